"""GPU parity of the teacher-forced backward (training) against the CPU
oracle, through the C ABI.

dW2w and dW1 elements must be bit-identical to the oracle's or lie in its
admissible interval for fp32 accumulation in any order
(oracle.backward_bounds); fp32 weights must also be within 1e-5 relative
with the forward's floor of 1e-2 (sums over V cancel).  Rows of dW1 that no
valid id refers to must be exactly zero.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import rank_markov_draft_amd as rmd
from oracle import oracle as orc
from rank_markov_draft_amd import workloads as wl
from tests.gpu_util import device_inputs, from_dev

pytestmark = pytest.mark.gpu

REPORT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out",
                      "parity_report.txt")


def _report(name, **kw):
    line = f"[parity] {name}: " + ", ".join(f"{k}={v}" for k, v in kw.items())
    print(line, flush=True)
    os.makedirs(os.path.dirname(REPORT), exist_ok=True)
    with open(REPORT, "a") as f:
        f.write(line + "\n")


def _f32(a):
    return wl.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def run_backward(inp, ws=None):
    d = device_inputs({k: inp[k] for k in ("grad", "token_ids", "w1", "w2")})
    gw1, gw2 = rmd.apply_block_logits_backward(d["grad"], d["token_ids"], d["w1"], d["w2"], workspace=ws)
    torch.cuda.synchronize()
    return from_dev(gw1), from_dev(gw2)


def _check(kind, gpu, inp, ids_valid, which, cols, name):
    """Elements (which[i], cols[i]) of dW2 (kind 'dw2') or dW1 ('dw1')."""
    g = _f32(gpu)[which, cols]
    lo, mid, hi = orc.backward_bounds(inp["grad"].reshape(-1, inp["grad"].shape[-1])[ids_valid],
                                      inp["token_ids"].reshape(-1)[ids_valid], inp["w1"], inp["w2"], kind,
                                      which, cols)
    same = g.view(np.uint32) == mid.view(np.uint32)
    inside = (lo <= g) & (g <= hi)
    bad = ~(same | inside)
    assert not bad.any(), (f"{name} {kind}: {int(bad.sum())} of {g.size} outside the interval; first "
                           f"{int(np.argmax(bad))}: gpu {g[bad][0]!r} oracle {mid[bad][0]!r} "
                           f"[{lo[bad][0]!r}, {hi[bad][0]!r}]")
    if gpu.dtype != np.uint16:   # the forward's fp32 rule: 1e-5 relative, floor 1e-2
        err = np.abs(g.astype(np.float64) - mid)
        ok = err <= 1e-5 * np.maximum(np.abs(mid), 1e-2)
        assert ok.all(), (f"{name} {kind}: {int((~ok).sum())} fp32 elements beyond 1e-5 relative "
                          f"(max abs diff {float(err.max())!r})")
    return int((~same).sum()), g.size


def check_backward(inp, gdw1, gdw2, n_dw2=None, n_dw1=None, name="", seed=0):
    V, r = inp["w1"].shape
    flat = inp["token_ids"].reshape(-1)
    valid = (flat >= 0) & (flat < V)
    rng = np.random.default_rng(seed)
    if n_dw2 is None:
        v2, j2 = (a.reshape(-1) for a in np.meshgrid(np.arange(V), np.arange(r), indexing="ij"))
    else:
        v2, j2 = rng.integers(0, V, n_dw2), rng.integers(0, r, n_dw2)
        v2 = np.concatenate([v2, [0, V - 1]])
        j2 = np.concatenate([j2, [0, r - 1]])
    m2, t2 = _check("dw2", gdw2, inp, valid, v2, j2, name)
    ids = np.unique(flat[valid])
    if n_dw1 is None:
        x1, j1 = (a.reshape(-1) for a in np.meshgrid(ids, np.arange(r), indexing="ij"))
    else:
        x1, j1 = rng.choice(ids, n_dw1), rng.integers(0, r, n_dw1)
    m1, t1 = _check("dw1", gdw1, inp, valid, x1, j1, name)
    untouched = np.setdiff1d(np.arange(V), ids)
    assert not _f32(gdw1)[untouched].any(), "dW1 rows no id refers to must be zero"
    _report(name, dw2_elements=t2, dw2_mismatches=m2, dw1_elements=t1, dw1_mismatches=m1)


def _inputs(dtype=wl.BF16, ldt=None, seed=0, **sizes):
    w = dataclasses.replace(wl.WORKLOADS["teacher_forced_320_backward"], dtype=dtype,
                            logits_dtype=-1 if ldt is None else ldt)
    return wl.make_inputs(w, seed=seed, **sizes)


def test_teacher_forced_320_backward(native):
    w = wl.WORKLOADS["teacher_forced_320_backward"]
    inp = wl.make_inputs(w)
    gdw1, gdw2 = run_backward(inp)
    check_backward(inp, gdw1, gdw2, n_dw2=4000, n_dw1=600, name=w.name)
    # deterministic: a second call gives the same bits
    gdw1b, gdw2b = run_backward(inp)
    assert np.array_equal(gdw1, gdw1b) and np.array_equal(gdw2, gdw2b)


@pytest.mark.parametrize("B,M,V,r,dtype,ldt,ids", [
    (3, 5, 1000, 24, wl.BF16, None, "uniform"),      # rank padded to 32
    (2, 33, 4104, 64, wl.BF16, None, "repeats"),     # several rows per id, 66 rows
    (4, 9, 2048, 256, wl.BF16, wl.F32, "repeats"),   # fp32 gradient, bf16 weights
    (1, 300, 1040, 256, wl.BF16, None, "repeats"),   # 300 rows: two row groups in the de product
    (3, 4, 777, 12, wl.F32, None, "uniform"),        # fp32: scalar kernels
    (2, 3, 1001, 16, wl.BF16, None, "uniform"),      # V % 8 != 0: scalar kernels
    (2, 5, 640, 512, wl.BF16, None, "repeats"),      # rank 512: scalar kernels
])
def test_backward_shapes(native, B, M, V, r, dtype, ldt, ids):
    inp = _inputs(dtype, ldt, seed=B + M + V, B=B, M=M, V=V, r=r)
    if ids == "repeats":
        rng = np.random.default_rng(V)
        inp["token_ids"] = rng.integers(0, max(V // 50, 2), size=(B, M)).astype(np.int64)
    gdw1, gdw2 = run_backward(inp)
    check_backward(inp, gdw1, gdw2, name=f"backward B{B} M{M} V{V} r{r} W{dtype} L{ldt} {ids}")


def test_backward_rows_beyond_one_block(native):
    """4400 rows: the dW2 kernel walks two blocks of row offsets; sampled
    elements of both gradients."""
    inp = _inputs(seed=4, B=1100, M=4, V=1024, r=64)
    rng = np.random.default_rng(1)
    inp["token_ids"] = rng.integers(0, 300, size=(1100, 4)).astype(np.int64)
    gdw1, gdw2 = run_backward(inp)
    check_backward(inp, gdw1, gdw2, n_dw2=3000, n_dw1=400, name="backward 4400 rows")


def test_backward_bad_ids_and_empty(native):
    """Ids outside [0, V) contribute nothing and are counted; no rows gives
    zero gradients."""
    B, M, V, r = 3, 7, 2048, 64
    inp = _inputs(seed=2, B=B, M=M, V=V, r=r)
    ids = inp["token_ids"].copy()
    ids[0, 0], ids[1, 2], ids[2, 6] = -3, V, 2**40
    inp["token_ids"] = ids
    ws = rmd.Workspace(B, M, V, r, sample=False, backward=True)
    gdw1, gdw2 = run_backward(inp, ws=ws)
    assert rmd.read_device_error(ws) == 3
    check_backward(inp, gdw1, gdw2, name="backward bad ids")
    empty = dict(inp, grad=inp["grad"][:, :0], token_ids=ids[:, :0])
    gdw1, gdw2 = run_backward(empty)
    assert not _f32(gdw1).any() and not _f32(gdw2).any()
