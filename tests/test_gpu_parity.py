"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

The five workloads run at their full sizes in the launch configuration the
benchmark uses, and the oracle checks every row, token and element of
each.  Larger edge-size cases check sampled rows.  Element rule: bit-identical to the oracle or inside its admissible
interval for fp32 accumulation in any order; token rule: exactly the
selection on the GPU's own validated row (see tests/parity.py).
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import rank_markov_draft_amd as rmd
from oracle import oracle as orc
from rank_markov_draft_amd import workloads as wl
from tests import parity
from tests.gpu_util import device_inputs, from_dev, to_dev

pytestmark = pytest.mark.gpu


REPORT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out",
                      "parity_report.txt")


def _report(name, **kw):
    """Counts of each parity check, appended to gpurun_out/parity_report.txt."""
    line = f"[parity] {name}: " + ", ".join(f"{k}={v}" for k, v in kw.items())
    print(line)
    os.makedirs(os.path.dirname(REPORT), exist_ok=True)
    with open(REPORT, "a") as f:
        f.write(line + "\n")


def _chain_ids(first_prev, tokens):
    """Predecessors of a chain given its tokens: [first_prev, tok_0 .. tok_{M-2}]."""
    return np.concatenate([first_prev[:, None], tokens[:, :-1]], axis=1)


def run_apply(inp):
    d = device_inputs({k: inp[k] for k in ("base", "token_ids", "w1", "w2")})
    out = rmd.apply_block_logits(d["base"], d["token_ids"], d["w1"], d["w2"])
    torch.cuda.synchronize()
    return from_dev(out)


def run_sample(inp, T, seed=0, return_logits=True, position_offset=0, batch_offset=0):
    d = device_inputs({k: inp[k] for k in ("base", "first_prev", "w1", "w2")})
    B, M, V = inp["base"].shape
    ws = rmd.Workspace(B, M, V, inp["w1"].shape[1], sample=True)
    tok, corr = rmd.sample_block_tokens(d["base"], d["first_prev"], d["w1"], d["w2"], T, seed=seed,
                                        return_logits=return_logits, position_offset=position_offset,
                                        batch_offset=batch_offset, workspace=ws)
    assert rmd.read_device_error(ws) == 0      # synchronises; raises on a chain timeout
    return from_dev(tok), (from_dev(corr) if corr is not None else None)


def check_apply(inp, gpu, rows=None, name=""):
    """Oracle apply on all rows (rows=None) or on the flattened rows given."""
    B, M, V = inp["base"].shape
    if rows is None:
        ref = orc.apply_block(inp["base"], inp["token_ids"], inp["w1"], inp["w2"])
        rep = parity.check_logits(gpu, ref, inp["base"], inp["token_ids"], inp["w1"], inp["w2"])
    else:
        base = inp["base"].reshape(B * M, 1, V)[rows]
        ids = inp["token_ids"].reshape(B * M, 1)[rows]
        ref = orc.apply_block(base, ids, inp["w1"], inp["w2"])
        rep = parity.check_logits(gpu.reshape(B * M, 1, V)[rows], ref, base, ids, inp["w1"], inp["w2"])
    _report(name, **dataclasses.asdict(rep))
    return rep


def check_chain(inp, T, seed, tok, corr, brows=None, name=""):
    """Conditional per-step check of a sampled chain on batch rows `brows`."""
    B, M, V = inp["base"].shape
    brows = np.arange(B) if brows is None else np.asarray(brows)
    assert tok.shape == (B, M) and tok.min() >= 0 and tok.max() < V
    ids = _chain_ids(inp["first_prev"], tok)[brows]
    base = inp["base"][brows]
    ref = orc.apply_block(base, ids, inp["w1"], inp["w2"])
    lrep = parity.check_logits(corr[brows], ref, base, ids, inp["w1"], inp["w2"])
    b_abs = np.repeat(brows, M)
    k_abs = np.tile(np.arange(M), len(brows))
    trep = parity.check_tokens(tok[brows].reshape(-1), corr[brows].reshape(-1, V), ref.reshape(-1, V),
                               T, seed, b_abs, k_abs)
    _report(name, **dataclasses.asdict(lrep), **dataclasses.asdict(trep))
    return lrep, trep


# ------------------------------------------------------------ the five workloads
def test_tiny_fp32_apply_and_greedy(native):
    w = wl.WORKLOADS["tiny_fp32"]
    inp = wl.make_inputs(w)
    check_apply(inp, run_apply(inp), name=w.name + " apply")
    tok, corr = run_sample(inp, 0.0)
    check_chain(inp, 0.0, 0, tok, corr, name=w.name + " greedy")


def test_teacher_forced_320(native):
    w = wl.WORKLOADS["teacher_forced_320"]
    inp = wl.make_inputs(w)
    rep = check_apply(inp, run_apply(inp), name=w.name)
    assert rep.mismatches <= 1e-4 * rep.elements


def test_teacher_forced_320_f32logits(native):
    w = wl.WORKLOADS["teacher_forced_320_f32logits"]
    inp = wl.make_inputs(w)
    assert inp["base"].dtype == np.float32 and inp["w1"].dtype == np.uint16
    rep = check_apply(inp, run_apply(inp), name=w.name)
    assert rep.mismatches <= 1e-4 * rep.elements


def test_greedy_draft_64x5(native):
    w = wl.WORKLOADS["greedy_draft_64x5"]
    inp = wl.make_inputs(w)
    tok, corr = run_sample(inp, 0.0)
    lrep, trep = check_chain(inp, 0.0, 0, tok, corr, name=w.name)
    assert lrep.mismatches <= 1e-4 * lrep.elements
    # tokens-only call draws the same tokens
    tok2, none = run_sample(inp, 0.0, return_logits=False)
    assert none is None and np.array_equal(tok, tok2)


def test_temperature_draft_256x8(native):
    w = wl.WORKLOADS["temperature_draft_256x8"]
    inp = wl.make_inputs(w)
    tok, corr = run_sample(inp, w.temperature, seed=w.gumbel_seed)
    lrep, trep = check_chain(inp, w.temperature, w.gumbel_seed, tok, corr, name=w.name)
    assert trep.tokens == w.B * w.M and lrep.elements == w.elems
    assert trep.noise_ties <= 4 and lrep.mismatches <= 1e-4 * lrep.elements
    # the timed configuration returns tokens only: same draws
    tok2, _ = run_sample(inp, w.temperature, seed=w.gumbel_seed, return_logits=False)
    assert np.array_equal(tok, tok2)


@pytest.mark.parametrize("name", ["greedy_draft_64x5_f32logits", "temperature_draft_256x8_f32logits"])
def test_sampling_on_f32_logits(native, name):
    """Both drafts on fp32 base logits with bf16 weights, at full size, every
    row, token and element against the oracle (the step kernel's fp32-logit
    form: the bf16 bias widened exactly and added in fp32)."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    assert inp["base"].dtype == np.float32 and inp["w1"].dtype == np.uint16
    tok, corr = run_sample(inp, w.temperature, seed=w.gumbel_seed)
    lrep, trep = check_chain(inp, w.temperature, w.gumbel_seed, tok, corr, name=w.name)
    assert trep.tokens == w.B * w.M and lrep.elements == w.elems
    tok2, _ = run_sample(inp, w.temperature, seed=w.gumbel_seed, return_logits=False)
    assert np.array_equal(tok, tok2)


def test_teacher_forced_2560_zipf(native):
    w = wl.WORKLOADS["teacher_forced_2560_zipf"]
    inp = wl.make_inputs(w)
    gpu = run_apply(inp)
    rep = check_apply(inp, gpu, name=w.name)
    assert rep.elements == w.elems and rep.mismatches <= 1e-4 * rep.elements


# ------------------------------------------------------------ shapes and edges
@pytest.mark.parametrize("B,M,V,r,dtype", [
    (3, 7, 1000, 24, wl.BF16),      # ragged rows and last vocabulary tile, rank padded to 32
    (1, 1, 8, 8, wl.BF16),          # smallest tile case
    (2, 33, 4104, 40, wl.BF16),     # 66 rows (two tiles + 2), rank 40 -> 64
    (5, 5, 1001, 16, wl.BF16),      # V not a multiple of 8: generic kernel
    (2, 3, 640, 520, wl.BF16),      # rank above the tile kernel's 512: generic kernel
    (4, 6, 777, 12, wl.F32),        # fp32 generic kernel
    (2, 5, 2048, 512, wl.BF16),     # rank 512 tile kernel
])
def test_apply_shapes(native, B, M, V, r, dtype):
    w = dataclasses.replace(wl.WORKLOADS["teacher_forced_320"], dtype=dtype)
    inp = wl.make_inputs(w, B=B, M=M, V=V, r=r, seed=B * 1000 + V)
    check_apply(inp, run_apply(inp), name=f"apply B{B} M{M} V{V} r{r} dt{dtype}")


def _grouped_ids(kind, rng, n, V):
    if kind == "zipf":
        return wl.zipf_ids(rng, n, V, 1.1)
    if kind == "same":
        return np.full(n, V // 3, dtype=np.int64)
    if kind == "distinct":
        return rng.permutation(V)[:n].astype(np.int64)
    if kind == "bad-mix":                       # Zipf ids, one in eight out of range
        ids = wl.zipf_ids(rng, n, V, 1.1)
        bad = rng.random(n) < 0.125
        ids[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, V + 5)
        return ids
    raise ValueError(kind)


@pytest.mark.parametrize("B,M,V,r,kind", [
    (64, 64, 1024, 64, "zipf"),        # 4096 rows: the largest grouped call
    (17, 241, 512, 32, "zipf"),        # 4097 rows: the row-order kernel instead
    (31, 33, 700, 16, "zipf"),         # 1023 rows: no plan, rows in their own order
    (32, 33, 1000, 24, "same"),        # 1056 rows, one distinct token, rank padded to 32
    (2, 512, 4104, 40, "distinct"),    # 1024 rows: every chunk of 32 rows adds two tiles
    (5, 205, 2048, 512, "bad-mix"),    # rank 512, ids outside [0, V)
    (1024, 1, 8, 8, "zipf"),           # one 8-column slice
    (9, 115, 3000, 256, "zipf"),       # rank 256, ragged last chunk and vocabulary slice
])
def test_apply_repeated_predecessors(native, B, M, V, r, kind):
    """Batches whose rows share predecessors (one bias per distinct token)."""
    w = wl.WORKLOADS["teacher_forced_2560_zipf"]
    inp = wl.make_inputs(w, B=B, M=M, V=V, r=r, seed=B * 7 + V)
    rng = np.random.default_rng(B + M + V)
    ids = _grouped_ids(kind, rng, B * M, V).reshape(B, M)
    inp = dict(inp, token_ids=ids)
    d = device_inputs({k: inp[k] for k in ("base", "token_ids", "w1", "w2")})
    ws = rmd.Workspace(B, M, V, r, sample=False)
    out = from_dev(rmd.apply_block_logits(d["base"], d["token_ids"], d["w1"], d["w2"], workspace=ws))
    flat = ids.reshape(-1)
    bad = (flat < 0) | (flat >= V)
    assert rmd.read_device_error(ws) == int(bad.sum())
    flat_out = out.reshape(B * M, V)
    assert np.array_equal(flat_out[bad], inp["base"].reshape(B * M, V)[bad])
    good = np.nonzero(~bad)[0]
    check_apply(inp, out, rows=good, name=f"apply {kind} B{B} M{M} V{V} r{r}")


@pytest.mark.parametrize("B,M,V,r,kind", [
    (4, 300, 5000, 256, "zipf"),       # 1200 rows: one bias per distinct token
    (32, 33, 1000, 24, "same"),        # 1056 rows, one distinct token
    (31, 33, 700, 16, "zipf"),         # 1023 rows: no plan
    (9, 115, 3000, 512, "bad-mix"),    # rank 512, ids outside [0, V)
])
def test_apply_repeated_predecessors_f32_logits(native, B, M, V, r, kind):
    """fp32 logits with bf16 weights on the grouped path."""
    inp = _mixed_inputs(wl.F32, wl.BF16, B, M, V, r, seed=B * 5 + V)
    rng = np.random.default_rng(B + M + V + 1)
    ids = _grouped_ids(kind, rng, B * M, V).reshape(B, M)
    inp = dict(inp, token_ids=ids)
    d = device_inputs({k: inp[k] for k in ("base", "token_ids", "w1", "w2")})
    ws = rmd.Workspace(B, M, V, r, sample=False)
    out = from_dev(rmd.apply_block_logits(d["base"], d["token_ids"], d["w1"], d["w2"], workspace=ws))
    assert out.dtype == np.float32
    flat = ids.reshape(-1)
    bad = (flat < 0) | (flat >= V)
    assert rmd.read_device_error(ws) == int(bad.sum())
    flat_out = out.reshape(B * M, V)
    assert np.array_equal(flat_out[bad], inp["base"].reshape(B * M, V)[bad])
    good = np.nonzero(~bad)[0]
    check_apply(inp, out, rows=good, name=f"apply f32-logits {kind} B{B} M{M} V{V} r{r}")


@pytest.mark.parametrize("T", [0.0, 0.8])
@pytest.mark.parametrize("B,M,V,r,dtype", [
    (3, 4, 1000, 24, wl.BF16),
    (33, 2, 4104, 64, wl.BF16),
    (2, 3, 1001, 16, wl.BF16),
    (4, 5, 777, 12, wl.F32),
])
def test_sample_shapes(native, T, B, M, V, r, dtype):
    w = dataclasses.replace(wl.WORKLOADS["greedy_draft_64x5"], dtype=dtype)
    inp = wl.make_inputs(w, B=B, M=M, V=V, r=r, seed=7 + B + V)
    tok, corr = run_sample(inp, T, seed=11)
    check_chain(inp, T, 11, tok, corr, name=f"sample T{T} B{B} M{M} V{V} r{r} dt{dtype}")


@pytest.mark.parametrize("B,M,V,r", [
    (200, 3, 20000, 256),     # 13 groups of 16 rows (the last of 8), slices past the waves
    (17, 2, 8200, 128),       # two groups of 9 rows; a vocabulary of 256 + 8 slices
    (64, 1, 4096, 256),       # one step: only the first tokens' rows
    (5, 7, 65544, 32),        # one short group, seven steps, a ragged last slice
    (256, 2, 512, 64),        # 16 slices: most workgroups own no column
    (3, 2, 163840, 256),      # 20 slices a workgroup on 256 CUs: four slices' W2 rows in LDS
    (16, 2, 139264, 64),      # 17 slices a workgroup on 256 CUs: one LDS slice, rank 64
    (9, 3, 151928, 256),      # a ragged last slice among the LDS slices
])
def test_temperature_chain_shapes(native, B, M, V, r):
    """Temperature chains on the persistent sampling kernel (bf16, B <= 256,
    M * B <= 4096): every token and corrected logit against the oracle, and
    the tokens-only call gives the same tokens."""
    w = wl.WORKLOADS["temperature_draft_256x8"]
    inp = wl.make_inputs(w, B=B, M=M, V=V, r=r, seed=40 + B + M)
    tok, corr = run_sample(inp, 0.7, seed=77)
    check_chain(inp, 0.7, 77, tok, corr, name=f"temperature chain B{B} M{M} V{V} r{r}")
    tok2, _ = run_sample(inp, 0.7, seed=77, return_logits=False)
    assert np.array_equal(tok2, tok)


@pytest.mark.parametrize("B,M,V,r", [
    (200, 3, 20000, 256),     # 13 groups of 16 rows, one 1 KB segment a row
    (5, 7, 65544, 32),        # nine slices a workgroup: two segments, a ragged last slice
    (16, 2, 139264, 64),      # 17 slices on 256 CUs: one LDS slice, three segments (the last overlapping)
    (3, 2, 155648, 256),      # 19 slices on 256 CUs: three LDS slices, 608 columns
    (9, 3, 151928, 256),      # a ragged last slice among the LDS slices
    (256, 2, 512, 64),        # 16 slices: most workgroups own no column
])
def test_f32_logit_temperature_chain_shapes(native, B, M, V, r):
    """Temperature chains on fp32 logits (bf16 weights) run on the sampling
    chain's fp32-logit form (two staged units, up to 608 columns a CU):
    every token and corrected logit against the oracle, and the tokens-only
    call gives the same tokens."""
    w = wl.WORKLOADS["temperature_draft_256x8_f32logits"]
    inp = wl.make_inputs(w, B=B, M=M, V=V, r=r, seed=70 + B + M)
    assert inp["base"].dtype == np.float32
    tok, corr = run_sample(inp, 0.7, seed=78)
    check_chain(inp, 0.7, 78, tok, corr, name=f"f32-logit temperature chain B{B} M{M} V{V} r{r}")
    tok2, _ = run_sample(inp, 0.7, seed=78, return_logits=False)
    assert np.array_equal(tok2, tok)


@pytest.mark.parametrize("B,M,V,r", [
    (17, 3, 8200, 128),       # two groups of 9 rows, a ragged last workgroup
    (1, 7, 4096, 64),         # one row, seven steps
    (64, 1, 20000, 32),       # four groups, one step
    (33, 4, 65544, 256),      # three groups (the last of one row), a ragged last slice
])
def test_f32_logit_greedy_chain_shapes(native, B, M, V, r):
    """Greedy drafts on fp32 logits with bf16 weights run on the persistent
    chain's fp32-logit form: every token and corrected logit against the
    oracle, and the tokens-only call gives the same tokens."""
    w = wl.WORKLOADS["greedy_draft_64x5_f32logits"]
    inp = wl.make_inputs(w, B=B, M=M, V=V, r=r, seed=50 + B + M)
    assert inp["base"].dtype == np.float32
    tok, corr = run_sample(inp, 0.0)
    check_chain(inp, 0.0, 0, tok, corr, name=f"f32-logit chain B{B} M{M} V{V} r{r}")
    tok2, _ = run_sample(inp, 0.0, return_logits=False)
    assert np.array_equal(tok2, tok)


@pytest.mark.parametrize("B,M,V,r", [
    (65, 3, 20000, 256),      # one row past the greedy chain's 64: five groups
    (128, 2, 163840, 256),    # 20 slices a workgroup on 256 CUs (four in LDS)
    (256, 2, 8200, 64),       # 16 full groups, rank 64, a ragged last workgroup
    (48, 3, 163840, 256),     # a vocabulary past the greedy chain's 512 columns per CU (256 CUs)
])
def test_greedy_wide_batch_chain(native, B, M, V, r):
    """Greedy drafts the greedy chain does not take (65..256 rows, or more
    than 512 columns per CU) run on the sampling chain selecting the argmax
    of the corrected values: every token and corrected logit against the
    oracle, and the tokens-only call gives the same tokens."""
    w = wl.WORKLOADS["greedy_draft_64x5"]
    inp = wl.make_inputs(w, B=B, M=M, V=V, r=r, seed=60 + B + M)
    tok, corr = run_sample(inp, 0.0)
    check_chain(inp, 0.0, 0, tok, corr, name=f"greedy wide chain B{B} M{M} V{V} r{r}")
    tok2, _ = run_sample(inp, 0.0, return_logits=False)
    assert np.array_equal(tok2, tok)


def test_f32_logit_chain_equals_single_steps(native):
    """The fp32-logit chain over M steps equals M one-step calls fed the
    previous tokens (GPU against GPU, bitwise)."""
    w = wl.WORKLOADS["greedy_draft_64x5_f32logits"]
    inp = wl.make_inputs(w, B=40, M=5, V=8192, r=256)
    full_t, full_c = run_sample(inp, 0.0)
    prev = inp["first_prev"].copy()
    for k in range(5):
        step = dict(inp, base=np.ascontiguousarray(inp["base"][:, k:k + 1]), first_prev=prev)
        t, c = run_sample(step, 0.0, position_offset=k)
        assert np.array_equal(t[:, 0], full_t[:, k]) and np.array_equal(c[:, 0], full_c[:, k])
        prev = t[:, 0].copy()


def _mixed_inputs(ldt, wdt, B, M, V, r, seed):
    """Workload-shaped inputs with the logits in ldt and the weights in wdt."""
    w = dataclasses.replace(wl.WORKLOADS["teacher_forced_320"], dtype=wl.F32)
    inp = wl.make_inputs(w, B=B, M=M, V=V, r=r, seed=seed)
    if ldt == wl.BF16:
        inp["base"] = wl.to_bf16_bits(inp["base"])
    if wdt == wl.BF16:
        inp["w1"], inp["w2"] = wl.to_bf16_bits(inp["w1"]), wl.to_bf16_bits(inp["w2"])
    return inp


@pytest.mark.parametrize("ldt,wdt", [(wl.F32, wl.BF16), (wl.BF16, wl.F32)])
@pytest.mark.parametrize("B,M,V,r", [(3, 5, 1000, 24), (2, 33, 4104, 64)])
def test_apply_mixed_dtypes(native, ldt, wdt, B, M, V, r):
    inp = _mixed_inputs(ldt, wdt, B, M, V, r, seed=B + V)
    check_apply(inp, run_apply(inp), name=f"apply mixed L{ldt} W{wdt} B{B} M{M} V{V} r{r}")


@pytest.mark.parametrize("ldt,wdt,B,M,V,r,T", [
    (wl.F32, wl.F32, 16, 3, 129280, 256, 0.0),     # fp32 weights at the full vocabulary: matrix-core kernel
    (wl.F32, wl.F32, 8, 3, 129280, 256, 0.7),
    (wl.BF16, wl.F32, 12, 3, 129280, 256, 0.0),
    (wl.F32, wl.F32, 3, 4, 3001, 20, 0.7),         # V not a multiple of 4: the row-tile FMA kernel
    (wl.F32, wl.F32, 37, 2, 1000, 1040, 0.0),      # rank past 1024: 17 rank chunks; apply rows past one tile
    (wl.F32, wl.F32, 70, 2, 5000, 36, 0.7),        # 70 rows (two row tiles), a part rank chunk, an 8-column last tile
    (wl.BF16, wl.F32, 5, 3, 4100, 64, 0.7),        # bf16 logits, temperature, a ragged last tile
    (wl.F32, wl.F32, 2, 2, 1024, 4, 0.0),          # rank 4: one step of one block
])
def test_fp32_weight_kernel(native, ldt, wdt, B, M, V, r, T):
    """fp32 weights (and bf16 logits with fp32 weights) go to the
    matrix-core kernel (fp32 products, v_mfma_f32_16x16x4_f32) when r and V
    are multiples of 4, else to the row-tile FMA kernel: sampling and the
    teacher-forced apply against the oracle on every row."""
    inp = _mixed_inputs(ldt, wdt, B, M, V, r, seed=B * 31 + V)
    tok, corr = run_sample(inp, T, seed=3)
    check_chain(inp, T, 3, tok, corr, name=f"fp32-weight sample L{ldt} B{B} M{M} V{V} r{r} T{T}")
    check_apply(inp, run_apply(inp), name=f"fp32-weight apply L{ldt} B{B} M{M} V{V} r{r}")


@pytest.mark.parametrize("T", [0.0, 0.8])
@pytest.mark.parametrize("ldt,wdt", [(wl.F32, wl.BF16), (wl.BF16, wl.F32)])
def test_sample_mixed_dtypes(native, T, ldt, wdt):
    inp = _mixed_inputs(ldt, wdt, 5, 4, 2048, 32, seed=99)
    tok, corr = run_sample(inp, T, seed=5)
    check_chain(inp, T, 5, tok, corr, name=f"sample mixed T{T} L{ldt} W{wdt}")


def test_in_place_apply(native):
    w = wl.WORKLOADS["teacher_forced_320"]
    inp = wl.make_inputs(w, B=4, M=5, V=4096, r=256)
    d = device_inputs(inp)
    expect = from_dev(rmd.apply_block_logits(d["base"], d["token_ids"], d["w1"], d["w2"]))
    rmd.apply_block_logits(d["base"], d["token_ids"], d["w1"], d["w2"], out=d["base"])
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(d["base"]), expect)


def test_empty_inputs(native):
    w = wl.WORKLOADS["teacher_forced_320"]
    inp = wl.make_inputs(w, B=2, M=3, V=64, r=16)
    d = device_inputs(inp)
    out = rmd.apply_block_logits(d["base"][:, :0], d["token_ids"][:, :0], d["w1"], d["w2"])
    assert out.shape == (2, 0, 64)
    tok, corr = rmd.sample_block_tokens(d["base"][:, :0], d["first_prev"], d["w1"], d["w2"])
    assert tok.shape == (2, 0)
    tok, corr = rmd.sample_block_tokens(d["base"][:0], d["first_prev"][:0], d["w1"], d["w2"])
    assert tok.shape == (0, 3)


def test_out_of_range_ids_flag_device_error(native):
    w = wl.WORKLOADS["teacher_forced_320"]
    inp = wl.make_inputs(w, B=2, M=4, V=1024, r=32)
    ids = inp["token_ids"].copy()
    ids[0, 1] = 1024
    ids[1, 3] = -5
    d = device_inputs(dict(inp, token_ids=ids))
    ws = rmd.Workspace(2, 4, 1024, 32, sample=False)
    out = from_dev(rmd.apply_block_logits(d["base"], d["token_ids"], d["w1"], d["w2"], workspace=ws))
    assert rmd.read_device_error(ws) == 2
    assert rmd.read_device_error(ws) == 0            # the read clears the count
    # a bad row keeps its base logits (zero bias); good rows match the oracle
    assert np.array_equal(out[0, 1], inp["base"][0, 1]) and np.array_equal(out[1, 3], inp["base"][1, 3])
    good = np.array([0, 2, 3, 4, 5, 6])
    check_apply(dict(inp, token_ids=ids), out, rows=good, name="apply good rows beside bad ids")


def test_invalid_arguments_rejected_on_host(native):
    from rank_markov_draft_amd import _lib
    L = native
    w = wl.WORKLOADS["teacher_forced_320"]
    inp = wl.make_inputs(w, B=2, M=2, V=64, r=16)
    d = device_inputs(inp)
    ws = rmd.Workspace(2, 2, 64, 16, sample=True)
    out = torch.zeros_like(d["base"])
    p = lambda t: t.data_ptr()
    s = torch.cuda.current_stream().cuda_stream
    # r <= 0
    assert L.dspark_markov_apply_block(p(d["base"]), 1, p(d["token_ids"]), p(d["w1"]), p(d["w2"]), 1,
                                       2, 2, 64, 0, p(out), ws.ptr, ws.nbytes, s) == 1
    # workspace too small
    assert L.dspark_markov_apply_block(p(d["base"]), 1, p(d["token_ids"]), p(d["w1"]), p(d["w2"]), 1,
                                       2, 2, 64, 16, p(out), ws.ptr, 8, s) == 3
    # partial overlap of output and input
    assert L.dspark_markov_apply_block(p(d["base"]), 1, p(d["token_ids"]), p(d["w1"]), p(d["w2"]), 1,
                                       2, 2, 64, 16, p(d["base"]) + 2, ws.ptr, ws.nbytes, s) == 1
    # NaN temperature
    tok = torch.zeros((2, 2), dtype=torch.int64, device="cuda")
    assert L.dspark_markov_sample_block(p(d["base"]), 1, p(d["first_prev"]), p(d["w1"]), p(d["w2"]), 1,
                                        2, 2, 64, 16, float("nan"), 0, 0, 0, p(tok), None, ws.ptr,
                                        ws.nbytes, s) == 1
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0      # nothing was written


# ------------------------------------------------------------ invariants on the GPU
def test_equal_predecessors_identical_rows(native):
    """The vanilla bias is a pure function of the previous token: rows with
    equal predecessor and equal base rows are bit-identical, across row
    tiles and vocabulary slices."""
    w = wl.WORKLOADS["teacher_forced_320"]
    inp = wl.make_inputs(w, B=20, M=5, V=8192, r=256)
    base = inp["base"].copy()
    base[:] = base[0, 0]
    rng = np.random.default_rng(0)
    ids = rng.choice(np.array([3, 77, 8191]), size=(20, 5)).astype(np.int64)
    out = run_apply(dict(inp, base=base, token_ids=ids)).reshape(100, -1)
    for t in (3, 77, 8191):
        rows = out[ids.reshape(-1) == t]
        assert all(np.array_equal(rows[0], x) for x in rows[1:])


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_zero_w2_is_identity(native, dtype):
    w = dataclasses.replace(wl.WORKLOADS["teacher_forced_320"], dtype=dtype)
    inp = wl.make_inputs(w, B=3, M=5, V=4096, r=64)
    inp["w2"] = np.zeros_like(inp["w2"])
    out = run_apply(inp)
    assert np.array_equal(parity.as_f32(out), parity.as_f32(inp["base"]))
    tok, corr = run_sample(inp, 0.0)
    assert np.array_equal(parity.as_f32(corr), parity.as_f32(inp["base"]))
    assert np.array_equal(tok, np.argmax(parity.as_f32(inp["base"]), axis=-1))


@pytest.mark.parametrize("T", [0.0, 9.99e-6, -2.0])
def test_small_temperature_is_greedy(native, T):
    w = wl.WORKLOADS["greedy_draft_64x5"]
    inp = wl.make_inputs(w, B=16, M=5, V=8192, r=256)
    g, cg = run_sample(inp, 0.0)
    t, ct = run_sample(inp, T, seed=5)
    assert np.array_equal(g, t) and np.array_equal(cg, ct)


@pytest.mark.parametrize("T", [0.0, 0.7])
def test_chain_equals_single_steps(native, T):
    """One M-step call equals M one-step calls fed the previous tokens with
    position_offset = k (GPU against GPU, bitwise)."""
    w = wl.WORKLOADS["greedy_draft_64x5"]
    inp = wl.make_inputs(w, B=8, M=5, V=8192, r=256)
    full_t, full_c = run_sample(inp, T, seed=3)
    prev = inp["first_prev"].copy()
    for k in range(5):
        step = dict(inp, base=np.ascontiguousarray(inp["base"][:, k:k + 1]), first_prev=prev)
        t, c = run_sample(step, T, seed=3, position_offset=k)
        assert np.array_equal(t[:, 0], full_t[:, k]) and np.array_equal(c[:, 0], full_c[:, k])
        prev = t[:, 0].copy()


def test_batch_split_equals_whole(native):
    w = wl.WORKLOADS["temperature_draft_256x8"]
    inp = wl.make_inputs(w, B=12, M=3, V=8192, r=256)
    whole, _ = run_sample(inp, 0.7, seed=9)
    part = dict(inp, base=np.ascontiguousarray(inp["base"][4:10]),
                first_prev=np.ascontiguousarray(inp["first_prev"][4:10]))
    t, _ = run_sample(part, 0.7, seed=9, batch_offset=4)
    assert np.array_equal(t, whole[4:10])


def test_deterministic_and_workspace_reuse(native):
    w = wl.WORKLOADS["greedy_draft_64x5"]
    inp = wl.make_inputs(w, B=32, M=5, V=16384, r=256)
    d = device_inputs(inp)
    ws = rmd.Workspace(32, 5, 16384, 256, sample=True)
    outs = []
    for T in (0.0, 0.9, 0.0, 0.9):
        tok, corr = rmd.sample_block_tokens(d["base"], d["first_prev"], d["w1"], d["w2"], T, seed=1,
                                            workspace=ws)
        outs.append((from_dev(tok), from_dev(corr)))
    assert np.array_equal(outs[0][0], outs[2][0]) and np.array_equal(outs[0][1], outs[2][1])
    assert np.array_equal(outs[1][0], outs[3][0]) and np.array_equal(outs[1][1], outs[3][1])
    assert rmd.read_device_error(ws) == 0


@pytest.mark.parametrize("ldt", [wl.BF16, wl.F32])
# 8: the greedy chain; 70: the sampling chain selecting without noise; 300:
# step-by-step kernels
@pytest.mark.parametrize("B", [8, 70, 300])
def test_greedy_special_values(native, B, ldt):
    """Argmax semantics on planted values (W2 = 0, so corrected = base), on
    bf16 and fp32 logits: NaN ranks first (first NaN wins), exact ties go to
    the first column -- within a lane, across lanes and across workgroups --,
    -0 ties +0, and +-inf order."""
    V, M, r = 8192, 2, 32
    w = wl.WORKLOADS["greedy_draft_64x5"]
    inp = wl.make_inputs(w, B=B, M=M, V=V, r=r, seed=21)
    base = wl.bf16_bits_to_f32(inp["base"]).copy()
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    for b in range(B):
        kind = b % 8
        row = base[b]                       # [M, V] view
        if kind == 0:
            row[:, 3] = 100.0
            row[:, 777] = nan
            row[:, 5000] = nan
        elif kind == 1:
            row[:, [9, 4000, 4001]] = 50.0   # first of equal maxima
            row[:, 10] = 50.0                # same lane as column 9
        elif kind == 2:
            row[:, [7000, 6000]] = inf
        elif kind == 3:
            row[:] = -inf
            row[:, 8191] = -1e30
        elif kind == 4:
            row[:] = -inf                    # all equal: column 0
        elif kind == 5:
            row[:] = -np.abs(row) - 1.0
            row[:, [300, 299]] = 0.0
        elif kind == 6:
            row[:, 8191] = nan
        elif kind == 7:
            row[:] = -np.abs(row) - 1.0
            row[:, 4100] = np.float32(-0.0)   # -0 ties +0: the first column wins
            row[:, 4200] = 0.0
    inp["base"] = wl.to_bf16_bits(base) if ldt == wl.BF16 else base
    inp["w2"] = np.zeros_like(inp["w2"])
    tok, corr = run_sample(inp, 0.0)
    expect = {0: 777, 1: 9, 2: 6000, 3: 8191, 4: 0, 5: 299, 6: 8191, 7: 4100}
    for b in range(B):
        if b % 8 in expect:
            assert (tok[b] == expect[b % 8]).all(), (b, tok[b])
    check_chain(inp, 0.0, 0, tok, corr, name=f"greedy special values B{B} L{ldt}")


@pytest.mark.parametrize("ldt,V", [(wl.BF16, 8192), (wl.BF16, 163840), (wl.F32, 8192), (wl.F32, 151552)])
def test_temperature_special_values(native, ldt, V):
    """The temperature chain's selection on planted values (W2 = 0, so
    corrected = base, T = 0.7): a NaN ranks above every score and the first
    NaN wins, +inf scores tie and the first wins, all -inf rows take column
    0, and a single finite value among -inf wins.  At the large vocabularies
    the planted columns 512..639 lie in the slices whose W2 rows sit in LDS
    (bf16 logits: 640 columns a CU on 256 CUs; fp32: 608)."""
    B, M, r = 16, 2, 32
    w = wl.WORKLOADS["temperature_draft_256x8" if ldt == wl.BF16 else "temperature_draft_256x8_f32logits"]
    inp = wl.make_inputs(w, B=B, M=M, V=V, r=r, seed=23)
    base = (wl.bf16_bits_to_f32(inp["base"]) if ldt == wl.BF16 else inp["base"]).copy()
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    a, b2 = (600, 620) if V > 8192 else (777, 5000)
    for b in range(B):
        kind = b % 5
        row = base[b]
        if kind == 0:
            row[:, b2] = nan
            row[:, a] = nan
        elif kind == 1:
            row[:, [530, 515]] = inf
        elif kind == 2:
            row[:] = -inf
        elif kind == 3:
            row[:] = -inf
            row[:, a] = -1e30
    inp["base"] = wl.to_bf16_bits(base) if ldt == wl.BF16 else base
    inp["w2"] = np.zeros_like(inp["w2"])
    tok, corr = run_sample(inp, 0.7, seed=5)
    expect = {0: min(a, b2), 1: 515, 2: 0, 3: a}
    for b in range(B):
        if b % 5 in expect:
            assert (tok[b] == expect[b % 5]).all(), (b, tok[b])
    check_chain(inp, 0.7, 5, tok, corr, name=f"temperature special values L{ldt} V{V}")


def test_apply_beyond_31_bit_offsets(native):
    """16640 rows at V = 129280 (2.15e9 bf16 logits, 4.3 GB): element offsets
    pass 2^31, so the apply leaves the grouped and row-order kernels for the
    tile kernel with 64-bit offsets.  The base logits come from a seeded torch
    generator on the device; rows at the start, on both sides of element 2^31
    and at the end are copied back and checked against the oracle."""
    B, M, V, r = 3328, 5, 129280, 256
    n_rows = B * M
    assert n_rows * V > 2**31
    w = wl.WORKLOADS["teacher_forced_320"]
    small = wl.make_inputs(w)                  # W1 and W2 at this V and r
    assert small["w1"].shape == (V, r)
    ids = np.random.default_rng(12).integers(0, V, size=(B, M)).astype(np.int64)
    gen = torch.Generator(device="cuda").manual_seed(12)
    base = torch.empty((B, M, V), dtype=torch.bfloat16, device="cuda")
    for b0 in range(0, B, 256):                # slices bound the fp32 temporary
        nb = min(256, B - b0)
        base[b0:b0 + nb] = (2.0 * torch.randn((nb, M, V), generator=gen, device="cuda")).to(torch.bfloat16)
    d = device_inputs({"token_ids": ids, "w1": small["w1"], "w2": small["w2"]})
    out = rmd.apply_block_logits(base, d["token_ids"], d["w1"], d["w2"])
    torch.cuda.synchronize()
    edge = 2**31 // V                          # the row that holds element 2^31
    rows = np.array([0, 1, edge - 1, edge, edge + 1, n_rows - 2, n_rows - 1])
    sel = torch.as_tensor(rows, device="cuda")
    base_s = from_dev(base.view(n_rows, V).index_select(0, sel)).reshape(len(rows), 1, V)
    out_s = from_dev(out.view(n_rows, V).index_select(0, sel)).reshape(len(rows), 1, V)
    del base, out
    torch.cuda.empty_cache()
    ids_s = ids.reshape(n_rows, 1)[rows]
    ref = orc.apply_block(base_s, ids_s, small["w1"], small["w2"])
    rep = parity.check_logits(out_s, ref, base_s, ids_s, small["w1"], small["w2"])
    _report("apply beyond 2^31 elements", **dataclasses.asdict(rep))
    assert rep.mismatches <= 1e-4 * rep.elements


@pytest.mark.parametrize("B", [4096, 4097])
@pytest.mark.parametrize("T", [0.0, 0.7])
def test_sample_at_the_step_kernel_row_limit(native, B, T):
    """4096 batch rows are the most the step kernel stages in LDS; 4097 take
    the tile kernel.  Sampled batch rows (the first and last among them) are
    checked step by step against the oracle."""
    w = wl.WORKLOADS["temperature_draft_256x8"]
    inp = wl.make_inputs(w, B=B, M=2, V=512, r=64, seed=B)
    tok, corr = run_sample(inp, T, seed=3)
    rows = np.unique(np.concatenate([np.random.default_rng(B).choice(B, 60, replace=False), [0, B - 1]]))
    check_chain(inp, T, 3, tok, corr, brows=rows, name=f"sample B{B} T{T} at the step kernel's row limit")


def test_workspace_shared_across_shapes_and_operations(native):
    """One workspace serves calls of different shapes and operations in any
    order (one layout for every call; the chain's area holds nothing else):
    a temperature step call with more rows and a wider vocabulary, an apply
    and a backward, then greedy chains, each equal to its result on a fresh
    workspace."""
    w = wl.WORKLOADS["greedy_draft_64x5"]
    big = wl.make_inputs(wl.WORKLOADS["temperature_draft_256x8"], B=96, M=3, V=16384, r=256, seed=31)
    chain_in = wl.make_inputs(w, B=40, M=4, V=8192, r=256, seed=32)
    chain2_in = wl.make_inputs(w, B=64, M=7, V=8192, r=256, seed=33)
    ws = rmd.Workspace(96, 8, 16384, 256, sample=True, backward=True)
    db = device_inputs({k: big[k] for k in ("base", "first_prev", "token_ids", "w1", "w2")})
    dc = device_inputs({k: chain_in[k] for k in ("base", "first_prev", "w1", "w2")})
    dc2 = device_inputs({k: chain2_in[k] for k in ("base", "first_prev", "w1", "w2")})

    def chain(d, workspace=None):
        tok, corr = rmd.sample_block_tokens(d["base"], d["first_prev"], d["w1"], d["w2"], 0.0, workspace=workspace)
        torch.cuda.synchronize()
        return from_dev(tok), from_dev(corr)

    want1, want2 = chain(dc), chain(dc2)
    rmd.sample_block_tokens(db["base"], db["first_prev"], db["w1"], db["w2"], 0.7, seed=5, workspace=ws)
    got = chain(dc, ws)
    assert np.array_equal(got[0], want1[0]) and np.array_equal(got[1], want1[1])
    rmd.apply_block_logits(db["base"], db["token_ids"], db["w1"], db["w2"], workspace=ws)
    rmd.apply_block_logits_backward(db["base"], db["token_ids"], db["w1"], db["w2"], workspace=ws)
    got = chain(dc2, ws)
    assert np.array_equal(got[0], want2[0]) and np.array_equal(got[1], want2[1])
    got = chain(dc, ws)
    assert np.array_equal(got[0], want1[0])
    assert rmd.read_device_error(ws) == 0
