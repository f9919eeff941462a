"""The sampling entry point that allocates nothing
(dspark_markov_sample_block_static), called through the C ABI, against the
workspace entry point dspark_markov_sample_block on the same inputs: two
calls in a row, the second smaller, must give the same tokens and corrected
logits bit for bit (the same kernels run on the static scratch)."""
import ctypes

import numpy as np
import pytest
import torch

from rank_markov_draft_amd import _lib
from rank_markov_draft_amd import workloads as wl
from tests.gpu_util import device_inputs, from_dev

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _tag(t):
    return _lib.DSPARK_BF16 if t.dtype == torch.bfloat16 else _lib.DSPARK_F32


def _call(L, static, d, T, seed, logits):
    B, M, V = d["base"].shape
    r = d["w1"].shape[1]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    tok = torch.full((B, M), -7, dtype=torch.int64, device="cuda")
    corr = torch.empty_like(d["base"]) if logits else None
    args = (_p(d["base"]), _tag(d["base"]), _p(d["first_prev"]), _p(d["w1"]), _p(d["w2"]), _tag(d["w1"]),
            B, M, V, r, float(T), seed, 0, 0, _p(tok), _p(corr))
    if static:
        st = L.dspark_markov_sample_block_static(*args, stream)
    else:
        nb = int(L.dspark_markov_workspace_bytes(B, M, V, r, 1))
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        assert L.dspark_markov_workspace_init(_p(ws), nb, stream) == 0
        st = L.dspark_markov_sample_block(*args, _p(ws), nb, stream)
    assert st == 0, _lib.load().dspark_markov_last_error()
    torch.cuda.synchronize()
    return from_dev(tok), (from_dev(corr) if logits else None)


@pytest.mark.parametrize("order", ["chain-then-steps", "steps-then-chain"])
def test_static_scratch_entry_point_matches_workspace_entry_point(native, order):
    L = _lib.load()
    big = wl.make_inputs(wl.WORKLOADS["greedy_draft_64x5"])                         # persistent chain
    small = wl.make_inputs(wl.WORKLOADS["temperature_draft_256x8"], B=24, M=3, V=4096, r=256, seed=9)
    cases = [(big, 0.0, 0, True), (small, 0.7, 1234, True)]
    if order == "steps-then-chain":
        small2 = wl.make_inputs(wl.WORKLOADS["greedy_draft_64x5"], B=40, M=4, V=8192, r=256, seed=10)
        cases = [(wl.make_inputs(wl.WORKLOADS["temperature_draft_256x8"], B=96, M=4, V=16384, r=256, seed=11),
                  0.7, 77, True), (small2, 0.0, 0, True)]
    for inp, T, seed, logits in cases:
        d = device_inputs({k: inp[k] for k in ("base", "first_prev", "w1", "w2")})
        print(f"[no-alloc] {order}: B={inp['base'].shape[0]} M={inp['base'].shape[1]} V={inp['base'].shape[2]} "
              f"T={T}", flush=True)
        t_ref, c_ref = _call(L, False, d, T, seed, logits)
        t_got, c_got = _call(L, True, d, T, seed, logits)
        assert t_ref.min() >= 0
        assert np.array_equal(t_got, t_ref)
        assert np.array_equal(c_got, c_ref)


def test_static_scratch_rejects_sizes_beyond_it(native):
    L = _lib.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    B, M, V, r = 4096, 5, 151936, 256               # needs 39 MB of workspace
    fake = ctypes.c_void_p(0x1000)
    st = L.dspark_markov_sample_block_static(fake, _lib.DSPARK_BF16, fake, fake, fake, _lib.DSPARK_BF16,
                                             B, M, V, r, 0.0, 0, 0, 0, fake, None, stream)
    assert st == 3
    assert b"static scratch" in L.dspark_markov_last_error()
