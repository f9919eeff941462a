"""The persistent chain's failure path, forced from the host.

A workspace control word (byte 128) makes every device-wide wait of the
persistent chains (greedy and temperature) give up at once, as a real 1 s timeout would, while
every workgroup still exits normally.  The call must then return -1 for
every token, the library must report DSPARK_ERR_DEVICE on the next read of
the workspace's error words, and later persistent calls on the unread
workspace must refuse to produce tokens (-1) until that read clears it."""
import ctypes

import numpy as np
import pytest
import torch

import rank_markov_draft_amd as rmd
from rank_markov_draft_amd import _lib
from rank_markov_draft_amd import workloads as wl
from tests.gpu_util import device_inputs, from_dev

pytestmark = pytest.mark.gpu


def _raw_read(ws):
    n = ctypes.c_int64(-1)
    st = _lib.load().dspark_markov_read_device_error(
        ws.ptr, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(n))
    return st, int(n.value)


@pytest.mark.parametrize("T,B,name", [(0.0, 8, "greedy_draft_64x5"), (0.7, 8, "greedy_draft_64x5"),
                                      (0.7, 40, "greedy_draft_64x5"), (0.0, 24, "greedy_draft_64x5_f32logits"),
                                      (0.7, 24, "temperature_draft_256x8_f32logits")])
def test_forced_chain_timeout_gives_sentinel_tokens(native, T, B, name):
    M, V, r = 5, 4096, 256                   # bf16 weights: the persistent chains
    inp = wl.make_inputs(wl.WORKLOADS[name], B=B, M=M, V=V, r=r, seed=21)
    d = device_inputs({k: inp[k] for k in ("base", "first_prev", "w1", "w2")})
    ws = rmd.Workspace(B, M, V, r, sample=True)

    def call(**kw):
        return rmd.sample_block_tokens(d["base"], d["first_prev"], d["w1"], d["w2"], T, seed=4, workspace=ws,
                                       **kw)

    good, _ = call()
    assert rmd.read_device_error(ws) == 0
    good = from_dev(good)
    assert good.min() >= 0

    print(f"[chain failure] forced timeout, T={T} B={B} M=5 V=4096 r=256 {name}", flush=True)
    ws.set_chain_test_hook(True)
    tok, _ = call()
    torch.cuda.synchronize()
    assert np.all(from_dev(tok) == -1)
    st, _ = _raw_read(ws)
    assert st == _lib.DSPARK_ERR_DEVICE
    # the read cleared the record: with the hook off the chain runs again
    ws.set_chain_test_hook(False)
    tok, _ = call()
    assert rmd.read_device_error(ws) == 0
    assert np.array_equal(from_dev(tok), good)

    # an unread failure poisons the workspace: the next call does no work
    ws.set_chain_test_hook(True)
    call()
    ws.set_chain_test_hook(False)
    tok, _ = call()
    torch.cuda.synchronize()
    assert np.all(from_dev(tok) == -1)
    with pytest.raises(_lib.DsparkError):
        rmd.read_device_error(ws)
    tok, _ = call(check=True)                  # cleared: runs, and the check passes
    assert np.array_equal(from_dev(tok), good)

    # check=True raises on the failing call itself
    ws.set_chain_test_hook(True)
    with pytest.raises(_lib.DsparkError):
        call(check=True)
    ws.set_chain_test_hook(False)
    tok, _ = call(check=True)
    assert np.array_equal(from_dev(tok), good)
