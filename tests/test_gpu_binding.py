"""Binding checks that need a GPU tensor: mixed devices and caller buffers
that do not match the call are rejected on the host, before any launch."""
import pytest
import torch

import rank_markov_draft_amd as rmd

pytestmark = pytest.mark.gpu

B, M, V, r, d = 2, 3, 64, 16, 8


def _dev():
    g = torch.Generator().manual_seed(1)
    t = {
        "base": torch.randn(B, M, V, generator=g).to(torch.bfloat16),
        "ids": torch.randint(0, V, (B, M), generator=g),
        "first": torch.randint(0, V, (B,), generator=g),
        "w1": (0.02 * torch.randn(V, r, generator=g)).to(torch.bfloat16),
        "w2": (0.02 * torch.randn(V, r, generator=g)).to(torch.bfloat16),
        "h": torch.randn(B, M, d, generator=g).to(torch.bfloat16),
        "gw": (0.1 * torch.randn(r, d + r, generator=g)).to(torch.bfloat16),
        "gb": torch.zeros(r).to(torch.bfloat16),
    }
    return {k: v.cuda() for k, v in t.items()}


def test_mixed_devices_are_rejected(native):
    t = _dev()
    with pytest.raises(ValueError, match="token_ids is on cpu"):
        rmd.apply_block_logits(t["base"], t["ids"].cpu(), t["w1"], t["w2"])
    with pytest.raises(ValueError, match="w2 is on cpu"):
        rmd.sample_block_tokens(t["base"], t["first"], t["w1"], t["w2"].cpu())
    with pytest.raises(ValueError, match="hidden_states is on cpu"):
        rmd.apply_block_logits_gated(t["base"], t["ids"], t["w1"], t["w2"], t["gw"], t["gb"], t["h"].cpu())
    with pytest.raises(ValueError, match="gate_weight is on cpu"):
        rmd.sample_block_tokens_gated(t["base"], t["first"], t["w1"], t["w2"], t["gw"].cpu(), t["gb"], t["h"])
    with pytest.raises(ValueError, match="token_ids is on cpu"):
        rmd.apply_block_logits_backward(t["base"], t["ids"].cpu(), t["w1"], t["w2"])


def test_caller_buffers_must_match(native):
    t = _dev()
    with pytest.raises(ValueError, match="tokens_out"):
        rmd.sample_block_tokens(t["base"], t["first"], t["w1"], t["w2"],
                                tokens_out=torch.empty((B, M + 1), dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError, match="tokens_out"):
        rmd.sample_block_tokens(t["base"], t["first"], t["w1"], t["w2"],
                                tokens_out=torch.empty((B, M), dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError, match="logits_out"):
        rmd.sample_block_tokens(t["base"], t["first"], t["w1"], t["w2"],
                                logits_out=torch.empty((B, M, V), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="out must be"):
        rmd.apply_block_logits(t["base"], t["ids"], t["w1"], t["w2"],
                               out=torch.empty((B, M, V + 8), dtype=torch.bfloat16, device="cuda"))


def test_unused_gate_tensors_are_not_checked(native):
    """Without hidden states the gated call is the vanilla head; gate tensors
    it does not read may live anywhere."""
    t = _dev()
    out = rmd.apply_block_logits_gated(t["base"], t["ids"], t["w1"], t["w2"], t["gw"].cpu(), t["gb"].cpu(), None)
    ref = rmd.apply_block_logits(t["base"], t["ids"], t["w1"], t["w2"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_bandwidth_probes_are_exact(native):
    """The streaming copy and the read-mix pass that bench.py times as HBM
    ceilings move the bytes exactly, including a partial last pass of their
    workgroups, and write nothing past the end."""
    import ctypes
    from rank_markov_draft_amd import _lib
    bw = _lib.load_bandwidth()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for n in (16, 4096 + 16, (1 << 20) + 48, 64 << 20):
        src = torch.randint(0, 256, (2 * n,), dtype=torch.uint8, device="cuda")
        dst = torch.zeros(n + 64, dtype=torch.uint8, device="cuda")
        assert bw.dspark_bandwidth_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), n,
                                        stream) == 0
        torch.cuda.synchronize()
        assert torch.equal(dst[:n], src[:n]), n
        assert not dst[n:].any(), "bytes past the end were written"
        for m in (n, n + 16 * (n // 32), 2 * n):          # 1, ~1.5 and 2 source bytes per byte written
            dst.zero_()
            assert bw.dspark_bandwidth_read_mix(ctypes.c_void_p(dst.data_ptr()), n, ctypes.c_void_p(src.data_ptr()),
                                                m, stream) == 0
            torch.cuda.synchronize()
            s16 = src[:m].view(torch.int32).view(-1, 4).cpu()
            want = s16[: n // 16].clone()
            tail = s16[n // 16:]
            want[: tail.shape[0]] ^= tail
            assert torch.equal(dst[:n].view(torch.int32).view(-1, 4).cpu(), want), (n, m)
            assert not dst[n:].any()
