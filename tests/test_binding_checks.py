"""Host-side argument checks of the Python binding: tensors the kernels
would read or write must be on the logits' GPU, and caller-provided output
buffers must match the call.  Every case here is rejected before any
library or device call, so these run without a GPU."""
import pytest
import torch

import rank_markov_draft_amd as rmd

B, M, V, r, d = 2, 3, 64, 16, 8


def _cpu():
    g = torch.Generator().manual_seed(0)
    return {
        "base": torch.randn(B, M, V, generator=g),
        "ids": torch.randint(0, V, (B, M), generator=g),
        "first": torch.randint(0, V, (B,), generator=g),
        "w1": torch.randn(V, r, generator=g),
        "w2": torch.randn(V, r, generator=g),
        "h": torch.randn(B, M, d, generator=g),
        "gw": torch.randn(r, d + r, generator=g),
        "gb": torch.randn(r, generator=g),
    }


def test_host_tensors_are_rejected():
    t = _cpu()
    with pytest.raises(ValueError, match="runs on a GPU"):
        rmd.apply_block_logits(t["base"], t["ids"], t["w1"], t["w2"])
    with pytest.raises(ValueError, match="runs on a GPU"):
        rmd.sample_block_tokens(t["base"], t["first"], t["w1"], t["w2"], 0.7)
    with pytest.raises(ValueError, match="runs on a GPU"):
        rmd.apply_block_logits_gated(t["base"], t["ids"], t["w1"], t["w2"], t["gw"], t["gb"], t["h"])
    with pytest.raises(ValueError, match="runs on a GPU"):
        rmd.sample_block_tokens_gated(t["base"], t["first"], t["w1"], t["w2"], t["gw"], t["gb"], t["h"])
    with pytest.raises(ValueError, match="runs on a GPU"):
        rmd.apply_block_logits_backward(t["base"], t["ids"], t["w1"], t["w2"])


def test_empty_host_inputs_are_rejected_too():
    """The device check comes before the empty-input shortcut."""
    t = _cpu()
    with pytest.raises(ValueError, match="runs on a GPU"):
        rmd.apply_block_logits(t["base"][:, :0], t["ids"][:, :0], t["w1"], t["w2"])
    with pytest.raises(ValueError, match="runs on a GPU"):
        rmd.sample_block_tokens(t["base"][:, :0], t["first"], t["w1"], t["w2"])


def test_check_device_names_the_foreign_tensor():
    """_check_device compares every named tensor with the logits' device."""
    cuda0 = torch.device("cuda", 0)
    t = _cpu()
    with pytest.raises(ValueError, match="token_ids is on cpu"):
        rmd._check_device(cuda0, None, token_ids=t["ids"])
    rmd._check_device(cuda0, None, token_ids=None)   # absent tensors are skipped
