"""DSpark low-rank Markov head on MI355X (gfx950).

Python binding of libdspark_markov.so with the names of the pages'
VanillaMarkov methods (third-party markov_head.py page):

* ``apply_block_logits(base_logits, token_ids, w1, w2)`` -- teacher-forced
  bias of every block position by its given predecessor;
* ``sample_block_tokens(base_logits, first_prev_token_ids, w1, w2,
  temperature=0.0, ...)`` -- left-to-right sampling, each position biased by
  the token drawn at the previous one.

``apply_block_logits_backward`` gives the gradients of W1 and W2 for a
gradient of the teacher-forced corrected logits (training).
``apply_block_logits_lm_head`` fuses the drafter's FP32 vocabulary head
(the base logits) with the teacher-forced bias.

The gated head (the pages' GatedMarkovHead) has the same two operations,
``apply_block_logits_gated`` and ``sample_block_tokens_gated``, which also
take the backbone hidden states and the gate_proj weight and bias.

Tensors must live on the current HIP device.  ``w1`` is the Embedding
weight [V, r]; ``w2`` is the Linear(r, V) weight [V, r].  This module only
marshals arguments (dtype tags, pointers, sizes, the current stream) and
allocates outputs and workspace with torch: every step of the computation
runs in the library's kernels.  There is no fallback path: if the library
is missing, the first call raises.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

__all__ = ["apply_block_logits", "sample_block_tokens", "apply_block_logits_gated",
           "sample_block_tokens_gated", "apply_block_logits_backward", "apply_block_logits_lm_head", "Workspace",
           "read_device_error", "workspace_bytes"]


def _dtype_tag(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return _lib.DSPARK_F32
    if t.dtype == torch.bfloat16:
        return _lib.DSPARK_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; the head takes float32 or bfloat16")


def _stream_handle(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def workspace_bytes(B: int, M: int, V: int, r: int, sample: bool, hidden: int | None = None) -> int:
    """Workspace bytes of a call; ``hidden`` (the hidden size d, or 0 for the
    gated calls' vanilla fallback) sizes it for the gated calls."""
    if hidden is None:
        return int(_lib.load().dspark_markov_workspace_bytes(B, M, V, r, 1 if sample else 0))
    return int(_lib.load().dspark_markov_gated_workspace_bytes(B, M, V, r, hidden, 1 if sample else 0))


class Workspace:
    """Device workspace for a family of calls of at most the given sizes
    (``hidden``: the hidden size of gated calls; ``backward``: sized for the
    backward as well).

    Zero-filled once at creation; the library leaves it ready for the next
    call.  Calls sharing one workspace must be ordered on one stream."""

    def __init__(self, B: int, M: int, V: int, r: int, sample: bool, device=None,
                 hidden: int | None = None, backward: bool = False):
        device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.nbytes = max(workspace_bytes(B, M, V, r, sample, hidden), 256)
        if backward:
            self.nbytes = max(self.nbytes, int(_lib.load().dspark_markov_backward_workspace_bytes(B, M, V, r)))
        self.buffer = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        _lib.check(_lib.load().dspark_markov_workspace_init(
            _ptr(self.buffer), self.nbytes, _stream_handle(device)), "workspace_init")

    @property
    def ptr(self):
        return _ptr(self.buffer)

    def set_chain_test_hook(self, on: bool):
        """Tests of the failure path: with the hook on, the persistent chain's
        device-wide waits give up at once, so the call returns -1 tokens and
        records a failure without a stall (control word at byte 128)."""
        self.buffer[128:132].view(torch.int32).fill_(1 if on else 0)


def read_device_error(ws: Workspace) -> int:
    """Rows with out-of-range predecessor ids since the last read (synchronises).
    Raises DeviceError when a persistent sampling launch on ``ws`` failed since
    the last read (its tokens were -1); the record is cleared either way."""
    n = ctypes.c_int64(0)
    _lib.check(_lib.load().dspark_markov_read_device_error(
        ws.ptr, _stream_handle(ws.buffer.device), ctypes.byref(n)), "read_device_error")
    return int(n.value)


def _check_weights(w1: torch.Tensor, w2: torch.Tensor):
    if w1.dim() != 2 or w2.dim() != 2 or w1.shape != w2.shape:
        raise ValueError(f"w1 and w2 must both be [V, r], got {tuple(w1.shape)} and {tuple(w2.shape)}")
    if w1.dtype != w2.dtype:
        raise TypeError("w1 and w2 must share a dtype")


def apply_block_logits(base_logits: torch.Tensor, token_ids: torch.Tensor, w1: torch.Tensor,
                       w2: torch.Tensor, *, out: torch.Tensor | None = None,
                       workspace: Workspace | None = None) -> torch.Tensor:
    """Teacher-forced corrected logits base[..., M, V] + bias(token_ids[..., M]).

    ``out`` may be ``base_logits`` itself (in place).  An empty input returns
    ``base_logits`` (or ``out`` untouched), as the pages' method does."""
    _check_weights(w1, w2)
    if base_logits.dim() < 2:
        raise ValueError("base_logits must be [..., M, V]")
    V = base_logits.shape[-1]
    M = base_logits.shape[-2]
    B = 1
    for d in base_logits.shape[:-2]:
        B *= int(d)
    if tuple(token_ids.shape) != tuple(base_logits.shape[:-1]):
        raise ValueError(f"token_ids {tuple(token_ids.shape)} must be base_logits.shape[:-1]")
    if w1.shape[0] != V:
        raise ValueError(f"weights have vocabulary {w1.shape[0]}, logits {V}")
    _check_device(base_logits.device, workspace, token_ids=token_ids, w1=w1, w2=w2, out=out)
    if base_logits.numel() == 0:
        return base_logits if out is None else out
    base_c = base_logits.contiguous()
    ids = token_ids.to(torch.int64).contiguous()
    w1c, w2c = w1.contiguous(), w2.contiguous()
    if out is None:
        out = torch.empty_like(base_c)
    elif out.shape != base_logits.shape or out.dtype != base_logits.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like base_logits")
    r = w1.shape[1]
    if workspace is None:
        workspace = Workspace(B, M, V, r, sample=False, device=base_c.device)
    st = _lib.load().dspark_markov_apply_block(
        _ptr(base_c), _dtype_tag(base_c), _ptr(ids), _ptr(w1c), _ptr(w2c), _dtype_tag(w1c),
        B, M, V, r, _ptr(out), workspace.ptr, workspace.nbytes, _stream_handle(base_c.device))
    _lib.check(st, "apply_block_logits")
    return out


def sample_block_tokens(base_logits: torch.Tensor, first_prev_token_ids: torch.Tensor,
                        w1: torch.Tensor, w2: torch.Tensor, temperature: float | None = 0.0, *,
                        seed: int = 0, position_offset: int = 0, batch_offset: int = 0,
                        return_logits: bool = True, tokens_out: torch.Tensor | None = None,
                        logits_out: torch.Tensor | None = None,
                        workspace: Workspace | None = None, check: bool = False):
    """Left-to-right block sampling over base_logits [B, M, V].

    Returns ``(sampled_tokens [B, M] int64, corrected_logits [B, M, V] or None)``.
    ``temperature`` None or below 1e-5 is greedy argmax; otherwise Gumbel-max
    with Philox4x32-10 noise keyed by ``seed``.

    Greedy bf16 calls of up to 64 rows run as one persistent launch.  If its
    workgroups cannot all run (CUs held by other work), it gives up after 1 s
    and every token is -1; later persistent calls on the same workspace also
    return -1 tokens until ``read_device_error`` (which raises) clears the
    record.  ``check=True`` synchronises after the call and raises at once."""
    _check_weights(w1, w2)
    if base_logits.dim() != 3:
        raise ValueError("base_logits must be [B, M, V]")
    B, M, V = base_logits.shape
    if tuple(first_prev_token_ids.shape) != (B,):
        raise ValueError("first_prev_token_ids must be [B]")
    if w1.shape[0] != V:
        raise ValueError(f"weights have vocabulary {w1.shape[0]}, logits {V}")
    T = 0.0 if temperature is None else float(temperature)
    dev = base_logits.device
    _check_device(dev, workspace, first_prev_token_ids=first_prev_token_ids, w1=w1, w2=w2,
                  tokens_out=tokens_out, logits_out=logits_out if return_logits else None)
    if tokens_out is not None and (tuple(tokens_out.shape) != (B, M) or tokens_out.dtype != torch.int64
                                   or not tokens_out.is_contiguous()):
        raise ValueError(f"tokens_out must be a contiguous int64 tensor of shape {(B, M)}")
    if return_logits and logits_out is not None and (
            logits_out.shape != base_logits.shape or logits_out.dtype != base_logits.dtype
            or not logits_out.is_contiguous()):
        raise ValueError("logits_out must be a contiguous tensor shaped and typed like base_logits")
    if tokens_out is None:
        tokens_out = torch.empty((B, M), dtype=torch.int64, device=dev)
    if M == 0:
        return tokens_out, (base_logits if return_logits else None)
    base_c = base_logits.contiguous()
    first = first_prev_token_ids.to(torch.int64).contiguous()
    w1c, w2c = w1.contiguous(), w2.contiguous()
    corrected = None
    if return_logits:
        corrected = torch.empty_like(base_c) if logits_out is None else logits_out
    r = w1.shape[1]
    if workspace is None:
        workspace = Workspace(B, M, V, r, sample=True, device=dev)
    st = _lib.load().dspark_markov_sample_block(
        _ptr(base_c), _dtype_tag(base_c), _ptr(first), _ptr(w1c), _ptr(w2c), _dtype_tag(w1c),
        B, M, V, r, T, int(seed) & (2**64 - 1), int(position_offset), int(batch_offset),
        _ptr(tokens_out), _ptr(corrected), workspace.ptr, workspace.nbytes, _stream_handle(dev))
    _lib.check(st, "sample_block_tokens")
    if check:
        read_device_error(workspace)
    return tokens_out, corrected


def apply_block_logits_lm_head(hidden_states: torch.Tensor, lm_head_weight: torch.Tensor,
                               token_ids: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, *,
                               out: torch.Tensor | None = None,
                               workspace: Workspace | None = None) -> torch.Tensor:
    """The drafter's vocabulary head fused with the teacher-forced bias:
    hidden_states [..., M, d] and the head's Linear weight [V, d] give FP32
    base logits U (DeepseekV41DSparkModel.compute_logits), and the result is
    U + bias(token_ids[..., M]) as apply_block_logits would return it, in
    float32 [..., M, V], without U being materialised."""
    _check_weights(w1, w2)
    if hidden_states.dim() < 2:
        raise ValueError("hidden_states must be [..., M, d]")
    d = hidden_states.shape[-1]
    M = hidden_states.shape[-2]
    B = 1
    for x in hidden_states.shape[:-2]:
        B *= int(x)
    V, r = w1.shape
    if lm_head_weight.dim() != 2 or tuple(lm_head_weight.shape) != (V, d):
        raise ValueError(f"lm_head_weight must be [V, d] = {(V, d)}, got {tuple(lm_head_weight.shape)}")
    if tuple(token_ids.shape) != tuple(hidden_states.shape[:-1]):
        raise ValueError(f"token_ids {tuple(token_ids.shape)} must be hidden_states.shape[:-1]")
    dev = hidden_states.device
    _check_device(dev, workspace, lm_head_weight=lm_head_weight, token_ids=token_ids, w1=w1, w2=w2, out=out)
    shape = tuple(hidden_states.shape[:-1]) + (V,)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    elif tuple(out.shape) != shape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous float32 tensor of shape {shape}")
    if out.numel() == 0:
        return out
    h = hidden_states.contiguous()
    lm = lm_head_weight.contiguous()
    ids = token_ids.to(torch.int64).contiguous()
    w1c, w2c = w1.contiguous(), w2.contiguous()
    if workspace is None:
        workspace = Workspace(B, M, V, r, sample=False, device=dev)
    st = _lib.load().dspark_markov_apply_block_lm_head(
        _ptr(h), _dtype_tag(h), d, _ptr(lm), _dtype_tag(lm), _ptr(ids), _ptr(w1c), _ptr(w2c), _dtype_tag(w1c),
        B, M, V, r, _ptr(out), workspace.ptr, workspace.nbytes, _stream_handle(dev))
    _lib.check(st, "apply_block_logits_lm_head")
    return out


def _check_device(dev: torch.device, workspace: "Workspace | None" = None, **tensors):
    """Every tensor the kernels read or write must live on the GPU that holds
    the logits: a host or foreign-device pointer would reach the kernels."""
    if dev.type != "cuda":
        raise ValueError(f"the head runs on a GPU; the logits are on {dev}")
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the logits on {dev}")
    if workspace is not None and workspace.buffer.device != dev:
        raise ValueError(f"the workspace is on {workspace.buffer.device}, the logits on {dev}")


def _check_gate(hidden_states, gate_weight, gate_bias, lead, d_expected_rows, r, wdtype):
    if hidden_states is None:
        return 0
    if tuple(hidden_states.shape[:-1]) != tuple(lead):
        raise ValueError(f"hidden_states {tuple(hidden_states.shape)} must be {tuple(lead)} + (d,)")
    d = hidden_states.shape[-1]
    if gate_weight is None or gate_bias is None:
        raise ValueError("the gated head needs gate_weight [r, d + r] and gate_bias [r]")
    if tuple(gate_weight.shape) != (r, d + r) or tuple(gate_bias.shape) != (r,):
        raise ValueError(f"gate_weight must be [{r}, {d + r}] and gate_bias [{r}]")
    if gate_weight.dtype != wdtype or gate_bias.dtype != wdtype:
        raise TypeError("gate_weight and gate_bias must have the dtype of w1 and w2")
    return d


def apply_block_logits_gated(base_logits: torch.Tensor, token_ids: torch.Tensor, w1: torch.Tensor,
                             w2: torch.Tensor, gate_weight: torch.Tensor | None,
                             gate_bias: torch.Tensor | None, hidden_states: torch.Tensor | None, *,
                             out: torch.Tensor | None = None, return_latent: bool = False,
                             workspace: Workspace | None = None):
    """Teacher-forced corrected logits of the gated head (GatedMarkovHead):
    base[..., M, V] + W2 (sigmoid(gate_proj([h; W1[x]])) * W1[x]).

    ``hidden_states`` [..., M, d]; None is the pages' vanilla fallback.
    Returns the corrected logits, and with ``return_latent`` also the latent
    rows [..., M, r] the projection consumed."""
    _check_weights(w1, w2)
    if base_logits.dim() < 2:
        raise ValueError("base_logits must be [..., M, V]")
    V, M = base_logits.shape[-1], base_logits.shape[-2]
    B = 1
    for s_ in base_logits.shape[:-2]:
        B *= int(s_)
    if tuple(token_ids.shape) != tuple(base_logits.shape[:-1]):
        raise ValueError(f"token_ids {tuple(token_ids.shape)} must be base_logits.shape[:-1]")
    if w1.shape[0] != V:
        raise ValueError(f"weights have vocabulary {w1.shape[0]}, logits {V}")
    r = w1.shape[1]
    d = _check_gate(hidden_states, gate_weight, gate_bias, base_logits.shape[:-1], None, r, w1.dtype)
    dev = base_logits.device
    gated = hidden_states is not None
    _check_device(dev, workspace, token_ids=token_ids, w1=w1, w2=w2, hidden_states=hidden_states, out=out,
                  gate_weight=gate_weight if gated else None, gate_bias=gate_bias if gated else None)
    latent = torch.empty(tuple(base_logits.shape[:-1]) + (r,), dtype=w1.dtype, device=dev) if return_latent else None
    if base_logits.numel() == 0:
        res = base_logits if out is None else out
        return (res, latent) if return_latent else res
    base_c = base_logits.contiguous()
    ids = token_ids.to(torch.int64).contiguous()
    w1c, w2c = w1.contiguous(), w2.contiguous()
    hc = hidden_states.contiguous() if hidden_states is not None else None
    gwc = gate_weight.contiguous() if hc is not None else None
    gbc = gate_bias.contiguous() if hc is not None else None
    if out is None:
        out = torch.empty_like(base_c)
    elif out.shape != base_logits.shape or out.dtype != base_logits.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like base_logits")
    if workspace is None:
        workspace = Workspace(B, M, V, r, sample=False, device=dev, hidden=d)
    st = _lib.load().dspark_markov_apply_block_gated(
        _ptr(base_c), _dtype_tag(base_c), _ptr(ids), _ptr(hc), _dtype_tag(hc) if hc is not None else 0, d,
        _ptr(w1c), _ptr(w2c), _ptr(gwc), _ptr(gbc), _dtype_tag(w1c), B, M, V, r, _ptr(out), _ptr(latent),
        workspace.ptr, workspace.nbytes, _stream_handle(dev))
    _lib.check(st, "apply_block_logits_gated")
    return (out, latent) if return_latent else out


def sample_block_tokens_gated(base_logits: torch.Tensor, first_prev_token_ids: torch.Tensor,
                              w1: torch.Tensor, w2: torch.Tensor, gate_weight: torch.Tensor | None,
                              gate_bias: torch.Tensor | None, hidden_states: torch.Tensor | None,
                              temperature: float | None = 0.0, *, seed: int = 0, position_offset: int = 0,
                              batch_offset: int = 0, return_logits: bool = True,
                              return_latent: bool = False, workspace: Workspace | None = None):
    """Left-to-right sampling with the gated head; step k gates with
    hidden_states[:, k, :] ([B, M, d]; None: vanilla fallback) and the token
    drawn at k - 1.  Returns (tokens [B, M], corrected [B, M, V] or None) and,
    with ``return_latent``, the latent rows [B, M, r] as a third item."""
    _check_weights(w1, w2)
    if base_logits.dim() != 3:
        raise ValueError("base_logits must be [B, M, V]")
    B, M, V = base_logits.shape
    if tuple(first_prev_token_ids.shape) != (B,):
        raise ValueError("first_prev_token_ids must be [B]")
    if w1.shape[0] != V:
        raise ValueError(f"weights have vocabulary {w1.shape[0]}, logits {V}")
    r = w1.shape[1]
    d = _check_gate(hidden_states, gate_weight, gate_bias, (B, M), None, r, w1.dtype)
    T = 0.0 if temperature is None else float(temperature)
    dev = base_logits.device
    gated = hidden_states is not None
    _check_device(dev, workspace, first_prev_token_ids=first_prev_token_ids, w1=w1, w2=w2,
                  hidden_states=hidden_states, gate_weight=gate_weight if gated else None,
                  gate_bias=gate_bias if gated else None)
    tokens = torch.empty((B, M), dtype=torch.int64, device=dev)
    latent = torch.empty((B, M, r), dtype=w1.dtype, device=dev) if return_latent else None
    if M == 0 or B == 0:
        res = (tokens, base_logits if return_logits else None)
        return res + (latent,) if return_latent else res
    base_c = base_logits.contiguous()
    first = first_prev_token_ids.to(torch.int64).contiguous()
    w1c, w2c = w1.contiguous(), w2.contiguous()
    hc = hidden_states.contiguous() if hidden_states is not None else None
    gwc = gate_weight.contiguous() if hc is not None else None
    gbc = gate_bias.contiguous() if hc is not None else None
    corrected = torch.empty_like(base_c) if return_logits else None
    if workspace is None:
        workspace = Workspace(B, M, V, r, sample=True, device=dev, hidden=d)
    st = _lib.load().dspark_markov_sample_block_gated(
        _ptr(base_c), _dtype_tag(base_c), _ptr(first), _ptr(hc), _dtype_tag(hc) if hc is not None else 0, d,
        _ptr(w1c), _ptr(w2c), _ptr(gwc), _ptr(gbc), _dtype_tag(w1c), B, M, V, r, T, int(seed) & (2**64 - 1),
        int(position_offset), int(batch_offset), _ptr(tokens), _ptr(corrected), _ptr(latent),
        workspace.ptr, workspace.nbytes, _stream_handle(dev))
    _lib.check(st, "sample_block_tokens_gated")
    return (tokens, corrected, latent) if return_latent else (tokens, corrected)


def apply_block_logits_backward(grad_corrected: torch.Tensor, token_ids: torch.Tensor, w1: torch.Tensor,
                                w2: torch.Tensor, *, workspace: Workspace | None = None):
    """Gradients (grad_w1 [V, r], grad_w2 [V, r]) of the teacher-forced apply
    for the gradient of the corrected logits grad_corrected [..., M, V]; the
    base logits' gradient is grad_corrected itself."""
    _check_weights(w1, w2)
    if grad_corrected.dim() < 2:
        raise ValueError("grad_corrected must be [..., M, V]")
    V, M = grad_corrected.shape[-1], grad_corrected.shape[-2]
    B = 1
    for s_ in grad_corrected.shape[:-2]:
        B *= int(s_)
    if tuple(token_ids.shape) != tuple(grad_corrected.shape[:-1]):
        raise ValueError(f"token_ids {tuple(token_ids.shape)} must be grad_corrected.shape[:-1]")
    if w1.shape[0] != V:
        raise ValueError(f"weights have vocabulary {w1.shape[0]}, logits {V}")
    r = w1.shape[1]
    dev = grad_corrected.device
    _check_device(dev, workspace, token_ids=token_ids, w1=w1, w2=w2)
    g = grad_corrected.contiguous()
    ids = token_ids.to(torch.int64).contiguous()
    w1c, w2c = w1.contiguous(), w2.contiguous()
    gw1 = torch.empty_like(w1c)
    gw2 = torch.empty_like(w2c)
    if workspace is None:
        workspace = Workspace(B, M, V, r, sample=False, device=dev, backward=True)
    st = _lib.load().dspark_markov_apply_block_backward(
        _ptr(g), _dtype_tag(g), _ptr(ids), _ptr(w1c), _ptr(w2c), _dtype_tag(w1c), B, M, V, r, _ptr(gw1), _ptr(gw2),
        workspace.ptr, workspace.nbytes, _stream_handle(dev))
    _lib.check(st, "apply_block_logits_backward")
    return gw1, gw2
