"""ctypes wrapper around the CPU oracle (liboracle_dspark.so).

TEST INFRASTRUCTURE ONLY.  The test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module; the product path
(``rank_markov_draft_amd``) never does, and nothing here touches a GPU.

The oracle follows the DSpark pages step by step (see ``dspark_oracle.c``):
the third-party ``markov_head.py`` page (module docstring, ``_sample_tokens``,
``VanillaMarkov.apply_block_logits`` / ``sample_block_tokens``) and the NeMo
AutoModel ``speculative/dspark/markov_head`` API page; the gated head
follows ``GatedMarkovHead`` on both pages.

Arrays are numpy: float32 for fp32 data, uint16 bit patterns for bfloat16,
int64 for token ids.  W1 and W2w are both [V, r] (Embedding weight and
Linear(r, V) weight).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32 = 0
BF16 = 1
OK = 0
INVALID = 1
UNSUPPORTED = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_dspark.so")
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


def build(force: bool = False) -> str:
    """Compile the oracle with its Makefile (gcc, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["make", "-C", _HERE] + (["-B"] if force else [])
        subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        L.dspark_oracle_apply_block.argtypes = [_p, _int, _p, _p, _p, _int, _i64, _i64, _i64, _i64, _p, _int]
        L.dspark_oracle_apply_block.restype = _int
        L.dspark_oracle_sample_block.argtypes = [
            _p, _int, _p, _p, _p, _int, _i64, _i64, _i64, _i64,
            ctypes.c_double, ctypes.c_uint64, _i64, _i64, _p, _p, _int]
        L.dspark_oracle_sample_block.restype = _int
        L.dspark_oracle_select_token.argtypes = [
            _p, _int, _i64, ctypes.c_double, ctypes.c_uint64, _i64, _i64, _p, _p, _p]
        L.dspark_oracle_select_token.restype = _int
        L.dspark_oracle_apply_block_lm_head.argtypes = [_p, _int, _p, _int, _i64, _p, _p, _p, _int, _i64, _i64,
                                                        _i64, _p, _p, _int]
        L.dspark_oracle_apply_block_lm_head.restype = _int
        L.dspark_oracle_lm_head_bounds.argtypes = [_p, _int, _p, _int, _i64, _p, _p, _p, _int, _i64, _i64, _i64,
                                                   _p, _p, _p, _p, _p]
        L.dspark_oracle_lm_head_bounds.restype = _int
        L.dspark_oracle_select_tokens.argtypes = [
            _p, _int, _i64, _i64, ctypes.c_double, ctypes.c_uint64, _p, _p, _p, _p, _p, _int]
        L.dspark_oracle_select_tokens.restype = _int
        L.dspark_oracle_logit_bounds.argtypes = [
            _p, _int, _p, _p, _p, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p]
        L.dspark_oracle_logit_bounds.restype = _int
        L.dspark_oracle_gated_latent.argtypes = [
            _p, _int, _i64, _p, _p, _p, _p, _int, _i64, _i64, _i64, _p, _p, _p, _int]
        L.dspark_oracle_gated_latent.restype = _int
        L.dspark_oracle_apply_rows.argtypes = [_p, _int, _p, _p, _int, _i64, _i64, _i64, _p, _int]
        L.dspark_oracle_apply_rows.restype = _int
        L.dspark_oracle_logit_bounds_rows.argtypes = [
            _p, _int, _p, _p, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p]
        L.dspark_oracle_logit_bounds_rows.restype = _int
        L.dspark_oracle_apply_block_gated.argtypes = [
            _p, _int, _p, _p, _int, _i64, _p, _p, _p, _p, _int, _i64, _i64, _i64, _i64, _p, _p, _int]
        L.dspark_oracle_apply_block_gated.restype = _int
        L.dspark_oracle_sample_block_gated.argtypes = [
            _p, _int, _p, _p, _int, _i64, _p, _p, _p, _p, _int, _i64, _i64, _i64, _i64,
            ctypes.c_double, ctypes.c_uint64, _i64, _i64, _p, _p, _p, _int]
        L.dspark_oracle_sample_block_gated.restype = _int
        L.dspark_oracle_apply_block_backward.argtypes = [_p, _int, _p, _p, _p, _int, _i64, _i64, _i64, _p, _p, _int]
        L.dspark_oracle_apply_block_backward.restype = _int
        L.dspark_oracle_backward_bounds.argtypes = [
            _p, _int, _p, _p, _p, _int, _i64, _i64, _i64, _int, _i64, _p, _p, _p, _p, _p]
        L.dspark_oracle_backward_bounds.restype = _int
        L.dspark_oracle_philox4x32_10.argtypes = [_p, _p, _p]
        L.dspark_oracle_philox4x32_10.restype = None
        L.dspark_oracle_gumbel2.argtypes = [ctypes.c_uint64, _i64, _i64, _i64]
        L.dspark_oracle_gumbel2.restype = ctypes.c_float
        L.dspark_oracle_round_bf16.argtypes = [ctypes.c_float]
        L.dspark_oracle_round_bf16.restype = ctypes.c_uint16
        L.dspark_oracle_kappa.argtypes = [ctypes.c_double]
        L.dspark_oracle_kappa.restype = ctypes.c_float
        _lib = L
    return _lib


class OracleError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"oracle returned status {status}")
        self.status = status


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_tag(a) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported array dtype {a.dtype}")


def _check(status: int):
    if status != OK:
        raise OracleError(status)


def apply_block(base, token_ids, w1, w2, n_threads: int = 0, check: bool = True):
    """Teacher-forced corrected logits for base [..., M, V], token_ids [..., M]."""
    base = np.ascontiguousarray(base)
    token_ids = np.ascontiguousarray(token_ids, dtype=np.int64)
    w1 = np.ascontiguousarray(w1)
    w2 = np.ascontiguousarray(w2)
    V = base.shape[-1]
    M = base.shape[-2] if base.ndim >= 2 else 0
    B = int(np.prod(base.shape[:-2])) if base.ndim >= 2 else 0
    r = w1.shape[1]
    out = base.copy()
    st = lib().dspark_oracle_apply_block(
        _ptr(base), _dtype_tag(base), _ptr(token_ids), _ptr(w1), _ptr(w2), _dtype_tag(w1),
        B, M, V, r, _ptr(out), n_threads)
    if check:
        _check(st)
        return out
    return st, out


def sample_block(base, first_prev, w1, w2, temperature=0.0, seed=0, position_offset=0,
                 batch_offset=0, return_logits=True, n_threads: int = 0, check: bool = True):
    """Left-to-right sampling over base [B, M, V]; returns (tokens [B, M], corrected|None)."""
    base = np.ascontiguousarray(base)
    first_prev = np.ascontiguousarray(first_prev, dtype=np.int64)
    w1 = np.ascontiguousarray(w1)
    w2 = np.ascontiguousarray(w2)
    B, M, V = base.shape
    r = w1.shape[1]
    tokens = np.zeros((B, M), dtype=np.int64)
    corrected = base.copy() if return_logits else None
    st = lib().dspark_oracle_sample_block(
        _ptr(base), _dtype_tag(base), _ptr(first_prev), _ptr(w1), _ptr(w2), _dtype_tag(w1),
        B, M, V, r, float(temperature), int(seed) & (2**64 - 1), int(position_offset),
        int(batch_offset), _ptr(tokens), _ptr(corrected), n_threads)
    if check:
        _check(st)
        return tokens, corrected
    return st, tokens, corrected


def select_token(row, temperature=0.0, seed=0, b_abs=0, k_abs=0):
    """Token drawn from one corrected row; returns (token, best, second, runner_up)."""
    row = np.ascontiguousarray(row)
    tok = np.zeros(1, dtype=np.int64)
    sc = np.zeros(2, dtype=np.float32)
    ru = np.zeros(1, dtype=np.int64)
    _check(lib().dspark_oracle_select_token(
        _ptr(row), _dtype_tag(row), row.shape[-1], float(temperature),
        int(seed) & (2**64 - 1), int(b_abs), int(k_abs), _ptr(tok), _ptr(sc), _ptr(ru)))
    return int(tok[0]), float(sc[0]), float(sc[1]), int(ru[0])


def select_tokens(rows, temperature=0.0, seed=0, b_abs=None, k_abs=None, n_threads: int = 0):
    """select_token over rows [n, V] at once; returns (tokens [n], scores [n, 2]
    (winner, runner-up), runner_up [n])."""
    rows = np.ascontiguousarray(rows)
    V = rows.shape[-1]
    rows = rows.reshape(-1, V)
    n = rows.shape[0]
    b_abs = np.ascontiguousarray(np.zeros(n) if b_abs is None else b_abs, dtype=np.int64)
    k_abs = np.ascontiguousarray(np.zeros(n) if k_abs is None else k_abs, dtype=np.int64)
    tok = np.zeros(n, dtype=np.int64)
    sc = np.zeros((n, 2), dtype=np.float32)
    ru = np.zeros(n, dtype=np.int64)
    _check(lib().dspark_oracle_select_tokens(
        _ptr(rows), _dtype_tag(rows), n, V, float(temperature), int(seed) & (2**64 - 1),
        _ptr(b_abs), _ptr(k_abs), _ptr(tok), _ptr(sc), _ptr(ru), n_threads))
    return tok, sc, ru


def logit_bounds(base, token_ids, w1, w2, rows, cols):
    """Admissible [lo, hi] (and the oracle's own value) for corrected elements
    (rows[i], cols[i]) of the flattened [B*M, V] layout."""
    base = np.ascontiguousarray(base)
    token_ids = np.ascontiguousarray(token_ids, dtype=np.int64).reshape(-1)
    w1 = np.ascontiguousarray(w1)
    w2 = np.ascontiguousarray(w2)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    n = rows.shape[0]
    lo = np.zeros(n, dtype=np.float32)
    mid = np.zeros(n, dtype=np.float32)
    hi = np.zeros(n, dtype=np.float32)
    _check(lib().dspark_oracle_logit_bounds(
        _ptr(base), _dtype_tag(base), _ptr(token_ids), _ptr(w1), _ptr(w2), _dtype_tag(w1),
        base.shape[-1], w1.shape[1], n, _ptr(rows), _ptr(cols), _ptr(lo), _ptr(mid), _ptr(hi)))
    return lo, mid, hi


def _c(a, dtype=None):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def gated_latent(hidden, token_ids, w1, gate_w, gate_b, bounds: bool = False, n_threads: int = 0):
    """Latent rows sigmoid(gate_proj([h; W1[x]])) * W1[x] of the gated head for
    hidden [..., d] and token_ids [...] (flattened); returns latent [rows, r]
    (weight dtype), plus (lo, hi) float32 [rows, r] when bounds is set."""
    w1, gate_w, gate_b = _c(w1), _c(gate_w), _c(gate_b)
    d = hidden.shape[-1]
    hidden = _c(hidden).reshape(-1, d)
    ids = _c(token_ids, np.int64).reshape(-1)
    rows, r = ids.shape[0], w1.shape[1]
    lat = np.zeros((rows, r), dtype=w1.dtype)
    lo = np.zeros((rows, r), dtype=np.float32) if bounds else None
    hi = np.zeros((rows, r), dtype=np.float32) if bounds else None
    _check(lib().dspark_oracle_gated_latent(
        _ptr(hidden), _dtype_tag(hidden), d, _ptr(ids), _ptr(w1), _ptr(gate_w), _ptr(gate_b),
        _dtype_tag(w1), rows, w1.shape[0], r, _ptr(lat), _ptr(lo), _ptr(hi), n_threads))
    return (lat, lo, hi) if bounds else lat


def apply_rows(base, latent, w2, n_threads: int = 0):
    """Corrected rows: base [..., V] row n biased by project_bias(latent[n])."""
    base, latent, w2 = _c(base), _c(latent), _c(w2)
    V = base.shape[-1]
    rows = base.size // V if V else 0
    out = base.copy()
    _check(lib().dspark_oracle_apply_rows(
        _ptr(base), _dtype_tag(base), _ptr(latent), _ptr(w2), _dtype_tag(w2), rows, V,
        w2.shape[1], _ptr(out), n_threads))
    return out


def logit_bounds_rows(base, latent, w2, rows, cols):
    """logit_bounds with every row biased by its own latent row."""
    base, latent, w2 = _c(base), _c(latent), _c(w2)
    rows, cols = _c(rows, np.int64), _c(cols, np.int64)
    n = rows.shape[0]
    lo, mid, hi = (np.zeros(n, dtype=np.float32) for _ in range(3))
    _check(lib().dspark_oracle_logit_bounds_rows(
        _ptr(base), _dtype_tag(base), _ptr(latent), _ptr(w2), _dtype_tag(w2), base.shape[-1],
        w2.shape[1], n, _ptr(rows), _ptr(cols), _ptr(lo), _ptr(mid), _ptr(hi)))
    return lo, mid, hi


def apply_block_gated(base, token_ids, hidden, w1, w2, gate_w, gate_b, n_threads: int = 0,
                      check: bool = True):
    """Gated teacher-forced corrected logits; returns (corrected, latent [B, M, r]).
    hidden None is the vanilla fallback."""
    base, w1, w2 = _c(base), _c(w1), _c(w2)
    ids = _c(token_ids, np.int64)
    hidden, gate_w, gate_b = _c(hidden), _c(gate_w), _c(gate_b)
    V, M = base.shape[-1], base.shape[-2]
    B = int(np.prod(base.shape[:-2]))
    r = w1.shape[1]
    d = hidden.shape[-1] if hidden is not None else 0
    out = base.copy()
    lat = np.zeros(base.shape[:-1] + (r,), dtype=w1.dtype)
    st = lib().dspark_oracle_apply_block_gated(
        _ptr(base), _dtype_tag(base), _ptr(ids), _ptr(hidden),
        _dtype_tag(hidden) if hidden is not None else 0, d, _ptr(w1), _ptr(w2), _ptr(gate_w),
        _ptr(gate_b), _dtype_tag(w1), B, M, V, r, _ptr(out), _ptr(lat), n_threads)
    if check:
        _check(st)
        return out, lat
    return st, out, lat


def sample_block_gated(base, first_prev, hidden, w1, w2, gate_w, gate_b, temperature=0.0, seed=0,
                       position_offset=0, batch_offset=0, n_threads: int = 0):
    """Gated left-to-right sampling; returns (tokens [B, M], corrected, latent [B, M, r])."""
    base, w1, w2 = _c(base), _c(w1), _c(w2)
    first = _c(first_prev, np.int64)
    hidden, gate_w, gate_b = _c(hidden), _c(gate_w), _c(gate_b)
    B, M, V = base.shape
    r = w1.shape[1]
    d = hidden.shape[-1] if hidden is not None else 0
    tokens = np.zeros((B, M), dtype=np.int64)
    corrected = base.copy()
    lat = np.zeros((B, M, r), dtype=w1.dtype)
    _check(lib().dspark_oracle_sample_block_gated(
        _ptr(base), _dtype_tag(base), _ptr(first), _ptr(hidden),
        _dtype_tag(hidden) if hidden is not None else 0, d, _ptr(w1), _ptr(w2), _ptr(gate_w),
        _ptr(gate_b), _dtype_tag(w1), B, M, V, r, float(temperature), int(seed) & (2**64 - 1),
        int(position_offset), int(batch_offset), _ptr(tokens), _ptr(corrected), _ptr(lat),
        n_threads))
    return tokens, corrected, lat


def apply_block_backward(grad, token_ids, w1, w2, n_threads: int = 0):
    """Gradients (dW1 [V, r], dW2w [V, r]) of the teacher-forced apply for the
    upstream gradient grad [..., V] of the corrected logits."""
    grad, w1, w2 = _c(grad), _c(w1), _c(w2)
    ids = _c(token_ids, np.int64).reshape(-1)
    V, r = w1.shape
    dw1 = np.zeros_like(w1)
    dw2 = np.zeros_like(w2)
    _check(lib().dspark_oracle_apply_block_backward(
        _ptr(grad), _dtype_tag(grad), _ptr(ids), _ptr(w1), _ptr(w2), _dtype_tag(w1), ids.shape[0], V, r,
        _ptr(dw1), _ptr(dw2), n_threads))
    return dw1, dw2


def backward_bounds(grad, token_ids, w1, w2, kind, which, cols):
    """Admissible [lo, hi] and the oracle's value for backward outputs:
    kind "dw2" (which = vocabulary rows v) or "dw1" (which = token ids x)."""
    grad, w1, w2 = _c(grad), _c(w1), _c(w2)
    ids = _c(token_ids, np.int64).reshape(-1)
    which, cols = _c(which, np.int64), _c(cols, np.int64)
    n = which.shape[0]
    lo, mid, hi = (np.zeros(n, dtype=np.float32) for _ in range(3))
    V, r = w1.shape
    _check(lib().dspark_oracle_backward_bounds(
        _ptr(grad), _dtype_tag(grad), _ptr(ids), _ptr(w1), _ptr(w2), _dtype_tag(w1), ids.shape[0], V, r,
        2 if kind == "dw2" else 1, n, _ptr(which), _ptr(cols), _ptr(lo), _ptr(mid), _ptr(hi)))
    return lo, mid, hi


def apply_block_lm_head(hidden, lm_head, token_ids, w1, w2, n_threads: int = 0, return_base: bool = False):
    """Fused LM head and bias: hidden [..., d] -> corrected fp32 [..., V] with
    U = hidden . lm_head^T in FP32 (lm_head [V, d]) plus the bias of token_ids
    [...]; with return_base also U."""
    hidden, lm_head, w1, w2 = _c(hidden), _c(lm_head), _c(w1), _c(w2)
    ids = _c(token_ids, np.int64)
    d = hidden.shape[-1]
    V, r = w1.shape
    rows = ids.size
    out = np.zeros(ids.shape + (V,), dtype=np.float32)
    base = np.zeros_like(out) if return_base else None
    _check(lib().dspark_oracle_apply_block_lm_head(
        _ptr(hidden), _dtype_tag(hidden), _ptr(lm_head), _dtype_tag(lm_head), d, _ptr(ids), _ptr(w1), _ptr(w2),
        _dtype_tag(w1), rows, V, r, _ptr(out), _ptr(base), n_threads))
    return (out, base) if return_base else out


def lm_head_bounds(hidden, lm_head, token_ids, w1, w2, rows, cols):
    """Admissible [lo, hi] and the oracle's value for fused elements (rows[i], cols[i])."""
    hidden, lm_head, w1, w2 = _c(hidden), _c(lm_head), _c(w1), _c(w2)
    ids = _c(token_ids, np.int64).reshape(-1)
    rows, cols = _c(rows, np.int64), _c(cols, np.int64)
    n = rows.shape[0]
    lo, mid, hi = (np.zeros(n, dtype=np.float32) for _ in range(3))
    d = hidden.shape[-1]
    V, r = w1.shape
    _check(lib().dspark_oracle_lm_head_bounds(
        _ptr(hidden), _dtype_tag(hidden), _ptr(lm_head), _dtype_tag(lm_head), d, _ptr(ids), _ptr(w1), _ptr(w2),
        _dtype_tag(w1), V, r, n, _ptr(rows), _ptr(cols), _ptr(lo), _ptr(mid), _ptr(hi)))
    return lo, mid, hi


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().dspark_oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def gumbel2(seed, b_abs, k_abs, v) -> float:
    return float(lib().dspark_oracle_gumbel2(int(seed) & (2**64 - 1), int(b_abs), int(k_abs), int(v)))


def round_bf16(x: float) -> int:
    return int(lib().dspark_oracle_round_bf16(float(x)))


def kappa(temperature: float) -> float:
    return float(lib().dspark_oracle_kappa(float(temperature)))
