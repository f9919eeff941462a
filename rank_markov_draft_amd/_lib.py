"""ctypes loader of libdspark_markov.so (the C ABI in include/dspark_markov.h).

torch is imported first: its bundled HIP runtime carries the same SONAME
(libamdhip64.so.7) that the library needs, so both share one runtime and
torch's device pointers and streams are valid handles for the library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import torch  # noqa: F401  (must load the HIP runtime before the library)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdspark_markov.so")
CSRC = os.path.join(_HERE, "csrc")

DSPARK_F32 = 0
DSPARK_BF16 = 1
DSPARK_ERR_DEVICE = 4

STATUS = {
    0: "DSPARK_OK",
    1: "DSPARK_ERR_INVALID_ARGUMENT",
    2: "DSPARK_ERR_UNSUPPORTED",
    3: "DSPARK_ERR_WORKSPACE_TOO_SMALL",
    4: "DSPARK_ERR_DEVICE",
}

# Every symbol include/dspark_markov.h declares.
EXPORTS = (
    "dspark_markov_workspace_bytes",
    "dspark_markov_workspace_init",
    "dspark_markov_apply_block",
    "dspark_markov_sample_block",
    "dspark_markov_sample_block_static",
    "dspark_markov_gated_workspace_bytes",
    "dspark_markov_apply_block_gated",
    "dspark_markov_sample_block_gated",
    "dspark_markov_backward_workspace_bytes",
    "dspark_markov_apply_block_backward",
    "dspark_markov_apply_block_lm_head",
    "dspark_markov_read_device_error",
    "dspark_status_string",
    "dspark_markov_last_error",
)

_lib = None


class DsparkError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        msg = f"{what}: {STATUS.get(status, status)}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)
        self.status = status


def build(force: bool = False) -> str:
    """Compile the HIP library for gfx950 in-tree (make in csrc/)."""
    cmd = ["make", "-C", CSRC] + (["-B"] if force else [])
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
    return LIB_PATH


def load():
    """Load the built library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (rank_markov_draft_amd._lib.build())")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, u64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_int
    L.dspark_markov_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    L.dspark_markov_workspace_bytes.restype = sz
    L.dspark_markov_workspace_init.argtypes = [p, sz, p]
    L.dspark_markov_workspace_init.restype = i32
    L.dspark_markov_apply_block.argtypes = [p, i32, p, p, p, i32, i64, i64, i64, i64, p, p, sz, p]
    L.dspark_markov_apply_block.restype = i32
    L.dspark_markov_sample_block.argtypes = [p, i32, p, p, p, i32, i64, i64, i64, i64,
                                             ctypes.c_double, u64, i64, i64, p, p, p, sz, p]
    L.dspark_markov_sample_block.restype = i32
    L.dspark_markov_sample_block_static.argtypes = [p, i32, p, p, p, i32, i64, i64, i64, i64,
                                                    ctypes.c_double, u64, i64, i64, p, p, p]
    L.dspark_markov_sample_block_static.restype = i32
    L.dspark_markov_gated_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
    L.dspark_markov_gated_workspace_bytes.restype = sz
    L.dspark_markov_apply_block_gated.argtypes = [p, i32, p, p, i32, i64, p, p, p, p, i32,
                                                  i64, i64, i64, i64, p, p, p, sz, p]
    L.dspark_markov_apply_block_gated.restype = i32
    L.dspark_markov_sample_block_gated.argtypes = [p, i32, p, p, i32, i64, p, p, p, p, i32,
                                                   i64, i64, i64, i64, ctypes.c_double, u64, i64, i64,
                                                   p, p, p, p, sz, p]
    L.dspark_markov_sample_block_gated.restype = i32
    L.dspark_markov_backward_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.dspark_markov_backward_workspace_bytes.restype = sz
    L.dspark_markov_apply_block_backward.argtypes = [p, i32, p, p, p, i32, i64, i64, i64, i64, p, p, p, sz, p]
    L.dspark_markov_apply_block_backward.restype = i32
    L.dspark_markov_apply_block_lm_head.argtypes = [p, i32, i64, p, i32, p, p, p, i32, i64, i64, i64, i64, p, p,
                                                    sz, p]
    L.dspark_markov_apply_block_lm_head.restype = i32
    L.dspark_markov_read_device_error.argtypes = [p, p, ctypes.POINTER(i64)]
    L.dspark_markov_read_device_error.restype = i32
    L.dspark_status_string.argtypes = [i32]
    L.dspark_status_string.restype = ctypes.c_char_p
    L.dspark_markov_last_error.argtypes = []
    L.dspark_markov_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


BANDWIDTH_LIB_PATH = os.path.join(_HERE, "libdspark_bandwidth.so")
_bw = None


def load_bandwidth():
    """The probes the benchmark times as HBM and matrix-core ceilings (not
    part of the head): dspark_bandwidth_copy, dspark_bandwidth_read_mix and
    dspark_bandwidth_mfma."""
    global _bw
    if _bw is None:
        if not os.path.exists(BANDWIDTH_LIB_PATH):
            raise ImportError(f"{BANDWIDTH_LIB_PATH} is missing: build it first")
        L = ctypes.CDLL(BANDWIDTH_LIB_PATH)
        p, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.dspark_bandwidth_copy.argtypes = [p, p, sz, p]
        L.dspark_bandwidth_copy.restype = i32
        L.dspark_bandwidth_read_mix.argtypes = [p, sz, p, sz, p]
        L.dspark_bandwidth_read_mix.restype = i32
        L.dspark_bandwidth_mfma.argtypes = [p, sz, i32, i32, i32, p]
        L.dspark_bandwidth_mfma.restype = i32
        _bw = L
    return _bw


def check(status: int, what: str):
    if status != 0:
        detail = load().dspark_markov_last_error().decode() if status == 4 else ""
        raise DsparkError(status, what, detail)
