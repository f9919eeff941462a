"""CPU checks of the C ABI: the library loads, exports every symbol that
include/dspark_markov.h declares, and rejects bad arguments on the host
(before any device work) with the documented status codes.  No call here
reaches a kernel."""
import ctypes
import os
import re

import pytest

from rank_markov_draft_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark_markov.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        _lib.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_strings(L):
    for code in range(5):
        assert L.dspark_status_string(code)
    assert L.dspark_status_string(0) == b"ok"
    assert L.dspark_markov_last_error() == b""


def _align256(x):
    return (x + 255) // 256 * 256


HEAD = 256                           # control block
CHAIN = 4096 + 16 * 8 * 64 * 64      # the persistent chain's area: counters, then keys for up to 16 steps
DATA = HEAD + CHAIN                  # where every call's own data starts


def test_workspace_bytes(L):
    """One layout for every call: the control block, the chain's area (only
    the chain writes there and leaves it zeroed), then the call's data:
    apply, a 16 KB store sink for lanes past the edges; sample, the step
    partials (B * ceil(V/128) keys), at least the sink's size."""
    assert L.dspark_markov_workspace_bytes(64, 5, 129280, 256, 0) == DATA + 16384
    assert L.dspark_markov_workspace_bytes(64, 5, 129280, 256, 1) == DATA + _align256(64 * 1010 * 8)
    assert L.dspark_markov_workspace_bytes(256, 8, 151936, 256, 1) == DATA + _align256(256 * 1187 * 8)
    assert DATA % 256 == 0
    # a sampling workspace holds at least the apply's sink, so it serves the apply too
    assert L.dspark_markov_workspace_bytes(2, 2, 64, 16, 1) == DATA + 16384


FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: every call below fails validation


@pytest.mark.parametrize("args,code", [
    # (logits dtype, weight dtype, B, M, V, r) -> status
    ((1, 1, 2, 3, 64, 0), 1),        # rank must be positive
    ((1, 1, 2, 3, 64, -4), 1),
    ((1, 1, -1, 3, 64, 16), 1),      # negative sizes
    ((1, 1, 2, -3, 64, 16), 1),
    ((1, 1, 2, 3, -64, 16), 1),
    ((7, 7, 2, 3, 64, 16), 1),       # unknown dtype tag
    ((1, 1, 2**40, 2**20, 2**20, 16), 1),   # element count overflows int64
])
def test_apply_argument_errors(L, args, code):
    ldt, wdt, B, M, V, r = args
    st = L.dspark_markov_apply_block(FAKE, ldt, FAKE, FAKE, FAKE, wdt, B, M, V, r, FAKE, FAKE, 1 << 20, None)
    assert st == code


def test_mixed_dtype_pairs_pass_validation(L):
    """Both mixed (logits, weights) pairs are accepted: with no workspace the
    call stops at the workspace check, before anything is enqueued."""
    for ldt, wdt in ((0, 1), (1, 0)):
        assert L.dspark_markov_apply_block(FAKE, ldt, FAKE, FAKE, FAKE, wdt, 2, 3, 64, 16, FAKE, None, 0, None) == 3
        assert L.dspark_markov_sample_block(FAKE, ldt, FAKE, FAKE, FAKE, wdt, 2, 3, 64, 16, 0.0, 0, 0, 0,
                                            FAKE, FAKE, None, 0, None) == 3


def test_apply_empty_is_ok_and_touches_nothing(L):
    assert L.dspark_markov_apply_block(FAKE, 1, FAKE, FAKE, FAKE, 1, 0, 5, 64, 16, FAKE, None, 0, None) == 0
    assert L.dspark_markov_apply_block(FAKE, 1, FAKE, FAKE, FAKE, 1, 3, 0, 64, 16, FAKE, None, 0, None) == 0
    assert L.dspark_markov_apply_block(None, 1, None, None, None, 1, 3, 5, 0, 16, None, None, 0, None) == 0


def test_apply_null_pointers_and_workspace(L):
    assert L.dspark_markov_apply_block(None, 1, FAKE, FAKE, FAKE, 1, 2, 3, 64, 16, FAKE, FAKE, 1 << 20, None) == 1
    assert L.dspark_markov_apply_block(FAKE, 1, None, FAKE, FAKE, 1, 2, 3, 64, 16, FAKE, FAKE, 1 << 20, None) == 1
    assert L.dspark_markov_apply_block(FAKE, 1, FAKE, FAKE, FAKE, 1, 2, 3, 64, 16, None, FAKE, 1 << 20, None) == 1
    assert L.dspark_markov_apply_block(FAKE, 1, FAKE, FAKE, FAKE, 1, 2, 3, 64, 16, FAKE, None, 1 << 20, None) == 3
    assert L.dspark_markov_apply_block(FAKE, 1, FAKE, FAKE, FAKE, 1, 2, 3, 64, 16, FAKE, FAKE, DATA + 16383, None) == 3


def test_apply_overlap_rejected(L):
    base = 0x200000
    out = ctypes.c_void_p(base + 64)          # partial overlap with base
    st = L.dspark_markov_apply_block(ctypes.c_void_p(base), 1, FAKE, ctypes.c_void_p(0x900000),
                                     ctypes.c_void_p(0xA00000), 1, 2, 3, 64, 16, out, FAKE, 1 << 20, None)
    assert st == 1


def _sample(L, T=0.0, B=2, M=3, V=64, r=16, first=FAKE, tok=FAKE, ws=FAKE, wsb=1 << 20):
    return L.dspark_markov_sample_block(FAKE, 1, first, FAKE, FAKE, 1, B, M, V, r, T, 0, 0, 0, tok, None,
                                        ws, wsb, None)


def test_sample_argument_errors(L):
    assert _sample(L, T=float("nan")) == 1
    assert _sample(L, r=0) == 1
    assert _sample(L, V=0) == 1          # nothing to draw from
    assert _sample(L, M=0) == 0          # empty work
    assert _sample(L, B=0) == 0
    assert _sample(L, first=None) == 1
    assert _sample(L, tok=None) == 1
    assert _sample(L, ws=None) == 3
    assert _sample(L, wsb=256) == 3


# ------------------------------------------------------------ gated head
def _gate_splits(rows, r, d):
    """Splits of the gate GEMM's inner dimension: at most 512 workgroups of
    64 x 64 output tiles, at most 32 splits, whole 32-column steps."""
    K = d + r
    tiles = ((rows + 63) // 64) * ((r + 63) // 64)
    steps = (K + 31) // 32
    want = max(min(512 // tiles, 32, steps), 1)
    kchunk = (steps + want - 1) // want * 32
    return (K + kchunk - 1) // kchunk


def test_gated_workspace_bytes(L):
    """Gated calls: the vanilla layout, then the latent rows of the call (4
    bytes per element at most) and, when the gate GEMM splits, its split
    sums."""
    for B, M, V, r, d, sample in ((64, 5, 129280, 256, 5120, 0), (64, 5, 129280, 256, 5120, 1),
                                  (512, 5, 129280, 512, 5120, 0), (3, 4, 700, 16, 40, 1), (2, 3, 64, 16, 0, 0)):
        rows = B if sample else B * M
        S = _gate_splits(rows, r, d) if d else 1
        want = (_align256(L.dspark_markov_workspace_bytes(B, M, V, r, sample)) + _align256(rows * r * 4)
                + (_align256(S * rows * r * 4) if S > 1 else 0))
        assert L.dspark_markov_gated_workspace_bytes(B, M, V, r, d, sample) == want
    assert _gate_splits(320, 256, 5120) == 24 and _gate_splits(64, 256, 5120) == 28
    assert _gate_splits(2560, 512, 5120) == 1


def _gapply(L, ldt=1, hdt=1, d=32, B=2, M=3, V=64, r=16, hidden=FAKE, gw=FAKE, gb=FAKE, out=FAKE,
            latent=None, ws=FAKE, wsb=1 << 24, base=FAKE):
    return L.dspark_markov_apply_block_gated(base, ldt, FAKE, hidden, hdt, d, FAKE, FAKE, gw, gb, 1,
                                             B, M, V, r, out, latent, ws, wsb, None)


def _gsample(L, T=0.0, hdt=1, d=32, B=2, M=3, V=64, r=16, hidden=FAKE, gw=FAKE, gb=FAKE, ws=FAKE, wsb=1 << 24):
    return L.dspark_markov_sample_block_gated(FAKE, 1, FAKE, hidden, hdt, d, FAKE, FAKE, gw, gb, 1,
                                              B, M, V, r, T, 0, 0, 0, FAKE, None, None, ws, wsb, None)


def test_gated_argument_errors(L):
    assert _gapply(L, d=0) == 1                 # a hidden state needs d > 0
    assert _gapply(L, d=-5) == 1
    assert _gapply(L, hdt=9) == 1               # unknown hidden dtype
    assert _gapply(L, gw=None) == 1             # gate weight and bias required
    assert _gapply(L, gb=None) == 1
    assert _gapply(L, r=0) == 1
    assert _gapply(L, out=None) == 1
    assert _gapply(L, ws=None) == 3
    assert _gapply(L, wsb=1024) == 3
    assert _gapply(L, B=0) == 0                 # empty work
    assert _gapply(L, V=0) == 0
    # vanilla fallback: the gate arguments are not looked at
    assert _gapply(L, hidden=None, d=0, gw=None, gb=None, ws=None) == 3
    assert _gsample(L, T=float("nan")) == 1
    assert _gsample(L, d=0) == 1
    assert _gsample(L, gw=None) == 1
    assert _gsample(L, V=0) == 1
    assert _gsample(L, M=0) == 0
    assert _gsample(L, ws=None) == 3
    assert _gsample(L, hidden=None, d=0, gw=None, gb=None, ws=None) == 3


def test_gated_overlaps_rejected(L):
    base = 0x200000
    # latent rows written over the base logits, or over the hidden states
    assert _gapply(L, base=ctypes.c_void_p(base), latent=ctypes.c_void_p(base + 32)) == 1
    assert _gapply(L, hidden=ctypes.c_void_p(0x400000), latent=ctypes.c_void_p(0x400000 + 64)) == 1
    # corrected logits over the gate weight
    assert _gapply(L, gw=ctypes.c_void_p(0x600000), out=ctypes.c_void_p(0x600000 + 16)) == 1


# ------------------------------------------------------------ backward
def test_backward_workspace_bytes(L):
    """The common head (control block and chain area), the de rows (4 bytes
    per element at most), the split sums of the de product over 1024-column
    slices of V, and two row links."""
    for B, M, V, r in ((64, 5, 129280, 256), (3, 4, 700, 16), (0, 5, 64, 8)):
        rows = B * M
        S = (V + 1023) // 1024
        want = DATA + _align256(rows * r * 4) + _align256(S * rows * r * 4) + _align256(rows * 8)
        assert L.dspark_markov_backward_workspace_bytes(B, M, V, r) == want


def _bwd(L, B=2, M=3, V=64, r=16, grad=FAKE, ids=FAKE, gw1=ctypes.c_void_p(0x700000),
         gw2=ctypes.c_void_p(0x800000), ws=FAKE, wsb=1 << 24, wdt=1):
    return L.dspark_markov_apply_block_backward(grad, 1, ids, ctypes.c_void_p(0x500000), ctypes.c_void_p(0x600000),
                                                wdt, B, M, V, r, gw1, gw2, ws, wsb, None)


def test_backward_argument_errors(L):
    assert _bwd(L, r=0) == 1
    assert _bwd(L, B=-1) == 1
    assert _bwd(L, grad=None) == 1
    assert _bwd(L, ids=None) == 1
    assert _bwd(L, gw1=None) == 1
    assert _bwd(L, gw2=None) == 1
    assert _bwd(L, ws=None) == 3
    assert _bwd(L, wsb=256) == 3
    assert _bwd(L, V=0) == 0                                    # no parameters: nothing to do
    assert _bwd(L, wdt=7) == 1
    # gradients over each other or over an input
    assert _bwd(L, gw1=ctypes.c_void_p(0x700000), gw2=ctypes.c_void_p(0x700000 + 64)) == 1
    assert _bwd(L, gw1=ctypes.c_void_p(0x500000 + 16)) == 1    # over W1


def test_bandwidth_probe_argument_errors():
    """The bandwidth and matrix-core probes (a separate library, not the
    head's ABI) take 16-byte aligned, non-overlapping buffers and whole
    16-byte pieces; zero bytes is a no-op.  Every call here is rejected
    before any launch or device query."""
    from rank_markov_draft_amd import _lib
    bw = _lib.load_bandwidth()
    a, b = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    bad = 1
    assert bw.dspark_bandwidth_copy(b, a, 0, None) == 0
    assert bw.dspark_bandwidth_copy(None, a, 4096, None) == bad
    assert bw.dspark_bandwidth_copy(b, None, 4096, None) == bad
    assert bw.dspark_bandwidth_copy(ctypes.c_void_p(0x200008), a, 4096, None) == bad
    assert bw.dspark_bandwidth_copy(b, ctypes.c_void_p(0x100004), 4096, None) == bad
    assert bw.dspark_bandwidth_copy(b, a, 4100, None) == bad
    assert bw.dspark_bandwidth_copy(ctypes.c_void_p(0x100800), a, 4096, None) == bad   # overlap
    assert bw.dspark_bandwidth_read_mix(b, 0, a, 0, None) == 0
    assert bw.dspark_bandwidth_read_mix(b, 4096, a, 2048, None) == bad                   # reads fewer than writes
    assert bw.dspark_bandwidth_read_mix(b, 4096, a, 4096 * 5, None) == bad               # more than four passes
    assert bw.dspark_bandwidth_read_mix(b, 4096, a, 4100, None) == bad
    assert bw.dspark_bandwidth_read_mix(ctypes.c_void_p(0x100800), 4096, a, 8192, None) == bad
    # the matrix-core probe: one of two product forms, 4, 8 or 16 waves per
    # CU, at least one round, an aligned output buffer
    assert bw.dspark_bandwidth_mfma(None, 1 << 20, 0, 16, 10, None) == bad
    assert bw.dspark_bandwidth_mfma(ctypes.c_void_p(0x100004), 1 << 20, 0, 16, 10, None) == bad
    assert bw.dspark_bandwidth_mfma(a, 1 << 20, 2, 16, 10, None) == bad
    assert bw.dspark_bandwidth_mfma(a, 1 << 20, 1, 12, 10, None) == bad
    assert bw.dspark_bandwidth_mfma(a, 1 << 20, 0, 16, 0, None) == bad


def test_product_abi_has_no_benchmark_utility(L):
    assert not hasattr(L, "dspark_markov_stream_copy")


def test_static_scratch_entry_point_rejects_oversize_on_the_host(L):
    """dspark_markov_sample_block_static refuses sizes whose workspace exceeds
    its 4 MiB static scratch before touching the device."""
    f = ctypes.c_void_p(0x1000)
    st = L.dspark_markov_sample_block_static(f, 1, f, f, f, 1, 4096, 5, 151936, 256, 0.0, 0, 0, 0, f, None, None)
    assert st == 3
    assert b"static scratch" in L.dspark_markov_last_error()
    # no work at all is a successful no-op, as for the workspace entry point
    assert L.dspark_markov_sample_block_static(f, 1, f, f, f, 1, 0, 5, 151936, 256, 0.0, 0, 0, 0, f, None, None) == 0


def test_rank_above_the_limit_is_unsupported(L):
    """Ranks above 16384 return DSPARK_ERR_UNSUPPORTED, on the host, before
    anything is enqueued (distinct fake buffers pass the overlap checks)."""
    mb = 1 << 24
    base, ids, w1, w2, out, ws = (ctypes.c_void_p(mb * (i + 1)) for i in range(6))
    for ldt, wdt in ((0, 0), (1, 0), (1, 1)):
        assert L.dspark_markov_apply_block(base, ldt, ids, w1, w2, wdt, 2, 3, 64, 16385, out, ws, 1 << 20, None) == 2
        assert L.dspark_markov_sample_block(base, ldt, ids, w1, w2, wdt, 2, 3, 64, 16385, 0.0, 0, 0, 0,
                                            ctypes.c_void_p(mb * 8), None, ws, 1 << 20, None) == 2
