"""Seeded synthetic inputs for the DSpark Markov head.

This module draws random inputs and holds none of the head's arithmetic.
It is shared by the GPU tests, the oracle tests and the benchmark so that
both sides read identical bytes.

Shapes follow the DSpark pages: vocabulary 129280, Markov rank 256 and
block size 5 for DeepSeek-V4.1 (NeMo AutoModel ``deepseek_v41/config`` page,
``DeepseekV41TextConfig``: ``vocab_size``, ``dspark_markov_rank``,
``dspark_block_size``; ``initializer_range=0.02`` matches the N(0, 0.02^2)
weights), many anchors per sequence (``models/deepseek_v41/dspark`` page,
module summary), and an 8-position block at vocabulary 151936 for the
second drafter (third-party ``markov_head.py`` page, suffix-decay note).
The pages name no dataset; real backbone logits and trained weights are
replaced by normal draws.

Draw order for every workload: base logits, W1, W2w, then the token ids,
from ``numpy.random.default_rng(seed)``; float32 draws are rounded to
bfloat16 by torch's own conversion.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

F32 = 0
BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int                 # batch rows (B * num_anchors for the training layout)
    M: int                 # block size / proposal length
    V: int                 # vocabulary
    r: int                 # Markov rank
    dtype: int             # F32 or BF16, both logits and weights
    base_sigma: float
    w_sigma: float
    seed: int
    mode: str              # "apply", "greedy", "temperature", "apply+greedy", "backward"
    temperature: float = 0.0
    gumbel_seed: int = 0
    ids: str = "uniform"   # "uniform" or "zipf1.1"
    boost: float = 0.0     # added at one random position per (b, k) row
    return_logits: bool = True
    logits_dtype: int = -1  # the logits' dtype when it differs from the weights' (-1: same)
    hidden: int = 0         # gated head: backbone hidden size d (0: vanilla head)
    lm_head: int = 0        # fused vocabulary head: hidden size d (0: base logits given)

    @property
    def ldtype(self) -> int:
        return self.dtype if self.logits_dtype < 0 else self.logits_dtype

    @property
    def rows(self) -> int:
        return self.B * self.M

    @property
    def elems(self) -> int:
        return self.B * self.M * self.V


WORKLOADS = {
    # Tiny fp32 check: apply plus greedy left-to-right sampling.
    "tiny_fp32": Workload("tiny_fp32", B=2, M=5, V=1024, r=16, dtype=F32, base_sigma=1.0,
                          w_sigma=0.02, seed=0, mode="apply+greedy"),
    # Teacher-forced training forward: 4 sequences x 16 anchors, block 5.
    "teacher_forced_320": Workload("teacher_forced_320", B=64, M=5, V=129280, r=256, dtype=BF16,
                                   base_sigma=2.0, w_sigma=0.02, seed=2, mode="apply"),
    # Greedy left-to-right draft, batch 64, block 5, corrected logits returned.
    "greedy_draft_64x5": Workload("greedy_draft_64x5", B=64, M=5, V=129280, r=256, dtype=BF16,
                                  base_sigma=2.0, w_sigma=0.02, seed=3, mode="greedy",
                                  boost=6.0),
    # Temperature draft at the 151936 vocabulary, batch 256, block 8, tokens only.
    "temperature_draft_256x8": Workload("temperature_draft_256x8", B=256, M=8, V=151936, r=256,
                                        dtype=BF16, base_sigma=2.0, w_sigma=0.02, seed=4,
                                        mode="temperature", temperature=0.7, gumbel_seed=1234,
                                        return_logits=False),
    # The 320-row teacher-forced batch with fp32 base logits (an fp32 LM head
    # output) and bf16 weights.
    "teacher_forced_320_f32logits": Workload("teacher_forced_320_f32logits", B=64, M=5, V=129280,
                                             r=256, dtype=BF16, base_sigma=2.0, w_sigma=0.02, seed=2,
                                             mode="apply", logits_dtype=F32),
    # The greedy and temperature drafts on fp32 base logits (the fp32 LM head
    # output of DeepSeek-V4.1's compute_logits) with bf16 weights.
    "greedy_draft_64x5_f32logits": Workload("greedy_draft_64x5_f32logits", B=64, M=5, V=129280, r=256, dtype=BF16,
                                            base_sigma=2.0, w_sigma=0.02, seed=3, mode="greedy", boost=6.0,
                                            logits_dtype=F32),
    "temperature_draft_256x8_f32logits": Workload("temperature_draft_256x8_f32logits", B=256, M=8, V=151936,
                                                  r=256, dtype=BF16, base_sigma=2.0, w_sigma=0.02, seed=4,
                                                  mode="temperature", temperature=0.7, gumbel_seed=1234,
                                                  return_logits=False, logits_dtype=F32),
    # The greedy draft with fp32 logits and fp32 weights (the row-tile FMA kernel).
    "greedy_draft_64x5_fp32": Workload("greedy_draft_64x5_fp32", B=64, M=5, V=129280, r=256, dtype=F32,
                                       base_sigma=2.0, w_sigma=0.02, seed=3, mode="greedy", boost=6.0),
    # Gated head (GatedMarkovHead) at the DeepSeek-V4.1 hidden size 5120:
    # teacher-forced 320 rows, and a greedy draft of batch 64, block 5.
    "gated_teacher_forced_320": Workload("gated_teacher_forced_320", B=64, M=5, V=129280, r=256,
                                         dtype=BF16, base_sigma=2.0, w_sigma=0.02, seed=6,
                                         mode="apply", hidden=5120),
    "gated_greedy_draft_64x5": Workload("gated_greedy_draft_64x5", B=64, M=5, V=129280, r=256,
                                        dtype=BF16, base_sigma=2.0, w_sigma=0.02, seed=7,
                                        mode="greedy", boost=6.0, hidden=5120),
    # Backward of the 320-row teacher-forced batch (training): a gradient of
    # the corrected logits per element.
    "teacher_forced_320_backward": Workload("teacher_forced_320_backward", B=64, M=5, V=129280, r=256,
                                            dtype=BF16, base_sigma=2.0, w_sigma=0.02, seed=8,
                                            mode="backward"),
    # The drafter's FP32 vocabulary head fused with the teacher-forced bias:
    # the 320-row batch from hidden states of size 5120 (DeepSeek-V4.1).
    "lm_head_teacher_forced_320": Workload("lm_head_teacher_forced_320", B=64, M=5, V=129280, r=256, dtype=BF16,
                                           base_sigma=2.0, w_sigma=0.02, seed=9, mode="apply", lm_head=5120),
    # Large teacher-forced batch: 8 sequences x 64 anchors, rank 512, Zipf ids.
    "teacher_forced_2560_zipf": Workload("teacher_forced_2560_zipf", B=512, M=5, V=129280, r=512,
                                         dtype=BF16, base_sigma=2.0, w_sigma=0.02, seed=5,
                                         mode="apply", ids="zipf1.1"),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), via torch's conversion."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def zipf_ids(rng: np.random.Generator, n: int, V: int, s: float) -> np.ndarray:
    """n draws from P(i) proportional to (i+1)^-s on [0, V), by inverse CDF."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    ids = np.searchsorted(cdf, rng.random(n), side="right")
    return np.minimum(ids, V - 1).astype(np.int64)


def make_inputs(w: Workload, *, B: int | None = None, M: int | None = None,
                V: int | None = None, r: int | None = None, seed: int | None = None,
                hidden: int | None = None, lm_head: int | None = None):
    """Draw inputs for workload ``w`` (optionally at other sizes).

    Returns a dict of numpy arrays: base [B, M, V], w1 [V, r], w2 [V, r]
    (float32 or uint16 bf16 bits), token_ids [B, M] and first_prev [B] (int64).
    With a hidden size d (gated head) it also holds hidden [B, M, d] ~ N(0, 1)
    (a normalised backbone state) and the gate_proj weight [r, d + r] and
    bias [r], both U(-1/sqrt(d + r), 1/sqrt(d + r)) (nn.Linear's default
    initialisation), drawn after everything else in that order, in the
    weight dtype.  With a fused vocabulary head (lm_head = d) it holds
    lm_hidden [B, M, d] ~ N(0, 1) and lm_head [V, d] ~ N(0, 0.02^2), bf16,
    drawn last.
    """
    B = w.B if B is None else B
    M = w.M if M is None else M
    V = w.V if V is None else V
    r = w.r if r is None else r
    d = w.hidden if hidden is None else hidden
    if lm_head is not None:
        w = dataclasses.replace(w, lm_head=lm_head)
    rng = np.random.default_rng(w.seed if seed is None else seed)
    base = rng.standard_normal((B, M, V), dtype=np.float32) * np.float32(w.base_sigma)
    if w.boost and B * M > 0 and V > 0:
        pos = rng.integers(0, V, size=(B, M))
        bi, ki = np.meshgrid(np.arange(B), np.arange(M), indexing="ij")
        base[bi, ki, pos] += np.float32(w.boost)
    w1 = rng.standard_normal((V, r), dtype=np.float32) * np.float32(w.w_sigma)
    w2 = rng.standard_normal((V, r), dtype=np.float32) * np.float32(w.w_sigma)
    if w.ids == "zipf1.1":
        token_ids = zipf_ids(rng, B * M, V, 1.1).reshape(B, M) if V > 0 else np.zeros((B, M), np.int64)
    else:
        token_ids = rng.integers(0, max(V, 1), size=(B, M), dtype=np.int64)
    first_prev = rng.integers(0, max(V, 1), size=(B,), dtype=np.int64)
    out = {"token_ids": token_ids, "first_prev": first_prev}
    if w.mode == "backward":
        # gradient of the loss w.r.t. the corrected logits, N(0, 1), in the
        # logits dtype, drawn after the ids
        g = rng.standard_normal((B, M, V), dtype=np.float32)
        out["grad"] = to_bf16_bits(g) if w.ldtype == BF16 else g
    if d:
        bound = np.float32(1.0 / np.sqrt(d + r))
        hid = rng.standard_normal((B, M, d), dtype=np.float32)
        gw = (rng.random((r, d + r), dtype=np.float32) * 2 - 1) * bound
        gb = (rng.random((r,), dtype=np.float32) * 2 - 1) * bound
        if w.dtype == BF16:
            hid, gw, gb = to_bf16_bits(hid), to_bf16_bits(gw), to_bf16_bits(gb)
        out.update(hidden=hid, gate_w=gw, gate_b=gb)
    if w.lm_head:
        # fused head: hidden states N(0, 1) [B, M, d] and the head's weight
        # [V, d] ~ N(0, 0.02^2) (initializer_range), bf16, drawn last
        dl = w.lm_head
        hs = rng.standard_normal((B, M, dl), dtype=np.float32)
        lw = np.empty((V, dl), dtype=np.uint16)
        for v0 in range(0, V, 8192):   # in slices: the fp32 draw of the whole head is 2.6 GB
            v1 = min(V, v0 + 8192)
            lw[v0:v1] = to_bf16_bits(rng.standard_normal((v1 - v0, dl), dtype=np.float32) * np.float32(w.w_sigma))
        out.update(lm_hidden=to_bf16_bits(hs), lm_head=lw)
    if w.ldtype == BF16:
        base = to_bf16_bits(base)
    if w.dtype == BF16:
        w1, w2 = to_bf16_bits(w1), to_bf16_bits(w2)
    out.update(base=base, w1=w1, w2=w2)
    return out
