"""Comparison of GPU outputs with the CPU oracle (test infrastructure).

Corrected logits: every element must be bit-identical to the oracle's, or
lie in the oracle's admissible interval [lo, hi] -- the result of pushing the
dot product to -/+ 2r*2^-24*sum|e_j W2w[v,j]| (any fp32 accumulation order)
through the monotone rounding chain.  Elements outside the stated tolerance
(fp32: 1e-5 relative; bf16: 2e-2 absolute) but inside the interval are
rounding flips; they are counted and reported.

Tokens: the GPU token of each (b, k) must be exactly the oracle's selection
applied to the GPU's own (validated) corrected row; tokens that differ from
the oracle's selection on the oracle's own row are near-ties, counted.
Sampling is checked conditionally per step: the oracle is teacher-forced
with the GPU's previous tokens, so one near-tie cannot cascade.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from oracle import oracle as orc
from rank_markov_draft_amd import workloads as wl


@dataclasses.dataclass
class LogitReport:
    elements: int = 0
    mismatches: int = 0      # not bit-identical to the oracle
    flips: int = 0           # beyond the stated tolerance, inside the admissible interval
    max_abs_diff: float = 0.0


@dataclasses.dataclass
class TokenReport:
    tokens: int = 0
    near_ties: int = 0       # GPU token != oracle token on the oracle's own row
    noise_ties: int = 0      # GPU token == runner-up of a near-tied score on its own row
    max_tie_gap: float = 0.0  # largest oracle-row gap (value or score) behind a near-tie


def as_f32(a: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)


def tolerance_ok(gpu: np.ndarray, ref: np.ndarray, is_bf16: bool) -> np.ndarray:
    d = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    if is_bf16:
        return d <= 2e-2
    return d <= 1e-5 * np.maximum(np.abs(ref.astype(np.float64)), 1e-2)


def check_logits(gpu, ref, base, ids, w1, w2, report: LogitReport | None = None,
                 latent=None) -> LogitReport:
    """gpu, ref: oracle-typed arrays [R, M, V] (or [N, V]); base/ids/w1/w2 the
    oracle's inputs for the same rows (ids: the predecessor of every row).
    With ``latent`` [N, r] (gated head) row n is biased by latent[n] instead
    of w1[ids[n]], and ids/w1 are not used."""
    rep = report or LogitReport()
    V = gpu.shape[-1]
    g = as_f32(gpu).reshape(-1, V)
    o = as_f32(ref).reshape(-1, V)
    rep.elements += g.size
    same = (g.view(np.uint32) == o.view(np.uint32)) | (np.isnan(g) & np.isnan(o))
    bad_r, bad_c = np.nonzero(~same)
    rep.mismatches += int(bad_r.size)
    if bad_r.size:
        rep.max_abs_diff = max(rep.max_abs_diff, float(np.max(np.abs(g[bad_r, bad_c] - o[bad_r, bad_c]))))
        if latent is None:
            lo, mid, hi = orc.logit_bounds(base, ids, w1, w2, bad_r, bad_c)
        else:
            lo, mid, hi = orc.logit_bounds_rows(base.reshape(-1, V), latent.reshape(-1, latent.shape[-1]),
                                                w2, bad_r, bad_c)
        gv = g[bad_r, bad_c]
        assert np.array_equal(mid, o[bad_r, bad_c]), "oracle bounds disagree with oracle values"
        inside = (lo <= gv) & (gv <= hi)
        if not inside.all():
            i = int(np.argmin(inside))
            raise AssertionError(
                f"{int((~inside).sum())} of {g.size} corrected logits outside the admissible interval; "
                f"first at row {bad_r[i]} col {bad_c[i]}: gpu {gv[i]!r} oracle {o[bad_r[i], bad_c[i]]!r} "
                f"interval [{lo[i]!r}, {hi[i]!r}]")
        rep.flips += int((~tolerance_ok(gv, o[bad_r, bad_c], gpu.dtype == np.uint16)).sum())
    return rep


@dataclasses.dataclass
class LatentReport:
    elements: int = 0
    mismatches: int = 0      # not bit-identical to the oracle's latent
    max_rel_diff: float = 0.0


def check_latent(gpu_latent, hidden, ids, w1, gate_w, gate_b, report: LatentReport | None = None) -> LatentReport:
    """Gated head: the GPU's latent rows [N, r] against the oracle's for the
    same hidden rows [N, d] and predecessors [N].  Every element must lie in
    the oracle's admissible interval (fp32 accumulation of the gate in any
    order, fp32 logistic within 2^-20 relative); fp32 latents must also be
    within 1e-5 relative of the oracle's."""
    rep = report or LatentReport()
    r = w1.shape[1]
    lat, lo, hi = orc.gated_latent(hidden, ids, w1, gate_w, gate_b, bounds=True)
    g = as_f32(gpu_latent).reshape(-1, r)
    o = as_f32(lat).reshape(-1, r)
    rep.elements += g.size
    rep.mismatches += int((g.view(np.uint32) != o.view(np.uint32)).sum())
    inside = (lo <= g) & (g <= hi)
    if not inside.all():
        i, j = (int(t[0]) for t in np.nonzero(~inside))
        raise AssertionError(f"{int((~inside).sum())} of {g.size} latent elements outside the admissible "
                             f"interval; first at row {i} col {j}: gpu {g[i, j]!r} oracle {o[i, j]!r} "
                             f"interval [{lo[i, j]!r}, {hi[i, j]!r}]")
    rel = np.abs(g.astype(np.float64) - o) / np.maximum(np.abs(o.astype(np.float64)), 1e-30)
    rel[(g == o)] = 0.0
    rep.max_rel_diff = max(rep.max_rel_diff, float(rel.max()) if rel.size else 0.0)
    if gpu_latent.dtype != np.uint16:
        e = as_f32(w1)[np.asarray(ids).reshape(-1)]
        ok = np.abs(g - o) <= 1e-5 * np.maximum(np.abs(o), 1e-6 * np.abs(e))
        assert ok.all(), f"{int((~ok).sum())} fp32 latent elements beyond 1e-5 relative"
    return rep


def _bf16_ulp(x: float) -> float:
    return float(np.spacing(np.float32(abs(x)))) * 2.0 ** 16


def check_tokens(gpu_tokens, gpu_rows, oracle_rows, temperature, seed, b_abs, k_abs,
                 report: TokenReport | None = None) -> TokenReport:
    """gpu_tokens [N]; gpu_rows/oracle_rows: oracle-typed [N, V] corrected rows;
    b_abs/k_abs [N] noise indices of each row.

    Greedy: the GPU token must be exactly the first argmax of its own row.
    Temperature: it must be the oracle's Gumbel-max selection on that row, or
    -- the device log2 may differ from libm's by an ulp -- the runner-up when
    the top-2 scores are within 1e-5 relative (a counted noise near-tie).

    Near-ties (GPU token != the oracle's selection on the oracle's own row)
    are counted and bounded: on the oracle's row, the gap between the
    oracle's winner and the GPU's token must be explained by the GPU row's
    admissible deviation at those two columns (already validated against the
    oracle's intervals) plus the float tolerance (fp32: 1e-5 relative of the
    winner; temperature scores: 1e-5 relative), and for bf16 greedy rows it
    must be at most one bf16 ulp of the winner."""
    rep = report or TokenReport()
    greedy = temperature < 1e-5
    gpu_tokens = np.asarray(gpu_tokens).reshape(-1)
    n = gpu_tokens.shape[0]
    V = gpu_rows.shape[-1]
    g_rows = np.asarray(gpu_rows).reshape(n, V)
    b_abs = np.asarray(b_abs).reshape(-1)
    k_abs = np.asarray(k_abs).reshape(-1)
    t_own, sc, runner = orc.select_tokens(g_rows, temperature, seed, b_abs, k_abs)
    rep.tokens += n
    for i in np.nonzero(t_own != gpu_tokens)[0]:
        tg, best, second = int(gpu_tokens[i]), float(sc[i, 0]), float(sc[i, 1])
        assert not greedy, f"row {i}: GPU token {tg} is not the first argmax {t_own[i]} of its own row"
        assert runner[i] == tg and abs(best - second) <= 1e-5 * max(1.0, abs(best)), (
            f"row {i}: GPU token {tg} vs oracle selection {t_own[i]} on the same row is not a near-tie "
            f"(scores {best!r}, {second!r}, runner-up {runner[i]})")
        rep.noise_ties += 1
    if oracle_rows is None:
        return rep
    o_rows = np.asarray(oracle_rows).reshape(n, V)
    t_ref = orc.select_tokens(o_rows, temperature, seed, b_abs, k_abs)[0]
    is_bf16 = g_rows.dtype == np.uint16
    kappa = 0.0 if greedy else orc.kappa(temperature)
    for i in np.nonzero(t_ref != gpu_tokens)[0]:
        tg, tr = int(gpu_tokens[i]), int(t_ref[i])
        og = as_f32(o_rows[i, [tg, tr]]).astype(np.float64)
        gg = as_f32(g_rows[i, [tg, tr]]).astype(np.float64)
        dev = float(np.max(np.abs(gg - og)))
        if greedy:
            gap = og[1] - og[0]
            allowed = dev + (0.0 if is_bf16 else 1e-5 * max(1.0, abs(og[1])))
            ok = gap <= allowed and (not is_bf16 or gap <= _bf16_ulp(og[1]))
        else:
            noise = [orc.gumbel2(seed, b_abs[i], k_abs[i], t) for t in (tg, tr)]
            s_g, s_r = (float(np.float32(og[j] * kappa + noise[j])) for j in range(2))
            gap = s_r - s_g
            ok = gap <= 1e-5 * max(1.0, abs(s_r)) + kappa * dev
        assert ok, (f"row {i}: GPU token {tg} differs from the oracle's {tr} by a gap of {gap!r} on the "
                    f"oracle's row, beyond the GPU row's deviation {dev!r} at those columns and the tolerance")
        rep.near_ties += 1
        rep.max_tie_gap = max(rep.max_tie_gap, float(gap))
    return rep
