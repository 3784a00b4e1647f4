"""Comparison rules between the HIP path and the CPU oracle.

Scores: the standard any-order floating-point dot-product bound. With fp32
accumulation over n = H_s * D_i products, |S_gpu - S_exact| <= gamma_n * max_t,s
sum |q_idx . k_idx terms| <= gamma_n * max||q|| * max||k|| (Cauchy-Schwarz),
gamma_n = n u / (1 - n u), u = 2^-24. The max-pool keeps the bound.

Ids: bit-identical wherever the oracle's K-1-th and K-th best candidate scores
differ by more than 1e-3 relative; inside such a near tie, any block whose
oracle score is within 1e-3 relative of the swapped one is accepted, and the
attention outputs are then compared with the oracle recomputed on the GPU's ids.

Outputs: max-abs 2e-2 (bf16) or 1e-5 (fp32) on out, 1e-3 absolute on lse.
"""

import numpy as np

from oracle import msa_oracle as O

REL_GAP = 1e-3
OUT_TOL = {"bf16": 2e-2, "f32": 1e-5}
LSE_TOL = 1e-3


def gamma(n, u=2.0 ** -24):
    return n * u / (1 - n * u)


def score_tolerance(q_idx, k_idx, n_sel):
    """Per-group absolute tolerance [n_sel] from the dot-product bound."""
    T, Hi, Di = q_idx.shape
    Hs = Hi // n_sel
    qn = np.linalg.norm(q_idx.reshape(T, n_sel, Hs * Di).astype(np.float64), axis=2).max(0)
    kf = np.transpose(k_idx, (0, 2, 1, 3)).reshape(-1, n_sel, Hs * Di).astype(np.float64)
    kn = np.linalg.norm(kf, axis=2).max(0)
    return gamma(Hs * Di) * qn * kn * 1.0001 + 1e-30


def check_scores(gpu, ref, tol, where=""):
    """gpu, ref [U][n_sel][row]; infinities must match exactly."""
    gpu = np.asarray(gpu, dtype=np.float64)
    inf = ~np.isfinite(ref)
    assert np.array_equal(gpu[inf], ref[inf]), f"{where}: +-inf pattern differs"
    err = np.zeros_like(ref)
    err[~inf] = np.abs(gpu[~inf] - ref[~inf])
    worst = (err / tol[None, :, None]).max() if err.size else 0.0
    assert worst <= 1.0, f"{where}: score error {err.max():.3e} exceeds the bound " \
                         f"(ratio {worst:.3f})"
    return float(err.max()) if err.size else 0.0


def ids_acceptable(gpu_ids, ref_scores_row, tau, topk):
    """Whether one row of GPU ids is correct under the near-tie rule.
    Returns (ok, exact) where exact says the ids equal the oracle's."""
    ref_ids = O.select_blocks(ref_scores_row, tau, topk)
    gpu_ids = [int(x) for x in gpu_ids]
    if gpu_ids == ref_ids:
        return True, True
    K = min(topk, tau + 1)
    kept = [b for b in gpu_ids if b >= 0]
    # structural validity: ascending, unique, diagonal present, right count, -1 tail
    if kept != sorted(set(kept)) or tau not in kept or len(kept) != K:
        return False, False
    if gpu_ids[len(kept):] != [-1] * (topk - len(kept)) or max(kept) > tau:
        return False, False
    m = K - 1
    cand = sorted((float(ref_scores_row[b]) for b in range(tau)), reverse=True)
    if len(cand) <= m:
        return False, False
    cm, cn = cand[m - 1] if m > 0 else np.inf, cand[m]
    gap = (cm - cn) / max(abs(cm), abs(cn), 1e-30) if m > 0 else np.inf
    if gap > REL_GAP:
        return False, False
    A, Oset = set(kept) - {tau}, set(ref_ids) - {tau, -1}
    for a in A - Oset:
        for o in Oset - A:
            sa, so = float(ref_scores_row[a]), float(ref_scores_row[o])
            if abs(sa - so) > REL_GAP * max(abs(sa), abs(so), 1e-30):
                return False, False
    return True, False


def check_ids(gpu_ids, ref_scores, units, topk, where=""):
    """Returns the number of rows whose ids differ from the oracle's (near ties)."""
    U, n_sel, _ = ref_scores.shape
    differ = 0
    for u in range(U):
        for g in range(n_sel):
            ok, exact = ids_acceptable(gpu_ids[u, g], ref_scores[u, g], units[u]["tau"], topk)
            assert ok, f"{where}: unit {u} group {g}: ids {list(gpu_ids[u, g])} vs oracle " \
                       f"{O.select_blocks(ref_scores[u, g], units[u]['tau'], topk)}"
            differ += not exact
    return differ


def check_attention(gpu_out, gpu_lse, ref_out, ref_lse, dtype, where=""):
    d_out = float(np.abs(np.asarray(gpu_out, np.float64) - ref_out).max()) if ref_out.size else 0
    d_lse = float(np.abs(np.asarray(gpu_lse, np.float64) - ref_lse).max()) if ref_lse.size else 0
    assert d_out <= OUT_TOL[dtype], f"{where}: out max-abs error {d_out:.3e}"
    assert d_lse <= LSE_TOL, f"{where}: lse error {d_lse:.3e}"
    return d_out, d_lse
