"""Comparison rules between the HIP path and the oracle (the project's parity tolerances).

Indexer: (i) |g - o| <= 1e-3 * A everywhere in the causal range, A = sum_j |w| qs ks sum_i |dec q8 * dec k8|
         (the magnitude scale of the sum, A >= |o|); (ii) |g - o| / |o| <= 1e-3 where the relative error is
         meaningful: |o| >= c * A with c = (oracle fp32 error bound + FP8 MFMA accumulation bound) / 1e-3,
         i.e. ((D_I + H_I + 4) 2^-24 + 2^-14) / 1e-3.  Below that, the oracle's own rounding alone may exceed
         1e-3 |o|.  The GPU error against the exact fp64 value is pinned separately to <= 2^-14 A.
Top-k:   the GPU selection run on the GPU's own logits must equal the oracle's selection on those
         same logits exactly (ties included); against the oracle's own logits the sets may differ
         only by swaps at the k-th boundary whose oracle scores lie within 1e-3 relative of the
         k-th score (plus 1e-6 of the row maximum, for a k-th score of 0).
Attention (on the same index lists): bf16 output max abs error <= 2e-2; fp32 output per (t, h)
         row max_d |g - o| / max_d |o| <= 1e-3; |lse_g - lse_o| <= 1e-3 * max(1, |lse_o|).
"""
from __future__ import annotations

import numpy as np

IDX_ABS = 1e-3
IDX_REL = 1e-3
TOPK_REL = 1e-3
MLA_BF16_ABS = 2e-2
MLA_F32_REL = 1e-3
LSE_TOL = 1e-3


def e4m3_abs_table() -> np.ndarray:
    import torch
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    t = np.nan_to_num(t, nan=0.0)
    return np.abs(t).astype(np.float32)


def magnitude(q8, qs, w, k8, ks, rows_pos, S, chunk: int = 16) -> np.ndarray:
    """A[t, s] (fp32) for the given rows; NaN outside the causal range."""
    tab = e4m3_abs_table()
    kd = tab[k8] * np.abs(ks)[:, None]                       # [S, D]
    out = np.empty((q8.shape[0], S), dtype=np.float32)
    for a in range(0, q8.shape[0], chunk):
        b = min(a + chunk, q8.shape[0])
        qd = tab[q8[a:b]] * np.abs(qs[a:b])[..., None]       # [c, H, D]
        m = np.einsum("chd,sd->chs", qd, kd, optimize=True)   # [c, H, S]
        out[a:b] = np.einsum("ch,chs->cs", np.abs(w[a:b]), m, optimize=True)
    n = np.minimum(S, np.asarray(rows_pos) + 1)
    out[np.arange(S)[None, :] >= n[:, None]] = np.nan
    return out


MFMA_FP8_BOUND = 2.0 ** -14   # accumulation error allowance of the gfx950 FP8 MFMA, relative to A


def rel_threshold(D_I: int, H_I: int) -> float:
    return ((D_I + H_I + 4) * 2.0 ** -24 + MFMA_FP8_BOUND) / IDX_REL


def check_indexer(g: np.ndarray, o: np.ndarray, A: np.ndarray, D_I: int, H_I: int, what: str = "indexer"):
    m = ~np.isnan(o)
    gm, om, Am = g[m].astype(np.float64), o[m].astype(np.float64), A[m].astype(np.float64)
    err = np.abs(gm - om)
    bad = err > IDX_ABS * Am
    assert not bad.any(), "%s: %d entries exceed 1e-3*A (worst %.3e of A)" % (
        what, bad.sum(), np.max(err / np.maximum(Am, 1e-30)))
    big = np.abs(om) >= rel_threshold(D_I, H_I) * Am
    rel = err[big] / np.abs(om[big])
    assert rel.size == 0 or rel.max() <= IDX_REL, "%s: relative error %.3e" % (what, rel.max())
    return float(np.max(err / np.maximum(Am, 1e-30))) if err.size else 0.0


def check_indexer_exact(g: np.ndarray, exact: np.ndarray, A: np.ndarray, what: str = "indexer vs exact"):
    """GPU scores against the exact (fp64) value: within the FP8 MFMA accumulation bound plus fp32 epilogue."""
    m = ~np.isnan(exact)
    err = np.abs(g[m].astype(np.float64) - exact[m]) / np.maximum(A[m].astype(np.float64), 1e-30)
    assert err.max() <= MFMA_FP8_BOUND + 2.0 ** -20, "%s: %.3e of A" % (what, err.max())
    return float(err.max())


def valid_set(row: np.ndarray) -> np.ndarray:
    return np.sort(row[row >= 0])


def check_topk_exact(g_idx: np.ndarray, o_idx: np.ndarray, what: str = "top-k"):
    for t in range(g_idx.shape[0]):
        gs, os_ = valid_set(g_idx[t]), valid_set(o_idx[t])
        assert len(gs) == len(np.unique(gs)), "%s row %d: duplicate indices" % (what, t)
        assert np.array_equal(gs, os_), "%s row %d: sets differ (%d vs %d, %d common)" % (
            what, t, len(gs), len(os_), len(np.intersect1d(gs, os_)))
        assert np.all(g_idx[t][len(gs):] == -1), "%s row %d: -1 padding not at the end" % (what, t)


def check_topk_boundary(g_idx: np.ndarray, o_idx: np.ndarray, o_logits: np.ndarray, n: np.ndarray,
                        what: str = "top-k vs oracle logits"):
    swaps = 0
    for t in range(g_idx.shape[0]):
        gs, os_ = valid_set(g_idx[t]), valid_set(o_idx[t])
        assert len(gs) == len(os_), "%s row %d: %d vs %d selected" % (what, t, len(gs), len(os_))
        assert len(gs) == len(np.unique(gs)) and (len(gs) == 0 or (gs.min() >= 0 and gs.max() < n[t]))
        diff = np.setxor1d(gs, os_)
        if diff.size == 0:
            continue
        row = o_logits[t, :n[t]].astype(np.float64)
        tau = np.sort(row)[::-1][len(os_) - 1]
        tol = TOPK_REL * abs(tau) + 1e-6 * np.max(np.abs(row))
        assert np.all(np.abs(row[diff] - tau) <= tol), "%s row %d: swap outside the boundary band" % (what, t)
        swaps += diff.size // 2
    return swaps


def check_mla(g_bf16: np.ndarray, g_f32: np.ndarray, g_lse: np.ndarray, o_f32: np.ndarray, o_lse: np.ndarray,
              what: str = "sparse MLA"):
    """g_bf16 as float32 values."""
    abs_err = np.abs(g_bf16.astype(np.float64) - o_f32)
    assert abs_err.max() <= MLA_BF16_ABS, "%s: bf16 max abs error %.3e" % (what, abs_err.max())
    num = np.abs(g_f32.astype(np.float64) - o_f32).max(axis=-1)
    den = np.abs(o_f32).max(axis=-1)
    rel = num / np.maximum(den, 1e-30)
    assert rel.max() <= MLA_F32_REL, "%s: fp32 row-relative error %.3e" % (what, rel.max())
    fin = np.isfinite(o_lse)
    assert np.array_equal(fin, np.isfinite(g_lse)), "%s: lse finiteness differs" % what
    le = np.abs(g_lse[fin].astype(np.float64) - o_lse[fin]) / np.maximum(1.0, np.abs(o_lse[fin]))
    assert le.size == 0 or le.max() <= LSE_TOL, "%s: lse error %.3e" % (what, le.max())
    return float(abs_err.max()), float(rel.max())
