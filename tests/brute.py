"""fp64 brute-force forms of the method, used only to pin the oracle.

Written independently of oracle/: FP8 and bf16 decoding go through torch's
own casts, contractions through numpy/torch fp64 matmuls.  Nothing here is
blocked, fused or reordered beyond the definitions.
"""
from __future__ import annotations

import numpy as np
import torch


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def visible(pos: np.ndarray, S: int) -> np.ndarray:
    return np.minimum(S, np.asarray(pos, dtype=np.int64) + 1)


def indexer(q8, qs, w, pos, k8, ks):
    """(I, A): index scores and their magnitude scale, fp64, NaN outside the causal range.

    A[t,s] = sum_j |w| * sum_i |q_I[t,j,i] * k_I[s,i]| bounds |I| and every partial sum.
    """
    qd = e4m3_decode(q8) * np.asarray(qs, np.float64)[..., None]        # [T,H,D]
    kd = e4m3_decode(k8) * np.asarray(ks, np.float64)[:, None]          # [S,D]
    w64 = np.asarray(w, np.float64)
    dots = np.einsum("tjd,sd->tjs", qd, kd)                              # exact: 18-bit integers x 2^-18
    I = np.einsum("tj,tjs->ts", w64, np.maximum(dots, 0.0))
    A = np.einsum("tj,tjs->ts", np.abs(w64), np.einsum("tjd,sd->tjs", np.abs(qd), np.abs(kd)))
    n = visible(pos, kd.shape[0])
    mask = np.arange(kd.shape[0])[None, :] >= n[:, None]
    I[mask] = np.nan
    A[mask] = np.nan
    return I, A


def topk_lexsort(scores_row: np.ndarray, n: int, k: int) -> np.ndarray:
    """numpy lexsort by (score descending, index ascending) over the first n entries."""
    s = np.asarray(scores_row[:n], np.float64)
    s = np.where(s == 0.0, 0.0, s)
    order = np.lexsort((np.arange(n), -s))
    out = np.full(k, -1, dtype=np.int64)
    m = min(k, n)
    out[:m] = order[:m]
    return out


def sparse_mla(q, idx, pos, kv, D_v, sm_scale):
    """fp64 attention over the listed rows (duplicates with multiplicity, invalid skipped)."""
    qd = bf16_decode(q)                  # [T,H,Dqk]
    kvd = bf16_decode(kv)                # [S,Dqk]
    T, H, _ = qd.shape
    S = kvd.shape[0]
    n = visible(pos, S)
    out = np.zeros((T, H, D_v))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        sel = [int(s) for s in idx[t] if 0 <= s < n[t]]
        if not sel:
            continue
        K = kvd[sel]                     # [m, Dqk]
        z = sm_scale * (qd[t] @ K.T)     # [H, m]
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        l = e.sum(axis=1, keepdims=True)
        out[t] = (e @ K[:, :D_v]) / l
        lse[t] = (m + np.log(l))[:, 0]
    return out, lse
