"""Sparse-MLA backward (dsa_sparse_mla_bwd) against the oracle, through the C ABI (needs an MI355X).

Bar (the project's 1e-3 relative reading applied to gradients, as for the indexer backward): every
dq and dkv entry within 1e-3 of the sum of the absolute values of its terms (dq[t,h,d]: sm_scale
|ds_i| |k_i[d]| over the row's entries; dkv[s,c]: sm_scale |ds| |q[t,h,c]| + p |dout[t,h,c]| over
every (t, h, entry) selecting s), plus 1e-6 of the array's largest such sum.  The term magnitudes
come from a float64 recomputation of p and ds (a tolerance scale, not an expected value).  At the
workload sizes dout is nonzero on sampled query rows only, so every other row contributes exactly
nothing and the oracle, run on the sampled rows, gives the complete dkv of the full-size launch.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import brute
import oracle
from dsa_inputs import get, prefill_inputs
from dsa_inputs.generate import block_rng, to_bf16_bits
from gpu_helpers import PrefillDev, dget, dput

pytestmark = pytest.mark.gpu
REL = 1e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_02_amd as dsa
    dsa.load()
    return torch.device("cuda:0")


def _log(*a):
    print(*a, flush=True)


def term_magnitudes(q, kv, dout, idx, pos, D_v, sm, rows):
    """(A_dq [R, H, D_qk], A_dkv [S, D_qk]): sums of |terms| of dq on the given rows and of dkv over
    those rows' entries, float64."""
    qd, kvd, gd = brute.bf16_decode(q), brute.bf16_decode(kv), brute.bf16_decode(dout)
    S, D_qk = kvd.shape
    H = qd.shape[1]
    A_dq = np.zeros((len(rows), H, D_qk))
    A_dkv = np.zeros((S, D_qk))
    for r, t in enumerate(rows):
        n = min(S, int(pos[t]) + 1)
        sel = np.array([int(s) for s in idx[t] if 0 <= s < n], dtype=np.int64)
        if len(sel) == 0:
            continue
        K = kvd[sel]                                              # [m, D_qk]
        z = sm * qd[t] @ K.T                                      # [H, m]
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = gd[t] @ K[:, :D_v].T
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        A_dq[r] = sm * np.abs(ds) @ np.abs(K)
        contrib = sm * np.abs(ds).T @ np.abs(qd[t])               # [m, D_qk]
        contrib[:, :D_v] += p.T @ np.abs(gd[t])
        np.add.at(A_dkv, sel, contrib)
    return A_dq, A_dkv


def check_grad(g, o, A, what):
    err = np.abs(g.astype(np.float64) - o)
    bar = REL * A + 1e-6 * A.max()
    worst = float(np.max(err / bar))
    assert worst <= 1.0, "%s: %d entries over the bar (worst %.3f of it, max err %.3e)" % (
        what, int((err > bar).sum()), worst, err.max())
    return worst


def run(dev, q, kv, idx, dout, sm, D_v, q_start):
    import dsa_lightning_indexer_02_amd as dsa
    qd, kvd = dput(q, dev).view(torch.bfloat16), dput(kv, dev).view(torch.bfloat16)
    it = dput(idx.astype(np.int32), dev)
    out, _, lse = dsa.dsa_sparse_mla_fwd(qd, kvd, it, sm, D_v, q_start=q_start)
    dq, dkv = dsa.dsa_sparse_mla_bwd(qd, kvd, it, lse, dput(dout, dev).view(torch.bfloat16), sm,
                                     q_start=q_start)
    torch.cuda.synchronize()
    return dget(dq), dget(dkv)


def _case(dev, T, S, H, k, q_start, idx, name, seed, rows=None, sm=1 / np.sqrt(192)):
    _log("case", name, "T", T, "S", S, "H", H, "k", k)
    g = block_rng(seed, T, S)
    q = to_bf16_bits(g.standard_normal((T, H, 576)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((S, 576)).astype(np.float32))
    dout = to_bf16_bits(g.standard_normal((T, H, 512)).astype(np.float32))
    rows = np.arange(T) if rows is None else np.asarray(rows)
    dq, dkv = run(dev, q, kv, idx, dout, sm, 512, q_start)
    pos = q_start + np.arange(T)
    odq, odkv = oracle.sparse_mla_bwd(q[rows], idx[rows], pos[rows], kv, 512, sm, dout[rows])
    A_dq, A_dkv = term_magnitudes(q, kv, dout, idx, pos, 512, sm, rows)
    w1 = check_grad(dq[rows], odq, A_dq, name + " dq")
    w2 = check_grad(dkv, odkv, A_dkv, name + " dkv")
    _log("  dq worst %.3f of the bar, dkv worst %.3f of the bar" % (w1, w2))
    return dq, dkv


def test_bwd_invalid_duplicate_entries(dev):
    g = block_rng(141, 0, 0)
    T, S, k = 24, 3000, 2048
    idx = g.integers(-5, S + 50, size=(T, k))
    idx[:, 10:20] = idx[:, 0:10]            # duplicates
    idx[5] = -1                             # nothing valid in row 5: dq = 0, no dkv contribution
    idx[6, 1:] = -1                         # a single entry: ds = 0 exactly
    dq, _ = _case(dev, T, S, 128, k, 2000, idx, "invalid/duplicate", 142)
    assert np.all(dq[5] == 0.0)


def test_bwd_short_lists_partial_heads(dev):
    # 100 heads (the second head half holds a partial group), lists of 64 with early rows seeing
    # fewer keys than the list length
    g = block_rng(143, 0, 0)
    T, S, k = 40, 300, 64
    idx = np.stack([g.permutation(S)[:k] for _ in range(T)]).astype(np.int64)
    _case(dev, T, S, 100, k, 0, idx, "H=100, k=64", 144)


def _workload(dev, name, rows, seed):
    import dsa_lightning_indexer_02_amd as dsa
    wl = get(name)
    _log("case", name, "sampled dout rows", len(rows))
    inp = prefill_inputs(wl)
    d = PrefillDev(inp, dev)
    lg = dsa.dsa_indexer_logits(d.q8, d.qs, d.w, d.k8, d.ks, q_start=wl.q_start)
    idx = dsa.dsa_topk(lg, wl.topk, wl.S, q_start=wl.q_start)
    del lg
    out, _, lse = dsa.dsa_sparse_mla_fwd(d.q, d.kv, idx, wl.sm_scale, wl.D_v, q_start=wl.q_start)
    g = block_rng(seed, len(rows), 0)
    dout = np.zeros((wl.T, wl.H, wl.D_v), np.uint16)
    dout[rows] = to_bf16_bits(g.standard_normal((len(rows), wl.H, wl.D_v)).astype(np.float32))
    dq, dkv = dsa.dsa_sparse_mla_bwd(d.q, d.kv, idx, lse, dput(dout, dev).view(torch.bfloat16), wl.sm_scale,
                                     q_start=wl.q_start)
    torch.cuda.synchronize()
    dq, dkv, idx = dget(dq), dget(dkv), dget(idx)
    # rows with dout = 0 get dq = 0 exactly
    others = np.setdiff1d(np.arange(wl.T), rows)
    assert np.all(dq[others] == 0.0), "rows without an output gradient must get dq = 0"
    pos = wl.q_start + np.arange(wl.T)
    odq, odkv = oracle.sparse_mla_bwd(inp.q[rows], idx[rows], pos[rows], inp.kv, wl.D_v, wl.sm_scale, dout[rows])
    A_dq, A_dkv = term_magnitudes(inp.q, inp.kv, dout, idx, pos, wl.D_v, wl.sm_scale, rows)
    w1 = check_grad(dq[rows], odq, A_dq, name + " dq")
    w2 = check_grad(dkv, odkv, A_dkv, name + " dkv")
    _log("  dq worst %.3f of the bar, dkv worst %.3f of the bar" % (w1, w2))


def test_bwd_prefill_4k_sampled(dev):
    _workload(dev, "prefill_4k", np.array([0, 1, 17, 1000, 2046, 2047, 2048, 2049, 3001, 4094, 4095]), 145)


def test_bwd_prefill_32k_sampled(dev):
    """The full-size launch (every row processed) with the output gradient on 24 rows spread over
    the causal triangle: dq on those rows, the complete dkv."""
    rows = np.unique(np.concatenate([np.linspace(0, 32767, 20).round().astype(np.int64), [1, 2047, 2048, 32767]]))
    _workload(dev, "prefill_32k", rows, 146)


def test_bwd_chunks_and_few_heads(dev):
    # 1100 rows: three chunks of the dKV buffers (512, 512, 76); 16 heads (a 64-head contraction
    # padded with zeros); repeated keys, including one repeated three times in a row's list
    g = block_rng(148, 0, 0)
    T, S, k, q_start = 1100, 1300, 96, 100
    idx = g.integers(-3, S, size=(T, k))
    idx[:, 40:44] = idx[:, 0:4]
    idx[:, 50] = idx[:, 0]
    _case(dev, T, S, 16, k, q_start, idx, "3 chunks, H=16", 149)


def test_bwd_determinism(dev):
    g = block_rng(147, 0, 0)
    T, S, k = 16, 2500, 2048
    idx = g.integers(0, S, size=(T, k))
    q = to_bf16_bits(g.standard_normal((T, 128, 576)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((S, 576)).astype(np.float32))
    dout = to_bf16_bits(g.standard_normal((T, 128, 512)).astype(np.float32))
    a = run(dev, q, kv, idx, dout, 0.07, 512, 2400)
    b = run(dev, q, kv, idx, dout, 0.07, 512, 2400)
    assert np.array_equal(a[0].view(np.int32), b[0].view(np.int32)), "dq must be bitwise reproducible"
    assert np.array_equal(a[1].view(np.int32), b[1].view(np.int32)), "dkv must be bitwise reproducible"
