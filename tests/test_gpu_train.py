"""The indexer's training signal (KL loss toward the head-averaged main attention) and the indexer
backward through the C ABI against the oracle (needs an MI355X).

Shapes cover the workloads' widths (H = 128 heads of 576-wide latent rows, H_I = 64 indexer heads
of 128) and the small configuration's (8 heads of 80, 4 indexer heads of 32), an odd number of
query rows (the last workgroup holds one row), partial head groups, a latent row width that is
not a multiple of 16, every supported D_I, rows that end inside a key block, the in-place score
gradient, and the whole chain (indexer -> loss -> backward) at the 4K prefill shape on sampled
rows."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import parity
from dsa_inputs.generate import block_rng, quantize_fp8_rows, to_bf16_bits
from gpu_helpers import dget, dput

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_02_amd as dsa
    dsa.load()
    return torch.device("cuda:0")


def _kl_case(dev, T, S, q_start, H, D, sm, seed, scale=2.0, in_place=False):
    import dsa_lightning_indexer_02_amd as dsa
    print("case kl", T, S, q_start, H, D, "in_place" if in_place else "", flush=True)
    g = block_rng(seed, T, S)
    q = to_bf16_bits(g.standard_normal((T, H, D)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((S, D)).astype(np.float32))
    ld = dsa.ld_for(S)
    logits = np.zeros((T, ld), np.float32)
    logits[:, :S] = (g.standard_normal((T, S)) * scale).astype(np.float32)
    lg = dput(logits, dev)
    loss, d = dsa.dsa_indexer_kl_loss(dput(q, dev).view(torch.bfloat16), dput(kv, dev).view(torch.bfloat16), lg,
                                      sm, q_start=q_start, in_place=in_place)
    torch.cuda.synchronize()
    pos = q_start + np.arange(T)
    lo, do = oracle.indexer_kl(q, kv, pos, sm, logits[:, :S])
    worst = parity.check_kl(dget(loss), dget(d)[:, :S], lo, do, logits[:, :S], pos, "kl %dx%d H=%d D=%d" % (T, S, H, D))
    print("  worst error / bar: %.3e" % worst, flush=True)
    if in_place:
        assert d.data_ptr() == lg.data_ptr()


@pytest.mark.parametrize("T,S,q_start,H,D,sm", [
    (40, 64, 24, 8, 80, 80 ** -0.5),          # the small configuration's attention shape
    (67, 300, 250, 128, 576, 192 ** -0.5),    # full width, odd row count, rows ending mid-block
    (33, 100, 80, 20, 72, 0.11),              # partial head group, row width padded to 80
    (16, 16, 0, 128, 576, 192 ** -0.5),       # causal from the first key (rows of 1 .. 16 keys)
])
def test_kl_loss_vs_oracle(dev, T, S, q_start, H, D, sm):
    _kl_case(dev, T, S, q_start, H, D, sm, 81)


def test_kl_loss_in_place_and_sharp(dev):
    _kl_case(dev, 31, 97, 70, 64, 576, 192 ** -0.5, 82, in_place=True)
    # sharp indexer distributions (scores spread over ~60 nats)
    _kl_case(dev, 20, 50, 30, 16, 80, 0.5, 83, scale=20.0)


def _bwd_case(dev, T, S, q_start, H_I, D_I, seed):
    import dsa_lightning_indexer_02_amd as dsa
    print("case bwd", T, S, q_start, H_I, D_I, flush=True)
    g = block_rng(seed, T, S)
    q8, qs = quantize_fp8_rows(g.standard_normal((T, H_I, D_I)).astype(np.float32))
    k8, ks = quantize_fp8_rows(g.standard_normal((S, D_I)).astype(np.float32))
    w = (g.uniform(0.0, 1.0, (T, H_I)) / H_I).astype(np.float32)
    ld = dsa.ld_for(S)
    dI = np.zeros((T, ld), np.float32)
    dI[:, :S] = (g.standard_normal((T, S)) * 1e-2).astype(np.float32)
    dq, dw, dk = dsa.dsa_indexer_bwd(dput(q8, dev), dput(qs, dev), dput(w, dev), dput(k8, dev), dput(ks, dev),
                                     dput(dI, dev), q_start=q_start)
    torch.cuda.synchronize()
    pos = q_start + np.arange(T)
    oq, ow, ok = oracle.indexer_bwd(q8, qs, w, pos, k8, ks, dI[:, :S])
    amb, worst = parity.check_indexer_bwd(dget(dq), dget(dw), dget(dk), oq, ow, ok, q8, qs, w, k8, ks, dI[:, :S], pos,
                                   "bwd %dx%d H_I=%d D_I=%d" % (T, S, H_I, D_I))
    print("  ambiguous ReLU signs: %d, worst error / bar: %.3e" % (amb, worst), flush=True)


@pytest.mark.parametrize("T,S,q_start,H_I,D_I", [
    (256, 256, 0, 4, 32),        # the small configuration
    (100, 300, 200, 64, 128),    # full heads; ragged rows, keys and query chunks
    (50, 50, 0, 20, 64),         # partial head group
    (40, 170, 130, 8, 96),
    (300, 700, 400, 64, 128),    # several dk query chunks, key groups that no row sees
])
def test_indexer_bwd_vs_oracle(dev, T, S, q_start, H_I, D_I):
    _bwd_case(dev, T, S, q_start, H_I, D_I, 84)


def _distinct_lists(T, S, pos, k, seed):
    """Index lists with distinct valid entries (as top-k writes them), -1 padding and one entry
    beyond the causal range per row."""
    g = block_rng(seed, T, k)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = min(S, int(pos[t]) + 1)
        m = min(n, k)
        idx[t, :m] = g.permutation(n)[:m]
        if m > 3:
            idx[t, 2] = n + 5
    return idx


def _bwd_listed_case(dev, T, S, q_start, H_I, D_I, k, seed):
    import dsa_lightning_indexer_02_amd as dsa
    print("case bwd listed", T, S, q_start, H_I, D_I, k, flush=True)
    g = block_rng(seed, T, S)
    q8, qs = quantize_fp8_rows(g.standard_normal((T, H_I, D_I)).astype(np.float32))
    k8, ks = quantize_fp8_rows(g.standard_normal((S, D_I)).astype(np.float32))
    w = (g.uniform(0.0, 1.0, (T, H_I)) / H_I).astype(np.float32)
    pos = q_start + np.arange(T)
    idx = _distinct_lists(T, S, pos, k, seed + 1)
    ld = dsa.ld_for(S)
    dI = np.zeros((T, ld), np.float32)      # nonzero at the valid listed keys only
    for t in range(T):
        keys = idx[t][(idx[t] >= 0) & (idx[t] < pos[t] + 1) & (idx[t] < S)]
        dI[t, keys] = (g.standard_normal(keys.size) * 1e-2).astype(np.float32)
    dq, dw, dk = dsa.dsa_indexer_bwd_listed(dput(q8, dev), dput(qs, dev), dput(w, dev), dput(k8, dev),
                                            dput(ks, dev), dput(idx, dev), dput(dI, dev), q_start=q_start)
    torch.cuda.synchronize()
    oq, ow, ok = oracle.indexer_bwd(q8, qs, w, pos, k8, ks, dI[:, :S])
    amb, worst = parity.check_indexer_bwd(dget(dq), dget(dw), dget(dk), oq, ow, ok, q8, qs, w, k8, ks, dI[:, :S], pos,
                                          "bwd listed %dx%d H_I=%d D_I=%d k=%d" % (T, S, H_I, D_I, k))
    print("  ambiguous ReLU signs: %d, worst error / bar: %.3e" % (amb, worst), flush=True)


@pytest.mark.parametrize("T,S,q_start,H_I,D_I,k", [
    (256, 256, 0, 4, 32, 64),        # the small configuration (rows shorter than their lists)
    (40, 3000, 2900, 64, 128, 2048),  # full heads and list length
    (50, 50, 0, 20, 64, 16),         # partial head group, one list block
    (40, 170, 130, 8, 96, 48),       # a ragged list block
    (33, 300, 100, 60, 128, 100),    # a partial wave of heads
])
def test_indexer_bwd_listed_vs_oracle(dev, T, S, q_start, H_I, D_I, k):
    _bwd_listed_case(dev, T, S, q_start, H_I, D_I, k, 88)


def test_train_chain_prefill_4k_rows(dev):
    """indexer -> KL loss (in place) -> backward at the 4K prefill shape; the loss and dI of
    sampled rows against the oracle (its own scores), the backward against the oracle fed the same
    GPU-independent inputs on a slice of the rows."""
    import dsa_lightning_indexer_02_amd as dsa
    from dsa_inputs import get, prefill_inputs
    wl = get("prefill_4k")
    inp = prefill_inputs(wl)
    print("case train chain prefill_4k", flush=True)
    lg = dsa.dsa_indexer_logits(dput(inp.q8, dev), dput(inp.qs, dev), dput(inp.w, dev), dput(inp.k8, dev),
                                dput(inp.ks, dev), 0)
    q = dput(inp.q, dev).view(torch.bfloat16)
    kv = dput(inp.kv, dev).view(torch.bfloat16)
    loss, d = dsa.dsa_indexer_kl_loss(q, kv, lg, wl.sm_scale, in_place=True)
    dq, dw, dk = dsa.dsa_indexer_bwd(dput(inp.q8, dev), dput(inp.qs, dev), dput(inp.w, dev), dput(inp.k8, dev),
                                     dput(inp.ks, dev), d)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 17, 1000, 2047, 3333, 4095])
    pos = rows.astype(np.int64)
    o_lg = oracle.indexer(inp.q8[rows], inp.qs[rows], inp.w[rows], pos, inp.k8, inp.ks)
    o_lg = np.nan_to_num(o_lg, nan=0.0)
    lo, do = oracle.indexer_kl(inp.q[rows], inp.kv, pos, wl.sm_scale, o_lg)
    # the GPU's scores differ from the oracle's within the indexer bar; the loss moves by at most
    # sum |dI| |dlogit| <= 2 max |dlogit|, dI by at most (e - 1)-relative of pi
    A = parity.magnitude(inp.q8[rows], inp.qs[rows], inp.w[rows], inp.k8, inp.ks, pos, wl.S)
    dmax = np.nanmax(A, axis=1) * (parity.indexer_beta(wl.D_I, wl.H_I) + (wl.H_I + 3) * 2.0 ** -24)
    g_loss, g_d = dget(loss)[rows], dget(d)[rows, :wl.S]
    for i, t in enumerate(rows):
        n = t + 1
        x = o_lg[i, :n].astype(np.float64)
        pi = np.exp(x - x.max()) / np.sum(np.exp(x - x.max()))
        p = pi - do[i, :n]
        tol = parity.KL_REL * (np.abs(p) + pi) + pi * (np.exp(2 * dmax[i]) - 1) + 1e-9
        assert np.all(np.abs(g_d[i, :n] - do[i, :n]) <= tol), "chain dI row %d" % t
        assert abs(g_loss[i] - lo[i]) <= parity.KL_REL * (lo[i] + 1.0) + 2 * dmax[i], "chain loss row %d" % t
    assert np.all(np.isfinite(dget(dq))) and np.all(np.isfinite(dget(dw))) and np.all(np.isfinite(dget(dk)))
    # the backward on the GPU's own dI is checked elementwise by the shape tests above; at full size
    # it must satisfy Euler's identity: I is homogeneous of degree 2 in (q_I, k_I) jointly and of
    # degree 1 in w, so (sum dq . q_I + sum dk . k_I) / 2 = sum dI I = sum dw . w
    tab = parity.e4m3_abs_table().astype(np.float64) * np.where(np.arange(256) & 0x80, -1.0, 1.0)
    qd = tab[inp.q8] * inp.qs.astype(np.float64)[..., None]
    kd = tab[inp.k8] * inp.ks.astype(np.float64)[:, None]
    gq, gk, gw = (dget(x).astype(np.float64) for x in (dq, dk, dw))
    lhs = (np.sum(gq * qd) + np.sum(gk * kd)) / 2.0
    rhs = np.sum(gw * inp.w.astype(np.float64))
    scale = (np.sum(np.abs(gq * qd)) + np.sum(np.abs(gk * kd))) / 2.0 + np.sum(np.abs(gw * inp.w))
    assert abs(lhs - rhs) <= parity.KL_REL * scale, "Euler identity of the backward: %.6e vs %.6e" % (lhs, rhs)


# ------------------------------------------------------------------ sparse-stage loss
def _sparse_lists(T, S, pos, k, seed):
    g = block_rng(seed, T, k)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = min(S, int(pos[t]) + 1)
        m = min(n, k)
        idx[t, :m] = g.permutation(n)[:m]
        if m > 3:
            idx[t, 1] = idx[t, 0]           # a repeated key
            idx[t, 2] = n + 5               # beyond the causal range: skipped
    return idx


def _kl_sparse_case(dev, T, S, q_start, H, D, D_v, k, sm, seed, in_place=False, gpu_lse=True):
    import dsa_lightning_indexer_02_amd as dsa
    print("case kl sparse", T, S, q_start, H, D, k, "in_place" if in_place else "", flush=True)
    g = block_rng(seed, T, S)
    q = to_bf16_bits(g.standard_normal((T, H, D)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((S, D)).astype(np.float32))
    pos = q_start + np.arange(T)
    idx = _sparse_lists(T, S, pos, k, seed + 1)
    ld = dsa.ld_for(S)
    logits = np.zeros((T, ld), np.float32)
    logits[:, :S] = (g.standard_normal((T, S)) * 2.0).astype(np.float32)
    qd, kvd, idd = dput(q, dev).view(torch.bfloat16), dput(kv, dev).view(torch.bfloat16), dput(idx, dev)
    if gpu_lse:   # the sparse forward's normaliser over the same lists
        _, _, lse = dsa.dsa_sparse_mla_fwd(qd, kvd, idd, sm, D_v, q_start=q_start)
    else:         # a width the forward does not take: the oracle forward's normaliser as the input
        _, _, lse_o = oracle.sparse_mla(q, idx, pos, kv, D_v, sm)
        lse = dput(lse_o, dev)
    lg = dput(logits, dev)
    loss, d = dsa.dsa_indexer_kl_loss_sparse(qd, kvd, idd, lse, lg, sm, q_start=q_start, in_place=in_place)
    torch.cuda.synchronize()
    lo, do = oracle.indexer_kl_sparse(q, kv, pos, sm, idx, logits[:, :S])
    worst = parity.check_kl_sparse(dget(loss), dget(d)[:, :S], lo, do, logits[:, :S], pos, idx,
                                   "kl sparse %dx%d H=%d D=%d k=%d" % (T, S, H, D, k))
    print("  worst error / bar: %.3e" % worst, flush=True)


@pytest.mark.parametrize("T,S,q_start,H,D,D_v,k,sm,gpu_lse", [
    (40, 64, 24, 8, 80, 64, 16, 80 ** -0.5, True),          # the small configuration's shapes
    (21, 3000, 2900, 128, 576, 512, 2048, 192 ** -0.5, True),  # full width and k
    (33, 100, 80, 20, 72, 64, 48, 0.11, False),             # partial head group, padded width
    (10, 40, 0, 128, 576, 512, 64, 192 ** -0.5, True),      # rows shorter than their lists (-1 padded)
])
def test_kl_sparse_vs_oracle(dev, T, S, q_start, H, D, D_v, k, sm, gpu_lse):
    _kl_sparse_case(dev, T, S, q_start, H, D, D_v, k, sm, 85, gpu_lse=gpu_lse)


def test_kl_sparse_in_place(dev):
    _kl_sparse_case(dev, 17, 500, 450, 64, 576, 512, 256, 192 ** -0.5, 86, in_place=True)


def test_sparse_stage_chain_prefill_4k(dev):
    """indexer -> top-2048 -> sparse attention (lse) -> sparse-stage loss in place -> backward at the
    4K prefill shape.  Invariants of every row: keys outside the list get exactly 0, the gradient
    sums to 0 (both distributions sum to 1), the loss is non-negative, all finite."""
    import dsa_lightning_indexer_02_amd as dsa
    from dsa_inputs import get, prefill_inputs
    wl = get("prefill_4k")
    inp = prefill_inputs(wl)
    print("case sparse-stage chain prefill_4k", flush=True)
    q8, qs, w, k8, ks = (dput(x, dev) for x in (inp.q8, inp.qs, inp.w, inp.k8, inp.ks))
    q = dput(inp.q, dev).view(torch.bfloat16)
    kv = dput(inp.kv, dev).view(torch.bfloat16)
    lg = dsa.dsa_indexer_logits(q8, qs, w, k8, ks, 0)
    idx = dsa.dsa_topk(lg, wl.topk, wl.S)
    _, _, lse = dsa.dsa_sparse_mla_fwd(q, kv, idx, wl.sm_scale, wl.D_v)
    loss, d = dsa.dsa_indexer_kl_loss_sparse(q, kv, idx, lse, lg, wl.sm_scale, in_place=True)
    dq, dw, dk = dsa.dsa_indexer_bwd(q8, qs, w, k8, ks, d)
    torch.cuda.synchronize()
    L, D, I = dget(loss), dget(d)[:, :wl.S], dget(idx)
    assert np.all(np.isfinite(L)) and np.all(L >= -1e-5), "sparse-stage loss must be finite and non-negative"
    for t in [0, 1, 100, 2047, 2048, 3000, 4095]:
        n = t + 1
        listed = np.zeros(n, bool)
        listed[I[t][I[t] >= 0]] = True
        assert np.all(D[t, :n][~listed] == 0.0)
        assert abs(float(np.sum(D[t, :n].astype(np.float64)))) <= 1e-5, "row %d gradient does not sum to 0" % t
    for x in (dq, dw, dk):
        assert np.all(np.isfinite(dget(x)))
    # the listed backward on the same lists: dk through the same kernels, dq / dw summed in
    # another order over the same nonzero terms
    lq, lw, lk = dsa.dsa_indexer_bwd_listed(q8, qs, w, k8, ks, idx, d)
    torch.cuda.synchronize()
    assert np.array_equal(dget(lk), dget(dk))
    for a, b, name in ((lq, dq, "dq"), (lw, dw, "dw")):
        a, b = dget(a), dget(b)
        assert np.max(np.abs(a - b)) <= 1e-4 * np.max(np.abs(b)), "listed %s differs from the dense backward" % name


def test_train_long_context_rows(dev):
    """The chunked-prefill shape: 64 query rows at positions 131008 .. 131071 over a 131072-key
    context (4096 key blocks per row in the loss, key groups and query chunks far from the origin
    in the backward); loss and dI of two rows against the oracle, the backward on a 16-row slice and
    the listed backward (2048-entry lists over the whole context) on 8 rows."""
    import dsa_lightning_indexer_02_amd as dsa
    T, S, H, D, H_I, D_I = 64, 131072, 128, 576, 64, 128
    q_start = S - T
    sm = 192 ** -0.5
    print("case long context", T, S, flush=True)
    g = block_rng(87, T, S)
    q = to_bf16_bits(g.standard_normal((T, H, D)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((S, D)).astype(np.float32))
    ld = dsa.ld_for(S)
    logits = (g.standard_normal((T, ld)) * 2.0).astype(np.float32)
    loss, d = dsa.dsa_indexer_kl_loss(dput(q, dev).view(torch.bfloat16), dput(kv, dev).view(torch.bfloat16),
                                      dput(logits, dev), sm, q_start=q_start)
    torch.cuda.synchronize()
    rows = np.array([0, T - 1])
    pos = q_start + rows
    lo, do = oracle.indexer_kl(q[rows], kv, pos, sm, logits[rows, :S])
    worst = parity.check_kl(dget(loss)[rows], dget(d)[rows, :S], lo, do, logits[rows, :S], pos, "kl long context")
    print("  loss worst error / bar: %.3e" % worst, flush=True)
    # backward over the same context for 16 rows (q_start leaves them 131056 .. 131071)
    Tb = 16
    q8, qs = quantize_fp8_rows(g.standard_normal((Tb, H_I, D_I)).astype(np.float32))
    k8, ks = quantize_fp8_rows(g.standard_normal((S, D_I)).astype(np.float32))
    w = (g.uniform(0.0, 1.0, (Tb, H_I)) / H_I).astype(np.float32)
    dI = (g.standard_normal((Tb, ld)) * 1e-4).astype(np.float32)
    dq, dw, dk = dsa.dsa_indexer_bwd(dput(q8, dev), dput(qs, dev), dput(w, dev), dput(k8, dev), dput(ks, dev),
                                     dput(dI, dev), q_start=S - Tb)
    torch.cuda.synchronize()
    posb = S - Tb + np.arange(Tb)
    oq, ow, ok = oracle.indexer_bwd(q8, qs, w, posb, k8, ks, dI[:, :S])
    # the dk of 1024 sampled keys and every dq / dw (the magnitude scales need the whole sum)
    amb, worst = parity.check_indexer_bwd(dget(dq), dget(dw), dget(dk), oq, ow, ok, q8, qs, w, k8, ks, dI[:, :S],
                                          posb, "bwd long context")
    print("  backward: ambiguous ReLU signs %d, worst error / bar %.3e" % (amb, worst), flush=True)
    # the listed backward over 2048-entry lists spread across the whole context (8 rows)
    Tl = 8
    posl = S - Tl + np.arange(Tl)
    idx = _distinct_lists(Tl, S, posl, 2048, 89)
    dIl = np.zeros((Tl, ld), np.float32)
    for t in range(Tl):
        keys = idx[t][(idx[t] >= 0) & (idx[t] <= posl[t])]
        dIl[t, keys] = (g.standard_normal(keys.size) * 1e-2).astype(np.float32)
    lq, lw, lk = dsa.dsa_indexer_bwd_listed(dput(q8[:Tl], dev), dput(qs[:Tl], dev), dput(w[:Tl], dev), dput(k8, dev),
                                            dput(ks, dev), dput(idx, dev), dput(dIl, dev), q_start=S - Tl)
    torch.cuda.synchronize()
    oq, ow, ok = oracle.indexer_bwd(q8[:Tl], qs[:Tl], w[:Tl], posl, k8, ks, dIl[:, :S])
    amb, worst = parity.check_indexer_bwd(dget(lq), dget(lw), dget(lk), oq, ow, ok, q8[:Tl], qs[:Tl], w[:Tl], k8, ks,
                                          dIl[:, :S], posl, "bwd listed long context")
    print("  listed backward: ambiguous ReLU signs %d, worst error / bar %.3e" % (amb, worst), flush=True)
