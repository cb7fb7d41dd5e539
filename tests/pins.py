"""Checks that pin the oracle to things other than itself.

Each check takes an oracle library handle (so the same check can be run
against deliberately broken copies of the oracle) and raises AssertionError
when the oracle disagrees with the pages' definitions, a library routine, a
closed form, an error bound or an invariant.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from dsa_inputs import get, prefill_inputs
from dsa_inputs.generate import bf16_bits_to_f32, block_rng, quantize_fp8_rows, to_bf16_bits

import brute

U = 2.0 ** -24   # unit roundoff of fp32


def indexer_bound(D_I: int, H_I: int) -> float:
    """First-order forward error bound of the fp32 oracle relative to the magnitude scale A:
    dequantization (2 roundings), products and D_I-term dot (gamma_{D_I}), weighting and
    H_I-term sum (gamma_{H_I + 1})."""
    return 1.01 * (D_I + H_I + 4) * U


# ---------------------------------------------------------------- formats
def check_e4m3_table(lib):
    t = oracle.e4m3_table(lib)
    ref = brute.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float32)
    assert np.array_equal(t, ref, equal_nan=True), "E4M3 table differs from torch.float8_e4m3fn"
    # closed forms from the format definition
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and not np.isinf(t).any()


def check_bf16_round(lib):
    g = block_rng(123, 99, 0)
    x = np.concatenate([g.standard_normal(20000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.0e38, -3.0e38, 1e-40, np.inf, -np.inf], np.float32)])
    mine = oracle.bf16_round(x, lib)
    ref = to_bf16_bits(x)
    assert np.array_equal(mine, ref), "bf16 rounding differs from torch"


# ---------------------------------------------------------------- indexer
def check_indexer_tiny(lib):
    wl = get("tiny")
    inp = prefill_inputs(wl)
    o = oracle.indexer(inp.q8, inp.qs, inp.w, inp.pos, inp.k8, inp.ks, lib=lib)
    b, A = brute.indexer(inp.q8, inp.qs, inp.w, inp.pos, inp.k8, inp.ks)
    m = ~np.isnan(b)
    assert np.array_equal(m, ~np.isnan(o)), "causal region of the oracle is wrong"
    err = np.abs(o[m] - b[m])
    assert np.all(err <= indexer_bound(wl.D_I, wl.H_I) * A[m] + 1e-30), \
        "indexer exceeds fp32 error bound (max %.3e of A)" % np.max(err / np.maximum(A[m], 1e-30))


def check_indexer_full_heads(lib, rows=(0, 1, 777, 2047, 2048, 4095)):
    wl = get("prefill_4k")
    inp = prefill_inputs(wl, rows=rows, with_q=False)
    o = oracle.indexer(inp.q8, inp.qs, inp.w, inp.pos, inp.k8, inp.ks, lib=lib)
    b, A = brute.indexer(inp.q8, inp.qs, inp.w, inp.pos, inp.k8, inp.ks)
    m = ~np.isnan(b)
    assert np.array_equal(m, ~np.isnan(o))
    assert np.all(np.abs(o[m] - b[m]) <= indexer_bound(wl.D_I, wl.H_I) * A[m])


def check_indexer_relu_matmul(lib):
    """H_I = 1, w = 1, unit scales: I = ReLU(Q K^T) (library matmul in fp64)."""
    g = block_rng(7, 1, 0)
    T, S, D = 40, 40, 64
    q8 = g.integers(0, 256, size=(T, 1, D)).astype(np.uint8)
    k8 = g.integers(0, 256, size=(S, D)).astype(np.uint8)
    q8[(q8 & 0x7F) == 0x7F] = 0x10    # no NaN codes
    k8[(k8 & 0x7F) == 0x7F] = 0x20
    ones_q = np.ones((T, 1), np.float32)
    o = oracle.indexer(q8, ones_q, ones_q, np.arange(T), k8, np.ones(S, np.float32), lib=lib)
    Q = torch.from_numpy(brute.e4m3_decode(q8[:, 0, :]))
    K = torch.from_numpy(brute.e4m3_decode(k8))
    ref = torch.relu(torch.matmul(Q, K.T)).numpy()
    tri = np.tril(np.ones((T, S), bool))
    # integer-valued products x 2^-18 summed exactly in fp64; fp32 may round the sum
    A = torch.matmul(Q.abs(), K.abs().T).numpy()
    assert np.all(np.abs(o[tri] - ref[tri]) <= (D + 2) * U * A[tri])
    assert np.all(np.isnan(o[~tri]))


def check_indexer_scale_invariants(lib):
    wl = get("tiny")
    inp = prefill_inputs(wl)
    o = oracle.indexer(inp.q8, inp.qs, inp.w, inp.pos, inp.k8, inp.ks, lib=lib)
    o2 = oracle.indexer(inp.q8, inp.qs, 2.0 * inp.w, inp.pos, inp.k8, inp.ks, lib=lib)
    m = ~np.isnan(o)
    assert np.array_equal(o2[m], 2.0 * o[m]), "doubling w must double every score exactly"
    # a negative weight is used literally (no clamping of w)
    wneg = inp.w.copy()
    wneg[:, 0] = -wneg[:, 0]
    o3 = oracle.indexer(inp.q8, inp.qs, wneg, inp.pos, inp.k8, inp.ks, lib=lib)
    b3, A3 = brute.indexer(inp.q8, inp.qs, wneg, inp.pos, inp.k8, inp.ks)
    assert np.all(np.abs(o3[m] - b3[m]) <= indexer_bound(wl.D_I, wl.H_I) * A3[m] + 1e-30)
    assert (o3[m] < 0).any()


# ---------------------------------------------------------------- top-k
def _rows_check(o, scores, pos, k):
    S = scores.shape[1]
    for t in range(scores.shape[0]):
        n = int(min(S, pos[t] + 1))
        ref = brute.topk_lexsort(scores[t], n, k)
        assert np.array_equal(o[t].astype(np.int64), ref), "top-k row %d differs from lexsort" % t


def check_topk_lexsort(lib):
    g = block_rng(11, 2, 0)
    T, S, k = 64, 300, 37
    scores = g.standard_normal((T, S)).astype(np.float32)
    pos = g.integers(0, S + 20, size=T)
    o = oracle.topk(scores, pos, k, lib=lib)
    _rows_check(o, scores, pos, k)


def check_topk_ties(lib):
    """Integer scores from {0..7}: massive ties, the lower index must win."""
    g = block_rng(12, 2, 0)
    T, S, k = 48, 257, 64
    scores = g.integers(0, 8, size=(T, S)).astype(np.float32)
    scores[:, 5] = -0.0      # -0.0 ties with +0.0
    pos = np.arange(T) * 5 + 10
    o = oracle.topk(scores, pos, k, lib=lib)
    _rows_check(o, scores, pos, k)


def check_topk_special_cases(lib):
    g = block_rng(13, 2, 0)
    T, S = 20, 50
    scores = g.standard_normal((T, S)).astype(np.float32)
    pos = np.arange(T)
    # k >= n_t: every visible key, then -1
    o = oracle.topk(scores, pos, 64, lib=lib)
    for t in range(T):
        n = t + 1
        assert sorted(o[t, :n].tolist()) == list(range(n))
        assert np.all(o[t, n:] == -1)
    # k = 1: first argmax
    pos2 = np.full(T, S - 1)
    o1 = oracle.topk(scores, pos2, 1, lib=lib)
    assert np.array_equal(o1[:, 0], np.argmax(scores, axis=1))
    # causal: nothing past the query's own position
    o3 = oracle.topk(scores, pos, 5, lib=lib)
    assert np.all(o3 <= pos[:, None])
    # -0.0 and +0.0 are equal: the lower index wins
    z = np.zeros((1, 4), np.float32)
    z[0, 0] = -0.0
    z[0, 1] = 0.0
    z[0, 2:] = -1.0
    assert oracle.topk(z, np.array([3]), 1, lib=lib)[0, 0] == 0


# ---------------------------------------------------------------- sparse MLA
def _mla_inputs(T, S, H, D_qk, seed):
    g = block_rng(seed, 3, 0)
    q = to_bf16_bits(g.standard_normal((T, H, D_qk)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((S, D_qk)).astype(np.float32))
    return q, kv


def check_mla_dense_equivalence(lib):
    """k >= n_t with every visible key listed: equals dense causal attention (torch SDPA, fp64)."""
    T = S = 64
    H, D_qk, D_v = 8, 80, 64
    sm = 1.0 / np.sqrt(80.0)
    q, kv = _mla_inputs(T, S, H, D_qk, 21)
    k = 64
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        idx[t, :t + 1] = np.arange(t + 1)[::-1]    # any order
    out, _, lse = oracle.sparse_mla(q, idx, np.arange(T), kv, D_v, sm, lib=lib)
    Q = torch.from_numpy(brute.bf16_decode(q)).permute(1, 0, 2)             # [H,T,D]
    KV = torch.from_numpy(brute.bf16_decode(kv))
    K = KV[None].expand(H, S, D_qk)
    V = KV[None, :, :D_v].expand(H, S, D_v)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=sm)
    ref = ref.permute(1, 0, 2).numpy()
    rel = np.abs(out - ref).max(axis=2) / np.abs(ref).max(axis=2)
    assert rel.max() < 2e-5, "oracle MLA differs from dense causal attention (%.2e)" % rel.max()
    z = sm * np.einsum("htd,sd->hts", Q.numpy(), KV.numpy())
    z = np.where(np.tril(np.ones((T, S), bool))[None], z, -np.inf)
    lse_ref = torch.logsumexp(torch.from_numpy(z), dim=-1).numpy().T
    assert np.abs(lse - lse_ref).max() < 2e-5


def check_mla_brute(lib):
    """Random index lists with duplicates and invalid entries vs the fp64 brute force."""
    T, S, H, D_qk, D_v = 16, 200, 8, 80, 64
    q, kv = _mla_inputs(T, S, H, D_qk, 22)
    g = block_rng(22, 4, 0)
    k = 32
    pos = g.integers(40, S, size=T)
    idx = g.integers(-3, S, size=(T, k)).astype(np.int32)
    idx[:, 3] = idx[:, 2]                            # duplicates
    out, _, lse = oracle.sparse_mla(q, idx, pos, kv, D_v, 0.125, lib=lib)
    ref, lse_ref = brute.sparse_mla(q, idx, pos, kv, D_v, 0.125)
    rel = np.abs(out - ref).max(axis=2) / np.abs(ref).max(axis=2)
    assert rel.max() < 2e-5 and np.abs(lse - lse_ref).max() < 2e-5


def check_mla_special_cases(lib):
    T, S, H, D_qk, D_v = 8, 64, 8, 80, 64
    q, kv = _mla_inputs(T, S, H, D_qk, 23)
    kvf = brute.bf16_decode(kv)
    pos = np.full(T, S - 1)
    # k = 1: output is the selected V row exactly, lse = the one logit
    idx1 = (np.arange(T) * 7 % S).astype(np.int32)[:, None]
    out, outb, lse = oracle.sparse_mla(q, idx1, pos, kv, D_v, 0.1, lib=lib)
    for t in range(T):
        assert np.array_equal(out[t], np.broadcast_to(kvf[idx1[t, 0], :D_v], (H, D_v)).astype(np.float32))
        assert np.array_equal(outb[t], np.broadcast_to(kv[idx1[t, 0], :D_v], (H, D_v)))
    z = 0.1 * np.einsum("thd,td->th", brute.bf16_decode(q), kvf[idx1[:, 0]])
    assert np.abs(lse - z).max() < 1e-5
    # q = 0: uniform weights, output is the mean of the selected V rows, lse = log(count)
    q0 = np.zeros_like(q)
    idx = np.stack([np.arange(10) * 3 + t for t in range(T)]).astype(np.int32)
    out0, _, lse0 = oracle.sparse_mla(q0, idx, pos, kv, D_v, 0.3, lib=lib)
    for t in range(T):
        mean = kvf[idx[t], :D_v].mean(axis=0)
        assert np.abs(out0[t] - mean[None]).max() <= 16 * U * np.abs(kvf[idx[t], :D_v]).max() * 10
    assert np.abs(lse0 - np.log(10.0)).max() < 1e-6
    # invalid entries are skipped exactly; an all-invalid row gives 0 and -inf
    idx2 = np.concatenate([idx, np.full((T, 3), -1, np.int32), np.full((T, 2), S + 5, np.int32)], axis=1)
    outa, _, lsea = oracle.sparse_mla(q, idx, pos, kv, D_v, 0.3, lib=lib)
    outb2, _, lseb = oracle.sparse_mla(q, idx2, pos, kv, D_v, 0.3, lib=lib)
    assert np.array_equal(outa, outb2) and np.array_equal(lsea, lseb)
    # keys beyond the query position are invalid too
    posn = np.full(T, 5)
    outc, _, lsec = oracle.sparse_mla(q, idx, posn, kv, D_v, 0.3, lib=lib)
    keep = np.where((idx >= 0) & (idx <= 5), idx, -1).astype(np.int32)
    outd, _, lsed = oracle.sparse_mla(q, keep, pos, kv, D_v, 0.3, lib=lib)
    assert np.array_equal(outc, outd) and np.array_equal(lsec, lsed)
    none = np.full((T, 4), -1, np.int32)
    oute, _, lsee = oracle.sparse_mla(q, none, pos, kv, D_v, 0.3, lib=lib)
    assert np.all(oute == 0) and np.all(np.isneginf(lsee))
    # index order does not change the result beyond fp32 rounding
    perm = idx[:, ::-1].copy()
    outp, _, lsep = oracle.sparse_mla(q, perm, pos, kv, D_v, 0.3, lib=lib)
    assert np.abs(outp - outa).max() < 1e-5 and np.abs(lsep - lsea).max() < 1e-5


# ---------------------------------------------------------------- end to end
def check_dense_when_k_covers(lib, rows=(0, 1, 5, 1000, 2047)):
    """Invariant: when k >= n_t, sparse attention equals dense causal MLA."""
    wl = get("prefill_4k")
    inp = prefill_inputs(wl, rows=rows)
    logits, idx, out, _, lse = oracle.prefill(inp, lib=lib)
    Q = brute.bf16_decode(inp.q)
    KV = brute.bf16_decode(inp.kv)
    for r, t in enumerate(rows):
        n = t + 1
        assert sorted(idx[r][:n].tolist()) == list(range(n)) and np.all(idx[r][n:] == -1)
        z = wl.sm_scale * (Q[r] @ KV[:n].T)
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        ref = (e @ KV[:n, :wl.D_v]) / e.sum(axis=1, keepdims=True)
        rel = np.abs(out[r] - ref).max(axis=1) / np.abs(ref).max(axis=1)
        assert rel.max() < 1e-4


def check_causal_end_to_end(lib):
    wl = get("tiny")
    inp = prefill_inputs(wl)
    logits, idx, out, _, lse = oracle.prefill(inp, lib=lib)
    pos = inp.pos
    assert np.all(idx <= pos[:, None])
    for t in range(wl.T):
        n = t + 1
        v = idx[t][idx[t] >= 0]
        assert len(v) == min(n, wl.topk) and len(set(v.tolist())) == len(v)


# ---------------------------------------------------------------- FP8 quantize + paged append
FP8_MAX = 448.0


def _torch_e4m3(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def check_e4m3_encode_round_trip(lib):
    t = oracle.e4m3_table(lib)
    codes = np.arange(256, dtype=np.uint8)
    fin = ~np.isnan(t)
    assert fin.sum() == 254                      # 0x7F and 0xFF are NaN
    assert np.array_equal(oracle.e4m3_encode(t[fin], lib), codes[fin]), "E4M3 encode does not invert decode"


def check_e4m3_encode_midpoints(lib):
    t = oracle.e4m3_table(lib).astype(np.float64)
    lo = np.arange(0, 0x7E)
    mid = ((t[lo] + t[lo + 1]) / 2).astype(np.float32)      # exact: at most 5 significant bits
    assert np.array_equal(mid.astype(np.float64), (t[lo] + t[lo + 1]) / 2)
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(oracle.e4m3_encode(mid, lib), even), "halfway values must take the even code"
    assert np.array_equal(oracle.e4m3_encode(-mid, lib), even | 0x80)
    above = np.nextafter(mid, np.float32(np.inf))
    below = np.nextafter(mid, np.float32(0))
    assert np.array_equal(oracle.e4m3_encode(above, lib), (lo + 1).astype(np.uint8))
    assert np.array_equal(oracle.e4m3_encode(below[1:], lib), lo[1:].astype(np.uint8))
    assert oracle.e4m3_encode(np.array([0.0, -0.0], np.float32), lib).tolist() == [0x00, 0x80]


def check_e4m3_encode_vs_torch(lib):
    g = block_rng(50, 0, 0)
    u = g.uniform(-FP8_MAX, FP8_MAX, 200_000).astype(np.float32)
    small = (g.choice([-1.0, 1.0], 100_000) * np.exp2(g.uniform(-12, 2, 100_000))).astype(np.float32)
    t = oracle.e4m3_table(lib).astype(np.float64)
    lo = np.arange(0, 0x7E)
    mids = ((t[lo] + t[lo + 1]) / 2).astype(np.float32)
    y = np.concatenate([u, small, mids, -mids, np.float32([FP8_MAX, -FP8_MAX, 0.0])])
    assert np.array_equal(oracle.e4m3_encode(y, lib), _torch_e4m3(y)), "E4M3 encode differs from torch's cast"


def check_quantize_rows_closed_forms(lib):
    x = np.zeros((3, 128), np.float32)
    x[1, 5] = -3.0
    x[1, 7] = 1.5
    x[2] = np.linspace(-2, 7, 128)
    codes, scales = oracle.quantize_rows(to_bf16_bits(x), lib)
    assert scales[0] == 1.0 and not codes[0].any()                       # all-zero row
    assert scales[1] == np.float32(3.0) / np.float32(FP8_MAX)
    assert codes[1, 5] == 0xFE and codes[1, 7] == _torch_e4m3(np.float32([224.0]))[0]
    assert codes[2, 127] == 0x7E and (codes[2] & 0x7F).max() == 0x7E   # the row maximum codes 448
    dec = oracle.e4m3_table(lib)[codes[2]].astype(np.float64) * scales[2]
    xb = bf16_bits_to_f32(to_bf16_bits(x[2])).astype(np.float64)
    # E4M3 keeps 4 significant bits: within 2^-4 relative (normal range) or half a subnormal step
    assert np.all(np.abs(dec - xb) <= np.maximum(np.abs(xb) * 2.0 ** -4, 2.0 ** -10 * scales[2]))


def check_quantize_rows_vs_generator(lib):
    # the input generator quantizes the same definition through torch (fp32 division, RNE cast)
    g = block_rng(51, 0, 0)
    x = (g.standard_normal((257, 128)) * np.exp2(g.uniform(-6, 6, (257, 1)))).astype(np.float32)
    x[3] = 0.0
    x[4, :7] = 1e-30
    bits = to_bf16_bits(x)
    xv = bf16_bits_to_f32(bits)
    codes, scales = oracle.quantize_rows(bits, lib)
    gc, gs = quantize_fp8_rows(xv)
    assert np.array_equal(scales, gs), "row scales differ from amax / 448"
    assert np.array_equal(codes, gc), "row codes differ from the torch quantizer"


def check_append_paged_round_trip(lib, bs=16):
    g = block_rng(52, 0, bs)
    D_I, D_qk, NB = 64, 80, 12
    k8 = g.integers(0, 255, (NB, bs, D_I), dtype=np.uint8)
    ks = g.uniform(0.1, 1.0, (NB, bs)).astype(np.float32)
    kv = g.integers(0, 65535, (NB, bs, D_qk), dtype=np.uint16)
    table = np.array([[3, 7, 1, -1], [0, 11, -1, -1]], np.int32)
    seq = np.array([0, 0, 0, 1, 1], np.int32)
    pos = np.array([0, bs + 2, 3 * bs - 1, 1, 2 * bs - 1], np.int32)
    kn = to_bf16_bits(g.standard_normal((5, D_I)).astype(np.float32))
    vn = g.integers(0, 65535, (5, D_qk), dtype=np.uint16)
    k8n, ksn, kvn = oracle.append_paged(k8, ks, kv, table, seq, pos, kn, vn, lib)
    qc, qsc = oracle.quantize_rows(kn, lib)
    written = np.zeros((NB, bs), bool)
    for i in range(5):
        written[table[seq[i], pos[i] // bs], pos[i] % bs] = True
        # through the paged gather: logical row pos[i] of sequence seq[i]
        n = int(pos[i]) + 1
        assert np.array_equal(oracle.gather_rows(k8n, table[seq[i]], n, lib)[-1], qc[i]), "appended codes misplaced"
        assert oracle.gather_rows(ksn[..., None], table[seq[i]], n, lib)[-1, 0] == qsc[i]
        assert np.array_equal(oracle.gather_rows(kvn, table[seq[i]], n, lib)[-1], vn[i]), "appended row misplaced"
    assert np.array_equal(k8n[~written], k8[~written]), "append touched other slots"
    assert np.array_equal(ksn[~written], ks[~written])
    assert np.array_equal(kvn[~written], kv[~written])


def check_quantize_ue8m0(lib):
    # UE8M0 reading: s = 2^p, the smallest power of two >= amax / 448 (p >= -127); codes as the
    # plain quantizer with that scale.  Pinned to the closed form in float64 and torch's cast.
    g = block_rng(53, 0, 0)
    x = (g.standard_normal((300, 128)) * np.exp2(g.uniform(-30, 30, (300, 1)))).astype(np.float32)
    x[0] = 0.0
    x[1] = 0.0
    x[1, 3] = 448.0 * 2.0 ** -5          # amax / 448 exactly a power of two
    x[2] = 0.0
    x[2, 9] = -7.0                       # 7 / 448 = 2^-6 exactly
    x[3] = np.float32(1e-38) * g.standard_normal(128).astype(np.float32)   # p clamps to -127
    bits = to_bf16_bits(x)
    xv = bf16_bits_to_f32(bits)
    codes, exps, scales = oracle.quantize_rows_ue8m0(bits, lib)
    amax = np.abs(xv).max(axis=1)
    t = np.where(amax > 0, (amax / np.float32(FP8_MAX)).astype(np.float32), np.float32(1.0)).astype(np.float64)
    p = np.maximum(np.ceil(np.log2(t)), -127).astype(np.int64)
    assert np.array_equal(exps.astype(np.int64), p + 127), "E8M0 exponent is not ceil(log2(amax / 448))"
    assert np.array_equal(scales.astype(np.float64), np.exp2(p.astype(np.float64))), "scale is not 2^p"
    assert scales[1] == 2.0 ** -5 and scales[2] == 2.0 ** -6 and exps[0] == 127
    y = np.clip(xv.astype(np.float64) / scales[:, None].astype(np.float64), -FP8_MAX, FP8_MAX).astype(np.float32)
    assert np.array_equal(codes, _torch_e4m3(y)), "UE8M0 codes differ from the torch cast of x / 2^p"
    assert np.all((codes & 0x7F) <= 0x7E)


# ---------------------------------------------------------------- indexer training signal
# Reading (DeepSeek-V3.2-Exp summary page, "Method", dense warm-up): the row loss is
# KL(p || softmax(I)) with p the main attention's distribution averaged over the heads; the
# backward passes the FP8 quantization straight through.
def _kl_inputs(T, S, q_start, H, D, seed, scale=2.0):
    g = block_rng(seed, T, S)
    q = to_bf16_bits(g.standard_normal((T, H, D)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((S, D)).astype(np.float32))
    logits = (g.standard_normal((T, S)) * scale).astype(np.float32)
    return q, kv, logits, q_start + np.arange(T)


def torch_kl(q, kv, logits, pos, sm):
    """(loss [T], dI [T, S]) by torch in float64: per-head softmax over the visible keys, mean over
    heads, F.kl_div against log_softmax of the scores, gradient by autograd."""
    qf = torch.from_numpy(brute.bf16_decode(q))
    kf = torch.from_numpy(brute.bf16_decode(kv))
    T, S = logits.shape
    vis = torch.from_numpy(np.arange(S)[None, :] < np.minimum(S, pos + 1)[:, None])
    z = torch.matmul(qf, kf.T) * sm                                    # [T, H, S]
    p = torch.softmax(z.masked_fill(~vis[:, None, :], float("-inf")), dim=-1).mean(dim=1)
    I = torch.from_numpy(logits.astype(np.float64)).requires_grad_(True)
    logpi = torch.log_softmax(I.masked_fill(~vis, float("-inf")), dim=-1).masked_fill(~vis, 0.0)
    loss = torch.nn.functional.kl_div(logpi, p, reduction="none").sum(dim=-1)
    loss.sum().backward()
    return loss.detach().numpy(), np.where(vis.numpy(), I.grad.numpy(), np.nan)


def check_kl_vs_torch(lib):
    for (T, S, q0, H, D, sm) in [(24, 40, 16, 4, 24, 0.3), (9, 9, 0, 3, 80, 80 ** -0.5)]:
        q, kv, logits, pos = _kl_inputs(T, S, q0, H, D, 71)
        loss, d = oracle.indexer_kl(q, kv, pos, sm, logits, lib=lib)
        tl, td = torch_kl(q, kv, logits, pos, sm)
        assert np.all(np.abs(loss - tl) <= 1e-12 * (1.0 + np.abs(tl))), "KL loss differs from torch kl_div"
        m = ~np.isnan(td)
        assert np.array_equal(m, ~np.isnan(d)), "visible region of dI is wrong"
        assert np.max(np.abs(d[m] - td[m])) <= 1e-13, "dI differs from torch autograd"
        assert np.all(loss >= -1e-15), "KL divergence must be non-negative"


def check_kl_closed_forms(lib):
    # a row that sees one key: both distributions are that key
    q, kv, logits, pos = _kl_inputs(3, 8, 0, 2, 16, 72)
    loss, d = oracle.indexer_kl(q, kv, pos, 0.25, logits, lib=lib)
    assert loss[0] == 0.0 and d[0, 0] == 0.0
    # identical heads and scores equal to that head's attention logits (+ a constant): pi = p
    T, S, H, D, sm = 6, 20, 3, 16, 0.25
    q, kv, _, pos = _kl_inputs(T, S, 14, H, D, 73)
    q[:, 1:] = q[:, :1]
    z = brute.bf16_decode(q)[:, 0] @ brute.bf16_decode(kv).T * sm
    loss, d = oracle.indexer_kl(q, kv, pos, sm, (z + 1.5).astype(np.float32), lib=lib)
    assert np.all(loss <= 1e-10) and np.nanmax(np.abs(d)) <= 1e-5, "pi = p must give zero loss"
    # uniform scores: loss = log n + sum p log p, with p = 1/n - dI
    q, kv, _, pos = _kl_inputs(T, S, 14, H, D, 74)
    loss, d = oracle.indexer_kl(q, kv, pos, sm, np.full((T, S), 0.37, np.float32), lib=lib)
    for t in range(T):
        n = min(S, pos[t] + 1)
        p = 1.0 / n - d[t, :n]
        assert abs(p.sum() - 1.0) <= 1e-12
        assert abs(loss[t] - (np.log(n) + np.sum(p * np.log(p)))) <= 1e-12
    # two sharp heads on two different keys: p = 1/2 on each (head average, not a sum or a max)
    S = 10
    q = to_bf16_bits(np.array([[[60.0, 0.0], [0.0, 60.0]]], np.float32))
    kvf = np.zeros((S, 2), np.float32)
    kvf[3] = [1.0, 0.0]
    kvf[7] = [0.0, 1.0]
    logits = block_rng(75, 0, 0).standard_normal((1, S)).astype(np.float32)
    loss, d = oracle.indexer_kl(q, to_bf16_bits(kvf), np.array([S - 1]), 1.0, logits, lib=lib)
    lp = logits[0].astype(np.float64) - np.log(np.sum(np.exp(logits[0].astype(np.float64))))
    ref = 0.5 * (np.log(0.5) - lp[3]) + 0.5 * (np.log(0.5) - lp[7])
    assert abs(loss[0] - ref) <= 1e-12
    pi = np.exp(lp)
    assert abs(d[0, 3] - (pi[3] - 0.5)) <= 1e-12 and abs(d[0, 0] - pi[0]) <= 1e-12


def check_kl_finite_difference(lib):
    # dI against central differences of the oracle's own loss (the exact perturbation of the fp32
    # score is used)
    q, kv, logits, pos = _kl_inputs(4, 30, 26, 2, 16, 76)
    sm = 0.3
    _, d = oracle.indexer_kl(q, kv, pos, sm, logits, lib=lib)
    for (t, s) in [(0, 0), (1, 5), (2, 28), (3, 29), (3, 11)]:
        up, dn = logits.copy(), logits.copy()
        up[t, s] = np.float32(logits[t, s] + np.float32(2.0 ** -9))
        dn[t, s] = np.float32(logits[t, s] - np.float32(2.0 ** -9))
        lu, _ = oracle.indexer_kl(q, kv, pos, sm, up, lib=lib)
        ld_, _ = oracle.indexer_kl(q, kv, pos, sm, dn, lib=lib)
        fd = (lu[t] - ld_[t]) / (float(up[t, s]) - float(dn[t, s]))
        assert abs(fd - d[t, s]) <= 1e-5, "dI[%d,%d] differs from the finite difference" % (t, s)


def _bwd_inputs(T, S, q_start, H_I, D_I, seed):
    g = block_rng(seed, T, S)
    q8, qs = quantize_fp8_rows(g.standard_normal((T, H_I, D_I)).astype(np.float32))
    k8, ks = quantize_fp8_rows(g.standard_normal((S, D_I)).astype(np.float32))
    w = (g.uniform(-1.0, 1.0, (T, H_I)) / H_I).astype(np.float32)      # any sign (weights are literal)
    dI = (g.standard_normal((T, S)) * 1e-2).astype(np.float32)
    return q8, qs, w, k8, ks, dI, q_start + np.arange(T)


def _indexer_linear_form(qd, kd, w, dI, pos):
    """L = sum over visible (t, s) of dI[t,s] I[t,s], in float64 from dequantized inputs."""
    T, S = dI.shape
    z = np.einsum("tjd,sd->tjs", qd, kd)
    I = np.einsum("tj,tjs->ts", w.astype(np.float64), np.maximum(z, 0.0))
    vis = np.arange(S)[None, :] < np.minimum(S, pos + 1)[:, None]
    return float(np.sum(np.where(vis, dI.astype(np.float64) * I, 0.0)))


def check_indexer_bwd_vs_torch(lib):
    T, S, H_I, D_I = 20, 36, 4, 32
    q8, qs, w, k8, ks, dI, pos = _bwd_inputs(T, S, 16, H_I, D_I, 77)
    dq, dw, dk = oracle.indexer_bwd(q8, qs, w, pos, k8, ks, dI, lib=lib)
    qd = torch.from_numpy(qs.astype(np.float64)[:, :, None] * brute.e4m3_decode(q8)).requires_grad_(True)
    kd = torch.from_numpy(ks.astype(np.float64)[:, None] * brute.e4m3_decode(k8)).requires_grad_(True)
    wt = torch.from_numpy(w.astype(np.float64)).requires_grad_(True)
    vis = torch.from_numpy(np.arange(S)[None, :] < np.minimum(S, pos + 1)[:, None])
    I = (wt[:, :, None] * torch.relu(torch.matmul(qd, kd.T))).sum(dim=1)
    (torch.from_numpy(dI.astype(np.float64)) * I).masked_fill(~vis, 0.0).sum().backward()
    for name, mine, ref in [("dq", dq, qd.grad.numpy()), ("dw", dw, wt.grad.numpy()), ("dk", dk, kd.grad.numpy())]:
        assert np.max(np.abs(mine - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref))), "%s differs from autograd" % name


def check_indexer_bwd_finite_difference(lib):
    # I is linear in each row scale qs[t,j], key scale ks[s] and weight w[t,j] (positive scales do
    # not move the ReLU kink), so central differences of L = sum dI * I are exact up to rounding
    # and fix the projections dq[t,j] . dec(q8[t,j]), dk[s] . dec(k8[s]) and dw[t,j]
    T, S, H_I, D_I = 10, 16, 3, 16
    q8, qs, w, k8, ks, dI, pos = _bwd_inputs(T, S, 6, H_I, D_I, 78)
    dq, dw, dk = oracle.indexer_bwd(q8, qs, w, pos, k8, ks, dI, lib=lib)
    qdec, kdec = brute.e4m3_decode(q8), brute.e4m3_decode(k8)

    def L(qs_, ks_, w_):
        return _indexer_linear_form(qs_.astype(np.float64)[:, :, None] * qdec,
                                    ks_.astype(np.float64)[:, None] * kdec, w_, dI, pos)
    h = 1e-3
    for (t, j) in [(0, 0), (4, 2), (9, 1)]:
        a, b = qs.astype(np.float64).copy(), qs.astype(np.float64).copy()
        a[t, j] += h
        b[t, j] -= h
        fd = (L(a, ks, w) - L(b, ks, w)) / (2 * h)
        assert abs(fd - np.dot(dq[t, j], qdec[t, j])) <= 1e-9 * (1.0 + abs(fd)), "dq projection"
        a, b = w.astype(np.float64).copy(), w.astype(np.float64).copy()
        a[t, j] += h
        b[t, j] -= h
        fd = (L(qs, ks, a) - L(qs, ks, b)) / (2 * h)
        assert abs(fd - dw[t, j]) <= 1e-9 * (1.0 + abs(fd)), "dw"
    for s in [0, 7, 15]:
        a, b = ks.astype(np.float64).copy(), ks.astype(np.float64).copy()
        a[s] += h
        b[s] -= h
        fd = (L(qs, a, w) - L(qs, b, w)) / (2 * h)
        assert abs(fd - np.dot(dk[s], kdec[s])) <= 1e-9 * (1.0 + abs(fd)), "dk projection"


# Sparse stage (reading: the loss restricted to each row's index-list entries).
def torch_kl_sparse(q, kv, logits, pos, sm, idx):
    """(loss [T], dI [T, S]) by torch in float64 over the valid entries of idx (rows with at least
    one valid entry): gathered scores, per-head softmax over the entries, head mean, kl_div against
    log_softmax of the gathered scores, autograd through the gather (repeated keys accumulate)."""
    qf = torch.from_numpy(brute.bf16_decode(q))
    kf = torch.from_numpy(brute.bf16_decode(kv))
    T, S = logits.shape
    n = np.minimum(S, pos + 1)
    valid = torch.from_numpy((idx >= 0) & (idx < n[:, None]))
    ic = torch.from_numpy(np.where(idx >= 0, np.minimum(idx, S - 1), 0).astype(np.int64))
    z = torch.einsum("thd,tkd->thk", qf, kf[ic]) * sm
    p = torch.softmax(z.masked_fill(~valid[:, None, :], float("-inf")), dim=-1).mean(dim=1)
    I = torch.from_numpy(logits.astype(np.float64)).requires_grad_(True)
    g = torch.gather(I, 1, ic).masked_fill(~valid, float("-inf"))
    logpi = torch.log_softmax(g, dim=-1).masked_fill(~valid, 0.0)
    loss = torch.nn.functional.kl_div(logpi, p, reduction="none").sum(dim=-1)
    loss.sum().backward()
    vis = np.arange(S)[None, :] < n[:, None]
    return loss.detach().numpy(), np.where(vis, I.grad.numpy(), np.nan)


def _sparse_lists(T, S, pos, k, seed):
    g = block_rng(seed, T, k)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = min(S, pos[t] + 1)
        m = min(n, k)
        idx[t, :m] = g.permutation(n)[:m]
        if m > 3:
            idx[t, 1] = idx[t, 0]               # a repeated key
            idx[t, 2] = n + 5                   # beyond the causal range: skipped
    return idx


def check_kl_sparse_vs_torch(lib):
    T, S, q0, H, D, sm, k = 12, 40, 20, 3, 24, 0.3, 16
    q, kv, logits, pos = _kl_inputs(T, S, q0, H, D, 91)
    idx = _sparse_lists(T, S, pos, k, 92)
    loss, d = oracle.indexer_kl_sparse(q, kv, pos, sm, idx, logits, lib=lib)
    tl, td = torch_kl_sparse(q, kv, logits, pos, sm, idx)
    assert np.all(np.abs(loss - tl) <= 1e-12 * (1.0 + np.abs(tl))), "sparse KL loss differs from torch"
    m = ~np.isnan(td)
    assert np.array_equal(m, ~np.isnan(d)), "visible region of the sparse dI is wrong"
    assert np.max(np.abs(d[m] - td[m])) <= 1e-13, "sparse dI differs from torch autograd"
    for t in range(T):                          # keys not listed get exactly 0
        listed = set(int(x) for x in idx[t] if 0 <= x < min(S, pos[t] + 1))
        for s in range(min(S, pos[t] + 1)):
            if s not in listed:
                assert d[t, s] == 0.0


def check_kl_sparse_closed_forms(lib):
    T, S, q0, H, D, sm = 8, 30, 22, 4, 16, 0.25
    q, kv, logits, pos = _kl_inputs(T, S, q0, H, D, 93)
    # every visible key listed once (any order, -1 padding): the dense loss
    k = 40
    g = block_rng(94, 0, 0)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = min(S, pos[t] + 1)
        idx[t, :n] = g.permutation(n)
    ls, ds = oracle.indexer_kl_sparse(q, kv, pos, sm, idx, logits, lib=lib)
    ld_, dd = oracle.indexer_kl(q, kv, pos, sm, logits, lib=lib)
    assert np.all(np.abs(ls - ld_) <= 1e-12 * (1 + np.abs(ld_))), "full list must give the dense loss"
    m = ~np.isnan(dd)
    assert np.max(np.abs(ds[m] - dd[m])) <= 1e-14
    # no valid entry: 0; one valid entry: 0
    idx = np.full((T, 4), -1, np.int32)
    idx[1, 2] = 5
    ls, ds = oracle.indexer_kl_sparse(q, kv, pos, sm, idx, logits, lib=lib)
    assert ls[0] == 0.0 and np.all(ds[0][~np.isnan(ds[0])] == 0.0)
    assert ls[1] == 0.0 and ds[1, 5] == 0.0
    # a key listed twice next to another with the same row: p = 1/3 per entry
    kvf = np.zeros((S, D), np.float32)
    kvf[3] = kvf[9] = 1.0
    idx = np.array([[3, 3, 9, -1]] * T, np.int32)
    ls, ds = oracle.indexer_kl_sparse(q, to_bf16_bits(kvf), pos, sm, idx, logits, lib=lib)
    for t in range(T):
        a, b = float(logits[t, 3]), float(logits[t, 9])
        zt = 2 * np.exp(a) + np.exp(b)
        pa, pb = np.exp(a) / zt, np.exp(b) / zt
        ref = 2 * (1 / 3) * (np.log(1 / 3) - np.log(pa)) + (1 / 3) * (np.log(1 / 3) - np.log(pb))
        assert abs(ls[t] - ref) <= 1e-12
        assert abs(ds[t, 3] - 2 * (pa - 1 / 3)) <= 1e-12 and abs(ds[t, 9] - (pb - 1 / 3)) <= 1e-12


# ---------------------------------------------------------------- sparse MLA backward
def _mla_bwd_case(T, S, H, D_qk, D_v, k, seed, dup=True):
    """Inputs with duplicates, entries past the causal range and -1 padding in the lists."""
    g = block_rng(seed, 5, 0)
    q = to_bf16_bits(g.standard_normal((T, H, D_qk)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((S, D_qk)).astype(np.float32))
    dout = to_bf16_bits(g.standard_normal((T, H, D_v)).astype(np.float32))
    pos = g.integers(k // 2, S, size=T).astype(np.int64)
    idx = g.integers(-2, S, size=(T, k)).astype(np.int32)
    if dup:
        idx[:, 1] = idx[:, 0]
        idx[:, 5] = idx[:, 4]
    idx[:, -1] = -1
    return q, kv, dout, pos, idx


def torch_mla_bwd(q, kv, dout, pos, idx, D_v, sm):
    """(dq, dkv) by torch autograd in float64 through the gather of each row's valid entries."""
    qf = torch.from_numpy(brute.bf16_decode(q)).requires_grad_(True)
    kvf = torch.from_numpy(brute.bf16_decode(kv)).requires_grad_(True)
    gf = torch.from_numpy(brute.bf16_decode(dout))
    S = kvf.shape[0]
    n = np.minimum(S, pos + 1)
    total = 0.0
    for t in range(q.shape[0]):
        sel = [int(s) for s in idx[t] if 0 <= s < n[t]]
        if not sel:
            continue
        K = kvf[torch.tensor(sel)]                              # [m, D_qk], repeated rows allowed
        p = torch.softmax(sm * qf[t] @ K.T, dim=-1)             # [H, m]
        total = total + (p @ K[:, :D_v] * gf[t]).sum()
    if isinstance(total, torch.Tensor):
        total.backward()
    dq = qf.grad.numpy() if qf.grad is not None else np.zeros(qf.shape)
    dkv = kvf.grad.numpy() if kvf.grad is not None else np.zeros(kvf.shape)
    return dq, dkv


def check_mla_bwd_vs_torch(lib):
    T, S, H, D_qk, D_v, k, sm = 6, 50, 3, 24, 16, 20, 0.3
    q, kv, dout, pos, idx = _mla_bwd_case(T, S, H, D_qk, D_v, k, 95)
    dq, dkv = oracle.sparse_mla_bwd(q, idx, pos, kv, D_v, sm, dout, lib=lib)
    tq, tkv = torch_mla_bwd(q, kv, dout, pos, idx, D_v, sm)
    assert np.max(np.abs(dq - tq)) <= 1e-12 * (1 + np.abs(tq).max()), "sparse MLA dq differs from torch autograd"
    assert np.max(np.abs(dkv - tkv)) <= 1e-12 * (1 + np.abs(tkv).max()), "sparse MLA dkv differs from torch autograd"


def _mla_loss_f64(qd, kvd, gd, pos, idx, D_v, sm):
    """L = sum_{t,h} g[t,h] . out[t,h] of the forward's definition, float64 inputs."""
    S = kvd.shape[0]
    n = np.minimum(S, pos + 1)
    L = 0.0
    for t in range(qd.shape[0]):
        sel = [int(s) for s in idx[t] if 0 <= s < n[t]]
        if not sel:
            continue
        K = kvd[sel]
        z = sm * qd[t] @ K.T
        e = np.exp(z - z.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        L += float(np.sum((p @ K[:, :D_v]) * gd[t]))
    return L


def check_mla_bwd_finite_difference(lib):
    """Central differences of L = sum g . out along single coordinates of q and of listed kv rows."""
    T, S, H, D_qk, D_v, k, sm = 4, 30, 2, 12, 8, 10, 0.4
    q, kv, dout, pos, idx = _mla_bwd_case(T, S, H, D_qk, D_v, k, 96)
    dq, dkv = oracle.sparse_mla_bwd(q, idx, pos, kv, D_v, sm, dout, lib=lib)
    qd, kvd, gd = brute.bf16_decode(q), brute.bf16_decode(kv), brute.bf16_decode(dout)
    h = 1e-6
    g = block_rng(97, 0, 0)
    for _ in range(12):
        t, hh, d = int(g.integers(T)), int(g.integers(H)), int(g.integers(D_qk))
        a, b = qd.copy(), qd.copy()
        a[t, hh, d] += h
        b[t, hh, d] -= h
        fd = (_mla_loss_f64(a, kvd, gd, pos, idx, D_v, sm) - _mla_loss_f64(b, kvd, gd, pos, idx, D_v, sm)) / (2 * h)
        assert abs(fd - dq[t, hh, d]) <= 1e-6 * (1 + abs(fd)), "dq vs central difference"
    listed = sorted(set(int(s) for t in range(T) for s in idx[t] if 0 <= s <= pos[t]))
    for _ in range(12):
        s, d = listed[int(g.integers(len(listed)))], int(g.integers(D_qk))
        a, b = kvd.copy(), kvd.copy()
        a[s, d] += h
        b[s, d] -= h
        fd = (_mla_loss_f64(qd, a, gd, pos, idx, D_v, sm) - _mla_loss_f64(qd, b, gd, pos, idx, D_v, sm)) / (2 * h)
        assert abs(fd - dkv[s, d]) <= 1e-6 * (1 + abs(fd)), "dkv vs central difference"


def check_mla_bwd_dense_equivalence(lib):
    """Every visible key listed once (k >= n_t): the gradients of dense causal attention, torch SDPA
    autograd in float64 with K = kv and V = kv[:, :D_v] shared by every head."""
    T = S = 24
    H, D_qk, D_v, sm = 4, 20, 16, 1.0 / np.sqrt(20.0)
    g = block_rng(98, 0, 0)
    q = to_bf16_bits(g.standard_normal((T, H, D_qk)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((S, D_qk)).astype(np.float32))
    dout = to_bf16_bits(g.standard_normal((T, H, D_v)).astype(np.float32))
    idx = np.full((T, S), -1, np.int32)
    for t in range(T):
        idx[t, :t + 1] = g.permutation(t + 1)
    dq, dkv = oracle.sparse_mla_bwd(q, idx, np.arange(T), kv, D_v, sm, dout, lib=lib)
    Q = torch.from_numpy(brute.bf16_decode(q)).permute(1, 0, 2).contiguous().requires_grad_(True)   # [H,T,D]
    KV = torch.from_numpy(brute.bf16_decode(kv)).requires_grad_(True)
    out = torch.nn.functional.scaled_dot_product_attention(Q, KV[None].expand(H, S, D_qk),
                                                           KV[None, :, :D_v].expand(H, S, D_v),
                                                           is_causal=True, scale=sm)
    (out * torch.from_numpy(brute.bf16_decode(dout)).permute(1, 0, 2)).sum().backward()
    assert np.max(np.abs(dq - Q.grad.permute(1, 0, 2).numpy())) <= 1e-12, "dq differs from dense attention"
    assert np.max(np.abs(dkv - KV.grad.numpy())) <= 1e-12, "dkv differs from dense attention"


def check_mla_bwd_closed_forms(lib):
    T, S, H, D_qk, D_v = 5, 40, 3, 16, 8
    g = block_rng(99, 0, 0)
    q = to_bf16_bits(g.standard_normal((T, H, D_qk)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((S, D_qk)).astype(np.float32))
    dout = to_bf16_bits(g.standard_normal((T, H, D_v)).astype(np.float32))
    gd, qd = brute.bf16_decode(dout), brute.bf16_decode(q)
    pos = np.full(T, S - 1)
    # one valid entry: p = 1, ds = 0, so dq = 0 and the key gets sum_h g in its value columns
    idx1 = np.array([[3 * t + 1, -1, S + 2] for t in range(T)], np.int32)
    dq, dkv = oracle.sparse_mla_bwd(q, idx1, pos, kv, D_v, 0.2, dout, lib=lib)
    assert np.all(dq == 0.0)
    ref = np.zeros((S, D_qk))
    for t in range(T):
        ref[3 * t + 1, :D_v] += gd[t].sum(axis=0)
    assert np.max(np.abs(dkv - ref)) <= 1e-12
    # q = 0: uniform p over the m entries, the key columns of dkv get nothing (ds q = 0), each
    # entry's value columns get sum_h g / m
    m = 7
    idx = np.stack([np.arange(m) * 5 + t for t in range(T)]).astype(np.int32)
    dq0, dkv0 = oracle.sparse_mla_bwd(np.zeros_like(q), idx, pos, kv, D_v, 0.2, dout, lib=lib)
    ref = np.zeros((S, D_qk))
    for t in range(T):
        for s in idx[t]:
            ref[s, :D_v] += gd[t].sum(axis=0) / m
    assert np.max(np.abs(dkv0 - ref)) <= 1e-12
    # the softmax gradient sums to zero over a row's entries: summed over all keys, the columns past
    # D_v vanish and the value columns add up to sum_{t,h} g (rows with a valid entry)
    q_, kv_, dout_, pos_, idx_ = _mla_bwd_case(8, 60, 4, 24, 16, 24, 100)
    dq_, dkv_ = oracle.sparse_mla_bwd(q_, idx_, pos_, kv_, 16, 0.3, dout_, lib=lib)
    has = np.array([np.any((r >= 0) & (r <= p)) for r, p in zip(idx_, pos_)])
    assert np.abs(dkv_[:, 16:].sum(axis=0)).max() <= 1e-10
    assert np.abs(dkv_[:, :16].sum(axis=0) - brute.bf16_decode(dout_)[has].sum(axis=(0, 1))).max() <= 1e-10
    # rows without a valid entry: dq = 0 and no contribution
    none = np.full((T, 3), -1, np.int32)
    dqn, dkvn = oracle.sparse_mla_bwd(q, none, pos, kv, D_v, 0.2, dout, lib=lib)
    assert np.all(dqn == 0.0) and np.all(dkvn == 0.0)
    del qd
