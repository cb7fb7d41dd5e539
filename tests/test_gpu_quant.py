"""On-device FP8 quantization and paged append vs the oracle, bit for bit (needs an MI355X)."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import decode_inputs, get, to_bf16_bits
from dsa_inputs.generate import block_rng
from gpu_helpers import bf16_vals, dget, dims_of, dput

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_02_amd as dsa
    dsa.load()
    return torch.device("cuda:0")


def _rows(rng, rows: int, D: int) -> np.ndarray:
    """bf16 rows spanning magnitudes, with the special rows of the definition."""
    x = (rng.standard_normal((rows, D)) * np.exp2(rng.uniform(-20, 20, (rows, 1)))).astype(np.float32)
    x[0] = 0.0                                   # all-zero row: scale 1
    x[1] = 0.0
    x[1, D // 2] = -3.0                          # one element: codes -448 and zeros
    x[2] = np.float32(1e-38) * rng.standard_normal(D).astype(np.float32)   # near the bottom of bf16
    x[3, ::2] = 3.0e38                           # near the top of bf16
    x[3, 1::2] = -1.0
    x[4] = -0.0                                  # negative zeros keep their sign bit
    return to_bf16_bits(x)


@pytest.mark.parametrize("D", [8, 32, 64, 96, 128, 512])
def test_quantize_rows_bit_exact(dev, D):
    import dsa_lightning_indexer_02_amd as dsa
    rng = block_rng(60, D, 0)
    bits = _rows(rng, 1000 + D, D)
    print("case quantize rows", bits.shape, flush=True)
    codes, scales = dsa.dsa_quantize_fp8_rows(dput(bits, dev).view(torch.bfloat16))
    oc, osc = oracle.quantize_rows(bits)
    assert np.array_equal(dget(scales), osc)
    assert np.array_equal(dget(codes), oc)


def test_quantize_queries_shape(dev):
    # the indexer's query layout [T, H_I, D_I]: one scale per (token, head)
    import dsa_lightning_indexer_02_amd as dsa
    rng = block_rng(61, 0, 0)
    q = to_bf16_bits(rng.standard_normal((37, 64, 128)).astype(np.float32))
    codes, scales = dsa.dsa_quantize_fp8_rows(dput(q, dev).view(torch.bfloat16))
    oc, osc = oracle.quantize_rows(q)
    assert tuple(scales.shape) == (37, 64)
    assert np.array_equal(dget(codes), oc) and np.array_equal(dget(scales), osc)


def _cache(rng, NB, bs, D_I, D_qk):
    k8 = rng.integers(0, 255, (NB, bs, D_I), dtype=np.uint8)
    ks = rng.uniform(0.1, 1.0, (NB, bs)).astype(np.float32)
    kv = rng.integers(0, 65535, (NB, bs, D_qk), dtype=np.uint16)
    return k8, ks, kv


@pytest.mark.parametrize("bs,D_I,D_qk", [(16, 128, 576), (64, 128, 576), (256, 32, 80)])
def test_append_paged_bit_exact(dev, bs, D_I, D_qk):
    import dsa_lightning_indexer_02_amd as dsa
    rng = block_rng(62, bs, D_I)
    NB, B, maxb = 40, 5, 8
    k8, ks, kv = _cache(rng, NB, bs, D_I, D_qk)
    table = np.full((B, maxb), -1, np.int32)
    perm = rng.permutation(NB).astype(np.int32)
    for b in range(B):
        table[b, :6] = perm[6 * b:6 * b + 6]
    # distinct slots: positions drawn without replacement per sequence
    seq, pos = [], []
    for b in range(B):
        p = rng.choice(6 * bs, size=min(6 * bs, 50), replace=False)
        seq += [b] * len(p)
        pos += p.tolist()
    seq = np.array(seq, np.int32)
    pos = np.array(pos, np.int32)
    n = len(seq)
    kn = _rows(rng, n, D_I)
    vn = rng.integers(0, 65535, (n, D_qk), dtype=np.uint16)
    print("case append", n, "tokens, block", bs, flush=True)
    cache = dsa.PagedKV(dput(k8, dev), dput(ks, dev), dput(kv, dev).view(torch.bfloat16), dput(table, dev))
    dsa.dsa_append_paged(cache, dput(seq, dev), dput(pos, dev), dput(kn, dev).view(torch.bfloat16),
                         dput(vn, dev).view(torch.bfloat16))
    ok8, oks, okv = oracle.append_paged(k8, ks, kv, table, seq, pos, kn, vn)
    assert np.array_equal(dget(cache.k8), ok8)
    assert np.array_equal(dget(cache.k_scale), oks)
    assert np.array_equal(dget(cache.kv.view(torch.int16)).view(np.uint16), okv)


def test_append_paged_skips_tokens_outside_the_cache(dev):
    import dsa_lightning_indexer_02_amd as dsa
    rng = block_rng(63, 0, 0)
    bs, D_I, D_qk, NB = 16, 64, 80, 6
    k8, ks, kv = _cache(rng, NB, bs, D_I, D_qk)
    table = np.array([[2, -1, 9], [4, 1, 0]], np.int32)           # -1 unmapped, 9 outside the pool
    seq = np.array([0, 0, 0, 1, 1, 2, -1, 1], np.int32)
    pos = np.array([3, 20, 40, 0, 47, 1, 1, 48], np.int32)         # 48: past the table row
    n = len(seq)
    kn = _rows(rng, n, D_I)
    vn = rng.integers(0, 65535, (n, D_qk), dtype=np.uint16)
    cache = dsa.PagedKV(dput(k8, dev), dput(ks, dev), dput(kv, dev).view(torch.bfloat16), dput(table, dev))
    dsa.dsa_append_paged(cache, dput(seq, dev), dput(pos, dev), dput(kn, dev).view(torch.bfloat16),
                         dput(vn, dev).view(torch.bfloat16))
    keep = np.array([0, 3, 4])                                     # the tokens with a valid slot
    ok8, oks, okv = oracle.append_paged(k8, ks, kv, table, seq[keep], pos[keep], kn[keep], vn[keep])
    assert np.array_equal(dget(cache.k8), ok8)
    assert np.array_equal(dget(cache.k_scale), oks)
    assert np.array_equal(dget(cache.kv.view(torch.int16)).view(np.uint16), okv)


def test_quantize_append_then_decode(dev):
    # the decode step fed by the on-device path: queries quantized on the GPU, each sequence's
    # newest token appended on the GPU, then the fused decode; the same steps through the oracle
    import dsa_lightning_indexer_02_amd as dsa
    import parity
    wl = dataclasses.replace(get("tiny"), kind="decode", T=6, S=3000, decode_len_lo=1, decode_len_hi=3000,
                             block_size=16)
    lens = np.array([1, 2, 17, 64, 700, 2999], np.int32)
    inp = decode_inputs(wl, seq_lens=lens)
    rng = block_rng(64, 0, 0)
    B = len(lens)
    q_bf = to_bf16_bits(rng.standard_normal((B, wl.H_I, wl.D_I)).astype(np.float32))
    k_new = to_bf16_bits(rng.standard_normal((B, wl.D_I)).astype(np.float32))
    kv_new = to_bf16_bits(rng.standard_normal((B, wl.D_qk)).astype(np.float32))
    seq = np.arange(B, dtype=np.int32)
    pos = (lens - 1).astype(np.int32)
    print("case quantize + append + decode", lens.tolist(), flush=True)
    cache = dsa.PagedKV(dput(inp.k8_pool, dev), dput(inp.ks_pool, dev),
                        dput(inp.kv_pool, dev).view(torch.bfloat16), dput(inp.block_table, dev),
                        dput(inp.seq_lens, dev))
    dsa.dsa_append_paged(cache, dput(seq, dev), dput(pos, dev), dput(k_new, dev).view(torch.bfloat16),
                         dput(kv_new, dev).view(torch.bfloat16))
    q8, qs = dsa.dsa_quantize_fp8_rows(dput(q_bf, dev).view(torch.bfloat16))
    out, f32, lse, idx = dsa.dsa_decode_paged(cache, int(lens.max()), dims_of(wl), q8, qs, dput(inp.w, dev),
                                              dput(inp.q, dev).view(torch.bfloat16), want_f32=True,
                                              want_indices=True)
    torch.cuda.synchronize()
    # oracle: the same append and quantization, then the decode definition
    ok8, oks, okv = oracle.append_paged(inp.k8_pool, inp.ks_pool, inp.kv_pool, inp.block_table, seq, pos,
                                        k_new, kv_new)
    oq8, oqs = oracle.quantize_rows(q_bf)
    assert np.array_equal(dget(q8), oq8) and np.array_equal(dget(qs), oqs)
    oinp = dataclasses.replace(inp, k8_pool=ok8, ks_pool=oks, kv_pool=okv, q8=oq8, qs=oqs)
    g_idx = dget(idx)
    g_out = bf16_vals(out)
    for b in range(B):
        o_lg, o_ix, _, _, _ = oracle.decode(oinp, seqs=[b], nthreads=1)[0]
        n = int(lens[b])
        parity.check_topk_boundary(g_idx[b:b + 1], o_ix[None], o_lg[None], np.array([n]), "decode top-k %d" % b)
        kvr = oracle.gather_rows(okv, inp.block_table[b], n)
        oo, _, ol = oracle.sparse_mla(inp.q[b:b + 1], g_idx[b:b + 1].astype(np.int32), np.array([n - 1]), kvr,
                                      wl.D_v, wl.sm_scale)
        parity.check_mla(g_out[b:b + 1], dget(f32)[b:b + 1], dget(lse)[b:b + 1], oo, ol,
                         "decode seq %d" % b)



# ----------------------------------------------------------------- UE8M0 scales (next row 2)
@pytest.mark.parametrize("D", [32, 128])
def test_quantize_ue8m0_bit_exact(dev, D):
    import dsa_lightning_indexer_02_amd as dsa
    rng = block_rng(65, D, 0)
    bits = _rows(rng, 777, D)
    print("case quantize ue8m0", bits.shape, flush=True)
    codes, exps, scales = dsa.dsa_quantize_fp8_rows_ue8m0(dput(bits, dev).view(torch.bfloat16))
    oc, oe, osc = oracle.quantize_rows_ue8m0(bits)
    assert np.array_equal(dget(exps), oe)
    assert np.array_equal(dget(scales), osc)
    assert np.array_equal(dget(codes), oc)


@pytest.mark.parametrize("T,S,q_start,H_I,D_I", [(300, 700, 400, 64, 128), (77, 200, 123, 4, 32),
                                                 (1000, 1000, 0, 64, 128)])
def test_indexer_ue8m0_scaled_mfma(dev, T, S, q_start, H_I, D_I):
    # scores from UE8M0-quantized inputs, exponents applied inside the MFMA, against the oracle
    # indexer fed the same codes with fp32 scales 2^(e - 127)
    import dsa_lightning_indexer_02_amd as dsa
    import parity
    rng = block_rng(66, T, H_I)
    q = to_bf16_bits((rng.standard_normal((T, H_I, D_I)) * np.exp2(rng.uniform(-8, 8, (T, H_I, 1)))).astype(np.float32))
    k = to_bf16_bits((rng.standard_normal((S, D_I)) * np.exp2(rng.uniform(-8, 8, (S, 1)))).astype(np.float32))
    w = (rng.uniform(0, 1, (T, H_I)) / H_I).astype(np.float32)
    print("case indexer ue8m0", T, S, q_start, H_I, D_I, flush=True)
    q8, qe, qs = dsa.dsa_quantize_fp8_rows_ue8m0(dput(q, dev).view(torch.bfloat16))
    k8, ke, ks = dsa.dsa_quantize_fp8_rows_ue8m0(dput(k, dev).view(torch.bfloat16))
    lg = dsa.dsa_indexer_logits_ue8m0(q8, qe, dput(w, dev), k8, ke, q_start=q_start)
    # the same scores through the fp32-scale entry point (scales 2^(e - 127), applied in the epilogue)
    lg32 = dsa.dsa_indexer_logits(q8, qs, dput(w, dev), k8, ks, q_start=q_start)
    torch.cuda.synchronize()
    oq8, oqe, oqs = oracle.quantize_rows_ue8m0(q)
    ok8, oke, oks = oracle.quantize_rows_ue8m0(k)
    assert np.array_equal(dget(q8), oq8) and np.array_equal(dget(ke), oke)
    pos = q_start + np.arange(T)
    o = oracle.indexer(oq8, oqs, w, pos, ok8, oks)
    A = parity.magnitude(oq8, oqs, w, ok8, oks, pos, S)
    g = dget(lg)[:, :S]
    # codes of rows scaled over 2^+-8 with power-of-two scales: the block-max allowance (any codes)
    B = parity.block_magnitude(oq8, oqs, w, ok8, oks, pos, S)
    _, share = parity.check_indexer(g, o, A, D_I, H_I, "indexer ue8m0", B=B)
    print("  relative term dominates on %.1f%% of entries" % (100 * share), flush=True)
    m = ~np.isnan(o)
    g32 = dget(lg32)[:, :S]
    assert np.all(np.abs(g[m] - g32[m]) <= 2.0 ** -20 * A[m]), "scaled MFMA and epilogue scaling disagree"
