"""Fused paged decode vs the oracle, per sequence (needs an MI355X)."""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import parity
from dsa_inputs import decode_inputs, get
from gpu_helpers import DecodeDev, bf16_vals, dget, dims_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_02_amd as dsa
    dsa.load()
    return torch.device("cuda:0")


def _check(inp, res, seqs):
    """Every listed sequence through all three steps: the decode indexer's scores entry by entry
    against the oracle (the indexer bar), the decode top-k exactly against the oracle's selection
    on the GPU's own scores and by the boundary rule against the oracle's scores, attention on the
    GPU's own index lists."""
    out, out_f32, lse, idx, scores = (dget(x) if x.dtype != torch.bfloat16 else bf16_vals(x) for x in res)
    wl = inp.wl

    def one(b):
        return b, oracle.decode(inp, seqs=[b], nthreads=2)[0]

    with ThreadPoolExecutor(8) as ex:
        results = list(ex.map(one, seqs))
    entries, rel_entries, worst = 0, 0.0, 0.0
    for b, (o_lg, o_ix, o_out, _, o_lse) in results:
        n = int(inp.seq_lens[b])
        pos = np.array([n - 1])
        # 1. scores of the visible keys, read through the sequence's block table
        k8 = oracle.gather_rows(inp.k8_pool, inp.block_table[b], n)
        ks = oracle.gather_rows(inp.ks_pool[..., None], inp.block_table[b], n)[:, 0]
        g_lg = scores[b:b + 1, :n].astype(np.float32)
        A = parity.magnitude(inp.q8[b:b + 1], inp.qs[b:b + 1], inp.w[b:b + 1], k8, ks, pos, n)
        wr, share = parity.check_indexer(g_lg, o_lg[None], A, wl.D_I, wl.H_I, "decode indexer seq %d" % b)
        worst = max(worst, wr)
        entries += n
        rel_entries += share * n
        # 2. top-k: exact on the GPU's own scores, boundary rule against the oracle's scores
        parity.check_topk_exact(idx[b:b + 1], oracle.topk(g_lg, pos, wl.topk), "decode top-k seq %d" % b)
        parity.check_topk_boundary(idx[b:b + 1], o_ix[None], o_lg[None], np.array([n]), "decode top-k")
        # 3. attention on the GPU's own indices
        kv = oracle.gather_rows(inp.kv_pool, inp.block_table[b], n)
        oo, _, ol = oracle.sparse_mla(inp.q[b:b + 1], idx[b:b + 1].astype(np.int32), pos, kv, wl.D_v, wl.sm_scale)
        parity.check_mla(out[b:b + 1], out_f32[b:b + 1], lse[b:b + 1], oo, ol, "decode seq %d" % b)
    print("  %d sequences, %d scores: worst %.3f of the indexer bar, the 1e-3 relative term dominates on %.1f%%"
          % (len(results), entries, worst, 100 * rel_entries / max(entries, 1)), flush=True)


def test_decode_short_sequences(dev):
    wl = get("decode_64")
    lens = np.array([1, 2, 63, 64, 65, 100, 2047, 2048, 2049, 5000, 40000, 70001], dtype=np.int32)
    print("case decode short", lens.tolist(), flush=True)
    inp = decode_inputs(wl, seq_lens=lens)
    d = DecodeDev(inp, dev)
    res = d.run()
    torch.cuda.synchronize()
    _check(inp, res, range(len(lens)))


def test_decode_64_full_size(dev):
    wl = get("decode_64")
    inp = decode_inputs(wl)
    print("case decode_64 lens", int(inp.seq_lens.min()), int(inp.seq_lens.max()), flush=True)
    d = DecodeDev(inp, dev)
    res = d.run()
    torch.cuda.synchronize()
    _check(inp, res, range(len(inp.seq_lens)))        # all 64 sequences


@pytest.mark.parametrize("block_size", [16, 256])
def test_decode_other_block_sizes(dev, block_size):
    # blocks under 64 rows take the per-lane table lookup in the decode indexer; larger ones the
    # per-workgroup block-id preload (a 64-key group never straddles two blocks)
    wl = dataclasses.replace(get("decode_64"), block_size=block_size)
    lens = np.array([1, 17, 64, 255, 257, 4097, 9000, 20001], dtype=np.int32)
    print("case decode block_size", block_size, lens.tolist(), flush=True)
    inp = decode_inputs(wl, seq_lens=lens)
    d = DecodeDev(inp, dev)
    res = d.run()
    torch.cuda.synchronize()
    _check(inp, res, range(len(lens)))


@pytest.mark.parametrize("block_size", [16, 64])
def test_decode_small_dims(dev, block_size):
    # 4 indexer heads of width 32 (one 16-head MFMA tile, lanes past D_I re-read in-row bytes
    # against zero query bytes), 8 attention heads of 80/64 and top-64: the combine over 64-wide
    # partial rows
    wl = dataclasses.replace(get("tiny"), kind="decode", T=7, S=5000, decode_len_lo=1, decode_len_hi=5000,
                             block_size=block_size)
    lens = np.array([1, 5, 64, 65, 300, 1000, 4097], dtype=np.int32)
    print("case decode small dims block_size", block_size, lens.tolist(), flush=True)
    inp = decode_inputs(wl, seq_lens=lens)
    d = DecodeDev(inp, dev)
    res = d.run()
    torch.cuda.synchronize()
    _check(inp, res, range(len(lens)))


def _bulk_decode_inputs(wl, lens, seed):
    """Decode inputs for many short sequences drawn in one pass (the per-sequence streams of
    decode_inputs take minutes at 12288 sequences): same recipe, per-row absmax FP8 keys and queries,
    bf16 N(0,1) latent rows and queries, one seeded permutation of the exact pool cut into tables."""
    from dsa_inputs.generate import DecodeInputs, block_rng, quantize_fp8_rows, to_bf16_bits
    g = block_rng(seed, 0, 0)
    bs, B = wl.block_size, len(lens)
    nblk = (lens.astype(np.int64) + bs - 1) // bs
    NB = int(nblk.sum())
    perm = g.permutation(NB).astype(np.int32)
    table = np.full((B, int(nblk.max())), -1, np.int32)
    starts = np.concatenate([[0], np.cumsum(nblk)[:-1]])
    for j in range(int(nblk.max())):
        has = nblk > j
        table[has, j] = perm[starts[has] + j]
    k8, ks = quantize_fp8_rows(g.standard_normal((NB * bs, wl.D_I)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((NB * bs, wl.D_qk)).astype(np.float32))
    q8, qs = quantize_fp8_rows(g.standard_normal((B, wl.H_I, wl.D_I)).astype(np.float32))
    w = (g.random((B, wl.H_I)) / wl.H_I).astype(np.float32)
    q = to_bf16_bits(g.standard_normal((B, wl.H, wl.D_qk)).astype(np.float32))
    return DecodeInputs(wl, lens.astype(np.int32), table, k8.reshape(NB, bs, wl.D_I), ks.reshape(NB, bs),
                        kv.reshape(NB, bs, wl.D_qk), q8, qs, w, q)


def test_decode_largest_batch(dev):
    # the largest batch one decode call takes (12288 sequences: the indexer's per-sequence prefix
    # table fills most of the LDS), with short sequences and the small attention dims; every
    # 97th sequence plus the first and last are checked
    import dsa_lightning_indexer_02_amd as dsa
    B = 12288
    lens = (np.arange(B) % 97 + 1).astype(np.int32)
    wl = dataclasses.replace(get("tiny"), kind="decode", T=B, S=128, decode_len_lo=1, decode_len_hi=128,
                             block_size=64)
    print("case decode largest batch", B, flush=True)
    inp = _bulk_decode_inputs(wl, lens, seed=91)
    d = DecodeDev(inp, dev)
    res = d.run()
    torch.cuda.synchronize()
    _check(inp, res, sorted(set(range(0, B, 97)) | {0, 1, B - 1}))
    # one more sequence is refused on the host (tests/test_abi.py covers the status code)
    assert dsa.decode_workspace_size(dims_of(wl), B + 1, 128) > 0
