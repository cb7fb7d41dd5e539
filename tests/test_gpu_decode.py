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
from gpu_helpers import DecodeDev, bf16_vals, dget

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_02_amd as dsa
    dsa.load()
    return torch.device("cuda:0")


def _check(inp, res, seqs):
    out, out_f32, lse, idx = (dget(x) if x.dtype != torch.bfloat16 else bf16_vals(x) for x in res)
    wl = inp.wl

    def one(b):
        return b, oracle.decode(inp, seqs=[b], nthreads=1)[0]

    with ThreadPoolExecutor(8) as ex:
        results = list(ex.map(one, seqs))
    for b, (o_lg, o_ix, o_out, _, o_lse) in results:
        n = int(inp.seq_lens[b])
        # top-k against the oracle's logits (boundary rule); attention on the GPU's own indices
        parity.check_topk_boundary(idx[b:b + 1], o_ix[None], o_lg[None], np.array([n]), "decode top-k")
        kv = oracle.gather_rows(inp.kv_pool, inp.block_table[b], n)
        oo, _, ol = oracle.sparse_mla(inp.q[b:b + 1], idx[b:b + 1].astype(np.int32), np.array([n - 1]), kv,
                                      wl.D_v, wl.sm_scale)
        parity.check_mla(out[b:b + 1], out_f32[b:b + 1], lse[b:b + 1], oo, ol, "decode seq %d" % b)


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
    order = np.argsort(inp.seq_lens)
    _check(inp, res, [int(order[0]), int(order[1]), int(order[32]), int(order[-2]), int(order[-1])])


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
