"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds no arithmetic of the method itself.  It draws random
numbers and encodes them into the input formats the method consumes:

* FP8 E4M3 (OCP "fn" variant: max 448, no infinities) codes with one fp32
  scale per row of the last dimension (the indexer listing on the createthis
  gist page quantizes its inputs along the last dimension; the indexer runs in
  FP8 per the DeepSeek-V3.2-Exp summary page, section "Method").  The encoding is torch's own
  ``float8_e4m3fn`` cast (round to nearest even) after clamping to +-448.
* bf16 bit patterns (round to nearest even, torch's cast).

Random streams.  Every tensor is cut into blocks of ``ROWS_PER_BLOCK`` rows of
its first dimension; block ``b`` of tensor ``tid`` is drawn from its own
``PCG64(SeedSequence(seed, spawn_key=(tid, ..., b)))`` stream.  Any subset of
rows can therefore be regenerated exactly without drawing the rest, and
blocks are drawn in parallel threads.  Tensor ids, in draw order:
0 q_I, 1 k_I, 2 w, 3 q, 4 kv, 5 outlier positions, 6 decode lengths,
7 decode block permutation.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from .configs import Workload

ROWS_PER_BLOCK = 16
FP8_MAX = 448.0

TID_QI, TID_KI, TID_W, TID_Q, TID_KV, TID_OUTLIER, TID_LENS, TID_PERM = range(8)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def block_rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=tuple(key))))


def _draw_rows(seed: int, key: tuple, n_rows: int, row_shape: tuple, kind: str,
               rows: Optional[np.ndarray] = None, scale: float = 1.0) -> np.ndarray:
    """float32 rows [len(rows) or n_rows, *row_shape]; 'normal' N(0,1) or 'uniform' U[0,1) times scale."""
    per_row = int(np.prod(row_shape)) if row_shape else 1
    sel = np.arange(n_rows, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(sel), per_row), dtype=np.float32)
    if len(sel) == 0:
        return out.reshape((0,) + tuple(row_shape))
    blocks = np.unique(sel // ROWS_PER_BLOCK)

    def fill(b: int):
        g = block_rng(seed, *key, int(b))
        if kind == "normal":
            vals = g.standard_normal(ROWS_PER_BLOCK * per_row, dtype=np.float32)
        else:
            vals = g.random(ROWS_PER_BLOCK * per_row, dtype=np.float32)
        vals = vals.reshape(ROWS_PER_BLOCK, per_row)
        lo = b * ROWS_PER_BLOCK
        m = (sel >= lo) & (sel < lo + ROWS_PER_BLOCK)
        where = np.nonzero(m)[0]
        out[where] = vals[sel[where] - lo]

    if len(blocks) > 4:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, blocks))
    else:
        for b in blocks:
            fill(b)
    if scale != 1.0:
        out *= np.float32(scale)
    return out.reshape((len(sel),) + tuple(row_shape))


def quantize_fp8_rows(x: np.ndarray):
    """Per-row (last dim) absmax scaling to OCP E4M3: returns (uint8 codes, fp32 scales).

    scale = amax / 448 (1.0 for an all-zero row); code = e4m3(clamp(x / scale, -448, 448)).
    """
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    amax = t.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    y = (t / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy(), scale.numpy().astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class PrefillInputs:
    wl: Workload
    rows: np.ndarray          # query rows present (int64), positions q_start + rows
    q8: np.ndarray            # [R, H_I, D_I] uint8
    qs: np.ndarray            # [R, H_I] f32
    w: np.ndarray             # [R, H_I] f32
    k8: np.ndarray            # [S, D_I] uint8
    ks: np.ndarray            # [S] f32
    q: np.ndarray             # [R, H, D_qk] uint16 (bf16)
    kv: np.ndarray            # [S, D_qk] uint16 (bf16)
    outliers: np.ndarray      # key positions scaled before quantization

    @property
    def pos(self) -> np.ndarray:
        return self.wl.q_start + self.rows


def _keys(wl: Workload, seed: int, key_prefix: tuple, n: int, outlier_pos=None):
    kI = _draw_rows(seed, key_prefix + (TID_KI,), n, (wl.D_I,), "normal")
    if outlier_pos is not None and len(outlier_pos):
        kI[outlier_pos] *= np.float32(wl.outlier_factor)
    k8, ks = quantize_fp8_rows(kI)
    del kI
    kv = to_bf16_bits(_draw_rows(seed, key_prefix + (TID_KV,), n, (wl.D_qk,), "normal"))
    return k8, ks, kv


def prefill_inputs(wl: Workload, rows: Optional[Sequence[int]] = None, seed: Optional[int] = None,
                   with_q: bool = True) -> PrefillInputs:
    """Inputs of a prefill workload; ``rows`` restricts the query-side tensors to those rows."""
    seed = wl.seed if seed is None else seed
    sel = np.arange(wl.T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    qI = _draw_rows(seed, (TID_QI,), wl.T, (wl.H_I, wl.D_I), "normal", sel)
    q8, qs = quantize_fp8_rows(qI)
    del qI
    outl = np.zeros(0, dtype=np.int64)
    if wl.outlier_frac > 0:
        n_out = int(round(wl.outlier_frac * wl.S))
        outl = np.sort(block_rng(seed, TID_OUTLIER, 0).choice(wl.S, size=n_out, replace=False)).astype(np.int64)
    k8, ks, kv = _keys(wl, seed, (), wl.S, outl)
    w = _draw_rows(seed, (TID_W,), wl.T, (wl.H_I,), "uniform", sel, scale=1.0 / wl.H_I)
    if with_q:
        q = to_bf16_bits(_draw_rows(seed, (TID_Q,), wl.T, (wl.H, wl.D_qk), "normal", sel))
    else:
        q = np.zeros((len(sel), wl.H, wl.D_qk), dtype=np.uint16)
    return PrefillInputs(wl, sel, q8, qs, w, k8, ks, q, kv, outl)


@dataclass
class DecodeInputs:
    wl: Workload
    seq_lens: np.ndarray      # [B] int32, context length incl. the new token
    block_table: np.ndarray   # [B, max_blocks] int32, -1 past a sequence's blocks
    k8_pool: np.ndarray       # [NB, bs, D_I] uint8
    ks_pool: np.ndarray       # [NB, bs] f32
    kv_pool: np.ndarray       # [NB, bs, D_qk] uint16
    q8: np.ndarray            # [B, H_I, D_I]
    qs: np.ndarray            # [B, H_I]
    w: np.ndarray             # [B, H_I]
    q: np.ndarray             # [B, H, D_qk]

    @property
    def num_blocks(self) -> int:
        return self.k8_pool.shape[0]


def decode_lengths(wl: Workload, seed: Optional[int] = None) -> np.ndarray:
    seed = wl.seed if seed is None else seed
    return block_rng(seed, TID_LENS, 0).integers(wl.decode_len_lo, wl.decode_len_hi, size=wl.T,
                                                 endpoint=True).astype(np.int32)


def decode_inputs(wl: Workload, seed: Optional[int] = None, seq_lens: Optional[np.ndarray] = None) -> DecodeInputs:
    """Paged decode inputs: one query per sequence at position seq_len - 1.

    The pool holds exactly sum(ceil(n_b / bs)) blocks; one seeded permutation of all
    block ids is cut into consecutive per-sequence slices (the block tables).
    """
    seed = wl.seed if seed is None else seed
    bs = wl.block_size
    lens = decode_lengths(wl, seed) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    B = len(lens)
    nblk = (lens.astype(np.int64) + bs - 1) // bs
    NB = int(nblk.sum())
    perm = block_rng(seed, TID_PERM, 0).permutation(NB).astype(np.int32)
    maxb = int(nblk.max())
    table = np.full((B, maxb), -1, dtype=np.int32)
    k8_pool = np.zeros((NB, bs, wl.D_I), dtype=np.uint8)
    ks_pool = np.zeros((NB, bs), dtype=np.float32)
    kv_pool = np.zeros((NB, bs, wl.D_qk), dtype=np.uint16)
    off = 0
    for b in range(B):
        n = int(lens[b])
        blocks = perm[off:off + nblk[b]]
        off += int(nblk[b])
        table[b, :len(blocks)] = blocks
        k8, ks, kv = _keys(wl, seed, (b,), n)
        pad = len(blocks) * bs - n
        if pad:
            k8 = np.concatenate([k8, np.zeros((pad, wl.D_I), np.uint8)])
            ks = np.concatenate([ks, np.zeros(pad, np.float32)])
            kv = np.concatenate([kv, np.zeros((pad, wl.D_qk), np.uint16)])
        k8_pool[blocks] = k8.reshape(-1, bs, wl.D_I)
        ks_pool[blocks] = ks.reshape(-1, bs)
        kv_pool[blocks] = kv.reshape(-1, bs, wl.D_qk)
    qI = _draw_rows(seed, (TID_QI,), B, (wl.H_I, wl.D_I), "normal")
    q8, qs = quantize_fp8_rows(qI)
    w = _draw_rows(seed, (TID_W,), B, (wl.H_I,), "uniform", scale=1.0 / wl.H_I)
    q = to_bf16_bits(_draw_rows(seed, (TID_Q,), B, (wl.H, wl.D_qk), "normal"))
    return DecodeInputs(wl, lens, table, k8_pool, ks_pool, kv_pool, q8, qs, w, q)
