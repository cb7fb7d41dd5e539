"""Python wrapper of the DSA oracle (oracle/dsa_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
cpu_baseline leg of bench.py may import this package.  The product library
(dsa_lightning_indexer_02_amd) never imports it, and this package never
imports the product library.

Every function takes host numpy arrays in the input formats of the method
(FP8 E4M3 codes as uint8, bf16 as uint16 bit patterns) and returns numpy
arrays.  ``pos`` is the absolute position of each query row; row t sees keys
0 .. min(S, pos[t] + 1) - 1.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def load(path: Optional[str] = None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        from . import build as _b
        _b.build(out=p)
    lib = ctypes.CDLL(p)
    lib.oracle_e4m3_table.argtypes = [_p]
    lib.oracle_e4m3_table.restype = None
    lib.oracle_bf16_round.argtypes = [_p, _p, _i64]
    lib.oracle_bf16_round.restype = None
    lib.oracle_gather_rows.argtypes = [_p, _i64, _p, _i32, _i64, _p]
    lib.oracle_gather_rows.restype = ctypes.c_int
    lib.oracle_indexer.argtypes = [_p, _p, _p, _p, _i64, _p, _p, _i64, _i32, _i32, _p, _i64, _i32]
    lib.oracle_indexer.restype = ctypes.c_int
    lib.oracle_topk.argtypes = [_p, _i64, _p, _i64, _i64, _i32, _p, _i32]
    lib.oracle_topk.restype = ctypes.c_int
    lib.oracle_sparse_mla.argtypes = [_p, _p, _p, _i64, _i32, _i32, _i32, _i32, _p, _i64,
                                      ctypes.c_float, _p, _p, _p, _i32]
    lib.oracle_sparse_mla.restype = ctypes.c_int
    lib.oracle_e4m3_encode.argtypes = [_p, _p, _i64]
    lib.oracle_e4m3_encode.restype = None
    lib.oracle_quantize_rows.argtypes = [_p, _i64, _i32, _p, _p]
    lib.oracle_quantize_rows.restype = None
    lib.oracle_quantize_rows_ue8m0.argtypes = [_p, _i64, _i32, _p, _p, _p]
    lib.oracle_quantize_rows_ue8m0.restype = None
    lib.oracle_append_paged.argtypes = [_p, _p, _p, _i32, _p, _i64, _p, _p, _i64, _i32, _i32, _p, _p]
    lib.oracle_append_paged.restype = _i64
    lib.oracle_indexer_kl.argtypes = [_p, _p, _p, _i64, _i64, _i32, _i32, ctypes.c_double, _p, _i64, _p, _p,
                                      _i64, _i32]
    lib.oracle_indexer_kl.restype = ctypes.c_int
    lib.oracle_indexer_bwd.argtypes = [_p, _p, _p, _p, _i64, _p, _p, _i64, _i32, _i32, _p, _i64, _p, _p, _p,
                                       _i32]
    lib.oracle_indexer_bwd.restype = ctypes.c_int
    lib.oracle_indexer_kl_sparse.argtypes = [_p, _p, _p, _i64, _i64, _i32, _i32, ctypes.c_double, _p, _i32, _p,
                                             _i64, _p, _p, _i64, _i32]
    lib.oracle_indexer_kl_sparse.restype = ctypes.c_int
    lib.oracle_sparse_mla_bwd.argtypes = [_p, _p, _p, _i64, _i32, _i32, _i32, _i32, _p, _i64, ctypes.c_double, _p,
                                          _p, _p, _i32]
    lib.oracle_sparse_mla_bwd.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def e4m3_table(lib=None) -> np.ndarray:
    lib = lib or load()
    out = np.empty(256, dtype=np.float32)
    lib.oracle_e4m3_table(_ptr(out))
    return out


def bf16_round(x: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.oracle_bf16_round(_ptr(x), _ptr(out), x.size)
    return out


def gather_rows(pool: np.ndarray, block_table: np.ndarray, n: int, lib=None) -> np.ndarray:
    """Logical rows 0..n-1 of a paged pool [NB, bs, ...] via one sequence's block table."""
    lib = lib or load()
    pool = np.ascontiguousarray(pool)
    bs = pool.shape[1]
    row_shape = pool.shape[2:]
    row_bytes = int(np.prod(row_shape, dtype=np.int64)) * pool.itemsize
    out = np.empty((n,) + row_shape, dtype=pool.dtype)
    tbl = _c(block_table, np.int32)
    rc = lib.oracle_gather_rows(_ptr(pool), row_bytes, _ptr(tbl), bs, n, _ptr(out))
    if rc:
        raise ValueError("oracle_gather_rows: negative block id inside the sequence")
    return out


def indexer(q8, qs, w, pos, k8, ks, nthreads: int = 0, lib=None) -> np.ndarray:
    """Index scores [T, S] float32; entries past each row's visible range are NaN."""
    lib = lib or load()
    q8 = _c(q8, np.uint8)
    T, H_I, D_I = q8.shape
    k8 = _c(k8, np.uint8)
    S = k8.shape[0]
    qs, w, ks = _c(qs, np.float32), _c(w, np.float32), _c(ks, np.float32)
    pos = _c(pos, np.int64)
    out = np.full((T, S), np.nan, dtype=np.float32)
    rc = lib.oracle_indexer(_ptr(q8), _ptr(qs), _ptr(w), _ptr(pos), T, _ptr(k8), _ptr(ks), S,
                            H_I, D_I, _ptr(out), S, nthreads)
    if rc:
        raise RuntimeError("oracle_indexer failed (%d)" % rc)
    return out


def topk(logits, pos, k: int, nthreads: int = 0, lib=None) -> np.ndarray:
    """Top-k index lists [T, k] int32 (score descending, index ascending; -1 padded)."""
    lib = lib or load()
    logits = _c(logits, np.float32)
    T, S = logits.shape
    pos = _c(pos, np.int64)
    out = np.empty((T, k), dtype=np.int32)
    rc = lib.oracle_topk(_ptr(logits), S, _ptr(pos), T, S, k, _ptr(out), nthreads)
    if rc:
        raise RuntimeError("oracle_topk failed (%d)" % rc)
    return out


def sparse_mla(q, idx, pos, kv, D_v: int, sm_scale: float, nthreads: int = 0, lib=None):
    """(out fp32 [T,H,D_v], out bf16 bits [T,H,D_v], lse fp32 [T,H])."""
    lib = lib or load()
    q = _c(q, np.uint16)
    T, H, D_qk = q.shape
    idx = _c(idx, np.int32)
    k = idx.shape[1]
    kv = _c(kv, np.uint16)
    S = kv.shape[0]
    pos = _c(pos, np.int64)
    out = np.empty((T, H, D_v), dtype=np.float32)
    outb = np.empty((T, H, D_v), dtype=np.uint16)
    lse = np.empty((T, H), dtype=np.float32)
    rc = lib.oracle_sparse_mla(_ptr(q), _ptr(idx), _ptr(pos), T, H, D_qk, D_v, k, _ptr(kv), S,
                               ctypes.c_float(sm_scale), _ptr(out), _ptr(outb), _ptr(lse), nthreads)
    if rc:
        raise RuntimeError("oracle_sparse_mla failed (%d)" % rc)
    return out, outb, lse


def prefill(inp, nthreads: int = 0, lib=None):
    """Whole path for prefill inputs (dsa_inputs.PrefillInputs): logits, indices, out, out_bf16, lse."""
    wl = inp.wl
    pos = inp.pos
    logits = indexer(inp.q8, inp.qs, inp.w, pos, inp.k8, inp.ks, nthreads, lib)
    idx = topk(logits, pos, wl.topk, nthreads, lib)
    out, outb, lse = sparse_mla(inp.q, idx, pos, inp.kv, wl.D_v, wl.sm_scale, nthreads, lib)
    return logits, idx, out, outb, lse


def decode(inp, nthreads: int = 0, lib=None, seqs=None):
    """Whole path for paged decode inputs (dsa_inputs.DecodeInputs), per sequence.

    Returns per-sequence lists (logits row of length n_b, indices [k], out [H, D_v] fp32,
    out bf16, lse [H]).  Keys and KV rows are read through each sequence's block table.
    """
    wl = inp.wl
    res = []
    seqs = range(len(inp.seq_lens)) if seqs is None else seqs
    for b in seqs:
        n = int(inp.seq_lens[b])
        tbl = inp.block_table[b]
        k8 = gather_rows(inp.k8_pool, tbl, n, lib)
        ks = gather_rows(inp.ks_pool[..., None], tbl, n, lib)[:, 0]
        kv = gather_rows(inp.kv_pool, tbl, n, lib)
        pos = np.array([n - 1], dtype=np.int64)
        lg = indexer(inp.q8[b:b + 1], inp.qs[b:b + 1], inp.w[b:b + 1], pos, k8, ks, nthreads, lib)
        ix = topk(lg, pos, wl.topk, nthreads, lib)
        o, ob, l = sparse_mla(inp.q[b:b + 1], ix, pos, kv, wl.D_v, wl.sm_scale, nthreads, lib)
        res.append((lg[0], ix[0], o[0], ob[0], l[0]))
    return res


def e4m3_encode(y: np.ndarray, lib=None) -> np.ndarray:
    """Nearest OCP E4M3 codes (ties to the even code) of finite fp32 values with |y| <= 448."""
    lib = lib or load()
    y = _c(y, np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib.oracle_e4m3_encode(_ptr(y), _ptr(out), y.size)
    return out


def quantize_rows(x_bf16: np.ndarray, lib=None):
    """Per-row (last dim) absmax FP8 quantization of bf16 bit patterns: (uint8 codes, f32 scales)."""
    lib = lib or load()
    x = _c(x_bf16, np.uint16)
    D = x.shape[-1]
    rows = x.size // D if D else 0
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    lib.oracle_quantize_rows(_ptr(x), rows, D, _ptr(codes), _ptr(scales))
    return codes, scales


def append_paged(k8_pool, ks_pool, kv_pool, block_table, seq, pos, k_bf16, kv_bf16, lib=None):
    """Copies of the three pools after appending tokens (seq[i], pos[i]) with indexer keys k_bf16
    [n, D_I] (quantized here) and latent rows kv_bf16 [n, D_qk]."""
    lib = lib or load()
    k8 = np.array(k8_pool, dtype=np.uint8, copy=True, order="C")
    ks = np.array(ks_pool, dtype=np.float32, copy=True, order="C")
    kv = np.array(kv_pool, dtype=np.uint16, copy=True, order="C")
    tbl = _c(block_table, np.int32)
    seq = _c(seq, np.int32)
    pos = _c(pos, np.int32)
    k = _c(k_bf16, np.uint16)
    v = _c(kv_bf16, np.uint16)
    n = len(seq)
    bad = lib.oracle_append_paged(_ptr(k8), _ptr(ks), _ptr(kv), k8.shape[1], _ptr(tbl), tbl.shape[1], _ptr(seq),
                                  _ptr(pos), n, k8.shape[2], kv.shape[2], _ptr(k), _ptr(v))
    if bad:
        raise ValueError("oracle_append_paged: %d tokens fall in blocks with a negative id" % bad)
    return k8, ks, kv


def quantize_rows_ue8m0(x_bf16: np.ndarray, lib=None):
    """Per-row FP8 quantization with power-of-two (UE8M0) scales: (uint8 codes, uint8 biased
    exponents, f32 scales = 2^(exponent - 127))."""
    lib = lib or load()
    x = _c(x_bf16, np.uint16)
    D = x.shape[-1]
    rows = x.size // D if D else 0
    codes = np.empty(x.shape, dtype=np.uint8)
    exps = np.empty(x.shape[:-1], dtype=np.uint8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    lib.oracle_quantize_rows_ue8m0(_ptr(x), rows, D, _ptr(codes), _ptr(exps), _ptr(scales))
    return codes, exps, scales


def indexer_kl(q, kv, pos, sm_scale: float, logits, nthreads: int = 0, lib=None):
    """KL(p || softmax(I)) per query row and its gradient with respect to the scores.

    q: bf16 bits [T, H, D_qk]; kv: bf16 bits [S, D_qk]; logits: fp32 [T, >= S] (each row's visible
    entries are read).  Returns (loss float64 [T], dlogits float64 [T, S], NaN past each row's
    visible range)."""
    lib = lib or load()
    q = _c(q, np.uint16)
    T, H, D_qk = q.shape
    kv = _c(kv, np.uint16)
    S = kv.shape[0]
    logits = _c(logits, np.float32)
    pos = _c(pos, np.int64)
    loss = np.empty(T, dtype=np.float64)
    d = np.full((T, S), np.nan, dtype=np.float64)
    rc = lib.oracle_indexer_kl(_ptr(q), _ptr(kv), _ptr(pos), T, S, H, D_qk, ctypes.c_double(sm_scale),
                               _ptr(logits), logits.shape[1], _ptr(loss), _ptr(d), S, nthreads)
    if rc:
        raise RuntimeError("oracle_indexer_kl failed (%d)" % rc)
    return loss, d


def indexer_bwd(q8, qs, w, pos, k8, ks, dlogits, nthreads: int = 0, lib=None):
    """Gradients (dq [T, H_I, D_I], dw [T, H_I], dk [S, D_I], float64) of a loss through the index
    scores, given dlogits fp32 [T, >= S] = dL/dI on the visible entries."""
    lib = lib or load()
    q8 = _c(q8, np.uint8)
    T, H_I, D_I = q8.shape
    k8 = _c(k8, np.uint8)
    S = k8.shape[0]
    qs, w, ks = _c(qs, np.float32), _c(w, np.float32), _c(ks, np.float32)
    dlogits = _c(dlogits, np.float32)
    pos = _c(pos, np.int64)
    dq = np.empty((T, H_I, D_I), dtype=np.float64)
    dw = np.empty((T, H_I), dtype=np.float64)
    dk = np.empty((S, D_I), dtype=np.float64)
    rc = lib.oracle_indexer_bwd(_ptr(q8), _ptr(qs), _ptr(w), _ptr(pos), T, _ptr(k8), _ptr(ks), S, H_I, D_I,
                                _ptr(dlogits), dlogits.shape[1], _ptr(dq), _ptr(dw), _ptr(dk), nthreads)
    if rc:
        raise RuntimeError("oracle_indexer_bwd failed (%d)" % rc)
    return dq, dw, dk


def indexer_kl_sparse(q, kv, pos, sm_scale: float, idx, logits, nthreads: int = 0, lib=None):
    """Sparse-stage loss: KL over each row's index-list entries (see oracle_indexer_kl_sparse).

    idx: int32 [T, k].  Returns (loss float64 [T], dlogits float64 [T, S], 0 on visible keys not
    listed, NaN past each row's visible range)."""
    lib = lib or load()
    q = _c(q, np.uint16)
    T, H, D_qk = q.shape
    kv = _c(kv, np.uint16)
    S = kv.shape[0]
    idx = _c(idx, np.int32)
    logits = _c(logits, np.float32)
    pos = _c(pos, np.int64)
    loss = np.empty(T, dtype=np.float64)
    d = np.full((T, S), np.nan, dtype=np.float64)
    rc = lib.oracle_indexer_kl_sparse(_ptr(q), _ptr(kv), _ptr(pos), T, S, H, D_qk, ctypes.c_double(sm_scale),
                                      _ptr(idx), idx.shape[1], _ptr(logits), logits.shape[1], _ptr(loss), _ptr(d),
                                      S, nthreads)
    if rc:
        raise RuntimeError("oracle_indexer_kl_sparse failed (%d)" % rc)
    return loss, d


def sparse_mla_bwd(q, idx, pos, kv, D_v: int, sm_scale: float, dout, nthreads: int = 0, lib=None):
    """Gradients of the sparse MLA forward (see oracle_sparse_mla_bwd) for dL/dout = dout (bf16 bits
    [T, H, D_v]): (dq float64 [T, H, D_qk], dkv float64 [S, D_qk])."""
    lib = lib or load()
    q = _c(q, np.uint16)
    T, H, D_qk = q.shape
    idx = _c(idx, np.int32)
    k = idx.shape[1]
    kv = _c(kv, np.uint16)
    S = kv.shape[0]
    pos = _c(pos, np.int64)
    dout = _c(dout, np.uint16)
    dq = np.empty((T, H, D_qk), dtype=np.float64)
    dkv = np.empty((S, D_qk), dtype=np.float64)
    rc = lib.oracle_sparse_mla_bwd(_ptr(q), _ptr(idx), _ptr(pos), T, H, D_qk, D_v, k, _ptr(kv), S,
                                   ctypes.c_double(sm_scale), _ptr(dout), _ptr(dq), _ptr(dkv), nthreads)
    if rc:
        raise RuntimeError("oracle_sparse_mla_bwd failed (%d)" % rc)
    return dq, dkv

