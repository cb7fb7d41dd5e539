"""ctypes binding of libdsa.so (the C ABI declared in include/dsa.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels.  Torch
tensors are accepted for their device pointers and the current HIP stream; no torch operator
computes any part of the method.  The library must have been built (``build.py``); a missing
library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

DSA_OK = 0
TOPK_NOALLOC_SCRATCH_BYTES = 32 << 20   # DSA_TOPK_NOALLOC_SCRATCH_BYTES of include/dsa.h
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARGUMENT", 2: "DSA_ERR_UNSUPPORTED",
                3: "DSA_ERR_WORKSPACE_TOO_SMALL", 4: "DSA_ERR_HIP"}

EXPORTS = [
    "dsa_status_string", "dsa_last_error", "dsa_abi_version", "dsa_profile_begin", "dsa_profile_end",
    "dsa_profile_kernel_name", "dsa_indexer_logits",
    "dsa_topk_workspace_size", "dsa_topk", "dsa_topk_noalloc",
    "dsa_sparse_mla_workspace_size", "dsa_sparse_mla_fwd", "dsa_sparse_mla_bwd_workspace_size",
    "dsa_sparse_mla_bwd",
    "dsa_prefill_workspace_size", "dsa_prefill_paged", "dsa_decode_workspace_size", "dsa_decode_paged",
    "dsa_quantize_fp8_rows", "dsa_append_paged", "dsa_quantize_fp8_rows_ue8m0", "dsa_indexer_logits_ue8m0",
    "dsa_indexer_kl_loss", "dsa_indexer_bwd_workspace_size", "dsa_indexer_bwd", "dsa_indexer_kl_loss_sparse",
    "dsa_indexer_bwd_listed",
]

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_f32 = ctypes.c_float


class PagedCache(ctypes.Structure):
    _fields_ = [("k8", _p), ("k_scale", _p), ("kv", _p), ("num_blocks", _i64), ("block_size", _i32),
                ("block_table", _p), ("max_blocks_per_seq", _i64), ("seq_lens", _p)]


class Dims(ctypes.Structure):
    _fields_ = [("H_I", _i32), ("D_I", _i32), ("H", _i32), ("D_qk", _i32), ("D_v", _i32),
                ("topk", _i32), ("sm_scale", _f32)]


class DSAError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__("%s failed: %s: %s" % (fn, STATUS_NAMES.get(status, status), message))
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libdsa.so once; raises OSError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError("libdsa.so not found at %s: run dsa_lightning_indexer_02_amd/build.py "
                      "(or __graft_entry__.build()) first" % path)
    lib = ctypes.CDLL(path)
    lib.dsa_status_string.argtypes = [ctypes.c_int]
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_abi_version.argtypes = []
    lib.dsa_abi_version.restype = ctypes.c_int
    lib.dsa_profile_begin.argtypes = [_p, _i32]
    lib.dsa_profile_begin.restype = ctypes.c_int
    lib.dsa_profile_end.argtypes = []
    lib.dsa_profile_end.restype = _i32
    lib.dsa_profile_kernel_name.argtypes = [_i32]
    lib.dsa_profile_kernel_name.restype = ctypes.c_char_p
    lib.dsa_indexer_logits.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i64, _p, _i64, _p]
    lib.dsa_topk_workspace_size.argtypes = [_i64, _i64, _i32]
    lib.dsa_topk_workspace_size.restype = _sz
    lib.dsa_topk.argtypes = [_p, _i64, _i64, _i64, _i64, _i32, _p, _p, _sz, _p]
    lib.dsa_topk_noalloc.argtypes = [_p, _i64, _i64, _i64, _i64, _i32, _p, _p]
    lib.dsa_topk_noalloc.restype = ctypes.c_int
    lib.dsa_sparse_mla_workspace_size.argtypes = [_i64, _i64, _i32, _i32, _i32, _i32]
    lib.dsa_sparse_mla_workspace_size.restype = _sz
    lib.dsa_sparse_mla_fwd.argtypes = [_p, _p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _i64, _f32, _p, _p,
                                       _p, _p, _sz, _p]
    lib.dsa_sparse_mla_bwd_workspace_size.argtypes = [_i64, _i64, _i32, _i32]
    lib.dsa_sparse_mla_bwd_workspace_size.restype = _sz
    lib.dsa_sparse_mla_bwd.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _i64, _f32, _p, _p, _p,
                                       _sz, _p]
    lib.dsa_sparse_mla_bwd.restype = ctypes.c_int
    lib.dsa_prefill_workspace_size.argtypes = [ctypes.POINTER(Dims), _i64, _i64]
    lib.dsa_prefill_workspace_size.restype = _sz
    lib.dsa_prefill_paged.argtypes = [ctypes.POINTER(PagedCache), _i32, ctypes.POINTER(Dims), _i64, _i64,
                                      _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]
    lib.dsa_decode_workspace_size.argtypes = [ctypes.POINTER(Dims), _i32, _i64]
    lib.dsa_decode_workspace_size.restype = _sz
    lib.dsa_decode_paged.argtypes = [ctypes.POINTER(PagedCache), _i32, _i64, ctypes.POINTER(Dims), _p, _p, _p,
                                     _p, _p, _p, _p, _p, _p, _sz, _p]
    lib.dsa_quantize_fp8_rows.argtypes = [_p, _i64, _i32, _p, _p, _p]
    lib.dsa_append_paged.argtypes = [ctypes.POINTER(PagedCache), _i32, _p, _p, _i64, _i32, _i32, _p, _p, _p]
    lib.dsa_quantize_fp8_rows_ue8m0.argtypes = [_p, _i64, _i32, _p, _p, _p, _p]
    lib.dsa_indexer_logits_ue8m0.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i64, _p, _i64, _p]
    lib.dsa_indexer_kl_loss.argtypes = [_p, _p, _i64, _i64, _i32, _i32, _f32, _i64, _p, _i64, _p, _p, _p]
    lib.dsa_indexer_kl_loss_sparse.argtypes = [_p, _p, _p, _i32, _p, _i64, _i64, _i32, _i32, _f32, _i64, _p, _i64,
                                               _p, _p, _p]
    lib.dsa_indexer_bwd_workspace_size.argtypes = [_i64, _i64, _i32]
    lib.dsa_indexer_bwd_workspace_size.restype = _sz
    lib.dsa_indexer_bwd.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i64, _p, _i64, _p, _p, _p, _p,
                                    _sz, _p]
    lib.dsa_indexer_bwd_listed.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i64, _p, _i32, _p, _i64, _p,
                                           _p, _p, _p, _sz, _p]
    for name in ("dsa_indexer_logits", "dsa_topk", "dsa_sparse_mla_fwd", "dsa_prefill_paged",
                 "dsa_decode_paged", "dsa_quantize_fp8_rows", "dsa_append_paged", "dsa_quantize_fp8_rows_ue8m0",
                 "dsa_indexer_logits_ue8m0", "dsa_indexer_kl_loss", "dsa_indexer_bwd",
                 "dsa_indexer_kl_loss_sparse", "dsa_indexer_bwd_listed"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def check(fn: str, status: int):
    if status != DSA_OK:
        msg = load().dsa_last_error().decode(errors="replace")
        raise DSAError(fn, status, msg)
