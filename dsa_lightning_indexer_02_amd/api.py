"""Python entry points with the same names as the C ABI, over torch device tensors.

Each function checks shapes and dtypes, allocates any output the caller did not pass (torch
as the device allocator), and calls the library on the current HIP stream.  Nothing here
computes any part of the method.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from ._lib import Dims, PagedCache, check, load

_BYTES = {1: (torch.uint8, torch.int8, torch.float8_e4m3fn),
          2: (torch.bfloat16, torch.int16, torch.uint16),
          4: (torch.float32, torch.int32)}


def _dev(t: torch.Tensor, name: str, ndim: int, itemsize: int) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %s" % (name, ndim, tuple(t.shape)))
    if t.element_size() != itemsize:
        raise ValueError("%s must have %d-byte elements, got %s" % (name, itemsize, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _opt(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def ld_for(S: int) -> int:
    return (S + 3) // 4 * 4


# ------------------------------------------------------------------------------------------------
_profile_handles = None  # the event-handle array the library records into (kept alive while active)


def dsa_profile_begin(events) -> None:
    """Start stage timing on this thread: the kernels of the following dsa_* calls record
    ``events`` (torch.cuda.Event(enable_timing=True) objects) in launch order, one after each kernel."""
    global _profile_handles
    lib = load()
    handles = []
    for ev in events:
        if not ev.cuda_event:       # torch creates the HIP event at its first record
            ev.record()
        handles.append(ev.cuda_event)
    _profile_handles = (ctypes.c_void_p * len(handles))(*handles)
    check("dsa_profile_begin", lib.dsa_profile_begin(ctypes.cast(_profile_handles, ctypes.c_void_p), len(handles)))


def dsa_profile_end():
    """Stop stage timing; returns the kernel names behind the events recorded, in order."""
    lib = load()
    n = lib.dsa_profile_end()
    return [lib.dsa_profile_kernel_name(i).decode() for i in range(n)]


def dsa_profile_kernel_name(i: int) -> str:
    return load().dsa_profile_kernel_name(i).decode()


# ------------------------------------------------------------------------------------------------
def dsa_indexer_logits(q8, q_scale, w, k8, k_scale, q_start: int = 0, logits=None) -> torch.Tensor:
    """Index scores into ``logits`` [T, ld >= S] float32 (entries past each row's causal range untouched)."""
    lib = load()
    T, H_I, D_I = q8.shape
    S = k8.shape[0]
    if logits is None:
        logits = torch.empty((T, ld_for(S)), dtype=torch.float32, device=q8.device)
    status = lib.dsa_indexer_logits(
        _dev(q8, "q8", 3, 1), _dev(q_scale, "q_scale", 2, 4), _dev(w, "w", 2, 4), _dev(k8, "k8", 2, 1),
        _dev(k_scale, "k_scale", 1, 4), T, S, H_I, D_I, q_start, _dev(logits, "logits", 2, 4),
        logits.shape[1], _stream(q8))
    check("dsa_indexer_logits", status)
    return logits


def dsa_topk(logits, k: int, S: int, q_start: int = 0, indices=None, workspace=None) -> torch.Tensor:
    """Top-k key indices [T, k] int32 of each logits row's visible part (-1 padded)."""
    lib = load()
    T = logits.shape[0]
    if indices is None:
        indices = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    need = lib.dsa_topk_workspace_size(T, S, k)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    status = lib.dsa_topk(_dev(logits, "logits", 2, 4), logits.shape[1], T, S, q_start, k,
                          _dev(indices, "indices", 2, 4), _opt(workspace), ws_bytes, _stream(logits))
    check("dsa_topk", status)
    return indices


def dsa_topk_noalloc(logits, k: int, S: int, q_start: int = 0, indices=None) -> torch.Tensor:
    """dsa_topk without a workspace (the library's own per-GPU scratch array); ``indices`` given
    makes the call allocate nothing at all."""
    lib = load()
    T = logits.shape[0]
    if indices is None:
        indices = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    status = lib.dsa_topk_noalloc(_dev(logits, "logits", 2, 4), logits.shape[1], T, S, q_start, k,
                                  _dev(indices, "indices", 2, 4), _stream(logits))
    check("dsa_topk_noalloc", status)
    return indices


def dsa_sparse_mla_fwd(q, kv, indices, sm_scale: float, D_v: int, q_start: int = 0, out=None,
                       out_f32=None, lse=None, want_f32: bool = False, want_lse: bool = True,
                       staging: str = "fp16", workspace=None):
    """(out bf16 [T,H,D_v], out_f32 or None, lse or None) of MQA-mode sparse MLA.  ``staging``
    "fp16" passes a workspace (the library's fp16 staging where the dims have it), "bf16" none."""
    lib = load()
    T, H, D_qk = q.shape
    S = kv.shape[0]
    k = indices.shape[1]
    dev = q.device
    if staging not in ("fp16", "bf16"):
        raise ValueError("staging must be 'fp16' or 'bf16'")
    ws_ptr, ws_bytes = None, 0
    if staging == "fp16":
        need = lib.dsa_sparse_mla_workspace_size(T, S, H, D_qk, D_v, k)
        if need > 0:
            workspace = _workspace(need, dev, workspace)
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty((T, H, D_v), dtype=torch.bfloat16, device=dev)
    if out_f32 is None and want_f32:
        out_f32 = torch.empty((T, H, D_v), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    status = lib.dsa_sparse_mla_fwd(
        _dev(q, "q", 3, 2), _dev(kv, "kv", 2, 2), _dev(indices, "indices", 2, 4), T, S, H, D_qk, D_v, k,
        q_start, ctypes.c_float(sm_scale), _dev(out, "out", 3, 2), _opt(out_f32), _opt(lse), ws_ptr, ws_bytes,
        _stream(q))
    check("dsa_sparse_mla_fwd", status)
    return out, out_f32, lse


def dsa_sparse_mla_bwd(q, kv, indices, lse, dout, sm_scale: float, q_start: int = 0, dq=None, dkv=None,
                       workspace=None):
    """(dq f32 [T, H, D_qk], dkv f32 [S, D_qk]): gradients through dsa_sparse_mla_fwd on the same index
    lists, given the forward's lse and dout = dL/dout (bf16 [T, H, D_v])."""
    lib = load()
    T, H, D_qk = q.shape
    S = kv.shape[0]
    k = indices.shape[1]
    D_v = dout.shape[2]
    dev = q.device
    if dq is None:
        dq = torch.empty((T, H, D_qk), dtype=torch.float32, device=dev)
    if dkv is None:
        dkv = torch.empty((S, D_qk), dtype=torch.float32, device=dev)
    workspace = _workspace(lib.dsa_sparse_mla_bwd_workspace_size(T, S, H, k), dev, workspace)
    status = lib.dsa_sparse_mla_bwd(
        _dev(q, "q", 3, 2), _dev(kv, "kv", 2, 2), _dev(indices, "indices", 2, 4), _dev(lse, "lse", 2, 4),
        _dev(dout, "dout", 3, 2), T, S, H, D_qk, D_v, k, q_start, ctypes.c_float(sm_scale),
        _dev(dq, "dq", 3, 4), _dev(dkv, "dkv", 2, 4), workspace.data_ptr(), workspace.numel(), _stream(q))
    check("dsa_sparse_mla_bwd", status)
    return dq, dkv


# ------------------------------------------------------------------------------------------------
@dataclass
class PagedKV:
    """Paged cache tensors: pools [NB, bs, ...], block_table [B, max_blocks] i32, seq_lens [B] i32."""
    k8: torch.Tensor
    k_scale: torch.Tensor
    kv: torch.Tensor
    block_table: torch.Tensor
    seq_lens: Optional[torch.Tensor] = None

    def struct(self) -> PagedCache:
        NB, bs, _ = self.k8.shape
        _dev(self.k8, "k8 pool", 3, 1)
        _dev(self.k_scale, "k_scale pool", 2, 4)
        _dev(self.kv, "kv pool", 3, 2)
        _dev(self.block_table, "block_table", 2, 4)
        if self.seq_lens is not None:
            _dev(self.seq_lens, "seq_lens", 1, 4)
        return PagedCache(self.k8.data_ptr(), self.k_scale.data_ptr(), self.kv.data_ptr(), NB, bs,
                          self.block_table.data_ptr(), self.block_table.shape[1], _opt(self.seq_lens))


def make_dims(H_I, D_I, H, D_qk, D_v, topk, sm_scale) -> Dims:
    return Dims(H_I, D_I, H, D_qk, D_v, topk, sm_scale)


def prefill_workspace_size(dims: Dims, T: int, S: int) -> int:
    return load().dsa_prefill_workspace_size(ctypes.byref(dims), T, S)


def decode_workspace_size(dims: Dims, B: int, max_seq_len: int) -> int:
    return load().dsa_decode_workspace_size(ctypes.byref(dims), B, max_seq_len)


def _workspace(nbytes: int, device, given=None):
    if given is not None and given.numel() * given.element_size() >= nbytes:
        return given
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def dsa_prefill_paged(cache: PagedKV, seq: int, dims: Dims, q_start: int, q8, q_scale, w, q, out=None,
                      want_f32: bool = False, want_lse: bool = True, want_indices: bool = False,
                      workspace=None):
    """Fused indexer -> top-k -> sparse MLA for T queries of sequence ``seq`` at q_start .. q_start+T-1."""
    lib = load()
    T = q8.shape[0]
    dev = q8.device
    if out is None:
        out = torch.empty((T, dims.H, dims.D_v), dtype=torch.bfloat16, device=dev)
    out_f32 = torch.empty((T, dims.H, dims.D_v), dtype=torch.float32, device=dev) if want_f32 else None
    lse = torch.empty((T, dims.H), dtype=torch.float32, device=dev) if want_lse else None
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device=dev) if want_indices else None
    ws = _workspace(prefill_workspace_size(dims, T, q_start + T), dev, workspace)
    c = cache.struct()
    status = lib.dsa_prefill_paged(
        ctypes.byref(c), seq, ctypes.byref(dims), T, q_start, _dev(q8, "q8", 3, 1),
        _dev(q_scale, "q_scale", 2, 4), _dev(w, "w", 2, 4), _dev(q, "q", 3, 2), _dev(out, "out", 3, 2),
        _opt(out_f32), _opt(lse), _opt(idx), ws.data_ptr(), ws.numel(), _stream(q8))
    check("dsa_prefill_paged", status)
    return out, out_f32, lse, idx


def dsa_decode_paged(cache: PagedKV, max_seq_len: int, dims: Dims, q8, q_scale, w, q, out=None,
                     want_f32: bool = False, want_lse: bool = True, want_indices: bool = False,
                     workspace=None):
    """Fused decode: one query per sequence at position seq_lens[b] - 1."""
    lib = load()
    B = q8.shape[0]
    dev = q8.device
    if out is None:
        out = torch.empty((B, dims.H, dims.D_v), dtype=torch.bfloat16, device=dev)
    out_f32 = torch.empty((B, dims.H, dims.D_v), dtype=torch.float32, device=dev) if want_f32 else None
    lse = torch.empty((B, dims.H), dtype=torch.float32, device=dev) if want_lse else None
    idx = torch.empty((B, dims.topk), dtype=torch.int32, device=dev) if want_indices else None
    ws = _workspace(decode_workspace_size(dims, B, max_seq_len), dev, workspace)
    c = cache.struct()
    status = lib.dsa_decode_paged(
        ctypes.byref(c), B, max_seq_len, ctypes.byref(dims), _dev(q8, "q8", 3, 1),
        _dev(q_scale, "q_scale", 2, 4), _dev(w, "w", 2, 4), _dev(q, "q", 3, 2), _dev(out, "out", 3, 2),
        _opt(out_f32), _opt(lse), _opt(idx), ws.data_ptr(), ws.numel(), _stream(q8))
    check("dsa_decode_paged", status)
    return out, out_f32, lse, idx


def decode_scores(workspace: torch.Tensor, B: int, max_seq_len: int) -> torch.Tensor:
    """The index scores a completed dsa_decode_paged call left at the start of its workspace:
    fp32 [B, ld] with ld = ld_for(max_seq_len); entries s < seq_lens[b] of row b are the scores
    the top-k selected from (the layout include/dsa.h documents for the decode workspace)."""
    ld = ld_for(max_seq_len)
    nbytes = B * ld * 4
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace smaller than the %d-byte score prefix" % nbytes)
    return workspace.view(torch.uint8).reshape(-1)[:nbytes].view(torch.float32).view(B, ld)


# ------------------------------------------------------------------------------------------------
def dsa_quantize_fp8_rows(x, codes=None, scales=None):
    """Per-row FP8 E4M3 codes (uint8, x's shape) and fp32 scales (x's shape without the last dim)
    of a bf16 tensor x [..., D]."""
    lib = load()
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    nd = x.dim()
    status = lib.dsa_quantize_fp8_rows(_dev(x, "x", nd, 2), rows, D, _dev(codes, "codes", nd, 1),
                                       _dev(scales, "scales", nd - 1, 4) if nd > 1 else scales.data_ptr(),
                                       _stream(x))
    check("dsa_quantize_fp8_rows", status)
    return codes, scales


def dsa_append_paged(cache: PagedKV, seq_ids, positions, k, kv):
    """Write tokens (seq_ids[i], positions[i]) into the cache's pools: the FP8 codes and scale of
    their bf16 indexer keys k [n, D_I] and their bf16 latent rows kv [n, D_qk]."""
    lib = load()
    n, D_I = k.shape
    D_qk = kv.shape[1]
    B = cache.block_table.shape[0]
    c = cache.struct()
    status = lib.dsa_append_paged(ctypes.byref(c), B, _dev(seq_ids, "seq_ids", 1, 4),
                                  _dev(positions, "positions", 1, 4), n, D_I, D_qk, _dev(k, "k", 2, 2),
                                  _dev(kv, "kv", 2, 2), _stream(k))
    check("dsa_append_paged", status)


def dsa_quantize_fp8_rows_ue8m0(x, codes=None, exps=None, scales=None, want_scales: bool = True):
    """Per-row FP8 codes with power-of-two scales: (codes uint8 [..., D], biased exponents uint8
    [...], scales fp32 [...] or None) of a bf16 tensor x [..., D]."""
    lib = load()
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if exps is None:
        exps = torch.empty(x.shape[:-1], dtype=torch.uint8, device=x.device)
    if scales is None and want_scales:
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    nd = x.dim()
    status = lib.dsa_quantize_fp8_rows_ue8m0(_dev(x, "x", nd, 2), rows, D, _dev(codes, "codes", nd, 1),
                                             _dev(exps, "exps", nd - 1, 1), _opt(scales), _stream(x))
    check("dsa_quantize_fp8_rows_ue8m0", status)
    return codes, exps, scales


def dsa_indexer_logits_ue8m0(q8, q_exp, w, k8, k_exp, q_start: int = 0, logits=None) -> torch.Tensor:
    """Index scores with UE8M0 exponent scales applied inside the FP8 MFMA (see dsa_indexer_logits)."""
    lib = load()
    T, H_I, D_I = q8.shape
    S = k8.shape[0]
    if logits is None:
        logits = torch.empty((T, ld_for(S)), dtype=torch.float32, device=q8.device)
    status = lib.dsa_indexer_logits_ue8m0(
        _dev(q8, "q8", 3, 1), _dev(q_exp, "q_exp", 2, 1), _dev(w, "w", 2, 4), _dev(k8, "k8", 2, 1),
        _dev(k_exp, "k_exp", 1, 1), T, S, H_I, D_I, q_start, _dev(logits, "logits", 2, 4), logits.shape[1],
        _stream(q8))
    check("dsa_indexer_logits_ue8m0", status)
    return logits


def dsa_indexer_kl_loss(q, kv, logits, sm_scale: float, q_start: int = 0, dlogits=None, loss=None,
                        in_place: bool = False):
    """(loss f32 [T], dlogits f32 [T, ld]) of the indexer's KL loss toward the head-averaged main
    attention; dlogits = softmax(logits) - p on each row's visible entries.  in_place overwrites
    logits with dlogits."""
    lib = load()
    T, H, D_qk = q.shape
    S = kv.shape[0]
    if dlogits is None:
        dlogits = logits if in_place else torch.empty_like(logits)
    if loss is None:
        loss = torch.empty((T,), dtype=torch.float32, device=q.device)
    status = lib.dsa_indexer_kl_loss(
        _dev(q, "q", 3, 2), _dev(kv, "kv", 2, 2), T, S, H, D_qk, ctypes.c_float(sm_scale), q_start,
        _dev(logits, "logits", 2, 4), logits.shape[1], _dev(dlogits, "dlogits", 2, 4), _dev(loss, "loss", 1, 4),
        _stream(q))
    check("dsa_indexer_kl_loss", status)
    return loss, dlogits


def dsa_indexer_kl_loss_sparse(q, kv, indices, lse, logits, sm_scale: float, q_start: int = 0, dlogits=None,
                               loss=None, in_place: bool = False):
    """(loss f32 [T], dlogits f32 [T, ld]) of the sparse-stage indexer loss over each row's index-list
    entries; lse is the sparse forward's [T, H] log-normaliser over the same lists."""
    lib = load()
    T, H, D_qk = q.shape
    S = kv.shape[0]
    k = indices.shape[1]
    if dlogits is None:
        dlogits = logits if in_place else torch.empty_like(logits)
    if loss is None:
        loss = torch.empty((T,), dtype=torch.float32, device=q.device)
    status = lib.dsa_indexer_kl_loss_sparse(
        _dev(q, "q", 3, 2), _dev(kv, "kv", 2, 2), _dev(indices, "indices", 2, 4), k, _dev(lse, "lse", 2, 4), T, S, H,
        D_qk, ctypes.c_float(sm_scale), q_start, _dev(logits, "logits", 2, 4), logits.shape[1],
        _dev(dlogits, "dlogits", 2, 4), _dev(loss, "loss", 1, 4), _stream(q))
    check("dsa_indexer_kl_loss_sparse", status)
    return loss, dlogits


def indexer_bwd_workspace_size(T: int, S: int, D_I: int) -> int:
    return load().dsa_indexer_bwd_workspace_size(T, S, D_I)


def dsa_indexer_bwd(q8, q_scale, w, k8, k_scale, dlogits, q_start: int = 0, dq=None, dw=None, dk=None,
                    workspace=None):
    """(dq [T, H_I, D_I], dw [T, H_I], dk [S, D_I]) f32: gradients through the index scores for
    dlogits = dL/dlogits, with respect to the dequantized q_I, k_I and the weights w."""
    lib = load()
    T, H_I, D_I = q8.shape
    S = k8.shape[0]
    dev = q8.device
    if dq is None:
        dq = torch.empty((T, H_I, D_I), dtype=torch.float32, device=dev)
    if dw is None:
        dw = torch.empty((T, H_I), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((S, D_I), dtype=torch.float32, device=dev)
    workspace = _workspace(lib.dsa_indexer_bwd_workspace_size(T, S, D_I), dev, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    status = lib.dsa_indexer_bwd(
        _dev(q8, "q8", 3, 1), _dev(q_scale, "q_scale", 2, 4), _dev(w, "w", 2, 4), _dev(k8, "k8", 2, 1),
        _dev(k_scale, "k_scale", 1, 4), T, S, H_I, D_I, q_start, _dev(dlogits, "dlogits", 2, 4), dlogits.shape[1],
        _dev(dq, "dq", 3, 4), _dev(dw, "dw", 2, 4), _dev(dk, "dk", 2, 4), _opt(workspace), ws_bytes, _stream(q8))
    check("dsa_indexer_bwd", status)
    return dq, dw, dk


def dsa_indexer_bwd_listed(q8, q_scale, w, k8, k_scale, indices, dlogits, q_start: int = 0, dq=None, dw=None,
                           dk=None, workspace=None):
    """dsa_indexer_bwd for a dlogits that vanishes off each row's index list (indices [T, k] i32,
    distinct valid entries per row): dq and dw are summed over the listed keys only."""
    lib = load()
    T, H_I, D_I = q8.shape
    S = k8.shape[0]
    k = indices.shape[1]
    dev = q8.device
    if dq is None:
        dq = torch.empty((T, H_I, D_I), dtype=torch.float32, device=dev)
    if dw is None:
        dw = torch.empty((T, H_I), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((S, D_I), dtype=torch.float32, device=dev)
    workspace = _workspace(lib.dsa_indexer_bwd_workspace_size(T, S, D_I), dev, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    status = lib.dsa_indexer_bwd_listed(
        _dev(q8, "q8", 3, 1), _dev(q_scale, "q_scale", 2, 4), _dev(w, "w", 2, 4), _dev(k8, "k8", 2, 1),
        _dev(k_scale, "k_scale", 1, 4), T, S, H_I, D_I, q_start, _dev(indices, "indices", 2, 4), k,
        _dev(dlogits, "dlogits", 2, 4), dlogits.shape[1], _dev(dq, "dq", 3, 4), _dev(dw, "dw", 2, 4),
        _dev(dk, "dk", 2, 4), _opt(workspace), ws_bytes, _stream(q8))
    check("dsa_indexer_bwd_listed", status)
    return dq, dw, dk
