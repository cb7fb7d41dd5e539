"""Shared helpers of the GPU tests: host <-> device copies and the standalone / fused runs."""
from __future__ import annotations

import numpy as np
import torch

import dsa_lightning_indexer_02_amd as dsa


def dput(a: np.ndarray, dev) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev)
    return torch.from_numpy(a).to(dev)


def dget(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_vals(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


class PrefillDev:
    """Device copies of dsa_inputs.PrefillInputs (all query rows present)."""

    def __init__(self, inp, dev):
        self.inp = inp
        self.q8 = dput(inp.q8, dev)
        self.qs = dput(inp.qs, dev)
        self.w = dput(inp.w, dev)
        self.k8 = dput(inp.k8, dev)
        self.ks = dput(inp.ks, dev)
        self.q = dput(inp.q, dev).view(torch.bfloat16)
        self.kv = dput(inp.kv, dev).view(torch.bfloat16)


def run_chain(d: PrefillDev, staging: str = "fp16"):
    wl = d.inp.wl
    S = d.k8.shape[0]
    logits = dsa.dsa_indexer_logits(d.q8, d.qs, d.w, d.k8, d.ks, q_start=wl.q_start)
    idx = dsa.dsa_topk(logits, wl.topk, S, q_start=wl.q_start)
    out, out_f32, lse = dsa.dsa_sparse_mla_fwd(d.q, d.kv, idx, wl.sm_scale, wl.D_v, q_start=wl.q_start,
                                               want_f32=True, staging=staging)
    return logits, idx, out, out_f32, lse


def dims_of(wl):
    return dsa.make_dims(wl.H_I, wl.D_I, wl.H, wl.D_qk, wl.D_v, wl.topk, wl.sm_scale)


def paged_from_contiguous(d: PrefillDev, block_size: int = 64, perm: np.ndarray = None):
    """One-sequence paged cache holding the prefill keys; ``perm`` permutes the physical blocks."""
    S = d.k8.shape[0]
    nb = (S + block_size - 1) // block_size
    pad = nb * block_size - S
    dev = d.k8.device
    k8 = torch.cat([d.k8, torch.zeros((pad, d.k8.shape[1]), dtype=d.k8.dtype, device=dev)])
    ks = torch.cat([d.ks, torch.zeros((pad,), dtype=d.ks.dtype, device=dev)])
    kv = torch.cat([d.kv, torch.zeros((pad, d.kv.shape[1]), dtype=d.kv.dtype, device=dev)])
    k8 = k8.view(nb, block_size, -1)
    ks = ks.view(nb, block_size)
    kv = kv.view(nb, block_size, -1)
    table = np.arange(nb, dtype=np.int32)
    if perm is not None:
        # logical block j lives in physical block perm[j]
        inv = np.empty_like(perm)
        inv[perm] = np.arange(nb)
        pidx = torch.from_numpy(inv.astype(np.int64)).to(dev)
        k8 = k8[pidx].contiguous()
        ks = ks[pidx].contiguous()
        kv = kv[pidx].contiguous()
        table = perm.astype(np.int32)
    return dsa.PagedKV(k8, ks, kv, dput(table[None, :], dev))


class DecodeDev:
    def __init__(self, inp, dev):
        self.inp = inp
        self.cache = dsa.PagedKV(dput(inp.k8_pool, dev), dput(inp.ks_pool, dev),
                                 dput(inp.kv_pool, dev).view(torch.bfloat16), dput(inp.block_table, dev),
                                 dput(inp.seq_lens, dev))
        self.q8 = dput(inp.q8, dev)
        self.qs = dput(inp.qs, dev)
        self.w = dput(inp.w, dev)
        self.q = dput(inp.q, dev).view(torch.bfloat16)
        self.max_len = int(inp.seq_lens.max())

    def run(self):
        """(out, out_f32, lse, indices, scores): scores = the decode indexer's [B, ld] output, read from
        the workspace prefix the decode call documents."""
        wl = self.inp.wl
        B = self.q8.shape[0]
        ws = torch.empty(dsa.decode_workspace_size(dims_of(wl), B, self.max_len), dtype=torch.uint8,
                         device=self.q8.device)
        res = dsa.dsa_decode_paged(self.cache, self.max_len, dims_of(wl), self.q8, self.qs, self.w, self.q,
                                   want_f32=True, want_indices=True, workspace=ws)
        return res + (dsa.decode_scores(ws, B, self.max_len),)
