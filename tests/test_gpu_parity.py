"""HIP path vs the oracle on the same seeded inputs, through the C ABI (needs an MI355X)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import get, prefill_inputs
from dsa_inputs.configs import Workload
import parity
from gpu_helpers import PrefillDev, bf16_vals, dget, dims_of, dput, paged_from_contiguous, run_chain

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_02_amd as dsa
    dsa.load()
    return torch.device("cuda:0")


def _log(*a):
    print(*a, flush=True)


def _full_check(wl, dev, mla_rows=None, idx_rows=None):
    """Whole-path parity for a prefill workload; oracle on all rows or on the given subsets."""
    _log("case", wl.name, "T", wl.T, "S", wl.S)
    inp = prefill_inputs(wl)
    d = PrefillDev(inp, dev)
    logits, idx, out, out_f32, lse = run_chain(d)
    torch.cuda.synchronize()
    S = wl.S
    rows = np.arange(wl.T) if idx_rows is None else np.asarray(idx_rows)
    pos = wl.q_start + rows
    g_logits = dget(logits[torch.from_numpy(rows).to(dev)])[:, :S]
    n = np.minimum(S, pos + 1)
    g_logits[np.arange(S)[None, :] >= n[:, None]] = np.nan
    # 1. indexer
    o_logits = oracle.indexer(inp.q8[rows], inp.qs[rows], inp.w[rows], pos, inp.k8, inp.ks)
    A = parity.magnitude(inp.q8[rows], inp.qs[rows], inp.w[rows], inp.k8, inp.ks, pos, S)
    worst = parity.check_indexer(g_logits, o_logits, A, wl.D_I, wl.H_I)
    if len(rows) <= 64 or wl.S <= 4096:
        import brute
        exact, _ = brute.indexer(inp.q8[rows], inp.qs[rows], inp.w[rows], pos, inp.k8, inp.ks)
        vs_exact = parity.check_indexer_exact(g_logits, exact, A)
        _log("  indexer |g-exact|/A %.2e" % vs_exact)
    # 2. top-k: exact on the GPU's own logits, boundary rule against the oracle's logits
    g_idx = dget(idx)[rows]
    o_idx_same = oracle.topk(np.nan_to_num(g_logits, nan=0.0), pos, wl.topk)
    parity.check_topk_exact(g_idx, o_idx_same)
    o_idx = oracle.topk(np.nan_to_num(o_logits, nan=0.0), pos, wl.topk)
    swaps = parity.check_topk_boundary(g_idx, o_idx, o_logits, n)
    # 3. attention on the GPU's own index lists
    mrows = rows if mla_rows is None else np.asarray(mla_rows)
    mpos = wl.q_start + mrows
    o_out, _, o_lse = oracle.sparse_mla(inp.q[mrows], dget(idx)[mrows], mpos, inp.kv, wl.D_v, wl.sm_scale)
    sel = torch.from_numpy(mrows).to(dev)
    abs_err, rel = parity.check_mla(bf16_vals(out[sel]), dget(out_f32[sel]), dget(lse[sel]), o_out, o_lse)
    _log("  indexer worst |g-o|/A %.2e, boundary swaps %d, mla bf16 abs %.2e f32 rel %.2e"
         % (worst, swaps, abs_err, rel))
    return d, (logits, idx, out, out_f32, lse)


def test_tiny_full(dev):
    _full_check(get("tiny"), dev)


def test_prefill_4k(dev):
    wl = get("prefill_4k")
    rows = np.unique(np.concatenate([np.arange(0, 4096, 61), [0, 1, 2047, 2048, 2049, 4094, 4095]]))
    mla_rows = np.array([0, 1, 17, 1000, 2046, 2047, 2048, 2049, 3001, 4095])
    _full_check(wl, dev, mla_rows=mla_rows, idx_rows=rows)


def test_ragged_small_prefill(dev):
    """T not a multiple of any tile, q_start > 0, rows with n_t < k and n_t > k."""
    base = get("tiny")
    wl = Workload(**{**base.__dict__, "name": "ragged", "T": 77, "S": 150, "q_start": 20, "topk": 64})
    _full_check(wl, dev)


def test_prefill_32k_sampled(dev):
    """Full-size headline workload in the launch configuration the bench times; sampled rows."""
    wl = get("prefill_32k")
    rows = np.array([0, 1, 2047, 2048, 4095, 16383, 16384, 30001, 32766, 32767])
    _full_check(wl, dev, mla_rows=rows[[0, 2, 3, 6, 9]], idx_rows=rows)


def test_chunked_131k_sampled(dev):
    wl = get("chunked_131k")
    rows = np.array([0, 1, 4095, 8190, 8191])
    _full_check(wl, dev, mla_rows=rows[[0, 2, 4]], idx_rows=rows)


# ----------------------------------------------------------------------------------- structure
def test_paged_equals_contiguous_and_fused_equals_chain(dev):
    import dsa_lightning_indexer_02_amd as dsa
    for name in ("tiny", "prefill_4k"):
        wl = get(name)
        _log("case paged/fused", name)
        inp = prefill_inputs(wl)
        d = PrefillDev(inp, dev)
        logits, idx, out, out_f32, lse = run_chain(d)
        nb = (wl.S + 63) // 64
        perm = np.random.Generator(np.random.PCG64(5)).permutation(nb).astype(np.int32)
        for p in (None, perm):
            cache = paged_from_contiguous(d, 64, p)
            o2, f2, l2, i2 = dsa.dsa_prefill_paged(cache, 0, dims_of(wl), wl.q_start, d.q8, d.qs, d.w, d.q,
                                                   want_f32=True, want_indices=True)
            torch.cuda.synchronize()
            assert torch.equal(i2, idx), "fused indices differ from the standalone chain"
            assert torch.equal(o2.view(torch.int16), out.view(torch.int16))
            assert torch.equal(f2, out_f32) and torch.equal(l2, lse)


def _bits(x: torch.Tensor) -> torch.Tensor:
    return x.view(torch.int32) if x.element_size() == 4 else x.view(torch.int16)


def test_determinism(dev):
    wl = get("prefill_4k")
    inp = prefill_inputs(wl)
    d = PrefillDev(inp, dev)
    a = run_chain(d)
    b = run_chain(d)
    torch.cuda.synchronize()
    S = wl.S
    assert torch.equal(_bits(a[0][:, :S].nan_to_num(0).tril()), _bits(b[0][:, :S].nan_to_num(0).tril()))
    for x, y in zip(a[1:], b[1:]):
        assert torch.equal(_bits(x), _bits(y))


def test_t_zero_is_noop(dev):
    import dsa_lightning_indexer_02_amd as dsa
    wl = get("tiny")
    inp = prefill_inputs(wl)
    d = PrefillDev(inp, dev)
    logits = torch.full((0, 256), 7.0, device=dev)
    out = dsa.dsa_indexer_logits(d.q8[:0], d.qs[:0], d.w[:0], d.k8, d.ks, 0, logits)
    assert out.shape == (0, 256)
    idx = dsa.dsa_topk(logits, 64, 256)
    assert idx.shape == (0, 64)
