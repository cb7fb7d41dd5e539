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


def _full_check(wl, dev, mla_rows=None, idx_rows=None, staging="fp16"):
    """Whole-path parity for a prefill workload; oracle on all rows or on the given subsets."""
    _log("case", wl.name, "T", wl.T, "S", wl.S, "staging", staging)
    inp = prefill_inputs(wl)
    d = PrefillDev(inp, dev)
    logits, idx, out, out_f32, lse = run_chain(d, staging)
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
    worst, share = parity.check_indexer(g_logits, o_logits, A, wl.D_I, wl.H_I)
    _log("  indexer: %d causal entries, worst %.3f of the bar, the 1e-3 relative term dominates on %.1f%%"
         % (int(np.sum(~np.isnan(o_logits))), worst, 100 * share))
    if len(rows) <= 64 or wl.S <= 4096:
        import brute
        exact, _ = brute.indexer(inp.q8[rows], inp.qs[rows], inp.w[rows], pos, inp.k8, inp.ks)
        vs_exact = parity.check_indexer_exact(g_logits, exact, A, wl.D_I, wl.H_I)
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
    _log("  boundary swaps %d, mla rows %d, bf16 abs %.2e f32 rel %.2e" % (swaps, len(mrows), abs_err, rel))
    return d, (logits, idx, out, out_f32, lse)


def test_tiny_full(dev):
    _full_check(get("tiny"), dev)


@pytest.mark.parametrize("staging", ["fp16", "bf16"])
def test_prefill_4k(dev, staging):
    """fp16 staging (latent rows converted in the workspace) and bf16 staging (no workspace)."""
    wl = get("prefill_4k")
    rows = np.unique(np.concatenate([np.arange(0, 4096, 61), [0, 1, 2047, 2048, 2049, 4094, 4095]]))
    mla_rows = np.array([0, 1, 17, 1000, 2046, 2047, 2048, 2049, 3001, 4095])
    _full_check(wl, dev, mla_rows=mla_rows, idx_rows=rows, staging=staging)


def test_ragged_small_prefill(dev):
    """T not a multiple of any tile, q_start > 0, rows with n_t < k and n_t > k."""
    base = get("tiny")
    wl = Workload(**{**base.__dict__, "name": "ragged", "T": 77, "S": 150, "q_start": 20, "topk": 64})
    _full_check(wl, dev)


def _spread(T: int, n: int, extra) -> np.ndarray:
    """n rows evenly spread over [0, T) plus the given ones (the causal triangle's edges)."""
    return np.unique(np.concatenate([np.linspace(0, T - 1, n).round().astype(np.int64), np.asarray(extra)]))


def test_prefill_32k_sampled(dev):
    """Full-size headline workload in the launch configuration the bench times; 66 rows spread over
    the causal triangle, every one checked in all three steps."""
    wl = get("prefill_32k")
    rows = _spread(wl.T, 60, [0, 1, 2047, 2048, 4095, 16383, 16384, 30001, 32766, 32767])
    assert len(rows) >= 64
    _full_check(wl, dev, mla_rows=rows, idx_rows=rows)


def test_chunked_131k_sampled(dev):
    wl = get("chunked_131k")
    rows = _spread(wl.T, 28, [0, 1, 4095, 8190, 8191])
    _full_check(wl, dev, mla_rows=rows, idx_rows=rows)


@pytest.mark.parametrize("D_I", [32, 64, 96, 128])
def test_fp8_mfma_accumulation_bound(dev, D_I):
    """The per-dot accumulation allowance of the FP8 MFMA that the indexer bar uses, re-measured.

    One indexer head with unit weight and unit scales scores relu(dec q8 . dec k8) exactly as the
    MFMA sums it (the epilogue multiplies by 1.0).  The exact dot comes from an fp64 matmul of the
    decoded codes: every E4M3 value is an integer times 2^-9, so products are integers times 2^-18
    below 2^36 and a sum of 128 stays below 2^53 (exact).  Three code distributions: per-row
    absmax-scaled N(0,1) (the workloads' recipe), cubed normals (heavy tails) and codes drawn
    uniformly from all finite codes (subnormals to 448).  The error is reported against several
    magnitude measures of the dot: the sum of |products|, the sum over 32-element blocks of the
    largest |product|, and the sum over blocks of (largest |q|) x (largest |k|)."""
    import brute
    import dsa_lightning_indexer_02_amd as dsa
    from dsa_inputs.generate import block_rng, quantize_fp8_rows
    T, S = 256, 4096
    worst = {}
    normal_worst = 0.0
    for kind in ("normal", "cubed", "uniform-codes"):
        g = block_rng(71, D_I, len(kind))
        if kind == "uniform-codes":
            finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
            q8 = finite[g.integers(0, len(finite), (T, 1, D_I))]
            k8 = finite[g.integers(0, len(finite), (S, D_I))]
        else:
            qx = g.standard_normal((T, 1, D_I)).astype(np.float32)
            kx = g.standard_normal((S, D_I)).astype(np.float32)
            if kind == "cubed":
                qx, kx = qx ** 3, kx ** 3
            q8, _ = quantize_fp8_rows(qx)
            k8, _ = quantize_fp8_rows(kx)
        ones_q = np.ones((T, 1), np.float32)
        lg = dsa.dsa_indexer_logits(dput(np.ascontiguousarray(q8), dev), dput(ones_q, dev), dput(ones_q, dev),
                                    dput(np.ascontiguousarray(k8), dev), dput(np.ones(S, np.float32), dev),
                                    q_start=S)       # every row sees all S keys
        torch.cuda.synchronize()
        gl = dget(lg)[:, :S].astype(np.float64)
        qd, kd = brute.e4m3_decode(q8[:, 0, :]), brute.e4m3_decode(k8)
        err = np.abs(gl - np.maximum(qd @ kd.T, 0.0))
        nb = D_I // 32
        qb = np.abs(qd).reshape(T, nb, 32).max(axis=2)
        kb = np.abs(kd).reshape(S, nb, 32).max(axis=2)
        measures = {"sum|p|": np.abs(qd) @ np.abs(kd).T, "sum_b max|q|max|k|": qb @ kb.T}
        bmax = np.zeros((T, S))
        aq, ak = np.abs(qd).astype(np.float32), np.abs(kd).astype(np.float32)
        for a in range(0, T, 32):
            pr = aq[a:a + 32, None, :] * ak[None, :, :]                   # [32, S, D] exact in fp32
            bmax[a:a + 32] = pr.reshape(len(pr), S, nb, 32).max(axis=3).sum(axis=2)
        measures["sum_b max|p|"] = bmax
        for name, m in measures.items():
            r = float(np.max(err / np.maximum(m, 1e-300)))
            worst[name] = max(worst.get(name, 0.0), r)
            if kind == "normal" and name == "sum|p|":
                normal_worst = r
            _log("  D_I=%d %-13s max err / %-18s = 2^%.2f" % (D_I, kind, name, np.log2(max(r, 1e-300))))
    _log("  D_I=%d worst over the distributions: %s" % (
        D_I, ", ".join("%s 2^%.2f" % (k, np.log2(max(v, 1e-300))) for k, v in worst.items())))
    assert normal_worst <= parity.MFMA_FP8_DOT[D_I], \
        "FP8 MFMA accumulation 2^%.2f of sum|p| on workload-like codes above the allowance 2^%.2f" % (
            np.log2(normal_worst), np.log2(parity.MFMA_FP8_DOT[D_I]))
    assert worst["sum_b max|q|max|k|"] <= parity.MFMA_FP8_BLOCK[D_I], \
        "FP8 MFMA accumulation 2^%.2f of sum_b max|q| max|k| above the allowance 2^%.2f" % (
            np.log2(worst["sum_b max|q|max|k|"]), np.log2(parity.MFMA_FP8_BLOCK[D_I]))


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
