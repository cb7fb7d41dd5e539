"""Edge cases of the top-k and sparse-MLA kernels through the C ABI vs the oracle (needs an MI355X)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import parity
from dsa_inputs.generate import block_rng, to_bf16_bits
from gpu_helpers import bf16_vals, dget, dput

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_02_amd as dsa
    dsa.load()
    return torch.device("cuda:0")


def _topk_case(dev, scores: np.ndarray, q_start: int, k: int, name: str):
    import dsa_lightning_indexer_02_amd as dsa
    print("case", name, scores.shape, "k", k, flush=True)
    T, S = scores.shape
    ld = dsa.ld_for(S)
    host = np.zeros((T, ld), np.float32)
    host[:, :S] = scores
    g = dget(dsa.dsa_topk(dput(host, dev), k, S, q_start=q_start))
    pos = q_start + np.arange(T)
    o = oracle.topk(scores, pos, k)
    parity.check_topk_exact(g, o, name)
    # ordering contract: keys above the k-th score first (ascending), then the ties (ascending)
    for t in range(T):
        v = g[t][g[t] >= 0]
        if min(S, pos[t] + 1) <= k:      # every visible key: ascending index order
            assert np.array_equal(v, np.arange(len(v)))
            continue
        sc = scores[t][v]
        tau = sc.min()
        gt = v[sc > tau]
        eq = v[sc == tau]
        assert np.array_equal(v, np.concatenate([np.sort(gt), np.sort(eq)]))


def test_topk_random_rows(dev):
    g = block_rng(31, 0, 0)
    _topk_case(dev, g.standard_normal((300, 5000)).astype(np.float32), 4000, 2048, "normal")


def test_topk_massive_ties(dev):
    g = block_rng(32, 0, 0)
    s = g.integers(0, 8, size=(64, 6000)).astype(np.float32)
    s[:, ::7] = -0.0
    _topk_case(dev, s, 5900, 2048, "ties")
    _topk_case(dev, np.zeros((8, 3000), np.float32), 2990, 2048, "all-equal")
    _topk_case(dev, s[:, :200], 0, 64, "short rows n_t < k")


def test_topk_k1_and_negative(dev):
    g = block_rng(33, 0, 0)
    s = -np.abs(g.standard_normal((40, 999))).astype(np.float32)
    _topk_case(dev, s, 998, 1, "k=1")
    _topk_case(dev, s, 500, 300, "negative scores")


def test_topk_long_rows_split(dev):
    """Rows longer than one workgroup's chunk (split + merge path), including ties across chunks."""
    g = block_rng(34, 0, 0)
    S = 131072
    s = g.standard_normal((6, S)).astype(np.float32)
    s[1] = np.round(s[1] * 2)          # heavy ties straddling chunk borders
    s[2, 100000:] += 5.0               # all winners in the last chunks
    s[3] = 1.0                         # all equal
    _topk_case(dev, s, S - 6, 2048, "long rows")
    _topk_case(dev, s[:, :70001], 70000 - 5, 2048, "rows of 70001")


def test_topk_heavy_tail(dev):
    g = block_rng(35, 0, 0)
    s = (g.standard_normal((16, 40000)) ** 3).astype(np.float32)
    s[:, g.choice(40000, 400, replace=False)] *= 64.0
    _topk_case(dev, s, 39990, 2048, "heavy tail")


@pytest.mark.parametrize("S", [32768, 131072])
def test_topk_value_range_extremes(dev, S):
    """The pivot and the exact selects bin scores by value over their range: a lone outlier crowds
    every other score into one bin (refinement, then the key radix), a range beyond the float range
    skips the value bins altogether; rows of 32768 take the whole-row kernel, 131072 the chunks and
    the merge."""
    g = block_rng(38, 0, S)
    s = g.standard_normal((6, S)).astype(np.float32)
    s[0, g.integers(0, S)] = 1.0e4                       # crowded bins, refined
    s[1, g.integers(0, S)] = 1.0e6                       # crowded beyond the refinement
    s[2, ::2] = 3.0e38                                   # max - min overflows the float range
    s[2, 1::2] = -3.0e38 * g.random(S // 2).astype(np.float32)
    s[3, g.choice(S, S // 50, replace=False)] *= 1000.0  # a heavy upper tail
    s[4] = np.float32(1.0) + np.float32(2.0 ** -23) * g.integers(0, 4, S).astype(np.float32)  # four values
    s[5, : S // 2] = -0.0
    s[5, S // 2:] = 0.0                                  # signed zeros only
    _topk_case(dev, s, S - 6, 2048, "value-range extremes, rows of %d" % S)


@pytest.mark.parametrize("S", [8192, 16384, 32768])
def test_topk_sample_adversarial(dev, S):
    # A row of n <= 32768 scores is held as EPT = 16, 32 or 64 elements per thread (the narrowest
    # that fits); the pivot comes from a fixed 1-in-16 sample of positions (element 17 i,
    # i < EPT / 16, of every thread: position 64 EPT w + 1024 i + 4 lane + i).  Rows that defeat
    # that sample must still come out exact through the full select: sampled scores far above the
    # rest leave too few candidates above the pivot, far below leave too many.
    ept = S // 512
    sampled = np.array([64 * ept * w + 1024 * i + 4 * l + i
                        for w in range(8) for i in range(ept // 16) for l in range(64)])
    g = block_rng(36, 0, S)
    s = g.standard_normal((4, S)).astype(np.float32)
    s[0, sampled] += 100.0
    s[1, sampled] -= 100.0
    s[2, sampled] = 7.0        # sampled scores all tied, above the rest
    s[3, sampled[::3]] += 50.0
    _topk_case(dev, s, S - 4, 2048, "sample-adversarial rows of %d" % S)


def test_topk_row_lengths_across_layouts(dev):
    # rows whose visible lengths select every register layout, on both sides of each boundary
    g = block_rng(37, 0, 0)
    for n in [4097, 5000, 8191, 8193, 12000, 16383, 16385, 20000]:
        _topk_case(dev, g.standard_normal((1, n)).astype(np.float32), n - 1, 2048, "row of %d" % n)
    # one launch whose consecutive row lengths cross a boundary (rows of 8161 .. 8224 and 16353 .. 16416)
    for first in (8161, 16353):
        _topk_case(dev, g.standard_normal((64, first + 63)).astype(np.float32), first - 1, 2048,
                   "rows of %d .. %d" % (first, first + 63))


# ------------------------------------------------------------------------------------- MLA
def _mla_case(dev, T, S, H, D_qk, D_v, k, idx, q_start, sm, name, seed=40, staging="fp16", q=None, kv=None):
    import dsa_lightning_indexer_02_amd as dsa
    print("case", name, "staging", staging, flush=True)
    g = block_rng(seed, 0, 0)
    if q is None:
        q = to_bf16_bits(g.standard_normal((T, H, D_qk)).astype(np.float32))
    if kv is None:
        kv = to_bf16_bits(g.standard_normal((S, D_qk)).astype(np.float32))
    out, f32, lse = dsa.dsa_sparse_mla_fwd(dput(q, dev).view(torch.bfloat16), dput(kv, dev).view(torch.bfloat16),
                                           dput(idx.astype(np.int32), dev), sm, D_v, q_start=q_start, want_f32=True,
                                           staging=staging)
    o, _, ol = oracle.sparse_mla(q, idx.astype(np.int32), q_start + np.arange(T), kv, D_v, sm)
    parity.check_mla(bf16_vals(out), dget(f32), dget(lse), o, ol, name)
    return dget(f32), dget(lse)


@pytest.mark.parametrize("staging", ["fp16", "bf16"])
def test_mla_invalid_duplicate_entries(dev, staging):
    g = block_rng(41, 0, 0)
    T, S, k = 24, 3000, 2048
    idx = g.integers(-5, S + 50, size=(T, k))
    idx[:, 10:20] = idx[:, 0:10]          # duplicates
    idx[5] = -1                           # nothing valid in row 5
    idx[6, 1:] = -1                       # a single entry
    _mla_case(dev, T, S, 128, 576, 512, k, idx, 2000, 1 / np.sqrt(192), "invalid/duplicate", staging=staging)


def test_mla_small_dims_and_heads(dev):
    g = block_rng(42, 0, 0)
    T, S, k = 40, 256, 64
    idx = np.stack([g.permutation(S)[:k] for _ in range(T)])
    _mla_case(dev, T, S, 8, 80, 64, k, idx, 200, 1 / np.sqrt(80), "tiny dims")
    _mla_case(dev, T, S, 100, 576, 512, k, idx, 200, 0.07, "H=100 (partial head tile)")


@pytest.mark.parametrize("staging", ["fp16", "bf16"])
def test_mla_k1_and_large_logits(dev, staging):
    g = block_rng(43, 0, 0)
    T, S = 16, 500
    idx1 = g.integers(0, S, size=(T, 1))
    f32, lse = _mla_case(dev, T, S, 128, 576, 512, 1, idx1, S, 1 / np.sqrt(192), "k=1", staging=staging)
    idx = np.stack([g.permutation(S)[:256] for _ in range(T)])
    _mla_case(dev, T, S, 128, 576, 512, 256, idx, S, 2.0, "sharp softmax (rescale path)", staging=staging)


@pytest.mark.parametrize("staging", ["fp16", "bf16"])
def test_mla_value_magnitude_spread(dev, staging):
    """q and kv with magnitudes from 2^-24 up to a few units (every element N(0,1) times 2^e, e
    uniform in [-24, 0]): fp16 staging meets fp16's subnormal range and rounds the values below
    2^-17 to its 2^-24 grid; the results still meet the attention bar against the exact oracle."""
    g = block_rng(46, 0, 0)
    T, S, k = 20, 1500, 512
    q = g.standard_normal((T, 128, 576)) * np.exp2(g.integers(-24, 1, size=(T, 128, 576)))
    kv = g.standard_normal((S, 576)) * np.exp2(g.integers(-24, 1, size=(S, 576)))
    idx = np.stack([g.permutation(S)[:k] for _ in range(T)])
    _mla_case(dev, T, S, 128, 576, 512, k, idx, S, 1 / np.sqrt(192), "magnitude spread", staging=staging,
              q=to_bf16_bits(q.astype(np.float32)), kv=to_bf16_bits(kv.astype(np.float32)))


def test_many_rows_one_launch(dev):
    """70,000 query rows in one call (one workgroup per row, more than 65,536 of them): top-k and
    sparse attention at small widths, the oracle on rows on both sides of 65,536."""
    import dsa_lightning_indexer_02_amd as dsa
    T, S, k, q_start = 70000, 200, 64, 100
    print("case many rows", T, flush=True)
    g = block_rng(44, T, S)
    scores = g.standard_normal((T, S)).astype(np.float32)
    ld = dsa.ld_for(S)
    host = np.zeros((T, ld), np.float32)
    host[:, :S] = scores
    gi = dget(dsa.dsa_topk(dput(host, dev), k, S, q_start=q_start))
    rows = np.array([0, 1, 65534, 65535, 65536, 65537, T - 1])
    pos = q_start + rows
    parity.check_topk_exact(gi[rows], oracle.topk(scores[rows], pos, k), "top-k, many rows")
    H, D_qk, D_v, km = 8, 80, 64, 16
    q = to_bf16_bits(g.standard_normal((T, H, D_qk)).astype(np.float32))
    kv = to_bf16_bits(g.standard_normal((S, D_qk)).astype(np.float32))
    idx = g.integers(-2, S, size=(T, km)).astype(np.int32)   # some skipped and some non-causal entries
    sm = 1 / np.sqrt(80)
    out, f32, lse = dsa.dsa_sparse_mla_fwd(dput(q, dev).view(torch.bfloat16), dput(kv, dev).view(torch.bfloat16),
                                           dput(idx, dev), sm, D_v, q_start=q_start, want_f32=True)
    torch.cuda.synchronize()
    o, _, ol = oracle.sparse_mla(q[rows], idx[rows], pos, kv, D_v, sm)
    parity.check_mla(bf16_vals(out)[rows], dget(f32)[rows], dget(lse)[rows], o, ol, "MLA, many rows")
