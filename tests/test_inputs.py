"""The seeded input generator: determinism, row-subset regeneration, encodings."""
import numpy as np

import oracle
from dsa_inputs import decode_inputs, get, prefill_inputs, quantize_fp8_rows
from dsa_inputs.configs import Workload
from dsa_inputs.generate import block_rng


def test_prefill_deterministic_and_row_subsets():
    wl = get("tiny")
    a = prefill_inputs(wl)
    b = prefill_inputs(wl)
    for f in ("q8", "qs", "w", "k8", "ks", "q", "kv"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    rows = [0, 17, 31, 32, 200, 255]
    c = prefill_inputs(wl, rows=rows)
    for f in ("q8", "qs", "w", "q"):
        assert np.array_equal(getattr(c, f), getattr(a, f)[rows]), f
    assert np.array_equal(c.k8, a.k8) and np.array_equal(c.kv, a.kv)


def test_distributions_tiny():
    wl = get("tiny")
    a = prefill_inputs(wl)
    assert a.q8.shape == (256, 4, 32) and a.k8.shape == (256, 32)
    assert a.q.shape == (256, 8, 80) and a.kv.shape == (256, 80)
    assert a.w.min() >= 0 and a.w.max() < 1.0 / wl.H_I
    kvf = (a.kv.astype(np.uint32) << 16).view(np.float32)
    assert abs(kvf.mean()) < 0.05 and abs(kvf.std() - 1.0) < 0.05


def _nearest_e4m3(y, table):
    """Independent round-to-nearest-even over the finite E4M3 values (codes with even mantissa win ties)."""
    codes = np.array([c for c in range(256) if not np.isnan(table[c])], dtype=np.int64)
    vals = table[codes].astype(np.float64)
    d = np.abs(y[:, None].astype(np.float64) - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    out = np.empty(len(y), dtype=np.int64)
    for i in range(len(y)):
        cs = codes[cand[i]]
        cs_val = table[cs]
        if len(cs) > 1:
            # +0 / -0 are the same value: keep the sign of y; otherwise pick the even mantissa
            if np.all(cs_val == 0):
                cs = cs[(cs >> 7) == (1 if np.signbit(y[i]) else 0)]
            else:
                cs = cs[(cs & 1) == 0]
        out[i] = cs[0]
    return out


def test_quantizer_is_round_to_nearest_even():
    table = oracle.e4m3_table()
    g = block_rng(5, 0, 0)
    x = np.concatenate([g.standard_normal((64, 32)), g.standard_normal((4, 32)) * 1e-3,
                        np.zeros((1, 32))]).astype(np.float32)
    codes, scale = quantize_fp8_rows(x)
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(scale, np.where(amax > 0, amax / np.float32(448.0), 1.0).astype(np.float32))
    y = np.clip(x / scale[:, None], -448, 448).ravel()
    ref = _nearest_e4m3(y, table)
    assert np.array_equal(codes.ravel().astype(np.int64), ref)
    # the absmax element of every non-zero row encodes to +-448
    nz = amax > 0
    assert np.all(np.abs(table[codes[nz]]).max(axis=1) == 448.0)


def test_chunked_outliers():
    wl = get("chunked_131k")
    small = Workload(**{**wl.__dict__, "S": 4096, "T": 16, "q_start": 4080, "name": "chunked_small"})
    a = prefill_inputs(small, with_q=False)
    assert len(a.outliers) == round(0.01 * 4096) == len(np.unique(a.outliers))
    med = np.median(a.ks)
    assert np.median(a.ks[a.outliers]) > 5 * med


def test_decode_paging_structure():
    wl = get("decode_64")
    lens = np.array([70, 64, 1, 200], dtype=np.int32)
    d = decode_inputs(wl, seq_lens=lens)
    nblk = (lens + 63) // 64
    assert d.num_blocks == nblk.sum()
    used = np.concatenate([d.block_table[b, :nblk[b]] for b in range(len(lens))])
    assert sorted(used.tolist()) == list(range(d.num_blocks))
    for b in range(len(lens)):
        assert np.all(d.block_table[b, nblk[b]:] == -1)
    e = decode_inputs(wl, seq_lens=lens)
    assert np.array_equal(d.kv_pool, e.kv_pool) and np.array_equal(d.block_table, e.block_table)
    full = get("decode_64")
    L = decode_inputs.__globals__["decode_lengths"](full)
    assert L.min() >= 8192 and L.max() <= 131072 and len(L) == 64
