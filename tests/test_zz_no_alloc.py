"""The allocation-free top-k entry point (dsa_topk_noalloc) against dsa_topk with a caller
workspace, through the C ABI: identical index lists on two calls in a row, the second smaller,
both taking the split-row path that keeps its candidates in the library's per-GPU scratch array
(needs an MI355X)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from dsa_inputs.generate import block_rng
from gpu_helpers import dput

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_02_amd as dsa
    dsa.load()
    return torch.device("cuda:0")


def _rows(T, S, seed):
    g = block_rng(seed, T, S)
    s = g.standard_normal((T, S)).astype(np.float32)
    s[::3] = np.round(s[::3] * 2)        # ties straddling the chunk borders
    return s


def _compare(dev, T, S, q_start, k, seed):
    import dsa_lightning_indexer_02_amd as dsa
    print("case no-alloc top-k T=%d S=%d q_start=%d k=%d" % (T, S, q_start, k), flush=True)
    ld = dsa.ld_for(S)
    host = np.zeros((T, ld), np.float32)
    host[:, :S] = _rows(T, S, seed)
    lg = dput(host, dev)
    ref = dsa.dsa_topk(lg, k, S, q_start=q_start)
    got = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    dsa.dsa_topk_noalloc(lg, k, S, q_start=q_start, indices=got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "dsa_topk_noalloc differs from dsa_topk"
    need = dsa.load().dsa_topk_workspace_size(T, S, k)
    return need


def test_noalloc_topk_two_calls_second_smaller(dev):
    import dsa_lightning_indexer_02_amd as dsa
    # first call: 200 rows of up to 131072 scores (4 chunks, 13 MB of the 32 MiB scratch)
    need1 = _compare(dev, 200, 131072, 131072 - 200, 2048, 81)
    # second call, smaller: 37 rows of up to 70001 scores (3 chunks), over the first call's contents
    need2 = _compare(dev, 37, 70001, 70001 - 37, 2048, 82)
    assert 0 < need2 < need1 <= dsa.TOPK_NOALLOC_SCRATCH_BYTES
    # rows that fit one chunk take no scratch at all
    assert _compare(dev, 50, 20000, 19950, 2048, 83) == 0


def test_noalloc_topk_rejects_oversize(dev):
    import dsa_lightning_indexer_02_amd as dsa
    lg = torch.zeros((600, 131072), dtype=torch.float32, device=dev)
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_topk_noalloc(lg, 2048, 131072, q_start=131072)
    assert "scratch" in str(ei.value)
    # the refused call enqueued nothing; a call that fits still matches dsa_topk afterwards
    _compare(dev, 16, 40000, 39990, 2048, 84)
