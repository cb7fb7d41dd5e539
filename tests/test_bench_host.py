"""Host-side parts of bench.py (no GPU): the one-GPU contract and the algorithmic work counts that
every roofline fraction in its JSON line is computed from."""
from __future__ import annotations

import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_work_model_closed_forms():
    wl = SimpleNamespace(T=6, S=10, q_start=2, H_I=4, D_I=32, H=8, D_qk=80, D_v=64, topk=4)
    m = bench.work_model(wl)
    n = np.minimum(10, 2 + np.arange(6) + 1)          # 3 4 5 6 7 8 visible keys
    assert m["visible_pairs"] == 33 and m["visible_pairs"] == int(n.sum())
    assert m["selected_rows"] == 3 + 4 * 5           # min(n, 4)
    assert m["indexer_flop"] == 2 * 4 * 32 * 33
    assert m["mla_flop"] == 2 * 8 * (80 + 64) * 23
    assert m["topk_bytes"] == 4 * 33 + 4 * 6 * 4
    # an explicit row-length vector (decode) replaces the causal counts
    d = bench.work_model(wl, n=[10, 1])
    assert d["visible_pairs"] == 11 and d["selected_rows"] == 4 + 1


def test_percentiles():
    p = bench.percentiles([1.0, 2.0, 3.0, 4.0, 5.0])
    assert p["p50"] == 3.0 and p["p10"] < p["p50"] < p["p90"]
