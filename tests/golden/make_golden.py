"""Write tests/golden/oracle_topk_sha256.json from the oracle alone.

Fixed-token / hash regression idea from the weekinpapers summary of the
DeepSeek-V4-Flash-on-gfx90a paper (abstract): the SHA-256 of each workload's
selected index sets (each row's valid indices sorted ascending, int32
little-endian, rows concatenated) as produced by the oracle on the seeded
inputs.  Only oracle/ and dsa_inputs/ are used.
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from dsa_inputs import get, prefill_inputs  # noqa: E402

CASES = {
    "tiny": None,
    "prefill_4k": [2048, 2049, 3000, 4094, 4095],
}


def index_set_hash(idx: np.ndarray) -> str:
    h = hashlib.sha256()
    for row in idx:
        v = np.sort(row[row >= 0]).astype("<i4")
        h.update(v.tobytes())
    return h.hexdigest()


def compute(name, rows):
    wl = get(name)
    inp = prefill_inputs(wl, rows=rows, with_q=False)
    logits = oracle.indexer(inp.q8, inp.qs, inp.w, inp.pos, inp.k8, inp.ks)
    idx = oracle.topk(logits, inp.pos, wl.topk)
    return index_set_hash(idx)


def main():
    out = {}
    for name, rows in CASES.items():
        out[name] = {"rows": rows, "sha256": compute(name, rows)}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_topk_sha256.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
