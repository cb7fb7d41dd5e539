"""Oracle index sets against the stored SHA-256 fixtures (tests/golden/make_golden.py)."""
import json
import os

import pytest

from golden.make_golden import compute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_topk_sha256.json")


with open(GOLDEN) as _f:
    _CASES = json.load(_f)


@pytest.mark.parametrize("name", sorted(_CASES))
def test_oracle_topk_hash(name):
    case = _CASES[name]
    assert compute(name, case["rows"]) == case["sha256"]
