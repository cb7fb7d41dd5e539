"""Pins of the oracle's sparse-MLA backward (DeepSeek-V3.2-Exp summary page, "Method": the sparse
training stage runs the main attention over the selected rows only, so its gradients flow through
those rows): torch autograd in float64 through the gather (repeated and skipped entries), central
differences of the forward's definition, dense causal attention (torch SDPA autograd) when every
visible key is listed, and closed forms (a single entry, q = 0, the zero-sum of the softmax
gradient, rows without entries).  The checks live in pins.py (the mutant tests reuse them)."""
from __future__ import annotations

import pytest

import oracle
import pins


@pytest.mark.parametrize("check", [pins.check_mla_bwd_vs_torch, pins.check_mla_bwd_finite_difference,
                                   pins.check_mla_bwd_dense_equivalence, pins.check_mla_bwd_closed_forms],
                         ids=lambda c: c.__name__)
def test_mla_bwd_pin(check):
    check(oracle.load())
