"""Pins of the oracle's indexer training signal (KL loss toward the head-averaged main attention,
DeepSeek-V3.2-Exp summary page, "Method", dense warm-up) and of the indexer backward.

The loss and its score gradient are pinned to torch's kl_div and autograd in float64, to closed
forms (a single visible key, pi = p, uniform scores, two sharp heads) and to central differences;
the backward is pinned to torch autograd through ReLU and to exact finite differences along the
row scales and weights.  The sparse-stage loss (each row's index-list entries only) is pinned to
torch through the gather (repeated and skipped entries), to the dense loss when the list holds
every visible key, and to closed forms (no or one valid entry, a repeated key).  The checks live in pins.py (the mutant tests reuse them).
"""
from __future__ import annotations

import pytest

import oracle
import pins


@pytest.mark.parametrize("check", [pins.check_kl_vs_torch, pins.check_kl_closed_forms,
                                   pins.check_kl_finite_difference, pins.check_indexer_bwd_vs_torch,
                                   pins.check_indexer_bwd_finite_difference, pins.check_kl_sparse_vs_torch,
                                   pins.check_kl_sparse_closed_forms],
                         ids=lambda c: c.__name__)
def test_kl_pin(check):
    check(oracle.load())
