"""Pins of the oracle's FP8 quantizer and paged append (the on-device quantize + append step).

The codec is pinned to what the format and a reference cast fix: every finite code survives a
round trip, values exactly halfway between neighbouring codes take the even code, and random
values agree bit for bit with torch's float8_e4m3fn cast.  The row quantizer (per-row absmax
scale, createthis gist page, indexer listing) is pinned to its closed-form cases and to the input
generator's torch implementation of the same definition; the append is pinned through the
already-pinned paged gather.  The checks live in pins.py (the mutant tests reuse them).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import pins
from dsa_inputs import to_bf16_bits


@pytest.mark.parametrize("check", [pins.check_e4m3_encode_round_trip, pins.check_e4m3_encode_midpoints,
                                   pins.check_e4m3_encode_vs_torch, pins.check_quantize_rows_closed_forms,
                                   pins.check_quantize_rows_vs_generator, pins.check_quantize_ue8m0],
                         ids=lambda c: c.__name__)
def test_quantizer_pin(check):
    check(oracle.load())


@pytest.mark.parametrize("bs", [16, 64])
def test_append_paged_round_trip(bs):
    pins.check_append_paged_round_trip(oracle.load(), bs)


def test_append_paged_rejects_unmapped_block():
    k8 = np.zeros((4, 16, 32), np.uint8)
    ks = np.zeros((4, 16), np.float32)
    kv = np.zeros((4, 16, 80), np.uint16)
    table = np.array([[1, -1]], np.int32)
    with pytest.raises(ValueError):
        oracle.append_paged(k8, ks, kv, table, np.array([0], np.int32), np.array([20], np.int32),
                            to_bf16_bits(np.ones((1, 32), np.float32)), np.zeros((1, 80), np.uint16))
