"""The oracle against the pages' definitions, library routines, closed forms and invariants."""
import pytest

import pins


@pytest.mark.parametrize("check", [
    pins.check_e4m3_table,
    pins.check_bf16_round,
    pins.check_indexer_tiny,
    pins.check_indexer_full_heads,
    pins.check_indexer_relu_matmul,
    pins.check_indexer_scale_invariants,
    pins.check_topk_lexsort,
    pins.check_topk_ties,
    pins.check_topk_special_cases,
    pins.check_mla_dense_equivalence,
    pins.check_mla_brute,
    pins.check_mla_special_cases,
    pins.check_causal_end_to_end,
    pins.check_dense_when_k_covers,
], ids=lambda f: f.__name__)
def test_pin(check, oracle_lib):
    check(oracle_lib)
