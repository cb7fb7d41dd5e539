"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that a pin catches each.

Every mutant is the oracle source with one textual edit, compiled with gcc
into a temporary library; the real oracle source is never modified.
"""
import os

import pytest

import oracle
from oracle import build as obuild

import pins

MUTANTS = [
    # (name, original text, replacement, checks expected to fail)
    ("relu_dropped", "float r = d > 0.0f ? d : 0.0f;", "float r = d;",
     [pins.check_indexer_tiny]),
    ("diagonal_excluded", "int64_t n = pos + 1;", "int64_t n = pos;",
     [pins.check_indexer_tiny]),
    ("key_dim_reversed", "d += qdec[j * D_I + i] * kdec[s * D_I + i];",
     "d += qdec[j * D_I + i] * kdec[s * D_I + (D_I - 1 - i)];", [pins.check_indexer_tiny]),
    ("key_scale_dropped", "kdec[s * D_I + i] = ks[s] * g_e4m3[k8[s * D_I + i]];",
     "kdec[s * D_I + i] = g_e4m3[k8[s * D_I + i]];", [pins.check_indexer_tiny]),
    ("head_weight_index", "I += w[t * H_I + j] * r;", "I += w[t * H_I + (H_I - 1 - j)] * r;",
     [pins.check_indexer_tiny]),
    ("e4m3_bias", "ldexpf(1.0f + (float)m / 8.0f, e - 7)", "ldexpf(1.0f + (float)m / 8.0f, e - 8)",
     [pins.check_e4m3_table]),
    ("e4m3_subnormal", "ldexpf((float)m, -9)", "ldexpf((float)m, -10)", [pins.check_e4m3_table]),
    ("tie_to_higher_index", "return (x->i > y->i) - (x->i < y->i);",
     "return (x->i < y->i) - (x->i > y->i);", [pins.check_topk_ties]),
    ("ascending_scores", "if (x->v > y->v)\n        return -1;", "if (x->v < y->v)\n        return -1;",
     [pins.check_topk_lexsort]),
    ("topk_no_causal", "int64_t n = visible_keys(pos[t], S);\n        scored_t",
     "int64_t n = S;\n        scored_t", [pins.check_topk_special_cases]),
    ("mla_scale_dropped", "z[i] = sm_scale * dot;", "z[i] = dot;", [pins.check_mla_brute]),
    ("mla_value_columns", "acc[d] += e * bf16_value(vr[d]);",
     "acc[d] += e * bf16_value(vr[d + (D_qk - D_v)]);", [pins.check_mla_brute]),
    ("mla_lse_no_max", "lse[t * H + h] = m + logf(l);", "lse[t * H + h] = logf(l);",
     [pins.check_mla_dense_equivalence]),
    ("e4m3_ties_up", "return (uint8_t)((lo & 1) ? hi : lo);", "return (uint8_t)hi;",
     [pins.check_e4m3_encode_midpoints, pins.check_e4m3_encode_vs_torch]),
    ("e4m3_round_down", "    if (dl < dh)\n        return (uint8_t)lo;", "    if (dl <= dh + 1.0)\n        return (uint8_t)lo;",
     [pins.check_e4m3_encode_midpoints, pins.check_e4m3_encode_vs_torch]),
    ("quant_scale_447", "float s = amax > 0.0f ? amax / 448.0f : 1.0f", "float s = amax > 0.0f ? amax / 447.0f : 1.0f",
     [pins.check_quantize_rows_closed_forms, pins.check_quantize_rows_vs_generator]),
    ("quant_sign_dropped", "return (uint8_t)((signbit(y) ? 0x80 : 0) | e4m3_encode_abs(fabsf(y)));",
     "return (uint8_t)(e4m3_encode_abs(fabsf(y)));", [pins.check_e4m3_encode_round_trip]),
    ("ue8m0_floor", "int p = m == 0.5f ? e - 1 : e;", "int p = e - 1;", [pins.check_quantize_ue8m0]),
    ("ue8m0_no_clamp", "    if (p < -127)\n        p = -127;\n", "", [pins.check_quantize_ue8m0]),
    ("append_slot_shift", "int64_t row = (int64_t)blk * bs + pos[i] % bs;",
     "int64_t row = (int64_t)blk * bs + (pos[i] + 1) % bs;", [pins.check_append_paged_round_trip]),
    ("mla_future_keys", "int64_t n = visible_keys(pos[t], S);\n        const int32_t *row",
     "int64_t n = S;\n        const int32_t *row", [pins.check_mla_brute]),
    ("kl_head_sum", "p[s] += exp(z[s] - m) / l / (double)H;", "p[s] += exp(z[s] - m) / l;",
     [pins.check_kl_vs_torch]),
    ("kl_reversed", "acc += p[s] * (log(p[s]) - log_pi);", "acc += exp(log_pi) * (log_pi - log(p[s]));",
     [pins.check_kl_vs_torch, pins.check_kl_closed_forms]),
    ("kl_grad_sign", "dlogits[t * ld_d + s] = exp(log_pi) - p[s];", "dlogits[t * ld_d + s] = p[s] - exp(log_pi);",
     [pins.check_kl_vs_torch, pins.check_kl_finite_difference]),
    ("kl_scale_dropped", "z[s] = sm_scale * dot;", "z[s] = dot;", [pins.check_kl_vs_torch]),
    ("bwd_dk_unmasked", "if (z > 0.0)\n                    for", "if (1)\n                    for",
     [pins.check_indexer_bwd_vs_torch, pins.check_indexer_bwd_finite_difference]),
    ("bwd_dq_no_weight", "g[i] += di * (double)w[t * H_I + j] * kv_[i];", "g[i] += di * kv_[i];",
     [pins.check_indexer_bwd_vs_torch, pins.check_indexer_bwd_finite_difference]),
    ("bwd_dw_no_relu", "if (z > 0.0) {\n                    gw += di * z;",
     "gw += di * z;\n                if (z > 0.0) {", [pins.check_indexer_bwd_vs_torch,
                                                      pins.check_indexer_bwd_finite_difference]),
    ("kl_sparse_repeat_overwrites", "dlogits[t * ld_d + row[i]] += exp(log_pi) - p[i];",
     "dlogits[t * ld_d + row[i]] = exp(log_pi) - p[i];", [pins.check_kl_sparse_vs_torch,
                                                          pins.check_kl_sparse_closed_forms]),
    ("mla_bwd_no_delta", "const double ds = p * (dp[i] - D);", "const double ds = p * dp[i];",
     [pins.check_mla_bwd_vs_torch, pins.check_mla_bwd_finite_difference, pins.check_mla_bwd_closed_forms]),
    ("mla_bwd_dq_unscaled", "dqh[d] += sm_scale * ds * (double)bf16_value(kr[d]);",
     "dqh[d] += ds * (double)bf16_value(kr[d]);",
     [pins.check_mla_bwd_vs_torch, pins.check_mla_bwd_finite_difference, pins.check_mla_bwd_dense_equivalence]),
    ("mla_bwd_dv_without_p", "c[d] += p * (double)bf16_value(gh[d]);", "c[d] += (double)bf16_value(gh[d]);",
     [pins.check_mla_bwd_vs_torch, pins.check_mla_bwd_closed_forms]),
    ("mla_bwd_dk_from_key", "c[d] += sm_scale * ds * (double)bf16_value(qh[d]);",
     "c[d] += sm_scale * ds * (double)bf16_value(kr[d]);",
     [pins.check_mla_bwd_vs_torch, pins.check_mla_bwd_finite_difference]),
    ("mla_bwd_repeat_once", "                dst[d] += c[d];", "                dst[d] = c[d];",
     [pins.check_mla_bwd_vs_torch, pins.check_mla_bwd_closed_forms]),
    ("kl_sparse_all_keys", "p[i] += exp(z[i] - m) / l / (double)H;", "p[i] += exp(z[i] - m) / l / (double)(H + 1);",
     [pins.check_kl_sparse_vs_torch]),
]


@pytest.fixture(scope="module")
def source():
    with open(obuild.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,orig,repl,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_mutant(name, orig, repl, checks, source, tmp_path):
    assert source.count(orig) == 1, "mutation anchor for %s must occur exactly once" % name
    src = tmp_path / ("mutant_%s.c" % name)
    src.write_text(source.replace(orig, repl))
    lib_path = obuild.build(str(src), str(tmp_path / ("libmutant_%s.so" % name)))
    lib = oracle.load(lib_path)
    for check in checks:
        with pytest.raises(AssertionError):
            check(lib)
