"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU), builds it,
points the oracle module at the mutant and runs every pin: at least one must fail.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "dsa_oracle.c")

MUTATIONS = {
    "relu_dropped": ("double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;"),
    "relu_after_head_sum": ("total += oracle_bf16_to_double(wrow[j]) * relu;",
                            "total += oracle_bf16_to_double(wrow[j]) * dot;"),
    "head_weight_dropped": ("total += oracle_bf16_to_double(wrow[j]) * relu;", "total += relu;"),
    "causal_off_by_one": ("if (s > p) {", "if (s >= p) {"),
    "key_row_of_query": ("const uint16_t* krow = c->k + ((int64_t)b * c->Tk + s) * c->D;",
                         "const uint16_t* krow = c->k + ((int64_t)b * c->Tk + i) * c->D;"),
    "tie_prefers_higher_index": ("return (a->index > b->index) - (a->index < b->index);",
                                 "return (a->index < b->index) - (a->index > b->index);"),
    "padding_with_zero": ("for (int64_t j = kept; j < c->k; ++j) out[j] = -1;",
                          "for (int64_t j = kept; j < c->k; ++j) out[j] = 0;"),
    "short_rows_skip_own_key": ("for (int64_t j = 0; j < n; ++j) out[j] = (int32_t)j;",
                                "for (int64_t j = 0; j < n - 1; ++j) out[j] = (int32_t)j; kept = n - 1; if (0)"),
    "descending_output": ("return (a > b) - (a < b);", "return (a < b) - (a > b);"),
    "scale_dropped": ("z[j] = c->sm_scale * dot;", "z[j] = dot;"),
    "lse_without_max": ("c->lse[row * c->H + h] = m + log(denom);", "c->lse[row * c->H + h] = log(denom);"),
    "fp8_bias_8": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "fp8_scale_dropped": ("(double)c->kv_scale[(int64_t)b * c->Tk + s];", "1.0;"),
    "e2m1_bias_0": ("ldexp(1.0 + (double)m / 2.0, e - 1);", "ldexp(1.0 + (double)m / 2.0, e);"),
    "e2m1_subnormal_as_normal": ("double v = e == 0 ? (double)m / 2.0 :", "double v = 0 ? (double)m / 2.0 :"),
    "mxfp4_nibbles_swapped": ("(i % 2 == 0) ? (uint8_t)(byte & 15) : (uint8_t)(byte >> 4);",
                              "(i % 2 == 1) ? (uint8_t)(byte & 15) : (uint8_t)(byte >> 4);"),
    "mxfp4_scale_position": ("row[D / 2 + 4 * (j % 8) + j / 8];", "row[D / 2 + j];"),
    "mxfp4_row_stride": ("r * oracle_mxfp4_row_bytes(c->Dqk), c->Dqk, d);", "r * (c->Dqk / 2), c->Dqk, d);"),
    "kl_gradient_sign": ("G[e] = exp(logQ) - P[e];", "G[e] = P[e] - exp(logQ);"),
    "kl_target_head_sum": ("P[e] += exp(z[e] - m) / sum / c->H;", "P[e] += exp(z[e] - m) / sum;"),
    "kl_relu_dropped": ("total += wi[j] * (dot > 0.0 ? dot : 0.0);", "total += wi[j] * dot;"),
    "kl_dq_without_weight": ("dq[j * c->d_I + d] += G[e] * wi[j] * kr[d];", "dq[j * c->d_I + d] += G[e] * kr[d];"),
    "kl_dk_from_key": ("dk[d] += c.G[row * width + e] * wi[j] * qi[j * d_I + d];",
                       "dk[d] += c.G[row * width + e] * wi[j] * kr[d];"),
    "kl_scale_dropped": ("z[e] = c->sm_scale * dot;", "z[e] = dot;"),
    "kl_reverse_direction": ("if (P[e] > 0.0) L += P[e] * (log(P[e]) - logQ);",
                             "L += exp(logQ) * (logQ - log(P[e]));"),
    "stream_row_excludes_own_key": ("int32_t kv_len = t + 1;", "int32_t kv_len = t;"),
    "stream_row_query_of_previous_row": ("attn_ctx ac = {c->q + (int64_t)t * c->H * c->Dqk,",
                                         "attn_ctx ac = {c->q + (int64_t)(t > 0 ? t - 1 : 0) * c->H * c->Dqk,"),
    "value_from_key_tail": ("if (!c->v) return kv_value(c, b, s, g, d);",
                            "if (!c->v) return kv_value(c, b, s, g, d + (c->Dqk - c->Dv));"),
}

PIN_TESTS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_") and callable(getattr(pins, n))]


def _run_pins():
    failed = []
    for t in PIN_TESTS:
        try:
            if t.__name__ == "test_topk_matches_numpy_lexsort_with_heavy_ties":
                for k in (1, 3, 8, 33):
                    t(k)
            elif t.__name__ == "test_streamed_rows_equal_scores_topk_attention_composed":
                for fmt in ("bf16", "fp8", "mxfp4"):
                    t(fmt)
            else:
                t()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(t.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(before) >= 1, f"mutation anchor not found: {before}"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(before, after))
    so = tmp_path / "libmutant.so"
    inc = os.path.dirname(SRC)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-I", inc, str(mutant), "-o", str(so),
                           "-lm", "-lpthread"])
    saved_so, saved_lib = oracle._SO, oracle._lib
    try:
        oracle._SO, oracle._lib = str(so), None
        failed = _run_pins()
    finally:
        oracle._SO, oracle._lib = saved_so, saved_lib
    assert failed, f"no pin caught mutation {name}"
