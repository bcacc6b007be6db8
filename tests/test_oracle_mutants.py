"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake in a temporary copy of the oracle's C source
(a dropped term, a wrong sign, a wrong index or order, a transposed operand,
a wrong rounding), builds it, points the oracle wrapper at it and runs the
pin tests: at least one of them has to fail.  The committed oracle itself
is never changed."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from tests import test_oracle_combine as tc
from tests import test_oracle_config as tcfg
from tests import test_oracle_layout as tl
from tests import test_oracle_staged as ts

_SRC = os.path.join(os.path.dirname(oracle.__file__), "afd_oracle.c")

MUTANTS = {
    "combine_drops_accumulated_terms": ("acc[h] = acc[h] + p;", "acc[h] = p;"),
    "combine_wrong_sign": ("acc[h] = acc[h] + p;", "acc[h] = acc[h] - p;"),
    "combine_wrong_column": ("y[f][(int64_t)r * H + h]", "y[f][(int64_t)r * H + (h ^ 1)]"),
    "combine_weight_of_other_k": ("float wk = w[g * K + k];", "float wk = w[g * K + (K - 1 - k)];"),
    "layout_start_not_aligned": ("start[e] = align_up(prev_end, alpha);", "start[e] = prev_end;"),
    "layout_reverse_rank": ("slot_row[g * K + k] = (int32_t)(start[e] + cursor[e]);",
                            "slot_row[g * K + k] = (int32_t)(start[e] + C[e] - 1 - cursor[e]);"),
    "layout_dup_misses_neighbour": ("for (kk = 0; kk < k; ++kk)", "for (kk = 0; kk + 1 < k; ++kk)"),
    "layout_ends_aligned": ("ends[e] = (int32_t)(start[e] + C[e]);",
                            "ends[e] = (int32_t)align_up(start[e] + C[e], alpha);"),
    "dispatch_transposed_row": ("x + g * row_bytes, (size_t)row_bytes",
                                "x + (ntok - 1 - g) * row_bytes, (size_t)row_bytes"),
    "expert_scale_off_by_one": ("return 1.0f + (float)e / (float)E;", "return 1.0f + (float)(e + 1) / (float)E;"),
    "bf16_round_half_up": ("u += 0x7FFFu + lsb;", "u += 0x8000u;"),
    "scales_ignore_stride": ("(int64_t)b * stride_g[s]]", "(int64_t)b]"),
    # per-stage combine
    "partial_rounding_drops_lsb": ("partial[((int64_t)f * ntok + g) * H + h] = f32_to_bf16_rne(acc[h]);",
                                   "partial[((int64_t)f * ntok + g) * H + h] = (uint16_t)(f32_to_bf16_rne(acc[h]) & 0xFFFE);"),
    "stages_first_lane_order": ("for (kk = k + 1; kk < K; ++kk)", "for (kk = 0; kk < k; ++kk)"),
    "stages_skip_rounding_stage": ("v = bf16_to_f32(partial[((int64_t)f * ntok + g) * H + h]);",
                                   "v = bf16_to_f32(partial[((int64_t)f * ntok + g) * H + h]) * 1.00390625f;"),
    "fp8_clamp_off_by_one": ("int e = -117;", "int e = -116;"),
    "fp8_exponent_off_by_one": ("while ((double)amax > 448.0 * ldexp(1.0, e)) e += 1;",
                                "while ((double)amax > 224.0 * ldexp(1.0, e)) e += 1;"),
    "fp8_scale_not_applied": ("f32_to_e4m3_rne(ldexpf(bf16_to_f32(partial[b * 128 + i]), -e));",
                              "f32_to_e4m3_rne(ldexpf(bf16_to_f32(partial[b * 128 + i]), -e - (i == 5)));"),
    "fp8_dequant_bias": ("(int)row[H + h / 128] - 127);", "(int)row[H + h / 128] - 126);"),
    "fp8_ties_up": ("((c + 1) & 1) == 0)) c = c + 1;", "1)) c = c + 1;"),
    "fp8_nan_in_amax": ("if (v == v && v > amax) amax = v;", "if (v > amax || v != v) amax = v;"),
    # configuration and shape check
    "config_hidden_multiple_of_128": ("if (H % 256 != 0) return ORC_BAD_CONFIG;", "if (H % 128 != 0) return ORC_BAD_CONFIG;"),
    "config_topk_limit_dropped": ("if (K > 32 || K > E) return ORC_BAD_CONFIG;", "if (K > E) return ORC_BAD_CONFIG;"),
    "config_uneven_split_accepted": ("    if (E % F != 0) return ORC_BAD_CONFIG;\n", "\n"),
    "config_bucket_past_capacity": ("if (bucket < 1 || bucket > capacity)", "if (bucket < 1)"),
    "config_tokens_past_bucket": ("if (T[s] < 0 || T[s] > bucket)", "if (T[s] < 0)"),
}


def _pins():
    """The pin tests, as zero-argument callables."""
    out = []
    for case in tl.SWEEP[:12]:
        out.append(lambda c=case: tl.test_layout_matches_brute_force(c))
    for name in ("tiny", "2a2f_decode", "1a3f_e96"):
        out.append(lambda n=name: tc.test_rows_scales_weights_are_copies(n))
        out.append(lambda n=name: tc.test_identity_experts_bit_exact(n))
        out.append(lambda n=name: tc.test_combine_closed_form(n))
    out += [tc.test_strided_scales_equal_dense, tc.test_combine_sparse_routing_matrix_any_replies,
            tc.test_combine_exact_special_cases, tc.test_padding_rows_never_read,
            tc.test_oracle_number_formats, tl.test_first_offender_codes,
            tl.test_single_source_single_partition_is_stable_argsort]
    out += [ts.test_e4m3_encoder_matches_torch, ts.test_quantization_error_bound,
            ts.test_stage_two_order_is_last_lane, ts.test_fp8_partials_exact_for_short_integers,
            ts.test_single_partition_reduces_to_single_rounding,
            lambda: ts.test_quantized_rows_match_torch_and_closed_form(256)]
    out.insert(0, tcfg.test_config_pins_all)   # fast, so first
    for i in (0, 3, 4):
        out.append(lambda i=i: ts.test_partials_equal_masked_single_rounding_combine(i))
        out.append(lambda i=i: ts.test_stage_two_equals_single_rounding_combine_of_partials(i, False))
        out.append(lambda i=i: ts.test_stage_two_equals_single_rounding_combine_of_partials(i, True))
    return out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    src = open(_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mut.c")
        lib = os.path.join(d, "libmut.so")
        open(path, "w").write(src.replace(old, new))
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared", path, "-o", lib, "-lm"])
        import ctypes
        saved = oracle._lib
        oracle._lib = ctypes.CDLL(lib)
        caught = []
        try:
            for pin in _pins():
                try:
                    pin()
                except (AssertionError, ValueError, IndexError):
                    caught.append(pin)
                    break
        finally:
            oracle._lib = saved
        assert caught, f"no pin failed for planted mistake {name}"


def test_unmutated_oracle_passes_every_pin():
    for pin in _pins():
        pin()
    assert np.all(np.asarray([1]))
