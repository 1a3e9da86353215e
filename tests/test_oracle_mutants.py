"""The pins are strong enough: plant plausible mistakes in a copy of the oracle.

Each mutant is the oracle's C source with one edit (a wrong bucket map, a
dropped term, an off-by-one, a transposed index, a wrong tie rule ...), built
into its own library in a temporary directory.  The pin battery below must
pass on the real oracle and fail on every mutant.  Every mutant stays memory
safe (no edit can move an index outside its array).
"""

import os

import numpy as np
import pytest

import oracle as om
from tests import test_oracle_fp8_modes as fm
from tests import test_oracle_handworked as hw
from tests import test_oracle_properties as pr

MUTANTS = {
    "bucket_map_mod": ("is_token_in_rank[t * R + (int)(e / P)] = 1;",
                       "is_token_in_rank[t * R + (int)(e % R)] = 1;"),
    "channel_floor": ("int64_t per = (T + C - 1) / C;", "int64_t per = T / C;"),
    "recv_prefix_inclusive": ("recv_channel_prefix_matrix[r * C + c] = (int32_t)count;\n            count += n_rc;",
                              "count += n_rc;\n            recv_channel_prefix_matrix[r * C + c] = (int32_t)count;"),
    "src_idx_value": ("recv_src_idx[base + seen] = (int32_t)t;", "recv_src_idx[base + seen] = (int32_t)seen;"),
    "local_expert_id": ("recv_topk_idx[row * K + k] = mine ? e - (int64_t)r * P : -1;",
                        "recv_topk_idx[row * K + k] = mine ? e - (int64_t)r : -1;"),
    "weight_not_zeroed": ("mine ? topk_weights[t * K + k] : 0.0f;", "topk_weights[t * K + k];"),
    "fp8_fnuz_max": ("if (mode == ORACLE_FP8_AMAX) s = ap / 448.0f;",
                     "if (mode == ORACLE_FP8_AMAX) s = ap / 240.0f;"),
    "pow2_floor": ("return (float)ldexp(1.0, m == 0.5 ? e - 1 : e);", "return (float)ldexp(1.0, e - 1);"),
    "ue8m0_bias": ("(uint8_t)(ilogbf(s) + 127)", "(uint8_t)(ilogbf(s) + 126)"),
    "tensor_scale_ignored": ("else if (mode == ORACLE_FP8_TENSOR) s = tensor_scale;",
                             "else if (mode == ORACLE_FP8_TENSOR) s = 1.0f;"),
    "passthrough_row": ("memcpy(dst + row * W, src + t * W, (size_t)W);",
                        "memcpy(dst + row * W, src + (t > 0 ? t - 1 : 0) * W, (size_t)W);"),
    "fp8_tie_odd": ("else code = (uint8_t)((c & 1) ? c + 1 : c);", "else code = (uint8_t)((c & 1) ? c : c + 1);"),
    "fp8_no_floor": ("float ap = a > 1e-4f ? a : 1e-4f;", "float ap = a;"),
    "combine_no_dedup": ("if (seen) continue;", "(void)seen;"),
    "combine_per_slot_weight": ("if (e2 >= 0 && (int)(e2 / P) == r) w = w + gate_weights[t * K + k2];",
                                "if (k2 == k) w = w + gate_weights[t * K + k2];"),
    "combine_dropped_acc": ("send_head[t * R + r];\n            for (int64_t h = 0; h < H; ++h)\n"
                            "                acc[h] = fmaf(w, oracle_bf16_to_f32(y[row * H + h]), acc[h]);",
                            "send_head[t * R + r];\n            for (int64_t h = 0; h < H; ++h)\n"
                            "                acc[h] = w * oracle_bf16_to_f32(y[row * H + h]);"),
    "bf16_tie_odd": ("else pick = ((lo >> 16) & 1u) ? hi : lo;", "else pick = ((lo >> 16) & 1u) ? lo : hi;"),
    "bf16_half_down": ("if (dlo < dhi) pick = lo;", "if (dlo <= dhi) pick = lo;"),
    "ll_src_transposed": ("src_idx[e * cap + s] = (int32_t)t;", "src_idx[s * E + e] = (int32_t)t;"),
    "ll_dropped_slot": ("int64_t row = e * cap + slot_of[t * K + k];", "int64_t row = e * cap;"),
}

# fixed cases for the property pins (seed, T, (E, R), K, C, p_empty)
CASES = [(1, 37, (16, 4), 3, 5, 0.2), (2, 40, (8, 4), 2, 3, 0.0), (3, 23, (12, 3), 4, 8, 0.0),
         (4, 9, (16, 16), 4, 2, 0.0), (5, 40, (16, 4), 6, 7, 0.0)]


def battery(o: om.Oracle) -> None:
    """Every pin that can run on a given oracle; raises on the first failure."""
    for f in (hw.test_layout_by_hand, hw.test_handle_by_hand, hw.test_pack_by_hand,
              hw.test_combine_by_hand, hw.test_ll_by_hand):
        f(o)
    for case in CASES:
        pr.test_layout_and_handle_against_numpy.hypothesis.inner_test(o, case)
        pr.test_pack_against_index_select.hypothesis.inner_test(o, case, 128)
    pr.test_bf16_round_matches_torch_cast(o)
    for v, c in pr.E4M3_WORKED:
        pr.test_e4m3_worked_values(o, v, c)
    pr.test_e4m3_midpoints_round_to_even(o)
    pr.test_fp8_worked_block(o)
    pr.test_fp8_all_zero_block_and_negative_zero(o)
    for w in (pr.wl.TINY, pr.wl.PREFILL):
        pr.test_combine_identity_closed_forms(o, w)
    pr.test_ll_layout_properties.hypothesis.inner_test(o, 3, 40, 16, 4, 0.0)
    pr.test_ll_combine_unit_weights(o)
    fm.test_pow2_scale_worked_values(o)
    for mode in ("pow2", "ue8m0"):
        fm.test_pow2_block_codes_and_scale(o, mode)
    fm.test_tensor_scale_codes_and_saturation(o)
    fm.test_pack_modes_and_rows_bytes_against_indexing(o, 1)


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def test_battery_passes_on_oracle(oracle):
    with np.errstate(all="ignore"):
        battery(oracle)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(mutant_dir, name):
    find, repl = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(om.__file__), "oracle.c")).read()
    assert src.count(find) == 1, f"mutation site for {name} not found exactly once"
    path = os.path.join(str(mutant_dir), f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(find, repl))
    lib = om.build(src=path, out=os.path.join(str(mutant_dir), f"lib{name}.so"))
    o = om.Oracle(lib)
    with np.errstate(all="ignore"):
        with pytest.raises((AssertionError, ValueError)):
            battery(o)
