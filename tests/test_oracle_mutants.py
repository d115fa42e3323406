"""The pins catch plausible mistakes in the oracle.

Each case copies oracle.c to a temporary directory, plants one mistake (a
dropped term, a wrong sign or index, a transposed operand, a wrong rounding),
builds it with the same gcc flags, swaps it in for the real oracle, and runs
the CPU pins. At least one pin must fail for every planted mistake. The real
oracle source is never modified.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_adam as TA
import test_oracle_bf16 as TB
import test_oracle_layout as TL
import test_oracle_memory as TM
import test_oracle_reduce as TR
import test_oracle_ring as TG
import test_oracle_step as TS
import test_oracle_gather as TGA
import test_oracle_golden as TGO
import test_oracle_wire as TW

MUTANTS = {
    "no_bias_correction_1": ("float mh = m1 / bc1;", "float mh = m1;"),
    "no_bias_correction_2": ("float vh = v1 / bc2;", "float vh = v1;"),
    "wrong_update_sign": ("float pn = p1 - lu;", "float pn = p1 + lu;"),
    "betas_transposed": ("float mt = b1 * m[i];", "float mt = b2 * m[i];"),
    "eps_inside_sqrt": ("float den = sqrtf(vh) + eps_f;", "float den = sqrtf(vh + eps_f);"),
    "no_weight_decay": ("float p1 = p[i] * decay;", "float p1 = p[i];"),
    "g_not_squared": ("float gg = gi * gi;", "float gg = gi;"),
    "dropped_last_replica": ("for (int32_t j = 1; j < N; j++)", "for (int32_t j = 1; j < N - 1; j++)"),
    "no_averaging": ("return (float)(1.0 / ((double)N * loss_scale));",
                     "return (float)(1.0 / loss_scale);"),
    "t_off_by_one": ("for (int64_t k = 0; k < t; k++)", "for (int64_t k = 0; k <= t; k++)"),
    "nan_not_flagged": ("if (!isfinite(g)) flag |= 1u;", "if (isinf(g)) flag |= 1u;"),
    "sumsq_not_squared": ("sumsq += (double)g * (double)g;", "sumsq += (double)g;"),
    "bf16_ties_up": ("return ((lo >> 16) & 1u) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);",
                     "return (uint16_t)(hi >> 16);"),
    "no_alignment": ("int64_t o = (i == 0) ? 0 : or_align_up(end, A);", "int64_t o = end;"),
    "segment_offset_wrong_base": ("out[4 * n + 1] = a - offsets[i];", "out[4 * n + 1] = a - lo;"),
    "shard_not_rounded_to_B": ("int64_t S = or_align_up(per_rank, B);", "int64_t S = per_rank;"),
    "stage2_grads_not_partitioned": ("case 2: par = P;  grd = Pn;", "case 2: par = P;  grd = P;"),
    "ring_adds_twice": ("partial[k * S + e] = or_hold(msg[k * S + e] + own[e], wire_dtype);",
                        "partial[k * S + e] = or_hold(msg[k * S + e] + own[e] + own[e], wire_dtype);"),
    "gather_uses_first_rank": ("        int64_t r = f / S;\n", "        int64_t r = offset / S;\n"),
    "gather_off_by_one": ("(size_t)(f - r * S) * (size_t)elem_bytes", "(size_t)(f - r * S + (e > 0)) * (size_t)elem_bytes"),
    "wire_not_rounded": ("return or_hold(acc + x, dtype == OR_BF16_WIRE ? OR_BF16 : OR_F32);",
                         "return acc + x;"),
    "wire_truncates": ("return wire_dtype == 0 ? x : or_bf16_to_f32(or_f32_to_bf16(x));",
                       "return wire_dtype == 0 ? x : or_bf16_to_f32((uint16_t)(or_bits(x) >> 16));"),
    "walk_skips_return_hop": ("for (int64_t h = 1; h <= N; h++) {", "for (int64_t h = 1; h < N; h++) {"),
    "bucket_never_cut": ("int cut = (k < S) && bucket_elems > 0 && (k % bucket_elems) == 0;",
                         "int cut = 0;"),
    "skip_rule_ignored": ("if (!flag) or_adam(", "if (1) or_adam("),
}


def all_pins(orc):
    """Run every CPU pin once; return the names of those that failed."""
    failed = []
    cases = [
        ("layout_tiny", lambda: TL.test_tiny_worked_example(orc)),
        ("layout_tiny3", lambda: TL.test_tiny_three_ranks_has_tail_padding(orc)),
        ("layout_align", lambda: TL.test_alignment_padding_between_tensors(orc)),
        ("layout_brute", lambda: [TL.test_brute_force_element_map(orc, s) for s in range(12)]),
        ("memory", lambda: [TM.test_page_formulas(orc, n) for n in ("tiny", "gpt2s")]),
        ("memory_small", lambda: TM.test_small_n_exact(orc)),
        ("ring_std", lambda: [TG.test_standard_ring_order_and_volume(orc, n) for n in (1, 2, 3, 8)]),
        ("ring_walk", lambda: [TG.test_page_walk_order_and_volume(orc, n) for n in (2, 8)]),
        ("ring_volumes", lambda: TG.test_page_volume_figures_for_eight_ranks(orc)),
        ("reduce_identity", lambda: TR.test_single_replica_is_identity(orc)),
        ("reduce_order", lambda: TR.test_left_fold_order_closed_form(orc)),
        ("reduce_inv", lambda: TR.test_inv_scale_rounding(orc)),
        ("reduce_higham", lambda: TR.test_higham_bound_against_fsum(orc, 8, "bf16")),
        ("reduce_overflow", lambda: TR.test_overflow_classes(orc)),
        ("reduce_sumsq", lambda: TR.test_sumsq_against_fsum(orc)),
        ("adam_torch", lambda: [TA.test_matches_torch_float64(orc, t, wd)
                                for t in (1, 3, 1000) for wd in (0.0, 0.01)]),
        ("adam_first", lambda: TA.test_first_step_closed_form(orc)),
        ("adam_const", lambda: TA.test_constant_gradient_moves_lr_per_step(orc)),
        ("adam_zero", lambda: TA.test_zero_gradient(orc)),
        ("adam_scalars", lambda: TA.test_scalars_use_t_fold_product(orc)),
        ("bf16", lambda: TB.test_ties_and_edges(orc)),
        ("step_skip", lambda: TS.test_overflow_skips_everything(orc)),
        ("step_trainer", lambda: TS.test_trainer_dynamic_scale_and_counter(orc)),
        ("wire_ties", lambda: TW.test_hand_computed_ties(orc)),
        ("wire_torch", lambda: [TW.test_matches_torch_bf16_tensor_adds(orc, n) for n in (2, 8)]),
        ("wire_ring", lambda: [TW.test_ring_with_bf16_messages_equals_wire_fold(orc, n)
                               for n in (2, 3)]),
        ("wire_exact", lambda: TW.test_no_rounding_when_sums_are_bf16_exact(orc)),
        ("wire_skip", lambda: TW.test_wire_rounding_can_decide_the_skip(orc)),
        ("gather_ring", lambda: [TGA.test_gather_equals_ring_all_gather_slices(orc, n)
                                 for n in (2, 3)]),
        ("gather_round_trip", lambda: TGA.test_round_trip_through_segments(orc, 1, 1)),
        ("gather_edges", lambda: TGA.test_tensor_spanning_every_rank_and_edges(orc)),
        ("golden_memory", lambda: [TGO.test_memory_per_device_matches_page(orc, n) for n in (2, 8)]),
        ("golden_reduction", lambda: TGO.test_stated_reductions_are_byte_model_limits(orc)),
        ("golden_ring", lambda: TGO.test_ring_fractions_for_eight_ranks(orc)),
    ]
    for name, fn in cases:
        try:
            fn()
        except Exception:          # a failed pin, or the mutant broke a call contract
            failed.append(name)
    return failed


def test_real_oracle_passes_all_pins():
    assert all_pins(oracle) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(before, after))
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", *oracle.GCC_FLAGS, str(mut), "-o", str(so), "-lm"], check=True)
    saved = oracle._lib
    oracle._lib = oracle.load(str(so))
    try:
        failed = all_pins(oracle)
    finally:
        oracle._lib = saved
    assert failed, f"planted mistake {name} passed every pin"
