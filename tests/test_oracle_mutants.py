"""Plants plausible mistakes in a copy of the oracle's source (on the CPU,
never in the library) and checks that the pins catch every one of them."""
import os
import types

import pytest

from tests import (helpers, test_fp8_codec, test_oracle, test_oracle_blocks,
                   test_oracle_slots)

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "rpa_oracle.py")
SRC = open(SRC_PATH).read()

MUTANTS = [
    ("gqa_mapping", "g = h // G", "g = h % Hkv"),
    ("causal_off_by_one", "m = j <= p", "m = j < p"),
    ("window_off_by_one", "(p - j) < sliding_window", "(p - j) <= sliding_window"),
    ("sink_not_in_denominator", "z = z + np.exp(sink[h] - m)", "z = z"),
    ("soft_cap_form", "logits_soft_cap * np.tanh(s / logits_soft_cap)",
     "np.tanh(s) * logits_soft_cap"),
    ("k_v_swapped_in_gather", "k = to_f64(rows[:, 0::2", "k = to_f64(rows[:, 1::2"),
    ("v_written_with_k", "out[page, off, 2 * h + 1, :D] = v[:, h, :]",
     "out[page, off, 2 * h + 1, :D] = k[:, h, :]"),
    ("context_off_by_one", "return q0, q_len, kv_len - q_len, kv_len",
     "return q0, q_len, kv_len - q_len - 1, kv_len"),
    ("page_index_and_offset_swapped",
     "page = np.asarray(block_tables, dtype=np.int64)[s * pages_per_seq + pos // page_size]\n"
     "    return page, pos % page_size",
     "page = np.asarray(block_tables, dtype=np.int64)[s * pages_per_seq + pos % page_size]\n"
     "    return page, pos // page_size"),
    ("q_scale_ignored", "scale = softmax_scale * (q_scale if q_scale else 1.0)",
     "scale = softmax_scale"),
    ("k_scale_ignored", "return k * (k_scale if k_scale else 1.0), v", "return k, v"),
    ("pad_lanes_kept", "            out[page, off, 2 * h, :] = 0\n", ""),
    ("ties_to_odd", "(lo % 2 == 0)", "(lo % 2 == 1)"),
    ("quantise_multiplies", "y = np.asarray(x_f32, dtype=np.float32) / s",
     "y = np.asarray(x_f32, dtype=np.float32) * s"),
    ("no_clamp", "y = np.clip(y, np.float32(-448.0), np.float32(448.0))", "y = y"),
    ("num_seqs_drops_mixed", "return int(d[0] + d[1] + d[2])", "return int(d[0] + d[1])"),
    ("pv_wrong_operand", "out[:, h, :] = _weighted_sum(w, v[:, g, :], mask) / z[:, None]",
     "out[:, h, :] = _weighted_sum(w, k[:, g, :], mask) / z[:, None]"),
    ("exp_sign", "w = np.where(mask, np.exp(s - m[:, None]), 0.0)",
     "w = np.where(mask, np.exp(m[:, None] - s), 0.0)"),
    ("subnormal_scale", "return s * (m / 8.0) * 2.0 ** -6", "return s * (m / 8.0) * 2.0 ** -7"),
    ("bf16_shift", "(bits.astype(np.uint32) << np.uint32(16))",
     "(bits.astype(np.uint32) << np.uint32(15))"),
    ("slot_offset_dropped", "out[q0:q0 + q_len] = page.astype(np.int64) * page_size + off",
     "out[q0:q0 + q_len] = page.astype(np.int64) * page_size"),
    ("padding_rows_get_slot_0", "out = np.full(total_tokens, PAD_SLOT, dtype=np.int64)",
     "out = np.zeros(total_tokens, dtype=np.int64)"),
    ("split_v_gets_k", "vc[b, o, :, :D] = v[i]", "vc[b, o, :, :D] = k[i]"),
    ("pad_slot_stored", "if sl < 0 or sl >= nb * bs:", "if sl >= nb * bs:"),
    ("split_pad_lanes_kept", "        kc[b, o] = 0\n", ""),
    ("swap_direction", "out[d] = src_cache[s]", "out[s] = src_cache[d]"),
    ("copy_reads_destination", "o[d] = c[s]", "o[d] = c[d]"),
    ("visible_window_off_by_one", "lo = max(0, ctx - sliding_window + 1) if sliding_window else 0",
     "lo = max(0, ctx - sliding_window) if sliding_window else 0"),
    ("visible_window_ignored", "lo = max(0, ctx - sliding_window + 1) if sliding_window else 0",
     "lo = 0"),
    ("visible_stops_before_last_key",
     "page, off = slot_of(block_tables, pages_per_seq, page_size, s, np.arange(lo, kv_len))",
     "page, off = slot_of(block_tables, pages_per_seq, page_size, s, np.arange(lo, kv_len - 1))"),
    ("scale_sign_dropped", "scale = softmax_scale * (q_scale if q_scale else 1.0)",
     "scale = abs(softmax_scale) * (q_scale if q_scale else 1.0)"),
]

T = test_oracle
PINS = [
    lambda: T.test_no_context_prefill_equals_sdpa(7, 4, 2, 16),
    T.test_window_equals_sdpa_with_band_mask,
    T.test_context_tail_alignment_equals_sdpa_slice,
    T.test_single_key_returns_v_exactly,
    T.test_single_key_with_sink_closed_form,
    T.test_window_one_returns_own_value,
    T.test_uniform_keys_average_visible_values,
    T.test_soft_cap_closed_form_two_keys,
    T.test_weights_sum_to_one,
    T.test_bruteforce_all_features,
    T.test_scatter_matches_hand_derived_slots,
    T.test_scatter_zero_fills_pad_lanes_and_roundtrips,
    T.test_scatter_fp8_quantises_with_scale,
    T.test_distribution_only_sets_num_seqs,
    T.test_chunked_prefill_and_decode_consistency,
    T.test_tiny_config_bruteforce_end_to_end,
    T.test_fp8_prefill_equals_sdpa_on_library_dequant,
    T.test_q_scale_multiplies_logits,
    T.test_fp8_queries_equal_sdpa_on_torch_dequant,
    T.test_masked_slots_may_hold_nan,
    lambda: T.test_visible_slots_match_hand_derived_slots(0),
    lambda: T.test_visible_slots_match_hand_derived_slots(4),
    lambda: T.test_visible_slots_match_hand_derived_slots(2),
    T.test_zero_scale_averages_visible_values,
    T.test_negative_scale_equals_sdpa,
    test_fp8_codec.test_decode_all_codes_match_torch,
    test_fp8_codec.test_closed_forms,
    test_fp8_codec.test_encode_every_bf16_pattern_matches_torch,
    test_oracle_slots.test_slot_mapping_matches_hand_derived_slots,
    lambda: test_oracle_slots.test_split_update_equals_combined_update("mixed_bf16"),
    test_oracle_slots.test_pad_and_out_of_pool_slots_are_skipped,
    test_oracle_blocks.test_swap_blocks_hand_example,
    test_oracle_blocks.test_copy_blocks_every_layer_same_pairs,
]


def load(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
    mod = types.ModuleType("rpa_oracle_mutant")
    exec(compile(SRC.replace(old, new), SRC_PATH + ":mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, monkeypatch):
    mod = load(old, new)
    for m in (helpers, test_oracle, test_fp8_codec, test_oracle_slots, test_oracle_blocks):
        monkeypatch.setattr(m, "O", mod)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except Exception:
            caught += 1
    assert caught > 0, f"no pin catches mutant {name}"


def test_unmutated_source_passes_all_pins(monkeypatch):
    mod = load("import math\n", "import math\n")
    for m in (helpers, test_oracle, test_fp8_codec, test_oracle_slots, test_oracle_blocks):
        monkeypatch.setattr(m, "O", mod)
    for pin in PINS:
        pin()
