"""Planted mistakes in a copy of the oracle must each fail at least one pin.

The oracle's source is read, one plausible slip is written into the copy (a
dropped term, a wrong sign, index or base, a transposed operand) and the copy
is executed as a fresh module; the real oracle is never modified.
"""

import pathlib
import types

import pytest

import pins

SRC = (pathlib.Path(__file__).resolve().parents[1] / "oracle" / "ref.py").read_text()

MUTANTS = {
    "head_map_modulo": ("return head // (num_qo_heads // num_kv_heads)",
                        "return head % num_kv_heads"),
    "scale_dropped": ("s = sm_scale * (q @ k.T)", "s = (q @ k.T)"),
    "scale_squared": ("s = sm_scale * (q @ k.T)", "s = sm_scale * sm_scale * (q @ k.T)"),
    "lse_natural_log": ("lse = (m[:, 0] + np.log(z)) / LN2", "lse = (m[:, 0] + np.log(z))"),
    "lse_max_dropped": ("lse = (m[:, 0] + np.log(z)) / LN2", "lse = np.log(z) / LN2"),
    "not_normalised": ("out = (w @ v) / z[:, None]", "out = (w @ v)"),
    "empty_lse_plus_inf": ("return np.zeros((h, v.shape[1])), np.full(h, -np.inf)",
                           "return np.zeros((h, v.shape[1])), np.full(h, np.inf)"),
    "k_head_zero": ("k = bf16_to_f64(k_bits[pages, 0, g, :])",
                    "k = bf16_to_f64(k_bits[pages, 0, 0, :])"),
    "v_from_k": ("v = bf16_to_f64(v_bits[pages, 0, g, :])",
                 "v = bf16_to_f64(k_bits[pages, 0, g, :])"),
    "bf16_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "exp_sign": ("w = np.exp(s - m)", "w = np.exp(m - s)"),
    "token_offset": ("pages = np.asarray(kv_indices[base + tok_begin: base + tok_end]",
                     "pages = np.asarray(kv_indices[base + tok_begin + 1: base + tok_end + 1]"),
    "merge_base_e": ("np.exp2(parts_lse - safe_top[None, :])",
                     "np.exp(parts_lse - safe_top[None, :])"),
    "merge_lse_no_log": ("safe_top + np.log2(np.where(empty, 1.0, den))", "safe_top"),
    "mla_upper_mask_dropped": ("ids = ids[(ids >= 0) & (ids < pool_tokens)]",
                               "ids = ids[(ids >= 0)]"),
    "mla_v_tail": ("attend(q, rows, rows[:, :d_v], sm_scale)",
                   "attend(q, rows, rows[:, -d_v:], sm_scale)"),
    "mla_sink_v_tail": ("(w @ rows[:, :d_v])", "(w @ rows[:, -d_v:])"),
    "bt_page_from_remainder": ("[j // page_size]", "[j % page_size]"),
    "bt_slot_shifted": ("slots = j % page_size", "slots = (j + 1) % page_size"),
    "bt_slot_ignored": ("k = bf16_to_f64(k_bits[pages, slots, g, :])",
                        "k = bf16_to_f64(k_bits[pages, 0, g, :])"),
    "bt_v_slot_reversed": ("v = bf16_to_f64(v_bits[pages, slots, g, :])",
                           "v = bf16_to_f64(v_bits[pages, page_size - 1 - slots, g, :])"),
    "bt_whole_pages": ("j = np.arange(int(seq_lens[b]), dtype=np.int64)",
                       "j = np.arange(-(-int(seq_lens[b]) // page_size) * page_size, dtype=np.int64)"),
    "bt_one_short": ("j = np.arange(int(seq_lens[b]), dtype=np.int64)",
                     "j = np.arange(max(int(seq_lens[b]) - 1, 0), dtype=np.int64)"),
    "append_slot_swapped": ("k_out[slot // page_size, slot % page_size] = k_rows[i]",
                            "k_out[slot % num_pages, slot // num_pages] = k_rows[i]"),
    "append_upper_bound_dropped": ("if 0 <= slot < num_pages * page_size:", "if 0 <= slot:"),
    "append_v_from_k": ("v_out[slot // page_size, slot % page_size] = v_rows[i]",
                        "v_out[slot // page_size, slot % page_size] = k_rows[i]"),
    "topk_length_off_by_one": ("ids = np.asarray(indices[b][:length], dtype=np.int64)",
                               "ids = np.asarray(indices[b][:length + 1], dtype=np.int64)"),
    "topk_length_unclamped": ("min(max(int(topk_length[b]), 0), topk)", "int(topk_length[b])"),
    "sink_in_lse": ("lse[b] = (m + np.log(z_keys)) / LN2",
                    "lse[b] = (m + np.log(z_keys + np.exp(sink - m))) / LN2"),
    "sink_base_2": ("(z_keys + np.exp(sink - m))[:, None]", "(z_keys + np.exp2(sink - m))[:, None]"),
    "sink_ignored": ("(z_keys + np.exp(sink - m))[:, None]", "(z_keys)[:, None]"),
    "e4m3_bias_8": ("(1.0 + m / 8.0) * np.exp2(e - 7.0)", "(1.0 + m / 8.0) * np.exp2(e - 8.0)"),
    "e4m3_subnormal_scale": ("(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7"),
    "fp8_scale_index_modulo": ("(vals.reshape(n, 4, 128) * scales[:, :, None])",
                               "(vals.reshape(n, 128, 4) * scales[:, None, :])"),
    "fp8_rope_offset": ("tokens[:, 528:656].copy()", "tokens[:, 512:640].copy()"),
    "fp8_no_bf16_rounding": ("((u + 0x7FFF + ((u >> 16) & 1)) >> 16)", "(u >> 16)"),
    "scores_transposed_q": ("s = sm_scale * (q @ k.T)", "s = sm_scale * (q[::-1] @ k.T)"),
}


def _load_mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load_mutant(*MUTANTS[name])
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception:  # AssertionError or a crash both count as caught
            return
    pytest.fail(f"no pin fails for mutant {name}")
