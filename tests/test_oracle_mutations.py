"""Planted mistakes in a copy of the oracle must each trip at least one pin.

Each mutation rewrites one line of the oracle's source text (a dropped term, a
wrong sign or index, a transposed operand), loads the result as a separate
module on the CPU and runs every pin against it.
"""

import importlib.util
import os
import types

import pytest

import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "paged_attention.py")

MUTATIONS = {
    "gqa_modulo_mapping": ("g = h // group\n            out[b, h]", "g = h % num_kv_heads\n            out[b, h]"),
    "page_slot_swapped": ("logical_page = t // PAGE_SIZE", "logical_page = t % PAGE_SIZE"),
    "slot_from_page": ("slot = t % PAGE_SIZE\n        physical", "slot = (t + 1) % PAGE_SIZE\n        physical"),
    "block_table_ignored": ("physical = int(block_table_row[logical_page])", "physical = logical_page"),
    "v_read_k_layout": ("vc[t] = bf16_bits_to_f64(v_pool[physical, :, :, slot])",
                        "vc[t] = bf16_bits_to_f64(v_pool[physical, :, slot % v_pool.shape[2], :slot + 1].repeat(v_pool.shape[2], axis=-1)[:, :v_pool.shape[2]])"),
    "dropped_scale": ("scores = scale * (keys @ q_vec)", "scores = (keys @ q_vec)"),
    "keys_values_swapped": ("scores = scale * (keys @ q_vec)", "scores = scale * (values @ q_vec)"),
    "softmax_sign": ("e = np.exp(scores - m)", "e = np.exp(m - scores)"),
    "min_instead_of_max": ("m = np.max(scores)", "m = np.min(scores)"),
    "dropped_normaliser": ("return (e @ values) / z", "return (e @ values)"),
    "normalise_by_count": ("return (e @ values) / z", "return (e @ values) / len(e) * (z / z)"),
    "bf16_shift": ("(bits.astype(np.uint32) << 16)", "(bits.astype(np.uint32) << 15)"),
    "query_head_kv_row": ("out[b, h] = attend_one_head(qb[h], kc[:, g, :], vc[:, g, :], scale)",
                          "out[b, h] = attend_one_head(qb[g], kc[:, g, :], vc[:, g, :], scale)"),
    "append_wrong_slot": ("set_k_slot_row(k_out, physical, slot, k_new[b])",
                          "set_k_slot_row(k_out, physical, (slot + 1) % PAGE_SIZE, k_new[b])"),
    "append_v_wrong_head": ("v_out[physical, :, :, slot] = v_new[b]",
                            "v_out[physical, :, :, slot] = v_new[b, :1]"),
    "k_read_slabs_transposed": ("return k_pool[physical, :, :, slot, :].reshape(",
                                "return k_pool[physical, :, :, slot, :].transpose(0, 2, 1).reshape("),
    "k_write_slabs_reversed": ("k_pool[physical, :, :, slot, :] = rows.reshape(rows.shape[0], -1, K_SLAB)",
                               "k_pool[physical, :, :, slot, :] = rows.reshape(rows.shape[0], -1, K_SLAB)[:, ::-1]"),
    "append_ignores_skip": ("if pos < 0:\n            continue", "if pos < -10**9:\n            continue"),
    "ctx_zero_not_zero": ("if n == 0:\n            continue\n        kc, vc",
                          "if n == 0:\n            out[b] = 1.0\n            continue\n        kc, vc"),
    "off_by_one_ctx": ("kc, vc = gather_sequence(k_pool, v_pool, block_tables[b], n)",
                       "kc, vc = gather_sequence(k_pool, v_pool, block_tables[b], max(1, n - 1))"),
    "prefill_not_causal": ("kc[:p + 1, g, :], vc[:p + 1, g, :]", "kc[:, g, :], vc[:, g, :]"),
    "prefill_causal_off_by_one": ("kc[:p + 1, g, :], vc[:p + 1, g, :]", "kc[:p + 2, g, :], vc[:p + 2, g, :]"),
    "prefill_ignores_cache": ("p = before + row - first", "p = row - first"),
    "prefill_gqa_modulo": ("g = h // group\n                out[row, h]",
                           "g = h % k_pool.shape[1]\n                out[row, h]"),
    "write_ignores_cache": ("pos = int(ctx_before[b]) + row - int(query_start[b])",
                            "pos = row - int(query_start[b])"),
    "write_v_from_k": ("v_out[physical, :, :, slot] = v_rows[row]", "v_out[physical, :, :, slot] = k_rows[row]"),
    "prefill_reads_old_pool": ("kc, vc = gather_sequence(k_new_pool, v_new_pool,",
                               "kc, vc = gather_sequence(k_pool, v_pool,"),
}


def load_mutant(name):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation {name}: anchor not found exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(text.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mutant = load_mutant(name)
    tripped = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception as exc:  # AssertionError or a crash both count
            tripped.append((pin.__name__, type(exc).__name__))
    assert tripped, f"no pin caught the planted mistake {name!r}"
