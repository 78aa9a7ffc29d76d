"""Planted mistakes in the CPU oracle must be caught by its pins.

Each case copies oracle/pa_oracle.c, plants one plausible mistake (a wrong
index, a dropped term, a flipped sign, a transposed operand), builds the copy
with gcc into a temporary directory, and runs every pin of oracle_pins.py on
it: at least one pin must fail.  Everything runs on the CPU.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "pa_oracle.c")

# (name, text in pa_oracle.c, replacement)
MUTANTS = [
    ("gqa_modulo_map", "elem(pb->key_cache, key_index(pb, s, h / G, t, d), pb->dtype);",
     "elem(pb->key_cache, key_index(pb, s, h % pb->num_kv_heads, t, d), pb->dtype);"),
    ("value_head_map", "elem(pb->value_cache, value_index(pb, s, hv / G, t, d), pb->dtype);",
     "elem(pb->value_cache, value_index(pb, s, hv % pb->num_kv_heads, t, d), pb->dtype);"),
    ("logical_not_physical_block",
     "int32_t phys = pb->block_tables[(size_t)s * pb->max_blocks_per_seq + t / pb->block_size];",
     "int32_t phys = t / pb->block_size; (void)s;"),
    ("slab_axes_swapped", "return (size_t)phys * pb->num_kv_heads + kvh;",
     "return (size_t)kvh * pb->num_kv_heads + phys;"),
    ("key_layout_unsplit",
     "return ((slab * (size_t)(pb->head_dim / x) + (size_t)(d / x)) * pb->block_size + slot) * x +\n"
     "           d % x;",
     "return (slab * pb->block_size + slot) * (size_t)pb->head_dim + d + 0 * x;"),
    ("key_group_fixed", "return dtype == ORACLE_BF16 ? 8 : 4;", "return 8 + 0 * dtype;"),
    ("value_layout_token_major",
     "return (slab * (size_t)pb->head_dim + (size_t)d) * pb->block_size + slot;",
     "return (slab * pb->block_size + slot) * (size_t)pb->head_dim + d;"),
    ("scale_dropped", "return pb->scale * dot;", "return dot;"),
    ("scale_squared", "return pb->scale * dot;", "return pb->scale * pb->scale * dot;"),
    ("tail_not_masked", "if (attend_range(&pb, s, h, 0, L, o, &m, &den)) {",
     "if (attend_range(&pb, s, h, 0, (L + 15) / 16 * 16, o, &m, &den)) {"),
    ("first_token_dropped", "if (attend_range(&pb, s, h, 0, L, o, &m, &den)) {",
     "if (attend_range(&pb, s, h, L > 1 ? 1 : 0, L, o, &m, &den)) {"),
    ("softmax_sign", "double w = exp(z[t - t0] - zmax);", "double w = exp(zmax - z[t - t0]);"),
    ("unnormalised_output", "for (int d = 0; d < pb->head_dim; ++d) o[d] /= sum;",
     "for (int d = 0; d < pb->head_dim; ++d) o[d] /= 1.0;"),
    ("query_row_of_kv_head",
     "size_t qoff = ((size_t)s * pb->q_len * pb->num_q_heads + h) * pb->head_dim;",
     "size_t qoff = ((size_t)s * pb->q_len * pb->num_q_heads + h / G) * pb->head_dim;"),
    ("merge_sign", "double wgt = exp(m[p] - gmax) * es[p] / total;",
     "double wgt = exp(gmax - m[p]) * es[p] / total;"),
    ("merge_drops_exp_sum", "double wgt = exp(m[p] - gmax) * es[p] / total;",
     "double wgt = exp(m[p] - gmax) / total;"),
    ("partition_overlap", "int t1 = t0 + partition_size < L ? t0 + partition_size : L;",
     "int t1 = t0 + partition_size + 1 < L ? t0 + partition_size + 1 : L;"),
    ("partition_count_floor",
     "long parts = L > 0 ? ((long)L + partition_size - 1) / partition_size : 0;",
     "long parts = L > 0 ? (long)L / partition_size : 0;"),
    ("causal_off_by_one", "int visible = seq_lens[s] - q_len + j + 1; /* tokens 0 .. L - q_len + j */",
     "int visible = seq_lens[s] - q_len + j;"),
    ("query_token_ignored",
     "size_t qoff = ((size_t)s * pb->q_len * pb->num_q_heads + h) * pb->head_dim;",
     "size_t qoff = ((size_t)s * pb->q_len * pb->num_q_heads + h % pb->num_q_heads) * pb->head_dim;"),
    ("bf16_widen_wrong_half", "uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;",
     "uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 15;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_c = tmp_path / f"{name}.c"
    mutant_c.write_text(src.replace(old, new))
    lib_path = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                    "-o", str(lib_path), str(mutant_c), "-lm"], check=True)
    lib = oracle.load(str(lib_path))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
