"""Planted mistakes in the oracle must fail its pins.

Each case copies the oracle's C source, plants one plausible mistake (a wrong
index, a dropped term, a flipped sign, a transposed operand), compiles the copy
with gcc into a temporary directory and runs a set of pin checks from
test_oracle_pins against it.  At least one pin must fail for every mutation.
Nothing here touches a GPU.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle.build import SRC, build
from tests import test_oracle_pins as pins
from tests.conftest import golden

MUTATIONS = {
    "gqa_head_modulo": ("const int64_t kvh = h / g;", "const int64_t kvh = h % a->Hkv;"),
    "slot_offset_shift": ("const int64_t b = table[t / a->B], off = t % a->B;\n    int64_t krow;",
                          "const int64_t b = table[t / a->B], off = (t + 1) % a->B;\n    int64_t krow;"),
    "scale_dropped": ("x[t - t0] = a->scale * acc;", "x[t - t0] = acc;"),
    "max_sign_flipped": ("const double w = exp(x[t - t0] - m);", "const double w = exp(m - x[t - t0]);"),
    "merge_weight_flipped": ("w = exp(m - M);", "w = exp(M - m);"),
    "physical_index_transposed": ("return (int64_t)table[pos / block_size] * block_size + pos % block_size;",
                                  "return (int64_t)table[pos % block_size] * block_size + pos / block_size;"),
    "write_offset_transposed": ("const int64_t dst = (b * block_size + o) * row;",
                                "const int64_t dst = (o * block_size + b) * row;"),
    "bf16_widening_wrong_half": ("w = (uint32_t)h << 16;", "w = (uint32_t)h;"),
    "copy_direction_swapped": ("memcpy((char *)k_cache + d * blk, (const char *)k_cache + s * blk, (size_t)blk);",
                               "memcpy((char *)k_cache + s * blk, (const char *)k_cache + d * blk, (size_t)blk);"),
    "v_row_uses_k_head": ("const int64_t vrow = ((b * a->B + off) * a->Hkv + kvh) * a->D;",
                          "const int64_t vrow = ((b * a->B + off) * a->Hkv + (h % a->Hkv)) * a->D;"),
}


def _pin_checks():
    yield lambda: pins.test_physical_index_page_examples(None)
    for c in golden("physical_index.json")["cases"]:
        yield lambda c=c: pins.test_kv_write_lands_at_page_slot(c)
    yield pins.test_kv_write_then_gather_reads_back_bf16
    yield pins.test_copy_on_write_keeps_parent_bytes
    for case in pins.ATTN_CASES:
        yield lambda case=case: pins.test_attention_equals_library_sdpa_and_dense(case)
    yield pins.test_attention_single_token_returns_v
    yield pins.test_attention_uniform_weights_give_mean
    yield lambda: pins.test_split_k_equals_unsplit(8)
    yield pins.test_split_k_reduce_closed_form


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = build(src=str(mutated), lib=str(tmp_path / "libmutant.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.load(lib))
    caught = []
    for check in _pin_checks():
        try:
            check()
        except (AssertionError, oracle.OracleError) as e:
            caught.append(repr(e)[:80])
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_the_same_checks():
    for check in _pin_checks():
        check()
