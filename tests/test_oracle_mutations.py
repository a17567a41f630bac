"""Planted mistakes in the oracle must fail its pins.

Each case copies the oracle's C source, plants one plausible mistake (a wrong
index, a dropped term, a flipped sign, a transposed operand), compiles the copy
with gcc into a temporary directory and runs a set of pin checks from
test_oracle_pins against it.  The Python parts of the oracle (the block model, the
prefix-reuse model and the decode-step builder) get the same treatment: a copy of
the source with one planted mistake is loaded as a module of its own and put in
place of the original for the pins.  At least one pin must fail for every mutation.
Nothing here touches a GPU.
"""
import math
import os
import types

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


# ---------------------------------------------------------------------------
# the Python parts of the oracle
# ---------------------------------------------------------------------------

ORACLE_DIR = os.path.dirname(SRC)
BLOCKS_PY = os.path.join(ORACLE_DIR, "blocks.py")
BATCH_PY = os.path.join(ORACLE_DIR, "batch.py")
BATCH_IMPORT = "from oracle.blocks import BlockModel, build_tables"

PY_MUTATIONS = {
    # the block model
    "allocate_newest_first": (BLOCKS_PY, "return newest[::-1]", "return newest"),
    "free_while_still_held": (BLOCKS_PY, "if self._holders[b] == 0:", "if self._holders[b] <= 1:"),
    "fork_adds_no_holder": (BLOCKS_PY, "self._holders[b] += 1", "self._holders[b] += 0"),
    "cow_only_above_two_holders": (BLOCKS_PY, "if self._holders[old] > 1:", "if self._holders[old] > 2:"),
    "cow_keeps_writer_on_old_block": (BLOCKS_PY, "self.release([old])          # the old block keeps its other holders",
                                      "pass"),
    "grow_one_token_late": (BLOCKS_PY, 'missing = self.blocks_needed(seq["len"] + 1) - len(seq["table"])',
                            'missing = self.blocks_needed(seq["len"]) - len(seq["table"])'),
    # the prefix-reuse model
    "prefix_key_own_block_only": (BLOCKS_PY, "return tuple(tokens[:(j + 1) * self.m.B])",
                                  "return tuple(tokens[j * self.m.B:(j + 1) * self.m.B])"),
    "prefix_partial_block_entered": (BLOCKS_PY, "full = len(tokens) // self.m.B",
                                     "full = self.m.blocks_needed(len(tokens))"),
    "prefix_map_outlives_blocks": (BLOCKS_PY, "del self.by_prefix[self.prefix_of.pop(b)]", "pass"),
    # the fork workload's step builder
    "parent_writes_before_children": (BATCH_PY,
                                      "for i, s in [(i + 1, k) for i, k in enumerate(kids)] + [(0, parent)]:",
                                      "for i, s in [(0, parent)] + [(i + 1, k) for i, k in enumerate(kids)]:"),
    "parent_without_first_token": (BATCH_PY, "parent = m.new_sequence(prompt_tokens + 1)\n    kids",
                                   "parent = m.new_sequence(prompt_tokens)\n    kids"),
    "steady_writes_skip_cow": (BATCH_PY, "                m.write_slot(seqs[i], pos)\n", "                pass\n"),
}


def _module(name, text, inject=None):
    mod = types.ModuleType(name)
    mod.__dict__.update(inject or {})
    exec(compile(text, f"<{name}>", "exec"), mod.__dict__)
    return mod


def _py_oracle(blocks_text, batch_text):
    blocks = _module("mutant_blocks", blocks_text)
    assert BATCH_IMPORT in batch_text
    batch = _module("mutant_batch", batch_text.replace(BATCH_IMPORT, ""),
                    {"BlockModel": blocks.BlockModel, "build_tables": blocks.build_tables})
    return blocks, batch


def _py_pin_checks():
    yield pins.test_go_scenario_block_model
    yield pins.test_sharing_counts
    yield pins.test_block_model_oom_leaves_state_unchanged
    yield pins.test_block_model_append_growth_rule
    yield pins.test_block_model_random_ops_invariants
    yield pins.test_copy_on_write_keeps_parent_bytes
    for case in golden("prefix_sharing.json")["cases"]:
        yield lambda case=case: pins.test_prefix_model_ten_requests_share_one_prompt(case)
    yield pins.test_prefix_model_divergent_shifted_and_released
    yield pins.test_prefix_model_same_block_ids_under_two_prefixes
    yield pins.test_prefix_model_out_of_blocks_changes_nothing
    yield pins.test_oracle_fork_step_counts
    yield pins.test_oracle_steady_fork_step_counts


def _run_py_checks(blocks_text, batch_text, monkeypatch):
    blocks, batch = _py_oracle(blocks_text, batch_text)
    monkeypatch.setattr(pins, "BlockModel", blocks.BlockModel)
    monkeypatch.setattr(pins, "PrefixModel", blocks.PrefixModel)
    monkeypatch.setattr(pins, "obatch", batch)
    failed = []
    for check in _py_pin_checks():
        try:
            check()
        except (Exception, pytest.fail.Exception) as e:   # a wrong value or a crash: the pin fails
            failed.append(repr(e)[:80])
    return failed


@pytest.mark.parametrize("name", sorted(PY_MUTATIONS))
def test_planted_mistake_in_python_oracle_is_caught(name, monkeypatch):
    path, old, new = PY_MUTATIONS[name]
    texts = {p: open(p).read() for p in (BLOCKS_PY, BATCH_PY)}
    assert texts[path].count(old) == 1, f"mutation anchor for {name} not found once"
    texts[path] = texts[path].replace(old, new, 1)
    caught = _run_py_checks(texts[BLOCKS_PY], texts[BATCH_PY], monkeypatch)
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmutated_python_oracle_passes_the_same_checks(monkeypatch):
    assert _run_py_checks(open(BLOCKS_PY).read(), open(BATCH_PY).read(), monkeypatch) == []
