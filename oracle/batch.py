"""Decode-step inputs derived with the oracle's block model -- TEST INFRASTRUCTURE ONLY.

Independent of the product's block manager: tests check that both produce the
same block tables, slots and copy-on-write pairs from the same free-stack order.

Readings (where the pages leave the step open):
  * each step writes the newest token at position ctx - 1, then attends over ctx
    tokens including it;
  * fork workload: the parent holds the 2000-token prompt and its first generated
    token (2001 tokens), 15 children fork from it; at the fork step every
    sequence writes position 2001, children first (each copies the shared, partly
    filled block: copy-on-write, nano-vLLM Ch04 section 6), then the parent, who
    is by then the block's only holder and writes in place;
  * steady step: sequences grow one position at a time, children then parent at
    each position, to 2001 + their own generated tokens.
"""
from __future__ import annotations

import numpy as np

from oracle.blocks import BlockModel, build_tables


def _pack(m, seqs, ctx, slots, pairs):
    ctx = np.asarray(ctx, dtype=np.int32)
    width = m.blocks_needed(int(ctx.max()))
    return {
        "block_tables": build_tables(seqs, width),
        "context_lens": ctx,
        "slot_mapping": np.asarray(slots, dtype=np.int64),
        "copy_pairs": np.asarray(pairs, dtype=np.int64).reshape(-1, 2),
        "holders": np.asarray(m.holder_counts(), dtype=np.int32),   # per block id, after the step
    }


def decode_step(context_lens, num_blocks, block_size, free_order):
    m = BlockModel(num_blocks, block_size, free_order)
    seqs = [m.new_sequence(int(c)) for c in context_lens]
    slots = [m.physical_index(s, int(c) - 1) for s, c in zip(seqs, context_lens)]
    return _pack(m, seqs, context_lens, slots, [])


def fork_step(prompt_tokens, children, num_blocks, block_size, free_order):
    m = BlockModel(num_blocks, block_size, free_order)
    parent = m.new_sequence(prompt_tokens + 1)
    kids = [{"table": m.fork(parent["table"]), "len": parent["len"]} for _ in range(children)]
    pos = prompt_tokens + 1
    slots, pairs = [None] * (children + 1), []
    for i, s in [(i + 1, k) for i, k in enumerate(kids)] + [(0, parent)]:
        assert m.append_token(s)
        slots[i], pair = m.write_slot(s, pos)
        if pair:
            pairs.append(pair)
    m.check([parent] + kids)
    return _pack(m, [parent] + kids, [pos + 1] * (children + 1), slots, pairs)


def steady_fork_step(prompt_tokens, generated, num_blocks, block_size, free_order):
    m = BlockModel(num_blocks, block_size, free_order)
    parent = m.new_sequence(prompt_tokens + 1)
    seqs = [parent] + [{"table": m.fork(parent["table"]), "len": parent["len"]} for _ in range(len(generated) - 1)]
    ctx = [prompt_tokens + 1 + int(x) for x in generated]
    for pos in range(prompt_tokens + 1, max(ctx)):
        for i in list(range(1, len(seqs))) + [0]:
            if pos < ctx[i]:
                assert m.append_token(seqs[i])
                m.write_slot(seqs[i], pos)
    m.check(seqs)
    slots = [m.physical_index(s, c - 1) for s, c in zip(seqs, ctx)]
    return _pack(m, seqs, ctx, slots, [])


def step_for(wl, which: str = "steady"):
    """Oracle-side step inputs of a workloads.Workload ('steady' or 'fork' for the fork workload)."""
    cfg = wl.cfg
    if cfg.ctx[0] == "fork":
        prompt = cfg.ctx[1]
        if which == "fork":
            return fork_step(prompt, cfg.num_seqs - 1, wl.num_blocks, cfg.block_size, wl.free_order)
        return steady_fork_step(prompt, wl.fork_generated, wl.num_blocks, cfg.block_size, wl.free_order)
    return decode_step(wl.context_lens, wl.num_blocks, cfg.block_size, wl.free_order)
