"""Host-side construction of one decode step and its upload to the GPU.

A decode step writes each sequence's newest token (position ctx - 1) through the
slot mapping, then attends over ctx tokens including it.  The block tables, the
slot mapping and any copy-on-write pairs are built on the CPU by the block
manager, once per batch (page "nano-vLLM . Ch04 . PagedAttention", section 9,
Myth 2: the slot mapping is computed on the CPU and handed to the GPU as a tensor).

Fork workload (one 2000-token prompt shared by 16 sequences):
  * the parent holds the prompt plus its first generated token (2001 tokens, the
    last of 126 blocks partly filled) and 15 children fork from it (refcount 16);
  * fork step: every sequence writes position 2001; the children meet refcount > 1
    and copy the partly filled block first, the parent (last holder) writes in
    place; then attention over 2002 tokens;
  * steady step: each sequence has grown to 2001 + its own generated tokens, token
    by token in sequence order at every position; the step writes the newest
    token (no copies remain to be made) and attends.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .block_manager import BlockManager


@dataclass
class DecodeStep:
    block_tables: np.ndarray     # int32 [S, max_blocks]
    context_lens: np.ndarray     # int32 [S]
    slot_mapping: np.ndarray     # int64 [S] slot of each sequence's newest token
    copy_pairs: np.ndarray       # int64 [P, 2] (src, dst) copies to run before the write
    max_context_len: int
    utilization: float           # fraction of pool blocks in use after the step's allocations


def _finish(bm: BlockManager, seqs, ctx, slots, pairs) -> DecodeStep:
    ctx = np.asarray(ctx, dtype=np.int32)
    max_ctx = int(ctx.max())
    tables = bm.block_tables(seqs, max_blocks=bm.blocks_needed(max_ctx))
    pr = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    return DecodeStep(tables, ctx, np.asarray(slots, dtype=np.int64), pr, max_ctx, bm.utilization())


def decode_step(context_lens, num_blocks: int, block_size: int, free_order) -> DecodeStep:
    """Independent sequences admitted in order; each holds ctx tokens, the newest at ctx - 1."""
    bm = BlockManager(num_blocks, block_size, free_order)
    seqs = []
    for c in np.asarray(context_lens).tolist():
        s = bm.new_sequence(int(c))
        if s is None:
            raise MemoryError(f"pool of {num_blocks} blocks cannot hold the batch")
        seqs.append(s)
    ctx = np.asarray(context_lens, dtype=np.int64)
    slots = bm.slot_mapping(seqs, ctx - 1)
    return _finish(bm, seqs, ctx, slots, [])


def _fork_family(bm: BlockManager, prompt_tokens: int, children: int):
    parent = bm.new_sequence(prompt_tokens + 1)
    if parent is None:
        raise MemoryError("pool too small for the shared prompt")
    kids = [bm.fork(parent) for _ in range(children)]
    return parent, kids


def fork_step(prompt_tokens: int, children: int, num_blocks: int, block_size: int, free_order) -> DecodeStep:
    bm = BlockManager(num_blocks, block_size, free_order)
    parent, kids = _fork_family(bm, prompt_tokens, children)
    pos = prompt_tokens + 1
    slots, pairs = {}, []
    for idx, seq in [(i + 1, k) for i, k in enumerate(kids)] + [(0, parent)]:
        if not bm.append_token(seq):
            raise MemoryError("pool exhausted")
        r = bm.prepare_write(seq, pos)
        if r is None:
            raise MemoryError("no free block for copy-on-write")
        slots[idx], pair = r
        if pair is not None:
            pairs.append(pair)
    seqs = [parent] + kids
    return _finish(bm, seqs, [pos + 1] * len(seqs), [slots[i] for i in range(len(seqs))], pairs)


def steady_fork_step(prompt_tokens: int, generated, num_blocks: int, block_size: int, free_order) -> DecodeStep:
    generated = [int(x) for x in np.asarray(generated).tolist()]
    bm = BlockManager(num_blocks, block_size, free_order)
    parent, kids = _fork_family(bm, prompt_tokens, len(generated) - 1)
    seqs = [parent] + kids
    ctx = [prompt_tokens + 1 + gi for gi in generated]
    order = list(range(1, len(seqs))) + [0]            # children, then the parent
    for pos in range(prompt_tokens + 1, max(ctx)):
        for i in order:
            if pos < ctx[i]:
                if not bm.append_token(seqs[i]) or bm.prepare_write(seqs[i], pos) is None:
                    raise MemoryError("pool exhausted")
    slots = bm.slot_mapping(seqs, np.asarray(ctx) - 1)
    return _finish(bm, seqs, ctx, slots, [])


def balanced_partition(num_seqs: int, num_kv_heads: int, max_context_len: int, block_size: int,
                       num_cus: int) -> int:
    """A partition size for a batch with too few (sequence, KV head) work items to give every
    compute unit one: the fewest equal pieces per sequence whose items cover every unit once,
    rounded up to whole blocks (16 sequences x 8 KV heads on 256 units: two pieces).  0 (unsplit)
    when the unsplit batch already covers them or a piece would be the whole context."""
    units = num_seqs * num_kv_heads
    if units <= 0 or units >= num_cus or max_context_len <= block_size:
        return 0
    parts = -(-num_cus // units)
    p = -(-max_context_len // parts)
    p = -(-p // block_size) * block_size
    return p if p < max_context_len else 0


# ---------------------------------------------------------------------------
# upload
# ---------------------------------------------------------------------------

def to_torch(a: np.ndarray, device, bf16: bool = False):
    """numpy -> torch on ``device``; uint16 arrays holding bf16 bit patterns become bfloat16."""
    import torch
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def from_torch_bits(t) -> np.ndarray:
    """Device tensor -> numpy; bfloat16 comes back as uint16 bit patterns, fp32 as float32."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def to_head_major(k_cache, v_cache):
    """Row-layout device caches [N, B, Hkv, D] placed in the head-major layout:
    k [N, Hkv, D/x, B, x] with x = 16 / element bytes, v [N, Hkv, D, B] (the same values)."""
    N, B, Hkv, D = k_cache.shape
    x = 16 // k_cache.element_size()
    k = k_cache.reshape(N, B, Hkv, D // x, x).permute(0, 2, 3, 1, 4).contiguous()
    v = v_cache.permute(0, 2, 3, 1).contiguous()
    return k, v


def step_for(wl, which: str = "steady") -> DecodeStep:
    """The decode step of a synthetic workload ('steady' or 'fork' for the fork workload)."""
    cfg = wl.cfg
    if cfg.ctx[0] == "fork":
        prompt = cfg.ctx[1]
        if which == "fork":
            return fork_step(prompt, cfg.num_seqs - 1, wl.num_blocks, cfg.block_size, wl.free_order)
        return steady_fork_step(prompt, wl.fork_generated, wl.num_blocks, cfg.block_size, wl.free_order)
    return decode_step(wl.context_lens, wl.num_blocks, cfg.block_size, wl.free_order)
