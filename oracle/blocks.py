"""Block-manager model -- TEST INFRASTRUCTURE ONLY (part of the CPU oracle).

A plain model of the host-side bookkeeping that feeds the decode kernels, used to
derive block tables, slots and copy-on-write pairs independently of the product's
own block manager.

Sources:
  * page "PagedAttention" (PidokuInfra, topic 10), section 4 "Tiny example":
    the free stack (Allocate takes the last n ids, in stack order), Free (an id
    returns to the stack only when its refcount reaches 0), Fork (share the ids,
    bump every refcount), BlocksNeeded = ceil(tokens / B), AppendToken (grow by
    one block when BlocksNeeded exceeds the table length), PhysicalIndex.
  * page "nano-vLLM . Ch04 . PagedAttention", section 6 "Copy-on-write block
    sharing": before writing into a block with refcount > 1, copy it, decrement
    the old block's count, give the copy to the writer, then write; with
    refcount 1, write in place.  Section 7: allocation failure returns a value
    (no exception) and changes nothing.

Readings: the growth rule is section 4's BlocksNeeded comparison (exact at every
length); an allocation that cannot be met leaves the model unchanged.
"""
from __future__ import annotations


class OutOfBlocks(Exception):
    pass


class BlockModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.B = block_size
        self.num_blocks = num_blocks
        # the free stack; its last element is handed out first
        self.free = list(range(num_blocks - 1, -1, -1)) if free_order is None else [int(b) for b in free_order]
        assert sorted(self.free) == list(range(num_blocks))
        self.ref: dict[int, int] = {}

    # -- allocator -----------------------------------------------------------
    def allocate(self, n: int):
        """n fresh ids (the top n of the stack, in stack order), or None if fewer are free."""
        if len(self.free) < n:
            return None
        taken = self.free[len(self.free) - n:]
        del self.free[len(self.free) - n:]
        for b in taken:
            self.ref[b] = 1
        return taken

    def release(self, blocks) -> None:
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                del self.ref[b]
                self.free.append(b)

    def fork(self, blocks):
        for b in blocks:
            self.ref[b] += 1
        return list(blocks)

    def blocks_needed(self, tokens: int) -> int:
        return (tokens + self.B - 1) // self.B

    # -- sequences: dicts {"table": [...], "len": n} ---------------------------
    def new_sequence(self, prompt_len: int):
        t = self.allocate(self.blocks_needed(prompt_len))
        if t is None:
            return None
        return {"table": t, "len": prompt_len}

    def append_token(self, seq) -> bool:
        if self.blocks_needed(seq["len"] + 1) > len(seq["table"]):
            t = self.allocate(1)
            if t is None:
                return False
            seq["table"].extend(t)
        seq["len"] += 1
        return True

    def physical_index(self, seq, pos: int) -> int:
        return seq["table"][pos // self.B] * self.B + pos % self.B

    def write_slot(self, seq, pos: int):
        """Slot for writing position pos, applying copy-on-write.

        Returns (slot, pair) where pair = (old, new) if the block had to be copied first.
        Raises OutOfBlocks (and changes nothing) if a copy is needed and no block is free.
        """
        j = pos // self.B
        b = seq["table"][j]
        pair = None
        if self.ref[b] > 1:
            fresh = self.allocate(1)
            if fresh is None:
                raise OutOfBlocks
            nb = fresh[0]
            self.ref[b] -= 1
            seq["table"][j] = nb
            pair = (b, nb)
        return self.physical_index(seq, pos), pair

    # -- invariants ----------------------------------------------------------
    def check(self, seqs) -> None:
        counts: dict[int, int] = {}
        for s in seqs:
            for b in s["table"]:
                counts[b] = counts.get(b, 0) + 1
        assert counts == self.ref, "refcounts must equal the number of tables holding each block"
        assert set(self.free).isdisjoint(self.ref), "a block is free iff its refcount is 0"
        assert len(self.free) + len(self.ref) == self.num_blocks
        assert len(set(self.free)) == len(self.free)


def build_tables(seqs, max_blocks: int | None = None, pad: int = 0):
    """[S, max_blocks] int rows of the sequences' tables, padded with ``pad``."""
    import numpy as np
    mb = max(len(s["table"]) for s in seqs) if max_blocks is None else max_blocks
    out = np.full((len(seqs), mb), pad, dtype=np.int32)
    for i, s in enumerate(seqs):
        out[i, :len(s["table"])] = s["table"]
    return out


class PrefixModel:
    """Prefix reuse of full prompt blocks, as a plain model (test infrastructure): a new
    prompt's leading blocks are reused when its first j * B tokens equal those of a block
    held in the map (PidokuInfra page, section 5 "The relationship to prefix caching"; the
    block's identity is its whole token prefix).  Keys are the literal token tuples, not
    hashes.  A block leaves the map when its refcount reaches zero."""

    def __init__(self, model: BlockModel):
        self.m = model
        self.by_prefix: dict[tuple, int] = {}
        self.prefix_of: dict[int, tuple] = {}

    def new_sequence(self, tokens):
        B = self.m.B
        tokens = [int(t) for t in tokens]
        full = len(tokens) // B
        hits = []
        while len(hits) < full:
            b = self.by_prefix.get(tuple(tokens[:(len(hits) + 1) * B]))
            if b is None:
                break
            hits.append(b)
        fresh = self.m.allocate(self.m.blocks_needed(len(tokens)) - len(hits))
        if fresh is None:
            return None
        table = self.m.fork(hits) + fresh
        for j in range(len(hits), full):
            self.by_prefix[tuple(tokens[:(j + 1) * B])] = table[j]
            self.prefix_of[table[j]] = tuple(tokens[:(j + 1) * B])
        return {"table": table, "len": len(tokens)}, len(hits)

    def release(self, seq) -> None:
        table = list(seq["table"])
        self.m.release(table)
        for b in table:
            if b not in self.m.ref and b in self.prefix_of:
                del self.by_prefix[self.prefix_of.pop(b)]
