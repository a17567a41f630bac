"""Block-manager model -- TEST INFRASTRUCTURE ONLY (part of the CPU oracle).

A plain model of the host-side bookkeeping that feeds the decode kernels, used to
derive block tables, slots and copy-on-write pairs independently of the product's
own block manager.  It is written from the rules the pages state, not from their
listing, and keeps its state in its own form: a holder count per physical block and,
for every free block, the time at which it became free.

The rules (and where the pages state them):
  * Free blocks are reused most-recently-freed first, and a request for n blocks
    receives the n most recently freed ones, oldest of them first ("PagedAttention",
    PidokuInfra topic 10, section 4 "Tiny example": the allocator is a stack whose
    top n entries are handed out in stack order; the section's scenario, worked by
    hand in tests/golden/go_scenario.json, pins the order).  A request that cannot be
    met gets nothing and changes nothing (same section, ErrNoBlocks; nano-vLLM Ch04
    section 7: allocation failure is a return value).
  * A block becomes free when its last holder lets it go; sharing a table adds one
    holder to each of its blocks (PidokuInfra section 4, Fork; nano-vLLM section 6,
    "Copy-on-write block sharing": reference counts).
  * A sequence of n tokens holds exactly ceil(n / B) blocks, its table listing them
    in logical order (PidokuInfra section 4, BlocksNeeded; nano-vLLM section 4
    "The Three Mechanisms", the block table).
  * Token t of a sequence lives at slot table[t // B] * B + t % B (nano-vLLM
    section 4, Mechanism 3; PidokuInfra section 4, PhysicalIndex).
  * Writing into a block that has other holders first moves the writer onto a
    private copy: a fresh block, the old block loses the writer as a holder, the
    writer's table points at the copy, and the (old, copy) pair tells the GPU what to
    copy; with no other holder the write happens in place (nano-vLLM section 6).

Readings: a sequence grows its table only when a token needs a new block (the
growth rule follows from the ceil(n / B) rule at every length); a copy-on-write
that finds no free block raises and changes nothing.
"""
from __future__ import annotations

import heapq


class OutOfBlocks(Exception):
    pass


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class BlockModel:
    """Holder counts and free times of num_blocks physical blocks of block_size slots.

    free_order: the initial free blocks, least recently freed first (the last entry is
    handed out first); by default every id is free and id 0 was freed last."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.B = block_size
        self.num_blocks = num_blocks
        order = list(range(num_blocks - 1, -1, -1)) if free_order is None else [int(b) for b in free_order]
        assert sorted(order) == list(range(num_blocks)), "the free order must list every block once"
        self._holders = [0] * num_blocks
        self._freed_at: dict[int, int] = {b: i for i, b in enumerate(order)}
        self._clock = len(order)
        # the free blocks as a max-queue on their free time; an entry whose block has been
        # taken since (or freed again later) is stale and skipped
        self._queue = [(-t, b) for b, t in self._freed_at.items()]
        heapq.heapify(self._queue)

    # -- views of the state ----------------------------------------------------
    @property
    def free(self) -> list:
        """Free blocks, least recently freed first."""
        return sorted(self._freed_at, key=self._freed_at.__getitem__)

    @property
    def ref(self) -> dict:
        """Holder count of every held block."""
        return {b: n for b, n in enumerate(self._holders) if n}

    def holder_counts(self) -> list:
        """Holder count of every block id, 0 for free blocks."""
        return list(self._holders)

    def blocks_needed(self, tokens: int) -> int:
        return _ceil_div(tokens, self.B)

    # -- blocks -----------------------------------------------------------------
    def allocate(self, n: int):
        """The n most recently freed blocks, oldest of them first, each with one holder;
        None (and nothing changes) if fewer than n are free."""
        if n > len(self._freed_at):
            return None
        newest = []
        while len(newest) < n:
            t, b = heapq.heappop(self._queue)
            if self._freed_at.get(b) == -t:
                del self._freed_at[b]
                newest.append(b)
        for b in newest:
            self._holders[b] = 1
        return newest[::-1]

    def release(self, blocks) -> None:
        """One holder fewer for each block, in order; a block with none left is free from now."""
        for b in blocks:
            assert self._holders[b] > 0, f"block {b} is not held"
            self._holders[b] -= 1
            if self._holders[b] == 0:
                self._freed_at[b] = self._clock
                heapq.heappush(self._queue, (-self._clock, b))
                self._clock += 1

    def fork(self, blocks):
        """A new table sharing these blocks: one more holder for each."""
        for b in blocks:
            assert self._holders[b] > 0, f"block {b} is not held"
            self._holders[b] += 1
        return list(blocks)

    # -- sequences: dicts {"table": [...], "len": n} ------------------------------
    def new_sequence(self, prompt_len: int):
        table = self.allocate(self.blocks_needed(prompt_len))
        return None if table is None else {"table": table, "len": prompt_len}

    def append_token(self, seq) -> bool:
        """Length + 1, holding ceil(len / B) blocks afterwards; False (nothing changes) if the
        block the new token needs cannot be had."""
        missing = self.blocks_needed(seq["len"] + 1) - len(seq["table"])
        if missing > 0:
            got = self.allocate(missing)
            if got is None:
                return False
            seq["table"] = seq["table"] + got
        seq["len"] += 1
        return True

    def physical_index(self, seq, pos: int) -> int:
        block, offset = divmod(pos, self.B)
        return seq["table"][block] * self.B + offset

    def write_slot(self, seq, pos: int):
        """Slot for writing position pos, after copy-on-write if the block has other holders.

        Returns (slot, pair) where pair = (old, copy) if the writer was moved onto a copy.
        Raises OutOfBlocks (and changes nothing) if a copy is needed and no block is free."""
        j = pos // self.B
        old = seq["table"][j]
        pair = None
        if self._holders[old] > 1:
            got = self.allocate(1)
            if got is None:
                raise OutOfBlocks
            self.release([old])          # the old block keeps its other holders
            seq["table"] = seq["table"][:j] + got + seq["table"][j + 1:]
            pair = (old, got[0])
        return self.physical_index(seq, pos), pair

    # -- invariants -------------------------------------------------------------
    def check(self, seqs) -> None:
        counts = [0] * self.num_blocks
        for s in seqs:
            assert len(s["table"]) == self.blocks_needed(s["len"]), "a sequence holds ceil(len / B) blocks"
            for b in s["table"]:
                counts[b] += 1
        assert counts == self._holders, "holder counts must equal the number of tables holding each block"
        for b in range(self.num_blocks):
            assert (b in self._freed_at) == (self._holders[b] == 0), "a block is free iff nobody holds it"
        assert len(set(self._freed_at.values())) == len(self._freed_at)


def build_tables(seqs, max_blocks: int | None = None, pad: int = 0):
    """[S, max_blocks] int rows of the sequences' tables, padded with ``pad``."""
    import numpy as np
    mb = max(len(s["table"]) for s in seqs) if max_blocks is None else max_blocks
    out = np.full((len(seqs), mb), pad, dtype=np.int32)
    for i, s in enumerate(seqs):
        out[i, :len(s["table"])] = s["table"]
    return out


class PrefixModel:
    """Prefix reuse of full prompt blocks, as a plain model (test infrastructure).

    A block of a prompt can stand for the same block of another prompt only when the two
    agree on every token up to its end: its identity is the whole prefix it closes
    (PidokuInfra page, section 5 "The relationship to prefix caching": full blocks are
    looked up by their token ids, and a hit on the first j blocks means the first j * B
    tokens match).  Keys here are the literal token tuples, not hashes.  Only full blocks
    are entered; the last, partly filled block of a prompt stays private.  A block leaves
    the map when nobody holds it any more."""

    def __init__(self, model: BlockModel):
        self.m = model
        self.by_prefix: dict[tuple, int] = {}
        self.prefix_of: dict[int, tuple] = {}

    def _key(self, tokens, j: int) -> tuple:
        """Identity of full block j of a prompt: every token up to the block's end."""
        return tuple(tokens[:(j + 1) * self.m.B])

    def new_sequence(self, tokens):
        """(sequence, number of leading blocks reused), or None (nothing changes) when the
        blocks the prompt still needs cannot be had."""
        tokens = [int(t) for t in tokens]
        full = len(tokens) // self.m.B
        hits = []
        for j in range(full):
            b = self.by_prefix.get(self._key(tokens, j))
            if b is None:
                break
            hits.append(b)
        fresh = self.m.allocate(self.m.blocks_needed(len(tokens)) - len(hits))
        if fresh is None:
            return None
        table = self.m.fork(hits) + fresh
        for j in range(len(hits), full):
            key = self._key(tokens, j)
            self.by_prefix[key] = table[j]
            self.prefix_of[table[j]] = key
        return {"table": table, "len": len(tokens)}, len(hits)

    def release(self, seq) -> None:
        table = list(seq["table"])
        self.m.release(table)
        for b in table:
            if b not in self.m.ref and b in self.prefix_of:
                del self.by_prefix[self.prefix_of.pop(b)]
