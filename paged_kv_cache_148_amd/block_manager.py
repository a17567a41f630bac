"""Host-side block manager: the CPU bookkeeping that feeds the decode kernels.

The pool of ``num_blocks`` physical blocks is handed out from a free stack; each
sequence holds a block table (logical block -> physical id); a refcount per
block allows sharing between forked sequences, with copy-on-write before a
write into a shared block.  Sources:

* page "nano-vLLM . Ch04 . PagedAttention": section 4 (free list, block table,
  slot mapping computed on the CPU once per batch), section 6 (refcounts and
  copy-on-write: copy first, drop the old block's count, hand the copy to the
  writer, then write; with a count of one write in place), section 7
  (allocation failure is a return value, not an exception).
* page "PagedAttention" (PidokuInfra, topic 10), section 4: Allocate takes the
  top n ids of the stack in stack order, Free returns an id when its count
  reaches zero, Fork bumps every count, AppendToken grows the table by one block
  when BlocksNeeded(len) exceeds its length, PhysicalIndex.

Everything here is integer bookkeeping on the host; nothing is timed on the GPU.
A failed allocation or copy-on-write leaves every structure unchanged.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Sequence:
    """One request: its block table and its length in tokens."""
    table: list = field(default_factory=list)
    length: int = 0


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        # free stack: the last element is handed out first; by default ids N-1..0 are
        # pushed in that order, so id 0 is on top
        if free_order is None:
            self._free = list(range(num_blocks - 1, -1, -1))
        else:
            self._free = [int(b) for b in free_order]
            if sorted(self._free) != list(range(num_blocks)):
                raise ValueError("free_order must be a permutation of range(num_blocks)")
        self._ref = np.zeros(num_blocks, dtype=np.int32)

    # ------------------------------------------------------------------ pool
    @property
    def free_blocks(self) -> list:
        return list(self._free)

    def num_free(self) -> int:
        return len(self._free)

    def refcount(self, block: int) -> int:
        return int(self._ref[block])

    def utilization(self) -> float:
        """Fraction of the pool's blocks held by at least one sequence."""
        return 1.0 - len(self._free) / self.num_blocks

    def blocks_needed(self, tokens: int) -> int:
        return -(-tokens // self.block_size)

    def allocate(self, n: int):
        """Pop n ids (top of the stack, in stack order) with refcount 1, or None if short."""
        if n < 0:
            raise ValueError("n must be >= 0")
        if n > len(self._free):
            return None
        cut = len(self._free) - n
        ids = self._free[cut:]
        del self._free[cut:]
        self._ref[ids] = 1
        return ids

    def free(self, blocks) -> None:
        """Drop one reference to each block; a block returns to the stack at zero."""
        for b in blocks:
            if self._ref[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
            self._ref[b] -= 1
            if self._ref[b] == 0:
                self._free.append(int(b))

    def fork_table(self, blocks) -> list:
        """Share the blocks with a new table (every refcount + 1)."""
        for b in blocks:
            if self._ref[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
        for b in blocks:
            self._ref[b] += 1
        return list(blocks)

    # ------------------------------------------------------------- sequences
    def new_sequence(self, prompt_tokens: int):
        ids = self.allocate(self.blocks_needed(prompt_tokens))
        return None if ids is None else Sequence(ids, prompt_tokens)

    def fork(self, seq: Sequence) -> Sequence:
        return Sequence(self.fork_table(seq.table), seq.length)

    def release(self, seq: Sequence) -> None:
        self.free(seq.table)
        seq.table = []
        seq.length = 0

    def append_token(self, seq: Sequence) -> bool:
        """Grow the sequence by one token, taking one more block when it needs one."""
        if self.blocks_needed(seq.length + 1) > len(seq.table):
            ids = self.allocate(1)
            if ids is None:
                return False
            seq.table.extend(ids)
        seq.length += 1
        return True

    def physical_index(self, seq: Sequence, pos: int) -> int:
        B = self.block_size
        return seq.table[pos // B] * B + pos % B

    def prepare_write(self, seq: Sequence, pos: int):
        """Slot for writing position ``pos`` of ``seq``, applying copy-on-write.

        Returns ``(slot, copy_pair)``; ``copy_pair`` is ``(src, dst)`` when the block was
        shared and had to be copied to a fresh block first, else None.  Returns None
        (and changes nothing) when a copy is needed but no block is free.
        """
        j = pos // self.block_size
        old = seq.table[j]
        if self._ref[old] > 1:
            ids = self.allocate(1)
            if ids is None:
                return None
            new = ids[0]
            self._ref[old] -= 1
            seq.table[j] = new
            return self.physical_index(seq, pos), (old, new)
        return self.physical_index(seq, pos), None

    # ------------------------------------------------------------ batch views
    def slot_mapping(self, seqs, positions) -> np.ndarray:
        """int64 slots of one batch: slot_i = table_i[pos_i // B] * B + pos_i % B."""
        B = self.block_size
        pos = np.asarray(positions, dtype=np.int64)
        phys = np.array([s.table[p // B] for s, p in zip(seqs, pos.tolist())], dtype=np.int64)
        return phys * B + pos % B

    @staticmethod
    def block_tables(seqs, max_blocks: int | None = None, pad: int = 0) -> np.ndarray:
        """int32 [len(seqs), max_blocks] table rows, padded with ``pad``."""
        width = max(len(s.table) for s in seqs) if max_blocks is None else max_blocks
        out = np.full((len(seqs), width), pad, dtype=np.int32)
        for i, s in enumerate(seqs):
            if len(s.table) > width:
                raise ValueError("table longer than max_blocks")
            out[i, :len(s.table)] = s.table
        return out

    def check(self, seqs) -> None:
        """Invariants: each refcount equals the number of tables holding the block; a block
        is on the free stack exactly when its refcount is zero; the stack has no repeats."""
        counts = np.zeros(self.num_blocks, dtype=np.int64)
        for s in seqs:
            np.add.at(counts, np.asarray(s.table, dtype=np.int64), 1)
        if not np.array_equal(counts, self._ref):
            raise AssertionError("refcounts do not match the tables")
        free = np.zeros(self.num_blocks, dtype=bool)
        free[self._free] = True
        if len(set(self._free)) != len(self._free):
            raise AssertionError("free stack holds a block twice")
        if not np.array_equal(free, self._ref == 0):
            raise AssertionError("free stack and zero refcounts disagree")


class DecodeBatch:
    """The running batch of a decode loop held as arrays, so that a step's host work -- every
    sequence gains its newest token, takes a block when that token starts one, copies a shared
    block before writing into it, and the slot mapping of the new tokens -- is a few array
    operations rather than a loop over sequences (page "nano-vLLM . Ch04 . PagedAttention",
    section 4: the slot mapping is built on the CPU once per batch; section 9: no Python per
    token while the GPU runs the step).

    ``tables`` [S, capacity] int32 rows (zeros past each row's ``nblocks``), ``lengths`` [S].
    ``step()`` gives exactly what BlockManager.append_token then prepare_write would give,
    sequence by sequence: a sequence whose new token starts a block takes the top of the free
    stack, in sequence order; a write into a block shared with another sequence (after a fork)
    takes the manager's per-sequence copy-on-write rules for that step.
    """

    def __init__(self, bm: BlockManager, seqs, capacity: int = 0):
        self.bm = bm
        self.lengths = np.array([s.length for s in seqs], dtype=np.int64)
        self.nblocks = np.array([len(s.table) for s in seqs], dtype=np.int64)
        width = max(int(self.nblocks.max(initial=0)) + 1, capacity)
        self.tables = np.zeros((len(seqs), width), dtype=np.int32)
        for i, s in enumerate(seqs):
            self.tables[i, :len(s.table)] = s.table
        self._rows = np.arange(len(seqs))

    def _ensure(self, cols: int) -> None:
        if cols > self.tables.shape[1]:
            grown = np.zeros((self.tables.shape[0], max(cols, 2 * self.tables.shape[1])), dtype=np.int32)
            grown[:, :self.tables.shape[1]] = self.tables
            self.tables = grown

    def block_tables(self) -> np.ndarray:
        """int32 [S, max blocks] view of the tables (the kernels' block_tables)."""
        return self.tables[:, :max(1, int(self.nblocks.max(initial=1)))]

    def context_lens(self) -> np.ndarray:
        return self.lengths.astype(np.int32)

    def sequences(self) -> list:
        return [Sequence(self.tables[i, :n].tolist(), int(l))
                for i, (n, l) in enumerate(zip(self.nblocks.tolist(), self.lengths.tolist()))]

    def step(self):
        """One decode step.  Returns ``(slot_mapping, copy_pairs)`` (int64 [S] and [P, 2]), or
        None -- changing nothing -- when the pool cannot supply the step's blocks."""
        bm, B = self.bm, self.bm.block_size
        pos = self.lengths                      # the new tokens' positions
        col = pos // B
        fresh = col >= self.nblocks             # the token starts a block the table lacks
        keep = np.nonzero(~fresh)[0]
        targets = self.tables[keep, col[keep]]
        if (bm._ref[targets] > 1).any():
            out = self._step_each(pos, col, fresh)
        else:
            idx = np.nonzero(fresh)[0]
            if len(idx) > bm.num_free():
                return None
            if len(idx):
                ids = bm.allocate(len(idx))     # the stack's top len(idx), bottom to top:
                self._ensure(int(col[idx].max()) + 1)
                self.tables[idx, col[idx]] = ids[::-1]   # one at a time, the top goes first
                self.nblocks[idx] += 1
            slots = self.tables[self._rows, col].astype(np.int64) * B + pos % B
            out = slots, np.zeros((0, 2), dtype=np.int64)
        if out is not None:
            self.lengths += 1
        return out

    def _step_each(self, pos, col, fresh):
        """The step sequence by sequence, with copy-on-write (BlockManager.prepare_write's
        rules: copy, drop the old block's count, write the copy; the last holder of a block
        writes in place).  A dry run first counts the blocks it takes."""
        bm, B = self.bm, self.bm.block_size
        takes, ref = int(fresh.sum()), {}
        for i in np.nonzero(~fresh)[0].tolist():
            b = int(self.tables[i, col[i]])
            r = ref.get(b, int(bm._ref[b]))
            if r > 1:
                takes += 1
                ref[b] = r - 1
        if takes > bm.num_free():
            return None
        self._ensure(int(col.max()) + 1)
        slots = np.empty(len(pos), dtype=np.int64)
        pairs = []
        for i in range(len(pos)):
            c = int(col[i])
            if fresh[i]:
                self.tables[i, c] = bm.allocate(1)[0]
                self.nblocks[i] += 1
            else:
                old = int(self.tables[i, c])
                if bm._ref[old] > 1:
                    new = bm.allocate(1)[0]
                    bm._ref[old] -= 1
                    self.tables[i, c] = new
                    pairs.append((old, new))
            slots[i] = int(self.tables[i, c]) * B + int(pos[i]) % B
        return slots, np.asarray(pairs, dtype=np.int64).reshape(-1, 2)


class PrefixCache:
    """Reuse of full prompt blocks across requests (page "PagedAttention", PidokuInfra topic
    10, section 5 "The relationship to prefix caching": hash the token ids of each block,
    keep a hash -> block id map, and point a new sequence's leading blocks that hash to
    existing blocks at them, raising their refcounts, instead of computing them again).

    Reading: a block's hash covers its own token ids *and* the hash of the block before it,
    so that "the first N blocks hash to existing blocks" means "the first N * B tokens are
    those of an earlier prompt" -- K/V of a token depend on every token before it, so a block
    with the same ids after a different prefix holds different K/V.  Only full prompt blocks
    are entered; a partly filled last block stays private, so a sequence's own writes never
    land in a shared block.  Entries leave the map when their block returns to the free
    stack.
    """

    def __init__(self, bm: BlockManager):
        self.bm = bm
        self._block_of: dict[bytes, int] = {}
        self._key_of: dict[int, bytes] = {}

    @staticmethod
    def block_keys(token_ids, block_size: int) -> list:
        """Chained SHA-256 digests of the full blocks of ``token_ids``."""
        import hashlib
        ids = np.asarray(token_ids, dtype=np.int64)
        keys, prev = [], b""
        for j in range(len(ids) // block_size):
            prev = hashlib.sha256(prev + ids[j * block_size:(j + 1) * block_size].tobytes()).digest()
            keys.append(prev)
        return keys

    def cached_blocks(self) -> int:
        return len(self._block_of)

    def new_sequence(self, token_ids):
        """A sequence for a prompt, reusing its leading cached blocks.

        Returns ``(sequence, hit_blocks)``, or None (changing nothing) if the uncached part
        cannot be allocated."""
        bm = self.bm
        keys = self.block_keys(token_ids, bm.block_size)
        hits = []
        for k in keys:
            b = self._block_of.get(k)
            if b is None:
                break
            hits.append(b)
        fresh = bm.allocate(bm.blocks_needed(len(token_ids)) - len(hits))
        if fresh is None:
            return None
        table = bm.fork_table(hits) + fresh
        for j in range(len(hits), len(keys)):   # the new full blocks become reusable
            self._block_of[keys[j]] = table[j]
            self._key_of[table[j]] = keys[j]
        return Sequence(table, len(token_ids)), len(hits)

    def release(self, seq: Sequence) -> None:
        table = list(seq.table)
        self.bm.release(seq)
        for b in table:
            if self.bm.refcount(b) == 0 and b in self._key_of:
                del self._block_of[self._key_of.pop(b)]
