"""Block allocator, slot translation and block counting: the oracle's host side.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the CPU
baseline leg of bench.py, never by the library.

Sources (page titles as printed at the head of each page):
  * "vLLM PagedAttention: from fragmentation to slot mapping"
      - section 2: n = ceil(S/B) blocks per request, tail waste w = nB - S.
      - section 3: logical block = p // B, offset = p % B,
        slot = table[p // B] * B + p % B.
      - section 4 (allocator timeline and the minimal allocator): a FIFO free
        list (take from the front, give back at the end), a capacity check
        that takes nothing when short (MemoryError), KeyError for a duplicate
        request, IndexError for a position outside [0, length).
      - section 5 (block life cycle and reference counts): acquiring a block
        at ref 0 removes it from the free queue; releasing to 0 appends it.
  * "vLLM source walkthrough: PagedAttention and continuous batching",
    section 1.6: freeing walks the table in order, only ref-0 blocks return.
  * Glossary page "PagedAttention", worked example: unique live positions,
    allocated slots and the slots saved by sharing a prefix block.
  * nxmr.cn article, section 5.2: block utilisation = live tokens /
    (allocated blocks * B).
  * nxmr.cn article, sections 4.1-4.3 (copy-on-write): branches of one
    sequence (beam search, parallel sampling) share its blocks by reference;
    a full block is immutable and safely shared; before a sequence writes
    into its last, partly filled block it checks the block's reference
    count: 1 -> write in place; > 1 -> take a fresh block, copy the old
    block's contents into it, point the table entry at it, drop one
    reference from the old block, then write. A full last block means a
    fresh block and no copy. The paper-notes page adds that only the one
    modified block is copied, never the whole cache, as with Unix fork().

The free list is a plain deque; the pages' O(1) intrusive list is only needed
for prefix-cache eviction, which this oracle does not model.
"""
from __future__ import annotations

from collections import deque


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """n = ceil(S / B) (fragmentation page, section 2)."""
    if num_tokens < 0 or block_size <= 0:
        raise ValueError((num_tokens, block_size))
    return -(-num_tokens // block_size)


def tail_waste(num_tokens: int, block_size: int) -> int:
    """w = n*B - S, 0 <= w < B for S > 0 (fragmentation page, section 2)."""
    return blocks_needed(num_tokens, block_size) * block_size - num_tokens


def translate(table, position: int, block_size: int) -> int:
    """slot = table[p // B] * B + p % B (fragmentation page, section 3)."""
    if position < 0:
        raise IndexError(position)
    logical, offset = divmod(position, block_size)
    return table[logical] * block_size + offset


class _Seq:
    """One request: the physical blocks of its logical blocks, in order, and
    how many tokens it holds."""

    __slots__ = ("blocks", "length")

    def __init__(self, blocks, length: int):
        self.blocks = blocks
        self.length = length


class BlockAllocator:
    """FIFO block allocator with per-block reference counts.

    Blocks are ints in [0, num_blocks). ``initial_free`` sets the order of the
    free queue (default: 0..N-1, as in the pages' timeline); a seeded
    permutation gives the shuffled pools of the larger workloads. Every
    operation either completes or raises before changing anything.
    """

    def __init__(self, num_blocks: int, block_size: int, initial_free=None):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError((num_blocks, block_size))
        queue = range(num_blocks) if initial_free is None else [int(b) for b in initial_free]
        if sorted(queue) != list(range(num_blocks)):
            raise ValueError("initial_free must be a permutation of range(num_blocks)")
        self.block_size = block_size
        self.num_blocks = num_blocks
        self.ref = [0] * num_blocks
        self._queue = deque(queue)     # unreferenced blocks; the head goes out first
        self._seqs: dict = {}

    # -- views ---------------------------------------------------------------
    @property
    def tables(self) -> dict:
        """Request id -> its block table (a copy)."""
        return {rid: list(q.blocks) for rid, q in self._seqs.items()}

    @property
    def lengths(self) -> dict:
        """Request id -> tokens held."""
        return {rid: q.length for rid, q in self._seqs.items()}

    def free_list(self) -> list:
        return list(self._queue)

    # -- block reference counting -------------------------------------------
    def _check_room(self, wanted: int) -> None:
        if wanted > len(self._queue):
            raise MemoryError(f"{wanted} block(s) wanted, {len(self._queue)} unreferenced")

    def _fresh(self, count: int) -> list:
        """``count`` blocks off the head of the queue, each now referenced
        once; nothing is taken when the queue is too short."""
        self._check_room(count)
        got = []
        while len(got) < count:
            blk = self._queue.popleft()
            assert self.ref[blk] == 0
            self.ref[blk] = 1
            got.append(blk)
        return got

    def _ref_up(self, blk: int) -> None:
        if self.ref[blk] == 0:           # leaves the queue wherever it waits
            self._queue.remove(blk)
        self.ref[blk] += 1

    def _ref_down(self, blk: int) -> None:
        assert self.ref[blk] > 0, f"refcount underflow on block {blk}"
        self.ref[blk] -= 1
        if self.ref[blk] == 0:           # back in line, at the tail
            self._queue.append(blk)

    # -- requests ------------------------------------------------------------
    def add(self, rid, num_tokens: int, shared_prefix=()) -> list:
        """Admit request ``rid`` with ``num_tokens`` tokens.

        ``shared_prefix`` lists physical blocks (already owned by others, or
        free) that become this request's first logical blocks by reference;
        the remaining blocks are taken fresh.
        """
        if rid in self._seqs:
            raise KeyError(rid)
        total = blocks_needed(num_tokens, self.block_size)
        prefix = [int(b) for b in shared_prefix]
        if len(prefix) > total:
            raise ValueError("shared prefix longer than the request")
        # a prefix block at ref 0 leaves the free queue as well
        self._check_room(total - len(prefix) + len({b for b in prefix if self.ref[b] == 0}))
        for blk in prefix:
            self._ref_up(blk)
        blocks = prefix + self._fresh(total - len(prefix))
        self._seqs[rid] = _Seq(blocks, num_tokens)
        return list(blocks)

    def extend(self, rid, new_tokens: int) -> list:
        """``new_tokens`` more tokens for ``rid``: the blocks the longer
        length covers beyond the current ones, ceil((L+k)/B) - ceil(L/B)."""
        seq = self._seqs[rid]
        target = seq.length + new_tokens
        have = blocks_needed(seq.length, self.block_size)
        added = self._fresh(blocks_needed(target, self.block_size) - have)
        seq.blocks.extend(added)
        seq.length = target
        return added

    def fork(self, parent, child) -> list:
        """``child`` starts as a copy of ``parent``: the same blocks, by
        reference (every block gains one reference), the same length."""
        if child in self._seqs:
            raise KeyError(child)
        src = self._seqs[parent]
        for blk in src.blocks:
            self._ref_up(blk)
        self._seqs[child] = _Seq(list(src.blocks), src.length)
        return list(src.blocks)

    def append_slot(self, rid):
        """Make room for one more token of ``rid`` (copy-on-write rule).

        Returns (slot, copy): the slot the new token goes to, and (src, dst)
        when the last block had to be copied first, else None.
        """
        seq = self._seqs[rid]
        B = self.block_size
        filled = seq.length % B
        if filled == 0:                  # no block yet, or the last one is full
            (blk,) = self._fresh(1)
            seq.blocks.append(blk)
            seq.length += 1
            return blk * B, None
        last = seq.blocks[-1]
        if self.ref[last] == 1:          # sole owner: write in place
            seq.length += 1
            return last * B + filled, None
        (blk,) = self._fresh(1)          # shared partial block: copy on write
        seq.blocks[-1] = blk
        self._ref_down(last)
        seq.length += 1
        return blk * B + filled, (last, blk)

    def release(self, rid) -> None:
        """Drop ``rid``; its blocks lose one reference each, in table order."""
        for blk in self._seqs.pop(rid).blocks:
            self._ref_down(blk)

    def slot(self, rid, position: int) -> int:
        """Slot of one of ``rid``'s existing positions."""
        seq = self._seqs[rid]
        if position < 0 or position >= seq.length:
            raise IndexError(f"position {position} outside [0, {seq.length})")
        return translate(seq.blocks, position, self.block_size)


def slot_mapping(tables, positions, block_size: int) -> list:
    """Slot of each sequence's token at ``positions[s]``; a negative position
    maps to -1 (no write)."""
    out = []
    for table, p in zip(tables, positions):
        out.append(-1 if p < 0 else translate(table, p, block_size))
    return out


def sharing_stats(tables, lengths, block_size: int) -> dict:
    """Counts of the glossary page's worked example, for any set of tables.

    live = distinct physical slots holding a live token of some sequence;
    allocated = distinct blocks in use * B; waste = allocated - live;
    unshared = sum of per-sequence block counts * B (no sharing).
    """
    live = set()
    used = set()
    for table, n in zip(tables, lengths):
        nb = blocks_needed(n, block_size)
        used.update(int(b) for b in table[:nb])
        for t in range(n):
            live.add(translate(table, t, block_size))
    allocated = len(used) * block_size
    unshared = sum(blocks_needed(n, block_size) for n in lengths) * block_size
    return {
        "unique_blocks": len(used),
        "allocated_slots": allocated,
        "live_positions": len(live),
        "waste_slots": allocated - len(live),
        "unshared_slots": unshared,
        "saved_slots": unshared - allocated,
        "utilisation": (len(live) / allocated) if allocated else 0.0,
    }
