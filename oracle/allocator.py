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


class BlockAllocator:
    """FIFO block allocator with per-block reference counts.

    Blocks are ints in [0, num_blocks). ``initial_free`` sets the order of the
    free list (default: 0..N-1, as in the pages' timeline); a seeded
    permutation gives the shuffled pools of the larger workloads.
    """

    def __init__(self, num_blocks: int, block_size: int, initial_free=None):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError((num_blocks, block_size))
        self.block_size = block_size
        self.num_blocks = num_blocks
        order = list(range(num_blocks)) if initial_free is None else list(initial_free)
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_free must be a permutation of range(num_blocks)")
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.tables: dict = {}
        self.lengths: dict = {}

    # -- internals ---------------------------------------------------------
    def _take(self, n: int) -> list:
        # Capacity is checked before anything moves: a short pool takes nothing.
        if n > len(self.free):
            raise MemoryError(f"need {n}, free {len(self.free)}")
        out = [self.free.popleft() for _ in range(n)]
        for b in out:
            assert self.ref[b] == 0
            self.ref[b] = 1
        return out

    def _acquire(self, block: int) -> None:
        if self.ref[block] == 0:
            self.free.remove(block)
        self.ref[block] += 1

    def _release(self, block: int) -> None:
        assert self.ref[block] > 0, f"refcount underflow on block {block}"
        self.ref[block] -= 1
        if self.ref[block] == 0:
            self.free.append(block)

    # -- public API --------------------------------------------------------
    def add(self, rid, num_tokens: int, shared_prefix=()) -> list:
        """Admit request ``rid`` with ``num_tokens`` tokens.

        ``shared_prefix`` lists physical blocks (already owned by others, or
        free) that become this request's first logical blocks by reference;
        the remaining blocks are taken fresh. Atomic: on MemoryError nothing
        changes.
        """
        if rid in self.tables:
            raise KeyError(rid)
        need = blocks_needed(num_tokens, self.block_size)
        shared = list(shared_prefix)
        if len(shared) > need:
            raise ValueError("shared prefix longer than the request")
        fresh_needed = need - len(shared)
        # blocks at ref 0 in the prefix leave the free list too
        revived = len({b for b in shared if self.ref[b] == 0})
        if fresh_needed + revived > len(self.free):
            raise MemoryError(f"need {fresh_needed + revived}, free {len(self.free)}")
        for b in shared:
            self._acquire(b)
        blocks = shared + self._take(fresh_needed)
        self.tables[rid] = blocks
        self.lengths[rid] = num_tokens
        return list(blocks)

    def grow(self, rid, new_tokens: int) -> list:
        """Extend ``rid`` by ``new_tokens``; take ceil((L+k)/B) - ceil(L/B) blocks."""
        old = self.lengths[rid]
        extra = blocks_needed(old + new_tokens, self.block_size) - blocks_needed(
            old, self.block_size)
        got = self._take(extra)
        self.tables[rid].extend(got)
        self.lengths[rid] = old + new_tokens
        return got

    def fork(self, parent, child) -> list:
        """``child`` starts as a copy of ``parent``: the same blocks, by
        reference (every block gains one reference), the same length."""
        if child in self.tables:
            raise KeyError(child)
        blocks = list(self.tables[parent])
        for b in blocks:
            self._acquire(b)
        self.tables[child] = blocks
        self.lengths[child] = self.lengths[parent]
        return list(blocks)

    def append_slot(self, rid):
        """Make room for one more token of ``rid`` (copy-on-write rule).

        Returns (slot, copy): the slot the new token goes to, and (src, dst)
        when the last block had to be copied first, else None. Atomic: on
        MemoryError nothing changes.
        """
        n = self.lengths[rid]
        table = self.tables[rid]
        used = n % self.block_size
        if used == 0:                      # no block, or the last one is full
            (fresh,) = self._take(1)
            table.append(fresh)
            self.lengths[rid] = n + 1
            return fresh * self.block_size, None
        last = table[-1]
        if self.ref[last] == 1:            # sole owner: write in place
            self.lengths[rid] = n + 1
            return last * self.block_size + used, None
        (fresh,) = self._take(1)           # shared partial block: copy on write
        table[-1] = fresh
        self._release(last)
        self.lengths[rid] = n + 1
        return fresh * self.block_size + used, (last, fresh)

    def free_request(self, rid) -> None:
        """Release every block of ``rid`` in table order."""
        for b in self.tables.pop(rid):
            self._release(b)
        del self.lengths[rid]

    def slot(self, rid, position: int) -> int:
        if not 0 <= position < self.lengths[rid]:
            raise IndexError(position)
        return translate(self.tables[rid], position, self.block_size)

    def free_list(self) -> list:
        return list(self.free)


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
