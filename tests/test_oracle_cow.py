"""Pins for the oracle's copy-on-write: fork, the append rule and the block
copy.

  * tests/golden/cow.json: the nxmr.cn article's section 4.2 rule applied by
    hand to a FIFO pool (every case of the rule: write in place, copy a
    shared partial block, fresh block after a full one with no copy, freeing
    a branch);
  * a simulation over random add / fork / append / free sequences on a real
    pool, with every copy made by the oracle's copy_blocks and every token
    stored by its scatter: after every step each live sequence reads back
    exactly its own token history through its table (branch integrity: no
    branch ever overwrote another's data), reference counts equal the number
    of tables holding each block, the free list holds exactly the
    unreferenced blocks, a full block is never written or copied, and each
    append copies at most one block and changes no block but its destination
    (the paper-notes page: only the modified block is copied, as with fork());
  * planted mistakes in the append rule, and in the block copy (direction
    swapped, the whole pool overwritten, the copy left out, one head or one
    slot row only, the destination off by one), fail the simulation;
  * the block copy against a per-element loop.
"""
import numpy as np
import pytest

from oracle import allocator as A
from oracle.scatter import copy_blocks, scatter


def test_cow_timeline(golden):
    g = golden("cow.json")
    a = A.BlockAllocator(g["num_blocks"], g["block_size"])
    for st in g["steps"]:
        if st["op"] == "add":
            a.add(st["rid"], st["n"])
        elif st["op"] == "fork":
            a.fork(st["rid"], st["child"])
        elif st["op"] == "append":
            slot, cp = a.append_slot(st["rid"])
            assert slot == st["slot"], st
            assert (list(cp) if cp else None) == st["copy"], st
        else:
            a.release(st["rid"])
        assert a.tables == st["tables"], st
        assert a.free_list() == st["free"], st
    assert a.ref == g["final_refs"]
    assert a.lengths == g["final_lengths"]


def test_append_is_atomic_when_the_pool_is_empty():
    a = A.BlockAllocator(2, 4)
    a.add("p", 3)
    a.fork("p", "q")
    a.add("r", 1)                      # takes the last free block
    before = (a.free_list(), {k: v[:] for k, v in a.tables.items()}, dict(a.lengths),
              list(a.ref))
    with pytest.raises(MemoryError):
        a.append_slot("q")             # would need a fresh block for the copy
    assert before == (a.free_list(), {k: v[:] for k, v in a.tables.items()},
                      dict(a.lengths), list(a.ref))
    with pytest.raises(KeyError):
        a.fork("p", "q")


HKV, DIM = 2, 3     # the simulation's pool geometry (block size varies)


def _token_rows(tokens):
    """K/V content of each token: [len, HKV, DIM] int32, distinct for every
    (token, head, dim), so a byte that lands in the wrong place is seen."""
    t = np.asarray(tokens, np.int32)[:, None, None]
    return t * 16 + np.arange(HKV, dtype=np.int32)[None, :, None] * 4 + \
        np.arange(DIM, dtype=np.int32)[None, None, :]


class _Sim:
    """Branches of sequences over a real [N, HKV, B, DIM] pool. The oracle
    allocator decides blocks, slots and copies; every copy goes through the
    block-copy function under test and every token is stored with the
    oracle's scatter. Reading a sequence back walks its table position by
    position."""

    def __init__(self, alloc, copy_fn=copy_blocks):
        self.a = alloc
        self.B = alloc.block_size
        self.copy_fn = copy_fn
        self.pool = np.full((alloc.num_blocks, HKV, self.B, DIM), -1, np.int32)
        self.hist = {}
        self.next_tok = 1

    def _store(self, slots, tokens):
        self.pool = scatter(self.pool, _token_rows(tokens), slots)

    def add(self, rid, n):
        self.a.add(rid, n)
        toks = list(range(self.next_tok, self.next_tok + n))
        self.next_tok += n
        self._store([self.a.slot(rid, p) for p in range(n)], toks)
        self.hist[rid] = toks

    def fork(self, parent, child):
        self.a.fork(parent, child)
        self.hist[child] = list(self.hist[parent])

    def append(self, rid):
        slot, cp = self.a.append_slot(rid)
        copies = 0
        if cp is not None:
            src, dst = cp
            # only a partly filled last block is copied: the new token does
            # not start the fresh block
            assert slot // self.B == dst and slot % self.B != 0
            before = self.pool
            self.pool = self.copy_fn(before, [cp])
            # the paper-notes page: only the one modified block is copied;
            # every other block keeps its bytes
            changed = np.flatnonzero((self.pool != before).reshape(len(before), -1).any(1))
            assert set(changed.tolist()) <= {dst}, f"copy {cp} changed blocks {changed}"
            copies = 1
        # the block written to is referenced by this sequence alone
        assert self.a.ref[slot // self.B] == 1, "write into a shared block"
        tok = self.next_tok
        self.next_tok += 1
        self._store([slot], [tok])
        self.hist[rid].append(tok)
        return copies

    def free(self, rid):
        self.a.release(rid)
        del self.hist[rid]

    def read(self, rid):
        """The sequence's K/V rows, gathered position by position."""
        rows = []
        for p in range(self.a.lengths[rid]):
            blk, off = divmod(self.a.slot(rid, p), self.B)
            rows.append(self.pool[blk, :, off, :])
        return np.array(rows, np.int32).reshape(-1, HKV, DIM)

    def check(self):
        a = self.a
        for rid, h in self.hist.items():
            assert a.lengths[rid] == len(h)
            got = self.read(rid)
            assert np.array_equal(got, _token_rows(h)), f"sequence {rid} reads other data"
        held = [0] * a.num_blocks
        for t in a.tables.values():
            for b in t:
                held[b] += 1
        assert held == a.ref
        assert sorted(a.free_list()) == [b for b in range(a.num_blocks) if a.ref[b] == 0]
        assert len(set(a.free_list())) == len(a.free_list())


def _random_run(seed, alloc_cls=A.BlockAllocator, copy_fn=copy_blocks):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 4, 8]))
    sim = _Sim(alloc_cls(64, B, rng.permutation(64).tolist()), copy_fn)
    names = 0
    for _ in range(200):
        live = list(sim.hist)
        op = rng.choice(["add", "fork", "append", "append", "append", "free"])
        try:
            if op == "add" or not live:
                sim.add(f"r{names}", int(rng.integers(1, 3 * B + 2)))
                names += 1
            elif op == "fork":
                sim.fork(live[int(rng.integers(len(live)))], f"r{names}")
                names += 1
            elif op == "append":
                assert sim.append(live[int(rng.integers(len(live)))]) <= 1
            else:
                sim.free(live[int(rng.integers(len(live)))])
        except MemoryError:
            pass
        sim.check()


@pytest.mark.parametrize("seed", range(25))
def test_cow_simulation_keeps_every_branch_intact(seed):
    _random_run(seed)


# -- planted mistakes in the append rule ----------------------------------------

class _InPlaceWhenShared(A.BlockAllocator):
    def append_slot(self, rid):
        seq = self._seqs[rid]
        n = seq.length
        if n % self.block_size:
            seq.length = n + 1
            return seq.blocks[-1] * self.block_size + n % self.block_size, None
        return super().append_slot(rid)


class _CopyWithoutRelease(A.BlockAllocator):
    def _ref_down(self, block):
        import inspect
        if inspect.stack()[1].function == "append_slot":
            return
        super()._ref_down(block)


class _NoCopy(A.BlockAllocator):
    def append_slot(self, rid):
        slot, cp = super().append_slot(rid)
        return slot, None


@pytest.mark.parametrize("cls", [_InPlaceWhenShared, _CopyWithoutRelease, _NoCopy])
def test_planted_cow_mistakes_fail_the_simulation(cls):
    failures = 0
    for seed in range(10):
        try:
            _random_run(seed, cls)
        except AssertionError:
            failures += 1
    assert failures >= 5


# -- planted mistakes in the block copy -------------------------------------------
# Each is the oracle's copy_blocks with one mistake; the branch-integrity
# simulation above must catch every one of them.

def _copy_reversed(pool, pairs):           # direction swapped: src <- dst
    out = pool.copy()
    for s, d in pairs:
        out[int(s)] = pool[int(d)]
    return out


def _copy_everywhere(pool, pairs):         # src spread over the whole pool
    out = pool.copy()
    for s, _ in pairs:
        out[:] = pool[int(s)]
    return out


def _copy_nothing(pool, pairs):            # the copy left out
    return pool.copy()


def _copy_first_head(pool, pairs):         # one KV head only
    out = pool.copy()
    for s, d in pairs:
        out[int(d), 0] = pool[int(s), 0]
    return out


def _copy_first_slot(pool, pairs):         # one slot row only
    out = pool.copy()
    for s, d in pairs:
        out[int(d), :, 0] = pool[int(s), :, 0]
    return out


def _copy_next_block(pool, pairs):         # destination off by one
    out = pool.copy()
    for s, d in pairs:
        out[(int(d) + 1) % len(pool)] = pool[int(s)]
    return out


@pytest.mark.parametrize("fn", [_copy_reversed, _copy_everywhere, _copy_nothing,
                                _copy_first_head, _copy_first_slot, _copy_next_block])
def test_planted_copy_mistakes_fail_the_simulation(fn):
    failures = 0
    for seed in range(10):
        try:
            _random_run(seed, copy_fn=fn)
        except AssertionError:
            failures += 1
    assert failures >= 5, fn.__name__


def test_copy_blocks_definition():
    rng = np.random.default_rng(2)
    pool = rng.integers(0, 1 << 16, size=(9, 3, 4, 5), dtype=np.uint16)
    pairs = [(1, 7), (1, 8), (4, 2)]
    got = copy_blocks(pool, pairs)
    want = pool.copy()
    for s, d in pairs:
        for h in range(3):
            for o in range(4):
                for e in range(5):
                    want[d, h, o, e] = pool[s, h, o, e]
    assert np.array_equal(got, want)
    assert np.array_equal(copy_blocks(pool, pairs[::-1]), got)   # order does not matter
    assert np.array_equal(copy_blocks(pool, []), pool)
    with pytest.raises(AssertionError):
        copy_blocks(pool, [(1, 7), (2, 7)])
    with pytest.raises(AssertionError):
        copy_blocks(pool, [(1, 7), (7, 3)])


def test_cow_workload_is_what_the_allocator_decides():
    """The parallel-sampling workload's copies, slots and tables are exactly
    what the oracle allocator's fork + append rule produces."""
    import workloads as W
    b = W.cow_fork_bf16(num_prompts=40, lo=1, hi=300, num_layers=1)
    a = A.BlockAllocator(b.num_blocks, b.block_size, b.free_order.tolist())
    for p, L in enumerate(b.prompt_lens):
        a.add(("p", p), int(L))
        for j in range(1, b.branches):
            a.fork(("p", p), ("b", p, j))
    pairs, slots = [], []
    for p in range(len(b.prompt_lens)):
        for j in list(range(1, b.branches)) + [0]:
            slot, cp = a.append_slot(("b", p, j) if j else ("p", p))
            slots.append(slot)
            if cp:
                pairs.append(cp)
    assert pairs == [tuple(x) for x in b.copy_pairs.tolist()]
    assert slots == b.slots.tolist()
    for s, rid in enumerate(b.rids):
        t = a.tables[rid]
        assert t == b.block_table[s, :len(t)].tolist()
        assert (b.block_table[s, len(t):] == -1).all()
