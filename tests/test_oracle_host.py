"""Pins for the oracle's host side: translation, allocator, counting, scatter.

Every expected value here is printed on the pages (tests/golden/*.json, each
with its citation) or follows from a definition checked by brute force.
"""
import os

import numpy as np
import pytest

from oracle import allocator as A
from oracle.scatter import scatter
import workloads as W


def test_translation_pins(golden):
    g = golden("translation.json")
    for case in g["cases"]:
        b = case["block_size"]
        for p, slot, lb, off in zip(case["positions"], case["slots"], case["logical_blocks"],
                                    case["offsets"]):
            assert A.translate(case["table"], p, b) == slot
            assert divmod(p, b) == (lb, off)
        assert A.slot_mapping([case["table"]] * len(case["positions"]), case["positions"],
                              b) == case["slots"]


def test_slot_mapping_negative_position_is_no_write():
    assert A.slot_mapping([[7, 3, 11], [1]], [-1, 2], 4) == [-1, 6]


def test_allocator_timeline(golden):
    g = golden("allocator_timeline.json")
    a = A.BlockAllocator(g["num_blocks"], g["block_size"])
    for st in g["steps"]:
        if st["op"] == "add":
            a.add(st["rid"], st["n"])
        elif st["op"] == "grow":
            a.extend(st["rid"], st["n"])
        else:
            a.release(st["rid"])
        assert a.tables == st["tables"], st
        assert a.free_list() == st["free"], st
    for c in g["slot_checks"]:
        assert a.slot(c["rid"], c["position"]) == c["slot"]
    before = (a.free_list(), {k: v[:] for k, v in a.tables.items()}, dict(a.lengths),
              list(a.ref))
    with pytest.raises(MemoryError):
        a.extend(g["failing_grow"]["rid"], g["failing_grow"]["n"])
    after = (a.free_list(), {k: v[:] for k, v in a.tables.items()}, dict(a.lengths),
             list(a.ref))
    assert before == after


def test_allocator_error_paths():
    a = A.BlockAllocator(4, 4)
    a.add("x", 5)
    with pytest.raises(KeyError):
        a.add("x", 1)
    with pytest.raises(IndexError):
        a.slot("x", 5)
    with pytest.raises(IndexError):
        a.slot("x", -1)
    with pytest.raises(MemoryError):
        a.add("y", 13)          # needs 4 blocks, 2 free
    assert a.free_list() == [2, 3] and "y" not in a.tables
    with pytest.raises(KeyError):
        a.extend("nope", 1)


def test_refcount_sharing(golden):
    g = golden("refcount.json")
    bl = g["blocks"]
    a = A.BlockAllocator(g["num_blocks"], g["block_size"])
    a.add("A", 3 * g["block_size"])
    assert a.tables["A"] == [bl["b0"], bl["b1"], bl["b2"]]
    a.add("B", 3 * g["block_size"], shared_prefix=[bl["b0"], bl["b1"]])
    assert a.tables["B"] == [bl["b0"], bl["b1"], bl["b3"]]
    assert a.ref == g["after_add"]["ref"]
    a.release("A")
    assert a.ref == g["after_free_A"]["ref"]
    assert a.free_list() == [bl[n] for n in g["after_free_A"]["returned"]]
    a.release("B")
    assert a.ref == g["after_free_B"]["ref"]
    assert a.free_list() == [bl[n] for n in g["after_free_B"]["returned"]]


def test_acquire_of_free_block_leaves_free_list():
    a = A.BlockAllocator(4, 2)
    a.add("A", 2, shared_prefix=[2])      # block 2 was free: acquired by reference
    assert a.tables["A"] == [2] and a.ref[2] == 1 and 2 not in a.free_list()
    with pytest.raises(MemoryError):      # 3 free blocks, needs 1 shared + 4 fresh
        a.add("B", 10, shared_prefix=[2])
    assert a.ref[2] == 1 and a.free_list() == [0, 1, 3]


def test_block_counting(golden):
    g = golden("counting.json")
    b = g["block_size"]
    blocks = [A.blocks_needed(n, b) for n in g["lengths"]]
    assert blocks == g["blocks"]
    assert sum(blocks) > g["pool_blocks"]
    assert [A.tail_waste(n, b) for n in g["lengths"]] == g["waste"]
    assert len(g["lengths"]) * g["max_len_reservation"] == g["reserved_slots"]
    assert sum(g["lengths"]) == g["live_tokens"]
    bm = g["max_waste_block_size"]
    assert max(A.tail_waste(n, bm) for n in range(1, 200)) == g["max_waste"]
    with pytest.raises(MemoryError):      # 9 blocks do not fit in 8
        a = A.BlockAllocator(g["pool_blocks"], b)
        for i, n in enumerate(g["lengths"]):
            a.add(i, n)


def test_sharing_counts(golden):
    g = golden("sharing.json")
    st = A.sharing_stats(g["tables"], g["lengths"], g["block_size"])
    for k in ("unique_blocks", "allocated_slots", "live_positions", "waste_slots",
              "unshared_slots", "saved_slots"):
        assert st[k] == g[k], k
    assert st["utilisation"] == pytest.approx(13 / 16)


def test_scatter_definition():
    rng = np.random.default_rng(0)
    pool = rng.standard_normal((5, 2, 4, 3)).astype(np.float16)
    new = rng.standard_normal((3, 2, 3)).astype(np.float16)
    out = scatter(pool, new, [9, -1, 0])
    # slot 9 = block 2 offset 1; slot 0 = block 0 offset 0; token 1 skipped
    assert np.array_equal(out[2, :, 1, :].view(np.int16), new[0].view(np.int16))
    assert np.array_equal(out[0, :, 0, :].view(np.int16), new[2].view(np.int16))
    mask = np.ones(pool.shape[:1] + pool.shape[2:3], bool)
    mask[2, 1] = mask[0, 0] = False
    assert np.array_equal(out.transpose(0, 2, 1, 3)[mask].view(np.int16),
                          pool.transpose(0, 2, 1, 3)[mask].view(np.int16))
    with pytest.raises(AssertionError):
        scatter(pool, new, [3, 3, -1])
    with pytest.raises(AssertionError):
        scatter(pool, new, [20, -1, -1])


def test_scatter_then_translate_reads_back():
    """Writing position p's token through the allocator's slot, then reading
    the pool at table[p // B], p % B, returns it (slot and layout agree)."""
    rng = np.random.default_rng(1)
    a = A.BlockAllocator(6, 4, initial_free=[3, 0, 5, 1, 4, 2])
    a.add("s", 7)
    a.extend("s", 1)                     # position 7 now exists
    pool = np.zeros((6, 2, 4, 8), np.float32)
    new = rng.standard_normal((1, 2, 8)).astype(np.float32)
    out = scatter(pool, new, [a.slot("s", 7)])
    blk = a.tables["s"][7 // 4]
    assert np.array_equal(out[blk, :, 7 % 4], new[0])


def _alloc_tables(batch):
    """Drive the oracle allocator with the batch's lengths and free order."""
    a = A.BlockAllocator(batch.num_blocks, batch.block_size, initial_free=batch.free_order)
    lens = batch.live_lens() if batch.positions is not None else batch.context_lens
    shared = list(batch.shared_blocks)
    sharer_set = set(int(s) for s in batch.sharers)
    if shared:
        a.add("__prefix__", len(shared) * batch.block_size)   # takes the shared blocks first
        assert a.tables["__prefix__"] == shared
    for s, n in enumerate(lens):
        a.add(s, int(n), shared_prefix=shared if s in sharer_set else ())
    if shared:
        a.release("__prefix__")
    if batch.positions is not None:
        for s in range(batch.num_seqs):
            a.extend(s, 1)
    return a


@pytest.mark.parametrize("make", [
    lambda: W.mha_fp16(num_seqs=16, lo=20, hi=300),
    lambda: W.gqa_shared_bf16(num_seqs=40, median=300.0, prefix_blocks=4),
    lambda: W.long_split_bf16(num_seqs=3, lo=600, hi=3000),
    lambda: W.decode_step_bf16(num_seqs=50, lo=1, hi=100, num_layers=1),
])
def test_dealt_tables_match_allocator(make):
    batch = make()
    a = _alloc_tables(batch)
    for s in range(batch.num_seqs):
        n = A.blocks_needed(int(batch.context_lens[s]), batch.block_size)
        assert a.tables[s] == batch.block_table[s, :n].tolist()
        assert (batch.block_table[s, n:] == -1).all()
    if len(batch.sharers):
        for b in batch.shared_blocks:
            assert a.ref[int(b)] == len(batch.sharers)


def test_new_token_slots_take_fresh_block_on_boundary():
    """A cached length that is a multiple of B makes the new token start a
    fresh block (paper-notes page, block life-cycle table, step 3)."""
    batch = W.decode_step_bf16(num_seqs=64, lo=1, hi=64, num_layers=1)
    a = _alloc_tables(batch)
    slots = A.slot_mapping([a.tables[s] for s in range(batch.num_seqs)],
                           batch.positions.tolist(), batch.block_size)
    for s, (p, slot) in enumerate(zip(batch.positions, slots)):
        assert slot == a.slot(s, int(p))
        if p % batch.block_size == 0:
            assert slot % batch.block_size == 0
            assert a.tables[s][-1] == slot // batch.block_size


@pytest.mark.parametrize("make", ["tiny", "gqa_shared_bf16", "mha_fp16"])
def test_bench_block_utilisation_matches_oracle(make):
    """The bench line's block utilisation equals the oracle's sharing
    statistics on the same tables (the glossary page's example: 13 live
    positions in 16 slots)."""
    import bench
    b = W.CASES[make]()
    tables = [row[row >= 0].tolist() for row in b.block_table]
    want = A.sharing_stats(tables, b.context_lens.tolist(), b.block_size)
    assert bench.block_utilisation(b) == round(want["utilisation"], 4)
    if make == "tiny":
        assert (want["live_positions"], want["allocated_slots"]) == (13, 16)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for more, it exits with status 2 and
    says why, before touching a GPU."""
    import subprocess
    import sys
    from conftest import ROOT
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_traffic_lookup_follows_sources():
    """The bench line's traffic figure comes from the committed counter
    summary only while the kernel sources' hash matches it."""
    import json
    import bench
    from conftest import ROOT
    path = os.path.join(ROOT, "profiles", "decode_split_decode_step_bf16_traffic.json")
    rec = json.load(open(path))
    assert bench.traffic_for("decode_step_bf16") == (
        rec["hbm_bytes_per_launch"]
        if rec["kernel_source_sha256"] == bench.kernel_source_hash() else None)
    assert bench.traffic_for("no_such_workload") is None
