"""Pins for the oracle's swap out / swap in (preemption by swapping).

What fixes the expected values (none is the oracle's own output):
  * a hand case: two layers of a four-block pool whose every element says
    where it lives (layer, K or V, block, slot), and the host buffer written
    out by hand from the layout reading [layer][K or V][i][Hkv][B][D];
  * the nxmr.cn article, section 6.2, as a property: a preempted request's
    blocks go to host memory, its blocks are freed and reused by another
    request that overwrites them, the request comes back into newly
    allocated blocks and its table is rewritten; read through the new table
    (the oracle's C gather, which shares nothing with the swap code) every
    layer's K and V equal what it held before, and the other requests' data
    is untouched;
  * planted mistakes in copies of the two functions (K and V exchanged,
    layers exchanged, block order reversed, the wrong destination) fail one
    of the above.
"""
import numpy as np
import pytest

import oracle
from oracle import allocator as A
from oracle.scatter import scatter, swap_in, swap_out


def _labelled_pools():
    """Layer l's K pool holds 1000*l + 10*block + slot, its V pool the same
    plus 500: Hkv = 1, B = 2, D = 1, four blocks."""
    ks, vs = [], []
    for l in range(2):
        k = np.zeros((4, 1, 2, 1), np.int32)
        for b in range(4):
            for o in range(2):
                k[b, 0, o, 0] = 1000 * l + 10 * b + o
        ks.append(k)
        vs.append(k + 500)
    return ks, vs


def test_swap_out_hand_case():
    ks, vs = _labelled_pools()
    host = swap_out(ks, vs, [3, 0])
    # [layer][K=0 / V=1][i][Hkv][slot][D], blocks 3 then 0
    want = [[[[[[30], [31]]], [[[0], [1]]]],
             [[[[530], [531]]], [[[500], [501]]]]],
            [[[[[1030], [1031]]], [[[1000], [1001]]]],
             [[[[1530], [1531]]], [[[1500], [1501]]]]]]
    assert host.tolist() == want
    assert swap_out(ks, vs, []).shape == (2, 2, 0, 1, 2, 1)
    with pytest.raises(AssertionError):
        swap_out(ks, vs, [4])


def test_swap_in_hand_case():
    ks, vs = _labelled_pools()
    host = swap_out(ks, vs, [3, 0])
    # back into blocks 1 and 2: block 1 gets old block 3, block 2 old block 0
    k2, v2 = swap_in(ks, vs, host, [1, 2])
    assert [k2[0][b, 0, :, 0].tolist() for b in range(4)] == [[0, 1], [30, 31], [0, 1], [30, 31]]
    assert [v2[1][b, 0, :, 0].tolist() for b in range(4)] == \
        [[1500, 1501], [1530, 1531], [1500, 1501], [1530, 1531]]
    # the inputs are left as they were
    assert ks[0][1, 0, 0, 0] == 10
    with pytest.raises(AssertionError):
        swap_in(ks, vs, host, [1, 1])


def _preempt_and_resume(seed, out_fn=swap_out, in_fn=swap_in):
    """Three requests on a tight pool; request 1 is swapped out, its blocks
    reused by a newcomer that overwrites them, then swapped back into fresh
    blocks. Checks every layer of every request through the C gather."""
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 4]))
    hkv, d, layers = int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.integers(1, 4))
    lens = [int(x) for x in rng.integers(1, 4 * B + 1, size=3)]
    need = sum(A.blocks_needed(n, B) for n in lens)
    n_blocks = need + 1
    a = A.BlockAllocator(n_blocks, B, rng.permutation(n_blocks).tolist())
    ks = [rng.standard_normal((n_blocks, hkv, B, d)).astype(np.float32) for _ in range(layers)]
    vs = [rng.standard_normal((n_blocks, hkv, B, d)).astype(np.float32) for _ in range(layers)]
    for r, n in enumerate(lens):
        a.add(r, n)

    def read(rid, length):
        table = np.array(a.tables[rid], np.int32)
        return [oracle.gather(ks[l], vs[l], table, length, "f32") for l in range(layers)]

    before = {r: read(r, lens[r]) for r in range(3)}
    # preempt request 1: its blocks to the host, then freed
    host = out_fn(ks, vs, a.tables[1])
    a.release(1)
    # a newcomer takes the freed blocks (the pool has one spare) and writes them
    n_new = (A.blocks_needed(lens[1], B) + 1) * B
    a.add("new", n_new)
    slots = [a.slot("new", p) for p in range(n_new)]
    rows = lambda: rng.standard_normal((n_new, hkv, d)).astype(np.float32)  # noqa: E731
    for l in range(layers):
        ks[l] = scatter(ks[l], rows(), slots)
        vs[l] = scatter(vs[l], rows(), slots)
    newcomer = read("new", n_new)
    # the newcomer finishes; request 1 resumes in newly allocated blocks
    a.release("new")
    a.add(1, lens[1])
    ks, vs = in_fn(ks, vs, host, a.tables[1])
    for r in range(3):
        got = read(r, lens[r])
        for l in range(layers):
            assert np.array_equal(got[l][0], before[r][l][0]), (r, l, "K")
            assert np.array_equal(got[l][1], before[r][l][1]), (r, l, "V")
    return newcomer


@pytest.mark.parametrize("seed", range(20))
def test_swap_round_trip_restores_the_request(seed):
    _preempt_and_resume(seed)


def _out_kv_exchanged(k_pools, v_pools, ids):
    return swap_out(v_pools, k_pools, ids)


def _out_layers_exchanged(k_pools, v_pools, ids):
    host = swap_out(k_pools, v_pools, ids)
    return host[::-1].copy()


def _out_reversed(k_pools, v_pools, ids):
    host = swap_out(k_pools, v_pools, ids)
    return host[:, :, ::-1].copy()


def _in_next_block(k_pools, v_pools, host, ids):
    n = len(k_pools[0])
    return swap_in(k_pools, v_pools, host, [(int(b) + 1) % n for b in ids])


@pytest.mark.parametrize("out_fn,in_fn", [(_out_kv_exchanged, swap_in),
                                          (_out_layers_exchanged, swap_in),
                                          (_out_reversed, swap_in),
                                          (swap_out, _in_next_block)])
def test_planted_swap_mistakes_fail(out_fn, in_fn):
    failures = 0
    for seed in range(20):
        try:
            _preempt_and_resume(seed, out_fn, in_fn)
        except AssertionError:
            failures += 1
    # a single-layer or single-block draw can hide the layer or order mistake
    assert failures >= 8, failures
    ks, vs = _labelled_pools()
    hand = swap_out(ks, vs, [3, 0])
    try:
        host = out_fn(ks, vs, [3, 0])
        got_in = in_fn(ks, vs, hand, [1, 2])[0][0][1:3, 0, :, 0].tolist()
    except AssertionError:
        return
    assert host.tolist() != hand.tolist() or got_in != [[30, 31], [0, 1]]
