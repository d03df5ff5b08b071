"""New-token K/V write and whole-block copy in the paged pool: the oracle's
plain definitions.

TEST INFRASTRUCTURE ONLY (tests/, smoke check, CPU baseline leg of bench.py).

Source: "vLLM PagedAttention: from fragmentation to slot mapping", section 6
(the backend writes new K/V to physical slots; the slot mapping says which),
and section 3 (one slot holds one token's [num_kv_heads, head_dim] K and V
for a layer). Slot s lives in block s // B at offset s % B of a
[num_blocks, Hkv, B, D] pool. A negative slot means "no write".

Block copy (copy-on-write, nxmr.cn article, section 4.2: the old block's
KV data is copied into the fresh block): every byte of block dst, all KV
heads and all slots, becomes the byte of block src.

Swap out / in (preemption by swapping: the paper-notes page's preemption
table, "Swapping" row, moves a preempted request's KV blocks to CPU memory
and back; nxmr.cn article, section 6.2: on resumption the request gets
newly allocated blocks, its KV data is copied back into them and its table
is rewritten). The pages fix no host layout; the reading taken here is one
host buffer [layer][K or V][i][Hkv][B][D], i following the listed block
order.

Works on raw bytes (numpy views of any element type), so the comparison with
the GPU is bitwise.
"""
from __future__ import annotations

import numpy as np


def scatter(pool: np.ndarray, new: np.ndarray, slots) -> np.ndarray:
    """Return a copy of ``pool`` [N, Hkv, B, D] with new[i] [Hkv, D] stored at
    slot slots[i] for every slots[i] >= 0. Slots must be distinct (one writer
    per slot) and below N*B."""
    out = pool.copy()
    n_blocks, hkv, block_size, d = pool.shape
    assert new.shape[1:] == (hkv, d) and new.dtype == pool.dtype
    seen = set()
    for i, s in enumerate(int(x) for x in slots):
        if s < 0:
            continue
        assert s < n_blocks * block_size, f"slot {s} outside the pool"
        assert s not in seen, f"slot {s} written twice"
        seen.add(s)
        out[s // block_size, :, s % block_size, :] = new[i]
    return out


def copy_blocks(pool: np.ndarray, pairs) -> np.ndarray:
    """Return a copy of ``pool`` [N, Hkv, B, D] in which block dst holds the
    old contents of block src for every (src, dst) in ``pairs``. Destinations
    are distinct and no destination is another pair's source, so the result
    does not depend on the order of the pairs."""
    out = pool.copy()
    n_blocks = pool.shape[0]
    dsts = [int(d) for _, d in pairs]
    srcs = {int(s) for s, _ in pairs}
    assert len(set(dsts)) == len(dsts), "a block is copied into twice"
    assert not srcs & set(dsts), "a destination is also a source"
    for s, d in pairs:
        s, d = int(s), int(d)
        assert 0 <= s < n_blocks and 0 <= d < n_blocks
        out[d] = pool[s]
    return out


def swap_out(k_pools, v_pools, block_ids) -> np.ndarray:
    """Host buffer [L, 2, n, Hkv, B, D] for layers' pools k_pools[l] /
    v_pools[l] (each [N, Hkv, B, D]): entry [l, 0, i] holds block
    block_ids[i] of layer l's K pool, entry [l, 1, i] the same block of its
    V pool."""
    layers = len(k_pools)
    assert len(v_pools) == layers and layers > 0
    shape, dtype = k_pools[0].shape, k_pools[0].dtype
    ids = [int(b) for b in block_ids]
    for b in ids:
        assert 0 <= b < shape[0], f"block {b} outside the pool"
    host = np.empty((layers, 2, len(ids)) + tuple(shape[1:]), dtype)
    for l in range(layers):
        for pools, which in ((k_pools, 0), (v_pools, 1)):
            assert pools[l].shape == shape and pools[l].dtype == dtype
            for i, b in enumerate(ids):
                host[l, which, i] = pools[l][b]
    return host


def swap_in(k_pools, v_pools, host: np.ndarray, block_ids):
    """Copies of the layers' pools in which block block_ids[i] of layer l's
    K pool holds host[l, 0, i] and the same block of its V pool host[l, 1, i].
    The destinations are distinct (each receives one block)."""
    layers = len(k_pools)
    ids = [int(b) for b in block_ids]
    assert len(set(ids)) == len(ids), "a block is swapped into twice"
    assert host.shape[:3] == (layers, 2, len(ids))
    ks = [p.copy() for p in k_pools]
    vs = [p.copy() for p in v_pools]
    for l in range(layers):
        for pools, which in ((ks, 0), (vs, 1)):
            assert host.shape[3:] == pools[l].shape[1:] and host.dtype == pools[l].dtype
            for i, b in enumerate(ids):
                assert 0 <= b < len(pools[l]), f"block {b} outside the pool"
                pools[l][b] = host[l, which, i]
    return ks, vs
