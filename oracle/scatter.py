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
