"""Seeded synthetic inputs for paged-KV decode: the only code shared by the
HIP path's callers (bench, tests) and the oracle's callers.

This module holds input construction only: random lengths, a shuffled free
list, block tables dealt from it, and N(0,1) K/V/q tensors. It computes no
attention, no slot mapping and no scatter. The one piece of block arithmetic
it needs is how many blocks a length occupies (ceil(len / B)), since a block
table cannot be built without it.

Shapes follow the pages:
  * pool [num_blocks, Hkv, B, D] (glossary page "PagedAttention", teaching
    layout), block table [num_seqs, max_blocks] int32 padded with -1
    (same page, and the source-walkthrough page, section 1.7);
  * the tiny case is the glossary page's worked example (its tables,
    lengths and shapes; seed 53; V prefix = 0.5 * K prefix), drawn as pools;
  * the larger cases use the geometry of the nxmr.cn article, section 1.1
    (32 layers x 32 heads x 128 dims, fp16), the default block of 16 from the
    paper-notes page, prefix sharing from the glossary and walkthrough pages,
    and long contexts split into partitions (walkthrough page, section 1.8).

Recipe (for every case): lengths from numpy PCG64 ``default_rng(seed)``; the
free list is a seeded permutation of range(num_blocks) drawn next; sequences
take blocks in index order from the front of the free list; the pool holds
ceil(1.1 * blocks in use) blocks. Tensor values are N(0,1) float32 draws from a
torch generator seeded per (case seed, layer, tensor), rounded once to the
storage type; slots no live token occupies are NaN ("poison"), so any read of
them shows up in the output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def _torch_dtype(name):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def _nblocks(n: int, b: int) -> int:
    return -(-int(n) // b)


@dataclass
class Batch:
    """One decode batch: tables and lengths on the host; tensors made per layer."""
    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    block_table: np.ndarray          # int32 [S, max_blocks], -1 padded
    context_lens: np.ndarray         # int32 [S]: positions attention reads
    free_order: np.ndarray           # the permuted free list the tables came from
    seed: int
    num_layers: int = 1
    positions: np.ndarray | None = None   # int32 [S]: new-token position, or None
    partition_size: int = 0          # split size the case asks for (0: unsplit)
    sharers: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    shared_blocks: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    page_example: bool = False       # tensors come from the glossary page's recipe
    query_lens: np.ndarray | None = None  # int32 [S]: query tokens per sequence (multi-token
                                          # queries at the last positions), or None (one each)
    # parallel sampling (copy-on-write): prompts, branches per prompt, the
    # sequences' ids, the (src, dst) block copies and the new tokens' slots
    prompt_lens: np.ndarray | None = None
    branches: int = 1
    rids: list | None = None
    copy_pairs: np.ndarray | None = None
    slots: np.ndarray | None = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def num_tokens(self) -> int:
        """Query rows: one per sequence, or the sum of query_lens."""
        if self.query_lens is None:
            return self.num_seqs
        return int(self.query_lens.sum())

    @property
    def query_start_loc(self) -> np.ndarray:
        """int32 [S + 1]: sequence s owns query rows [qsl[s], qsl[s+1])."""
        q = np.ones(self.num_seqs, np.int64) if self.query_lens is None else self.query_lens
        return np.concatenate([[0], np.cumsum(q)]).astype(np.int32)

    def live_lens(self) -> np.ndarray:
        """Positions holding data before this step's write (ctx - 1 when a
        new token is written at position ctx - 1, else ctx)."""
        if self.positions is None:
            return self.context_lens.copy()
        return self.positions.copy()

    def max_partitions(self, partition_size: int | None = None) -> int:
        p = self.partition_size if partition_size is None else partition_size
        if p <= 0:
            return 1
        return max(1, _nblocks(int(self.context_lens.max(initial=0)), p))


def deal_tables(lengths, block_size: int, free_order, shared_blocks=(), sharers=(),
                width: int | None = None):
    """Block tables dealt from the front of ``free_order``.

    ``shared_blocks`` (taken first) become the first logical blocks of every
    sequence in ``sharers``. Returns (table int32 [S, width], blocks used).
    """
    free = list(int(b) for b in free_order)
    pos = 0
    shared = list(shared_blocks)
    if shared:
        assert free[:len(shared)] == shared
        pos = len(shared)
    sharer_set = set(int(s) for s in sharers)
    rows = []
    for s, n in enumerate(lengths):
        nb = _nblocks(n, block_size)
        row = []
        if s in sharer_set:
            row = list(shared)
            assert nb >= len(shared)
        take = nb - len(row)
        row += free[pos:pos + take]
        assert len(row) == nb, "pool too small"
        pos += take
        rows.append(row)
    w = max((len(r) for r in rows), default=0) if width is None else width
    w = max(w, 1)
    table = np.full((len(rows), w), -1, dtype=np.int32)
    for s, r in enumerate(rows):
        table[s, :len(r)] = r
    return table, pos


# --------------------------------------------------------------------------
# cases
# --------------------------------------------------------------------------

def tiny_page_example() -> Batch:
    """The glossary page's worked example: lengths 10 and 7, B=4, Hq=4,
    Hkv=2, D=8, fp32, 7 physical blocks, tables [5,1,6] and [5,3,-1] sharing
    physical block 5 (the common 4-token prefix)."""
    table = np.array([[5, 1, 6], [5, 3, -1]], dtype=np.int32)
    return Batch(name="tiny", dtype="f32", num_heads=4, num_kv_heads=2, head_size=8,
                 block_size=4, num_blocks=7, block_table=table,
                 context_lens=np.array([10, 7], dtype=np.int32),
                 free_order=np.arange(7, dtype=np.int32), seed=53,
                 sharers=np.array([0, 1], dtype=np.int32),
                 shared_blocks=np.array([5], dtype=np.int32), page_example=True)


def _uniform_case(name, dtype, hq, hkv, d, b, num_seqs, lo, hi, seed, partition_size=0,
                  num_layers=1, new_token=False):
    rng = np.random.default_rng(seed)
    cached = rng.integers(lo, hi, size=num_seqs, endpoint=True).astype(np.int64)
    lens = cached + 1 if new_token else cached
    need = int(sum(_nblocks(n, b) for n in lens))
    n_blocks = max(1, math.ceil(1.1 * need))
    free_order = rng.permutation(n_blocks).astype(np.int32)
    if not new_token:
        table, _ = deal_tables(lens, b, free_order)
    else:
        # the cached lengths are dealt first; then, in sequence order, every
        # sequence whose new token starts a block takes the next free block
        width = max(_nblocks(n, b) for n in lens)
        table, pos = deal_tables(cached, b, free_order, width=width)
        for s in range(num_seqs):
            nb_old, nb_new = _nblocks(cached[s], b), _nblocks(lens[s], b)
            if nb_new > nb_old:
                table[s, nb_old] = free_order[pos]
                pos += 1
    return Batch(name=name, dtype=dtype, num_heads=hq, num_kv_heads=hkv, head_size=d,
                 block_size=b, num_blocks=n_blocks, block_table=table,
                 context_lens=lens.astype(np.int32), free_order=free_order, seed=seed,
                 num_layers=num_layers,
                 positions=cached.astype(np.int32) if new_token else None,
                 partition_size=partition_size)


def mha_fp16(num_seqs: int = 64, lo: int = 128, hi: int = 2048, seed: int = 1002,
             block_size: int = 16) -> Batch:
    """Single-layer MHA decode, fp16, Hq=Hkv=32, D=128, B=16, lengths U{lo..hi}."""
    return _uniform_case("mha_fp16", "f16", 32, 32, 128, block_size, num_seqs, lo, hi, seed)


def gqa_shared_bf16(num_seqs: int = 256, median: float = 1024.0, clip=(16, 8192),
                    sigma: float = 1.0, share_frac: float = 0.3, prefix_blocks: int = 32,
                    seed: int = 1003, block_size: int = 16) -> Batch:
    """Single-layer GQA decode with prefix sharing, bf16, Hq=32, Hkv=8, D=128,
    B=16; lengths clip(rint(median * exp(sigma * Z)), clip); round(share_frac *
    S) sequences whose length covers the prefix map their first
    ``prefix_blocks`` logical blocks to the same physical blocks. Another
    block size keeps the shared prefix at the same number of positions."""
    b = block_size
    prefix_blocks = max(1, prefix_blocks * 16 // b)
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(num_seqs)
    lens = np.clip(np.rint(median * np.exp(sigma * z)), clip[0], clip[1]).astype(np.int64)
    n_share = int(round(share_frac * num_seqs))
    eligible = np.flatnonzero(lens >= prefix_blocks * b)
    per_seq = [_nblocks(n, b) for n in lens]
    # unique need: the shared prefix counts once
    n_share = min(n_share, len(eligible))
    need = sum(per_seq) - max(0, n_share - 1) * prefix_blocks if n_share else sum(per_seq)
    n_blocks = max(1, math.ceil(1.1 * need))
    free_order = rng.permutation(n_blocks).astype(np.int32)
    sharers = np.sort(rng.permutation(eligible)[:n_share]).astype(np.int32)
    shared = free_order[:prefix_blocks].copy() if n_share else np.zeros(0, np.int32)
    table, _ = deal_tables(lens, b, free_order, shared, sharers)
    return Batch(name="gqa_shared_bf16", dtype="bf16", num_heads=32, num_kv_heads=8,
                 head_size=128, block_size=b, num_blocks=n_blocks, block_table=table,
                 context_lens=lens.astype(np.int32), free_order=free_order, seed=seed,
                 sharers=sharers, shared_blocks=shared.astype(np.int32))


def long_split_bf16(num_seqs: int = 8, lo: int = 32768, hi: int = 131072,
                    seed: int = 1004, partition_size: int = 512, block_size: int = 32) -> Batch:
    """Long-context split decode, bf16, Hq=64, Hkv=8, D=128, B=32, lengths
    U{lo..hi}, 512-token partitions."""
    return _uniform_case("long_split_bf16", "bf16", 64, 8, 128, block_size, num_seqs, lo, hi,
                         seed, partition_size=partition_size)


def decode_step_bf16(num_seqs: int = 512, lo: int = 64, hi: int = 4096,
                     num_layers: int = 32, seed: int = 1005, block_size: int = 16) -> Batch:
    """Full decode step, bf16, Hq=32, Hkv=8, D=128, B=16: cached lengths
    U{lo..hi}; each sequence grows by its new token (taking a fresh block when
    its cached length is a multiple of 16), ``num_layers`` layers with their
    own pools; tables and positions are shared by all layers."""
    return _uniform_case("decode_step_bf16", "bf16", 32, 8, 128, block_size, num_seqs, lo, hi,
                         seed, num_layers=num_layers, new_token=True)


def _varlen_case(name, dtype, hq, hkv, d, b, hist, qlens, seed, free_order=None,
                 rng=None):
    """Sequences with ``hist`` cached positions and ``qlens`` new query
    tokens each, whose K/V are already in the pool: ctx = hist + q. Tables
    dealt from a shuffled free list over ceil(1.1 * need) blocks."""
    hist = np.asarray(hist, np.int64)
    qlens = np.asarray(qlens, np.int64)
    lens = hist + qlens
    need = int(sum(_nblocks(n, b) for n in lens))
    n_blocks = max(1, math.ceil(1.1 * need))
    if free_order is None:
        rng = np.random.default_rng(seed) if rng is None else rng
        free_order = rng.permutation(n_blocks).astype(np.int32)
    table, _ = deal_tables(lens, b, free_order)
    return Batch(name=name, dtype=dtype, num_heads=hq, num_kv_heads=hkv, head_size=d,
                 block_size=b, num_blocks=n_blocks, block_table=table,
                 context_lens=lens.astype(np.int32), free_order=free_order, seed=seed,
                 query_lens=qlens.astype(np.int32))


def spec_verify_bf16(num_seqs: int = 512, draft: int = 4, lo: int = 64, hi: int = 4096,
                     seed: int = 1006, block_size: int = 16) -> Batch:
    """Speculative verification in the decode-step geometry (bf16, Hq=32,
    Hkv=8, D=128, B=16): every sequence brings ``draft`` query tokens on top
    of U{lo..hi} cached positions."""
    rng = np.random.default_rng(seed)
    hist = rng.integers(lo, hi, size=num_seqs, endpoint=True)
    return _varlen_case("spec_verify_bf16", "bf16", 32, 8, 128, block_size, hist,
                        np.full(num_seqs, draft), seed, rng=rng)


def mixed_prefill_bf16(num_decode: int = 504, num_prefill: int = 8, chunk: int = 512,
                       lo: int = 64, hi: int = 4096, seed: int = 1007,
                       block_size: int = 16) -> Batch:
    """A continuous-batching step in the decode-step geometry (bf16, Hq=32,
    Hkv=8, D=128, B=16): ``num_decode`` sequences with one new token on
    U{lo..hi} cached positions, then ``num_prefill`` chunked prefills of
    ``chunk`` tokens on U{0..hi - chunk} already-computed prompt positions."""
    rng = np.random.default_rng(seed)
    hist_d = rng.integers(lo, hi, size=num_decode, endpoint=True)
    hist_p = rng.integers(0, hi - chunk, size=num_prefill, endpoint=True)
    hist = np.concatenate([hist_d, hist_p])
    q = np.concatenate([np.ones(num_decode, np.int64), np.full(num_prefill, chunk)])
    return _varlen_case("mixed_prefill_bf16", "bf16", 32, 8, 128, block_size, hist, q, seed,
                        rng=rng)


def cow_fork_bf16(num_prompts: int = 128, branches: int = 4, lo: int = 64, hi: int = 4096,
                  num_layers: int = 32, seed: int = 1008, block_size: int = 16) -> Batch:
    """Parallel sampling in the decode-step geometry (bf16, Hq=32, Hkv=8,
    D=128, B=16, 32 layers): ``num_prompts`` prompts of U{lo..hi} tokens, each
    forked into ``branches`` sequences sharing its blocks; then every branch
    appends one token, prompt by prompt, the forked branches first and the
    original last.

    The situation, as input data: a prompt whose last block is partly filled
    has that block shared by all its branches, so each forked branch gets the
    next block of the free list as a copy of it, and the original, left the
    sole owner, writes in place; a prompt whose last block is full gives every
    branch a fresh block and no copy. Sequences are ordered prompt by prompt,
    forked branches first."""
    b = block_size
    rng = np.random.default_rng(seed)
    plens = rng.integers(lo, hi, size=num_prompts, endpoint=True).astype(np.int64)
    need = int(sum(_nblocks(n, b) for n in plens)) + num_prompts * branches
    n_blocks = max(1, math.ceil(1.1 * need))
    free_order = rng.permutation(n_blocks).astype(np.int32)
    ptab, pos = deal_tables(plens, b, free_order)
    rows, lens, positions, slots, pairs, rids = [], [], [], [], [], []
    for p in range(num_prompts):
        L = int(plens[p])
        nb = _nblocks(L, b)
        base = [int(x) for x in ptab[p, :nb]]
        for j in list(range(1, branches)) + [0]:
            row = list(base)
            if L % b == 0:
                row.append(int(free_order[pos]))
                pos += 1
                slot = row[-1] * b
            elif j != 0:
                fresh = int(free_order[pos])
                pos += 1
                pairs.append((row[-1], fresh))
                row[-1] = fresh
                slot = fresh * b + L % b
            else:
                slot = row[-1] * b + L % b
            rows.append(row)
            lens.append(L + 1)
            positions.append(L)
            slots.append(slot)
            rids.append(("b", p, j) if j else ("p", p))
    width = max(len(r) for r in rows)
    table = np.full((len(rows), width), -1, np.int32)
    for s, r in enumerate(rows):
        table[s, :len(r)] = r
    return Batch(name="cow_fork_bf16", dtype="bf16", num_heads=32, num_kv_heads=8,
                 head_size=128, block_size=b, num_blocks=n_blocks, block_table=table,
                 context_lens=np.array(lens, np.int32), free_order=free_order, seed=seed,
                 num_layers=num_layers, positions=np.array(positions, np.int32),
                 prompt_lens=plens.astype(np.int32), branches=branches, rids=rids,
                 copy_pairs=np.array(pairs, np.int64).reshape(-1, 2),
                 slots=np.array(slots, np.int64))


def prefix_requests(num: int = 512, lo: int = 64, hi: int = 4096, shared: int = 512,
                    share_frac: float = 0.3, vocab: int = 32000, seed: int = 1009):
    """Token ids of ``num`` requests with U{lo..hi} tokens; round(share_frac
    * num) of them (a seeded choice among those longer than the shared part)
    start with the same ``shared``-token system prompt. Returns a list of
    int32 arrays."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, size=num, endpoint=True)
    system = rng.integers(0, vocab, size=shared).astype(np.int32)
    eligible = np.flatnonzero(lens > shared)
    k = min(len(eligible), int(round(share_frac * num)))
    sharers = set(rng.permutation(eligible)[:k].tolist())
    out = []
    for i, n in enumerate(lens):
        t = rng.integers(0, vocab, size=int(n)).astype(np.int32)
        if i in sharers:
            t[:shared] = system
        out.append(t)
    return out


CASES = {
    "tiny": tiny_page_example,
    "mha_fp16": mha_fp16,
    "gqa_shared_bf16": gqa_shared_bf16,
    "long_split_bf16": long_split_bf16,
    "decode_step_bf16": decode_step_bf16,
    "spec_verify_bf16": spec_verify_bf16,
    "mixed_prefill_bf16": mixed_prefill_bf16,
    "cow_fork_bf16": cow_fork_bf16,
}


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------

def _page_example_tensors(batch: Batch):
    """The glossary page's worked example, stated as pools: q [S, Hq, D], the
    K pool and the V pool [N, Hkv, B, D] are N(0,1) float32 draws from numpy
    PCG64 seeded 53, in that order; the shared prefix block's V is 0.5 times
    its K (the example's V prefix = 0.5 x K prefix). Slots no live token
    occupies hold zeros, as the page's pools do."""
    import torch
    rng = np.random.default_rng(batch.seed)
    n, hkv, b, d = batch.num_blocks, batch.num_kv_heads, batch.block_size, batch.head_size
    q = rng.standard_normal((batch.num_seqs, batch.num_heads, d), dtype=np.float32)
    k = rng.standard_normal((n, hkv, b, d), dtype=np.float32)
    v = rng.standard_normal((n, hkv, b, d), dtype=np.float32)
    for blk in batch.shared_blocks:
        v[blk] = np.float32(0.5) * k[blk]
    unused = (np.arange(b)[None, :] >= live_counts(batch)[:, None])[:, None, :, None]
    k = np.where(unused, np.float32(0), k)
    v = np.where(unused, np.float32(0), v)
    return {"q": torch.from_numpy(q), "k_cache": torch.from_numpy(np.ascontiguousarray(k)),
            "v_cache": torch.from_numpy(np.ascontiguousarray(v))}


def live_counts(batch: Batch) -> np.ndarray:
    """Per physical block, how many leading slots hold live data before this
    step's write (0 for blocks no sequence uses)."""
    b = batch.block_size
    cnt = np.zeros(batch.num_blocks, dtype=np.int64)
    for s, n in enumerate(batch.live_lens()):
        nb = _nblocks(int(n), b)
        row = batch.block_table[s, :nb].astype(np.int64)
        if nb == 0:
            continue
        full = np.full(nb, b, dtype=np.int64)
        full[-1] = int(n) - (nb - 1) * b
        np.maximum.at(cnt, row, full)
    return cnt


def _randn(shape, seed: int, dtype: str, device, chunk_rows: int | None = None):
    """N(0,1) float32 from a torch generator seeded ``seed`` on ``device``,
    rounded once to ``dtype``. Large tensors are drawn in row chunks
    (``chunk_rows`` of the leading dimension) from the same generator."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    td = _torch_dtype(dtype)
    out = torch.empty(shape, dtype=td, device=device)
    n0 = shape[0]
    step = n0 if chunk_rows is None else max(1, chunk_rows)
    for i in range(0, n0, step):
        j = min(n0, i + step)
        out[i:j] = torch.randn((j - i,) + tuple(shape[1:]), generator=g, device=device,
                               dtype=torch.float32).to(td)
    return out


def _poison_(pool, counts_dev, block_size: int):
    """NaN into every slot at or beyond its block's live count."""
    import torch
    offs = torch.arange(block_size, device=pool.device)
    dead = offs[None, :] >= counts_dev[:, None]            # [N, B]
    pool.masked_fill_(dead[:, None, :, None], float("nan"))


def layer_tensors(batch: Batch, layer: int = 0, device="cpu", poison: bool = True):
    """q, k_cache, v_cache (+ k_new, v_new for a step with new tokens) of one
    layer, as torch tensors on ``device``."""
    import torch
    if batch.page_example:
        t = _page_example_tensors(batch)
        if poison:
            cnt = torch.as_tensor(live_counts(batch), device="cpu")
            _poison_(t["k_cache"], cnt, batch.block_size)
            _poison_(t["v_cache"], cnt, batch.block_size)
        return {k: (v.to(device) if hasattr(v, "to") else v) for k, v in t.items()}
    base = batch.seed * 1000 + layer * 8
    n, hkv, b, d = batch.num_blocks, batch.num_kv_heads, batch.block_size, batch.head_size
    rows = max(1, (1 << 26) // (hkv * b * d))  # ~64M elements per draw
    out = {
        "q": _randn((batch.num_tokens, batch.num_heads, d), base + 0, batch.dtype, device),
        "k_cache": _randn((n, hkv, b, d), base + 1, batch.dtype, device, rows),
        "v_cache": _randn((n, hkv, b, d), base + 2, batch.dtype, device, rows),
    }
    if batch.positions is not None:
        out["k_new"] = _randn((batch.num_seqs, hkv, d), base + 3, batch.dtype, device)
        out["v_new"] = _randn((batch.num_seqs, hkv, d), base + 4, batch.dtype, device)
    if poison:
        cnt = torch.as_tensor(live_counts(batch), device=device)
        _poison_(out["k_cache"], cnt, b)
        _poison_(out["v_cache"], cnt, b)
    return out


def random_partials(num_seqs: int, num_heads: int, head_size: int, max_partitions: int,
                    context_lens, partition_size: int, seed: int, device="cpu"):
    """Synthetic split partials for testing a merge on its own: m ~ N(0, 3^2),
    l ~ U(1, 64), o ~ N(0, 1) for partitions a sequence has; NaN beyond."""
    import torch
    g = torch.Generator().manual_seed(seed)
    shape = (num_seqs, num_heads, max_partitions)
    m = torch.randn(shape, generator=g) * 3.0
    l = 1.0 + 63.0 * torch.rand(shape, generator=g)
    o = torch.randn(shape + (head_size,), generator=g)
    ctx = torch.as_tensor(np.asarray(context_lens, dtype=np.int64))
    np_ = (ctx + partition_size - 1) // partition_size
    dead = torch.arange(max_partitions)[None, :] >= np_[:, None]     # [S, P]
    dead = dead[:, None, :].expand(shape)
    m[dead] = float("nan")
    l[dead] = float("nan")
    o[dead] = float("nan")
    return m.to(device), l.to(device), o.to(device)
