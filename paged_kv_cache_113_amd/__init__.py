"""Python binding of libpagedkv.so, the gfx950 paged-KV decode library.

Argument marshalling only: each function takes torch tensors, passes their
device pointers, sizes and torch's current HIP stream to the C entry point of
the same name (include/pagedkv.h) and raises on a non-zero status. Every step
of the computation runs in the library's HIP kernels; there is no fallback.
If the library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_F32, PKV_F16, PKV_BF16 = 0, 1, 2
_DTYPE = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}

# C signatures, mirrored from include/pagedkv.h
_P, _I32, _I64, _F32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
SIGNATURES = {
    "paged_slot_mapping": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P]),
    "paged_kv_write": (_I32, [_P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _P]),
    "paged_decode_attention": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                      _I64, _I32, _F32, _I32, _I32, _P, _P, _P, _I32, _P]),
    "paged_decode_attention_merged": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                             _I32, _I64, _I32, _F32, _I32, _I32, _P, _P, _P, _P,
                                             _I32, _P]),
    "paged_decode_attention_append": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                             _I32, _I32, _I64, _I32, _F32, _I32, _I32, _P, _P,
                                             _P, _P, _I32, _P]),
    "paged_attention_reduce": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P]),
    "paged_varlen_attention": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                      _I32, _I32, _I64, _I32, _F32, _I32, _P, _P, _P, _I32,
                                      _P]),
    "paged_kv_copy_blocks": (_I32, [_P, _P, _I32, _P, _I64, _I64, _I32, _I32, _I32, _I32,
                                    _P]),
    "paged_kv_swap_out": (_I32, [_P, _I64, _P, _P, _I32, _P, _I64, _I64, _I32, _I32, _I32,
                                 _I32, _P]),
    "paged_kv_swap_in": (_I32, [_P, _I64, _P, _P, _I32, _P, _I64, _I64, _I32, _I32, _I32,
                                _I32, _P]),
    "paged_varlen_attention_noalloc": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                              _I32, _I32, _I32, _I64, _I32, _F32, _I32, _I32,
                                              _P]),
    "paged_varlen_attention_noalloc_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32]),
    "paged_varlen_attention_noalloc_limit": (ctypes.c_size_t, []),
    "paged_attention_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32]),
    "paged_kv_gather": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I64, _I32,
                               _I32, _I32, _P]),
    "pkv_block_hashes": (_I64, [_P, _P, _I64, _I32, _P, _I64]),
    "pkv_pool_create": (_I32, [_P, _I32, _I32, _P]),
    "pkv_pool_destroy": (None, [_P]),
    "pkv_pool_num_free": (_I64, [_P]),
    "pkv_pool_longest_hit": (_I32, [_P, _P, _I32, _P]),
    "pkv_pool_touch": (_I32, [_P, _P, _I32]),
    "pkv_pool_allocate": (_I32, [_P, _I32, _P]),
    "pkv_pool_cache": (_I32, [_P, _I32, _P]),
    "pkv_pool_release": (_I32, [_P, _P, _I32]),
    "pkv_pool_admit": (_I32, [_P, _P, _I64, _P, _I64, _P, _P]),
    "pkv_pool_cache_full_blocks": (_I32, [_P, _P, _P, _I64, _P, _I64]),
    "pkv_pool_state": (_I32, [_P, _P, _P, _P]),
    "pkv_strerror": (ctypes.c_char_p, [_I32]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python __graft_entry__.py` "
            "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class PagedKVError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {code} ({lib.pkv_strerror(code).decode()})")
        self.code = code


def _check(fn, code):
    if code != 0:
        raise PagedKVError(fn, code)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def _need(cond, what):
    """Host-side argument check: the library trusts sizes it is given, so a
    tensor smaller than they say would be read or written out of bounds."""
    if not cond:
        raise ValueError(what)


def _pool_geometry(k_cache, v_cache):
    _need(k_cache.dim() == 4, "pools are [num_blocks, Hkv, B, D]")
    _need(k_cache.shape == v_cache.shape and k_cache.dtype == v_cache.dtype,
          "K and V pools differ in shape or dtype")
    _need(k_cache.dtype in _DTYPE, f"unsupported dtype {k_cache.dtype}")
    return k_cache.shape


def _i32(*ts):
    for t in ts:
        _need(t.dtype == torch.int32, "block tables, lengths, positions and query starts are "
                                      "int32")


def _workspace(rows, mp, d, max_logits, exp_sums, tmp_out):
    for t in (max_logits, exp_sums, tmp_out):
        _need(t is not None, "the split needs max_logits, exp_sums and tmp_out")
        _need(t.dtype == torch.float32, "the workspace is float32")
    _need(max_logits.numel() >= rows * mp and exp_sums.numel() >= rows * mp,
          f"max_logits / exp_sums need {rows} x {mp} floats")
    _need(tmp_out.numel() >= rows * mp * d, f"tmp_out needs {rows} x {mp} x {d} floats")


def paged_slot_mapping(slot_mapping, block_table, positions, block_size, stream=None):
    """slot_mapping[s] = block_table[s][p // B] * B + p % B, p = positions[s]."""
    _need(slot_mapping.dtype == torch.int64, "slot_mapping is int64")
    _i32(block_table, positions)
    _need(block_table.dim() == 2 and block_table.shape[0] == positions.numel(),
          "block_table is [num_seqs, max_blocks] with one row per position")
    _need(slot_mapping.numel() >= positions.numel(), "slot_mapping is shorter than positions")
    _dev(slot_mapping, block_table, positions)
    _check("paged_slot_mapping", lib.paged_slot_mapping(
        _ptr(slot_mapping), _ptr(block_table), _ptr(positions), positions.shape[0],
        block_table.shape[1], block_size, _stream(stream)))


def paged_kv_write(k_cache, v_cache, k_new, v_new, slot_mapping, stream=None):
    """Store k_new/v_new [T, Hkv, D] at their slots of [N, Hkv, B, D] pools."""
    n, hkv, b, d = _pool_geometry(k_cache, v_cache)
    _need(k_new.dim() == 3 and k_new.shape[1:] == (hkv, d) and v_new.shape == k_new.shape,
          "k_new / v_new are [num_tokens, Hkv, D] of the pools' geometry")
    _need(k_new.dtype == v_new.dtype == k_cache.dtype, "new K/V and pools differ in dtype")
    _need(slot_mapping.dtype == torch.int64, "slot_mapping is int64")
    _need(slot_mapping.numel() >= k_new.shape[0], "slot_mapping is shorter than k_new")
    _dev(k_cache, v_cache, k_new, v_new, slot_mapping)
    _check("paged_kv_write", lib.paged_kv_write(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
        k_new.shape[0], n, hkv, b, d, _DTYPE[k_cache.dtype], _stream(stream)))


def paged_decode_attention(out, query, k_cache, v_cache, block_table, context_lens, scale,
                           partition_size=0, max_partitions=0, max_logits=None,
                           exp_sums=None, tmp_out=None, stream=None):
    """Decode attention; split mode writes the partials (see include/pagedkv.h)."""
    n, hkv, b, d = _pool_geometry(k_cache, v_cache)
    _need(query.dim() == 3 and query.shape[2] == d, "query is [num_seqs, Hq, D]")
    _need(query.dtype == k_cache.dtype, "query and pools differ in dtype")
    s, hq, _ = query.shape
    _i32(block_table, context_lens)
    _need(block_table.dim() == 2 and block_table.shape[0] == s,
          "block_table is [num_seqs, max_blocks]")
    _need(context_lens.numel() == s, "context_lens has one entry per sequence")
    if partition_size > 0:
        _workspace(s * hq, max_partitions, d, max_logits, exp_sums, tmp_out)
    else:
        _need(out is not None, "out is needed without a split")
    if out is not None:
        _need(out.dtype == torch.float32 and out.numel() == s * hq * d,
              "out is float32 [num_seqs, Hq, D]")
    _dev(out, query, k_cache, v_cache, block_table, context_lens, max_logits, exp_sums,
         tmp_out)
    _check("paged_decode_attention", lib.paged_decode_attention(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(context_lens), s, hq, hkv, d, b, n, block_table.shape[1], float(scale),
        partition_size, max_partitions, _ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out),
        _DTYPE[query.dtype], _stream(stream)))


def paged_decode_attention_merged(out, query, k_cache, v_cache, block_table, context_lens, scale,
                                  partition_size, max_partitions, max_logits, exp_sums, tmp_out,
                                  counters, stream=None):
    """Split decode attention and its merge in one call into out [S, Hq, D];
    counters [S * Hkv] int32 are zero before and after the call."""
    n, hkv, b, d = _pool_geometry(k_cache, v_cache)
    _need(query.dim() == 3 and query.shape[2] == d, "query is [num_seqs, Hq, D]")
    _need(query.dtype == k_cache.dtype, "query and pools differ in dtype")
    s, hq, _ = query.shape
    _i32(block_table, context_lens, counters)
    _need(block_table.dim() == 2 and block_table.shape[0] == s,
          "block_table is [num_seqs, max_blocks]")
    _need(context_lens.numel() == s, "context_lens has one entry per sequence")
    _need(partition_size > 0, "the merged call splits: partition_size > 0")
    _workspace(s * hq, max_partitions, d, max_logits, exp_sums, tmp_out)
    _need(out is not None and out.dtype == torch.float32 and out.numel() == s * hq * d,
          "out is float32 [num_seqs, Hq, D]")
    _need(counters.numel() >= s * hkv, "counters need num_seqs x Hkv entries")
    _dev(out, query, k_cache, v_cache, block_table, context_lens, max_logits, exp_sums,
         tmp_out, counters)
    _check("paged_decode_attention_merged", lib.paged_decode_attention_merged(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(context_lens), s, hq, hkv, d, b, n, block_table.shape[1], float(scale),
        partition_size, max_partitions, _ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out),
        _ptr(counters), _DTYPE[query.dtype], _stream(stream)))


def paged_decode_attention_append(out, query, k_cache, v_cache, k_new, v_new, block_table,
                                  context_lens, scale, partition_size, max_partitions, max_logits,
                                  exp_sums, tmp_out, counters, stream=None):
    """One decode step of one layer: each sequence's new token k_new / v_new
    [S, Hkv, D] stored at its last position (context_lens - 1), then split
    attention merged into out [S, Hq, D]; counters [S * Hkv] int32 are zero
    before and after the call."""
    n, hkv, b, d = _pool_geometry(k_cache, v_cache)
    _need(query.dim() == 3 and query.shape[2] == d, "query is [num_seqs, Hq, D]")
    _need(query.dtype == k_cache.dtype, "query and pools differ in dtype")
    s, hq, _ = query.shape
    _need(k_new.shape == (s, hkv, d) and v_new.shape == k_new.shape,
          "k_new / v_new are [num_seqs, Hkv, D]")
    _need(k_new.dtype == v_new.dtype == k_cache.dtype, "new K/V and pools differ in dtype")
    _i32(block_table, context_lens, counters)
    _need(block_table.dim() == 2 and block_table.shape[0] == s,
          "block_table is [num_seqs, max_blocks]")
    _need(context_lens.numel() == s, "context_lens has one entry per sequence")
    _need(partition_size > 0, "the call splits: partition_size > 0")
    _workspace(s * hq, max_partitions, d, max_logits, exp_sums, tmp_out)
    _need(out is not None and out.dtype == torch.float32 and out.numel() == s * hq * d,
          "out is float32 [num_seqs, Hq, D]")
    _need(counters.numel() >= s * hkv, "counters need num_seqs x Hkv entries")
    _dev(out, query, k_cache, v_cache, k_new, v_new, block_table, context_lens, max_logits,
         exp_sums, tmp_out, counters)
    _check("paged_decode_attention_append", lib.paged_decode_attention_append(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
        _ptr(block_table), _ptr(context_lens), s, hq, hkv, d, b, n, block_table.shape[1],
        float(scale), partition_size, max_partitions, _ptr(max_logits), _ptr(exp_sums),
        _ptr(tmp_out), _ptr(counters), _DTYPE[query.dtype], _stream(stream)))


def paged_attention_reduce(out, max_logits, exp_sums, tmp_out, context_lens, partition_size,
                           stream=None):
    """Log-sum-exp merge of split partials [S, Hq, P(, D)] into out [S, Hq, D]."""
    _need(tmp_out.dim() == 4, "tmp_out is [num_seqs, Hq, max_partitions, D]")
    s, hq, p, d = tmp_out.shape
    _workspace(s * hq, p, d, max_logits, exp_sums, tmp_out)
    _need(out.dtype == torch.float32 and out.numel() == s * hq * d,
          "out is float32 [num_seqs, Hq, D]")
    _i32(context_lens)
    _need(context_lens.numel() == s, "context_lens has one entry per sequence")
    _dev(out, max_logits, exp_sums, tmp_out, context_lens)
    _check("paged_attention_reduce", lib.paged_attention_reduce(
        _ptr(out), _ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out), _ptr(context_lens), s, hq,
        d, partition_size, p, _stream(stream)))


def paged_varlen_attention(out, query, k_cache, v_cache, block_table, query_start_loc,
                           context_lens, scale, max_partitions, max_logits, exp_sums, tmp_out,
                           stream=None):
    """Causal attention of several query tokens per sequence (rows
    query_start_loc[s]..query_start_loc[s+1]-1, at the last positions of the
    sequence's context) into out [T, Hq, D]; partials go through the
    workspace [T, Hq, P(, D)]."""
    n, hkv, b, d = _pool_geometry(k_cache, v_cache)
    _need(query.dim() == 3 and query.shape[2] == d, "query is [num_tokens, Hq, D]")
    _need(query.dtype == k_cache.dtype, "query and pools differ in dtype")
    t, hq, _ = query.shape
    _i32(block_table, query_start_loc, context_lens)
    ns = context_lens.numel()
    _need(block_table.dim() == 2 and block_table.shape[0] == ns,
          "block_table is [num_seqs, max_blocks]")
    _need(query_start_loc.numel() == ns + 1, "query_start_loc has num_seqs + 1 entries")
    _need(out.dtype == torch.float32 and out.numel() == t * hq * d,
          "out is float32 [num_tokens, Hq, D]")
    _workspace(t * hq, max_partitions, d, max_logits, exp_sums, tmp_out)
    _dev(out, query, k_cache, v_cache, block_table, query_start_loc, context_lens, max_logits,
         exp_sums, tmp_out)
    _check("paged_varlen_attention", lib.paged_varlen_attention(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(query_start_loc), _ptr(context_lens), context_lens.shape[0], t, hq, hkv, d, b, n,
        block_table.shape[1], float(scale), max_partitions, _ptr(max_logits), _ptr(exp_sums),
        _ptr(tmp_out), _DTYPE[query.dtype], _stream(stream)))


def paged_varlen_attention_noalloc(out, query, k_cache, v_cache, block_table,
                                   query_start_loc, context_lens, scale, max_partitions,
                                   stream=None):
    """paged_varlen_attention without a workspace: the partials go to the
    library's static device buffer (no device allocation in the call). Calls
    that overlap on one GPU race on that buffer."""
    n, hkv, b, d = _pool_geometry(k_cache, v_cache)
    _need(query.dim() == 3 and query.shape[2] == d, "query is [num_tokens, Hq, D]")
    _need(query.dtype == k_cache.dtype, "query and pools differ in dtype")
    t, hq, _ = query.shape
    _i32(block_table, query_start_loc, context_lens)
    ns = context_lens.numel()
    _need(block_table.dim() == 2 and block_table.shape[0] == ns,
          "block_table is [num_seqs, max_blocks]")
    _need(query_start_loc.numel() == ns + 1, "query_start_loc has num_seqs + 1 entries")
    _need(out.dtype == torch.float32 and out.numel() == t * hq * d,
          "out is float32 [num_tokens, Hq, D]")
    _dev(out, query, k_cache, v_cache, block_table, query_start_loc, context_lens)
    _check("paged_varlen_attention_noalloc", lib.paged_varlen_attention_noalloc(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(query_start_loc), _ptr(context_lens), ns, t, hq, hkv, d, b, n,
        block_table.shape[1], float(scale), max_partitions, _DTYPE[query.dtype],
        _stream(stream)))


def paged_varlen_attention_noalloc_bytes(num_tokens, num_heads, head_size, max_partitions):
    return int(lib.paged_varlen_attention_noalloc_bytes(num_tokens, num_heads, head_size,
                                                        max_partitions))


def paged_varlen_attention_noalloc_limit():
    return int(lib.paged_varlen_attention_noalloc_limit())


class PoolSet:
    """Every layer's K and V pools, checked once (one shape and dtype, on the
    GPU, contiguous), with the host arrays of their device pointers that the
    block-move calls take. Pass it in place of the two lists to skip the
    per-call checks in a serving loop."""

    def __init__(self, k_caches, v_caches):
        if isinstance(k_caches, PoolSet):
            raise TypeError("already a PoolSet")
        if len(k_caches) != len(v_caches) or not k_caches:
            raise ValueError("one K and one V pool per layer")
        _dev(*k_caches, *v_caches)
        shape, dtype = k_caches[0].shape, k_caches[0].dtype
        for t in (*k_caches, *v_caches):
            if t.shape != shape or t.dtype != dtype:
                raise ValueError("every layer's pools share one shape and dtype")
        arr = ctypes.c_void_p * len(k_caches)
        self.k = arr(*[t.data_ptr() for t in k_caches])
        self.v = arr(*[t.data_ptr() for t in v_caches])
        self.tensors = (list(k_caches), list(v_caches))   # keeps the storage alive
        self.num_layers = len(k_caches)
        self.shape = shape
        self.dtype = dtype


def _pools(k_caches, v_caches):
    ps = k_caches if isinstance(k_caches, PoolSet) else PoolSet(k_caches, v_caches)
    return ps.k, ps.v, ps.num_layers, ps.shape, ps.dtype


def paged_kv_copy_blocks(k_caches, v_caches, block_mapping, stream=None):
    """Copy block src -> dst in every layer's K and V pool, for each row
    (src, dst) of block_mapping [n, 2] int64 (copy-on-write). k_caches may be
    a PoolSet (then v_caches is ignored)."""
    kp, vp, nl, (n, hkv, b, d), dtype = _pools(k_caches, v_caches)
    _dev(block_mapping)
    _need(block_mapping.dtype == torch.int64 and block_mapping.dim() == 2 and
          block_mapping.shape[1] == 2, "block_mapping is int64 [num_pairs, 2]")
    _check("paged_kv_copy_blocks", lib.paged_kv_copy_blocks(
        kp, vp, nl, _ptr(block_mapping), block_mapping.shape[0], n, hkv, b, d,
        _DTYPE[dtype], _stream(stream)))


def _host_buf(host, dtype):
    if host.is_cuda or not host.is_contiguous() or host.dtype != dtype:
        raise ValueError("the host buffer is a contiguous CPU tensor of the pools' dtype")
    return ctypes.c_void_p(host.data_ptr()), host.numel() * host.element_size()


def paged_kv_swap_out(host_dst, k_caches, v_caches, block_ids, stream=None):
    """host_dst [L, 2, n, Hkv, B, D] (pinned) <- blocks block_ids of every
    layer's K (index 0) and V (index 1) pool. k_caches may be a PoolSet."""
    kp, vp, nl, (n, hkv, b, d), dtype = _pools(k_caches, v_caches)
    _dev(block_ids)
    _need(block_ids.dtype == torch.int64, "block_ids is int64")
    hp, nbytes = _host_buf(host_dst, dtype)
    _check("paged_kv_swap_out", lib.paged_kv_swap_out(
        hp, nbytes, kp, vp, nl, _ptr(block_ids), block_ids.numel(), n, hkv, b, d,
        _DTYPE[dtype], _stream(stream)))


def paged_kv_swap_in(host_src, k_caches, v_caches, block_ids, stream=None):
    """Blocks block_ids of every layer's pools <- host_src [L, 2, n, Hkv, B, D].
    k_caches may be a PoolSet."""
    kp, vp, nl, (n, hkv, b, d), dtype = _pools(k_caches, v_caches)
    _dev(block_ids)
    _need(block_ids.dtype == torch.int64, "block_ids is int64")
    hp, nbytes = _host_buf(host_src, dtype)
    _check("paged_kv_swap_in", lib.paged_kv_swap_in(
        hp, nbytes, kp, vp, nl, _ptr(block_ids), block_ids.numel(), n, hkv, b, d,
        _DTYPE[dtype], _stream(stream)))


def paged_attention_workspace_bytes(num_seqs, num_heads, head_size, max_partitions):
    return int(lib.paged_attention_workspace_bytes(num_seqs, num_heads, head_size,
                                                   max_partitions))


def paged_kv_gather(k_out, v_out, k_cache, v_cache, block_table, context_lens, stream=None):
    """Contiguous copy [S, Hkv, max_ctx, D] of each sequence's K and V."""
    n, hkv, b, d = _pool_geometry(k_cache, v_cache)
    _need(k_out.dim() == 4 and k_out.shape == v_out.shape and k_out.shape[1] == hkv and
          k_out.shape[3] == d, "k_out / v_out are [num_seqs, Hkv, max_ctx, D]")
    _need(k_out.dtype == v_out.dtype == k_cache.dtype, "outputs and pools differ in dtype")
    s, _, max_ctx, _ = k_out.shape
    _i32(block_table, context_lens)
    _need(block_table.dim() == 2 and block_table.shape[0] == s,
          "block_table is [num_seqs, max_blocks]")
    _need(context_lens.numel() == s, "context_lens has one entry per sequence")
    _dev(k_out, v_out, k_cache, v_cache, block_table, context_lens)
    _check("paged_kv_gather", lib.paged_kv_gather(
        _ptr(k_out), _ptr(v_out), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(context_lens), s, hkv, d, b, n, block_table.shape[1], max_ctx,
        _DTYPE[k_cache.dtype], _stream(stream)))


# -- prefix caching (host side) ---------------------------------------------------

def _host_i32(x):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _bytes_ptr(b):
    if not b:
        return None, 0
    buf = ctypes.create_string_buffer(bytes(b), len(b))
    return buf, len(b)


def block_hashes(tokens, block_size, extra=b""):
    """32-byte identities of the full blocks of ``tokens`` (a list of bytes)."""
    a, ap = _host_i32(tokens)
    nb = len(a) // block_size
    out = ctypes.create_string_buffer(max(1, 32 * nb))
    eb, el = _bytes_ptr(extra)
    n = lib.pkv_block_hashes(out, ap, len(a), block_size, eb, el)
    _check("pkv_block_hashes", n if n < 0 else 0)
    raw = out.raw
    return [raw[32 * i:32 * i + 32] for i in range(n)]


class BlockPool:
    """The library's cached block pool (host memory, one caller at a time)."""

    def __init__(self, num_blocks, block_size, initial_free=None):
        self.num_blocks, self.block_size = num_blocks, block_size
        h = ctypes.c_void_p()
        if initial_free is None:
            code = lib.pkv_pool_create(ctypes.byref(h), num_blocks, block_size, None)
        else:
            a, ap = _host_i32(initial_free)
            code = lib.pkv_pool_create(ctypes.byref(h), num_blocks, block_size, ap)
        _check("pkv_pool_create", code)
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            lib.pkv_pool_destroy(h)
            self._h = None

    def num_free(self):
        return int(lib.pkv_pool_num_free(self._h))

    def longest_hit(self, hashes):
        buf = ctypes.create_string_buffer(b"".join(hashes), max(1, 32 * len(hashes)))
        out = (ctypes.c_int32 * max(1, len(hashes)))()
        k = lib.pkv_pool_longest_hit(self._h, buf, len(hashes), out)
        _check("pkv_pool_longest_hit", k if k < 0 else 0)
        return list(out[:k])

    def touch(self, blocks):
        a, ap = _host_i32(blocks)
        _check("pkv_pool_touch", lib.pkv_pool_touch(self._h, ap, len(a)))

    def allocate(self, n):
        out = (ctypes.c_int32 * max(1, n))()
        _check("pkv_pool_allocate", lib.pkv_pool_allocate(self._h, n, out))
        return list(out[:n])

    def cache(self, block, h):
        code = lib.pkv_pool_cache(self._h, block, ctypes.create_string_buffer(bytes(h), 32))
        _check("pkv_pool_cache", code if code < 0 else 0)
        return bool(code)

    def release(self, blocks):
        a, ap = _host_i32(blocks)
        _check("pkv_pool_release", lib.pkv_pool_release(self._h, ap, len(a)))

    def admit(self, tokens, extra=b""):
        a, ap = _host_i32(tokens)
        nb = -(-len(a) // self.block_size)
        out = (ctypes.c_int32 * max(1, nb))()
        cached = ctypes.c_int64()
        eb, el = _bytes_ptr(extra)
        _check("pkv_pool_admit", lib.pkv_pool_admit(self._h, ap, len(a), eb, el, out,
                                                    ctypes.byref(cached)))
        return list(out[:nb]), int(cached.value)

    def cache_full_blocks(self, table, tokens, extra=b""):
        t, tp = _host_i32(table)
        a, ap = _host_i32(tokens)
        eb, el = _bytes_ptr(extra)
        _check("pkv_pool_cache_full_blocks",
               lib.pkv_pool_cache_full_blocks(self._h, tp, ap, len(a), eb, el))

    def state(self):
        """(reference counts, free queue head to tail, cached flags)."""
        ref = (ctypes.c_int32 * self.num_blocks)()
        free = (ctypes.c_int32 * self.num_blocks)()
        cached = (ctypes.c_uint8 * self.num_blocks)()
        n = lib.pkv_pool_state(self._h, ref, free, cached)
        _check("pkv_pool_state", n if n < 0 else 0)
        return list(ref), list(free[:n]), [bool(c) for c in cached]


def pkv_strerror(code):
    return lib.pkv_strerror(code).decode()
