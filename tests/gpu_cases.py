"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
on a batch from ``workloads`` and compute the oracle's answer on the host
from the same inputs (never from the HIP path's outputs)."""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import oracle
import workloads as W

TOL = 2e-3                      # max abs error vs the fp64 oracle
THREADS = min(16, os.cpu_count() or 1)


def scale_of(batch):
    return float(np.float32(1.0 / math.sqrt(batch.head_size)))


def device_meta(batch, dev):
    m = {"table": torch.as_tensor(batch.block_table, device=dev),
         "ctx": torch.as_tensor(batch.context_lens, device=dev)}
    if batch.positions is not None:
        m["pos"] = torch.as_tensor(batch.positions, device=dev)
    return m


def gpu_write(pkv, batch, t, meta, dev):
    """Slot mapping + K/V write of the new tokens (decode step)."""
    slots = torch.empty(batch.num_seqs, dtype=torch.int64, device=dev)
    pkv.paged_slot_mapping(slots, meta["table"], meta["pos"], batch.block_size)
    pkv.paged_kv_write(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], slots)
    return slots


def gpu_attention(pkv, batch, t, meta, dev, partition_size=0, max_partitions=None):
    out = torch.empty(batch.num_seqs, batch.num_heads, batch.head_size, device=dev)
    scale = scale_of(batch)
    if partition_size == 0:
        pkv.paged_decode_attention(out, t["q"], t["k_cache"], t["v_cache"], meta["table"],
                                   meta["ctx"], scale)
        return out
    mp = batch.max_partitions(partition_size) if max_partitions is None else max_partitions
    shape = (batch.num_seqs, batch.num_heads, mp)
    ml = torch.full(shape, float("nan"), device=dev)
    es = torch.full(shape, float("nan"), device=dev)
    to = torch.full(shape + (batch.head_size,), float("nan"), device=dev)
    pkv.paged_decode_attention(None, t["q"], t["k_cache"], t["v_cache"], meta["table"],
                               meta["ctx"], scale, partition_size, mp, ml, es, to)
    pkv.paged_attention_reduce(out, ml, es, to, meta["ctx"], partition_size)
    return out


def host(t):
    return {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in t.items()}


def oracle_slots(batch):
    tables = [row[row >= 0].tolist() for row in batch.block_table]
    return oracle.allocator.slot_mapping(tables, batch.positions.tolist(), batch.block_size)


def oracle_pools_after_write(batch, th):
    """The oracle's own write of the new tokens into host copies of the
    pre-write pools (raw storage bits)."""
    slots = oracle_slots(batch)
    k = oracle._raw(th["k_cache"], batch.dtype)
    v = oracle._raw(th["v_cache"], batch.dtype)
    kn = oracle.scatter.scatter(k, oracle._raw(th["k_new"], batch.dtype), slots)
    vn = oracle.scatter.scatter(v, oracle._raw(th["v_new"], batch.dtype), slots)
    return kn, vn, slots


def oracle_attention(batch, q, k, v, seqs=None):
    return oracle.attention(q, k, v, batch.block_table, batch.context_lens, scale_of(batch),
                            batch.dtype, seqs=seqs, threads=THREADS)


def max_err(got, want):
    g = got.double().numpy() if hasattr(got, "numpy") else got
    assert np.isfinite(g).all(), "non-finite output"
    return float(np.abs(g - want).max()) if want.size else 0.0


def gpu_varlen(pkv, batch, t, meta, dev, max_partitions=8, scale=None):
    """Multi-token attention through the C ABI; the workspace starts as NaN
    so that a slot the kernels forget shows up in the output."""
    T, H, D = batch.num_tokens, batch.num_heads, batch.head_size
    out = torch.full((T, H, D), float("nan"), device=dev)
    shape = (T, H, max_partitions)
    ml = torch.full(shape, float("nan"), device=dev)
    es = torch.full(shape, float("nan"), device=dev)
    to = torch.full(shape + (D,), float("nan"), device=dev)
    qsl = torch.as_tensor(batch.query_start_loc, device=dev)
    pkv.paged_varlen_attention(out, t["q"], t["k_cache"], t["v_cache"], meta["table"], qsl,
                               meta["ctx"], scale_of(batch) if scale is None else scale,
                               max_partitions, ml, es, to)
    return out


def oracle_varlen(batch, q, k, v, seqs=None, scale=None):
    """The oracle's multi-token attention on the host copies; with ``seqs``,
    on those sequences only (returns their rows, in order)."""
    qsl = batch.query_start_loc
    if seqs is None:
        return oracle.attention_varlen(q, k, v, batch.block_table, qsl, batch.context_lens,
                                       scale_of(batch) if scale is None else scale,
                                       batch.dtype, threads=THREADS)
    rows = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in seqs]).astype(np.int64)
    sub_q = q[torch.as_tensor(rows)]
    ql = np.array([qsl[s + 1] - qsl[s] for s in seqs], np.int64)
    sub_qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    return oracle.attention_varlen(sub_q, k, v, batch.block_table[list(seqs)], sub_qsl,
                                   batch.context_lens[list(seqs)], scale_of(batch),
                                   batch.dtype, threads=THREADS), rows
