"""CPU oracle for paged-KV decode attention.

TEST INFRASTRUCTURE ONLY. Only tests/, ``__graft_entry__.smoke()`` and the
CPU baseline leg of ``bench.py`` may import this package. It shares no code
with the HIP library and never imports it.

Parts:
  * ``allocator``   -- FIFO block allocator with refcounts, slot translation,
                       block counting (Python).
  * ``scatter``     -- new-token K/V write, bytewise (numpy).
  * ``attn_ref.c``  -- gather + fp64 attention (one query token per sequence,
                       or several with a causal limit), fp64 split partials
                       and their log-sum-exp merge (plain C, pthreads),
                       loaded here via ctypes.

Every function is pinned by tests/test_oracle_*.py against values the pages
print, closed forms and brute force; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import allocator, scatter  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "attn_ref.c")

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
_ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def build(verbose: bool = False) -> str:
    """Compile attn_ref.c with gcc into liboracle.so (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
           "-pthread", "-o", LIB_PATH, SRC_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or (
                os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH)):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        lib.orc_widen.argtypes = [P, P, i64, i32]
        lib.orc_gather.argtypes = [P, P, P, P, i32, P, i32, i64, i32, i32, i32]
        lib.orc_attention.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, i32, i64,
                                      i32, f32, P, i32, i32]
        lib.orc_attention_partials.argtypes = [P, P, P, P, P, P, i32, P, P, i32, i32,
                                               i32, i32, i64, i32, f32, i32, i32, P,
                                               i32, i32]
        lib.orc_lse_combine.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32]
        lib.orc_attention_varlen.argtypes = [P, P, P, P, i32, P, P, P, i32, i32, i32, i32,
                                             i32, i64, i32, f32, i32]
        for f in ("orc_widen", "orc_gather", "orc_attention",
                  "orc_attention_partials", "orc_lse_combine", "orc_attention_varlen"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _raw(a, dtype: str) -> np.ndarray:
    """Contiguous numpy view of the storage bits for ``dtype``."""
    if hasattr(a, "detach"):  # torch tensor on the CPU
        import torch
        a = a.detach().contiguous()
        if a.dtype in (torch.float16, torch.bfloat16):
            a = a.view(torch.int16)
        a = a.numpy()
    a = np.ascontiguousarray(a)
    if a.itemsize != _ELEM_BYTES[dtype]:
        raise TypeError(f"{dtype} storage needs {_ELEM_BYTES[dtype]}-byte items, got {a.dtype}")
    return a


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def widen(a, dtype: str) -> np.ndarray:
    """Exact f32/f16/bf16 -> float64 from the storage bits."""
    raw = _raw(a, dtype)
    out = np.empty(raw.shape, dtype=np.float64)
    _check(_load().orc_widen(_ptr(out), _ptr(raw), raw.size, DTYPE_CODES[dtype]), "widen")
    return out


def gather(k_pool, v_pool, table_row, ctx: int, dtype: str):
    """Contiguous fp64 K, V [Hkv, ctx, D] of one sequence."""
    k = _raw(k_pool, dtype)
    v = _raw(v_pool, dtype)
    n, hkv, b, d = k.shape
    row = np.ascontiguousarray(table_row, dtype=np.int32)
    ko = np.empty((hkv, ctx, d), dtype=np.float64)
    vo = np.empty((hkv, ctx, d), dtype=np.float64)
    _check(_load().orc_gather(_ptr(ko), _ptr(vo), _ptr(k), _ptr(v), DTYPE_CODES[dtype],
                              _ptr(row), ctx, n, hkv, b, d), "gather")
    return ko, vo


def attention(q, k_pool, v_pool, block_table, ctx_lens, scale: float, dtype: str,
              seqs=None, threads: int = 1) -> np.ndarray:
    """fp64 decode attention; returns [len(seqs), Hq, D] (all sequences by default)."""
    qa = _raw(q, dtype)
    k = _raw(k_pool, dtype)
    v = _raw(v_pool, dtype)
    n, hkv, b, d = k.shape
    ns, hq, dq = qa.shape
    assert dq == d
    tab = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    sel = np.arange(ns, dtype=np.int32) if seqs is None else np.ascontiguousarray(seqs, dtype=np.int32)
    out = np.empty((len(sel), hq, d), dtype=np.float64)
    _check(_load().orc_attention(_ptr(out), _ptr(qa), _ptr(k), _ptr(v), DTYPE_CODES[dtype],
                                 _ptr(tab), _ptr(ctx), hq, hkv, d, b, n, tab.shape[1],
                                 float(scale), _ptr(sel), len(sel), int(threads)),
           "attention")
    return out


def attention_partials(q, k_pool, v_pool, block_table, ctx_lens, scale: float, dtype: str,
                       partition_size: int, max_partitions: int, seqs=None, threads: int = 1):
    """fp64 split partials (m, l, o) for the listed sequences."""
    qa = _raw(q, dtype)
    k = _raw(k_pool, dtype)
    v = _raw(v_pool, dtype)
    n, hkv, b, d = k.shape
    ns, hq, _ = qa.shape
    tab = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    sel = np.arange(ns, dtype=np.int32) if seqs is None else np.ascontiguousarray(seqs, dtype=np.int32)
    m = np.empty((len(sel), hq, max_partitions), dtype=np.float64)
    l = np.empty_like(m)
    o = np.empty((len(sel), hq, max_partitions, d), dtype=np.float64)
    _check(_load().orc_attention_partials(
        _ptr(m), _ptr(l), _ptr(o), _ptr(qa), _ptr(k), _ptr(v), DTYPE_CODES[dtype], _ptr(tab),
        _ptr(ctx), hq, hkv, d, b, n, tab.shape[1], float(scale), partition_size,
        max_partitions, _ptr(sel), len(sel), int(threads)), "partials")
    return m, l, o


def lse_combine(m, l, o, ctx_lens, partition_size: int) -> np.ndarray:
    """fp64 log-sum-exp merge of partials [S, Hq, P(, D)] -> [S, Hq, D]."""
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    o = np.ascontiguousarray(o, dtype=np.float64)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    s, hq, p, d = o.shape
    out = np.empty((s, hq, d), dtype=np.float64)
    _check(_load().orc_lse_combine(_ptr(out), _ptr(m), _ptr(l), _ptr(o), _ptr(ctx), s, hq, d,
                                   partition_size, p), "lse_combine")
    return out


def attention_varlen(q, k_pool, v_pool, block_table, query_start_loc, ctx_lens, scale: float,
                     dtype: str, threads: int = 1) -> np.ndarray:
    """fp64 attention of multi-token queries: q [num_tokens, Hq, D]; token i
    of sequence s (tokens qsl[s]..qsl[s+1]-1) attends positions 0 ..
    ctx_s - q_s + i. Returns [num_tokens, Hq, D]."""
    qa = _raw(q, dtype)
    k = _raw(k_pool, dtype)
    v = _raw(v_pool, dtype)
    n, hkv, b, d = k.shape
    nt, hq, _ = qa.shape
    tab = np.ascontiguousarray(block_table, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    assert qsl[-1] == nt and len(qsl) == len(ctx) + 1
    out = np.zeros((nt, hq, d), dtype=np.float64)
    _check(_load().orc_attention_varlen(_ptr(out), _ptr(qa), _ptr(k), _ptr(v),
                                        DTYPE_CODES[dtype], _ptr(tab), _ptr(qsl), _ptr(ctx),
                                        len(ctx), hq, hkv, d, b, n, tab.shape[1], float(scale),
                                        int(threads)), "attention_varlen")
    return out
