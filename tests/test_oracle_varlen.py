"""Pins for the oracle's multi-token (chunked prefill / speculative) attention.

A sequence with q_s new tokens has them at its last q_s positions; the token
at position p sees positions 0..p (causal). The expected values come from:
  * torch's fp64 scaled_dot_product_attention on the CPU with
    ``causal_lower_right`` -- a library definition of a causal mask aligned
    to the end of the key sequence -- over K/V rebuilt position by position
    from the pool and repeated per query head with ``repeat_interleave``;
  * closed forms: the first token of a fresh prefill sees one position and
    returns its value exactly; a zero query returns the mean of the visible
    values; the last token of a chunk sees the whole context (so one token
    per sequence is plain decode attention, pinned elsewhere).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
import workloads as W


def _to64(t, dtype):
    if dtype == "bf16":
        return t.to(torch.float64)
    return t.to(torch.float64) if isinstance(t, torch.Tensor) else torch.from_numpy(t)


def _case(rng, dtype, hq, hkv, d, b, lens, qlens, extra_blocks=2):
    need = sum(-(-L // b) for L in lens)
    n = need + extra_blocks
    perm = rng.permutation(n)
    width = max(1, max(-(-L // b) for L in lens))
    table = np.full((len(lens), width), -1, np.int32)
    pos = 0
    for s, L in enumerate(lens):
        nb = -(-L // b)
        table[s, :nb] = perm[pos:pos + nb]
        pos += nb
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    td = W._torch_dtype(dtype)
    g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
    q = torch.randn(int(qsl[-1]), hq, d, generator=g).to(td)
    kp = torch.randn(n, hkv, b, d, generator=g).to(td)
    vp = torch.randn(n, hkv, b, d, generator=g).to(td)
    return q, kp, vp, table, qsl, np.array(lens, np.int32)


def sdpa_reference(q, kp, vp, table, qsl, ctx, scale, dtype):
    """torch fp64 SDPA per sequence with a lower-right causal mask."""
    q64, k64, v64 = _to64(q, dtype), _to64(kp, dtype), _to64(vp, dtype)
    n, hkv, b, d = k64.shape
    hq = q64.shape[1]
    out = torch.zeros(q64.shape, dtype=torch.float64)
    for s in range(len(ctx)):
        L, r0, r1 = int(ctx[s]), int(qsl[s]), int(qsl[s + 1])
        if r1 == r0:
            continue
        K = torch.stack([k64[int(table[s][t // b]), :, t % b] for t in range(L)], dim=1)
        V = torch.stack([v64[int(table[s][t // b]), :, t % b] for t in range(L)], dim=1)
        K = K.repeat_interleave(hq // hkv, dim=0)   # [hq, L, d]
        V = V.repeat_interleave(hq // hkv, dim=0)
        Q = q64[r0:r1].transpose(0, 1)               # [hq, qn, d]
        mask = causal_lower_right(r1 - r0, L)
        o = F.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=mask,
                                           scale=float(scale))
        out[r0:r1] = o[0].transpose(0, 1)
    return out.numpy()


@pytest.mark.parametrize("seed", range(10))
def test_varlen_matches_sdpa_lower_right(seed):
    rng = np.random.default_rng(500 + seed)
    dtype = ["f32", "f16", "bf16"][seed % 3]
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([4, 8, 16]))
    b = int(rng.choice([1, 2, 4]))
    ns = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(1, 30, size=ns)]
    # mixes fresh prefills (q = ctx), chunks on top of a history, decode (1)
    # and empty query sets (0)
    qlens = [int(rng.choice([0, 1, min(3, L), L, int(rng.integers(1, L + 1))])) for L in lens]
    q, kp, vp, table, qsl, ctx = _case(rng, dtype, hq, hkv, d, b, lens, qlens)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    got = oracle.attention_varlen(q, kp, vp, table, qsl, ctx, scale, dtype)
    want = sdpa_reference(q, kp, vp, table, qsl, ctx, scale, dtype)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)
    got_t = oracle.attention_varlen(q, kp, vp, table, qsl, ctx, scale, dtype, threads=3)
    assert np.array_equal(got, got_t)


def test_first_prefill_token_sees_one_position():
    """Fresh prefill (q_s = ctx_s): row 0 attends position 0 alone, so its
    output is v_0 exactly, whatever the scores."""
    rng = np.random.default_rng(11)
    q, kp, vp, table, qsl, ctx = _case(rng, "bf16", 4, 2, 8, 4, [9, 6], [9, 6])
    out = oracle.attention_varlen(q, kp, vp, table, qsl, ctx, 0.3, "bf16")
    v64 = vp.to(torch.float64).numpy()
    for s in range(2):
        v0 = v64[int(table[s][0]), :, 0]                  # [hkv, d]
        assert np.array_equal(out[qsl[s]], np.repeat(v0, 2, axis=0))


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(12)
    q, kp, vp, table, qsl, ctx = _case(rng, "f32", 2, 1, 4, 2, [7], [3])
    q = torch.zeros_like(q)
    out = oracle.attention_varlen(q, kp, vp, table, qsl, ctx, 1.0, "f32")
    v64 = vp.numpy().astype(np.float64)
    V = np.stack([v64[int(table[0][t // 2]), 0, t % 2] for t in range(7)])
    for i in range(3):
        p = 7 - 3 + i
        np.testing.assert_allclose(out[i, 0], V[:p + 1].mean(axis=0), rtol=1e-14, atol=1e-15)


def test_one_token_per_sequence_is_decode():
    rng = np.random.default_rng(13)
    q, kp, vp, table, qsl, ctx = _case(rng, "f16", 8, 2, 16, 4, [13, 5, 22], [1, 1, 1])
    scale = float(np.float32(0.25))
    a = oracle.attention_varlen(q, kp, vp, table, qsl, ctx, scale, "f16")
    b = oracle.attention(q, kp, vp, table, ctx, scale, "f16")
    assert np.array_equal(a, b)


def test_last_token_of_chunk_sees_everything():
    """The chunk's last row equals a decode call over the whole context."""
    rng = np.random.default_rng(14)
    q, kp, vp, table, qsl, ctx = _case(rng, "bf16", 4, 1, 8, 4, [17, 10], [5, 10])
    scale = 0.35
    out = oracle.attention_varlen(q, kp, vp, table, qsl, ctx, scale, "bf16")
    last = torch.stack([q[qsl[1] - 1], q[qsl[2] - 1]])
    dec = oracle.attention(last, kp, vp, table, ctx, scale, "bf16")
    assert np.array_equal(out[qsl[1] - 1], dec[0]) and np.array_equal(out[qsl[2] - 1], dec[1])


def test_varlen_rejects_bad_metadata():
    rng = np.random.default_rng(15)
    q, kp, vp, table, qsl, ctx = _case(rng, "f32", 2, 1, 4, 2, [5], [3])
    with pytest.raises(RuntimeError):   # start locations must begin at 0
        oracle.attention_varlen(q, kp, vp, table, np.array([1, 3], np.int32), ctx, 1.0, "f32")
    with pytest.raises(RuntimeError):   # more query tokens than positions
        oracle.attention_varlen(q, kp, vp, table, qsl, np.array([2], np.int32), 1.0, "f32")
