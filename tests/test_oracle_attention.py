"""Pins for the oracle's gather, fp64 attention, split partials and LSE merge.

What fixes the expected values (none is the oracle's own output):
  * exact widening: numpy's float16 and torch's bfloat16 conversions over all
    65536 bit patterns;
  * the glossary page's worked example: paged == contiguous (its script
    prints max_attention_abs_diff=0.000e+00), and its fp32 torch attention
    within the script's own rtol=1e-5/atol=1e-6;
  * closed forms of softmax attention (one position, constant keys, zero
    query, the logistic function for two positions, per-KV-head constants
    that expose the query-head -> KV-head map);
  * brute force: contiguous K/V rebuilt position by position with numpy,
    scipy's softmax, explicit head repetition;
  * the log-sum-exp identity for partials, checked against the whole-context
    attention and against hand-weighted closed forms.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

import oracle
import workloads as W


# -- widening -----------------------------------------------------------------

def test_widen_f16_all_patterns():
    bits = np.arange(65536, dtype=np.uint16).view(np.float16)
    got = oracle.widen(bits, "f16")
    want = bits.astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_widen_bf16_all_patterns():
    t = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    got = oracle.widen(t, "bf16")
    want = t.to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def test_widen_f32_exact():
    x = np.random.default_rng(3).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.widen(x, "f32"), x.astype(np.float64))


# -- brute force --------------------------------------------------------------

def _np_dtype(dtype):
    return {"f32": np.float32, "f16": np.float16}.get(dtype)


def _to64(t, dtype):
    if dtype == "bf16":
        return t.to(torch.float64).numpy()
    return t.numpy().astype(np.float64)


def brute_force(q, kp, vp, table, ctx, scale, dtype):
    """Rebuild each sequence's contiguous K/V position by position from the
    pool, then softmax attention with scipy. Query head h reads KV head
    h // (Hq/Hkv) via np.repeat over the head axis."""
    q64, k64, v64 = _to64(q, dtype), _to64(kp, dtype), _to64(vp, dtype)
    n, hkv, b, d = k64.shape
    s_, hq, _ = q64.shape
    out = np.zeros((s_, hq, d))
    for s in range(s_):
        L = int(ctx[s])
        if L == 0:
            continue
        K = np.empty((hkv, L, d))
        V = np.empty((hkv, L, d))
        for t in range(L):
            blk = int(table[s][t // b])
            K[:, t] = k64[blk, :, t % b]
            V[:, t] = v64[blk, :, t % b]
        Kq = np.repeat(K, hq // hkv, axis=0)
        Vq = np.repeat(V, hq // hkv, axis=0)
        for h in range(hq):
            w = softmax(np.float64(scale) * (Kq[h] @ q64[s, h]))
            out[s, h] = w @ Vq[h]
    return out


def _random_case(rng, dtype, hq, hkv, d, b, lens, extra_blocks=3):
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
    td = W._torch_dtype(dtype)
    g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
    q = torch.randn(len(lens), hq, d, generator=g).to(td)
    kp = torch.randn(n, hkv, b, d, generator=g).to(td)
    vp = torch.randn(n, hkv, b, d, generator=g).to(td)
    return q, kp, vp, table, np.array(lens, np.int32)


@pytest.mark.parametrize("seed", range(12))
def test_attention_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    dtype = ["f32", "f16", "bf16"][seed % 3]
    hkv = int(rng.choice([1, 2, 3]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([1, 4, 8, 16]))
    b = int(rng.choice([1, 2, 4]))
    lens = [int(x) for x in rng.integers(0, 41, size=int(rng.integers(1, 5)))]
    lens[0] = max(lens[0], 1)
    q, kp, vp, table, ctx = _random_case(rng, dtype, hq, hkv, d, b, lens)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    got = oracle.attention(q, kp, vp, table, ctx, scale, dtype)
    want = brute_force(q, kp, vp, table, ctx, scale, dtype)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    got_t = oracle.attention(q, kp, vp, table, ctx, scale, dtype, threads=3)
    assert np.array_equal(got, got_t)


# -- the glossary page's worked example ----------------------------------------

def _page_contiguous(batch, t):
    """Each sequence's contiguous K and V [Hkv, L, D], rebuilt position by
    position from the page's tables (brute force, no oracle code)."""
    B = batch.block_size
    out = []
    for s, L in enumerate(batch.context_lens):
        rows = [int(batch.block_table[s][p // B]) for p in range(int(L))]
        k = torch.stack([t["k_cache"][r, :, p % B] for p, r in enumerate(rows)], 1)
        v = torch.stack([t["v_cache"][r, :, p % B] for p, r in enumerate(rows)], 1)
        out.append((k, v))
    return out


def test_page_example_paged_equals_contiguous(golden):
    """The glossary page's experiment: attention through the page tables
    equals attention over the contiguous histories, max abs diff 0.000e+00
    as printed, and standard fp32 attention agrees within the page's
    tolerance; the two sequences share their first block (same K and V for
    positions 0..3) and V there is 0.5 x K."""
    g = golden("sharing.json")
    batch = W.tiny_page_example()
    t = W.layer_tensors(batch, poison=False)
    scale = float(np.float32(1.0 / math.sqrt(batch.head_size)))
    cont = _page_contiguous(batch, t)
    assert torch.equal(cont[0][0][:, :4], cont[1][0][:, :4])
    assert torch.equal(cont[0][1][:, :4], cont[1][1][:, :4])
    assert torch.equal(cont[0][1][:, :4], 0.5 * cont[0][0][:, :4])
    for s, L in enumerate(batch.context_lens):
        k, v = oracle.gather(t["k_cache"], t["v_cache"], batch.block_table[s], int(L), "f32")
        assert np.array_equal(k, cont[s][0].double().numpy())
        assert np.array_equal(v, cont[s][1].double().numpy())
    paged = oracle.attention(t["q"], t["k_cache"], t["v_cache"], batch.block_table,
                             batch.context_lens, scale, "f32")
    G = batch.num_heads // batch.num_kv_heads
    for s, L in enumerate(batch.context_lens):
        L = int(L)
        kc, vc = cont[s]
        # contiguous attention: the same oracle over a pool of L one-slot
        # blocks laid out in position order (identity table)
        kd = kc.permute(1, 0, 2).unsqueeze(2).contiguous()
        vd = vc.permute(1, 0, 2).unsqueeze(2).contiguous()
        dense = oracle.attention(t["q"][s:s + 1], kd, vd, np.arange(L, dtype=np.int32)[None],
                                 np.array([L], np.int32), scale, "f32")
        assert np.abs(paged[s] - dense[0]).max() == g["max_attention_abs_diff"]
        # standard fp32 softmax attention, query head h on KV head h // G
        for h in range(batch.num_heads):
            w = torch.softmax((kc[h // G] @ t["q"][s, h]) / math.sqrt(batch.head_size), 0)
            ref = (w[:, None] * vc[h // G]).sum(0)
            np.testing.assert_allclose(paged[s, h], ref.double().numpy(), rtol=1e-5, atol=1e-6)


def test_page_example_poisoned_slots_unread():
    """NaN in every slot no live token uses changes nothing (masking reads
    only positions < ctx and table entries < ceil(ctx/B))."""
    batch = W.tiny_page_example()
    clean = W.layer_tensors(batch, poison=False)
    dirty = W.layer_tensors(batch, poison=True)
    assert torch.isnan(dirty["k_cache"]).any()
    scale = float(np.float32(1.0 / math.sqrt(8)))
    a = oracle.attention(clean["q"], clean["k_cache"], clean["v_cache"], batch.block_table,
                         batch.context_lens, scale, "f32")
    b = oracle.attention(dirty["q"], dirty["k_cache"], dirty["v_cache"], batch.block_table,
                         batch.context_lens, scale, "f32")
    assert np.array_equal(a, b)


def test_gather_invariant_under_block_permutation():
    """Moving physical blocks (and fixing the table) leaves the gathered
    sequence unchanged: logical order comes from the table alone."""
    rng = np.random.default_rng(7)
    q, kp, vp, table, ctx = _random_case(rng, "f16", 4, 2, 8, 4, [13, 9])
    n = kp.shape[0]
    perm = rng.permutation(n)            # new block id of old block i is perm[i]
    kp2 = torch.empty_like(kp)
    vp2 = torch.empty_like(vp)
    kp2[torch.as_tensor(perm)] = kp
    vp2[torch.as_tensor(perm)] = vp
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
    for s in range(2):
        a = oracle.gather(kp, vp, table[s], int(ctx[s]), "f16")
        b = oracle.gather(kp2, vp2, table2[s], int(ctx[s]), "f16")
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_gather_rejects_bad_table_entry():
    kp = torch.zeros(3, 1, 2, 4)
    with pytest.raises(RuntimeError):
        oracle.gather(kp, kp, np.array([0, 5], np.int32), 3, "f32")
    with pytest.raises(RuntimeError):
        oracle.gather(kp, kp, np.array([0, -1], np.int32), 3, "f32")


# -- closed forms -------------------------------------------------------------

def _one_seq(K, V, q, b=4, dtype="f32"):
    """Pool/table for one sequence with contiguous K, V [Hkv, L, D] laid into
    blocks 1, 3, 5, ... (non-contiguous on purpose)."""
    hkv, L, d = K.shape
    nb = max(1, -(-L // b))
    ids = [2 * i + 1 for i in range(nb)]
    kp = torch.full((2 * nb + 1, hkv, b, d), float("nan"))
    vp = torch.full_like(kp, float("nan"))
    for t in range(L):
        kp[ids[t // b], :, t % b] = K[:, t]
        vp[ids[t // b], :, t % b] = V[:, t]
    return q[None], kp, vp, np.array([ids], np.int32), np.array([L], np.int32)


def test_single_position_returns_its_value():
    g = torch.Generator().manual_seed(1)
    K, V, q = torch.randn(2, 1, 8, generator=g), torch.randn(2, 1, 8, generator=g), torch.randn(4, 8, generator=g)
    args = _one_seq(K, V, q)
    out = oracle.attention(*args, 0.35, "f32")[0]
    for h in range(4):
        assert np.array_equal(out[h], V[h // 2, 0].double().numpy())


def test_zero_query_or_equal_keys_give_mean_of_values():
    g = torch.Generator().manual_seed(2)
    V = torch.randn(1, 11, 8, generator=g)
    K = torch.randn(1, 11, 8, generator=g)
    out = oracle.attention(*_one_seq(K, V, torch.zeros(1, 8)), 0.35, "f32")[0, 0]
    np.testing.assert_allclose(out, V[0].double().numpy().mean(0), rtol=0, atol=1e-15)
    Keq = K[:, :1].expand(1, 11, 8).contiguous()
    out = oracle.attention(*_one_seq(Keq, V, torch.randn(1, 8, generator=g)), 0.35, "f32")[0, 0]
    np.testing.assert_allclose(out, V[0].double().numpy().mean(0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("a", [-9.0, -1.5, 0.0, 0.7, 3.0, 12.0])
def test_two_positions_give_logistic(a):
    """k0 = a e0, k1 = 0, v0 = 1, v1 = 0, q = e0: out = sigmoid(scale * a)."""
    d = 4
    K = torch.zeros(1, 2, d)
    K[0, 0, 0] = a
    V = torch.zeros(1, 2, d)
    V[0, 0] = 1.0
    q = torch.zeros(1, d)
    q[0, 0] = 1.0
    scale = float(np.float32(0.5))
    out = oracle.attention(*_one_seq(K, V, q, b=1), scale, "f32")[0, 0]
    a32 = float(np.float32(a))          # the value the fp32 pool stores
    np.testing.assert_allclose(out, np.full(d, expit(scale * a32)), rtol=1e-14, atol=1e-300)


def test_query_head_group_map():
    """KV head j holds V == j + 1 everywhere: query head h must return
    h // (Hq/Hkv) + 1 (consecutive query heads share a KV head)."""
    hkv, G, L, d = 3, 4, 9, 8
    g = torch.Generator().manual_seed(4)
    K = torch.randn(hkv, L, d, generator=g)
    V = torch.stack([torch.full((L, d), float(j + 1)) for j in range(hkv)])
    q = torch.randn(hkv * G, d, generator=g)
    out = oracle.attention(*_one_seq(K, V, q), 0.35, "f32")[0]
    for h in range(hkv * G):
        np.testing.assert_allclose(out[h], h // G + 1, rtol=1e-15)


def test_score_shift_invariance():
    """Adding c*q_dir to every key adds the same c*|q|^2 to every score:
    the output must not move."""
    g = torch.Generator().manual_seed(5)
    # multiples of 2^-10 with |K| < 8: K and K + 2 are both exact in fp32
    K = torch.round(torch.randn(1, 17, 8, generator=g, dtype=torch.float64) * 1024) / 1024
    V = torch.randn(1, 17, 8, generator=g)
    q = torch.zeros(1, 8)
    q[0, :] = 0.5                       # exact in fp32
    a = oracle.attention(*_one_seq(K.float(), V, q), 0.25, "f32")
    b = oracle.attention(*_one_seq((K + 2.0).float(), V, q), 0.25, "f32")
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_zero_length_gives_zero_output():
    q = torch.randn(2, 2, 4)
    kp = torch.full((2, 1, 4, 4), float("nan"))
    table = np.array([[0, 1], [-1, -1]], np.int32)
    ctx = np.array([3, 0], np.int32)
    kp[0, :, :3] = 1.0
    out = oracle.attention(q, kp, kp, table, ctx, 0.5, "f32")
    assert np.array_equal(out[1], np.zeros((2, 4)))
    assert np.isfinite(out[0]).all()


# -- partials and their merge -------------------------------------------------

@pytest.mark.parametrize("P", [1, 4, 8, 12, 64])
def test_partials_merge_equals_whole(P):
    rng = np.random.default_rng(11)
    q, kp, vp, table, ctx = _random_case(rng, "bf16", 8, 2, 16, 4, [1, 9, 33, 40, 0])
    scale = float(np.float32(0.25))
    mp = max(1, -(-int(ctx.max()) // P))
    m, l, o = oracle.attention_partials(q, kp, vp, table, ctx, scale, "bf16", P, mp)
    whole = oracle.attention(q, kp, vp, table, ctx, scale, "bf16")
    merged = oracle.lse_combine(m, l, o, ctx, P)
    np.testing.assert_allclose(merged, whole, rtol=1e-12, atol=1e-13)
    for s, L in enumerate(ctx):
        n_p = -(-int(L) // P)
        assert np.isneginf(m[s, :, n_p:]).all() and (l[s, :, n_p:] == 0).all()
        assert (o[s, :, n_p:] == 0).all()
    # permuting the partitions a sequence has changes nothing
    s = 3
    n_p = -(-int(ctx[s]) // P)
    perm = rng.permutation(n_p)
    m2, l2, o2 = m.copy(), l.copy(), o.copy()
    m2[s, :, :n_p], l2[s, :, :n_p], o2[s, :, :n_p] = m[s][:, perm], l[s][:, perm], o[s][:, perm]
    np.testing.assert_allclose(oracle.lse_combine(m2, l2, o2, ctx, P), merged, rtol=1e-13,
                               atol=1e-14)


def test_single_partition_is_whole_context():
    rng = np.random.default_rng(12)
    q, kp, vp, table, ctx = _random_case(rng, "f16", 4, 4, 8, 4, [21])
    scale = float(np.float32(0.3))
    m, l, o = oracle.attention_partials(q, kp, vp, table, ctx, scale, "f16", 64, 1)
    whole = oracle.attention(q, kp, vp, table, ctx, scale, "f16")
    np.testing.assert_allclose(o[:, :, 0], whole, rtol=1e-13, atol=1e-14)
    # m is the largest score; l = sum exp(z - m) (brute force)
    k, _ = oracle.gather(kp, vp, table[0], 21, "f16")
    q64 = q.to(torch.float64).numpy()
    for h in range(4):
        z = np.float64(scale) * (k[h] @ q64[0, h])
        assert m[0, h, 0] == pytest.approx(z.max(), rel=1e-14)
        assert l[0, h, 0] == pytest.approx(np.exp(z - z.max()).sum(), rel=1e-13)


def test_one_token_partitions():
    """P = 1: each partition holds one position, so m_p = z_p, l_p = 1 and
    o_p = v_p."""
    rng = np.random.default_rng(13)
    q, kp, vp, table, ctx = _random_case(rng, "f32", 2, 1, 4, 2, [5])
    m, l, o = oracle.attention_partials(q, kp, vp, table, ctx, 0.5, "f32", 1, 5)
    k, v = oracle.gather(kp, vp, table[0], 5, "f32")
    q64 = q.double().numpy()
    for h in range(2):
        np.testing.assert_allclose(m[0, h], 0.5 * (k[0] @ q64[0, h]), rtol=1e-14)
        assert (l[0, h] == 1.0).all()
        assert np.array_equal(o[0, h], v[0])


def test_lse_combine_closed_forms():
    o = np.random.default_rng(14).standard_normal((1, 1, 2, 6))
    ctx = np.array([2], np.int32)
    # equal maxima and sums: the plain average
    out = oracle.lse_combine(np.zeros((1, 1, 2)), np.ones((1, 1, 2)) * 5, o, ctx, 1)
    np.testing.assert_allclose(out[0, 0], o[0, 0].mean(0), rtol=1e-15)
    # m0 = m1 + ln 3 with equal l: weights 3 : 1
    m = np.array([[[math.log(3.0) + 1.0, 1.0]]])
    out = oracle.lse_combine(m, np.ones((1, 1, 2)), o, ctx, 1)
    np.testing.assert_allclose(out[0, 0], 0.75 * o[0, 0, 0] + 0.25 * o[0, 0, 1], rtol=1e-14)
    # l weights: l0 = 1, l1 = 3 with equal m: weights 1 : 3
    out = oracle.lse_combine(np.zeros((1, 1, 2)), np.array([[[1.0, 3.0]]]), o, ctx, 1)
    np.testing.assert_allclose(out[0, 0], 0.25 * o[0, 0, 0] + 0.75 * o[0, 0, 1], rtol=1e-14)
    # a sequence with no partitions gives zero and reads nothing
    nan = np.full((1, 1, 2), np.nan)
    out = oracle.lse_combine(nan, nan, np.full((1, 1, 2, 6), np.nan), np.array([0], np.int32), 1)
    assert (out == 0).all()
