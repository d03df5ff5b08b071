"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bit-exact: slot mapping, the K/V write, the block-table gather.
Attention: max abs error <= 2e-3 against fp64 (the bar for fp16/bf16 KV with
fp32 accumulation), unsplit and split + merge, at sizes the oracle checks
element by element (several tiles, ragged tails) and at the full workload
sizes on every sequence, in the launch configurations the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_cases import (TOL, device_meta, gpu_attention, gpu_write, host, max_err,
                       oracle_attention, oracle_pools_after_write, oracle_slots, scale_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def pkv(dev):
    import paged_kv_cache_113_amd as m
    return m


def say(*a):
    print(*a, flush=True)


SMALL = {
    "mha_fp16": lambda: W.mha_fp16(num_seqs=6, lo=1, hi=300),
    "gqa_shared_bf16": lambda: W.gqa_shared_bf16(num_seqs=24, median=200.0, prefix_blocks=4),
    "long_split_bf16": lambda: W.long_split_bf16(num_seqs=2, lo=1500, hi=3000),
    "decode_step_bf16": lambda: W.decode_step_bf16(num_seqs=32, lo=1, hi=200, num_layers=1),
    "gqa8_f16": lambda: W._uniform_case("gqa8_f16", "f16", 64, 8, 128, 32, 5, 1, 700, 77),
    "gqa16_bf16": lambda: W._uniform_case("gqa16_bf16", "bf16", 32, 2, 128, 64, 4, 1, 500, 78),
    "gqa3_bf16": lambda: W._uniform_case("gqa3_bf16", "bf16", 12, 4, 128, 16, 5, 1, 300, 79),
    "plain_f32_d64": lambda: W._uniform_case("plain_f32", "f32", 8, 2, 64, 8, 4, 1, 100, 80),
    "plain_bf16_d96": lambda: W._uniform_case("plain_bf16", "bf16", 6, 3, 96, 4, 4, 1, 90, 81),
}


def test_tiny_page_example(dev, pkv):
    say("case: tiny page example, unsplit and split P=4, 8")
    b = W.tiny_page_example()
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    th = host(t)
    want = oracle_attention(b, th["q"], th["k_cache"], th["v_cache"])
    for P in (0, 4, 8):
        got = gpu_attention(pkv, b, t, meta, dev, P)
        torch.cuda.synchronize()
        e = max_err(got.cpu(), want)
        say(f"  P={P}: max abs err {e:.3e}")
        assert e <= TOL


def test_tiny_page_example_paged_equals_contiguous_bitwise(dev, pkv):
    """The glossary page's experiment on the GPU (its plain kernel: fp32,
    D = 8, B = 4): attention through the page tables equals attention over
    the same histories laid out contiguously (each sequence's positions in
    consecutive blocks of its own, identity order), max abs diff 0 as the page
    prints; and moving the physical blocks (rewriting the tables) changes no
    output bit either."""
    say("case: tiny page example, paged vs contiguous, bitwise")
    b = W.tiny_page_example()
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    B = b.block_size
    # contiguous layout: sequence s's position p in block base_s + p // B
    width = b.max_blocks
    ck = torch.zeros((b.num_seqs * width,) + tuple(t["k_cache"].shape[1:]), device=dev)
    cv = torch.zeros_like(ck)
    ctab = torch.full((b.num_seqs, width), -1, dtype=torch.int32)
    for s, L in enumerate(b.context_lens):
        for p in range(int(L)):
            src = int(b.block_table[s][p // B])
            ck[s * width + p // B, :, p % B] = t["k_cache"][src, :, p % B]
            cv[s * width + p // B, :, p % B] = t["v_cache"][src, :, p % B]
            ctab[s, p // B] = s * width + p // B
    cmeta = dict(meta, table=ctab.to(dev))
    perm = torch.randperm(b.num_blocks, generator=torch.Generator().manual_seed(53)).to(dev)
    pk = torch.empty_like(t["k_cache"])
    pv = torch.empty_like(t["v_cache"])
    pk[perm] = t["k_cache"]
    pv[perm] = t["v_cache"]
    ptab = torch.where(meta["table"] >= 0, perm[meta["table"].clamp(min=0).long()].int(),
                       meta["table"]).contiguous()
    for P in (0, 4, 8):
        paged = gpu_attention(pkv, b, t, meta, dev, P)
        cont = gpu_attention(pkv, b, dict(t, k_cache=ck, v_cache=cv), cmeta, dev, P)
        moved = gpu_attention(pkv, b, dict(t, k_cache=pk, v_cache=pv), dict(meta, table=ptab),
                              dev, P)
        torch.cuda.synchronize()
        diff = float((paged - cont).abs().max())
        say(f"  P={P}: max abs diff paged vs contiguous {diff:.3e}")
        assert diff == 0.0 and torch.equal(paged, cont)
        assert torch.equal(paged, moved)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_attention_small(dev, pkv, name):
    b = SMALL[name]()
    say(f"case: {name} S={b.num_seqs} ctx={b.context_lens.min()}..{b.context_lens.max()}")
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    th = host(t)
    if b.positions is not None:
        k, v, _ = oracle_pools_after_write(b, th)
        gpu_write(pkv, b, t, meta, dev)
    else:
        k, v = th["k_cache"], th["v_cache"]
    want = oracle_attention(b, th["q"], k, v)
    for P in (0, b.block_size, 2 * b.block_size, 512 - 512 % b.block_size):
        got = gpu_attention(pkv, b, t, meta, dev, P)
        torch.cuda.synchronize()
        e = max_err(got.cpu(), want)
        say(f"  P={P}: max abs err {e:.3e}")
        assert e <= TOL, (name, P, e)


def test_slot_mapping_bit_exact(dev, pkv):
    b = W.decode_step_bf16(num_layers=1)
    say(f"case: slot mapping, decode step S={b.num_seqs}")
    meta = device_meta(b, dev)
    slots = torch.empty(b.num_seqs, dtype=torch.int64, device=dev)
    pkv.paged_slot_mapping(slots, meta["table"], meta["pos"], b.block_size)
    torch.cuda.synchronize()
    assert slots.cpu().tolist() == oracle_slots(b)
    # positions the table cannot cover, or negative ones, give -1
    pos = torch.tensor([-1, 0, b.max_blocks * b.block_size, 5], dtype=torch.int32, device=dev)
    tab = meta["table"][:4].clone()
    tab[3, 0] = -1
    s4 = torch.empty(4, dtype=torch.int64, device=dev)
    pkv.paged_slot_mapping(s4, tab, pos, b.block_size)
    torch.cuda.synchronize()
    row1 = b.block_table[1]
    assert s4.cpu().tolist() == [-1, int(row1[0]) * b.block_size, -1, -1]


@pytest.mark.parametrize("full", [False, True])
def test_kv_write_bit_exact(dev, pkv, full):
    b = W.decode_step_bf16(num_layers=1) if full else SMALL["decode_step_bf16"]()
    say(f"case: kv write S={b.num_seqs} blocks={b.num_blocks}")
    t = W.layer_tensors(b, device=dev)
    th = host(t)
    k, v, slots = oracle_pools_after_write(b, th)
    meta = device_meta(b, dev)
    gpu_write(pkv, b, t, meta, dev)
    torch.cuda.synchronize()
    assert np.array_equal(oracle._raw(t["k_cache"].cpu(), b.dtype), k)
    assert np.array_equal(oracle._raw(t["v_cache"].cpu(), b.dtype), v)


def test_kv_write_skips_negative_and_out_of_pool_slots(dev, pkv):
    say("case: kv write with skipped slots")
    pool = torch.zeros(4, 2, 4, 8, dtype=torch.float16, device=dev)
    vpool = torch.zeros_like(pool)
    new = torch.arange(3 * 2 * 8, dtype=torch.float16, device=dev).reshape(3, 2, 8) + 1
    slots = torch.tensor([5, -1, 16], dtype=torch.int64, device=dev)   # 16 = 4 blocks * 4
    pkv.paged_kv_write(pool, vpool, new, new, slots)
    torch.cuda.synchronize()
    want = np.zeros((4, 2, 4, 8), np.float16)
    want = oracle.scatter.scatter(want, new.cpu().numpy(), [5, -1, -1])
    assert np.array_equal(pool.cpu().numpy().view(np.int16), want.view(np.int16))


@pytest.mark.parametrize("name", ["mha_fp16", "gqa_shared_bf16", "long_split_bf16",
                                  "plain_f32_d64", "plain_bf16_d96"])
def test_gather_bit_exact(dev, pkv, name):
    b = SMALL[name]() if name in SMALL else None
    say(f"case: gather {name}")
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    mc = int(b.context_lens.max())
    shape = (b.num_seqs, b.num_kv_heads, mc, b.head_size)
    ko = torch.zeros(shape, dtype=t["k_cache"].dtype, device=dev)
    vo = torch.zeros_like(ko)
    pkv.paged_kv_gather(ko, vo, t["k_cache"], t["v_cache"], meta["table"], meta["ctx"])
    torch.cuda.synchronize()
    th = host(t)
    kg = oracle.widen(ko.cpu(), b.dtype)
    vg = oracle.widen(vo.cpu(), b.dtype)
    for s, L in enumerate(b.context_lens):
        k, v = oracle.gather(th["k_cache"], th["v_cache"], b.block_table[s], int(L), b.dtype)
        assert np.array_equal(kg[s, :, :L], k) and np.array_equal(vg[s, :, :L], v)
        assert (kg[s, :, L:] == 0).all()      # rows past ctx untouched


def test_reduce_random_partials(dev, pkv):
    say("case: reduce on synthetic partials")
    S, H, D, P, Psz = 7, 5, 128, 9, 64
    ctx = np.array([0, 1, 64, 65, 300, 576, 577], np.int32)   # 577 -> 10 > P partitions
    m, l, o = W.random_partials(S, H, D, P, ctx, Psz, seed=5)
    out = torch.empty(S, H, D, device=dev)
    pkv.paged_attention_reduce(out, m.to(dev), l.to(dev), o.to(dev),
                               torch.as_tensor(ctx, device=dev), Psz)
    torch.cuda.synchronize()
    # the merge clamps to max_partitions: give the oracle the same clamp
    want = oracle.lse_combine(m.double().numpy(), l.double().numpy(), o.double().numpy(),
                              np.minimum(ctx, P * Psz), Psz)
    e = max_err(out.cpu(), want)
    say(f"  max abs err {e:.3e}")
    assert e <= 1e-5


@pytest.mark.parametrize("D,mp", [(64, 40), (128, 300), (256, 17), (128, 64)])
def test_reduce_many_slots(dev, pkv, D, mp):
    """More slots per row than one 16-lane round covers (the wave-per-row
    merge): rows with 0, 1, a few, more than 64 and all slots live, NaN in
    the others, against the oracle's log-sum-exp merge."""
    say(f"case: reduce with many slots D={D} mp={mp}")
    Psz = 16
    ctx = np.array([0, 1, 17 * Psz, min(mp, 70) * Psz - 5, mp * Psz, 33 * Psz + 1], np.int32)
    S, H = len(ctx), 3
    m, l, o = W.random_partials(S, H, D, mp, ctx, Psz, seed=D + mp)
    out = torch.empty(S, H, D, device=dev)
    pkv.paged_attention_reduce(out, m.to(dev), l.to(dev), o.to(dev),
                               torch.as_tensor(ctx, device=dev), Psz)
    torch.cuda.synchronize()
    want = oracle.lse_combine(m.double().numpy(), l.double().numpy(), o.double().numpy(),
                              np.minimum(ctx, mp * Psz), Psz)
    e = max_err(out.cpu(), want)
    say(f"  max abs err {e:.3e}")
    assert e <= 1e-5
    assert (out[0] == 0).all()


def test_block_permutation_is_bitwise_invariant(dev, pkv):
    """Moving physical blocks (and rewriting the table) must not change one
    output bit: the kernels see the same data in the same order."""
    b = SMALL["gqa_shared_bf16"]()
    say("case: block permutation invariance")
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    outs = [gpu_attention(pkv, b, t, meta, dev, P) for P in (0, 64)]
    perm = torch.randperm(b.num_blocks, generator=torch.Generator().manual_seed(9))
    t2 = dict(t)
    for key in ("k_cache", "v_cache"):
        x = torch.empty_like(t[key])
        x[perm.to(dev)] = t[key]
        t2[key] = x
    tab = torch.where(meta["table"] >= 0, perm.to(dev)[meta["table"].clamp(min=0).long()].int(),
                      meta["table"])
    meta2 = dict(meta, table=tab.contiguous())
    outs2 = [gpu_attention(pkv, b, t2, meta2, dev, P) for P in (0, 64)]
    torch.cuda.synchronize()
    for a, c in zip(outs, outs2):
        assert torch.equal(a, c)


def test_group_heads_with_equal_queries_agree(dev, pkv):
    b = SMALL["gqa_shared_bf16"]()
    say("case: equal queries in a head group")
    t = W.layer_tensors(b, device=dev)
    G = b.num_heads // b.num_kv_heads
    q = t["q"].view(b.num_seqs, b.num_kv_heads, G, b.head_size)
    q[:] = q[:, :, :1].clone()
    meta = device_meta(b, dev)
    out = gpu_attention(pkv, b, t, meta, dev).view(b.num_seqs, b.num_kv_heads, G, -1)
    torch.cuda.synchronize()
    assert torch.equal(out, out[:, :, :1].expand_as(out))


def test_edge_lengths(dev, pkv):
    """ctx = 0, 1, B-1, B, B+1, 16k+1 and a table entry outside the pool
    (skipped, no fault) in one batch."""
    say("case: edge lengths")
    lens = [0, 1, 15, 16, 17, 33, 257, 5]
    b = W.Batch(name="edges", dtype="bf16", num_heads=8, num_kv_heads=2, head_size=128,
                block_size=16, num_blocks=64, block_table=np.full((8, 20), -1, np.int32),
                context_lens=np.array(lens, np.int32), free_order=np.arange(64, dtype=np.int32),
                seed=4242)
    tab, _ = W.deal_tables(lens, 16, np.random.default_rng(1).permutation(64), width=20)
    b.block_table = tab
    t = W.layer_tensors(b, device=dev)
    th = host(t)
    want = oracle_attention(b, th["q"], th["k_cache"], th["v_cache"])
    meta = device_meta(b, dev)
    for P in (0, 16, 64):
        got = gpu_attention(pkv, b, t, meta, dev, P)
        torch.cuda.synchronize()
        e = max_err(got.cpu(), want)
        say(f"  P={P}: max abs err {e:.3e}")
        assert e <= TOL
        assert (got[0] == 0).all()                               # ctx 0
        kv1 = th["v_cache"][int(b.block_table[1, 0]), :, 0]       # ctx 1 returns v_0
        assert torch.equal(got[1].cpu(), kv1.float().repeat_interleave(4, 0))
    # a table entry past the pool: the sequence's other positions still count,
    # other sequences are unaffected, nothing faults
    tab2 = meta["table"].clone()
    tab2[6, 3] = b.num_blocks + 1000
    got = gpu_attention(pkv, b, t, dict(meta, table=tab2), dev)
    torch.cuda.synchronize()
    keep = [s for s in range(8) if s != 6]
    assert max_err(got.cpu()[keep], want[keep]) <= TOL
    assert torch.isfinite(got[6]).all()


# every sequence at full size; the partition sizes include the ones the
# benchmark times (256 for the MHA case, 1024 for the others)
FULL = {
    "mha_fp16": (W.mha_fp16, None, (0, 256, 512)),
    "gqa_shared_bf16": (W.gqa_shared_bf16, None, (0, 512, 1024)),
    "long_split_bf16": (W.long_split_bf16, None, (512, 1024)),
}


@pytest.mark.parametrize("name", sorted(FULL))
def test_attention_full_size(dev, pkv, name):
    make, seqs, parts = FULL[name]
    b = make()
    say(f"case: full {name} S={b.num_seqs} blocks={b.num_blocks}")
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    th = host(t)
    want = oracle_attention(b, th["q"], th["k_cache"], th["v_cache"], seqs)
    for P in parts:
        got = gpu_attention(pkv, b, t, meta, dev, P)
        torch.cuda.synchronize()
        g = got.cpu() if seqs is None else got.cpu()[list(seqs)]
        e = max_err(g, want)
        say(f"  P={P}: max abs err {e:.3e}")
        assert e <= TOL


@pytest.mark.parametrize("layer", [0, 31])
def test_decode_step_full_size_layer(dev, pkv, layer):
    """One layer of the 32-layer decode step at full size: slot mapping and
    write bit-exact; attention of all 512 sequences at partition size 1024
    (the benchmark's launch: max_partitions = ceil(max ctx / 1024)) and 512."""
    b = W.decode_step_bf16()
    say(f"case: full decode step layer {layer} S={b.num_seqs} blocks={b.num_blocks}")
    t = W.layer_tensors(b, layer=layer, device=dev)
    th = host(t)
    k, v, slots = oracle_pools_after_write(b, th)
    meta = device_meta(b, dev)
    got_slots = gpu_write(pkv, b, t, meta, dev)
    outs = {P: gpu_attention(pkv, b, t, meta, dev, P) for P in (1024, 512)}
    torch.cuda.synchronize()
    assert got_slots.cpu().tolist() == slots
    assert np.array_equal(oracle._raw(t["k_cache"].cpu(), b.dtype), k)
    assert np.array_equal(oracle._raw(t["v_cache"].cpu(), b.dtype), v)
    want = oracle_attention(b, th["q"], k, v)
    for P, out in outs.items():
        e = max_err(out.cpu(), want)
        say(f"  P={P}, all {b.num_seqs} seqs: max abs err {e:.3e}")
        assert e <= TOL


@pytest.mark.parametrize("name,P,mp_override", [
    ("gqa_shared_bf16", 64, None), ("gqa_shared_bf16", 512, None),
    ("mha_fp16", 256, 2), ("gqa8_f16", 32, 1), ("long_split_bf16", 512, None)])
def test_split_slots_contract(dev, pkv, name, P, mp_override):
    """Split mode writes every slot of every (sequence, head) with ctx >= 1:
    a partial with l >= 1 or an unused slot with l = 0 and m = -inf; at most
    max_partitions pieces; and the merge of the used slots is the attention."""
    b = SMALL[name]()
    say(f"case: split slots {name} P={P} mp={mp_override}")
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    mp = b.max_partitions(P) if mp_override is None else mp_override
    shape = (b.num_seqs, b.num_heads, mp)
    ml = torch.full(shape, float("nan"), device=dev)
    es = torch.full(shape, float("nan"), device=dev)
    to = torch.full(shape + (b.head_size,), float("nan"), device=dev)
    pkv.paged_decode_attention(None, t["q"], t["k_cache"], t["v_cache"], meta["table"],
                               meta["ctx"], scale_of(b), P, mp, ml, es, to)
    out = torch.empty(b.num_seqs, b.num_heads, b.head_size, device=dev)
    pkv.paged_attention_reduce(out, ml, es, to, meta["ctx"], P)
    torch.cuda.synchronize()
    ml, es = ml.cpu(), es.cpu()
    live = torch.as_tensor(b.context_lens > 0)
    assert not torch.isnan(es[live]).any() and not torch.isnan(ml[live]).any()
    used = es > 0
    assert (es[used] >= 1.0 - 1e-6).all()
    unused = live[:, None, None] & ~used
    assert (es[unused] == 0).all() and torch.isinf(ml[unused]).all()
    # every live (sequence, head) has at least one piece, at most mp
    assert (used.sum(-1)[live] >= 1).all() and (used.sum(-1) <= mp).all()
    th = host(t)
    want = oracle_attention(b, th["q"], th["k_cache"], th["v_cache"])
    e = max_err(out.cpu(), want)
    say(f"  max abs err {e:.3e}, pieces per (seq, head) up to {int(used.sum(-1).max())}")
    assert e <= TOL


MANY = {
    # ~16 short sequences per wave and KV head: finished pieces outgrow a
    # wave's LDS staging area and are flushed before the wave's range ends
    "short_gqa4_s4000": lambda: W._uniform_case("short_gqa4", "bf16", 32, 8, 128, 16, 4000, 1,
                                                40, 91),
    # the largest batch the split kernel takes with a group of 16 heads: the
    # prefix leaves less staging room than one piece needs, pieces go out
    # directly
    "short_gqa16_s8192": lambda: W._uniform_case("short_gqa16", "f16", 32, 2, 128, 16, 8192, 1,
                                                 40, 92),
    # one sequence past the split kernel's LDS prefix: the plain kernel's
    # partitions, aligned to multiples of the partition size
    "short_gqa4_s8193": lambda: W._uniform_case("short_gqa4", "bf16", 32, 8, 128, 16, 8193, 1,
                                                40, 93),
}


@pytest.mark.parametrize("name", sorted(MANY))
def test_split_many_pieces_per_wave(dev, pkv, name):
    """Many short sequences in split mode: every (sequence, head) within
    2e-3 of the oracle, every slot a partial (l >= 1) or marked unused."""
    b = MANY[name]()
    P = 16
    mp = b.max_partitions(P)
    say(f"case: many pieces {name} S={b.num_seqs} G={b.num_heads // b.num_kv_heads} mp={mp}")
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    shape = (b.num_seqs, b.num_heads, mp)
    ml = torch.full(shape, float("nan"), device=dev)
    es = torch.full(shape, float("nan"), device=dev)
    to = torch.full(shape + (b.head_size,), float("nan"), device=dev)
    pkv.paged_decode_attention(None, t["q"], t["k_cache"], t["v_cache"], meta["table"],
                               meta["ctx"], scale_of(b), P, mp, ml, es, to)
    out = torch.empty(b.num_seqs, b.num_heads, b.head_size, device=dev)
    pkv.paged_attention_reduce(out, ml, es, to, meta["ctx"], P)
    torch.cuda.synchronize()
    es, ml = es.cpu(), ml.cpu()
    assert not torch.isnan(es).any() and not torch.isnan(ml).any()
    used = es > 0
    assert (es[used] >= 1.0 - 1e-6).all()
    assert torch.isinf(ml[~used]).all() and (used.sum(-1) >= 1).all()
    th = host(t)
    want = oracle_attention(b, th["q"], th["k_cache"], th["v_cache"])
    e = max_err(out.cpu(), want)
    say(f"  max abs err {e:.3e}")
    assert e <= TOL


# -- split decode and its merge in one call ------------------------------------

MERGED = {
    "tiny": (W.tiny_page_example, 4),
    "mha_fp16": (SMALL["mha_fp16"], 64),
    "gqa_shared_bf16": (SMALL["gqa_shared_bf16"], 64),
    "long_split_bf16": (SMALL["long_split_bf16"], 512),
    "decode_step_bf16": (SMALL["decode_step_bf16"], 16),
    "gqa16_bf16": (SMALL["gqa16_bf16"], 64),
    "gqa3_bf16": (SMALL["gqa3_bf16"], 16),
    "plain_bf16_d96": (SMALL["plain_bf16_d96"], 8),
    "short_gqa4_s4000": (MANY["short_gqa4_s4000"], 16),
    "short_gqa16_s8192": (MANY["short_gqa16_s8192"], 16),
    "short_gqa4_s8193": (MANY["short_gqa4_s8193"], 16),
    "full_mha_fp16": (W.mha_fp16, 256),
    "full_gqa_shared_bf16": (W.gqa_shared_bf16, 1024),
    "full_long_split_bf16": (W.long_split_bf16, 1024),
}


def _merged(pkv, b, t, meta, dev, P, mp, counters):
    out = torch.full((b.num_seqs, b.num_heads, b.head_size), float("nan"), device=dev)
    shape = (b.num_seqs, b.num_heads, mp)
    ml = torch.full(shape, float("nan"), device=dev)
    es = torch.full(shape, float("nan"), device=dev)
    to = torch.full(shape + (b.head_size,), float("nan"), device=dev)
    pkv.paged_decode_attention_merged(out, t["q"], t["k_cache"], t["v_cache"], meta["table"],
                                      meta["ctx"], scale_of(b), P, mp, ml, es, to, counters)
    return out


@pytest.mark.parametrize("name", sorted(MERGED))
def test_merged_call(dev, pkv, name):
    """paged_decode_attention_merged against the oracle (2e-3) and against
    the split call + paged_attention_reduce (1e-5: the same partials, merged
    in another order); twice in a row on the same counters, which it leaves
    at zero, with bit-equal outputs."""
    make, P = MERGED[name]
    b = make()
    mp = b.max_partitions(P)
    say(f"case: merged {name} S={b.num_seqs} P={P} mp={mp}")
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    th = host(t)
    if b.positions is not None:
        k, v, _ = oracle_pools_after_write(b, th)
        gpu_write(pkv, b, t, meta, dev)
    else:
        k, v = th["k_cache"], th["v_cache"]
    counters = torch.zeros(b.num_seqs * b.num_kv_heads, dtype=torch.int32, device=dev)
    first = _merged(pkv, b, t, meta, dev, P, mp, counters)
    second = _merged(pkv, b, t, meta, dev, P, mp, counters)
    two = gpu_attention(pkv, b, t, meta, dev, P, mp)
    torch.cuda.synchronize()
    assert int(counters.abs().sum()) == 0, "counters not re-armed"
    assert torch.equal(first, second)
    want = oracle_attention(b, th["q"], k, v)
    e = max_err(first.cpu(), want)
    d = float((first - two).abs().max())
    say(f"  max abs err {e:.3e}, vs split + merge {d:.3e}")
    assert e <= TOL and d <= 1e-5


@pytest.mark.parametrize("layer", [0, 31])
def test_merged_decode_step_full_size(dev, pkv, layer):
    """The benchmark's call on a whole layer of the 32-layer decode step
    (512 sequences, partition size 1024), after the write: every sequence
    against the oracle."""
    b = W.decode_step_bf16()
    say(f"case: merged full decode step layer {layer}")
    t = W.layer_tensors(b, layer=layer, device=dev)
    th = host(t)
    k, v, _ = oracle_pools_after_write(b, th)
    meta = device_meta(b, dev)
    gpu_write(pkv, b, t, meta, dev)
    counters = torch.zeros(b.num_seqs * b.num_kv_heads, dtype=torch.int32, device=dev)
    out = _merged(pkv, b, t, meta, dev, 1024, b.max_partitions(1024), counters)
    torch.cuda.synchronize()
    assert int(counters.abs().sum()) == 0
    e = max_err(out.cpu(), oracle_attention(b, th["q"], k, v))
    say(f"  all {b.num_seqs} seqs: max abs err {e:.3e}")
    assert e <= TOL


def test_merged_edge_lengths(dev, pkv):
    """ctx = 0 rows come out zero, ctx = 1 rows equal v_0, with one and two
    slots per row."""
    lens = [0, 1, 15, 16, 17, 33, 257, 0]
    b = W.Batch(name="edges", dtype="bf16", num_heads=8, num_kv_heads=2, head_size=128,
                block_size=16, num_blocks=64, block_table=np.full((8, 20), -1, np.int32),
                context_lens=np.array(lens, np.int32), free_order=np.arange(64, dtype=np.int32),
                seed=4243)
    tab, _ = W.deal_tables(lens, 16, np.random.default_rng(2).permutation(64), width=20)
    b.block_table = tab
    say("case: merged edge lengths")
    t = W.layer_tensors(b, device=dev)
    th = host(t)
    want = oracle_attention(b, th["q"], th["k_cache"], th["v_cache"])
    meta = device_meta(b, dev)
    counters = torch.zeros(8 * 2, dtype=torch.int32, device=dev)
    for P, mp in ((16, 17), (16, 2), (64, 1)):
        got = _merged(pkv, b, t, meta, dev, P, mp, counters)
        torch.cuda.synchronize()
        e = max_err(got.cpu(), want)
        say(f"  P={P} mp={mp}: max abs err {e:.3e}")
        assert e <= TOL
        assert (got[0] == 0).all() and (got[7] == 0).all()
        kv1 = th["v_cache"][int(b.block_table[1, 0]), :, 0]
        assert torch.equal(got[1].cpu(), kv1.float().repeat_interleave(4, 0))
        assert int(counters.abs().sum()) == 0


@pytest.mark.parametrize("B", [16, 32])
def test_shared_prefix_groups(dev, pkv, B):
    """Several groups of sequences sharing leading blocks (runs of 1 to 6
    blocks, a group whose members diverge after the first block, a member
    shorter than the run, single sequences): the split kernel finds them by
    their first block, reads the shared lines ahead and weighs shared tiles
    less in its split; the output equals the oracle's, split and unsplit,
    merged in one launch or two, down to two pieces per sequence."""
    rng = np.random.default_rng(77 + B)
    N = 400
    free = [int(x) for x in rng.permutation(N)]
    rows, lens = [], []

    def take(n):
        out = free[:n]
        del free[:n]
        return out

    for run, members in ((6, 5), (1, 3), (3, 4), (2, 2)):
        shared = take(run)
        for m in range(members):
            L = int(rng.integers(1, 12 * B))
            if m == 0:
                L = max(L, run * B)          # the lowest holder covers the run
            nb = -(-L // B)
            rows.append((shared + take(max(0, nb - run)))[:nb])
            lens.append(L)
    for _ in range(6):
        L = int(rng.integers(1, 20 * B))
        rows.append(take(-(-L // B)))
        lens.append(L)
    order = rng.permutation(len(rows))
    rows = [rows[i] for i in order]
    lens = [lens[i] for i in order]
    width = max(len(r) for r in rows)
    table = np.full((len(rows), width), -1, np.int32)
    for s, r in enumerate(rows):
        table[s, :len(r)] = r
    b = W.Batch(name="shared_groups", dtype="bf16", num_heads=32, num_kv_heads=8,
                head_size=128, block_size=B, num_blocks=N, block_table=table,
                context_lens=np.array(lens, np.int32), free_order=np.arange(N, dtype=np.int32),
                seed=4244)
    say(f"case: shared prefix groups S={b.num_seqs} B={B}")
    t = W.layer_tensors(b, device=dev)
    th = host(t)
    want = oracle_attention(b, th["q"], th["k_cache"], th["v_cache"])
    meta = device_meta(b, dev)
    counters = torch.zeros(b.num_seqs * b.num_kv_heads, dtype=torch.int32, device=dev)
    # (partitions are whole blocks; the last split leaves at most two pieces
    # per sequence)
    half = -(-int(max(lens)) // 2)
    for P in (0, B, 4 * B, -(-half // B) * B):
        got = gpu_attention(pkv, b, t, meta, dev, P)
        torch.cuda.synchronize()
        e = max_err(got.cpu(), want)
        say(f"  P={P}: max abs err {e:.3e}")
        assert e <= TOL
        if P:
            m = _merged(pkv, b, t, meta, dev, P, b.max_partitions(P), counters)
            torch.cuda.synchronize()
            assert max_err(m.cpu(), want) <= TOL


# -- one decode step of one layer in one call ---------------------------------------

APPEND = {
    "decode_step_small": lambda: W.decode_step_bf16(num_seqs=32, lo=1, hi=200, num_layers=1),
    "decode_step_short": lambda: W.decode_step_bf16(num_seqs=300, lo=1, hi=40, num_layers=1),
    # ~5 and ~23 sequence ends per wave's range: the second prefetched round
    # of new rows, and the tokens past the first eight over several windows
    "decode_step_mid": lambda: W.decode_step_bf16(num_seqs=700, lo=1, hi=120, num_layers=1),
    "decode_step_many": lambda: W.decode_step_bf16(num_seqs=3000, lo=1, hi=24, num_layers=1),
    # past the split kernel's sequence capacity: write, plain split kernel,
    # merge as three launches
    "decode_step_s8193": lambda: W.decode_step_bf16(num_seqs=8193, lo=1, hi=24, num_layers=1),
    "gqa8_f16_step": lambda: W._uniform_case("gqa8_step", "f16", 64, 8, 128, 32, 7, 1, 700, 83,
                                             new_token=True),
    "plain_f32_step": lambda: W._uniform_case("plain_step", "f32", 8, 2, 64, 8, 5, 1, 100, 84,
                                              new_token=True),
}


def _append(pkv, b, t, meta, dev, P, mp, counters):
    out = torch.full((b.num_seqs, b.num_heads, b.head_size), float("nan"), device=dev)
    shape = (b.num_seqs, b.num_heads, mp)
    ml = torch.full(shape, float("nan"), device=dev)
    es = torch.full(shape, float("nan"), device=dev)
    to = torch.full(shape + (b.head_size,), float("nan"), device=dev)
    pkv.paged_decode_attention_append(out, t["q"], t["k_cache"], t["v_cache"], t["k_new"],
                                      t["v_new"], meta["table"], meta["ctx"], scale_of(b), P, mp,
                                      ml, es, to, counters)
    return out


@pytest.mark.parametrize("name", sorted(APPEND))
def test_append_call(dev, pkv, name):
    """paged_decode_attention_append: the pools afterwards are bit for bit the
    oracle's scatter of the new tokens at the oracle's slots (positions
    ctx - 1), and the output is within 2e-3 of the oracle's attention over
    them; twice in a row on the same counters (left at zero), bit-equal."""
    b = APPEND[name]()
    P = 4 * b.block_size
    mp = b.max_partitions(P)
    say(f"case: append {name} S={b.num_seqs} P={P} mp={mp}")
    t = W.layer_tensors(b, device=dev)
    th = host(t)
    k, v, _ = oracle_pools_after_write(b, th)
    meta = device_meta(b, dev)
    counters = torch.zeros(b.num_seqs * b.num_kv_heads, dtype=torch.int32, device=dev)
    first = _append(pkv, b, t, meta, dev, P, mp, counters)
    second = _append(pkv, b, t, meta, dev, P, mp, counters)
    torch.cuda.synchronize()
    bits = lambda x: np.ascontiguousarray(x).view(np.uint8)   # noqa: E731  (NaN poison)
    assert np.array_equal(bits(oracle._raw(t["k_cache"].cpu(), b.dtype)), bits(k))
    assert np.array_equal(bits(oracle._raw(t["v_cache"].cpu(), b.dtype)), bits(v))
    assert int(counters.abs().sum()) == 0
    assert torch.equal(first, second)
    e = max_err(first.cpu(), oracle_attention(b, th["q"], k, v))
    say(f"  max abs err {e:.3e}")
    assert e <= TOL


@pytest.mark.parametrize("layer", [0, 31])
def test_append_decode_step_full_size(dev, pkv, layer):
    """The benchmark's call on a whole layer of the 32-layer decode step
    (512 sequences, partition size 1024): pools bit-exact after the write,
    every sequence's attention against the oracle."""
    b = W.decode_step_bf16()
    say(f"case: append full decode step layer {layer}")
    t = W.layer_tensors(b, layer=layer, device=dev)
    th = host(t)
    k, v, _ = oracle_pools_after_write(b, th)
    meta = device_meta(b, dev)
    counters = torch.zeros(b.num_seqs * b.num_kv_heads, dtype=torch.int32, device=dev)
    out = _append(pkv, b, t, meta, dev, 1024, b.max_partitions(1024), counters)
    torch.cuda.synchronize()
    assert np.array_equal(oracle._raw(t["k_cache"].cpu(), b.dtype), k)
    assert np.array_equal(oracle._raw(t["v_cache"].cpu(), b.dtype), v)
    assert int(counters.abs().sum()) == 0
    e = max_err(out.cpu(), oracle_attention(b, th["q"], k, v))
    say(f"  all {b.num_seqs} seqs: max abs err {e:.3e}")
    assert e <= TOL
