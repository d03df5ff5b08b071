"""GPU parity of multi-token (causal) attention over paged KV: the HIP
library's paged_varlen_attention against the CPU oracle, within max abs
error 2e-3 of fp64, on batches that mix fresh prefills, prefill chunks on
top of a history, speculative groups, decode tokens and sequences with no
query tokens; on the matrix-core path (16-bit, D = 128, B % 16 == 0, G <= 16,
any group size) and the plain path (fp32, other head sizes)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_cases import TOL, device_meta, gpu_varlen, host, max_err, oracle_varlen

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


def _mix(name, dtype, hq, hkv, d, b, seed, n=12, hmax=300, kinds=None):
    """Histories U{0..hmax}; query lengths cycle through the regimes: 0, 1
    (decode), 2..5 (speculative), a ragged chunk, a fresh prefill (no
    history), and chunks that span several tiles and blocks (long enough,
    at G >= 3, for the prefill kernel: >= 128 (token, head) columns)."""
    rng = np.random.default_rng(seed)
    hist = rng.integers(0, hmax, size=n, endpoint=True)
    kinds = kinds or [0, 1, 3, 4, 5, 17, 40, 1, 2, 33, 64, 1]
    q = np.array([kinds[i % len(kinds)] for i in range(n)], np.int64)
    hist[4] = 0          # a fresh prefill: the chunk is the whole context
    hist[0] = max(hist[0], 1)   # a sequence with history but no query rows
    return W._varlen_case(name, dtype, hq, hkv, d, b, hist, q, seed, rng=rng)


SMALL = {
    "bf16_g4_b16": lambda: _mix("bf16_g4_b16", "bf16", 32, 8, 128, 16, 201),
    "f16_mha_b32": lambda: _mix("f16_mha_b32", "f16", 8, 8, 128, 32, 202),
    "bf16_g8_b16": lambda: _mix("bf16_g8_b16", "bf16", 16, 2, 128, 16, 203),
    "f16_g16_b64": lambda: _mix("f16_g16_b64", "f16", 32, 2, 128, 64, 204),
    "bf16_g3_b16": lambda: _mix("bf16_g3_b16", "bf16", 12, 4, 128, 16, 205),
    # a block size that is a multiple of 16 but not a power of two
    "bf16_g4_b48": lambda: _mix("bf16_g4_b48", "bf16", 32, 8, 128, 48, 210),
    "f32_d8_b4": lambda: _mix("f32_d8_b4", "f32", 4, 2, 8, 4, 206, hmax=40),
    "bf16_d64_b8": lambda: _mix("bf16_d64_b8", "bf16", 8, 2, 64, 8, 207, hmax=100),
    # MHA: chunks of 128+ tokens reach the prefill kernel (one head per KV head)
    "f16_mha_long": lambda: _mix("f16_mha_long", "f16", 4, 4, 128, 16, 208, n=6,
                                 kinds=[1, 130, 4, 200, 127, 257]),
    # 3000 speculative groups of 4 tokens on short histories: every piece
    # fills all 16 columns and the LDS staging area holds one at a time
    "bf16_g4_spec_many": lambda: W._varlen_case(
        "bf16_g4_spec_many", "bf16", 32, 8, 128, 16,
        np.random.default_rng(209).integers(0, 60, size=3000, endpoint=True),
        np.full(3000, 4), 209),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_varlen_small(dev, pkv, name):
    b = SMALL[name]()
    detail = (f"q={b.query_lens.tolist()} ctx={b.context_lens.tolist()}" if b.num_seqs <= 64
              else f"q {b.query_lens.min()}..{b.query_lens.max()} "
                   f"ctx {b.context_lens.min()}..{b.context_lens.max()}")
    say(f"case: varlen {name} S={b.num_seqs} T={b.num_tokens} {detail}")
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    th = host(t)
    want = oracle_varlen(b, th["q"], th["k_cache"], th["v_cache"])
    for mp in (1, 2, 8, 64):
        got = gpu_varlen(pkv, b, t, meta, dev, mp)
        torch.cuda.synchronize()
        e = max_err(got.cpu(), want)
        say(f"  max_partitions={mp}: max abs err {e:.3e}")
        assert e <= TOL, (name, mp, e)


def test_varlen_growing_scores(dev, pkv):
    """K rows at position t scaled by 0.02 t: the scores' spread grows along
    the context, so a column's running max climbs many times, often by far
    more than the prefill kernel lets its reference max lag (and stays
    within it at other times), inside one piece and across pieces."""
    b = _mix("bf16_ramp", "bf16", 16, 4, 128, 16, 209, n=6, hmax=700,
             kinds=[96, 1, 40, 130, 64, 1])
    say(f"case: varlen growing scores q={b.query_lens.tolist()} ctx={b.context_lens.tolist()}")
    t = W.layer_tensors(b, device=dev)
    blk, off, fac = [], [], []
    for s in range(b.num_seqs):
        for p in range(int(b.context_lens[s])):
            blk.append(int(b.block_table[s][p // b.block_size]))
            off.append(p % b.block_size)
            fac.append(0.02 * p)
    blk = torch.as_tensor(blk, device=dev)
    off = torch.as_tensor(off, device=dev)
    fac = torch.as_tensor(fac, device=dev, dtype=torch.float32)
    kc = t["k_cache"]
    kc[blk, :, off, :] = (kc[blk, :, off, :].float() * fac[:, None, None]).to(kc.dtype)
    meta = device_meta(b, dev)
    th = host(t)
    want = oracle_varlen(b, th["q"], th["k_cache"], th["v_cache"])
    for mp in (1, 8):
        got = gpu_varlen(pkv, b, t, meta, dev, mp)
        torch.cuda.synchronize()
        e = max_err(got.cpu(), want)
        say(f"  max_partitions={mp}: max abs err {e:.3e}")
        assert e <= TOL, (mp, e)


def test_varlen_nonpositive_scale(dev, pkv):
    """A negative or zero scale is valid (softmax of the negated or of equal
    scores); the call routes it to the plain kernel."""
    b = SMALL["bf16_g4_b16"]()
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    th = host(t)
    for scale in (-0.0883883, 0.0):
        want = oracle_varlen(b, th["q"], th["k_cache"], th["v_cache"], scale=scale)
        got = gpu_varlen(pkv, b, t, meta, dev, 8, scale=scale)
        torch.cuda.synchronize()
        e = max_err(got.cpu(), want)
        say(f"case: varlen scale {scale}: max abs err {e:.3e}")
        assert e <= TOL, (scale, e)


def test_varlen_one_token_each_matches_decode(dev, pkv):
    """q_s = 1 everywhere: the same answer as decode attention (both within
    the bar of the oracle, and close to each other)."""
    b = W.decode_step_bf16(num_seqs=48, lo=1, hi=400, num_layers=1)
    b.positions = None
    b.query_lens = np.ones(b.num_seqs, np.int32)
    say(f"case: varlen with one token per sequence, S={b.num_seqs}")
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    got = gpu_varlen(pkv, b, t, meta, dev, 8)
    dec = torch.empty_like(got)
    pkv.paged_decode_attention(dec, t["q"], t["k_cache"], t["v_cache"], meta["table"],
                               meta["ctx"], float(np.float32(1 / np.sqrt(128))))
    torch.cuda.synchronize()
    th = host(t)
    want = oracle_varlen(b, th["q"], th["k_cache"], th["v_cache"])
    assert max_err(got.cpu(), want) <= TOL and max_err(dec.cpu(), want) <= TOL
    assert float((got - dec).abs().max()) <= 1e-4


def test_varlen_block_permutation_is_bitwise_invariant(dev, pkv):
    b = SMALL["bf16_g4_b16"]()
    say("case: varlen block permutation invariance")
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    a = gpu_varlen(pkv, b, t, meta, dev, 8)
    perm = torch.randperm(b.num_blocks, generator=torch.Generator().manual_seed(3)).to(dev)
    t2 = dict(t)
    for key in ("k_cache", "v_cache"):
        x = torch.empty_like(t[key])
        x[perm] = t[key]
        t2[key] = x
    tab = torch.where(meta["table"] >= 0, perm[meta["table"].clamp(min=0).long()].int(),
                      meta["table"])
    c = gpu_varlen(pkv, b, t2, dict(meta, table=tab.contiguous()), dev, 8)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


def test_varlen_first_prefill_row_is_v0(dev, pkv):
    """A fresh prefill's first row sees position 0 only: its output is v_0
    exactly (fp32 of the stored value)."""
    b = SMALL["bf16_g4_b16"]()
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    got = gpu_varlen(pkv, b, t, meta, dev, 8)
    torch.cuda.synchronize()
    s = 4
    assert b.context_lens[s] == b.query_lens[s]
    r = int(b.query_start_loc[s])
    v0 = t["v_cache"][int(b.block_table[s, 0]), :, 0].float()     # [Hkv, D]
    G = b.num_heads // b.num_kv_heads
    assert torch.equal(got[r], v0.repeat_interleave(G, 0))


FULL = {
    "spec_verify_bf16": W.spec_verify_bf16,
    "mixed_prefill_bf16": W.mixed_prefill_bf16,
}


@pytest.mark.parametrize("name", sorted(FULL))
def test_varlen_full_size(dev, pkv, name):
    """Full-size batches, in the launch configuration the benchmark times
    (max_partitions 8): every query row against the oracle."""
    b = FULL[name]()
    say(f"case: varlen full {name} S={b.num_seqs} T={b.num_tokens} blocks={b.num_blocks}")
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    got = gpu_varlen(pkv, b, t, meta, dev, 8)
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    th = host(t)
    want = oracle_varlen(b, th["q"], th["k_cache"], th["v_cache"])
    e = max_err(got.cpu(), want)
    say(f"  all {b.num_tokens} rows: max abs err {e:.3e}")
    assert e <= TOL
