"""Random decode batches through the split kernel against the fp64 oracle.

Each seeded case draws a geometry (block size 16/32/64, 1-8 query heads per
KV head, f16 or bf16, head size 128: the matrix-core path), a length mix
(empty, single-tile and long sequences side by side), groups of sequences
that share leading blocks (runs of 1 to 8 blocks, members that diverge
early or end inside the run), a partition size and a workspace at or above
the smallest that fits; then runs the split call + paged_attention_reduce
and the merged call (twice on the same counters, which it leaves at zero)
and compares both with the oracle within 2e-3. The cases reach the split's
every branch: ranges weighted by shared runs, sequences cut into the
workspace's last slot, waves with no range."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_cases import TOL, device_meta, gpu_attention, host, max_err, oracle_attention, scale_of

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def pkv(dev):
    import paged_kv_cache_113_amd as m
    return m


def _case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([16, 32, 64]))
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4]))
    dtype = str(rng.choice(["bf16", "f16"]))
    S = int(rng.integers(1, 121))
    kind = rng.integers(0, 4, size=S)
    lens = np.where(kind == 0, 0, np.where(kind == 1, rng.integers(1, 17, size=S),
                                           rng.integers(1, 1500, size=S)))
    need = int(sum(-(-int(n) // B) for n in lens)) + 64
    free = [int(x) for x in rng.permutation(need)]
    rows = [None] * S
    order = rng.permutation(S)
    pos = 0
    for _ in range(int(rng.integers(0, 5))):        # sharing groups
        members = [int(x) for x in order[pos:pos + int(rng.integers(2, 7))]]
        pos += len(members)
        if len(members) < 2:
            break
        run = int(rng.integers(1, 9))
        shared, free = free[:run], free[run:]
        for m in members:
            if lens[m] == 0:
                lens[m] = int(rng.integers(1, (run + 3) * B))
            nb = -(-int(lens[m]) // B)
            keep = run if rng.random() < 0.8 else int(rng.integers(1, run + 1))
            own, free = free[:max(0, nb - keep)], free[max(0, nb - keep):]
            rows[m] = (shared[:keep] + own)[:nb]
    for s in range(S):
        if rows[s] is None:
            nb = -(-int(lens[s]) // B)
            rows[s], free = free[:nb], free[nb:]
    width = max(1, max(len(r) for r in rows))
    table = np.full((S, width), -1, np.int32)
    for s, r in enumerate(rows):
        table[s, :len(r)] = r
    b = W.Batch(name=f"random_split_{seed}", dtype=dtype, num_heads=G * hkv, num_kv_heads=hkv,
                head_size=128, block_size=B, num_blocks=need, block_table=table,
                context_lens=lens.astype(np.int32), free_order=np.arange(need, dtype=np.int32),
                seed=7000 + seed)
    longest = max(1, int(lens.max()))
    P = B * int(rng.integers(1, max(2, -(-longest // B) + 1)))
    mp = b.max_partitions(P) + int(rng.choice([0, 0, 1, 3]))
    return b, P, mp


@pytest.mark.parametrize("seed", range(48))
def test_random_decode_split(dev, pkv, seed):
    b, P, mp = _case(seed)
    say(f"case: random split seed={seed} S={b.num_seqs} B={b.block_size} Hq={b.num_heads} "
        f"Hkv={b.num_kv_heads} {b.dtype} P={P} mp={mp} max_len={int(b.context_lens.max())}")
    t = W.layer_tensors(b, device=dev)
    th = host(t)
    want = oracle_attention(b, th["q"], th["k_cache"], th["v_cache"])
    meta = device_meta(b, dev)
    got = gpu_attention(pkv, b, t, meta, dev, P, mp)
    torch.cuda.synchronize()
    e = max_err(got.cpu(), want)
    say(f"  split + reduce: max abs err {e:.3e}")
    assert e <= TOL
    counters = torch.zeros(b.num_seqs * b.num_kv_heads, dtype=torch.int32, device=dev)
    shape = (b.num_seqs, b.num_heads, mp)
    for rep in range(2):
        out = torch.full((b.num_seqs, b.num_heads, b.head_size), float("nan"), device=dev)
        ml = torch.full(shape, float("nan"), device=dev)
        es = torch.full(shape, float("nan"), device=dev)
        to = torch.full(shape + (b.head_size,), float("nan"), device=dev)
        pkv.paged_decode_attention_merged(out, t["q"], t["k_cache"], t["v_cache"], meta["table"],
                                          meta["ctx"], scale_of(b), P, mp, ml, es, to, counters)
        torch.cuda.synchronize()
        e = max_err(out.cpu(), want)
        say(f"  merged (call {rep + 1}): max abs err {e:.3e}")
        assert e <= TOL
        assert int(counters.abs().sum()) == 0
