"""paged_varlen_attention_noalloc (the entry point for callers that cannot
allocate device memory) through the C ABI: bit for bit the output of
paged_varlen_attention with a workspace, on the same inputs and
max_partitions, and within 2e-3 of the fp64 oracle; two calls in a row, the
second with a smaller input, so that the second runs over what the first
left in the static buffer; calls beyond the buffer are refused."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_cases import TOL, device_meta, gpu_varlen, host, max_err, oracle_varlen, scale_of

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


def _noalloc(pkv, b, t, meta, dev, mp):
    out = torch.full((b.num_tokens, b.num_heads, b.head_size), float("nan"), device=dev)
    qsl = torch.as_tensor(b.query_start_loc, device=dev)
    pkv.paged_varlen_attention_noalloc(out, t["q"], t["k_cache"], t["v_cache"], meta["table"],
                                       qsl, meta["ctx"], scale_of(b), mp)
    return out


def _decode_as_varlen(num_seqs, seed):
    """Decode batches (one query token per sequence) in the decode-step
    geometry, written as multi-token calls."""
    b = W.decode_step_bf16(num_seqs=num_seqs, lo=1, hi=3000, num_layers=1, seed=seed)
    b.positions = None
    b.query_lens = np.ones(b.num_seqs, np.int32)
    return b


CASES = [
    # (first call, second call: smaller), max_partitions
    ("mixed prefill + decode, then spec verify",
     lambda: W.mixed_prefill_bf16(num_decode=60, num_prefill=3, chunk=300, hi=2000),
     lambda: W.spec_verify_bf16(num_seqs=40, draft=4, hi=1500), 8),
    ("decode 256, then decode 33",
     lambda: _decode_as_varlen(256, 31), lambda: _decode_as_varlen(33, 32), 8),
    ("spec verify 300, then mixed 20 + 1 chunk",
     lambda: W.spec_verify_bf16(num_seqs=300, draft=4, hi=2500),
     lambda: W.mixed_prefill_bf16(num_decode=20, num_prefill=1, chunk=200, hi=900), 4),
]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_noalloc_matches_workspace_call(dev, pkv, idx):
    name, first, second, mp = CASES[idx]
    say(f"case: no-alloc varlen, {name}, max_partitions {mp}")
    for which, make in (("first", first), ("second", second)):
        b = make()
        assert pkv.paged_varlen_attention_noalloc_bytes(
            b.num_tokens, b.num_heads, b.head_size, mp) <= pkv.paged_varlen_attention_noalloc_limit()
        say(f"  {which}: S={b.num_seqs} T={b.num_tokens}")
        t = W.layer_tensors(b, device=dev)
        meta = device_meta(b, dev)
        got = _noalloc(pkv, b, t, meta, dev, mp)
        ref = gpu_varlen(pkv, b, t, meta, dev, max_partitions=mp)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{which} call differs from the workspace call"
        th = host(t)
        want = oracle_varlen(b, th["q"], th["k_cache"], th["v_cache"])
        e = max_err(got.cpu(), want)
        say(f"  {which}: max abs err {e:.3e}")
        assert e <= TOL


def test_noalloc_refuses_more_than_the_buffer(dev, pkv):
    """A call whose partials exceed the static buffer is refused before any
    launch; the next call works."""
    say("case: no-alloc varlen beyond the buffer")
    b = W.spec_verify_bf16(num_seqs=16, draft=4, hi=500)
    t = W.layer_tensors(b, device=dev)
    meta = device_meta(b, dev)
    limit = pkv.paged_varlen_attention_noalloc_limit()
    mp = 1
    while pkv.paged_varlen_attention_noalloc_bytes(b.num_tokens, b.num_heads, b.head_size,
                                                   mp) <= limit:
        mp *= 2
    with pytest.raises(pkv.PagedKVError) as e:
        _noalloc(pkv, b, t, meta, dev, mp)
    assert e.value.code == -10
    got = _noalloc(pkv, b, t, meta, dev, 8)
    ref = gpu_varlen(pkv, b, t, meta, dev, max_partitions=8)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
