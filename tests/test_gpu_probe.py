"""The bench's read-stream probe (libpkvprobe.so, a measurement aid outside
the attention library): it runs on every block order it can be given,
including entries outside the pools (read as block 0) and waves with no
blocks, leaves the sink alone for ordinary data, and its rate is positive
and below the HBM datasheet peak."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("blocks,n,heads,tph,wg", [(64, 0, 8, 1, 1), (64, 1, 8, 1, 1),
                                                  (64, 37, 8, 2, 2), (512, 512, 32, 1, 2),
                                                  (512, 100_000, 8, 1, 1), (8, 5, 3, 1, 2)])
def test_probe_runs_on_any_order(dev, blocks, n, heads, tph, wg):
    import bench
    print(f"case: probe over {blocks} blocks of {heads}x{tph} tiles, order of {n}, {wg} "
          "workgroups per CU", flush=True)
    nbytes = blocks * heads * tph * 4096
    k = torch.full((nbytes,), 1, dtype=torch.uint8, device=dev)
    v = torch.full((nbytes,), 2, dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(n)
    order = rng.integers(-5, blocks + 5, size=max(n, 1)).astype(np.int32)[:n]
    order_t = torch.from_numpy(order).to(dev) if n else torch.empty(0, dtype=torch.int32,
                                                                    device=dev)
    sink = torch.full((4,), 7, dtype=torch.int32, device=dev)
    bench.run_read_probe(k, v, order_t, heads, tph, wg, sink)
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [7, 7, 7, 7]


def test_probe_rate_is_plausible(dev):
    import bench
    gbs = bench.read_probe(dev, 1e9, 8, 1, 1, reps=3)
    print(f"  read-stream probe {gbs:.0f} GB/s", flush=True)
    assert 1000.0 < gbs < 8000.0
