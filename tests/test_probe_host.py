"""The bench's read-stream probe library loads and rejects bad arguments on
the host, before any HIP call (no GPU needed)."""
import ctypes

P = ctypes.c_void_p(16)   # a non-NULL pointer that is never dereferenced


def test_probe_validation():
    import bench
    f = bench.probe_lib().pkvprobe_read_stream
    blk = 8 * 4096
    assert f(P, P, blk * 4 + 4096, P, 8, 8, 1, 1, P, None) == -2   # not whole blocks
    assert f(P, P, 0, P, 8, 8, 1, 1, P, None) == -2
    assert f(P, P, blk, P, -1, 8, 1, 1, P, None) == -2
    assert f(P, P, blk, P, 8, 0, 1, 1, P, None) == -2
    assert f(P, P, blk, P, 8, 8, 0, 1, P, None) == -2
    assert f(P, P, blk, P, 8, 8, 1, 3, P, None) == -2
    assert f(P, P, blk, P, 0, 8, 1, 1, P, None) == 0                # nothing to read
    assert f(None, P, blk, P, 8, 8, 1, 1, P, None) == -1
    assert f(P, P, blk, None, 8, 8, 1, 1, P, None) == -1
    assert f(P, P, blk, P, 8, 8, 1, 1, None, None) == -1
