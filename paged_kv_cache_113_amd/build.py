"""Build libpagedkv.so (gfx950) in-tree with hipcc.

Every HIP source is compiled to an object in parallel, then linked into
paged_kv_cache_113_amd/libpagedkv.so. The bench's read-stream probe is a
library of its own (paged_kv_cache_113_amd/libpkvprobe.so, from probe/),
outside the attention library's ABI. Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
LIB_PATH = os.path.join(HERE, "libpagedkv.so")
SOURCES = ["api.cpp", "cache_ops.hip", "decode_fast.hip", "decode_generic.hip", "block_ops.hip",
           "prefill.hip", "prefix_cache.cpp", "scratch.hip"]
PROBE_SOURCE = os.path.join(HERE, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(HERE, "libpkvprobe.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops (v_pk_*_f32) stay off: plain fp32 math only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in VGPRs: the attention accumulators are rescaled
    # on the VALU every tile, so AGPR-resident results would be copied back
    # and forth
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + [PROBE_SOURCE]))
    _link(objs[:-1], LIB_PATH, verbose)
    _link(objs[-1:], PROBE_LIB, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
