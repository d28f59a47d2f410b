"""Build libmoe.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree, and
libmoe_probe.so (the benchmark's measured-ceiling kernels, not part of the
library's ABI).

Every translation unit is compiled with -O3 for gfx950 and with the
packed-fp32 instructions switched off; objects go to csrc/_build/ and the
libraries to the package directory, where the binding and the benchmark load
them.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe.so")
PROBE_OUT = os.path.join(PKG, "libmoe_probe.so")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["abi.hip", "router.hip", "permute.hip", "ffn_stream.hip", "ffn_fp8.hip", "ffn_tile.hip", "ffn_tile_fp8.hip", "combine.hip", "norm.hip"]
PROBE_SOURCES = ["probe.hip"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-munsafe-fp-atomics", "-I", os.path.join(PKG, "..", "include")]


def _compile(src: str, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so and libmoe_probe.so; returns
    the library path."""
    build_dir = os.path.join(CSRC, "_build")
    os.makedirs(build_dir, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, build_dir), srcs)))
    _link([objs[s] for s in SOURCES], OUT)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_OUT)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
