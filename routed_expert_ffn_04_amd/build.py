"""Compile the gfx950 HIP kernels and the C ABI into libmoe_gfx950.so (in-tree).

Every translation unit is compiled on its own (in parallel) with hipcc for
gfx950 only, then linked into one shared library next to this file.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libmoe_gfx950.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["route.hip", "permute.hip", "quant.hip", "combine.hip", "gffn.hip", "gffn_tile.hip",
           "gffn_stream.hip", "gffn_mid.hip", "gffn_big.hip", "gffn_mx.hip", "gffn_mxbig.hip", "noalloc.hip", "api.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # fixed arithmetic: no contraction besides explicit fmaf, IEEE fp32 division
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, extra=(), build_dir=BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=(), lib_path: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source and link lib_path (extra_flags: additional hipcc
    flags, e.g. -D tuning macros for experiments built elsewhere)."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, tuple(extra_flags), build_dir), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(lib_path)
    return lib_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
