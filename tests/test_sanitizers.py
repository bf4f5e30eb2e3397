"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host code (every source, with the sanitizers on its host half
only: the C ABI's argument checks, the workspace and tile-list arithmetic)
and the oracle's C
router chain are rebuilt with -fsanitize=address,undefined, and the boundary
tests (test_abi.py) and the router pins (test_oracle_route.py) run against
those builds in a child Python process with the sanitizer runtime preloaded.
No device code runs here.  A planted out-of-bounds read (one element past a
heap array) in a throwaway C function, run the same way, must be reported,
so a silent run means something."""
import os
import subprocess
import sys
import concurrent.futures as cf

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from routed_expert_ffn_04_amd import build as B  # noqa: E402

LLVM = "/opt/rocm/llvm/bin"
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = "-fsanitize=address,undefined"


def _have_toolchain():
    return os.path.exists(B.HIPCC) and os.path.exists(os.path.join(LLVM, "clang"))


pytestmark = pytest.mark.skipif(not _have_toolchain(), reason="hipcc / clang not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"


def _host_object(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    _run([B.HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xarch_host", SAN, "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-shared-libasan",
          "-Wno-unused-command-line-argument", "-I", B.INCLUDE, "-c", os.path.join(B.CSRC, src), "-o", obj])
    return obj


def _c_library(src, out, extra=()):
    _run([os.path.join(LLVM, "clang"), "-O1", "-g", "-fPIC", "-shared", SAN, "-fno-sanitize-recover=all",
          "-shared-libasan", *extra, src, "-o", out, "-lm"])
    return out


@pytest.fixture(scope="module")
def builds():
    os.makedirs(OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(_host_object, B.SOURCES))
    lib = os.path.join(OUT, "libmoe_gfx950_host_asan.so")
    _run([os.path.join(LLVM, "clang++"), "-shared", SAN, "-shared-libasan", *objs, "-L/opt/rocm/lib",
          "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    router = _c_library(os.path.join(ROOT, "oracle", "router_chain.c"),
                        os.path.join(OUT, "oracle_router_asan.so"), ("-std=c99", "-ffp-contract=off", "-mavx2", "-mfma"))
    planted = os.path.join(OUT, "planted.c")
    with open(planted, "w") as f:
        f.write("#include <stdlib.h>\n"
                "float planted_read(int n) { float* x = (float*)calloc(n, sizeof(float)); float s = 0;"
                " for (int i = 0; i <= n; ++i) s += x[i]; free(x); return s; }\n")
    planted_lib = _c_library(planted, os.path.join(OUT, "planted_asan.so"))
    rt = subprocess.run([os.path.join(LLVM, "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    assert os.path.exists(rt), rt
    return dict(lib=lib, router=router, planted=planted_lib, runtime=rt)


def _env(b):
    env = dict(os.environ)
    env.update(LD_PRELOAD=b["runtime"], MOE_GFX950_LIB=b["lib"], MOE_ORACLE_ROUTER_LIB=b["router"],
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:alloc_dealloc_mismatch=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def test_boundary_and_router_pins_under_sanitizers(builds):
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_oracle_route.py")],
                       capture_output=True, text=True, env=_env(builds), cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out


def test_planted_out_of_bounds_read_is_reported(builds):
    code = ("import ctypes, sys; L = ctypes.CDLL(sys.argv[1]); L.planted_read.restype = ctypes.c_float;"
            "L.planted_read(8)")
    env = _env(builds)
    r = subprocess.run([sys.executable, "-c", code, builds["planted"]], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]
