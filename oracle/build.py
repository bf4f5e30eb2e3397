"""Build the oracle's C part (router logits) with the host compiler.

TEST INFRASTRUCTURE ONLY: the result is loaded by the oracle, which only the
test suite, the smoke check and the benchmark's CPU-baseline leg use.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "router_chain.c")
LIB = os.path.join(HERE, "_oracle_router.so")

# x86-64-v3 (AVX2 + FMA) so fmaf is one instruction and the e-loop vectorises;
# -ffp-contract=off: no contraction other than the explicit fmaf.
CFLAGS = ["-O3", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-mavx2", "-mfma"]


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
