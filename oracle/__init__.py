"""CPU oracle for the sparse MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import, call, link or execute anything in
this package.  It shares no code with the GPU library (no kernels, headers,
helpers, tables or pre/post-processing) and neither imports the other; the
seeded input generator (package `synth`) is the only thing both sides use.
"""
from . import codecs, moe  # noqa: F401
from .build import build  # noqa: F401
