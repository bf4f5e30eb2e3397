"""Oracle microscaling (MX) formats: MXFP4 weights and MXFP8 activations.

TEST INFRASTRUCTURE ONLY (part of the CPU oracle; shares no code with the GPU
library).  Written from the OCP Microscaling Formats (MX) v1.0 specification:

* An MX block is 32 consecutive elements with one shared scale X = 2^(E-127)
  stored as E8M0 (an 8-bit biased exponent; E = 255 is NaN).  The value of
  element i is X * P_i.
* FP4 E2M1 elements: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit:
  magnitudes 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6; no Inf or NaN.
* FP8 E4M3 elements: as in codecs.py (largest magnitude 448).
* Conversion of a block of fp32 values V (the specification's section on
  converting to MX): shared_exp = floor(log2(max_i |V_i|)) - emax_elem, with
  emax_elem the exponent of the element format's largest normal number (2 for
  E2M1: 6 = 1.5 * 2^2; 8 for E4M3: 448 = 1.75 * 2^8); X = 2^shared_exp;
  P_i = the element nearest to V_i / X, ties to even, magnitudes above the
  largest normal clamped to it.  shared_exp is clamped to the E8M0 range
  [-127, 127]; an all-zero block takes E = 0 and zero elements.

Packing (the library's storage): E2M1 codes two per byte along K, the lower K
index in the low nibble; scales one byte per row and 32 K positions.

The pages name FP4 MoE on Blackwell as a deployment lever (the lever table of
"How DeepSeek inference works"; "The Premise That Wasn't") without a format;
MXFP4 (E2M1 + E8M0 per 32) with MXFP8 (E4M3 + E8M0 per 32) activations, the
pairing gfx950's scaled MFMA takes, is the reading here.
"""
import numpy as np

from . import codecs

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
EMAX = {"e2m1": 2, "e4m3": 8}
BLOCK = 32


def e8m0_decode(E) -> np.ndarray:
    """uint8 biased exponents -> 2^(E-127) as float64 (NaN for 255)."""
    E = np.asarray(E, dtype=np.int64)
    return np.where(E == 255, np.nan, np.ldexp(1.0, E - 127))


def e2m1_decode(codes) -> np.ndarray:
    """4-bit codes (0..15) -> float64 values: bit 3 sign, bits 2..0 magnitude index."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where((c >> 3) & 1, -1.0, 1.0) * E2M1_VALUES[c & 7]


def e2m1_encode(v) -> np.ndarray:
    """Values -> 4-bit codes: nearest magnitude, ties to the even code (the one
    with mantissa bit 0), clamped to 6; the sign of the input is kept."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 6.0)
    # distance to each representable magnitude; ties go to the code with bit 0 clear
    d = np.abs(a[..., None] - E2M1_VALUES)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    even = cand & ((np.arange(8) & 1) == 0)
    idx = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return (idx | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def mx_quant(v32: np.ndarray, elem: str):
    """Blocks of 32 along the last axis -> (element codes uint8, E8M0 uint8).
    elem: 'e2m1' (codes 0..15, one per element, unpacked) or 'e4m3'."""
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    *lead, K = v.shape
    assert K % BLOCK == 0
    vb = v.reshape(*lead, K // BLOCK, BLOCK)
    amax = np.abs(vb).max(axis=-1)
    nz = amax > 0
    shared = np.zeros(amax.shape, dtype=np.int64)
    shared[nz] = codecs._floor_log2(amax[nz]) - EMAX[elem]
    shared = np.clip(shared, -127, 127)
    E = np.where(nz, shared + 127, 0).astype(np.uint8)
    scaled = vb / np.ldexp(1.0, shared)[..., None]          # exact: division by a power of two
    codes = e2m1_encode(scaled) if elem == "e2m1" else codecs.e4m3_encode(scaled)
    return codes.reshape(*lead, K).astype(np.uint8), E


def mx_dequant(codes, E, elem: str) -> np.ndarray:
    """Inverse of mx_quant (exact)."""
    codes = np.asarray(codes)
    *lead, K = codes.shape
    dec = e2m1_decode(codes) if elem == "e2m1" else codecs.e4m3_decode(codes)
    return (dec.reshape(*lead, K // BLOCK, BLOCK) * e8m0_decode(E)[..., None]).reshape(*lead, K)


def unpack_e2m1(packed) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] 4-bit codes (low nibble = lower K index)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def mxfp4_matrix(packed, E) -> np.ndarray:
    """A stored MXFP4 matrix [rows][K/2] bytes + [rows][K/32] E8M0 -> float64 [rows][K]."""
    return mx_dequant(unpack_e2m1(packed), E, "e2m1")


def mxfp8_round_trip(v) -> np.ndarray:
    """Values as an MXFP8 (E4M3 + E8M0 per 32 along the last axis) tensor
    holds them: quantised from their fp32 value and dequantised (exact)."""
    q, E = mx_quant(np.asarray(v, dtype=np.float64).astype(np.float32), "e4m3")
    return mx_dequant(q, E, "e4m3")
