"""Oracle number formats: bfloat16 round-to-nearest-even and OCP FP8 E4M3FN.

TEST INFRASTRUCTURE ONLY (part of the CPU oracle; shares no code with the GPU
library).  Written from the format definitions:

* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits, the same
  exponent range as IEEE binary32; rounding is to nearest, ties to even.
* E4M3FN (OCP 8-bit floating point specification, "E4M3" encoding): 1 sign
  bit, 4 exponent bits (bias 7), 3 mantissa bits; no infinities; the single
  NaN magnitude is S.1111.111; the largest finite magnitude is
  S.1111.110 = 1.75 * 2^8 = 448; subnormals (exponent field 0) are
  m * 2^-9.  Encoding here rounds to nearest, ties to even, and saturates
  magnitudes above 448 to 448 (the sign of the input is kept, so a negative
  value that rounds to zero encodes as negative zero, code 0x80).

The pages name FP8 GEMMs and a BF16-to-FP8 cast ("DeepSeek V3/R1 Inference
Efficiency (2)", sections 1.a and 2.3.1, the "BF16->FP8" operator) but do not
spell out a format; E4M3 with fp32 block scales is the reading taken.
"""
import numpy as np

E4M3_MAX = 448.0


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for finite a > 0, exactly (frexp gives a = m 2^ex, m in [0.5, 1))."""
    _, ex = np.frexp(a)
    return ex.astype(np.int64) - 1


def bf16_rne(v) -> np.ndarray:
    """Round each value (float64 or float32) to the nearest bfloat16, ties to
    even; the result is returned as float64 holding the bfloat16 value."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    a = np.abs(v)
    nz = (a > 0) & np.isfinite(a)
    e = np.maximum(_floor_log2(a[nz]), -126)
    spacing = np.ldexp(1.0, e - 7)
    q = np.rint(a[nz] / spacing) * spacing          # np.rint: ties to even
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    q = np.where(q > max_bf16, np.inf, q)
    out[nz] = np.copysign(q, v[nz])
    out[~nz] = v[~nz]
    return out


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    E = (c >> 3) & 15
    m = c & 7
    sub = np.ldexp(m.astype(np.float64), -9)
    nrm = np.ldexp(1.0 + m / 8.0, E - 7)
    val = np.where(E == 0, sub, nrm)
    val = np.where((E == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(v) -> np.ndarray:
    """float values -> uint8 E4M3FN codes, round to nearest even, saturating."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    code = np.zeros(v.shape, dtype=np.int64)
    nz = a > 0
    an = a[nz]
    e = np.maximum(_floor_log2(an), -6)               # below 2^-6 the spacing stays 2^-9
    spacing = np.ldexp(1.0, e - 3)
    r = np.rint(an / spacing) * spacing                # representable value, ties to even
    r = np.minimum(r, E4M3_MAX)
    sub = r < 2.0 ** -6
    c = np.empty(an.shape, dtype=np.int64)
    c[sub] = np.rint(r[sub] / 2.0 ** -9).astype(np.int64)
    rn = r[~sub]
    ern = _floor_log2(rn)
    c[~sub] = ((ern + 7) << 3) | (np.rint(rn / np.ldexp(1.0, ern - 3)).astype(np.int64) - 8)
    code[nz] = c
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


def quant_e4m3_1x128(v32: np.ndarray):
    """Per-row, per-128-column block quantisation in fp32 arithmetic.

    For each block: amax = max |v|; s = fl32(amax / 448) (s = 1 when the block
    is all zero); q = enc(fl32(v / s)).  Returns (codes uint8 [rows][cols],
    scales float32 [rows][cols/128]).  Every division is an IEEE binary32
    division (numpy float32), the precision in which the scales are stored.
    """
    v32 = np.asarray(v32, dtype=np.float32)
    rows, cols = v32.shape
    assert cols % 128 == 0
    vb = v32.reshape(rows, cols // 128, 128)
    amax = np.abs(vb).max(axis=2)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = e4m3_encode((vb / s[:, :, None]).astype(np.float32))
    return q.reshape(rows, cols), s


def dequant_e4m3_1x128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    rows, cols = q.shape
    return (e4m3_decode(q).reshape(rows, cols // 128, 128) * s.astype(np.float64)[:, :, None]).reshape(rows, cols)


def dequant_e4m3_block(q: np.ndarray, s: np.ndarray, br: int = 128, bc: int = 128) -> np.ndarray:
    """[..., R, C] codes with [..., R/br, C/bc] scales -> float64 values (exact)."""
    *lead, R, C = q.shape
    d = e4m3_decode(q).reshape(*lead, R // br, br, C // bc, bc)
    return (d * s.astype(np.float64)[..., :, None, :, None]).reshape(*lead, R, C)
