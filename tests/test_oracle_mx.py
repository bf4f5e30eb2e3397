"""Pins for the oracle's microscaling formats (OCP MX v1.0: E8M0 scales,
FP4 E2M1 and FP8 E4M3 elements in blocks of 32).

E8M0 decoding is checked against torch's float8_e8m0fnu cast (a library
codec); E2M1 against the generic sign/exponent/mantissa formula of a binary
float with 2 exponent bits (bias 1) and 1 mantissa bit; the block conversion
against a brute-force nearest-element search and hand-worked blocks."""
import numpy as np
import pytest
import torch

from oracle import codecs, mx


def test_e8m0_decode_matches_torch_cast():
    E = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(E).view(torch.float8_e8m0fnu).double().numpy()
    d = mx.e8m0_decode(E)
    np.testing.assert_array_equal(d[:255], t[:255])
    assert np.isnan(d[255]) and np.isnan(t[255])
    assert d[127] == 1.0 and d[0] == 2.0 ** -127 and d[254] == 2.0 ** 127


def test_e2m1_decode_is_the_binary_float_formula():
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        # exponent bias 1; exponent field 0 is subnormal (2^(1-1) * m/2)
        mag = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0)
        v = (-1.0) ** s * mag
        got = mx.e2m1_decode(np.array([c]))[0]
        assert got == v and np.signbit(got) == bool(s), c
    assert mx.e2m1_decode(np.array([7]))[0] == 6.0


def test_e2m1_encode_roundtrip_and_ties_to_even():
    codes = np.arange(16)
    np.testing.assert_array_equal(mx.e2m1_encode(mx.e2m1_decode(codes)), codes)
    vals = mx.e2m1_decode(np.arange(8))
    mids = (vals[:-1] + vals[1:]) / 2
    expect = np.where(np.arange(7) % 2 == 0, np.arange(7), np.arange(1, 8))
    np.testing.assert_array_equal(mx.e2m1_encode(mids), expect)
    np.testing.assert_array_equal(mx.e2m1_encode(-mids), expect | 8)
    # just off the midpoints: nearest wins
    np.testing.assert_array_equal(mx.e2m1_encode(mids - 1e-9), np.arange(7))
    np.testing.assert_array_equal(mx.e2m1_encode(mids + 1e-9), np.arange(1, 8))
    # saturation above 6
    np.testing.assert_array_equal(mx.e2m1_encode(np.array([6.5, 7.0, 1e30, -9.0])), [7, 7, 7, 15])


def _brute_nearest(x, elem_vals):
    """Nearest representable magnitude by exhaustive search (ties: the even
    code, i.e. the lower index in an ascending table with codes 0, 1, 2 ...
    whose mantissa LSB alternates)."""
    d = np.abs(np.abs(x)[:, None] - elem_vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.array([np.flatnonzero(r)[0] if not any(r[i] and i % 2 == 0 for i in np.flatnonzero(r))
                    else [i for i in np.flatnonzero(r) if i % 2 == 0][0] for r in cand])
    return np.copysign(elem_vals[idx], x)


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_mx_quant_is_nearest_element_at_the_spec_scale(elem):
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((40, 64)) * np.exp2(rng.integers(-20, 20, (40, 1)))).astype(np.float32)
    q, E = mx.mx_quant(v, elem)
    assert q.shape == v.shape and E.shape == (40, 2)
    vb = v.astype(np.float64).reshape(40, 2, 32)
    amax = np.abs(vb).max(axis=2)
    # the spec's shared exponent: floor(log2(amax)) - emax_elem
    shared = np.floor(np.log2(amax)).astype(np.int64) - (2 if elem == "e2m1" else 8)
    np.testing.assert_array_equal(E.astype(np.int64), shared + 127)
    if elem == "e2m1":
        table = mx.E2M1_VALUES
    else:
        table = np.sort(codecs.e4m3_decode(np.arange(0x7F)))
        table = table[np.concatenate([[True], np.diff(table) > 0])]
    X = np.exp2(shared)[:, :, None]
    clamp = np.minimum(np.abs(vb / X), table[-1]) * np.sign(vb / X)
    expect = _brute_nearest(clamp.reshape(-1), table).reshape(vb.shape) * X
    np.testing.assert_array_equal(mx.mx_dequant(q, E, elem), expect.reshape(40, 64))


def test_mx_quant_worked_blocks():
    # amax 6 * 2^-3: shared exponent -3, every multiple of 2^-4 up to 6 * 2^-3 on the grid is exact
    blk = np.zeros(32, dtype=np.float32)
    blk[:8] = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]) * 2.0 ** -3
    blk[8:16] = -blk[:8]
    q, E = mx.mx_quant(blk[None], "e2m1")
    assert E[0, 0] == 127 - 3
    np.testing.assert_array_equal(mx.mx_dequant(q, E, "e2m1")[0], blk)
    # amax 7: shared exponent 0 and 7 clamps to 6 (the spec's saturation);
    # 2.5 is a tie between 2 (code 4, even) and 3 (code 5)
    blk = np.zeros(32, dtype=np.float32)
    blk[0], blk[1], blk[2], blk[3] = 7.0, 2.5, -0.25, 0.26
    q, E = mx.mx_quant(blk[None], "e2m1")
    assert E[0, 0] == 127
    np.testing.assert_array_equal(mx.mx_dequant(q, E, "e2m1")[0, :4], [6.0, 2.0, -0.0, 0.5])
    # e4m3 elements: amax 500 -> shared exponent 0, 500 clamps to 448
    blk = np.zeros(32, dtype=np.float32)
    blk[0], blk[1] = 500.0, 1.0 + 2.0 ** -4
    q, E = mx.mx_quant(blk[None], "e4m3")
    assert E[0, 0] == 127
    d = mx.mx_dequant(q, E, "e4m3")[0]
    assert d[0] == 448.0 and d[1] == 1.0      # 1 + 2^-4 is a tie: even mantissa (1.0)
    # all-zero block: E = 0, zero elements
    q, E = mx.mx_quant(np.zeros((1, 32), np.float32), "e2m1")
    assert E[0, 0] == 0 and not q.any()


def test_mx_quant_scale_range_clamps():
    # tiny block: floor(log2) - 8 below -127 clamps to E = 0 (scale 2^-127)
    v = np.full((1, 32), 2.0 ** -130, dtype=np.float32)
    q, E = mx.mx_quant(v, "e4m3")
    assert E[0, 0] == 0
    np.testing.assert_array_equal(mx.mx_dequant(q, E, "e4m3"), v.astype(np.float64))
    # huge block: fp32 max -> shared exponent 127 - 2 = 125
    v = np.full((1, 32), np.finfo(np.float32).max, dtype=np.float32)
    q, E = mx.mx_quant(v, "e2m1")
    assert E[0, 0] == 127 + 125


def test_unpack_e2m1_nibble_order():
    np.testing.assert_array_equal(mx.unpack_e2m1(np.array([[0x21, 0xF8]], np.uint8)), [[1, 2, 8, 15]])
    packed = np.array([[0x7A]], np.uint8)
    E = np.array([[127]], np.uint8)
    m = mx.mxfp4_matrix(np.concatenate([packed, np.zeros((1, 15), np.uint8)], axis=1), E)
    assert m[0, 0] == -1.0 and m[0, 1] == 6.0


def test_mxfp8_round_trip_is_idempotent_and_bounded():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((16, 256)).astype(np.float32)
    r = mx.mxfp8_round_trip(v)
    np.testing.assert_array_equal(mx.mxfp8_round_trip(r.astype(np.float32)), r)
    vb = v.astype(np.float64).reshape(16, 8, 32)
    rb = r.reshape(16, 8, 32)
    amax = np.abs(vb).max(axis=2, keepdims=True)
    X = np.exp2(np.floor(np.log2(amax)) - 8)
    err = np.abs(rb - vb)
    # below the saturation point 448 X: half an e4m3 spacing (2^-4 relative,
    # 2^-10 X absolute in the subnormal range)
    ok = np.abs(vb) <= 448 * X
    assert np.all(err[ok] <= np.maximum(np.abs(vb) * 2.0 ** -4, 2.0 ** -10 * X)[ok])
    # above it (amax in (448 X, 512 X)): clamped to 448 X, at most 1/8 of the block max
    assert np.all(err <= amax / 8)
