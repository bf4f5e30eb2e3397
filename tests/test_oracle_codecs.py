"""Pins for the oracle's number formats (bf16 RNE, OCP E4M3FN).

Checked against the format definitions (special code values) and against
torch's own casts, a library codec independent of both the oracle and the
GPU library."""
import numpy as np
import pytest
import torch

from oracle import codecs


def _torch_bf16(v64):
    return torch.from_numpy(np.asarray(v64, dtype=np.float32)).to(torch.bfloat16).float().double().numpy()


def test_bf16_matches_torch_cast_on_fp32_values():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(200000) * np.exp2(rng.integers(-130, 120, 200000))).astype(np.float32)
    np.testing.assert_array_equal(codecs.bf16_rne(v), _torch_bf16(v))


def test_bf16_ties_to_even_at_midpoints():
    rng = np.random.default_rng(1)
    b = torch.from_numpy(rng.standard_normal(5000).astype(np.float32)).to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    lo = b.float().double().numpy()
    hi = torch.from_numpy(((bits + 1) & 0xFFFF).astype(np.int16)).view(torch.bfloat16).float().double().numpy()
    mid = (lo + hi) / 2                      # exact in fp64
    r = codecs.bf16_rne(mid)
    even = np.where(bits % 2 == 0, lo, hi)
    np.testing.assert_array_equal(r, even)


def test_e4m3_decode_definition_points():
    d = codecs.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0x7F, 0x80, 0xFE, 0xB8]))
    exp = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 448.0, np.nan, -0.0, -448.0, -1.0]
    np.testing.assert_array_equal(d, np.array(exp))
    assert np.signbit(d[8])


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    np.testing.assert_array_equal(codecs.e4m3_decode(codes), t)


def test_e4m3_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(codecs.e4m3_encode(codecs.e4m3_decode(codes)), codes)


def test_e4m3_encode_ties_to_even_at_every_midpoint():
    pos = np.arange(0, 0x7E + 1)
    vals = codecs.e4m3_decode(pos)
    mids = (vals[:-1] + vals[1:]) / 2
    enc = codecs.e4m3_encode(mids).astype(np.int64)
    expect = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])   # even mantissa wins
    np.testing.assert_array_equal(enc, expect)
    np.testing.assert_array_equal(codecs.e4m3_encode(-mids).astype(np.int64), expect | 0x80)


def test_e4m3_encode_matches_torch_within_range():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(300000) * np.exp2(rng.integers(-12, 9, 300000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codecs.e4m3_encode(v), t)


def test_e4m3_saturates_and_keeps_sign_of_zero():
    assert codecs.e4m3_encode(np.array([500.0]))[0] == 0x7E
    assert codecs.e4m3_encode(np.array([-1e30]))[0] == 0xFE
    assert codecs.e4m3_encode(np.array([-1e-9]))[0] == 0x80
    assert codecs.e4m3_encode(np.array([1e-9]))[0] == 0x00


def test_quant_1x128_scale_amax_and_error_bound():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((7, 512)).astype(np.float32)
    v[3, 128:256] = 0.0
    q, s = codecs.quant_e4m3_1x128(v)
    assert q.dtype == np.uint8 and s.dtype == np.float32 and s.shape == (7, 4)
    amax = np.abs(v.reshape(7, 4, 128)).max(axis=2)
    np.testing.assert_array_equal(s[amax > 0], (amax / np.float32(448)).astype(np.float32)[amax > 0])
    assert s[3, 1] == 1.0 and (q[3, 128:256] == 0).all()
    # the largest element of each non-zero block lands on +-448
    qb = q.reshape(7, 4, 128)
    idx = np.abs(v.reshape(7, 4, 128)).argmax(axis=2)
    top = np.take_along_axis(qb, idx[:, :, None], axis=2)[..., 0]
    assert ((top[amax > 0] & 0x7F) == 0x7E).all()
    # |v - s dec(q)| <= half a code spacing of v/s, times s
    r = (v.reshape(7, 4, 128) / s[:, :, None]).astype(np.float64)
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -20))), -6)
    half = np.exp2(e - 4) * s[:, :, None]
    deq = codecs.dequant_e4m3_1x128(q, s).reshape(7, 4, 128)
    assert (np.abs(deq - v.reshape(7, 4, 128)) <= half * (1 + 1e-6)).all()
