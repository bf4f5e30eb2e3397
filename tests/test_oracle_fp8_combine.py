"""Pins of the FP8 combine in the oracle (round_y 'e4m3'): the per-1x128 fp8
round trip of expert outputs before the weighted reduce ("DeepSeek V3/R1
Inference Efficiency (2)", section 2, FP8 for the combine payload)."""
import numpy as np

import synth
from oracle import codecs
from oracle import moe as om


def test_round_trip_is_exact_on_representable_rows():
    """Rows built from e4m3 codes times a power-of-two block scale, each
    block holding the code of 448, come back unchanged (amax/448 is then
    exactly the block scale)."""
    rng = np.random.default_rng(0)
    rows, cols = 5, 512
    codes = rng.integers(0, 0x7F, size=(rows, cols), dtype=np.uint8)   # finite codes, any sign bit below
    codes[:, ::128] = 0x7E                                              # 448 in every block
    codes |= (rng.integers(0, 2, size=(rows, cols)) << 7).astype(np.uint8)
    scale = 2.0 ** rng.integers(-20, 5, size=(rows, cols // 128))
    v = codecs.e4m3_decode(codes).reshape(rows, cols // 128, 128) * scale[:, :, None]
    v = v.reshape(rows, cols)
    np.testing.assert_array_equal(om.round_y(v, "e4m3"), v)


def test_round_trip_error_bound():
    """|round_y(v) - v| <= max(2^-4 |v|, s 2^-10): half a unit in the last
    place of a 3-bit mantissa, or half the subnormal step, per block scale s."""
    rng = np.random.default_rng(1)
    v = rng.standard_normal((7, 384)) * np.exp(rng.uniform(-8, 8, size=(7, 1)))
    got = om.round_y(v, "e4m3")
    amax = np.abs(v.astype(np.float32)).reshape(7, 3, 128).max(axis=2)
    s = np.repeat(amax / 448.0, 128, axis=1)
    bound = np.maximum(2.0 ** -4 * np.abs(v), s * 2.0 ** -10) * (1 + 1e-6) + np.abs(v) * 2.0 ** -23
    assert (np.abs(got - v) <= bound).all()
    assert (np.abs(got - v) > 0).any()


def test_layer_with_fp8_combine_stays_near_the_bf16_combine():
    """The same fp8 layer with and without the fp8 round trip of the routed
    outputs: different, and within the quantisation noise."""
    wl = synth.make_layer(40, 512, 8, 2, 256, w_dt="e4m3", out_dt="bf16", seed=11)
    a = om.moe_layer(wl)["out"]
    wl.y_dt = "e4m3"
    b = om.moe_layer(wl)["out"]
    rel = np.linalg.norm(a - b) / np.linalg.norm(a)
    assert 0 < rel < 2.0 ** -5


def test_token_sample_matches_full_layer_with_fp8_combine():
    wl = synth.make_layer(24, 256, 8, 2, 256, w_dt="e4m3", out_dt="bf16", seed=12)
    wl.y_dt = "e4m3"
    full = om.moe_layer(wl)["out"]
    part = om.moe_layer_tokens(wl, [0, 5, 23])["out"]
    np.testing.assert_array_equal(part, full[[0, 5, 23]])
