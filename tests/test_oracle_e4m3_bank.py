"""Pins for the oracle's decoding of block-scaled e4m3 storage: expert banks
(one fp32 scale per 128 x 128 block) and pre-routed activations (one fp32
scale per row and 128 columns), the FP8 operands of "DeepSeek V3/R1 Inference
Efficiency (2)", section 2.3.1.

* Element by element, the matrices the oracle multiplies equal the OCP E4M3FN
  value of the stored code, decoded here from its bits (sign, 4-bit exponent
  with bias 7, 3-bit mantissa, subnormals m * 2^-9), times the scale of the
  element's block.  The banks are not square (I != H, three scale blocks
  along H, two along I) so that a transposed or mis-broadcast scale index
  picks a different scale.
* The decoded values also agree with torch's own float8_e4m3fn decoding (a
  library codec), and lie within half an e4m3 spacing (times the block scale)
  of the fp32 draws they were quantised from, which synth regenerates.
"""
import math

import numpy as np
import torch

import synth
from oracle import moe


def _e4m3_bits(code: int) -> float:
    """Value of one OCP E4M3FN code from its bit fields (finite codes)."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    assert not (e == 15 and m == 7), "NaN code"
    if e == 0:
        return sign * math.ldexp(m, -9)
    return sign * math.ldexp(8 + m, e - 7 - 3)


def _half_spacing(v: np.ndarray) -> np.ndarray:
    """Half the e4m3 spacing at magnitude |v| (values of magnitude <= 448):
    spacing 2^(max(floor(log2|v|), -6) - 3)."""
    a = np.abs(v)
    e = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
    return 0.5 * np.ldexp(1.0, (np.maximum(e, -6) - 3).astype(np.int64))


SEED, STREAMS = 9, (synth.ST_RG, synth.ST_RU, synth.ST_RD)
N, H, I = 3, 384, 256


def _banks():
    e8 = synth._bank(N, H, I, "e4m3", SEED, STREAMS, 0.02, "cpu")
    f32 = synth._bank(N, H, I, "f32", SEED, STREAMS, 0.02, "cpu")
    return e8, f32


def test_bank_scale_layout_is_not_square():
    e8, _ = _banks()
    assert e8.s_gate.shape == (N, I // 128, H // 128) == (3, 2, 3)
    assert e8.s_down.shape == (N, H // 128, I // 128) == (3, 3, 2)


def test_bank_decodes_elementwise_from_code_bits():
    e8, _ = _banks()
    rng = np.random.default_rng(0)
    for e in range(N):
        mats = moe.bank_expert_f64(e8, e)
        assert mats[0].shape == (I, H) and mats[1].shape == (I, H) and mats[2].shape == (H, I)
        for mat, q, s in zip(mats, (e8.w_gate, e8.w_up, e8.w_down), (e8.s_gate, e8.s_up, e8.s_down)):
            qn, sn = q[e].numpy(), s[e].numpy()
            R, C = qn.shape
            # every scale block, at a few random positions inside it, plus its corners
            for br in range(R // 128):
                for bc in range(C // 128):
                    pts = [(0, 0), (127, 127), (0, 127), (127, 0)] + [tuple(rng.integers(0, 128, 2)) for _ in range(6)]
                    for dr, dc in pts:
                        r, c = br * 128 + int(dr), bc * 128 + int(dc)
                        want = _e4m3_bits(int(qn[r, c])) * float(sn[br, bc])
                        assert mat[r, c] == want, (e, r, c)


def test_bank_decode_matches_torch_float8():
    e8, _ = _banks()
    for e in range(N):
        for mat, q, s in zip(moe.bank_expert_f64(e8, e), (e8.w_gate, e8.w_up, e8.w_down),
                             (e8.s_gate, e8.s_up, e8.s_down)):
            vals = q[e].view(torch.float8_e4m3fn).to(torch.float64)
            sc = torch.repeat_interleave(torch.repeat_interleave(s[e].double(), 128, 0), 128, 1)
            np.testing.assert_array_equal(mat, (vals * sc).numpy())


def test_bank_is_within_half_spacing_of_its_fp32_draws():
    e8, f32 = _banks()
    for e in range(N):
        for mat, w, s in zip(moe.bank_expert_f64(e8, e), (f32.w_gate, f32.w_up, f32.w_down),
                             (e8.s_gate, e8.s_up, e8.s_down)):
            w = w[e].double().numpy()
            sc = np.repeat(np.repeat(s[e].double().numpy(), 128, 0), 128, 1)
            err = np.abs(mat - w)
            # the code of w / s is off by at most half a spacing; the division
            # itself (fp32) adds at most one fp32 ulp of w / s
            bound = (_half_spacing(w / sc) + np.abs(w / sc) * 2.0 ** -23) * sc
            assert (err <= bound).all()
            # each block's largest magnitude decodes to 448 * scale
            blocks = np.abs(mat / sc).reshape(mat.shape[0] // 128, 128, mat.shape[1] // 128, 128).max(axis=(1, 3))
            np.testing.assert_array_equal(blocks, 448.0)


def test_prerouted_activations_decode_elementwise():
    gm, sm = [130, 5], 40
    wl = synth.make_grouped(gm, sm, H, I, seed=21)
    rows = sum(gm) + sm
    qa, sa = wl.a_q.numpy(), wl.a_s.numpy()
    assert qa.shape == (rows, H) and sa.shape == (rows, H // 128)
    idx = np.arange(rows)
    a = moe.prerouted_rows(wl)(idx)
    rng = np.random.default_rng(1)
    for _ in range(400):
        r, c = int(rng.integers(0, rows)), int(rng.integers(0, H))
        assert a[r, c] == _e4m3_bits(int(qa[r, c])) * float(sa[r, c // 128]), (r, c)
    # the same rows from a subset of indices, in any order
    sub = np.array([134, 0, 77])
    np.testing.assert_array_equal(moe.prerouted_rows(wl)(sub), a[sub])
    # within half a spacing of the N(0, 1) draws they were quantised from
    x = synth.normal((rows, H), 21, synth.ST_X, 1.0, torch.float32, "cpu").double().numpy()
    sc = np.repeat(sa.astype(np.float64), 128, 1)
    assert (np.abs(a - x) <= (_half_spacing(x / sc) + np.abs(x / sc) * 2.0 ** -23) * sc).all()
