"""Pins for the oracle's MXFP4 layer (E2M1 weights with E8M0 per-32 scales,
MXFP8 activations and h).

* The stored bank decodes, element by element with explicit bit arithmetic,
  to the matrices the oracle multiplies (nibble order and scale indexing).
* The sparse layer with its rounding points disabled equals a brute-force
  dense evaluation (every expert on every token, masked by routing weights);
  with them, it stays close.
* h is MXFP8-representable with the shared exponent the spec fixes; the
  token-subset path reproduces the full layer; the pre-routed grouped path
  equals the direct expert FFN."""
import numpy as np
import pytest
import torch

import synth
from oracle import mx, moe


def _elem(packed, E, r, c):
    """Element (r, c) of a stored MXFP4 matrix by explicit bit arithmetic."""
    byte = int(packed[r, c // 2])
    nib = (byte >> 4) if c % 2 else (byte & 15)
    sign = -1.0 if nib & 8 else 1.0
    e, m = (nib >> 1) & 3, nib & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + 0.5 * m)
    return sign * mag * 2.0 ** (int(E[r, c // 32]) - 127)


def test_bank_decodes_elementwise():
    b = synth._bank(3, 128, 256, "mxfp4", 7, (10, 11, 12), 0.02, "cpu")
    wg, wu, wd = moe.bank_expert_f64(b, 2)
    assert wg.shape == (256, 128) and wd.shape == (128, 256)
    rng = np.random.default_rng(0)
    for (mat, w, s) in ((wg, b.w_gate, b.s_gate), (wu, b.w_up, b.s_up), (wd, b.w_down, b.s_down)):
        pw, ps = w[2].numpy(), s[2].numpy()
        for _ in range(200):
            r, c = rng.integers(0, mat.shape[0]), rng.integers(0, mat.shape[1])
            assert mat[r, c] == _elem(pw, ps, r, c)


def test_bank_slice_regenerates_identically():
    full = synth._bank(4, 128, 128, "mxfp4", 3, (10, 11, 12), 0.02, "cpu")
    part = synth._bank(1, 128, 128, "mxfp4", 3, (10, 11, 12), 0.02, "cpu", experts=[2])
    for a, b in ((full.w_gate, part.w_gate), (full.s_down, part.s_down)):
        assert torch.equal(a[2], b[0])


def _no_rounding(wl):
    x32, wr, b = moe.layer_inputs(wl)
    ids, w, _ = moe.route(x32, wr, b, wl.k, wl.score)
    counts, offsets, src, dest = moe.permute(ids, wl.E)
    a = moe.activation_rows(wl, x32)
    y = np.zeros((wl.T * wl.k, wl.H))
    for e in range(wl.E):
        p0, p1 = offsets[e], offsets[e + 1]
        if p1 > p0:
            y[p0:p1] = moe.expert_ffn(a[src[p0:p1] // wl.k], *moe.bank_expert_f64(wl.routed, e), "f32")
    ysh = moe.expert_ffn(a, *moe.bank_expert_f64(wl.shared, 0), "f32")
    return ids, w, moe.combine(y, ysh, dest, w, wl.k)


def test_sparse_equals_dense_brute_force():
    wl = synth.make_layer(20, 256, 8, 3, 128, w_dt="mxfp4", out_dt="f32", seed=31)
    ids, w, out = _no_rounding(wl)
    dense = moe.dense_moe(wl, ids, w)
    np.testing.assert_allclose(out, dense, rtol=1e-9, atol=1e-12 * np.abs(dense).max())
    r = moe.moe_layer(wl)
    np.testing.assert_array_equal(r["ids"], ids)
    rel = np.linalg.norm(r["out"] - dense) / np.linalg.norm(dense)
    assert rel < 5e-2


def test_activations_are_mxfp8_of_the_input():
    wl = synth.make_layer(6, 256, 8, 2, 128, w_dt="mxfp4", seed=32)
    x32, _, _ = moe.layer_inputs(wl)
    a = moe.activation_rows(wl, x32)
    amax = np.abs(x32.astype(np.float64)).reshape(6, 8, 32).max(axis=2)
    X = np.exp2(np.floor(np.log2(amax)) - 8)[:, :, None]
    codes = a.reshape(6, 8, 32) / X
    # every element is an e4m3 value at the block's spec scale
    from oracle import codecs
    np.testing.assert_array_equal(codecs.e4m3_decode(codecs.e4m3_encode(codes)), codes)


def test_h_is_mxfp8_at_the_spec_scale():
    rng = np.random.default_rng(33)
    a = rng.standard_normal((5, 128))
    wg, wu, wd = (rng.standard_normal(s) * 0.1 for s in ((96, 128), (96, 128), (128, 96)))
    _, h = moe.expert_ffn(a, wg, wu, wd, "mxfp8", return_h=True)
    _, h0 = moe.expert_ffn(a, wg, wu, wd, "f32", return_h=True)
    h0b = h0.astype(np.float32).astype(np.float64).reshape(5, 3, 32)
    X = np.exp2(np.floor(np.log2(np.abs(h0b).max(axis=2))) - 8)[:, :, None]
    from oracle import codecs
    codes = h.reshape(5, 3, 32) / X
    np.testing.assert_array_equal(codecs.e4m3_decode(codecs.e4m3_encode(codes)), codes)
    assert np.abs(codes).max() <= 448


def test_token_subset_path_matches_full_layer():
    wl = synth.make_layer(30, 256, 16, 4, 128, w_dt="mxfp4", out_dt="bf16", seed=34)
    full = moe.moe_layer(wl)
    toks = [0, 5, 29, 17]
    sub = moe.moe_layer_tokens(wl, toks)
    np.testing.assert_array_equal(sub["ids"], full["ids"][toks])
    np.testing.assert_allclose(sub["out"], full["out"][toks], rtol=1e-12, atol=1e-12)


def test_grouped_prerouted_matches_direct_expert_ffn():
    wl = synth.make_grouped([40, 3], 9, 256, 128, dt="mxfp4", seed=35, y_dt="f32")
    r = moe.grouped_ffn(wl)
    a = mx.mxfp8_round_trip(wl.x.float().numpy())
    y = moe.expert_ffn(a[40:43], *moe.bank_expert_f64(wl.routed, 1), "mxfp8")
    np.testing.assert_array_equal(r[1][1], y.astype(np.float32).astype(np.float64))
    ys = moe.expert_ffn(a[43:52], *moe.bank_expert_f64(wl.shared, 0), "mxfp8")
    np.testing.assert_array_equal(r["shared"][1], ys.astype(np.float32).astype(np.float64))
