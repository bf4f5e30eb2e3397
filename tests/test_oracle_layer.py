"""Pins for the oracle's expert FFN and whole layer.

* E = k = 1 with no shared expert reduces to a plain SwiGLU FFN, checked
  against torch's silu and matmul (library routines) in float64.
* The sparse layer agrees with a brute-force dense evaluation that runs every
  expert on every token and masks by the routing weights.
* Closed forms: x = 0 gives 0; zero routed down-projections leave only the
  shared expert; permuting tokens permutes outputs.
* The intermediate h is bf16-representable in bf16 layers and sits within
  half a bf16 ulp of the unrounded value; in fp8 layers its 128-blocks are
  e4m3 codes times an fp32 scale."""
import numpy as np
import pytest
import torch

import synth
from oracle import codecs, moe


def _torch_swiglu(a, wg, wu, wd):
    a, wg, wu, wd = (torch.from_numpy(m) for m in (a, wg, wu, wd))
    return (torch.nn.functional.silu(a @ wg.T) * (a @ wu.T) @ wd.T).numpy()


def test_single_expert_is_plain_swiglu():
    wl = synth.make_layer(17, 128, 1, 1, 256, x_dt="f32", w_dt="f32", score="softmax",
                          shared=False, seed=11)
    r = moe.moe_layer(wl)
    x = wl.x.double().numpy()
    ref = _torch_swiglu(x, *moe.bank_expert_f64(wl.routed, 0))
    assert (r["ids"] == 0).all() and (r["w"] == 1).all()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-6, atol=1e-9)


def _no_rounding(wl):
    """Sparse oracle with its rounding points disabled, for the dense check."""
    x32, wr, b = moe.layer_inputs(wl)
    ids, w, _ = moe.route(x32, wr, b, wl.k, wl.score)
    counts, offsets, src, dest = moe.permute(ids, wl.E)
    a = moe.activation_rows(wl, x32)
    y = np.zeros((wl.T * wl.k, wl.H))
    for e in range(wl.E):
        p0, p1 = offsets[e], offsets[e + 1]
        if p1 > p0:
            y[p0:p1] = moe.expert_ffn(a[src[p0:p1] // wl.k], *moe.bank_expert_f64(wl.routed, e), "f32")
    ysh = None if wl.shared is None else moe.expert_ffn(a, *moe.bank_expert_f64(wl.shared, 0), "f32")
    return ids, w, moe.combine(y, ysh, dest, w, wl.k)


@pytest.mark.parametrize("kind", ["config1", "bf16-shared", "e4m3-shared", "bias-sigmoid"])
def test_sparse_equals_dense_brute_force(kind):
    if kind == "config1":
        wl = synth.config(1)
    elif kind == "bf16-shared":
        wl = synth.make_layer(24, 256, 16, 4, 128, seed=12)
    elif kind == "e4m3-shared":
        wl = synth.make_layer(20, 256, 8, 3, 256, w_dt="e4m3", out_dt="bf16", seed=13)
    else:
        b, _ = synth.zipf_bias(16, 4, 1.2, seed=14)
        wl = synth.make_layer(30, 128, 16, 4, 128, bias=b, seed=14)
    ids, w, out = _no_rounding(wl)
    dense = moe.dense_moe(wl, ids, w)
    np.testing.assert_allclose(out, dense, rtol=1e-9, atol=1e-12 * np.abs(dense).max())
    # the full oracle (with rounding points) stays close to the unrounded sum
    r = moe.moe_layer(wl)
    np.testing.assert_array_equal(r["ids"], ids)
    rel = np.linalg.norm(r["out"] - dense) / np.linalg.norm(dense)
    assert rel < (5e-2 if wl.w_dt == "e4m3" else 1e-2)


def test_config1_full_oracle_vs_dense_fp32_rounding_only():
    wl = synth.config(1)
    r = moe.moe_layer(wl)
    dense = moe.dense_moe(wl, r["ids"], r["w"])
    np.testing.assert_allclose(r["out"], dense, rtol=1e-5, atol=1e-6 * np.abs(dense).max())


def test_zero_input_gives_zero_output():
    wl = synth.make_layer(8, 128, 8, 2, 128, seed=15)
    wl.x.zero_()
    r = moe.moe_layer(wl)
    assert (r["out"] == 0).all()


def test_zero_routed_down_leaves_shared_only():
    wl = synth.make_layer(12, 128, 8, 2, 128, seed=16)
    wl.routed.w_down.zero_()
    r = moe.moe_layer(wl)
    x = wl.x.float().double().numpy()
    wg, wu, wd = moe.bank_expert_f64(wl.shared, 0)
    h = codecs.bf16_rne(torch.nn.functional.silu(torch.from_numpy(x @ wg.T)).numpy() * (x @ wu.T))
    ref = (h @ wd.T).astype(np.float32)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-6, atol=1e-7)


def test_token_permutation_equivariance():
    wl = synth.make_layer(16, 128, 8, 2, 128, seed=17)
    r = moe.moe_layer(wl)
    perm = np.random.default_rng(0).permutation(16)
    wl.x = wl.x[torch.from_numpy(perm)].contiguous()
    r2 = moe.moe_layer(wl)
    np.testing.assert_array_equal(r2["ids"], r["ids"][perm])
    np.testing.assert_allclose(r2["out"], r["out"][perm], rtol=1e-12, atol=1e-12)


def test_token_subset_path_matches_full_layer():
    wl = synth.make_layer(40, 256, 16, 4, 128, w_dt="e4m3", out_dt="bf16", seed=18)
    full = moe.moe_layer(wl)
    toks = [0, 7, 39, 21]
    sub = moe.moe_layer_tokens(wl, toks)
    np.testing.assert_array_equal(sub["ids"], full["ids"][toks])
    np.testing.assert_allclose(sub["out"], full["out"][toks], rtol=1e-12, atol=1e-12)


def test_bf16_h_is_rounded_to_bf16():
    rng = np.random.default_rng(19)
    a = rng.standard_normal((9, 128))
    wg, wu, wd = (rng.standard_normal(s) * 0.1 for s in ((64, 128), (64, 128), (128, 64)))
    _, h = moe.expert_ffn(a, wg, wu, wd, "bf16", return_h=True)
    _, h0 = moe.expert_ffn(a, wg, wu, wd, "f32", return_h=True)
    np.testing.assert_array_equal(h, codecs.bf16_rne(h))
    assert (np.abs(h - h0) <= np.abs(h0) * 2.0 ** -8).all()
    assert (h != h0).any()


def test_e4m3_h_is_block_quantised():
    rng = np.random.default_rng(20)
    a = rng.standard_normal((5, 256))
    wg, wu, wd = (rng.standard_normal(s) * 0.1 for s in ((256, 256), (256, 256), (256, 256)))
    _, h = moe.expert_ffn(a, wg, wu, wd, "e4m3", return_h=True)
    _, h0 = moe.expert_ffn(a, wg, wu, wd, "f32", return_h=True)
    hb, h0b = h.reshape(5, 2, 128), h0.reshape(5, 2, 128)
    s = (np.abs(h0b).max(axis=2).astype(np.float32) / np.float32(448)).astype(np.float64)
    codes = hb / s[:, :, None]
    np.testing.assert_array_equal(codecs.e4m3_decode(codecs.e4m3_encode(codes)), codes)
    assert (np.abs(np.abs(hb).max(axis=2) - 448 * s) == 0).all()


def test_grouped_prerouted_matches_direct_expert_ffn():
    wl = synth.make_grouped([130, 5], 40, 256, 256, seed=21)
    r = moe.grouped_ffn(wl)
    qa = wl.a_q.numpy()
    sa = wl.a_s.numpy()
    a = codecs.dequant_e4m3_1x128(qa, sa)
    wg, wu, wd = (codecs.dequant_e4m3_block(q[1].numpy(), s[1].numpy()) for q, s in
                  ((wl.routed.w_gate, wl.routed.s_gate), (wl.routed.w_up, wl.routed.s_up),
                   (wl.routed.w_down, wl.routed.s_down)))
    y = moe.expert_ffn(a[130:135], wg, wu, wd, "e4m3")
    np.testing.assert_array_equal(r[1][1], codecs.bf16_rne(y))
    assert r["shared"][1].shape == (40, 256)


@pytest.mark.parametrize("w_dt,y_dt", [("e4m3", None), ("e4m3", "e4m3"), ("mxfp4", None), ("bf16", None)])
def test_forked_token_subset_matches_serial_and_full_layer(w_dt, y_dt):
    """The multi-process token path (experts spread over forked workers) gives
    the serial path's outputs bit for bit, and both the full layer's rows
    (to library rounding: its products run over more rows at once)."""
    wl = synth.make_layer(24, 256, 8, 2, 256, w_dt=w_dt, out_dt="bf16", seed=21)
    wl.y_dt = y_dt
    toks = [0, 3, 7, 11, 23]
    serial = moe.moe_layer_tokens(wl, toks)
    forked = moe.moe_layer_tokens(wl, toks, procs=3)
    np.testing.assert_array_equal(forked["ids"], serial["ids"])
    np.testing.assert_array_equal(forked["out"], serial["out"])
    full = moe.moe_layer(wl)
    np.testing.assert_allclose(serial["out"], full["out"][toks], rtol=1e-12, atol=1e-12)
