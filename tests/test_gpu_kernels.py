"""GPU parity of every step of the layer against the CPU oracle, at sizes the
oracle finishes in seconds that still span several tiles and ragged tails.

Bit-exact: expert ids, counts, offsets, src, dest, e4m3 codes and scales of
activations.  Tolerances (written here, from the layer's accuracy target):
  routing weights            |dw| <= 1e-6
  fp32/bf16-weight outputs   max-abs <= 2e-2 and rel-Frobenius <= 1e-2
  fp8-weight outputs         rel-Frobenius <= 1e-2
The fp8 floor is set by the matrix cores' fp8 sums, which are not rounded
like fp32 sums (about 2e-5 of the sum of the products' magnitudes on
average, 2e-4 at most, per 128-long block): a few e4m3 codes of h per row,
and of y when y is e4m3, land on the other side of a rounding boundary from
the oracle's.  Observed up to ~5e-3 at these sizes (a flipped code weighs
1/sqrt(I) of a row, I = 256 to 512), so the gate is twice that.
"""
import numpy as np
import pytest
import torch

import routed_expert_ffn_04_amd as moe
import synth
from oracle import codecs
from oracle import moe as om

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

TOL_W = 1e-6
TOL_MAXABS = 2e-2
TOL_FROB = 1e-2
TOL_FROB_FP8 = 1e-2


def rel_frob(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_out(got, ref, fp8: bool, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, what
    assert np.isfinite(got).all(), what
    rf = rel_frob(got, ref)
    ma = float(np.abs(got - ref).max()) if got.size else 0.0
    print(f"[{what}] rel_frob={rf:.3e} max_abs={ma:.3e} max|ref|={np.abs(ref).max() if ref.size else 0:.3e}", flush=True)
    if fp8:
        assert rf <= TOL_FROB_FP8, what
    else:
        assert rf <= TOL_FROB and ma <= TOL_MAXABS, what


def to_dev(wl):
    f = lambda t: None if t is None else t.to(DEV)
    wl.x, wl.w_router, wl.bias = f(wl.x), f(wl.w_router), f(wl.bias)
    wl.a_q, wl.a_s = f(wl.a_q), f(wl.a_s)
    wl.routed = wl.routed.to(DEV) if wl.routed is not None else None
    wl.shared = wl.shared.to(DEV) if wl.shared is not None else None
    return wl


# ---------------------------------------------------------------- route

ROUTE_CASES = [
    # T, H, E, k, score, x_dt, bias
    (64, 256, 8, 2, "softmax", "f32", False),
    (37, 384, 40, 5, "sigmoid", "bf16", True),        # ragged T and E
    (300, 1024, 256, 8, "sigmoid", "bf16", False),    # mid register tile
    (2100, 512, 256, 8, "sigmoid", "bf16", True),     # large register tile + ragged
    (5, 128, 16, 16, "softmax", "f32", False),        # k = E
    (9, 128, 1024, 3, "sigmoid", "bf16", False),      # E at the maximum
    (11, 128, 7, 1, "softmax", "f32", False),         # k = 1
    (20, 1536, 24, 4, "sigmoid", "bf16", True),       # 512-long h chunks, ragged T and E
    (3, 768, 12, 2, "softmax", "f32", False),         # 256-long h chunks, fp32 x
]


@pytest.mark.parametrize("T,H,E,k,score,x_dt,use_bias", ROUTE_CASES)
def test_route_parity(T, H, E, k, score, x_dt, use_bias):
    print(f"route T={T} H={H} E={E} k={k} {score} {x_dt} bias={use_bias}", flush=True)
    seed = T * 31 + E
    x = synth.normal((T, H), seed, 1, 1.0, torch.float32 if x_dt == "f32" else torch.bfloat16)
    wr = synth.normal((H, E), seed, 2, H ** -0.5)
    b = synth.normal((E,), seed, 3, 0.5) if use_bias else None
    ids_ref, w_ref, _ = om.route(x.float().numpy(), wr.numpy(), None if b is None else b.numpy(), k, score)
    ids, w = moe.route(x.to(DEV), wr.to(DEV), None if b is None else b.to(DEV), k, score)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(w.cpu().numpy() - w_ref).max() <= TOL_W


def test_route_exact_ties_pick_lowest_index():
    T, H, E, k = 20, 128, 64, 8
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    wr = synth.normal((H, E), 5, 2, 0.1)
    b = torch.zeros(E)
    b[10:30] = 1.0                      # 20 experts tie at the top
    ids, w = moe.route(x.to(DEV), wr.to(DEV), b.to(DEV), k, "sigmoid")
    ids_ref, w_ref, _ = om.route(x.float().numpy(), wr.numpy(), b.numpy(), k, "sigmoid")
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_array_equal(ids.cpu().numpy()[0], np.arange(10, 18))
    assert np.abs(w.cpu().numpy() - 1.0 / k).max() <= TOL_W


# ---------------------------------------------------------------- permute

PERMUTE_CASES = [
    ("uniform", 128, 8, 256),
    ("uniform", 3001, 8, 256),      # ragged, several chunks
    ("onehot", 2048, 8, 256),       # every assignment to expert 0 ... k-1
    ("skew", 5000, 6, 300),
    ("uniform", 1, 1, 1),
    ("uniform", 777, 3, 1024),      # E at the maximum
    ("uniform", 16384, 8, 256),
    # one-workgroup path (at most two chunks): E at the maximum, ragged second chunk, skew
    ("uniform", 256, 8, 1024),
    ("onehot", 200, 8, 256),
    ("skew", 100, 6, 300),
]


@pytest.mark.parametrize("kind,T,k,E", PERMUTE_CASES)
def test_permute_parity(kind, T, k, E):
    print(f"permute {kind} T={T} k={k} E={E}", flush=True)
    rng = np.random.default_rng(T + k + E)
    if kind == "onehot":
        ids = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    elif kind == "skew":
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        ids = np.stack([rng.choice(E, k, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    else:
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    ref = om.permute(ids, E)
    got = moe.permute(torch.from_numpy(ids).to(DEV), E)
    torch.cuda.synchronize()
    for g, r, name in zip(got, ref, ["counts", "offsets", "src", "dest"]):
        np.testing.assert_array_equal(g.cpu().numpy(), r, err_msg=name)


# ---------------------------------------------------------------- quant

@pytest.mark.parametrize("rows,cols,x_dt", [(1, 128, "bf16"), (37, 7168, "bf16"), (64, 256, "f32"), (1000, 512, "bf16")])
def test_quant_parity_bit_exact(rows, cols, x_dt):
    x = synth.normal((rows, cols), rows, 7, 1.0, torch.float32 if x_dt == "f32" else torch.bfloat16)
    x[0, :128] = 0                                 # all-zero block -> scale 1, codes 0
    if rows > 3:
        x[1, 5] = -3e-7                            # rounds to -0 (code 0x80)
        x[2, 128:256] *= 1e4                       # large magnitudes
    q_ref, s_ref = codecs.quant_e4m3_1x128(x.float().numpy())
    q, s = moe.quant_e4m3_1x128(x.to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


# ---------------------------------------------------------------- grouped FFN

GROUPED_CASES = [
    # group rows (0 = empty expert), shared rows, H, I, dt
    ([130, 5, 0, 64, 1], 40, 256, 256, "bf16"),
    ([3, 77, 200], 0, 384, 512, "bf16"),
    ([130, 5, 0, 64, 1], 40, 256, 256, "e4m3"),
    ([257, 9], 300, 512, 384, "e4m3"),
    ([70, 0, 12], 20, 256, 256, "f32"),
    # 36 and 31 groups of 17..116 rows: the 64-row ring tiles (bf16, H % 256 == 0)
    ([17 + (g * 37) % 100 for g in range(36)], 50, 512, 256, "bf16"),
    ([17 + (g * 37) % 100 for g in range(31)] + [3, 0], 0, 512, 256, "bf16"),
    # the 64-row ring tiles at their m-tile boundaries (one short, exact, one
    # over), several m-tiles per group, the shared expert among them, and the
    # shortest down K loop (I = 128: two stages)
    ([17, 63, 64, 65, 128, 129, 192, 255, 256, 3], 100, 512, 128, "bf16"),
    ([40, 90, 33, 250, 170], 0, 256, 256, "bf16"),
    # m-tile boundaries of the 256-row tiles: exact multiples, one short, one over
    ([256, 512, 255, 257, 1], 256, 512, 256, "e4m3"),
    ([256, 512, 255, 257, 1], 0, 512, 256, "bf16"),
    # partial m-tiles ending inside and at the edge of 8-row load groups and of
    # the first and second 64-row load waves
    ([265, 282, 320, 329, 263], 0, 512, 256, "e4m3"),
    ([265, 282, 320, 329, 263], 0, 512, 256, "bf16"),
]


@pytest.mark.parametrize("gm,sm,H,I,dt", GROUPED_CASES)
@pytest.mark.parametrize("y_dt", ["f32", "bf16", "e4m3"])
def test_grouped_ffn_parity(gm, sm, H, I, dt, y_dt):
    if y_dt == "e4m3" and (dt != "e4m3" or H % 256):
        pytest.skip("e4m3 expert outputs: e4m3 weights and H % 256 == 0 only")
    print(f"grouped gm={gm} sm={sm} H={H} I={I} {dt} y={y_dt}", flush=True)
    fp8_y = y_dt == "e4m3"
    wl = synth.make_grouped(gm, sm, H, I, dt=dt, seed=sum(gm) + sm, y_dt="bf16" if fp8_y else y_dt)
    wl.y_dt = "e4m3" if fp8_y else None
    ref = om.grouped_ffn(wl)
    wl = to_dev(wl)
    G = len(gm)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(gm)]), dtype=torch.int32, device=DEV)
    R = int(sum(gm))
    ydt = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8}[y_dt]
    if dt == "e4m3":
        a, a_s = wl.a_q, wl.a_s
        a_sh, a_sh_s = (wl.a_q[R:], wl.a_s[R:]) if sm else (None, None)
    else:
        a, a_s = wl.x, None
        a_sh, a_sh_s = (wl.x[R:], None) if sm else (None, None)
    y, y_sh = moe.grouped_ffn(a, offs, moe.Experts.from_bank(wl.routed), a_scale=a_s, R_max=R,
                              a_sh=a_sh, a_sh_scale=a_sh_s,
                              shared=moe.Experts.from_bank(wl.shared) if sm else None, y_dtype=ydt)
    torch.cuda.synchronize()
    if fp8_y:
        yc = codecs.dequant_e4m3_1x128(y[0].cpu().numpy(), y[1].cpu().numpy())
    else:
        yc = y.float().cpu().numpy()
    starts = np.concatenate([[0], np.cumsum(gm)])
    for g in range(G):
        check_out(yc[starts[g]:starts[g + 1]], ref[g][1], dt == "e4m3", f"group {g}")
    if sm:
        check_out(y_sh.float().cpu().numpy(), ref["shared"][1], dt == "e4m3", "shared")


# ---------------------------------------------------------------- combine

@pytest.mark.parametrize("y_dt,out_dt,shared,k", [("f32", "f32", True, 4), ("bf16", "bf16", True, 4), ("f32", "bf16", False, 4),
                                                 ("e4m3", "bf16", True, 4), ("e4m3", "f32", False, 4),
                                                 # expert rows in chunks of 8: one full chunk plus a remainder, two plus one
                                                 ("f32", "f32", True, 12), ("bf16", "bf16", False, 9), ("e4m3", "bf16", True, 17)])
def test_combine_parity(y_dt, out_dt, shared, k):
    T, H = 50, 384
    rng = np.random.default_rng(1)
    R = T * k
    dest = rng.permutation(R).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    ysc = None
    if y_dt == "e4m3":
        # codes of every finite value (no 0x7F / 0xFF) and positive fp32 block scales
        codes = rng.integers(0, 0x7F, size=(R, H), dtype=np.uint8) | (rng.integers(0, 2, size=(R, H)) << 7).astype(np.uint8)
        scales = np.exp(rng.uniform(-6, 2, size=(R, H // 128))).astype(np.float32)
        yp = torch.from_numpy(codes)
        ysc = torch.from_numpy(scales)
        yref = codecs.dequant_e4m3_1x128(codes, scales)
        ysh = synth.normal((T, H), 9, 2, 1.0, torch.bfloat16) if shared else None
    else:
        ydt = torch.float32 if y_dt == "f32" else torch.bfloat16
        yp = synth.normal((R, H), 9, 1, 1.0, ydt)
        yref = yp.float().numpy().astype(np.float64)
        ysh = synth.normal((T, H), 9, 2, 1.0, ydt) if shared else None
    ref = om.combine(yref, None if ysh is None else ysh.float().numpy(), dest, w, k)
    ref = om.round_to(ref, out_dt)
    out = moe.combine(yp.to(DEV), None if ysh is None else ysh.to(DEV), torch.from_numpy(dest).to(DEV),
                      torch.from_numpy(w).to(DEV), out_dtype=torch.float32 if out_dt == "f32" else torch.bfloat16,
                      y_scale=None if ysc is None else ysc.to(DEV))
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    # fp32 accumulation vs the oracle's fp64: a few ulps (then the output rounding)
    tol = 1e-5 if out_dt == "f32" else 2.0 ** -8
    assert (np.abs(o - ref) <= tol * (np.abs(ref) + 1)).all()


# ---------------------------------------------------------------- layer

LAYER_CASES = [
    dict(T=64, H=256, E=8, k=2, I=512, x_dt="f32", w_dt="f32", out_dt="f32", score="softmax", shared=False),
    dict(T=100, H=512, E=32, k=4, I=256, x_dt="bf16", w_dt="bf16", out_dt="f32", score="sigmoid", shared=True),
    dict(T=77, H=512, E=16, k=3, I=384, x_dt="bf16", w_dt="e4m3", out_dt="bf16", score="sigmoid", shared=True),
    dict(T=200, H=256, E=64, k=8, I=256, x_dt="bf16", w_dt="bf16", out_dt="bf16", score="softmax", shared=False),
    # the FP8 combine: routed outputs as e4m3 per 1x128 before the weighted reduce
    dict(T=90, H=512, E=16, k=4, I=256, x_dt="bf16", w_dt="e4m3", out_dt="bf16", score="sigmoid", shared=True,
         y_dt="e4m3"),
]


@pytest.mark.parametrize("cfg", LAYER_CASES, ids=lambda c: f"{c['w_dt']}-T{c['T']}-E{c['E']}-y{c.get('y_dt')}")
def test_layer_parity(cfg):
    print(f"layer {cfg}", flush=True)
    c = dict(cfg)
    y_dt = c.pop("y_dt", None)
    wl = synth.make_layer(c.pop("T"), c.pop("H"), c.pop("E"), c.pop("k"), c.pop("I"), seed=123, **c)
    wl.y_dt = y_dt
    ref = om.moe_layer(wl)
    wl = to_dev(wl)
    out, ids, w, counts = moe.layer(wl.x, wl.w_router, wl.bias, wl.k, wl.score, moe.Experts.from_bank(wl.routed),
                                    moe.Experts.from_bank(wl.shared) if wl.shared is not None else None,
                                    out_dtype=torch.float32 if wl.out_dt == "f32" else torch.bfloat16,
                                    want_routing=True, y_dtype=torch.uint8 if y_dt == "e4m3" else None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["ids"])
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.abs(w.cpu().numpy() - ref["w"]).max() <= TOL_W
    check_out(out.float().cpu().numpy(), ref["out"], wl.w_dt == "e4m3", "layer")


def test_layer_is_deterministic():
    wl = to_dev(synth.make_layer(96, 512, 16, 4, 256, w_dt="e4m3", out_dt="bf16", seed=7))
    run = lambda: moe.layer(wl.x, wl.w_router, None, 4, "sigmoid", moe.Experts.from_bank(wl.routed),
                            moe.Experts.from_bank(wl.shared), out_dtype=torch.bfloat16)
    a = run().clone()
    b = run().clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_layer_T0_is_noop():
    wl = to_dev(synth.make_layer(4, 256, 8, 2, 256, seed=3))
    out = moe.layer(wl.x[:0], wl.w_router, None, 2, "sigmoid", moe.Experts.from_bank(wl.routed),
                    moe.Experts.from_bank(wl.shared))
    torch.cuda.synchronize()
    assert out.shape == (0, 256)
