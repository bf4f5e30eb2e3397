"""GPU parity of the MXFP4 path (E2M1 expert weights with E8M0 per-32
exponents, MXFP8 activations and h) against the CPU oracle.

Bit-exact: MXFP8 codes and exponents of the activation quantisation.
Expert and layer outputs: rel-Frobenius <= 1e-2.  The weights and
activations are exact on both sides; the residual is the matrix cores' fp8
sums, which are not rounded like fp32 sums (about 2e-5 of the sum of the
products' magnitudes on average, 2e-4 at most, per 128-long block), and the
h elements whose MXFP8 code flips because of it.  A flipped code moves a row
of y by about 1/16 of one element over sqrt(I) of them: up to ~5e-3 here
(I = 256), the gate twice that."""
import numpy as np
import pytest
import torch

import routed_expert_ffn_04_amd as moe
import synth
from oracle import mx
from oracle import moe as om

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_FROB_FP8 = 1e-2


def rel_frob(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_out(got, ref, what):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all(), what
    rf = rel_frob(got, ref)
    print(f"[{what}] rel_frob={rf:.3e} max_abs={np.abs(got - ref).max():.3e} max|ref|={np.abs(ref).max():.3e}",
          flush=True)
    assert rf <= TOL_FROB_FP8, what


@pytest.mark.parametrize("rows,cols,x_dt", [(1, 32, "bf16"), (37, 7168, "bf16"), (64, 256, "f32"), (1000, 96, "bf16")])
def test_quant_mxfp8_bit_exact(rows, cols, x_dt):
    print(f"quant_mxfp8 rows={rows} cols={cols} {x_dt}", flush=True)
    x = synth.normal((rows, cols), rows + 5, 7, 1.0, torch.float32 if x_dt == "f32" else torch.bfloat16)
    x[0, :32] = 0                                  # all-zero block: E = 0, codes 0
    if rows > 3:
        x[1, 5] = -1e-6                            # rounds to -0 (code 0x80) at its block's scale
        x[2, 32:64] *= 1e4                         # large magnitudes
        x[3, 0:32] = 1.99                          # amax in (448 X, 512 X): saturates to 448 X
        if x_dt == "f32":
            x[3, 32:64] = 2.0 ** -132              # below 2^-127: E clamps to 0
    q_ref, e_ref = mx.mx_quant(x.float().numpy(), "e4m3")
    q, e = moe.quant_mxfp8(x.to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(e.cpu().numpy(), e_ref)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


GROUPED_CASES = [
    # group rows (0 = empty expert), shared rows, H, I
    ([130, 5, 0, 64, 1], 40, 256, 256),        # 16-row and 64-row tiles, a ragged 130
    ([3, 77, 200], 0, 384, 512),               # odd number of 128-wide k-steps (no K split)
    ([32, 33, 2], 17, 512, 384),               # class boundaries; odd k-steps in the down projection
    ([9, 40, 3], 20, 1280, 1152),              # full rings of loads in flight plus tails, both projections
    ([5, 30, 2], 18, 4352, 2176),              # exponents in 16-step blocks (2 blocks + 2 / 1 block + 1 tail steps)
    # five or more groups of 33..256 rows: promoted to the 256-row MX tiles
    # (up to four such groups are cut into 16-row tiles instead)
    ([20, 33, 50, 70, 100, 5, 250], 17, 512, 256),
    # H % 256 != 0 (no large MX tiles): groups of 33..256 rows on the 64-row streaming tiles
    ([40, 90, 33, 250, 170, 60], 0, 384, 256),
    # 256 x 256 MX tiles: exact, partial (one row over) and multi m-tiles, a large shared group
    ([300, 600, 257, 20, 512], 280, 512, 256),
    # a 16-stage K ring (three stages rotating) in gate/up, partial tiles
    ([700, 260], 0, 2048, 384),
    # 36 groups of 17..116 rows: promoted to the 256-row MX tiles
    ([17 + (g * 37) % 100 for g in range(36)], 50, 512, 256),
]


@pytest.mark.parametrize("gm,sm,H,I", GROUPED_CASES)
@pytest.mark.parametrize("y_dt", ["f32", "bf16"])
def test_grouped_ffn_mxfp4_parity(gm, sm, H, I, y_dt):
    print(f"grouped mxfp4 gm={gm} sm={sm} H={H} I={I} y={y_dt}", flush=True)
    wl = synth.make_grouped(gm, sm, H, I, dt="mxfp4", seed=sum(gm) + sm + 1, y_dt=y_dt)
    ref = om.grouped_ffn(wl)
    R = int(sum(gm))
    x = wl.x.to(DEV)
    a, a_e = moe.quant_mxfp8(x)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(gm)]), dtype=torch.int32, device=DEV)
    routed = moe.Experts.from_bank(wl.routed.to(DEV))
    shared = moe.Experts.from_bank(wl.shared.to(DEV)) if sm else None
    ydt = torch.float32 if y_dt == "f32" else torch.bfloat16
    y, y_sh = moe.grouped_ffn(a, offs, routed, a_scale=a_e, R_max=R,
                              a_sh=a[R:] if sm else None, a_sh_scale=a_e[R:] if sm else None,
                              shared=shared, y_dtype=ydt)
    torch.cuda.synchronize()
    yc = y.float().cpu().numpy()
    starts = np.concatenate([[0], np.cumsum(gm)])
    for g in range(len(gm)):
        if gm[g]:
            check_out(yc[starts[g]:starts[g + 1]], ref[g][1], f"group {g}")
    if sm:
        check_out(y_sh.float().cpu().numpy(), ref["shared"][1], "shared")


LAYER_CASES = [
    dict(T=100, H=512, E=32, k=4, I=256, out_dt="f32", score="sigmoid", shared=True),
    dict(T=37, H=384, E=16, k=3, I=384, out_dt="bf16", score="softmax", shared=True),
    dict(T=150, H=256, E=8, k=2, I=256, out_dt="f32", score="sigmoid", shared=False),
]


@pytest.mark.parametrize("cfg", LAYER_CASES, ids=lambda c: f"T{c['T']}-H{c['H']}-E{c['E']}")
def test_layer_mxfp4_parity(cfg):
    print(f"layer mxfp4 {cfg}", flush=True)
    c = dict(cfg)
    wl = synth.make_layer(c.pop("T"), c.pop("H"), c.pop("E"), c.pop("k"), c.pop("I"), w_dt="mxfp4",
                          seed=321, **c)
    ref = om.moe_layer(wl)
    f = lambda t: None if t is None else t.to(DEV)
    out, ids, w, counts = moe.layer(f(wl.x), f(wl.w_router), f(wl.bias), wl.k, wl.score,
                                    moe.Experts.from_bank(wl.routed.to(DEV)),
                                    moe.Experts.from_bank(wl.shared.to(DEV)) if wl.shared is not None else None,
                                    out_dtype=torch.float32 if wl.out_dt == "f32" else torch.bfloat16,
                                    want_routing=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["ids"])
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    check_out(out.float().cpu().numpy(), ref["out"], "layer")


# ---------------------------------------------------------------- packed exponents

def _pack_reference(sg, su, sd):
    """The packed layouts of include/moe.h (moe_mx_pack_scales), written out
    with numpy from their definition: byte q = 4 ss + b of lane c*16 + r."""
    n, I, KH = sg.shape
    H = KH * 32
    KI = sd.shape[2]
    gu = np.zeros((n, I // 32, H // 512, 64, 16), np.uint8)
    dn = np.zeros((n, H // 64, I // 512, 64, 16), np.uint8)
    for lane in range(64):
        c, r = lane // 16, lane % 16
        for q in range(16):
            ss, b = q // 4, q % 4
            src = sg if b < 2 else su
            rows = np.arange(I // 32) * 32 + 16 * (b & 1) + r
            cols = 4 * (4 * np.arange(H // 512) + ss) + c
            gu[:, :, :, lane, q] = src[:, rows][:, :, cols]
            rows = np.arange(H // 64) * 64 + 16 * b + r
            cols = 4 * (4 * np.arange(I // 512) + ss) + c
            dn[:, :, :, lane, q] = sd[:, rows][:, :, cols]
    return gu.reshape(-1), dn.reshape(-1)


def test_pack_mx_scales_layout():
    """The packing kernel against the layout's definition, byte for byte
    (a non-square bank: H = 2048, I = 1024, three experts)."""
    wl = synth.make_grouped([3, 1, 2], 0, 2048, 1024, dt="mxfp4", seed=77)
    bank = wl.routed
    ex = moe.Experts.from_bank(bank.to(DEV))
    assert ex.s_gate_up_packed is not None and ex.s_down_packed is not None
    torch.cuda.synchronize()
    gu_ref, dn_ref = _pack_reference(bank.s_gate.numpy(), bank.s_up.numpy(), bank.s_down.numpy())
    np.testing.assert_array_equal(ex.s_gate_up_packed.cpu().numpy(), gu_ref)
    np.testing.assert_array_equal(ex.s_down_packed.cpu().numpy(), dn_ref)


PACKED_CASES = [
    # 16-row tiles with packed exponents: groups of 1..32 rows, an empty expert, the shared expert
    ([1, 5, 16, 17, 32, 3, 0, 9], 20, 1024, 512),
    # a shared group of 100 rows (joins the 16-row tiles: fewer than five groups of 33..256 rows)
    ([4, 60], 100, 2048, 1024),
    # H = 8192: the tile's activation rows and the partial sums of the eight-wave
    # gate/up workgroup exceed LDS, so the four-wave kernel takes the tiles
    ([3, 20, 1], 10, 8192, 512),
]


@pytest.mark.parametrize("gm,sm,H,I", PACKED_CASES)
def test_grouped_ffn_mxfp4_packed_exponents(gm, sm, H, I):
    """Banks with packed exponents: outputs within the fp8 tolerance of the
    oracle and bit-identical to the same banks without them."""
    print(f"grouped mxfp4 packed gm={gm} sm={sm} H={H} I={I}", flush=True)
    wl = synth.make_grouped(gm, sm, H, I, dt="mxfp4", seed=sum(gm) + 3 * sm)
    ref = om.grouped_ffn(wl)
    R = int(sum(gm))
    a, a_e = moe.quant_mxfp8(wl.x.to(DEV))
    offs = torch.tensor(np.concatenate([[0], np.cumsum(gm)]), dtype=torch.int32, device=DEV)
    outs = []
    for pack in (True, False):
        routed = moe.Experts.from_bank(wl.routed.to(DEV), pack=pack)
        shared = moe.Experts.from_bank(wl.shared.to(DEV), pack=pack)
        assert (routed.s_gate_up_packed is not None) == pack
        outs.append(moe.grouped_ffn(a, offs, routed, a_scale=a_e, R_max=R, a_sh=a[R:], a_sh_scale=a_e[R:],
                                    shared=shared, y_dtype=torch.float32))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    yc = outs[0][0].cpu().numpy()
    starts = np.concatenate([[0], np.cumsum(gm)])
    for g in range(len(gm)):
        if gm[g]:
            check_out(yc[starts[g]:starts[g + 1]], ref[g][1], f"group {g}")
    check_out(outs[0][1].cpu().numpy(), ref["shared"][1], "shared")


def test_layer_mxfp4_packed_exponents():
    """The fused layer with packed exponents equals the layer without them."""
    wl = synth.make_layer(64, 1024, 32, 4, 512, w_dt="mxfp4", seed=99, out_dt="f32", score="sigmoid", shared=True)
    ref = om.moe_layer(wl)
    f = lambda t: None if t is None else t.to(DEV)
    outs = []
    for pack in (True, False):
        outs.append(moe.layer(f(wl.x), f(wl.w_router), f(wl.bias), wl.k, wl.score,
                              moe.Experts.from_bank(wl.routed.to(DEV), pack=pack),
                              moe.Experts.from_bank(wl.shared.to(DEV), pack=pack), out_dtype=torch.float32))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    check_out(outs[0].cpu().numpy(), ref["out"], "layer packed")


def test_grouped_ffn_mxfp4_packed_many_tiles():
    """Packed exponents where each persistent workgroup takes several tiles
    in a row: bit-identical to the same banks without packed exponents.
    48 experts of 0..32 rows and a shared group of 100 rows at H = 7168,
    I = 1024, about 65 m-tiles: ~1800 down and ~520 gate/up tiles.  Random
    E2M1 bytes and E8M0 exponents 2^-9 .. 2^-1, generated on the device."""
    n, S, H, I = 48, 100, 7168, 1024
    g = torch.Generator(device=DEV)
    g.manual_seed(1234)
    gm = torch.randint(0, 33, (n,), generator=g, device=DEV).cpu().numpy()
    gm[5] = 0
    R = int(gm.sum())
    print(f"grouped mxfp4 packed many tiles R={R} S={S} H={H} I={I}", flush=True)

    def bank(e):
        u8 = lambda *s: torch.randint(0, 256, s, generator=g, device=DEV, dtype=torch.uint8)
        ex = lambda *s: torch.randint(118, 127, s, generator=g, device=DEV, dtype=torch.uint8)
        return moe.Experts(u8(e, I, H // 2), u8(e, I, H // 2), u8(e, H, I // 2),
                           ex(e, I, H // 32), ex(e, I, H // 32), ex(e, H, I // 32), moe.MXFP4)

    routed, shared = bank(n), bank(1)
    x = torch.randn(R + S, H, generator=g, device=DEV).to(torch.bfloat16)
    a, a_e = moe.quant_mxfp8(x)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(gm)]), dtype=torch.int32, device=DEV)
    outs = []
    for r, s in ((routed.pack_mx_scales(), shared.pack_mx_scales()), (routed, shared)):
        outs.append(moe.grouped_ffn(a, offs, r, a_scale=a_e, R_max=R, a_sh=a[R:], a_sh_scale=a_e[R:],
                                    shared=s, y_dtype=torch.float32))
    torch.cuda.synchronize()
    assert outs[0][0].abs().max().item() > 0 and torch.isfinite(outs[0][0]).all()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])

