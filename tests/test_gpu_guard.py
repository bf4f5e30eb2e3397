"""Guard bands around every buffer the layer's calls write.

Each output, routing buffer and workspace of the benchmark's launch
configuration (bench.LayerRunner / GroupedRunner, full sizes) and of the
fused entry point is carved out of a larger allocation whose 64 KiB before
and after (and the alignment slack) hold a byte pattern; after the calls the
pattern must be intact, and the outputs must equal those of the same calls
on plain allocations bit for bit."""
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import routed_expert_ffn_04_amd as moe  # noqa: E402
import synth  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GUARD = 1 << 16
PATTERN = 0xA5


class Guarded:
    """A tensor of the given shape and dtype inside a guarded byte buffer."""

    def __init__(self, like: torch.Tensor):
        self.n = like.numel() * like.element_size()
        span = (self.n + 255) // 256 * 256
        self.raw = torch.full((GUARD + span + GUARD,), PATTERN, dtype=torch.uint8, device=like.device)
        self.t = self.raw[GUARD:GUARD + self.n].view(like.dtype).view(like.shape)

    def intact(self) -> bool:
        return bool((self.raw[:GUARD] == PATTERN).all()) and bool((self.raw[GUARD + self.n:] == PATTERN).all())


LAYER_BUFFERS = ("ws_route", "ws_perm", "ws_ffn", "ids", "w", "counts", "offsets", "src", "dest", "xq", "xs",
                 "y", "y_scale", "y_sh", "out")
OUTPUTS = ("ids", "w", "counts", "offsets", "src", "dest", "y", "y_sh", "out")


def _guard(run, names):
    guards = {}
    for n in names:
        t = getattr(run, n, None)
        if t is None:
            continue
        guards[n] = Guarded(t)
        setattr(run, n, guards[n].t)
    return guards


def _run(run):
    for _, f in run.calls():
        f()
    torch.cuda.synchronize()


@pytest.mark.parametrize("cid,fp8c,mxfp4", [(2, False, False), (2, False, True), (3, False, False),
                                            (5, False, False), (5, True, False), (5, False, True)])
def test_layer_calls_write_inside_their_buffers(cid, fp8c, mxfp4):
    print(f"config {cid} fp8c={fp8c} mxfp4={mxfp4}", flush=True)
    wl = synth.config_mxfp4(cid, device=DEV) if mxfp4 else synth.config(cid, device=DEV)
    wl.y_dt = "e4m3" if fp8c else None
    plain = bench.LayerRunner(wl, DEV, fp8_combine=fp8c)
    _run(plain)
    run = bench.LayerRunner(wl, DEV, fp8_combine=fp8c)
    guards = _guard(run, LAYER_BUFFERS)
    _run(run)
    bad = [n for n, g in guards.items() if not g.intact()]
    assert not bad, f"writes outside {bad}"
    for n in OUTPUTS:
        if getattr(plain, n, None) is not None:
            assert torch.equal(getattr(run, n), getattr(plain, n)), n


def test_grouped_call_writes_inside_its_buffers():
    wl = synth.config(4, device=DEV)
    plain = bench.GroupedRunner(wl, DEV)
    _run(plain)
    run = bench.GroupedRunner(wl, DEV)
    guards = _guard(run, ("ws", "y", "y_sh"))
    _run(run)
    bad = [n for n, g in guards.items() if not g.intact()]
    assert not bad, f"writes outside {bad}"
    assert torch.equal(run.y, plain.y) and torch.equal(run.y_sh, plain.y_sh)


@pytest.mark.parametrize("w_dt,y_fp8", [("bf16", False), ("e4m3", False), ("e4m3", True), ("mxfp4", False)])
def test_fused_layer_writes_inside_its_buffers(w_dt, y_fp8):
    wl = synth.make_layer(700, 1024, 32, 4, 512, w_dt=w_dt, out_dt="bf16", seed=31, device=DEV)
    routed = moe.Experts.from_bank(wl.routed)
    shared = moe.Experts.from_bank(wl.shared)
    ydt = torch.uint8 if y_fp8 else None
    ref = moe.layer(wl.x, wl.w_router, wl.bias, wl.k, wl.score, routed, shared, out_dtype=torch.bfloat16,
                    y_dtype=ydt)
    rs = routed.struct()
    need = moe.layer_workspace_size(wl.T, wl.H, wl.E, wl.k, wl.I, moe._dt_of(wl.x), rs.dt, True,
                                    moe._dt_of(ref), moe.E4M3 if y_fp8 else None)
    g_out = Guarded(torch.empty_like(ref))
    g_ws = Guarded(torch.empty(need, dtype=torch.uint8, device=DEV))
    moe.layer(wl.x, wl.w_router, wl.bias, wl.k, wl.score, routed, shared, out_dtype=torch.bfloat16,
              out=g_out.t, ws=g_ws.t, y_dtype=ydt)
    torch.cuda.synchronize()
    assert g_out.intact() and g_ws.intact()
    assert torch.equal(g_out.t, ref)
