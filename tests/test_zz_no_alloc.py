"""moe_layer_noalloc (the fused layer with the library's static scratch)
against moe_layer (caller workspace): the same kernels on the same inputs, so
every output must be bitwise equal.  Two calls in a row on one GPU, the second
with fewer tokens, so the second runs on the scratch the first left behind;
then a call too large for the scratch is refused before any launch."""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import routed_expert_ffn_04_amd as moe  # noqa: E402
import synth  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _layer_inputs(wl):
    return (wl.x, wl.w_router, wl.bias, wl.k, wl.score, moe.Experts.from_bank(wl.routed),
            moe.Experts.from_bank(wl.shared) if wl.shared is not None else None)


@pytest.mark.parametrize("w_dt,out_dt", [("bf16", torch.float32), ("e4m3", torch.bfloat16)])
def test_noalloc_layer_equals_workspace_layer_twice(w_dt, out_dt):
    # the DeepSeek-V3 layer shape at decode size, then a smaller batch
    full = synth.make_layer(128, 7168, 256, 8, 2048, x_dt="bf16", w_dt=w_dt,
                            out_dt="f32" if out_dt == torch.float32 else "bf16", seed=41, device=DEV)
    for T in (128, 37):
        print(f"noalloc vs workspace layer: weights {w_dt}, T={T}", flush=True)
        x = full.x[:T].contiguous()
        args = (x,) + _layer_inputs(full)[1:]
        ref = moe.layer(*args, out_dtype=out_dt, want_routing=True)
        got = moe.layer_noalloc(*args, out_dtype=out_dt, want_routing=True)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert a.shape == b.shape
            assert torch.equal(a, b)
        assert torch.isfinite(got[0].float()).all()


def test_noalloc_layer_tiny_fp32_after_large():
    wl = synth.config(1, device=DEV)
    args = _layer_inputs(wl)
    ref = moe.layer(*args, out_dtype=torch.float32, want_routing=True)
    got = moe.layer_noalloc(*args, out_dtype=torch.float32, want_routing=True)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_noalloc_refuses_calls_beyond_the_scratch():
    L = moe.lib()
    need = L.moe_layer_workspace_size(1024, 7168, 256, 8, 2048, moe.BF16, moe.BF16, 1, moe.BF16, moe.BF16)
    assert need > 64 << 20
    wl = synth.make_layer(8, 7168, 256, 8, 2048, x_dt="bf16", w_dt="bf16", out_dt="bf16", seed=42, device=DEV)
    x = torch.zeros((1024, 7168), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.layer_noalloc(x, wl.w_router, None, 8, "sigmoid", moe.Experts.from_bank(wl.routed),
                          moe.Experts.from_bank(wl.shared), out_dtype=torch.bfloat16)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    assert "static array" in str(ei.value)
