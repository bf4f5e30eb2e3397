"""GPU parity at the five workloads' full sizes, in the launch configurations
the benchmark times: the layer as its C-ABI calls (bench.LayerRunner /
GroupedRunner), and the fused moe_layer call (bench.FusedRunner), whose output
must equal the five calls' bit for bit.

Routing (expert ids) and the permutation (counts, offsets, src, dest) are
compared bit-exactly over every token against the oracle; routing weights
within 1e-6.  Layer outputs are compared on sampled tokens (or, for the
pre-routed workload, sampled rows of every group) that the oracle computes one
by one: max-abs <= 2e-2 and rel-Frobenius <= 1e-2 for fp32/bf16 weights; for
fp8 weights (e4m3, MXFP4) rel-Frobenius <= 5e-3 and max-abs <= 2^-6 max|ref|
(two bf16 spacings at the largest output).  The fp8 floor measured here is
1e-3 to 2.4e-3: the outputs are bf16, and the matrix cores' fp8 sums differ
from fp64 enough to move a few e4m3 codes of h per row and, through them,
bf16 roundings of the outputs; a dropped 128-wide K block would move a row
by about 1/sqrt(56) (gate/up) to 1/sqrt(16) (down) of its norm.
"""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402
from oracle import moe as om  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _check(got, ref, fp8, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rf = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    ma = float(np.abs(got - ref).max())
    print(f"[{what}] rel_frob={rf:.3e} max_abs={ma:.3e} max|ref|={np.abs(ref).max():.3e}", flush=True)
    assert np.isfinite(got).all()
    if fp8:
        assert rf <= 5e-3 and ma <= 2.0 ** -6 * np.abs(ref).max()
    else:
        assert rf <= 1e-2 and ma <= 2e-2


def _sample(T, n, seed):
    rng = np.random.default_rng(seed)
    return sorted(set([0, T - 1] + rng.choice(T, size=n, replace=False).tolist()))


def _layer_run_and_routing(cid, fp8c, mxfp4):
    """The layer through bench.LayerRunner at full size; routing and the
    permutation checked bit-exactly over every token, and the fused layer
    (bench.FusedRunner) checked to give the same output bits.  Returns
    (wl, run)."""
    print(f"config {cid}{' with the fp8 combine' if fp8c else ''}{' with MXFP4 weights' if mxfp4 else ''}: generating",
          flush=True)
    wl = synth.config_mxfp4(cid, device=DEV) if mxfp4 else synth.config(cid, device=DEV)
    wl.y_dt = "e4m3" if fp8c else None
    run = bench.LayerRunner(wl, DEV, fp8_combine=fp8c)
    for _, f in run.calls():
        f()
    torch.cuda.synchronize()
    ids = run.ids.cpu().numpy()
    print(f"config {cid}: oracle routing over {wl.T} tokens", flush=True)
    x32, wr, b = om.layer_inputs(wl)
    ids_ref, w_ref, _ = om.route(x32, wr, b, wl.k, wl.score)
    np.testing.assert_array_equal(ids, ids_ref)
    assert np.abs(run.w.cpu().numpy() - w_ref).max() <= 1e-6
    counts, offsets, src, dest = om.permute(ids_ref, wl.E)
    np.testing.assert_array_equal(run.counts.cpu().numpy(), counts)
    np.testing.assert_array_equal(run.offsets.cpu().numpy(), offsets)
    np.testing.assert_array_equal(run.src.cpu().numpy(), src)
    np.testing.assert_array_equal(run.dest.cpu().numpy(), dest)
    fused = bench.FusedRunner(run, DEV)
    for _, f in fused.calls():
        f()
    torch.cuda.synchronize()
    assert torch.equal(fused.out, run.out), "fused layer differs from the five calls"
    del fused
    return wl, run


@pytest.mark.parametrize("cid,nsample,fp8c,mxfp4", [(1, None, False, False), (2, 16, False, False),
                                                    (3, 6, False, False), (2, 16, False, True)])
def test_layer_config_full_size(cid, nsample, fp8c, mxfp4):
    wl, run = _layer_run_and_routing(cid, fp8c, mxfp4)
    out = run.out.float().cpu().numpy()
    fp8 = wl.w_dt in ("e4m3", "mxfp4")
    if nsample is None:
        ref = om.moe_layer(wl)
        _check(out, ref["out"], fp8, f"config {cid} all tokens")
    else:
        toks = _sample(wl.T, nsample, cid)
        print(f"config {cid}: oracle outputs for tokens {toks}", flush=True)
        ref = om.moe_layer_tokens(wl, toks)
        np.testing.assert_array_equal(ref["ids"], run.ids.cpu().numpy()[toks])
        _check(out[toks], ref["out"], fp8, f"config {cid} tokens {toks}")


# worker processes for the oracle's sampled outputs (its experts spread over
# them); a dozen leaves the card's process budget and the host share alone
ORACLE_PROCS = max(1, min(12, os.cpu_count() or 1))


def _tail_tokens(offsets, src, k, n_min, seed):
    """Sample tokens that reach every expert's last rows: the token of the
    last row of each expert's segment (the high end of the segment, which
    lies in the group's last, partial m-tile whenever the group spans more
    than one), then random tokens up to n_min, plus tokens 0 and T-1."""
    T = len(src) // k
    toks = {0, T - 1}
    for e in range(len(offsets) - 1):
        if offsets[e + 1] > offsets[e]:
            toks.add(int(src[offsets[e + 1] - 1]) // k)
    rng = np.random.default_rng(seed)
    while len(toks) < n_min:
        toks.add(int(rng.integers(T)))
    return sorted(toks)


@pytest.mark.parametrize("fp8c,mxfp4", [(False, False), (True, False), (False, True)])
def test_prefill_layer_full_size_every_expert(fp8c, mxfp4):
    """The T = 16384 fp8 layer (e4m3 weights; the same with the fp8 combine;
    MXFP4 weights) at full size in the benchmark's launch configuration:
    outputs of at least 256 tokens, among them for every expert the token of
    its segment's last row, so every group's last m-tile (partial or full)
    and every expert's weights are checked."""
    wl, run = _layer_run_and_routing(5, fp8c, mxfp4)
    out = run.out.float().cpu().numpy()
    offsets = run.offsets.cpu().numpy()
    src = run.src.cpu().numpy()
    toks = _tail_tokens(offsets, src, wl.k, 256, 55)
    covered = set(int(e) for e in run.ids.cpu().numpy()[toks].reshape(-1))
    assert covered == set(range(wl.E))
    print(f"config 5: oracle outputs for {len(toks)} tokens over {ORACLE_PROCS} processes", flush=True)
    ref = om.moe_layer_tokens(wl, toks, procs=ORACLE_PROCS)
    _check(out[toks], ref["out"], True, f"config 5 {len(toks)} tokens")


@pytest.mark.parametrize("cid,fp8c,mxfp4", [(3, False, False), (5, False, False), (5, True, False),
                                            (5, False, True)])
def test_layer_full_size_all_tokens_deterministic(cid, fp8c, mxfp4):
    """Two runs of the full-size layer give the same bits in every token's
    output (and in the routed expert outputs)."""
    wl = synth.config_mxfp4(cid, device=DEV) if mxfp4 else synth.config(cid, device=DEV)
    wl.y_dt = "e4m3" if fp8c else None
    run = bench.LayerRunner(wl, DEV, fp8_combine=fp8c)
    outs, ys = [], []
    for _ in range(2):
        for _, f in run.calls():
            f()
        torch.cuda.synchronize()
        outs.append(run.out.clone())
        ys.append(run.y.clone())
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(ys[0], ys[1])


def test_grouped_config_full_size():
    print("config 4: generating", flush=True)
    wl = synth.config(4, device=DEV)
    run = bench.GroupedRunner(wl, DEV)
    for _, f in run.calls():
        f()
    torch.cuda.synchronize()
    y = run.y.float().cpu().numpy()
    y_sh = run.y_sh.float().cpu().numpy()
    rng = np.random.default_rng(4)
    sample = {}
    for g, m in enumerate(wl.group_m):
        sample[g] = sorted(set([0, m - 1] + rng.choice(m, 2, replace=False).tolist()))
    sample["shared"] = sorted(set([0, wl.shared_m - 1] + rng.choice(wl.shared_m, 2, replace=False).tolist()))
    print("config 4: oracle rows", flush=True)
    ref = om.grouped_ffn(wl, group_sample=sample)
    starts = np.concatenate([[0], np.cumsum(wl.group_m)])
    got, want = [], []
    for g in range(len(wl.group_m)):
        rows, yr = ref[g]
        got.append(y[starts[g] + rows])
        want.append(yr)
    rows, yr = ref["shared"]
    got.append(y_sh[rows])
    want.append(yr)
    _check(np.concatenate(got), np.concatenate(want), True, "config 4 sampled rows")


def test_layer_full_size_is_deterministic():
    wl = synth.config(2, device=DEV)
    run = bench.LayerRunner(wl, DEV)
    outs = []
    for _ in range(2):
        for _, f in run.calls():
            f()
        torch.cuda.synchronize()
        outs.append(run.out.clone())
    assert torch.equal(outs[0], outs[1])
