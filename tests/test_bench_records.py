"""Host-side pieces of the benchmark's records (no GPU): the routing-input
dump that the counter runs replay, and the traffic record lookup."""
import json
import os

import pytest
import torch

import bench
import synth
from measure import accounting


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_routing_inputs_match_config(cid, monkeypatch):
    """synth.routing_inputs(cid) holds the same tokens, router and bias as
    synth.config(cid) (banks stubbed out: their values do not enter routing)."""
    monkeypatch.setattr(synth, "_bank", lambda *a, **k: None)
    T = 64 if cid == 1 else 32
    wl = synth.config(cid, T=T)
    r = synth.routing_inputs(cid)
    assert (r["H"], r["E"], r["k"], r["I"]) == (wl.H, wl.E, wl.k, wl.I)
    assert (r["x_dt"], r["w_dt"], r["out_dt"], r["score"]) == (wl.x_dt, wl.w_dt, wl.out_dt, wl.score)
    assert r["shared"] == (cid != 1)
    # the token draw of row t does not depend on T: compare the first rows
    assert torch.equal(r["x"][:T], wl.x)
    assert torch.equal(r["w_router"], wl.w_router)
    if wl.bias is None:
        assert r["bias"] is None
    else:
        assert torch.equal(r["bias"], wl.bias)


def test_dump_inputs_layout(tmp_path):
    bench.dump_inputs(1, str(tmp_path))
    meta = dict(line.split(" ", 1) for line in open(tmp_path / "meta.txt").read().splitlines())
    assert meta["kind"] == "layer" and meta["T"] == "64" and meta["E"] == "8" and meta["bias"] == "0"
    r = synth.routing_inputs(1)
    assert os.path.getsize(tmp_path / "x.bin") == r["x"].numel() * 4
    assert os.path.getsize(tmp_path / "w_router.bin") == r["w_router"].numel() * 4
    bench.dump_inputs(2, str(tmp_path / "m"), mxfp4=True)
    meta = dict(line.split(" ", 1) for line in open(tmp_path / "m" / "meta.txt").read().splitlines())
    assert meta["w_dt"] == "mxfp4" and meta["x_dt"] == "bf16" and meta["T"] == "128"
    bench.dump_inputs(4, str(tmp_path / "g"))
    meta = dict(line.split(" ", 1) for line in open(tmp_path / "g" / "meta.txt").read().splitlines())
    assert meta["kind"] == "grouped" and len(meta["groups"].split()) == 9


def test_traffic_lookup_requires_matching_sources(tmp_path, monkeypatch):
    rec = {"sources_sha256": "abc", "workloads": {"w": {"bytes": 123}}}
    (tmp_path / "profiles").mkdir()
    with open(tmp_path / "profiles" / "traffic.json", "w") as f:
        json.dump(rec, f)
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    monkeypatch.setattr(accounting, "sources_digest", lambda: "abc")
    assert bench.measured_traffic("w") == 123
    assert bench.measured_traffic("other") is None
    monkeypatch.setattr(accounting, "sources_digest", lambda: "changed")
    assert bench.measured_traffic("w") is None


def test_sources_digest_is_stable():
    assert accounting.sources_digest() == accounting.sources_digest()
    assert len(accounting.sources_digest()) == 64


def test_sources_digest_covers_grouped_ffn_only():
    # the digest keys the grouped-FFN traffic record: it covers the grouped-FFN
    # kernels and the C ABI, not the router / permute / quant / combine kernels
    assert accounting._gffn_source("gffn_big.hip") and accounting._gffn_source("gffn_common.h")
    assert accounting._gffn_source("api.cpp") and accounting._gffn_source("moe.h")
    for other in ("route.hip", "permute.hip", "quant.hip", "combine.hip", "moe_probe.cpp"):
        assert not accounting._gffn_source(other)
