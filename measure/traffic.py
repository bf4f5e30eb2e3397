"""Measured HBM traffic of the grouped FFN per call, for the benchmark's
roofline record.

Build the probe beside this file on any machine with hipcc, after the
library (python -m measure.traffic --build), then run on a machine with the
GPU (the parent process never touches it):

    python -m measure.traffic --configs 2 5

For every workload it writes the routing inputs (bench.py --dump-inputs),
then runs the native probe (no torch) on exactly that routing under two
rocprofv3 counter passes, FETCH_SIZE and WRITE_SIZE, and sums the counters of
the grouped-FFN kernels per call.  The counters are scaled by what they read
for a plain device copy of 1 GiB (probe mode "copy"), so the figures are
bytes.  A third pass reads SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE: the
fraction of SIMD cycles the matrix cores were busy during the grouped-FFN
kernels is busy / (active / XCDS x CUs x 4 SIMDs), GRBM_GUI_ACTIVE being
summed over the accelerator dies (each has its own graphics register bus
manager).  At T = 16384 this gives about 0.31 for 1.31 PFLOP/s, i.e. about
4.2 PFLOP/s at full occupancy of the matrix cores, the rate that
register-only MFMA loops reach on this chip.  The result goes to
profiles/traffic.json together with a digest of the kernel sources; bench.py
reports the figures only while the sources still match that digest.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from measure.accounting import sources_digest  # noqa: E402

PROBE = os.path.join(HERE, "moe_probe")
LIBDIR = os.path.join(ROOT, "routed_expert_ffn_04_amd")


def build_probe() -> str:
    """Compile moe_probe.cpp against the built library (hipcc, gfx950)."""
    from routed_expert_ffn_04_amd import build as libbuild
    cmd = [libbuild.HIPCC, *libbuild.FLAGS, "-I", libbuild.INCLUDE, os.path.join(HERE, "moe_probe.cpp"),
           "-o", PROBE + ".tmp", "-L", LIBDIR, "-lmoe_gfx950", "-Wl,-rpath,$ORIGIN/../routed_expert_ffn_04_amd"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"moe_probe build failed:\n{r.stderr}")
    os.replace(PROBE + ".tmp", PROBE)
    return PROBE
GFFN_KERNELS = ("moe::stream_", "moe::tile_", "moe::mid_kernel", "moe::big_kernel", "moe::mx_", "moe::mxbig_kernel",
                "moe::gffn_build_lists")
NOT_GFFN = ("moe::mx_pack_",)   # exponent packing: once per bank at weight-load time, not per call
XCDS = 8          # MI355X accelerator dies
NAMES = {
    1: "tiny-fp32-T64-H256-E8-top2",
    2: "dsv3-decode-bf16-T128-H7168-E256+1-top8",
    3: "dsv3-skew-bf16-T4096-H7168-E256+1-top8-zipf1.2",
    4: "ep-prefill-share-fp8-9+1groups-H7168-I2048",
    5: "dsv3-prefill-fp8-T16384-H7168-E256+1-top8",
}
MXFP4_NAMES = {2: "dsv3-decode-mxfp4-T128-H7168-E256+1-top8", 3: "dsv3-skew-mxfp4-T4096-H7168-E256+1-top8-zipf1.2",
               5: "dsv3-prefill-mxfp4-T16384-H7168-E256+1-top8"}


def run(cmd, log):
    with open(log, "w") as f:
        r = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, timeout=300)
    if r.returncode != 0:
        with open(log) as f:
            tail = f.read()[-2000:]
        raise RuntimeError(f"{' '.join(cmd)} failed ({r.returncode}):\n{tail}")


def counter_sums(out_dir, by_counter=False):
    """{kernel name: [per-dispatch counter values]} of one pass (summed over
    counters), or {kernel name: {counter: [per-dispatch values]}}."""
    files = glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise RuntimeError(f"no counter file under {out_dir}")
    per = {}
    for fn in files:
        for r in csv.DictReader(open(fn)):
            key = r["Counter_Name"] if by_counter else ""
            d = per.setdefault(r["Kernel_Name"], {}).setdefault(key, {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if by_counter:
        return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in per.items()}
    return {k: list(cs[""].values()) for k, cs in per.items()}


def pmc_pass(counters, probe_args, work, tag):
    """One rocprofv3 counter pass (space-separated counters of one pass)."""
    out = os.path.join(work, f"{tag}_{counters.split()[0]}")
    shutil.rmtree(out, ignore_errors=True)
    cmd = ["rocprofv3", "--pmc", *counters.split(), "--output-format", "csv", "-d", out, "-o", "run", "--", PROBE,
           *probe_args]
    run(["timeout", "-s", "KILL", "120", *cmd], out + ".log")
    return counter_sums(out, by_counter=len(counters.split()) > 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--configs", type=int, nargs="*", default=[2, 5])
    ap.add_argument("--fp8-combine-configs", type=int, nargs="*", default=[],
                    help="fp8 layer workloads to measure also with the FP8 combine")
    ap.add_argument("--mxfp4-configs", type=int, nargs="*", default=[],
                    help="layer workloads to measure also with MXFP4 expert weights")
    ap.add_argument("--calls", type=int, default=2, help="timed calls per probe run (one more is the warm-up)")
    ap.add_argument("--work", default="/tmp/moe_traffic", help="scratch (dumped inputs, raw counter files)")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    ap.add_argument("--build", action="store_true", help="only compile the probe (no GPU needed)")
    args = ap.parse_args()
    if args.build:
        print(build_probe())
        return
    if not os.path.exists(PROBE):
        raise SystemExit(f"{PROBE} is missing: build it first (python -m measure.traffic --build)")
    os.makedirs(args.work, exist_ok=True)
    os.environ.setdefault("TMPDIR", "/tmp")

    # calibration: a 1 GiB device copy (probe: one untimed + `calls` timed copies)
    gib = float(1 << 30)
    cal = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        per = pmc_pass(counter, ["copy", str(args.calls)], args.work, "copy")
        vals = [v for k, v in per.items() if "copy_u4" in k][0]
        kib = sum(vals) / len(vals)
        cal[counter] = {"kib_per_gib_copy": kib, "bytes_per_kib": gib / kib}
        print(f"calibration {counter}: {kib:.0f} KiB per 1 GiB copy -> {gib / kib:.1f} bytes per KiB", flush=True)

    cus = int(subprocess.run([sys.executable, "-c", "import torch; print(torch.cuda.get_device_properties(0).multi_processor_count)"],
                             capture_output=True, text=True, timeout=300).stdout.strip().splitlines()[-1])
    result = {"sources_sha256": sources_digest(), "calibration": cal, "compute_units": cus, "workloads": {}}
    runs = ([(c, "") for c in args.configs] + [(c, "fp8c") for c in args.fp8_combine_configs]
            + [(c, "mxfp4") for c in args.mxfp4_configs])
    for cid, var in runs:
        fp8c = var == "fp8c"
        tag = f"c{cid}" + {"": "", "fp8c": "f", "mxfp4": "m"}[var]
        flag = {"": [], "fp8c": ["--fp8-combine"], "mxfp4": ["--mxfp4"]}[var]
        d = os.path.join(args.work, f"inputs_{tag}")
        run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", str(cid), "--dump-inputs", d] + flag,
            os.path.join(args.work, f"dump_{tag}.log"))
        ncalls = args.calls + 1
        rec = {"calls": ncalls, "kernels": {}}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            per = pmc_pass(counter, ["file", d, str(args.calls)], args.work, tag)
            tot = 0.0
            for k, vals in per.items():
                if not any(s in k for s in GFFN_KERNELS) or any(s in k for s in NOT_GFFN):
                    continue
                b = sum(vals) / ncalls * cal[counter]["bytes_per_kib"]
                rec["kernels"].setdefault(k, {})[counter] = round(b)
                tot += b
            rec[counter.lower().replace("_size", "_bytes")] = round(tot)
        rec["bytes"] = rec["fetch_bytes"] + rec["write_bytes"]
        per = pmc_pass("SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE", ["file", d, str(args.calls)], args.work, tag + "_mfma")
        busy = active = 0.0
        for k, vals in per.items():
            if any(s in k for s in GFFN_KERNELS):
                busy += sum(vals["SQ_VALU_MFMA_BUSY_CYCLES"])
                active += sum(vals["GRBM_GUI_ACTIVE"])
        rec["mfma_busy_cycles"] = round(busy / ncalls)
        rec["grbm_gui_active"] = round(active / ncalls)
        rec["mfma_busy_frac"] = round(busy / (active / XCDS * cus * 4), 4) if active else None
        rec["command"] = (f"python -m measure.traffic --configs {' '.join(map(str, args.configs))}"
                          + (f" --fp8-combine-configs {' '.join(map(str, args.fp8_combine_configs))}"
                             if args.fp8_combine_configs else "")
                          + (f" --mxfp4-configs {' '.join(map(str, args.mxfp4_configs))}"
                             if args.mxfp4_configs else "")
                          + f" (probe: moe_probe file <dump of bench.py --config {cid}"
                          + "".join(" " + f for f in flag) + f"> {args.calls})")
        name = MXFP4_NAMES[cid] if var == "mxfp4" else NAMES[cid] + ("+fp8-combine" if fp8c else "")
        result["workloads"][name] = rec
        print(f"config {cid} {var}: grouped FFN per call: fetch {rec['fetch_bytes'] / 1e9:.3f} GB, "
              f"write {rec['write_bytes'] / 1e9:.3f} GB", flush=True)
    os.makedirs(os.path.dirname(args.out), exist_ok=True)
    with open(args.out, "w") as f:
        json.dump(result, f, indent=1)
    print(f"wrote {args.out}")


if __name__ == "__main__":
    main()
