"""Grouped-FFN time against rows per group (m_per_group) and group count.

For each weight type (bf16, e4m3, MXFP4) and group count G, G experts of the
DeepSeek-V3 shape (H = 7168, I = 2048) each take m rows, for m from 1 to
2048, and one moe_grouped_ffn call over them is timed (median of the timed
calls, torch events on the launch stream).  Printed per point: the call's
time, its algorithmic bytes / time against the 8 TB/s HBM peak and its
algorithmic FLOPs / time against the MFMA peak of the weight type.  The
rows-per-group axis is the one "DeepSeek V3/R1 Inference Efficiency (2)",
section 1.b, ties grouped-GEMM efficiency to (its m_per_group), and the
table shows where each tile class of the library takes over.

    python -m measure.sweep_groups [--dts bf16 e4m3 mxfp4] [--groups 16 256] [--out FILE]
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import routed_expert_ffn_04_amd as moe  # noqa: E402
import synth  # noqa: E402
from measure import accounting  # noqa: E402

H, I = 7168, 2048
M_LIST = [1, 2, 4, 8, 16, 17, 24, 32, 48, 64, 96, 128, 192, 256, 257, 384, 512, 1024, 2048]
PEAK_TFLOPS = {"bf16": 2500.0, "e4m3": 5000.0, "mxfp4": 5000.0}   # dense MFMA (fp8 x fp4 runs at the fp8 rate)
HBM_GBS = 8000.0


def sub_bank(bank: synth.Bank, G: int) -> synth.Bank:
    f = lambda t: None if t is None else t[:G]
    return synth.Bank(G, bank.H, bank.I, bank.dt, f(bank.w_gate), f(bank.w_up), f(bank.w_down),
                      f(bank.s_gate), f(bank.s_up), f(bank.s_down))


def time_call(fn, warmup: int, steps: int) -> float:
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    return ts[len(ts) // 2]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--dts", nargs="*", default=["bf16", "e4m3", "mxfp4"])
    ap.add_argument("--groups", type=int, nargs="*", default=[16, 256])
    ap.add_argument("--m", type=int, nargs="*", default=M_LIST)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--out", default=None, help="also write the table to this file")
    args = ap.parse_args()
    dev = torch.device("cuda:0")
    moe.lib()
    lines = [f"# grouped FFN, H={H}, I={I}, no shared expert, bf16 y; median of {args.steps} calls after "
             f"{args.warmup} (python -m measure.sweep_groups {' '.join(sys.argv[1:])})",
             f"{'w':>6} {'G':>4} {'m':>5} {'ms':>9} {'GB/s':>8} {'HBM%':>6} {'TFLOP/s':>8} {'MFMA%':>6}"]
    print(lines[0], flush=True)
    print(lines[1], flush=True)
    for dt in args.dts:
        t0 = time.time()
        wl = synth.make_grouped([1] * max(args.groups), 0, H, I, dt=dt, seed=41, device=dev)
        bank = wl.routed
        del wl
        for G in args.groups:
            experts = moe.Experts.from_bank(sub_bank(bank, G))
            for m in args.m:
                R = G * m
                offs = torch.arange(0, R + 1, m, dtype=torch.int32, device=dev)
                x = synth.normal((R, H), 41, synth.ST_X, 1.0, torch.float32, dev)
                if dt == "e4m3":
                    a, a_s = synth.block_quant_e4m3(x, 1, 128)
                elif dt == "mxfp4":
                    a, a_s = moe.quant_mxfp8(x.to(torch.bfloat16))
                else:
                    a, a_s = x.to(torch.bfloat16), None
                del x
                y = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
                L = moe.lib()
                ws = moe._workspace(L.moe_grouped_ffn_workspace_size(R, G, 0, H, I, experts.struct().dt), dev)
                fn = lambda: moe.grouped_ffn(a, offs, experts, a_scale=a_s, R_max=R, y=y, ws=ws)
                ms = time_call(fn, args.warmup, args.steps)
                a_dt = {"bf16": "bf16", "e4m3": "e4m3", "mxfp4": "mxfp8"}[dt]
                nbytes = accounting.grouped_ffn_bytes([m] * G, 0, H, I, a_dt, dt, "bf16")
                flops = accounting.ffn_flops(R, H, I)
                gbs = nbytes / (ms * 1e-3) / 1e9
                tfs = flops / (ms * 1e-3) / 1e12
                line = (f"{dt:>6} {G:>4} {m:>5} {ms:>9.4f} {gbs:>8.1f} {100 * gbs / HBM_GBS:>6.1f} {tfs:>8.1f} "
                        f"{100 * tfs / PEAK_TFLOPS[dt]:>6.1f}")
                lines.append(line)
                print(line, flush=True)
                del a, a_s, y, ws
        del bank
        torch.cuda.empty_cache()
        print(f"# {dt}: {time.time() - t0:.1f} s", flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
