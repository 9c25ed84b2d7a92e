#!/usr/bin/env python3
"""A short run of each hot kernel for profiler counter passes (rocprofv3
--pmc ...): few dispatches, each of a known workload, so a counter run
takes seconds.

  decode GEMV, one token:     gate_up 17408x5120 and down 5120x17408, both
                              packings (bgg_ternary_gemv, M = 1)
  decode GEMV, eight tokens:  the same matrices at M = 8
  prefill GEMM:               4096 tokens x the same matrices, both packings
                              (bgg_ternary_gemm on x' given rotated)
  transform:                  bgg_hadamard_rotate, 4096 x 17408
  calibration:                the probe's streaming read and write of
                              --calib MiB (known bytes for FETCH_SIZE /
                              WRITE_SIZE)

With --decode-layer it runs instead one layer of the 64-layer decode step
(q, k, v, o, gate, up, down at one token, both packings, each call on its
own weight copy) --reps times, plus the calibration: every decode kernel
then gets the same mix of shapes per dispatch as in the step, so its
per-dispatch counters compare with the step's bytes per launch.

Each workload runs --reps times over --copies weight copies (so the weights
come from HBM).  Inputs are the benchmark's seeded synthetic ones.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--reps", type=int, default=4)
    ap.add_argument("--copies", type=int, default=24)
    ap.add_argument("--calib", type=int, default=256, metavar="MIB")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--decode-layer", action="store_true")
    args = ap.parse_args()

    import torch

    import bit_gemv_gemm_amd as bgg
    import synth
    from bit_gemv_gemm_amd import probe

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.decode_layer:
        decode_layer(args, torch, bgg, synth, dev, stream)
        calibrate(args, torch, probe, dev)
        return 0
    pw = synth.WORKLOADS["projection"]
    for mat in pw["matrices"]:
        T, S = synth.workload_matrix(mat, pw["seed"])
        x = torch.from_numpy(synth.workload_x(pw["seed"], 8, mat.k)).to(dev)
        y = torch.empty((8, mat.n), dtype=torch.float16, device=dev)
        for fmt in ("PQ2_0", "PTQ1_0"):
            d = bgg.bgg_describe(fmt, mat.n, mat.k)
            host = bgg.bgg_pack_weights(d, T, S)
            copies = [bgg.upload(host, dev) for _ in range(args.copies)]
            ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d, 8), dev)
            for M in (1, 8):
                print(f"gemv {fmt} {mat.name} M={M}: {bgg.bgg_gemv_kernel_name(d, M)}", flush=True)
                for r in range(args.reps):
                    bgg.bgg_ternary_gemv(d, copies[r % args.copies], x, y, M, bgg.BGG_ROTATE_INPUT, ws, stream)
                torch.cuda.synchronize()
            del copies
        del T, S
    if not args.no_gemm:
        gw = synth.WORKLOADS["prefill"]
        M = gw["m"][0]
        for mat in gw["matrices"]:
            T, S = synth.workload_matrix(mat, gw["seed"])
            x = torch.from_numpy(synth.workload_x(gw["seed"], M, mat.k)).to(dev)
            xr = torch.empty_like(x)
            y = torch.empty((M, mat.n), dtype=torch.float16, device=dev)
            print(f"transform {M}x{mat.k}", flush=True)
            for _ in range(args.reps):
                bgg.bgg_hadamard_rotate(x, xr, M, mat.k, stream)
            for fmt in ("PQ2_0", "PTQ1_0"):
                d = bgg.bgg_describe(fmt, mat.n, mat.k)
                packed = bgg.upload(bgg.bgg_pack_weights(d, T, S), dev)
                wsg = bgg.workspace(bgg.bgg_gemm_workspace_size(d, M), dev)
                print(f"gemm {fmt} {M}x{mat.k}->{mat.n}", flush=True)
                for _ in range(args.reps):
                    bgg.bgg_ternary_gemm(d, packed, xr, y, M, 0, wsg, stream)
                torch.cuda.synchronize()
                del packed, wsg
            del T, S, x, xr, y
    calibrate(args, torch, probe, dev)
    return 0


def decode_layer(args, torch, bgg, synth, dev, stream) -> None:
    """One layer of the decode step per packing, --reps times (each call
    of a repetition on its own weight copy, as the step's layers are)."""
    w = synth.WORKLOADS["decode_step"]
    layer = synth.decode_stack(1)
    for fmt in ("PQ2_0", "PTQ1_0"):
        calls = []
        for mat in layer:
            T, S = synth.workload_matrix(mat, w["seed"])
            d = bgg.bgg_describe(fmt, mat.n, mat.k)
            host = bgg.bgg_pack_weights(d, T, S)
            copies = [bgg.upload(host, dev) for _ in range(args.reps)]
            x = torch.from_numpy(synth.workload_x(w["seed"], 1, mat.k)).to(dev)
            y = torch.empty((1, mat.n), dtype=torch.float16, device=dev)
            calls.append((mat.name, d, copies, x, y))
            del T, S, host
        ws = bgg.workspace(max(bgg.bgg_gemv_workspace_size(d, 1) for _, d, _, _, _ in calls), dev)
        for name, d, _, _, _ in calls:
            print(f"decode layer {fmt} {name} {int(d.N)}x{int(d.K)}: {bgg.bgg_gemv_kernel_name(d, 1)}", flush=True)
        for r in range(args.reps):
            for _, d, copies, x, y in calls:
                bgg.bgg_ternary_gemv(d, copies[r], x, y, 1, bgg.BGG_ROTATE_INPUT, ws, stream)
        torch.cuda.synchronize()
        del calls, ws


def calibrate(args, torch, probe, dev) -> None:
    cb = torch.empty(args.calib << 20, dtype=torch.uint8, device=dev)
    sink = probe.sink(dev)
    print(f"calibration: probe read and write of {args.calib} MiB", flush=True)
    for _ in range(args.reps):
        probe.read(cb, sink)
        probe.write(cb)
    torch.cuda.synchronize()
    print("done", flush=True)


if __name__ == "__main__":
    sys.exit(main())
