#!/usr/bin/env python3
"""Benchmark of the ternary linear-layer hot path on one MI355X.

Workload of one step (the headline): the full decode-step weight sweep of a
64-layer 27B-class stack at batch 1 -- per layer q 5120->6144, k and v
5120->1024, o 6144->5120, gate and up 5120->17408, down 17408->5120 -- in
both packings, PQ2_0 then PTQ1_0: 2 x 448 calls of bgg_ternary_gemv, each
applying the block-128 Hadamard transform to its own fp16 input and then
the GEMV (the literal 448 transforms + 448 GEMVs per packing; the transform
runs inside the GEMV launch).  Every matrix has its own device buffer
(10.5 GB of packed weights resident, far beyond the 256 MiB Infinity
Cache); inputs are seeded and synthetic (the trit, scale and activation
distributions of the 27B-class stack) and resident in HBM before timing.

value = packed weight bytes of the step (trits + fp16 scales, both
        packings) / wall time of one step.

The calls run one after the other on one stream.  (Running q, k and v at
once on three streams, and gate with up, the most a decoder layer's data
dependencies allow, measured slower: the cross-stream edges of the graph
cost more than the overlap gains.)  Each step is one replay of a captured
HIP graph of its 896 launches (a ctypes call from Python costs as long as a
launch, so eager launching would time the interpreter); --warmup untimed
replays, then exactly --steps timed replays between two device
synchronisations.

Also in the same JSON line:
  roofline      the dominant kernel of the step (the kernel, by name, with
                the largest share of the step's time): packed bytes of its
                launches / their average duration from HIP events around a
                graph of back-to-back launches over the 64 layers' buffers,
                against 8 TB/s; traffic from the committed FETCH_SIZE /
                WRITE_SIZE counters when they were taken on these sources;
  achievable_hbm  a plain streaming read of 2 GiB (this project's probe
                kernel): the rate HBM delivers to a kernel on this machine;
  launch_floor  a kernel that does no work, launched the way the step
                launches its calls (a graph of back-to-back launches on one
                stream): the fixed cost every launch of the step pays, and
                that cost times the step's launches;
  decode_step   per packing: the step's rate, the kernel breakdown, the
                shared-transform and grouped-projection variants, and the
                small-batch sweep M = 2, 4, 8, 16;
  projection    the single-projection workload (gate_up and down);
  prefill_gemm  4096 tokens, TFLOP/s against the fp16 MFMA peak, the
                transform alone over 4 rotating buffer pairs, and a dense
                fp16 GEMM on pre-dequantised weights (torch.matmul) as a
                comparison, run only;
  cpu_baseline  the CPU oracle on a sample of the step, on all host threads
                and on one (with the host CPU's model name);
  context       the pages' end-to-end model figures with their hardware.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
METRIC = "ternary GEMV packed-weight GB/s (% HBM peak) + prefill GEMM TFLOPS (% MFMA)"
FMTS = ("PQ2_0", "PTQ1_0")
PROJ = ("q", "k", "v", "o", "gate", "up", "down")

# End-to-end figures the pages print for the whole model, with their
# hardware: context for the numbers here, not a target.
PAGES_CONTEXT = [
    dict(tok_s=130, hardware="RTX 5090", model="27B, ternary (PQ2_0 file)",
         source="allhereai.com/news/1346 (27B 模型压到 5.95GB…), paragraph on what the size means for hardware"),
    dict(tok_s=30, hardware="NVIDIA L4 (72 W)", model="27B, ternary (PQ2_0 file)",
         source="allhereai.com/news/1346, same paragraph"),
    dict(tok_s=47, hardware="Apple M5 Max", model="27B, ternary (PQ2_0 file)",
         source="allhereai.com/news/1346, same paragraph"),
    dict(tok_s=134, hardware="RTX 5090", model="Ternary-Bonsai-27B (1.71 bpw)",
         source="wmrh.cn/news/471187, section 性能数据"),
    dict(tok_s=58, hardware="Apple M5 Max", model="Ternary-Bonsai-27B (1.71 bpw)",
         source="wmrh.cn/news/471187, section 性能数据"),
]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_gemv_gemm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` (its name as the profiler lists it)
    from the committed counter summary, if that was taken on the current
    kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "gemv_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else int(k["fetch_bytes"] + k["write_bytes"])


def cpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return platform.processor() or "unknown"


def make_capture(torch):
    def capture(fn):
        """A graph of fn(stream), captured after one eager run of fn."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return g
    return capture


def replay_us(torch, g, reps, warm=2):
    """Median wall time of one replay of g (HIP events on the replay
    stream), over `reps` replays after `warm` untimed ones."""
    import numpy as np
    cur = torch.cuda.current_stream()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(cur)
        g.replay()
        b.record(cur)
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    return float(np.median(times))


class Stack:
    """The 64-layer decode stack resident on the device in one packing:
    every projection has its own buffer (the layers repeat layer 0's
    generated values: the bytes streamed and the work do not depend on
    them)."""

    def __init__(self, bgg, torch, dev, fmt, seed, layers, xs, ys, mmax, grouped=False):
        import numpy as np
        import synth
        self.fmt = fmt
        t0 = time.time()
        base = {m.name.split(".")[1]: m for m in synth.decode_stack(1)}
        if not grouped:
            host = {}
            for p in PROJ:
                T, S = synth.workload_matrix(base[p], seed)
                d = bgg.bgg_describe(fmt, base[p].n, base[p].k)
                host[p] = (d, bgg.bgg_pack_weights(d, T, S))
                del T, S
            self.calls = [(p, host[p][0], bgg.upload(host[p][1], dev)) for _ in range(layers) for p in PROJ]
        else:
            # q|k|v and gate|up packed as one matrix each: four calls a layer
            gdefs = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")),
                     ("down", ("down",))]
            host = {}
            for gname, parts in gdefs:
                Ts, Ss = zip(*(synth.workload_matrix(base[q], seed) for q in parts))
                T, S = np.concatenate(Ts), np.concatenate(Ss)
                d = bgg.bgg_describe(fmt, T.shape[0], T.shape[1])
                host[gname] = (d, bgg.bgg_pack_weights(d, T, S))
                del Ts, Ss, T, S
            self.calls = [(g, host[g][0], bgg.upload(host[g][1], dev)) for _ in range(layers)
                          for g, _ in gdefs]
            for _, d, _ in self.calls:
                ys.setdefault(int(d.N), torch.empty((mmax, int(d.N)), dtype=torch.float16, device=dev))
        del host
        self.bytes = sum(int(d.format_bytes) for _, d, _ in self.calls)
        self.weights = sum(int(d.N) * int(d.K) for _, d, _ in self.calls)
        wsb = max(bgg.bgg_gemv_workspace_size(d, mmax) for _, d, _ in self.calls)
        self.ws = bgg.workspace(wsb, dev)
        self.xs, self.ys = xs, ys
        log(f"{fmt} stack{' (grouped)' if grouped else ''}: {self.bytes / 1e9:.3f} GB packed in "
            f"{len(self.calls)} buffers ({time.time() - t0:.1f}s)")

    def step(self, bgg, st, M=1):
        """Every call of the step one after the other on stream st."""
        for _, d, p in self.calls:
            bgg.bgg_ternary_gemv(d, p, self.xs[int(d.K)][:M], self.ys[int(d.N)][:M], M,
                                 bgg.BGG_ROTATE_INPUT, self.ws, st)


def sister_bench(args, bgg, torch, dev, capture):
    """The projection matrices (gate_up 17408x5120, down 5120x17408) in the
    sister formats Q1_0 (sign bits, scale per 128) and Q2_0_G64 (2-bit codes,
    scale per 64), at M = 1 and M = 16: microseconds per bgg_ternary_gemv
    call (prepare + matrix-core run) from HIP events around a graph of
    back-to-back calls that cycle through the weight copies, and GB/s of
    the format's packed bytes."""
    import synth
    w = synth.WORKLOADS["projection"]
    seed = w["seed"]
    reps = args.kernel_reps
    out = {}
    for fmt in ("Q1_0", "Q2_0_G64"):
        rows = []
        for mat in w["matrices"]:
            T, S = synth.workload_matrix(mat, seed, fmt)
            d = bgg.bgg_describe(fmt, mat.n, mat.k)
            host = bgg.bgg_pack_weights(d, T, S)
            del T, S
            copies = [bgg.upload(host, dev) for _ in range(args.copies)]
            x = torch.from_numpy(synth.workload_x(seed, 16, mat.k)).to(dev)
            y = torch.empty((16, mat.n), dtype=torch.float16, device=dev)
            ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d, 16), dev)
            for M in (1, 16):
                g = capture(lambda st, M=M: [
                    bgg.bgg_ternary_gemv(d, copies[r % args.copies], x, y, M, bgg.BGG_ROTATE_INPUT,
                                         ws, st) for r in range(reps)])
                g.replay()
                cur = torch.cuda.current_stream()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(cur)
                g.replay()
                b.record(cur)
                b.synchronize()
                us = a.elapsed_time(b) * 1e3 / reps
                rows.append(dict(matrix=mat.name, n=mat.n, k=mat.k, m=M,
                                 kernel=bgg.bgg_gemv_kernel_name(d, M),
                                 bytes_per_call=int(d.format_bytes), avg_us=round(us, 3),
                                 gbs=round(d.format_bytes / us / 1e3, 1)))
                del g
            del copies
        step = {}
        for M in (1, 16):
            r = [e for e in rows if e["m"] == M]
            tot_us = sum(e["avg_us"] for e in r)
            step[f"m{M}"] = dict(us=round(tot_us, 2),
                                 gbs=round(sum(e["bytes_per_call"] for e in r) / tot_us / 1e3, 1))
        out[fmt] = dict(calls=rows, gate_up_plus_down=step)
        log(f"sister {fmt}: " + ", ".join(f"{e['matrix']} M={e['m']} {e['avg_us']:.2f}us "
                                          f"{e['gbs']:.0f}GB/s" for e in rows))
    return out


def ternarize_bench(args, bgg, torch, dev):
    """The offline front end on the projection shapes: float32 weights ->
    trits and fp16 scales (bgg_rotate_ternarize), HIP events around 10
    back-to-back calls after 3 warm-up calls; GB/s of the algorithmic bytes
    (4 read + 1 written per weight, 2 written per 128-block)."""
    import synth
    w = synth.WORKLOADS["projection"]
    stream = torch.cuda.current_stream()
    rows = []
    for mat in w["matrices"]:
        W = torch.from_numpy(synth.float_weights(w["seed"], mat.matrix_id, mat.n, mat.k)).to(dev)
        T = torch.empty((mat.n, mat.k), dtype=torch.int8, device=dev)
        S = torch.empty((mat.n, mat.k // 128), dtype=torch.float16, device=dev)
        for _ in range(3):
            bgg.bgg_rotate_ternarize(W, mat.n, mat.k, T, S, stream)
        reps = 10
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            bgg.bgg_rotate_ternarize(W, mat.n, mat.k, T, S, stream)
        b.record(stream)
        b.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        nbytes = mat.n * mat.k * 5 + mat.n * (mat.k // 128) * 2
        rows.append(dict(matrix=mat.name, n=mat.n, k=mat.k, avg_us=round(us, 1), bytes=nbytes,
                         gbs=round(nbytes / us / 1e3, 1),
                         frac=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)))
        del W, T, S
    log("ternarize: " + ", ".join(f"{r['matrix']} {r['avg_us']}us {r['gbs']}GB/s" for r in rows))
    best = max(r["gbs"] for r in rows)
    return dict(kernel="k_rotate_ternarize", workload="float32 weights of the projection shapes "
                "-> trits + fp16 scales (rotate, mean-magnitude scale, nearest trit)",
                shapes=rows, roofline=dict(bound="hbm", achieved=best, peak=HBM_PEAK_GBS,
                                           unit="GB/s", frac=round(best / HBM_PEAK_GBS, 4)))


def stack_breakdown(bgg, torch, stack, capture, reps_layers):
    """Average launch time of each projection of one layer (a graph of
    back-to-back calls of that projection over the stack's layers, HIP
    events around its replay): kernel name, us, GB/s."""
    rows = []
    per = len(PROJ)
    layers = len(stack.calls) // per
    for j in range(per):
        calls = [stack.calls[i * per + j] for i in range(layers)][:reps_layers]
        name, d, _ = calls[0]

        def fn(st, calls=calls, d=d):
            for _, dd, p in calls:
                bgg.bgg_ternary_gemv(dd, p, stack.xs[int(d.K)][:1], stack.ys[int(d.N)][:1], 1,
                                     bgg.BGG_ROTATE_INPUT, stack.ws, st)
        g = capture(fn)
        us = replay_us(torch, g, 5) / len(calls)
        del g
        nb = int(d.format_bytes)
        rows.append(dict(matrix=name, n=int(d.N), k=int(d.K), kernel=bgg.bgg_gemv_kernel_name(d, 1),
                         bytes_per_launch=nb, launches_per_step=layers, avg_us=round(us, 3),
                         gbs=round(nb / us / 1e3, 1), frac=round(nb / us / 1e3 / HBM_PEAK_GBS, 4)))
    return rows


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=64, help="layers of the decode stack")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the timed steps and their kernel breakdown (for profiler runs)")
    ap.add_argument("--copies", type=int, default=24,
                    help="distinct device copies of the single-projection weights")
    ap.add_argument("--stack-replays", type=int, default=20,
                    help="timed graph replays per decode-step variant (median reported)")
    ap.add_argument("--gemm-warmup", type=int, default=40,
                    help="untimed rotate + GEMM pairs before the timed prefill launches")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the shared-transform, grouped and small-batch lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ternarize", action="store_true", help="skip the offline front end lines")
    ap.add_argument("--no-sister", action="store_true", help="skip the Q1_0 / Q2_0_G64 lines")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="oracle time on all host threads (then as long again on one)")
    ap.add_argument("--kernel-reps", type=int, default=100,
                    help="back-to-back launches per per-kernel timing")
    ap.add_argument("--calib", type=int, default=0, metavar="MIB",
                    help="also run the probe's streaming read and write of this many MiB "
                         "(counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the path has no multi-GPU part", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import bit_gemv_gemm_amd as bgg
    import synth
    from bit_gemv_gemm_amd import probe

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    capture = make_capture(torch)

    # ------------------------------------------------------------ the stack
    w = synth.WORKLOADS["decode_step"]
    seed = w["seed"]
    ms = [1] + list(synth.WORKLOADS["small_batch"]["m"])
    mmax = max(ms)
    widths = sorted({m.k for m in w["matrices"]})
    xs = {k: torch.from_numpy(synth.workload_x(seed, mmax, k)).to(dev) for k in widths}
    ys = {n: torch.empty((mmax, n), dtype=torch.float16, device=dev)
          for n in sorted({m.n for m in w["matrices"]})}
    stacks = {fmt: Stack(bgg, torch, dev, fmt, seed, args.layers, xs, ys, mmax) for fmt in FMTS}
    step_bytes = sum(s.bytes for s in stacks.values())
    n_calls = sum(len(s.calls) for s in stacks.values())

    # ---------------------------------------------------- the timed region
    g_step = capture(lambda st: [s.step(bgg, st) for s in stacks.values()])
    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        g_step.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    del g_step
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9
    log(f"headline: {n_calls} calls, {step_bytes / 1e9:.3f} GB per step, {ms_per_step:.3f} ms, "
        f"{value:.0f} GB/s")

    # ------------------------------------ per packing: step and breakdown
    per_fmt = {}
    kernels = []
    for fmt, s in stacks.items():
        g = capture(lambda st, s=s: s.step(bgg, st))
        us = replay_us(torch, g, args.stack_replays)
        del g
        rows = stack_breakdown(bgg, torch, s, capture, args.layers)
        for r in rows:
            r["format"] = fmt
        kernels += rows
        per_fmt[fmt] = dict(packed_bytes=s.bytes, launches=len(s.calls), us_per_step=round(us, 1),
                            gbs=round(s.bytes / us / 1e3, 1),
                            frac=round(s.bytes / us / 1e3 / HBM_PEAK_GBS, 4),
                            steps_per_s=round(1e6 / us, 1),
                            sum_of_launch_us=round(sum(r["avg_us"] * r["launches_per_step"] for r in rows), 1),
                            kernels=rows)
        log(f"{fmt} step {us:.0f} us, {s.bytes / us / 1e3:.0f} GB/s; " +
            ", ".join(f"{r['matrix']} {r['avg_us']:.2f}us {r['gbs']:.0f}GB/s" for r in rows))

    # the dominant kernel: the GEMV kernel (by name) with the largest share
    # of the step; its roofline counts the packed bytes of all its launches
    by_name = {}
    for k in kernels:
        e = by_name.setdefault(k["kernel"], dict(us=0.0, bytes=0, launches=0, calls=[]))
        e["us"] += k["avg_us"] * k["launches_per_step"]
        e["bytes"] += k["bytes_per_launch"] * k["launches_per_step"]
        e["launches"] += k["launches_per_step"]
        e["calls"].append(f"{k['format']} {k['matrix']} {k['n']}x{k['k']} x{k['launches_per_step']}")
    dom_name, dom = max(by_name.items(), key=lambda kv: kv[1]["us"])
    achieved = dom["bytes"] / dom["us"] / 1e3
    traffic = measured_traffic(dom_name)
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=traffic,
                    kernel=dom_name, share_of_step=round(dom["us"] / sum(e["us"] for e in by_name.values()), 3),
                    launches_per_step=dom["launches"], calls=dom["calls"],
                    bytes_per_launch=round(dom["bytes"] / dom["launches"]),
                    avg_us=round(dom["us"] / dom["launches"], 3))
    log(f"dominant kernel {dom_name}: {roofline['avg_us']} us per launch, {achieved:.0f} GB/s")

    # ------------------------------------------------ achievable HBM (probe)
    sink = probe.sink(dev)
    achievable = None
    if args.calib:
        # counter calibration runs: only probe launches of the known size
        cb = torch.empty(args.calib << 20, dtype=torch.uint8, device=dev)
        for _ in range(3):
            probe.read(cb, sink)
            probe.write(cb)
        torch.cuda.synchronize()
        log(f"calibration: probe read and write of {args.calib} MiB x 3")
        del cb
    else:
        big = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
        big.fill_(1)
        for _ in range(3):
            probe.read(big, sink)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(10):
            probe.read(big, sink)
        b.record(stream)
        b.synchronize()
        hbm = (2 << 30) * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
        achievable = dict(gbs=round(hbm, 1), frac=round(hbm / HBM_PEAK_GBS, 4), bytes=2 << 30,
                          kernel="k_probe_read (16-byte non-temporal loads, 4096 x 256 threads)")
        log(f"achievable HBM read: {hbm:.0f} GB/s")
        del big

    # ------------------------------------------- fixed cost of one launch
    def fn_empty(st):
        for _ in range(64):
            probe.empty(160, 512, sink, st)
    g = capture(fn_empty)
    floor_us = replay_us(torch, g, 7) / 64
    del g
    launch_floor = dict(us=round(floor_us, 3), kernel="k_probe_empty (160 x 512 threads, no work)",
                        launches_per_step=n_calls, step_ms=round(floor_us * n_calls / 1e3, 3),
                        share_of_step=round(floor_us * n_calls / 1e3 / ms_per_step, 4))
    log(f"launch floor: {floor_us:.2f} us per launch, {floor_us * n_calls / 1e3:.2f} ms of the step")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int15xternary->f32", "data": "synthetic",
        "config": {"workload": f"decode step: {args.layers}-layer 27B-class stack at batch 1 (q 5120->6144, "
                               "k/v 5120->1024, o 6144->5120, gate/up 5120->17408, down 17408->5120), "
                               "PQ2_0 then PTQ1_0, Hadamard transform before every projection "
                               f"({n_calls} calls, one after the other)",
                   "global_batch": 1, "layers": args.layers, "launches_per_step": n_calls,
                   "packed_bytes_per_step": step_bytes},
        "roofline": roofline,
        "achievable_hbm": achievable,
        "launch_floor": launch_floor,
        "cpu_baseline": None,
        "decode_step": per_fmt,
        "context": dict(pages_end_to_end=PAGES_CONTEXT,
                        note="whole-model figures on other hardware (attention, KV cache and "
                             "sampling included); here: the stack's projections alone"),
        "source_hash": source_hash(),
    }
    if args.headline_only:
        print(json.dumps(out), flush=True)
        return 0

    # ------------------- variants of the step: shared transform, grouped, M
    if not args.no_variants:
        for fmt, s in stacks.items():
            res = per_fmt[fmt]
            # one prepare for q, k and v, one for o, one for gate and up, one
            # for down, each followed by a run per matrix (the transform shared
            # the way a model can share it)
            groups = []
            for i in range(0, len(s.calls), 7):
                layer = s.calls[i:i + 7]
                groups += [layer[0:3], layer[3:4], layer[4:6], layer[6:7]]

            def step_shared(st, M=1, s=s, groups=groups):
                for grp in groups:
                    _, d0, _ = grp[0]
                    bgg.bgg_gemv_prepare(d0, s.xs[int(d0.K)][:M], M, bgg.BGG_ROTATE_INPUT, s.ws, st)
                    for _, d, p in grp:
                        bgg.bgg_gemv_run(d, p, s.ys[int(d.N)][:M], M, s.ws, st)
            g = capture(step_shared)
            us = replay_us(torch, g, args.stack_replays)
            del g
            res["shared_transform"] = dict(launches=len(groups) + len(s.calls), us_per_step=round(us, 1),
                                           gbs=round(s.bytes / us / 1e3, 1))
            small = {}
            for M in ms[1:]:
                g = capture(lambda st, M=M, s=s: s.step(bgg, st, M))
                us = replay_us(torch, g, args.stack_replays)
                del g
                small[str(M)] = dict(us_per_step=round(us, 1), gbs=round(s.bytes / us / 1e3, 1),
                                     frac=round(s.bytes / us / 1e3 / HBM_PEAK_GBS, 4),
                                     tflops=round(2.0 * M * s.weights / us / 1e6, 2),
                                     kernel=bgg.bgg_gemv_kernel_name(s.calls[0][1], M))
            res["small_batch"] = small
            log(f"{fmt} shared transform {res['shared_transform']['gbs']} GB/s; small batch " +
                ", ".join(f"M={M} {v['gbs']}GB/s" for M, v in small.items()))
        for fmt in FMTS:
            gs = Stack(bgg, torch, dev, fmt, seed, args.layers, xs, ys, mmax, grouped=True)
            gres = dict(packed_bytes=gs.bytes, launches=len(gs.calls), per_m={})
            for M in ms:
                g = capture(lambda st, M=M: gs.step(bgg, st, M))
                us = replay_us(torch, g, args.stack_replays)
                del g
                gres["per_m"][str(M)] = dict(us_per_step=round(us, 1), gbs=round(gs.bytes / us / 1e3, 1),
                                             frac=round(gs.bytes / us / 1e3 / HBM_PEAK_GBS, 4))
            per_fmt[fmt]["grouped"] = gres
            log(f"{fmt} grouped: " + ", ".join(f"M={M} {v['gbs']}GB/s" for M, v in gres["per_m"].items()))
            del gs
            torch.cuda.empty_cache()
    del stacks
    torch.cuda.empty_cache()

    # ---------------------------------------- single projection (gate_up, down)
    pw = synth.WORKLOADS["projection"]
    proj = []
    for mat in pw["matrices"]:
        T, S = synth.workload_matrix(mat, pw["seed"])
        x = torch.from_numpy(synth.workload_x(pw["seed"], 1, mat.k)).to(dev)
        y = torch.empty((1, mat.n), dtype=torch.float16, device=dev)
        for fmt in FMTS:
            d = bgg.bgg_describe(fmt, mat.n, mat.k)
            host = bgg.bgg_pack_weights(d, T, S)
            copies = [bgg.upload(host, dev) for _ in range(args.copies)]
            ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d, 1), dev)
            reps = args.kernel_reps
            g = capture(lambda st: [bgg.bgg_ternary_gemv(d, copies[r % args.copies], x, y, 1,
                                                         bgg.BGG_ROTATE_INPUT, ws, st) for r in range(reps)])
            us = replay_us(torch, g, 5) / reps
            del g, copies
            proj.append(dict(format=fmt, matrix=mat.name, n=mat.n, k=mat.k,
                             kernel=bgg.bgg_gemv_kernel_name(d, 1), bytes=int(d.format_bytes),
                             avg_us=round(us, 3), gbs=round(d.format_bytes / us / 1e3, 1),
                             frac=round(d.format_bytes / us / 1e3 / HBM_PEAK_GBS, 4)))
        del T, S
    pbytes = sum(p["bytes"] for p in proj)
    pus = sum(p["avg_us"] for p in proj)
    out["projection"] = dict(workload="gate_up 17408x5120 + down 5120x17408, batch 1, PQ2_0 and PTQ1_0, "
                                      f"{args.copies} rotating weight copies",
                             gbs=round(pbytes / pus / 1e3, 1), calls=proj)
    log("projection: " + ", ".join(f"{p['format']} {p['matrix']} {p['avg_us']}us {p['gbs']}GB/s" for p in proj))

    # --------------------------------------------------------- prefill GEMM
    if not args.no_prefill:
        pw = synth.WORKLOADS["prefill"]
        M = pw["m"][0]
        shapes, fwht, ptq1, dense = [], [], [], []
        for mat in pw["matrices"]:
            T, S = synth.workload_matrix(mat, pw["seed"])
            xs4 = [torch.from_numpy(synth.workload_x(pw["seed"] + i, M, mat.k)).to(dev) for i in range(4)]
            xr4 = [torch.empty_like(x) for x in xs4]
            y = torch.empty((M, mat.n), dtype=torch.float16, device=dev)
            # the transform alone over four rotating input/output pairs
            for i in range(4):
                bgg.bgg_hadamard_rotate(xs4[i], xr4[i], M, mat.k, stream)
            reps = 16
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for r in range(reps):
                bgg.bgg_hadamard_rotate(xs4[r % 4], xr4[r % 4], M, mat.k, stream)
            b.record(stream)
            b.synchronize()
            f_us = a.elapsed_time(b) * 1e3 / reps
            fbytes = 2 * M * mat.k * 2
            fwht.append(dict(m=M, k=mat.k, pairs=4, avg_us=round(f_us, 1), bytes=fbytes,
                             gbs=round(fbytes / f_us / 1e3, 1)))
            for fmt in FMTS:
                d = bgg.bgg_describe(fmt, mat.n, mat.k)
                packed = bgg.upload(bgg.bgg_pack_weights(d, T, S), dev)
                wsg = bgg.workspace(bgg.bgg_gemm_workspace_size(d, M), dev)
                # warm-up long enough (tens of ms of matrix work) for the clocks
                for i in range(args.gemm_warmup):
                    bgg.bgg_ternary_gemm(d, packed, xr4[i % 4], y, M, 0, wsg, stream)
                torch.cuda.synchronize()
                reps = 10
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for r in range(reps):
                    bgg.bgg_ternary_gemm(d, packed, xr4[r % 4], y, M, 0, wsg, stream)
                b.record(stream)
                b.synchronize()
                g_us = a.elapsed_time(b) * 1e3 / reps
                flops = 2.0 * M * mat.n * mat.k
                row = dict(matrix=mat.name, m=M, n=mat.n, k=mat.k, avg_us=round(g_us, 1),
                           tflops=round(flops / g_us / 1e6, 1))
                (shapes if fmt == "PQ2_0" else ptq1).append(row)
                del packed, wsg
            # comparison: dense fp16 GEMM on the dequantised weights (W^T
            # stored K x N, so the product is a plain row-major matmul)
            wt = torch.from_numpy((T.astype(np.float32) * np.repeat(S.astype(np.float32), 128, axis=1))
                                  .T.astype(np.float16).copy()).to(dev)
            for i in range(args.gemm_warmup // 4):
                torch.matmul(xr4[i % 4], wt, out=y)
            torch.cuda.synchronize()
            reps = 10
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for r in range(reps):
                torch.matmul(xr4[r % 4], wt, out=y)
            b.record(stream)
            b.synchronize()
            d_us = a.elapsed_time(b) * 1e3 / reps
            dense.append(dict(matrix=mat.name, m=M, n=mat.n, k=mat.k, avg_us=round(d_us, 1),
                              tflops=round(2.0 * M * mat.n * mat.k / d_us / 1e6, 1),
                              weight_bytes=int(wt.numel() * 2)))
            del T, S, xs4, xr4, y, wt
            torch.cuda.empty_cache()
        tot_flops = sum(2.0 * s_["m"] * s_["n"] * s_["k"] for s_ in shapes)
        tf = tot_flops / sum(s_["avg_us"] for s_ in shapes) / 1e6
        tf3 = tot_flops / sum(s_["avg_us"] for s_ in ptq1) / 1e6
        tfd = tot_flops / sum(s_["avg_us"] for s_ in dense) / 1e6
        fbest = max(f["gbs"] for f in fwht)
        out["prefill_gemm"] = dict(
            workload="prefill: 4096 tokens x (5120->17408, 17408->5120), x' precomputed",
            tflops=round(tf, 1), unit="TFLOP/s", shapes=shapes,
            roofline=dict(bound="mfma", achieved=round(tf, 1), peak=F16_MFMA_PEAK_TFLOPS,
                          unit="TFLOP/s", frac=round(tf / F16_MFMA_PEAK_TFLOPS, 4), traffic=None,
                          kernel="k_gemm_pq2 (fp16 MFMA, fp32 accumulate)"),
            ptq1_0=dict(kernel="k_ptq1_to_pq2 (weights rewritten to PQ2_0 once per call) + k_gemm_pq2",
                        tflops=round(tf3, 1),
                        frac=round(tf3 / F16_MFMA_PEAK_TFLOPS, 4), shapes=ptq1),
            dense_fp16_comparison=dict(kernel="torch.matmul (hipBLASLt) on dequantised fp16 W, run only",
                                       tflops=round(tfd, 1), frac=round(tfd / F16_MFMA_PEAK_TFLOPS, 4),
                                       shapes=dense),
            fwht=dict(kernel="k_hadamard_rotate", shapes=fwht,
                      roofline=dict(bound="hbm", achieved=fbest, peak=HBM_PEAK_GBS, unit="GB/s",
                                    frac=round(fbest / HBM_PEAK_GBS, 4))))
        log(f"prefill PQ2_0 {tf:.0f} TF, PTQ1_0 {tf3:.0f} TF, dense fp16 {tfd:.0f} TF; fwht " +
            ", ".join(f"K={f['k']} {f['gbs']}GB/s" for f in fwht))

    if not args.no_sister:
        out["sister_formats"] = sister_bench(args, bgg, torch, dev, capture)
    if not args.no_ternarize:
        out["ternarize"] = ternarize_bench(args, bgg, torch, dev)

    # ----------------------------------------------------------- CPU oracle
    if not args.no_cpu_baseline:
        import oracle
        base = {m.name.split(".")[1]: m for m in synth.decode_stack(1)}
        sample = []
        for p in PROJ:
            T, S = synth.workload_matrix(base[p], seed)
            xh = synth.workload_x(seed, 1, base[p].k)
            for fmt in FMTS:
                sample.append((p, fmt, oracle.pack(fmt, T), S, xh, oracle.format_bytes(fmt, base[p].n, base[p].k)))
            del T

        def timed(items, seconds):
            done, t, reps = 0, 0.0, 0
            while t < seconds:
                for _, fmt, P, S, xh, nb in items:
                    t1 = time.perf_counter()
                    oracle.linear(fmt, P, S, xh)
                    t += time.perf_counter() - t1
                    done += nb
                reps += 1
            return done / t / 1e9, t, reps

        nthreads = oracle.num_threads()
        v_all, t_all, r_all = timed(sample, args.cpu_seconds)
        oracle.set_num_threads(1)
        one = [it for it in sample if it[0] in ("k", "v")]
        v_one, t_one, r_one = timed(one, args.cpu_seconds)
        oracle.set_num_threads(nthreads)
        out["cpu_baseline"] = dict(
            value=round(v_all, 4), unit="GB/s", cores=nthreads, kind="oracle",
            sample=f"one layer of the step (q, k, v, o, gate, up, down; PQ2_0 and PTQ1_0; M=1; unpack + "
                   f"dense rotation + fp64 dot) run {r_all} times in {t_all:.1f} s",
            cpu_model=cpu_model(),
            one_thread=dict(value=round(v_one, 4), unit="GB/s", cores=1,
                            sample=f"k and v of one layer, both packings, run {r_one} times in {t_one:.1f} s"))
        log(f"cpu oracle {v_all:.4f} GB/s on {nthreads} threads, {v_one:.4f} GB/s on one ({cpu_model()})")

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
