#!/usr/bin/env python3
"""Benchmark of the ternary linear-layer hot path on one MI355X.

Workload (one step): the single-projection decode workload at batch 1 --
gate/up (K=5120 -> N=17408) and down (K=17408 -> N=5120), each in both
packings (PQ2_0, PTQ1_0), each call applying the block-128 Hadamard
transform to its fp16 input and then the GEMV.  Inputs are seeded and
synthetic (trit, scale and activation distributions of the 27B-class stack)
and resident in HBM before timing starts; the weights rotate over several
distinct device copies (> 512 MiB together) so the 256 MiB Infinity Cache
cannot serve them.

value = packed weight bytes of the step (format bytes: trits + fp16 scales)
        / wall time of one step.

The steps are launched from a captured HIP graph (replayed K/copies
times), so the timed region measures the GPU, not the Python interpreter
that would otherwise issue every launch.

Also printed in the same JSON line: the roofline of the dominant GEMV kernel
(the kernel, by name, with the largest share of a step; its launch duration
from HIP events around the replay of a graph of back-to-back launches of
each call, right after the timed region), per-kernel figures, the prefill
GEMM (4096 tokens) in TFLOP/s with its MFMA roofline and the activation
transform in GB/s, and the CPU oracle timed on this host on a sample of the
step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
METRIC = "ternary GEMV packed-weight GB/s (% HBM peak) + prefill GEMM TFLOPS (% MFMA)"


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


def decode_stack_bench(args, bgg, torch, dev, capture):
    """The full decode step of a 64-layer stack (q, k, v, o, gate, up, down
    per layer) at M = 1 and the small-batch sweep M = 2, 4, 8, 16, both
    packings.  Each projection is one bgg_ternary_gemv call that transforms
    and encodes its own x (448 calls per step).  At M = 1 a second line
    shares each transform the way a model can: one bgg_gemv_prepare for q, k
    and v, one for o, one for gate and up, one for down, each followed by
    bgg_gemv_run per matrix.  Every matrix has its own device buffer; the 64
    layers reuse layer 0's generated values (the work and the bytes streamed
    do not depend on them).  A third set of lines packs q, k, v and gate, up
    as one matrix each (four calls per layer), for every M.  GB/s = packed
    bytes of the step / median wall time of one graph replay."""
    import numpy as np
    import synth
    w = synth.WORKLOADS["decode_step"]
    seed, mats = w["seed"], w["matrices"]
    ms = [1] + list(synth.WORKLOADS["small_batch"]["m"])
    mmax = max(ms)
    stream = torch.cuda.current_stream()
    xs = {k: torch.from_numpy(synth.workload_x(seed, mmax, k)).to(dev)
          for k in sorted({m.k for m in mats})}
    ys = {n: torch.empty((mmax, n), dtype=torch.float16, device=dev) for n in sorted({m.n for m in mats})}
    weights = sum(m.n * m.k for m in mats)
    res = dict(workload=f"decode step: {len(mats) // 7} layers x (q 5120->6144, k/v 5120->1024, "
                        f"o 6144->5120, gate/up 5120->17408, down 17408->5120), "
                        f"Hadamard transform before every projection",
               layers=len(mats) // 7, matrices=len(mats), weights=weights, formats={})

    def median_replay_us(g, reps):
        cur = torch.cuda.current_stream()
        for _ in range(3):
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

    for fmt in ("PQ2_0", "PTQ1_0"):
        t0 = time.time()
        host = {}
        for m in mats[:7]:
            T, S = synth.workload_matrix(m, seed)
            d = bgg.bgg_describe(fmt, m.n, m.k)
            host[m.name.split(".")[1]] = (d, bgg.bgg_pack_weights(d, T, S))
            del T, S
        calls = []
        for m in mats:
            d, hp = host[m.name.split(".")[1]]
            calls.append((m, d, bgg.upload(hp, dev)))
        del host
        step_bytes = sum(int(d.format_bytes) for _, d, _ in calls)
        wsb = max(bgg.bgg_gemv_workspace_size(d, mmax) for _, d, _ in calls)
        ws = bgg.workspace(wsb, dev)
        log(f"decode step {fmt}: {step_bytes / 1e9:.2f} GB packed in {len(calls)} buffers "
            f"({time.time() - t0:.1f}s)")
        per_m = {}
        for M in ms:
            def step(st, M=M):
                for m, d, p in calls:
                    bgg.bgg_ternary_gemv(d, p, xs[m.k][:M], ys[m.n][:M], M, bgg.BGG_ROTATE_INPUT,
                                         ws, st)
            g = capture(step)
            us = median_replay_us(g, args.stack_replays)
            del g
            per_m[str(M)] = dict(us_per_step=round(us, 1), gbs=round(step_bytes / us / 1e3, 1),
                                 frac=round(step_bytes / us / 1e3 / HBM_PEAK_GBS, 4),
                                 tflops=round(2.0 * M * weights / us / 1e6, 2))
            log(f"  M={M}: {us:.0f} us per step, {step_bytes / us / 1e3:.0f} GB/s")

        # the transform shared as a model would share it: one prepare for
        # q, k and v, one for o, one for gate and up, one for down, each
        # followed by a run per matrix
        groups = []  # (input width, [calls])
        for i in range(0, len(calls), 7):
            layer = calls[i:i + 7]
            groups += [layer[0:3], layer[3:4], layer[4:6], layer[6:7]]
        shared = dict(launches=len(groups) + len(calls), per_m={})
        for M in ms:
            def step_shared(st, M=M):
                for grp in groups:
                    m0, d0, _ = grp[0]
                    bgg.bgg_gemv_prepare(d0, xs[m0.k][:M], M, bgg.BGG_ROTATE_INPUT, ws, st)
                    for m, d, p in grp:
                        bgg.bgg_gemv_run(d, p, ys[m.n][:M], M, ws, st)
            g = capture(step_shared)
            us = median_replay_us(g, args.stack_replays)
            del g
            shared["per_m"][str(M)] = dict(us_per_step=round(us, 1),
                                           gbs=round(step_bytes / us / 1e3, 1),
                                           frac=round(step_bytes / us / 1e3 / HBM_PEAK_GBS, 4))
            log(f"  M={M} shared transform: {us:.0f} us per step, {step_bytes / us / 1e3:.0f} GB/s")
        del calls
        torch.cuda.empty_cache()

        # Grouped projections: the rows of q, k and v packed as one matrix
        # (N = 8192), those of gate and up as another (N = 34816), so a layer
        # is four calls; each call transforms its input once.  The same
        # weights and packed bytes up to the padding of the groups' rows.
        t0 = time.time()
        byname = {m.name.split(".")[1]: m for m in mats[:7]}
        gdefs = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")),
                 ("down", ("down",))]
        ghost = {}
        for gname, parts in gdefs:
            Ts, Ss = zip(*(synth.workload_matrix(byname[q], seed) for q in parts))
            T, S = np.concatenate(Ts), np.concatenate(Ss)
            d = bgg.bgg_describe(fmt, T.shape[0], T.shape[1])
            ghost[gname] = (d, bgg.bgg_pack_weights(d, T, S))
            del Ts, Ss, T, S
        gcalls = [(ghost[gname][0], bgg.upload(ghost[gname][1], dev))
                  for _ in range(len(mats) // 7) for gname, _ in gdefs]
        del ghost
        gbytes = sum(int(d.format_bytes) for d, _ in gcalls)
        gys = {int(d.N): torch.empty((mmax, int(d.N)), dtype=torch.float16, device=dev)
               for d, _ in gcalls}
        wsb = max(bgg.bgg_gemv_workspace_size(d, mmax) for d, _ in gcalls)
        ws = bgg.workspace(wsb, dev)
        log(f"  grouped: {gbytes / 1e9:.2f} GB packed in {len(gcalls)} buffers ({time.time() - t0:.1f}s)")
        grouped = {}
        for M in ms:
            def step_grouped(st, M=M):
                for d, p in gcalls:
                    bgg.bgg_ternary_gemv(d, p, xs[int(d.K)][:M], gys[int(d.N)][:M], M,
                                         bgg.BGG_ROTATE_INPUT, ws, st)
            g = capture(step_grouped)
            us = median_replay_us(g, args.stack_replays)
            del g
            grouped[str(M)] = dict(us_per_step=round(us, 1), gbs=round(gbytes / us / 1e3, 1),
                                   frac=round(gbytes / us / 1e3 / HBM_PEAK_GBS, 4))
            log(f"  grouped M={M}: {us:.0f} us per step, {gbytes / us / 1e3:.0f} GB/s")
        res["formats"][fmt] = dict(packed_bytes=step_bytes, per_m=per_m, shared_transform=shared,
                                   grouped=dict(packed_bytes=gbytes, launches=len(gcalls),
                                                per_m=grouped))
        del gcalls, gys, ws
        torch.cuda.empty_cache()
    return res


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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=8, help="distinct device copies of the weights")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-decode-step", action="store_true",
                    help="skip the 64-layer decode step and the small-batch sweep")
    ap.add_argument("--stack-replays", type=int, default=20,
                    help="timed graph replays per decode-step configuration (median reported)")
    ap.add_argument("--gemm-warmup", type=int, default=40,
                    help="untimed rotate + GEMM pairs before the timed prefill launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ternarize", action="store_true",
                    help="skip the offline front end lines")
    ap.add_argument("--no-sister", action="store_true",
                    help="skip the Q1_0 / Q2_0_G64 lines")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--kernel-reps", type=int, default=100,
                    help="back-to-back launches per per-kernel timing")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="also run a device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the path has no multi-GPU part", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import bit_gemv_gemm_amd as bgg
    import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = synth.WORKLOADS["projection"]
    seed = w["seed"]
    fmts = ("PQ2_0", "PTQ1_0")

    # ------------------------------------------------------------------ data
    t0 = time.time()
    items = []  # one per (format, matrix)
    for mat in w["matrices"]:
        T, S = synth.workload_matrix(mat, seed)
        x = torch.from_numpy(synth.workload_x(seed, 1, mat.k)).to(dev)
        for fmt in fmts:
            d = bgg.bgg_describe(fmt, mat.n, mat.k)
            host = bgg.bgg_pack_weights(d, T, S)
            copies = [bgg.upload(host, dev) for _ in range(args.copies)]
            ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d, 1), dev)
            y = torch.empty((1, mat.n), dtype=torch.float16, device=dev)
            items.append(dict(fmt=fmt, name=mat.name, desc=d, copies=copies, ws=ws, x=x, y=y,
                              bytes=int(d.format_bytes), n=mat.n, k=mat.k))
        del T, S
    resident = sum(it["desc"].total_bytes * args.copies for it in items)
    log(f"setup {time.time() - t0:.1f}s; {resident / 2**20:.0f} MiB of packed weights resident")

    # Launches go through HIP graphs (captured once, replayed): a ctypes call
    # from Python costs several microseconds, as long as the kernels it
    # launches, so eager launching would time the interpreter.
    # One call per (format, matrix): at one token bgg_ternary_gemv is a
    # single kernel that transforms and encodes x and computes y.
    def step(c, st):
        for it in items:
            bgg.bgg_ternary_gemv(it["desc"], it["copies"][c], it["x"], it["y"], 1,
                                 bgg.BGG_ROTATE_INPUT, it["ws"], st)

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

    # one replay = one step per weight copy
    g_steps = capture(lambda st: [step(c, st) for c in range(args.copies)])
    rounds = max(1, args.steps // args.copies)
    steps = rounds * args.copies
    for _ in range(max(1, args.warmup // args.copies)):
        g_steps.replay()
    torch.cuda.synchronize()

    # ------------------------------------------------------ the timed region
    t_start = time.perf_counter()
    for _ in range(rounds):
        g_steps.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall / steps * 1e3
    step_bytes = sum(it["bytes"] for it in items)
    value = step_bytes / (wall / steps) / 1e9

    # ---------------------------------------------- per-kernel launch times
    # HIP events on the replay stream around a graph of `reps` back-to-back
    # launches of one call (an event pair around every single launch would
    # add the event overhead, microseconds, to each).  At M = 1
    # bgg_ternary_gemv, bgg_gemv_prepare and bgg_gemv_run are one kernel
    # launch each; the last two are the two-step form, timed for comparison.
    reps = args.kernel_reps

    def timed(fn):
        g = capture(lambda st: [fn(r, st) for r in range(reps)])
        g.replay()
        cur = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(cur)
        g.replay()
        b.record(cur)
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / reps  # us per launch

    kernels = []
    for it in items:
        d = it["desc"]
        one_us = timed(lambda r, st: bgg.bgg_ternary_gemv(d, it["copies"][r % args.copies], it["x"],
                                                          it["y"], 1, bgg.BGG_ROTATE_INPUT,
                                                          it["ws"], st))
        bgg.bgg_gemv_prepare(d, it["x"], 1, bgg.BGG_ROTATE_INPUT, it["ws"], stream)
        run_us = timed(lambda r, st: bgg.bgg_gemv_run(d, it["copies"][r % args.copies], it["y"], 1,
                                                      it["ws"], st))
        prep_us = timed(lambda r, st: bgg.bgg_gemv_prepare(d, it["x"], 1, bgg.BGG_ROTATE_INPUT,
                                                           it["ws"], st))
        kernels.append(dict(kernel=bgg.bgg_gemv_kernel_name(d, 1), format=it["fmt"],
                            matrix=it["name"], n=it["n"], k=it["k"],
                            bytes_per_launch=it["bytes"], avg_us=round(one_us, 3),
                            gbs=round(it["bytes"] / one_us / 1e3, 1),
                            frac=round(it["bytes"] / one_us / 1e3 / HBM_PEAK_GBS, 4),
                            two_step=dict(prep_kernel="k_gemv_prep", prep_avg_us=round(prep_us, 3),
                                          run_avg_us=round(run_us, 3))))
    # the dominant kernel: the GEMV kernel (by name) with the largest share
    # of a step; its roofline counts the packed bytes of all its launches
    by_name = {}
    for k in kernels:
        e = by_name.setdefault(k["kernel"], dict(us=0.0, bytes=0, calls=[]))
        e["us"] += k["avg_us"]
        e["bytes"] += k["bytes_per_launch"]
        e["calls"].append(f"{k['format']} {k['matrix']} {k['n']}x{k['k']}")
    dom_name, dom = max(by_name.items(), key=lambda kv: kv[1]["us"])
    n_launch = len(dom["calls"])
    achieved = dom["bytes"] / dom["us"] / 1e3
    traffic = measured_traffic(dom_name)
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel=dom_name, launches=dom["calls"],
                    bytes_per_launch=round(dom["bytes"] / n_launch),
                    avg_us=round(dom["us"] / n_launch, 3))
    log(f"step {ms_per_step * 1e3:.1f} us, {value:.0f} GB/s; kernels: " +
        ", ".join(f"{k['format']}/{k['matrix']} {k['kernel']} {k['avg_us']:.2f}us "
                  f"{k['gbs']:.0f}GB/s (two-step: prep {k['two_step']['prep_avg_us']:.2f}us + run "
                  f"{k['two_step']['run_avg_us']:.2f}us)" for k in kernels))
    for it in items:
        del it["copies"]

    # calibration for the HBM byte counters: a plain device-to-device copy
    # of known size (run only when asked, for the counter profiles)
    if args.calib_copy:
        src = torch.empty(args.calib_copy << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calib_copy} MiB x 3")
        del src, dst

    # --------------------------------------------------------- prefill GEMM
    prefill = None
    if not args.no_prefill:
        pw = synth.WORKLOADS["prefill"]
        M = pw["m"][0]
        shapes, fwht, ptq1 = [], [], []
        for fmt in ("PQ2_0", "PTQ1_0"):
            for mat in pw["matrices"]:
                T, S = synth.workload_matrix(mat, pw["seed"])
                d = bgg.bgg_describe(fmt, mat.n, mat.k)
                packed = bgg.upload(bgg.bgg_pack_weights(d, T, S), dev)
                x = torch.from_numpy(synth.workload_x(pw["seed"], M, mat.k)).to(dev)
                xr = torch.empty_like(x)
                y = torch.empty((M, mat.n), dtype=torch.float16, device=dev)
                # (the workspace holds the partial sums where the GEMM splits K)
                wsg = bgg.workspace(bgg.bgg_gemm_workspace_size(d, M), dev)
                # warm-up long enough (tens of ms of matrix work) for the clocks
                # to settle: the first launches after the GEMV part run up to
                # 25 % slower than the steady state
                reps = 10
                for _ in range(args.gemm_warmup):
                    bgg.bgg_hadamard_rotate(x, xr, M, mat.k, stream)
                    bgg.bgg_ternary_gemm(d, packed, xr, y, M, 0, wsg, stream)
                torch.cuda.synchronize()
                e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                      torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
                for r in range(reps):
                    e[r][0].record(stream)
                    bgg.bgg_hadamard_rotate(x, xr, M, mat.k, stream)
                    e[r][1].record(stream)
                    bgg.bgg_ternary_gemm(d, packed, xr, y, M, 0, wsg, stream)
                    e[r][2].record(stream)
                torch.cuda.synchronize()
                f_us = float(np.mean([a.elapsed_time(b) for a, b, _ in e])) * 1e3
                g_us = float(np.mean([b.elapsed_time(c) for _, b, c in e])) * 1e3
                flops = 2.0 * M * mat.n * mat.k
                row = dict(matrix=mat.name, m=M, n=mat.n, k=mat.k, avg_us=round(g_us, 1),
                           tflops=round(flops / g_us / 1e6, 1))
                if fmt == "PQ2_0":
                    shapes.append(row)
                    fbytes = 2 * M * mat.k * 2
                    fwht.append(dict(m=M, k=mat.k, avg_us=round(f_us, 1),
                                     gbs=round(fbytes / f_us / 1e3, 1)))
                else:
                    ptq1.append(row)
                del T, S, packed, x, xr, y, wsg
        tot_flops = sum(2.0 * s["m"] * s["n"] * s["k"] for s in shapes)
        tot_us = sum(s["avg_us"] for s in shapes)
        tf = tot_flops / tot_us / 1e6
        tf3 = tot_flops / sum(s["avg_us"] for s in ptq1) / 1e6
        prefill = dict(
            workload="prefill: 4096 tokens x (5120->17408, 17408->5120), PQ2_0, x' precomputed",
            tflops=round(tf, 1), unit="TFLOP/s", shapes=shapes,
            roofline=dict(bound="mfma", achieved=round(tf, 1), peak=F16_MFMA_PEAK_TFLOPS,
                          unit="TFLOP/s", frac=round(tf / F16_MFMA_PEAK_TFLOPS, 4), traffic=None,
                          kernel="k_gemm_pq2 (fp16 MFMA, fp32 accumulate)"),
            ptq1_0=dict(kernel="k_gemm_ptq1 (base-3 bytes -> 2-bit codes -> fp16 MFMA)",
                        tflops=round(tf3, 1), frac=round(tf3 / F16_MFMA_PEAK_TFLOPS, 4),
                        shapes=ptq1),
            fwht=dict(kernel="k_hadamard_rotate", shapes=fwht,
                      roofline=dict(bound="hbm", achieved=max(f["gbs"] for f in fwht),
                                    peak=HBM_PEAK_GBS, unit="GB/s",
                                    frac=round(max(f["gbs"] for f in fwht) / HBM_PEAK_GBS, 4))))
        log(f"prefill PQ2_0 {tf:.0f} TFLOP/s; " + ", ".join(f"{s['matrix']} {s['tflops']} TF" for s in shapes)
            + f"; PTQ1_0 {tf3:.0f} TFLOP/s; " + ", ".join(f"{s['matrix']} {s['tflops']} TF" for s in ptq1))

    # ------------------------------------- 64-layer decode step, M = 1 .. 16
    stack = None
    if not args.no_decode_step:
        stack = decode_stack_bench(args, bgg, torch, dev, capture)

    # ------------------------------------------ sister formats, M = 1 and 16
    sister = None
    if not args.no_sister:
        sister = sister_bench(args, bgg, torch, dev, capture)

    # ------------------------------------------- offline front end (float W)
    tern = None
    if not args.no_ternarize:
        tern = ternarize_bench(args, bgg, torch, dev)

    # ----------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        sample = []
        for mat in w["matrices"]:
            T, S = synth.workload_matrix(mat, seed)
            xh = synth.workload_x(seed, 1, mat.k)
            for fmt in fmts:
                sample.append((fmt, oracle.pack(fmt, T), S, xh, oracle.format_bytes(fmt, mat.n, mat.k)))
            del T
        done_bytes, t_cpu, reps = 0, 0.0, 0
        while t_cpu < args.cpu_seconds:
            for fmt, P, S, xh, nb in sample:
                t1 = time.perf_counter()
                oracle.linear(fmt, P, S, xh)
                t_cpu += time.perf_counter() - t1
                done_bytes += nb
            reps += 1
        cpu = dict(value=round(done_bytes / t_cpu / 1e9, 4), unit="GB/s", cores=oracle.num_threads(),
                   kind="oracle",
                   sample=f"the whole step (gate_up + down, PQ2_0 + PTQ1_0, M=1, unpack + dense "
                          f"rotation + fp64 dot) run {reps} times, {t_cpu:.1f} s")
        log(f"cpu oracle {cpu['value']} GB/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i32+f32", "data": "synthetic",
        "config": {"workload": "projection: gate_up 17408x5120 + down 5120x17408, batch 1, "
                               "PQ2_0 and PTQ1_0, Hadamard transform on every call",
                   "global_batch": 1, "copies": args.copies,
                   "packed_bytes_per_step": step_bytes},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "prefill_gemm": prefill,
        "decode_step": stack,
        "sister_formats": sister,
        "ternarize": tern,
        "source_hash": source_hash(),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
