#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE feed-forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_w4a16]

A step is one whole qre_moe_forward (permutation, gate/up+SiLU GEMM, down GEMM,
combine; plus the INT8 quantizers in INT8-activation mode) over one synthetic
batch already resident in HBM.  Steps rotate over R copies of the packed
weights, enough that the 256 MB last-level cache cannot serve them, and are
replayed from one HIP graph holding R consecutive forwards (as a decode graph
holds the feed-forward of many layers); `step.one_graph_per_forward_ms` gives
the same loop with one graph launch per forward.  Prints one JSON line.

The headline is the 32-token W4A16 block (decode_w4a16): `value` is its
tokens/s over exactly K timed steps.  By default the same process then times
the 8192-token W8A8 prefill (`prefill` object: its own timed steps, the
gate/up MFMA fraction and the whole step's INT8 MFMA fraction), the same
32-token block with NVFP4 (W4A4) experts (`nvfp4` object: timed steps, the
gate/up kernel's HBM fraction) and a plain streaming read of device memory
(`hbm_read_probe`: the measured read ceiling next to the published 8 TB/s).

The roofline object is for the dominant kernel (the fused gate/up GEMM): its
algorithmic bytes per launch (packed weights + scales of the touched experts)
over its average duration, measured here with two HIP events that the library
hands to that kernel's own launch (hipExtLaunchKernelGGL on the kernel's
stream): they take the dispatch's begin and end, the interval a kernel trace
reports.  The per-step breakdown (`kernels_us`) comes from events recorded
between the steps, less the duration of an empty event pair.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA, published
I8_PEAK_TOPS = 5000.0
METRIC = "routed-expert FFN tokens/s; % HBM peak (32-tok block) & % MFMA peak (prefill)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gate_up_{}.txt")
CSRC = os.path.join(ROOT, "quantized_routed_expert_top_amd", "csrc")
LAUNCH = ("hipGraph of {R} consecutive forwards over the {R} weight copies, replayed "
          "(one-forward graphs for a remainder)")
STAGES = ("route_and_quantize_x", "gate_up", "quantize_h", "down", "combine")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def is_big(wl) -> bool:
    return wl.T * wl.K >= 64 * wl.E


def gemm_sources(wl) -> list:
    """Source files of the dominant kernel a workload runs: the NVFP4 kernels,
    the 128-row tile kernels at 64 or more slots per expert, else the
    per-expert kernels."""
    main = "nvfp4.hip" if wl.fmt == "nvfp4" else "gemm_big.hip" if is_big(wl) else "gemm.hip"
    return [os.path.join(CSRC, f) for f in (main, "gemm_common.h")]


def source_digest(wl) -> str:
    h = hashlib.sha256()
    for path in gemm_sources(wl):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(wl):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter
    summary, or None if absent or taken on a different kernel source."""
    path = TRAFFIC_FILE.format(wl.name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha256") != source_digest(wl):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class HipEvents:
    """hipEvent_t handles through ctypes (recorded by the library on its stream)."""

    def __init__(self):
        import ctypes as C
        self.C = C
        self.lib = C.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.lib.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.lib.hipEventDestroy.argtypes = [C.c_void_p]
        self.events = []

    def create(self):
        h = self.C.c_void_p()
        if self.lib.hipEventCreate(self.C.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.events.append(h.value)
        return h.value

    def record(self, ev, stream_handle):
        if self.lib.hipEventRecord(ev, stream_handle) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.C.c_float()
        if self.lib.hipEventElapsedTime(self.C.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy_all(self):
        for h in self.events:
            self.lib.hipEventDestroy(h)
        self.events = []


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, x_bits, ids, w, budget_s=10.0, budget_1t_s=5.0):
    """The oracle as it stands, on this host's cores, over whole blocks of the
    same workload (repeated until ~budget_s of wall time, at least once),
    with all the threads OpenMP gives it and again with one thread."""
    import numpy as np
    import oracle
    from harness.synthetic import touched_experts
    if wl.T > 512:
        tokens = np.arange(min(wl.T, 64))
        sample = f"first {len(tokens)} tokens of the {wl.T}-token batch"
    else:
        tokens = None
        sample = f"whole {wl.T}-token batch"
    tok = np.arange(wl.T) if tokens is None else tokens
    Wo = oracle.workload_experts(wl, touched_experts(ids[tok], wl.E))

    def timed(budget):
        runs, t_total = 0, 0.0
        while runs == 0 or t_total < budget:
            t0 = time.perf_counter()
            oracle.moe_forward(x_bits, ids, w, Wo, E=wl.E, bits=wl.weight_bits, act_int8=wl.act_int8, tokens=tokens)
            t_total += time.perf_counter() - t0
            runs += 1
        return runs, t_total

    threads = oracle.num_threads()
    runs, t_total = timed(budget_s)
    oracle.set_num_threads(1)
    runs1, t1 = timed(budget_1t_s)
    oracle.set_num_threads(threads)
    return {"value": round(runs * len(tok) / t_total, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "sample": f"{sample}, {runs} run(s), {t_total:.1f} s",
            "one_thread": {"value": round(runs1 * len(tok) / t1, 2), "unit": "tokens/s", "cores": 1,
                           "sample": f"{sample}, {runs1} run(s), {t1:.1f} s"},
            "cpu_model": cpu_model(), "build": "gcc -O2 -ffp-contract=off -fopenmp, no intrinsics, no BLAS"}


def empty_pair_us(hip, stream_handle, n=50):
    """Mean duration of two events recorded back to back (the cost an event
    pair adds to a kernel's measured duration)."""
    import numpy as np
    pairs = [(hip.create(), hip.create()) for _ in range(n)]
    for a, b in pairs:
        hip.record(a, stream_handle)
        hip.record(b, stream_handle)
    import torch
    torch.cuda.synchronize()
    return float(np.mean([hip.elapsed_ms(a, b) for a, b in pairs[5:]])) * 1e3


def time_workload(wl, steps, warmup, eager, copies_arg, dev, hip):
    """Problem setup, K timed steps (graph replay), a median of 5 further
    loops, and per-kernel durations from the library's events.  Returns a
    dict of measurements plus the problem (for the CPU baseline)."""
    import numpy as np
    import torch
    import quantized_routed_expert_top_amd as qre
    from harness.synthetic import algorithmic_bytes, gpu_problem

    log(f"[bench] workload {wl.name}: generating and quantizing weights on the GPU")
    t0 = time.perf_counter()
    P = gpu_problem(wl, dev)
    log(f"[bench] problem ready in {time.perf_counter() - t0:.1f} s")
    alg = algorithmic_bytes(wl, P["ids"])
    W0 = P["W"]
    R = copies_arg or max(1, math.ceil((1 << 30) / max(alg["gate_up_weights"] + alg["down_weights"], 1)))
    copies = [W0] + [W0.clone() for _ in range(R - 1)]
    x, ids_t, w_t = P["x"], P["topk_ids"], P["topk_w"]
    fp4 = wl.fmt == "nvfp4"
    nb = (qre.nvfp4_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.K) if fp4 else
          qre.workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.K, wl.weight_bits, wl.act_int8))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)

    def step(i):
        if fp4:
            qre.nvfp4_moe_forward(x, ids_t, w_t, copies[i % R], out=out, workspace=ws)
        else:
            qre.moe_forward(x, ids_t, w_t, copies[i % R], act_int8=wl.act_int8, out=out, workspace=ws)

    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        eager_out = out.clone()
        chain = None
        if not eager:
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step(r)
                graphs.append(g)
            # R consecutive forwards over the R weight sets in one graph, as a
            # decode graph holds the feed-forward of many layers
            chain = torch.cuda.CUDAGraph()
            with torch.cuda.graph(chain, stream=stream):
                for r in range(R):
                    step(r)
            for i in range(2 * R):
                graphs[i % R].replay()
            torch.cuda.synchronize()
            if not torch.equal(out, eager_out):
                raise RuntimeError("graph replay differs from eager output")
            chain.replay()
            torch.cuda.synchronize()
            if not torch.equal(out, eager_out):
                raise RuntimeError("chained graph replay differs from eager output")

        def run_steps(n, single=False):
            """n whole forwards, in order over the weight sets: eager launches,
            else the chained graph for each full round of R forwards and the
            one-forward graphs for the rest (or one-forward graphs only)."""
            i = 0
            if eager:
                for i in range(n):
                    step(i)
                return
            if not single:
                while i + R <= n:
                    chain.replay()
                    i += R
            while i < n:
                graphs[i % R].replay()
                i += 1

        # the warmup steps again, replayed as they are timed (clocks and caches
        # settle on the replayed sequence, not on the eager one)
        if not eager:
            run_steps(max(warmup, 2 * R))
        # ---- timed region: K whole steps ----
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        run_steps(steps)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms = ev0.elapsed_time(ev1)
        if not torch.equal(out, eager_out):
            raise RuntimeError("timed steps changed the output")

        # ---- five further event-timed loops (median) ----
        nl = max(10, min(steps, 200))
        loop_ms = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run_steps(nl)
            b.record(stream)
            torch.cuda.synchronize()
            loop_ms.append(a.elapsed_time(b) / nl)
        # the same loops with one graph launch per forward (the graph-to-graph
        # gap paid on every step)
        single_ms = []
        if not eager:
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                run_steps(nl, single=True)
                b.record(stream)
                torch.cuda.synchronize()
                single_ms.append(a.elapsed_time(b) / nl)

        # ---- per-kernel durations: the same kernels, with HIP events between steps ----
        sh = stream.cuda_stream
        pair_us = empty_pair_us(hip, sh)
        nk = max(20, min(steps, 200))
        # two passes: the six step marks alone (the per-step breakdown), then
        # only the two events the gate/up launch takes itself
        evs = [[hip.create() for _ in range(6)] + [None, None] for _ in range(nk)]
        kev = [[None] * 6 + [hip.create(), hip.create()] for _ in range(nk)]
        for timed in (evs, kev):
            for i in range(nk):
                if fp4:
                    qre.nvfp4_moe_forward_timed(x, ids_t, w_t, copies[i % R], timed[i], out=out, workspace=ws)
                else:
                    qre.moe_forward_timed(x, ids_t, w_t, copies[i % R], timed[i], act_int8=wl.act_int8, out=out,
                                          workspace=ws)
            torch.cuda.synchronize()
            if not torch.equal(out, eager_out):
                raise RuntimeError("timed forward differs from qre_moe_forward")
    dur = np.array([[hip.elapsed_ms(e[j], e[j + 1]) for j in range(5)] for e in evs[2:]]).mean(axis=0) * 1e3
    dur = np.maximum(dur - pair_us, 0.0)
    gu_kernel_us = float(np.mean([hip.elapsed_ms(e[6], e[7]) for e in kev[2:]])) * 1e3
    plan = 0 if fp4 else qre.forward_plan(wl.T, wl.H, wl.I, wl.E, wl.K, wl.weight_bits, wl.act_int8)
    return {
        "wl": wl, "P": P, "alg": alg, "R": R, "steps": steps, "wall": wall, "gpu_ms": gpu_ms, "plan": plan,
        "median_loop_ms": float(np.median(loop_ms)), "loops_ms": [round(v, 5) for v in loop_ms],
        "one_graph_per_forward_ms": round(float(np.median(single_ms)), 5) if single_ms else None,
        "kernels_us": {k: round(float(v), 2) for k, v in zip(STAGES, dur)}, "event_pair_us": round(pair_us, 2),
        "gate_up_kernel_us": round(gu_kernel_us, 2), "timed_launches": nk - 2,
    }


def hbm_probe(dev, hip, nbytes=2 << 30, reps=10):
    """Plain streaming read of `nbytes` of device memory (8x the last-level
    cache), event-timed; returns GB/s."""
    import numpy as np
    import torch
    import quantized_routed_expert_top_amd as qre
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4096, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(3):
            qre.hbm_read_probe(buf, sink)
        sh = stream.cuda_stream
        evs = [(hip.create(), hip.create()) for _ in range(reps)]
        for a, b in evs:
            hip.record(a, sh)
            qre.hbm_read_probe(buf, sink)
            hip.record(b, sh)
        torch.cuda.synchronize()
    us = float(np.mean([hip.elapsed_ms(a, b) for a, b in evs])) * 1e3
    del buf
    return {"bytes": nbytes, "avg_us": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def roofline(res, probe_gbs=None):
    wl, alg = res["wl"], res["alg"]
    gu_us = res["gate_up_kernel_us"]
    timing = (f"HIP events taken by the gate/up launch itself (dispatch begin and end), mean of "
              f"{res['timed_launches']} launches")
    if is_big(wl):
        # prefill-sized: 64+ rows per expert on average (the 128-row MFMA
        # tiles); the gate/up GEMM is a dense contraction for the matrix cores
        S = wl.T * wl.K
        gu_flops = 2.0 * S * wl.H * 2 * wl.I
        peak = I8_PEAK_TOPS if wl.act_int8 else BF16_PEAK_TFLOPS
        achieved = gu_flops / (gu_us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": read_traffic(wl),
                "kernel": "fused gate/up + SiLU*mul GEMM", "avg_us": gu_us, "alg_flops_per_launch": gu_flops,
                "timing": timing}
    gu_bytes = alg["gate_up_weights"]
    kernel = ("fused permutation + gate/up + SiLU*mul GEMM" if res["plan"] & 1 else "fused gate/up + SiLU*mul GEMM")
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(wl),
         "kernel": kernel, "avg_us": gu_us, "alg_bytes_per_launch": int(gu_bytes),
         "timing": timing}
    if probe_gbs:
        r["frac_of_measured_read"] = round(achieved / probe_gbs, 4)
    return r


def step_summary(res):
    wl, alg = res["wl"], res["alg"]
    s = res["wall"] / res["steps"]
    peak = I8_PEAK_TOPS if wl.act_int8 else BF16_PEAK_TFLOPS
    return {"gpu_ms_per_step": round(res["gpu_ms"] / res["steps"], 5),
            "median_of_5_loops_ms": round(res["median_loop_ms"], 5),
            "one_graph_per_forward_ms": res["one_graph_per_forward_ms"],
            "alg_bytes": int(alg["total"]),
            "hbm_frac_whole_step": round(alg["total"] / s / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac_whole_step": round(alg["flops"] / s / 1e12 / peak, 5)}


def router_bench(args, wl):
    """--stage router: the router kernel alone (top-K + softmax over the
    workload's synthetic logits), replayed from a HIP graph; one JSON line."""
    import numpy as np
    import torch
    import quantized_routed_expert_top_amd as qre
    from harness.inputs import gen_router_logits

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    logits_np = gen_router_logits(wl)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        lg = torch.from_numpy(logits_np).to(dev)
        ids, w = qre.topk_softmax(lg, wl.K)
        for _ in range(args.warmup):
            qre.topk_softmax(lg, wl.K)
        torch.cuda.synchronize()
        ids_eager, w_eager = ids.clone(), w.clone()
        g = torch.cuda.CUDAGraph()
        outs = {}
        with torch.cuda.graph(g, stream=stream):
            outs["ids"], outs["w"] = qre.topk_softmax(lg, wl.K)
        g.replay()
        torch.cuda.synchronize()
        if not (torch.equal(outs["ids"], ids_eager) and torch.equal(outs["w"], w_eager)):
            raise RuntimeError("graph replay differs from eager router output")
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # kernel duration: events around single eager launches on the same stream
        nk = max(20, min(args.steps, 200))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nk)]
        for a, b in evs:
            a.record(stream)
            qre.topk_softmax(lg, wl.K)
            b.record(stream)
        torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs[2:]])) * 1e3
    nbytes = wl.T * wl.E * 4 + wl.T * wl.K * 8
    achieved = nbytes / (us * 1e-6) / 1e9
    result = {
        "metric": "router tokens/s (top-K selection + softmax weights)",
        "value": round(wl.T * args.steps / wall, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"router_{wl.name}", "T": wl.T, "E": wl.E, "K": wl.K, "launch": "hipGraph replay"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": None, "kernel": "k_topk_softmax",
                     "avg_us": round(us, 2), "alg_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        import oracle
        log("[bench] timing the CPU oracle router")
        runs, t_total = 0, 0.0
        while runs == 0 or t_total < 5.0:
            t1 = time.perf_counter()
            oracle.topk_softmax(logits_np, wl.K)
            t_total += time.perf_counter() - t1
            runs += 1
        result["cpu_baseline"] = {"value": round(runs * wl.T / t_total, 1), "unit": "tokens/s", "cores": 1,
                                  "kind": "oracle", "sample": f"whole batch of {wl.T} tokens, {runs} run(s), "
                                                              f"{t_total:.1f} s"}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode_w4a16")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: enough for >= 1 GiB)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill_w8a8 object of the default run")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read probe")
    ap.add_argument("--no-nvfp4", action="store_true", help="skip the decode_nvfp4 object of the default run")
    ap.add_argument("--stage", choices=["ffn", "router"], default="ffn",
                    help="ffn: the whole feed-forward (default); router: the top-K + softmax router alone")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration under rocprofv3 --pmc)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): the library has no "
              f"multi-GPU path; the per-GPU kernel is what it measures.", file=sys.stderr)
        sys.exit(2)

    import torch
    from harness.inputs import WORKLOADS

    wl = WORKLOADS[args.workload]
    if args.stage == "router":
        return router_bench(args, wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = HipEvents()

    probe = None if args.no_probe else hbm_probe(dev, hip)
    res = time_workload(wl, args.steps, args.warmup, args.eager, args.copies, dev, hip)
    pre = None
    if not args.no_prefill and wl.name != "prefill_w8a8":
        pw = WORKLOADS["prefill_w8a8"]
        pre = time_workload(pw, min(args.steps, 100), min(args.warmup, 10), args.eager, 0, dev, hip)
    f4 = None
    if not args.no_nvfp4 and wl.name != "decode_nvfp4":
        f4 = time_workload(WORKLOADS["decode_nvfp4"], args.steps, args.warmup, args.eager, 0, dev, hip)
    hip.destroy_all()

    ms_per_step = res["wall"] * 1e3 / args.steps
    result = {
        "metric": METRIC,
        "value": round(wl.T * args.steps / res["wall"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if wl.act_int8 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "K": wl.K,
                   "weight_bits": wl.weight_bits, "act_int8": wl.act_int8, "weight_copies": res["R"],
                   "launch": "eager" if args.eager else LAUNCH.format(R=res["R"]),
                   "touched_experts": res["alg"]["touched"]},
        "roofline": roofline(res, probe["gbs"] if probe else None),
        "step": step_summary(res),
        "kernels_us": res["kernels_us"],
        "event_pair_us": res["event_pair_us"],
        "plan": {"route_in_gate_up": bool(res["plan"] & 1), "combine_in_down": bool(res["plan"] & 2)},
    }
    if probe:
        result["hbm_read_probe"] = probe
        result["step"]["frac_of_measured_read_whole_step"] = round(
            res["alg"]["total"] / (res["wall"] / args.steps) / 1e9 / probe["gbs"], 4)
    if pre is not None:
        pw = pre["wl"]
        pr = roofline(pre)
        ps = step_summary(pre)
        result["prefill"] = {
            "workload": pw.name, "T": pw.T, "H": pw.H, "I": pw.I, "E": pw.E, "K": pw.K,
            "weight_bits": pw.weight_bits, "act_int8": pw.act_int8, "dtype": "i8", "weight_copies": pre["R"],
            "steps": pre["steps"], "ms_per_step": round(pre["wall"] * 1e3 / pre["steps"], 5),
            "tokens_per_s": round(pw.T * pre["steps"] / pre["wall"], 1),
            "gate_up_us": pr["avg_us"], "gate_up_mfma_frac": pr["frac"], "gate_up_tops": pr["achieved"],
            "step_i8_mfma_frac": ps["mfma_frac_whole_step"], "step": ps, "kernels_us": pre["kernels_us"],
            "gate_up_traffic": pr["traffic"],
        }
    if f4 is not None:
        fw = f4["wl"]
        fr = roofline(f4, probe["gbs"] if probe else None)
        result["nvfp4"] = {
            "workload": fw.name, "T": fw.T, "H": fw.H, "I": fw.I, "E": fw.E, "K": fw.K,
            "format": "E2M1 weights and inputs, E4M3 scale per 16, FP32 outer scale per matrix / input row",
            "dtype": "f16 MFMA on exactly rebuilt FP4 operands, FP32 accumulation", "weight_copies": f4["R"],
            "steps": f4["steps"], "ms_per_step": round(f4["wall"] * 1e3 / f4["steps"], 5),
            "tokens_per_s": round(fw.T * f4["steps"] / f4["wall"], 1), "touched_experts": f4["alg"]["touched"],
            "roofline": fr, "step": step_summary(f4), "kernels_us": f4["kernels_us"],
        }
    if args.copy_probe:
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = n
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        P = res["P"]
        result["cpu_baseline"] = cpu_baseline(wl, P["x_bits"], P["ids"], P["w"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
