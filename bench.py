#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE feed-forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_w4a16]

A step is one whole qre_moe_forward (permutation, gate/up+SiLU GEMM, down GEMM,
combine; plus the INT8 quantizers in INT8-activation mode) over one synthetic
batch already resident in HBM.  Steps are replayed from HIP graphs (one per
weight copy) and rotate over enough copies of the packed weights that the
256 MB last-level cache cannot serve them.  Prints one JSON line.

The roofline object is for the dominant kernel (the fused gate/up GEMM): its
algorithmic bytes per launch (packed weights + scales of the touched experts)
over its average duration, measured here with HIP events recorded on the
kernel's stream around each launch.
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_sources(wl) -> list:
    """Source files of the gate/up kernel a workload runs: the 128-row tile
    kernels at 64 or more slots per expert, else the per-expert kernels."""
    big = wl.T * wl.K >= 64 * wl.E
    return [os.path.join(CSRC, f) for f in (("gemm_big.hip" if big else "gemm.hip"), "gemm_common.h")]


def source_digest(wl) -> str:
    h = hashlib.sha256()
    for path in gemm_sources(wl):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(wl):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter
    summary, or None if absent or taken on a different kernel source."""
    workload = wl.name
    path = TRAFFIC_FILE.format(workload)
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
        self.lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.lib.hipEventDestroy.argtypes = [C.c_void_p]
        self.events = []

    def create(self):
        h = self.C.c_void_p()
        if self.lib.hipEventCreate(self.C.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.events.append(h.value)
        return h.value

    def elapsed_ms(self, a, b):
        ms = self.C.c_float()
        if self.lib.hipEventElapsedTime(self.C.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy_all(self):
        for h in self.events:
            self.lib.hipEventDestroy(h)
        self.events = []


def cpu_baseline(wl, x_bits, ids, w, budget_s=12.0):
    """The oracle as it stands, on this host's cores, over whole blocks of the
    same workload (repeated until ~budget_s of CPU time, at least once)."""
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
    runs, t_total = 0, 0.0
    while runs == 0 or t_total < budget_s:
        t0 = time.perf_counter()
        oracle.moe_forward(x_bits, ids, w, Wo, E=wl.E, bits=wl.weight_bits, act_int8=wl.act_int8, tokens=tokens)
        t_total += time.perf_counter() - t0
        runs += 1
        if t_total > 3 * budget_s:
            break
    return {"value": runs * len(tok) / t_total, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"{sample}, {runs} run(s), {t_total:.1f} s"}


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
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode_w4a16")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: enough for >= 1 GiB)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    import numpy as np
    import torch
    import quantized_routed_expert_top_amd as qre
    from harness.inputs import WORKLOADS
    from harness.synthetic import algorithmic_bytes, gpu_problem

    wl = WORKLOADS[args.workload]
    if args.stage == "router":
        return router_bench(args, wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {wl.name}: generating and quantizing weights on the GPU")
    t0 = time.perf_counter()
    P = gpu_problem(wl, dev)
    log(f"[bench] problem ready in {time.perf_counter() - t0:.1f} s")
    alg = algorithmic_bytes(wl, P["ids"])
    W0 = P["W"]
    R = args.copies or max(1, math.ceil((1 << 30) / max(alg["gate_up_weights"] + alg["down_weights"], 1)))
    copies = [W0] + [W0.clone() for _ in range(R - 1)]
    x, ids_t, w_t = P["x"], P["topk_ids"], P["topk_w"]
    ws = torch.empty(qre.workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.K, wl.weight_bits, wl.act_int8),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)

    def step(i):
        qre.moe_forward(x, ids_t, w_t, copies[i % R], act_int8=wl.act_int8, out=out, workspace=ws)

    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        eager_out = out.clone()
        if not args.eager:
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step(r)
                graphs.append(g)
            for i in range(min(args.warmup, 2 * R)):
                graphs[i % R].replay()
            torch.cuda.synchronize()
            if not torch.equal(out, eager_out):
                raise RuntimeError("graph replay differs from eager output")

        # ---- timed region: K whole steps ----
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(args.steps):
            if args.eager:
                step(i)
            else:
                graphs[i % R].replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms = ev0.elapsed_time(ev1)
        if not torch.equal(out, eager_out):
            raise RuntimeError("timed steps changed the output")

        # ---- per-kernel durations: the same kernels, with HIP events between steps ----
        hip = HipEvents()
        nk = max(20, min(args.steps, 200))
        evs = [[hip.create() for _ in range(6)] for _ in range(nk)]
        for i in range(nk):
            qre.moe_forward_timed(x, ids_t, w_t, copies[i % R], evs[i], act_int8=wl.act_int8, out=out,
                                  workspace=ws)
        torch.cuda.synchronize()
        if not torch.equal(out, eager_out):
            raise RuntimeError("timed forward differs from qre_moe_forward")
    dur = np.array([[hip.elapsed_ms(e[j], e[j + 1]) for j in range(5)] for e in evs[2:]]).mean(axis=0) * 1e3  # us
    hip.destroy_all()

    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = wl.T * args.steps / wall
    gu_us, dn_us = float(dur[1]), float(dur[3])
    gu_bytes = alg["gate_up_weights"]
    S = wl.T * wl.K
    if S >= 64 * wl.E:
        # prefill-sized: 64+ rows per expert on average (the 128-row MFMA
        # tiles); the gate/up GEMM is a dense contraction for the matrix cores
        gu_flops = 2.0 * S * wl.H * 2 * wl.I
        peak = I8_PEAK_TOPS if wl.act_int8 else BF16_PEAK_TFLOPS
        achieved = gu_flops / (gu_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": read_traffic(wl),
                    "kernel": "fused gate/up + SiLU*mul GEMM", "avg_us": round(gu_us, 2),
                    "alg_flops_per_launch": gu_flops}
    else:
        achieved = gu_bytes / (gu_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(wl),
                    "kernel": "fused gate/up + SiLU*mul GEMM", "avg_us": round(gu_us, 2),
                    "alg_bytes_per_launch": int(gu_bytes)}
    step_bytes = alg["total"]
    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
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
                   "weight_bits": wl.weight_bits, "act_int8": wl.act_int8, "weight_copies": R,
                   "launch": "eager" if args.eager else "hipGraph replay", "touched_experts": alg["touched"]},
        "roofline": roofline,
        "step": {"gpu_ms_per_step": round(gpu_ms / args.steps, 5),
                 "alg_bytes": int(step_bytes),
                 "hbm_frac_whole_step": round(step_bytes / (wall / args.steps) / 1e9 / HBM_PEAK_GBS, 4),
                 "mfma_frac_whole_step": round(alg["flops"] / (wall / args.steps) / 1e12 /
                                               (I8_PEAK_TOPS if wl.act_int8 else BF16_PEAK_TFLOPS), 5)},
        "kernels_us": {"route_and_quantize_x": round(float(dur[0]), 2), "gate_up": round(gu_us, 2),
                       "quantize_h": round(float(dur[2]), 2), "down": round(dn_us, 2),
                       "combine": round(float(dur[4]), 2)},
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
        result["cpu_baseline"] = cpu_baseline(wl, P["x_bits"], P["ids"], P["w"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
