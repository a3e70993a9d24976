"""The benchmark's output contract on the GPU: one JSON line with the metric,
throughput, roofline and CPU-baseline objects, for a short run of the default
workload and of the router stage."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    print(f"[bench contract] bench.py {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def _check_common(j, steps, warmup):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in j, k
    assert j["n_gpus"] == 1 and j["steps"] == steps and j["warmup"] == warmup
    assert j["value"] > 0 and j["ms_per_step"] > 0 and j["higher_is_better"] is True
    assert j["data"] == "synthetic" and "workload" in j["config"]
    rf = j["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] in ("hbm", "mfma", "alu") and 0 < rf["frac"] < 1
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3


def test_default_workload_line():
    j = _bench("--steps", "20", "--warmup", "3", "--no-cpu-baseline")
    _check_common(j, 20, 3)
    assert j["config"]["workload"] == "decode_w4a16" and j["dtype"] == "bf16"
    assert j["roofline"]["bound"] == "hbm" and j["roofline"]["unit"] == "GB/s"
    # steps replay a graph of R consecutive forwards; the one-forward-per-graph
    # loop is reported beside it
    assert j["step"]["one_graph_per_forward_ms"] > 0
    assert str(j["config"]["weight_copies"]) in j["config"]["launch"]
    # tokens/s and ms/step describe the same timed region
    assert abs(j["value"] * j["ms_per_step"] / 1e3 - j["config"]["T"]) / j["config"]["T"] < 1e-3
    # the prefill half of the metric and the measured read ceiling ride on the same line
    pf = j["prefill"]
    assert pf["workload"] == "prefill_w8a8" and pf["tokens_per_s"] > 0 and 0 < pf["gate_up_mfma_frac"] < 1
    assert 0 < pf["step_i8_mfma_frac"] < 1 and pf["steps"] == 20
    pr = j["hbm_read_probe"]
    assert 0 < pr["frac_of_peak"] < 1 and 0 < j["roofline"]["frac_of_measured_read"] < 1.2
    # the NVFP4 (W4A4) decode block
    f4 = j["nvfp4"]
    assert f4["workload"] == "decode_nvfp4" and f4["tokens_per_s"] > 0 and f4["steps"] == 20
    assert f4["roofline"]["bound"] == "hbm" and 0 < f4["roofline"]["frac"] < 1
    assert set(f4["kernels_us"]) == {"route_and_quantize_x", "gate_up", "quantize_h", "down", "combine"}


def test_router_stage_line_with_cpu_baseline():
    j = _bench("--stage", "router", "--workload", "decode_w4a16", "--steps", "50", "--warmup", "3")
    _check_common(j, 50, 3)
    cb = j["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]


class _Events:
    """hipEvent_t handles through ctypes, for the timed forward calls."""

    def __init__(self):
        import ctypes as C
        self.C = C
        self.lib = C.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.lib.hipEventDestroy.argtypes = [C.c_void_p]
        self.made = []

    def create(self):
        h = self.C.c_void_p()
        assert self.lib.hipEventCreate(self.C.byref(h)) == 0
        self.made.append(h.value)
        return h.value

    def ms(self, a, b):
        v = self.C.c_float()
        assert self.lib.hipEventElapsedTime(self.C.byref(v), a, b) == 0
        return v.value

    def close(self):
        for h in self.made:
            self.lib.hipEventDestroy(h)


@pytest.mark.parametrize("name,T,H,I,E,K,bits,a8,fmt", [
    ("decode_routed", 32, 2048, 512, 256, 8, 4, False, "int"),   # permutation folded into gate/up
    ("w8a8_big", 512, 512, 256, 16, 4, 8, True, "int"),           # routing launches, 128-row INT8 tiles
    ("decode_nvfp4", 32, 512, 256, 64, 8, 4, False, "nvfp4"),
])
def test_timed_forward_kernel_events(name, T, H, I, E, K, bits, a8, fmt):
    """The timed forward calls give the untimed call's output bit for bit; the
    two events handed to the gate/up launch itself bracket a positive
    interval that lies inside the interval of the events recorded around that
    step (the dispatch begins after the step's first event and ends before
    its second)."""
    import torch
    import quantized_routed_expert_top_amd as qre
    from harness.inputs import Workload
    from harness.synthetic import gpu_problem

    print(f"[timed forward] {name}", flush=True)
    wl = Workload(name, T=T, H=H, I=I, E=E, K=K, weight_bits=bits, act_int8=a8, fmt=fmt, seed=7)
    P = gpu_problem(wl, torch.device("cuda:0"))
    fp4 = fmt == "nvfp4"
    if fp4:
        ref = qre.nvfp4_moe_forward(P["x"], P["topk_ids"], P["topk_w"], P["W"])
    else:
        ref = qre.moe_forward(P["x"], P["topk_ids"], P["topk_w"], P["W"], act_int8=a8)
    hip = _Events()
    try:
        for _ in range(3):
            ev = [hip.create() for _ in range(8)]
            if fp4:
                out = qre.nvfp4_moe_forward_timed(P["x"], P["topk_ids"], P["topk_w"], P["W"], ev)
            else:
                out = qre.moe_forward_timed(P["x"], P["topk_ids"], P["topk_w"], P["W"], ev, act_int8=a8)
            torch.cuda.synchronize()
            assert torch.equal(out, ref)
            kernel = hip.ms(ev[6], ev[7])
            step = hip.ms(ev[1], ev[2])
            print(f"[timed forward] {name}: gate/up kernel {kernel * 1e3:.2f} us, step {step * 1e3:.2f} us", flush=True)
            assert kernel > 0
            # 0.5 us of slack for the rounding of the two timestamp sources
            assert hip.ms(ev[1], ev[6]) >= -5e-4 and hip.ms(ev[7], ev[2]) >= -5e-4
        # the binding insists on all eight handles (the library reads eight)
        timed = qre.nvfp4_moe_forward_timed if fp4 else qre.moe_forward_timed
        with pytest.raises(ValueError):
            timed(P["x"], P["topk_ids"], P["topk_w"], P["W"], [None] * 6)
    finally:
        hip.close()
