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
