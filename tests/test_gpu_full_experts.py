"""Whole experts at full size: the prefill (W8A8) and skewed (Zipf, W4A16)
workloads run through the stage entry points (the same kernels and launch
configuration as the whole feed-forward at these sizes: the big-tile MFMA
kernels),
and every row of three experts -- the hottest, one of median load and the
least loaded -- is compared with the oracle, which computes only those rows
(its row mask).  h must be at rounding level (one BF16 ulp, or 2^-10 of the
row RMS); h and y (y computed from the GPU's own h) within the 1e-2
element-wise bar."""
import numpy as np
import pytest
import torch

import oracle
import quantized_routed_expert_top_amd as qre
from harness.inputs import WORKLOADS
from harness.synthetic import gpu_problem
from gpu_helpers import assert_parity, assert_rounding_level, bf16_np, bf16_to_f64, oracle_experts

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pick_experts(counts):
    touched = np.nonzero(counts)[0]
    order = touched[np.argsort(counts[touched], kind="stable")]
    return [int(order[-1]), int(order[len(order) // 2]), int(order[0])]


@pytest.mark.parametrize("name", ["prefill_w8a8", "zipf_w4a16"])
def test_full_size_whole_experts(name):
    wl = WORKLOADS[name]
    print(f"[whole experts] {name}", flush=True)
    P = gpu_problem(wl, DEV)
    ids, x_bits = P["ids"], P["x_bits"]
    counts, offsets, sorted_slot, slot_row, _ = oracle.route(ids, wl.E)
    picked = _pick_experts(counts)
    print(f"  experts {picked} with {[int(counts[e]) for e in picked]} rows", flush=True)
    mask = np.zeros(wl.S, np.uint8)
    for e in picked:
        mask[offsets[e]:offsets[e + 1]] = 1
    rows = np.nonzero(mask)[0]
    shp = dict(T=wl.T, H=wl.H, I=wl.I, E=wl.E, K=wl.K, bits=wl.weight_bits)
    Wo = oracle_experts(wl, picked)

    # GPU, full size
    gc, go, gss, gsr, _ = qre.route(P["topk_ids"], wl.E)
    np.testing.assert_array_equal(go.cpu().numpy(), offsets)
    if wl.act_int8:
        xq, xs = qre.quantize_act(P["x"])
        h_gpu, hq, hs = qre.gate_up(None, gss, go, P["W"], wl.K, act_int8=True, xq=xq, xs=xs, want_hq=True)
        y_gpu = qre.down(None, go, P["W"], wl.T, wl.K, act_int8=True, hq=hq, hs=hs)
    else:
        h_gpu = qre.gate_up(P["x"], gss, go, P["W"], wl.K)
        y_gpu = qre.down(h_gpu, go, P["W"], wl.T, wl.K)
    torch.cuda.synchronize()
    h_g = bf16_np(h_gpu)[rows]
    y_g = bf16_np(y_gpu)[rows]

    # oracle, the picked experts' rows only
    if wl.act_int8:
        oxq, oxs = oracle.quantize_act(x_bits)
        h_ref = oracle.gate_up(None, sorted_slot, offsets, Wo, act_int8=True, xq=oxq, xs=oxs, row_mask=mask, **shp)
        ohq, ohs = oracle.quantize_act(h_ref)
        y_ref = oracle.down(None, offsets, Wo, act_int8=True, hq=ohq, hs=ohs, row_mask=mask, **shp)
    else:
        h_ref = oracle.gate_up(x_bits, sorted_slot, offsets, Wo, row_mask=mask, **shp)
        y_ref = oracle.down(h_ref, offsets, Wo, row_mask=mask, **shp)
    assert_rounding_level(h_g, h_ref[rows], what=f"h {name} experts {picked}")
    assert_parity(h_g, bf16_to_f64(h_ref[rows]), what=f"h {name} experts {picked}")
    assert_parity(y_g, bf16_to_f64(y_ref[rows]), what=f"y {name} experts {picked}")
