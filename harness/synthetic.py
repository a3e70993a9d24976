"""GPU-resident synthetic problems for the routed-expert feed-forward.

Draws the seeded inputs of ``inputs.py`` and converts the float32 expert
weights to the packed INT4/INT8 format on the GPU with the library's own
weight converter (``quantize_weights``, or ``nvfp4_quantize_weights`` for the
NVFP4 format), one expert at a time so host memory stays bounded.
"""
from __future__ import annotations

import numpy as np
import torch

from quantized_routed_expert_top_amd import Nvfp4Experts, QuantizedExperts, nvfp4_quantize_weights, quantize_weights
from harness.inputs import GATE, UP, DOWN, Workload, gen_routing, gen_x, iter_expert_weights


def x_tensor(x_bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).to(device)


def gpu_experts(wl: Workload, device="cuda", threads: int | None = None):
    if wl.fmt == "nvfp4":
        return gpu_nvfp4_experts(wl, device, threads)
    W = QuantizedExperts.empty(wl.E, wl.H, wl.I, wl.weight_bits, device=device)
    dst = {GATE: (W.gate_q, W.gate_s), UP: (W.up_q, W.up_s), DOWN: (W.down_q, W.down_s)}
    for e, mats in iter_expert_weights(wl, range(wl.E), threads=threads):
        for m, w in zip((GATE, UP, DOWN), mats):
            q, s = dst[m]
            wd = torch.from_numpy(w).to(device, non_blocking=False)
            quantize_weights(wd, wl.weight_bits, out=(q[e], s[e]))
    torch.cuda.synchronize(device)
    return W


def gpu_nvfp4_experts(wl: Workload, device="cuda", threads: int | None = None) -> Nvfp4Experts:
    W = Nvfp4Experts.empty(wl.E, wl.H, wl.I, device=device)
    dst = {GATE: (W.gate_q, W.gate_s, W.gate_o), UP: (W.up_q, W.up_s, W.up_o),
           DOWN: (W.down_q, W.down_s, W.down_o)}
    for e, mats in iter_expert_weights(wl, range(wl.E), threads=threads):
        for m, w in zip((GATE, UP, DOWN), mats):
            q, sc, o = dst[m]
            wd = torch.from_numpy(w).to(device, non_blocking=False)
            nvfp4_quantize_weights(wd[None], out=(q[e:e + 1], sc[e:e + 1], o[e:e + 1]))
    torch.cuda.synchronize(device)
    return W


def gpu_problem(wl: Workload, device="cuda", threads: int | None = None) -> dict:
    """x (bf16 [T,H]), topk_ids (int32 [T,K]), topk_w (fp32 [T,K]) and packed
    weights on `device`, plus the host copies of x and routing."""
    x_bits = gen_x(wl)
    ids, w = gen_routing(wl)
    return {
        "wl": wl,
        "x_bits": x_bits,
        "ids": ids,
        "w": w,
        "x": x_tensor(x_bits, device),
        "topk_ids": torch.from_numpy(ids).to(device),
        "topk_w": torch.from_numpy(w).to(device),
        "W": gpu_experts(wl, device, threads),
    }


def touched_experts(ids: np.ndarray, E: int) -> np.ndarray:
    ids = np.asarray(ids).reshape(-1)
    ids = ids[(ids >= 0) & (ids < E)]
    return np.unique(ids)


def algorithmic_bytes(wl: Workload, ids: np.ndarray) -> dict:
    """Bytes the feed-forward itself must move: packed weights and scales of
    the touched experts, plus x, the routing inputs and out."""
    n_touched = len(touched_experts(ids, wl.E))
    per_w = 0.5 + 1 / 16 if wl.fmt == "nvfp4" else wl.weight_bits / 8 + 2 / 128
    gate_up = 2 * wl.I * wl.H * per_w
    down = wl.H * wl.I * per_w
    io = wl.T * wl.H * 2 * 2 + wl.T * wl.K * 8
    return {
        "touched": n_touched,
        "gate_up_weights": n_touched * gate_up,
        "down_weights": n_touched * down,
        "io": io,
        "total": n_touched * (gate_up + down) + io,
        "flops": 2 * wl.T * wl.K * 3 * wl.H * wl.I,
    }
