"""Shared helpers of the GPU parity tests: oracle-side weights for a workload,
tensor <-> numpy conversion and the output tolerance metric."""
import numpy as np
import torch

import oracle
from quantized_routed_expert_top_amd.inputs import Workload

# Output tolerance.  The stated bar is a maximum relative error of 1e-2,
# normalised by the output RMS.  It is read per output row (one token, or one
# sorted expert row for the intermediate h and y): the RMS of the row's error
# over the RMS of the oracle row must be <= 1e-2 for every row.  The reference
# is the oracle's FP32 output before its final rounding.
#
# An element-wise bar of 1e-2 cannot hold for BF16 outputs: half a BF16 ulp at
# |v| in [4, 8) x rms is already 1.6e-2 x rms, and two correct implementations
# that sum in different orders may round an expert output y to neighbouring
# BF16 values (2^-7 relative) before the final rounding (2^-8).  As a guard
# against isolated wrong elements, every element must also satisfy
# |gpu - ref| <= 2e-2 x max(|ref|, rms(ref)): the 1e-2 bar plus one BF16 ulp
# (2^-7) of slack, rounded up.
TOL = 1e-2
ELEM_TOL = 2e-2


def bf16_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def parity_stats(gpu_bits: np.ndarray, ref: np.ndarray) -> dict:
    g = bf16_to_f64(gpu_bits)
    r = np.asarray(ref, np.float64)
    if r.size == 0:
        return {"row_rel": 0.0, "elem_rel": 0.0, "strict": 0.0, "rel_l2": 0.0}
    r2 = r.reshape(-1, r.shape[-1])
    g2 = g.reshape(r2.shape)
    d = np.abs(g2 - r2)
    rms = float(np.sqrt(np.mean(r2 * r2)))
    floor = rms * 1e-3 if rms > 0 else 1e-30
    rms_row = np.maximum(np.sqrt(np.mean(r2 * r2, axis=1)), floor)
    err_row = np.sqrt(np.mean(d * d, axis=1))
    return {
        "row_rel": float((err_row / rms_row).max()),
        "elem_rel": float((d / np.maximum(np.abs(r2), max(rms, 1e-30))).max()),
        "strict": float(d.max() / rms) if rms > 0 else float(d.max()),
        "rel_l2": float(np.sqrt(np.sum(d * d)) / max(np.sqrt(np.sum(r2 * r2)), 1e-300)),
    }


def assert_parity(gpu_bits, ref, tol=TOL, elem_tol=ELEM_TOL, what=""):
    assert np.all(np.isfinite(bf16_to_f64(gpu_bits))), f"{what}: non-finite output"
    st = parity_stats(gpu_bits, ref)
    assert st["row_rel"] <= tol and st["elem_rel"] <= elem_tol, f"{what}: {st}"
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
