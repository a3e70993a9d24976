"""Shared helpers of the GPU parity tests: oracle-side weights for a workload,
tensor <-> numpy conversion and the output tolerance metric."""
import numpy as np
import torch

import oracle
from harness.inputs import Workload

# Output tolerance: max_i |gpu_i - ref_i| / max(|ref_i|, rms(ref)) <= 1e-2,
# element by element, against the oracle's value (for the whole feed-forward,
# its FP32 sum before the final rounding to BF16).  The stated bar is a
# maximum relative error of 1e-2 normalised by the output RMS; normalising by
# the RMS alone cannot hold for any BF16 output (half a BF16 ulp at |v| in
# [4, 8) x rms is already 1.6e-2 x rms), so an element is measured against the
# larger of its own magnitude and the RMS.  Every check prints its measured
# statistics (element-wise, strict max|d|/rms, per-row RMS, relative L2).
TOL = 1e-2


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


def assert_parity(gpu_bits, ref, tol=TOL, what=""):
    assert np.all(np.isfinite(bf16_to_f64(gpu_bits))), f"{what}: non-finite output"
    st = parity_stats(gpu_bits, ref)
    print(f"[parity] {what}: elem_rel={st['elem_rel']:.3e} strict={st['strict']:.3e} "
          f"row_rel={st['row_rel']:.3e} rel_l2={st['rel_l2']:.3e} (bar {tol:g})", flush=True)
    assert st["elem_rel"] <= tol, f"{what}: {st}"
    return st


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of the BF16 grid at |v| (8 significant bits; 2^-133 below 2^-126)."""
    v = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(np.where(v == 0, 1.0, v))
    return np.where(v == 0, 2.0 ** -133, np.ldexp(1.0, np.maximum(e, -125) - 8))


def assert_rounding_level(gpu_bits, ref_bits, what=""):
    """An intermediate BF16 result (h or y: one rounding of a sum, FP32 on the
    GPU, exact on the oracle): every GPU element equals the oracle's, is its
    BF16 neighbour (the two sums straddled a rounding midpoint), or is off by
    less than 2^-10 of the oracle row's RMS (an element much smaller than its
    own terms, where the FP32 sum's absolute error spans several of its
    ulps).  Prints how many elements differ and the largest difference."""
    g = bf16_to_f64(gpu_bits)
    r = bf16_to_f64(ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    if r.size == 0:
        return
    r2, g2 = r.reshape(-1, r.shape[-1]), g.reshape(-1, r.shape[-1])
    d = np.abs(g2 - r2)
    row_rms = np.sqrt(np.mean(r2 * r2, axis=1, keepdims=True))
    lim = bf16_ulp(np.maximum(np.abs(g2), np.abs(r2))) + 2.0 ** -10 * row_rms
    n_diff = int(np.count_nonzero(d))
    n_flip = int(np.count_nonzero((d > 0) & (d <= bf16_ulp(np.maximum(np.abs(g2), np.abs(r2))))))
    print(f"[rounding] {what}: {n_diff} of {d.size} elements differ ({n_flip} by one BF16 ulp); "
          f"largest difference {float((d / lim).max()):.3f} of the limit", flush=True)
    bad = d > lim
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond one BF16 ulp + 2^-10 row RMS"


def assert_forward_parity(gpu_bits, ref32, y_tok_bits, w_tok, tol=TOL, what=""):
    """The whole feed-forward's output against the oracle's FP32 sum before
    its final rounding: |gpu - ref| <= tol * max(|ref|, rms(ref)) element-wise,
    plus, for each of the K expert outputs y_k the element combines, the one
    BF16 ulp of y_k by which a correct y_k may round the other way (the GPU's
    FP32 sum and the oracle's exact sum straddling a rounding midpoint; the
    stage tests check that every y is within one ulp).  Prints how many
    elements needed that allowance."""
    g = bf16_to_f64(gpu_bits)
    r = np.asarray(ref32, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    st = parity_stats(gpu_bits, r)
    if r.size == 0:
        return st
    rms = float(np.sqrt(np.mean(r * r)))
    base = tol * np.maximum(np.abs(r), max(rms, 1e-30))
    yv = bf16_to_f64(y_tok_bits)                               # [n, K, H]
    straddle = (np.abs(np.asarray(w_tok, np.float64))[:, :, None] * bf16_ulp(yv)).sum(axis=1)
    d = np.abs(g - r)
    over = d > base
    n_over = int(over.sum())
    excess = float(((d - base) / straddle)[over].max()) if n_over else 0.0
    print(f"[parity] {what}: elem_rel={st['elem_rel']:.3e} strict={st['strict']:.3e} "
          f"row_rel={st['row_rel']:.3e} rel_l2={st['rel_l2']:.3e} (bar {tol:g}); "
          f"{n_over} of {d.size} elements above the bar, using at most {excess:.2f} of their y-straddle allowance",
          flush=True)
    bad = d > base + straddle
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the bar plus the y-straddle allowance; {st}"
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
