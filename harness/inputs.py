"""Seeded synthetic inputs for the routed-expert MoE feed-forward.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random numbers and shapes them into the workloads; it holds
none of the feed-forward's own arithmetic (no quantization, no routing
permutation, no expert matmul, no combine).  Everything it returns is a plain
numpy array.

Workloads follow the block-diffusion server described on the minnow README
(section "Quantization" and the opening paragraphs): a 32-token refinement
block, sixteen such blocks batched together, long prefill, plus a large skewed
MoE.  Random streams are numpy PCG64 generators seeded with
``default_rng([seed, tag, ...])`` so every stream regenerates independently:

  tag 0            x, N(0,1) float32, rounded to bf16 storage
  tag 2            router logits, N(0,1) (or Gumbel(0,1) for the Zipf workload)
  tag 3            outlier-channel choice (prefill workload)
  tag 4            Zipf rank permutation (skewed workload)
  [seed,1,e,m]     float32 weights of expert e, matrix m (0 gate, 1 up, 2 down),
                   N(0, 0.02)
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

GATE, UP, DOWN = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # routed experts
    K: int            # experts per token
    weight_bits: int  # 4 or 8
    act_int8: bool    # INT8 activations (W4A8 / W8A8)
    fmt: str = "int"  # "int": INT4/INT8 codes, FP16 scale per 128; "nvfp4": E2M1, E4M3 per 16, FP32 outer (W4A4)
    seed: int = 0
    router: str = "normal"     # "normal": logits N(0,1); "zipf": Zipf-biased
    zipf_s: float = 1.1
    outlier_frac: float = 0.0  # fraction of x channels scaled by outlier_scale
    outlier_scale: float = 20.0
    w_std: float = 0.02

    @property
    def S(self) -> int:
        return self.T * self.K

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # one 32-token refinement block, small model, INT8 weights / bf16 activations
    "tiny_w8a16": Workload("tiny_w8a16", T=32, H=256, I=128, E=8, K=2, weight_bits=8, act_int8=False),
    # one 32-token block at the mini model's MoE shape, INT4 weights: weight-streaming bound
    "decode_w4a16": Workload("decode_w4a16", T=32, H=2048, I=512, E=256, K=8, weight_bits=4, act_int8=False),
    # sixteen 32-token blocks under continuous batching
    "cb_w4a16": Workload("cb_w4a16", T=512, H=2048, I=512, E=256, K=8, weight_bits=4, act_int8=False),
    "cb_w8a16": Workload("cb_w8a16", T=512, H=2048, I=512, E=256, K=8, weight_bits=8, act_int8=False),
    # 8192-token prefill with INT8 activations and 1% outlier channels (x20)
    "prefill_w8a8": Workload("prefill_w8a8", T=8192, H=2048, I=512, E=256, K=8, weight_bits=8,
                             act_int8=True, outlier_frac=0.01),
    # large MoE with Zipf(1.1) expert popularity
    "zipf_w4a16": Workload("zipf_w4a16", T=4096, H=4096, I=1536, E=256, K=8, weight_bits=4,
                           act_int8=False, seed=4, router="zipf"),
    # NVFP4 (W4A4): the small block and the decode block at the mini model's MoE shape
    "tiny_nvfp4": Workload("tiny_nvfp4", T=32, H=256, I=128, E=8, K=2, weight_bits=4, act_int8=False,
                           fmt="nvfp4", seed=5),
    "decode_nvfp4": Workload("decode_nvfp4", T=32, H=2048, I=512, E=256, K=8, weight_bits=4, act_int8=False,
                             fmt="nvfp4"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 storage (nearest, ties to even); returns uint16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(a)
    out = r.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(wl: Workload) -> np.ndarray:
    n = int(np.floor(wl.outlier_frac * wl.H))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([wl.seed, 3])
    return np.sort(rng.choice(wl.H, size=n, replace=False))


def gen_x(wl: Workload) -> np.ndarray:
    """x[T,H] as bf16 bits (uint16)."""
    rng = np.random.default_rng([wl.seed, 0])
    x = rng.standard_normal((wl.T, wl.H), dtype=np.float32)
    ch = outlier_channels(wl)
    if ch.size:
        x[:, ch] *= np.float32(wl.outlier_scale)
    return f32_to_bf16_bits(x)


def zipf_log_popularity(wl: Workload) -> np.ndarray:
    """log p for each expert, p_r proportional to r^-s over a seeded rank permutation."""
    rng = np.random.default_rng([wl.seed, 4])
    rank = rng.permutation(wl.E) + 1
    logp = -wl.zipf_s * np.log(rank.astype(np.float64))
    logp -= np.log(np.exp(logp).sum())
    return logp.astype(np.float32)


def gen_router_logits(wl: Workload) -> np.ndarray:
    rng = np.random.default_rng([wl.seed, 2])
    if wl.router == "normal":
        return rng.standard_normal((wl.T, wl.E), dtype=np.float32)
    if wl.router == "zipf":
        # log-popularity plus Gumbel noise: the top-K is then a draw without
        # replacement proportional to popularity (Gumbel-top-k)
        g = rng.gumbel(size=(wl.T, wl.E)).astype(np.float32)
        return (g + zipf_log_popularity(wl)[None, :]).astype(np.float32)
    raise ValueError(wl.router)


def topk_softmax(logits: np.ndarray, K: int):
    """Router stand-in: top-K by logit (ties to the lower expert id), weights =
    float32 softmax over the selected logits with the max subtracted."""
    logits = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :K]
    sel = np.take_along_axis(logits, order, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True)).astype(np.float32)
    w = (z / z.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return order.astype(np.int32), w


def gen_routing(wl: Workload):
    return topk_softmax(gen_router_logits(wl), wl.K)


def weight_shape(wl: Workload, m: int):
    """[out, in] of matrix m: gate/up are [I, H], down is [H, I]."""
    return (wl.I, wl.H) if m in (GATE, UP) else (wl.H, wl.I)


def gen_expert_weight(wl: Workload, e: int, m: int) -> np.ndarray:
    rng = np.random.default_rng([wl.seed, 1, e, m])
    w = rng.standard_normal(weight_shape(wl, m), dtype=np.float32)
    w *= np.float32(wl.w_std)
    return w


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def iter_expert_weights(wl: Workload, experts, threads: int | None = None, chunk: int = 8):
    """Yield (e, [gate, up, down]) float32 arrays for each expert in `experts`,
    generated on a thread pool a few experts at a time (bounded memory)."""
    experts = list(experts)
    threads = threads or default_threads()

    def one(e):
        return e, [gen_expert_weight(wl, e, m) for m in (GATE, UP, DOWN)]

    with ThreadPoolExecutor(threads) as ex:
        for i in range(0, len(experts), chunk * threads):
            for item in ex.map(one, experts[i:i + chunk * threads]):
                yield item


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    """A seeded, sorted sample of n token indices that always includes the first
    and last token (the ragged tail of the block)."""
    if n >= T:
        return np.arange(T, dtype=np.int64)
    rng = np.random.default_rng([seed, 9])
    mid = rng.choice(np.arange(1, T - 1), size=max(0, n - 2), replace=False)
    return np.unique(np.concatenate([[0, T - 1], mid])).astype(np.int64)
