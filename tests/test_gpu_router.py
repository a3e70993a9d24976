"""GPU parity of the router (top-K selection + softmax weights) against the
CPU oracle, through the C ABI: ids bit-exact, weights within the rounding
bound of the FP32 arithmetic, and the router's output feeding the
feed-forward."""
import numpy as np
import pytest
import torch

import oracle
import quantized_routed_expert_top_amd as qre
from harness.inputs import WORKLOADS, Workload, gen_router_logits, gen_x
from gpu_helpers import assert_forward_parity, bf16_np, oracle_experts, to_gpu_experts

pytestmark = pytest.mark.gpu
DEV = "cuda"
U = 2.0 ** -24


def _weight_tol(logits, ids):
    """Relative bound on each FP32 weight: the rounding of l_k - l_0 (|l_k - l_0|
    units), expf (two units), K rounded additions and one division (one unit
    each), plus slack of two units."""
    sel = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), axis=1)
    spread = np.abs(sel - sel[:, :1]).max(initial=0.0)
    return (spread + ids.shape[1] + 5) * U


def _check(logits, K):
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(DEV)
    ids, w = qre.topk_softmax(lg, K)
    ids2, w2 = qre.topk_softmax(lg, K)
    torch.cuda.synchronize()
    ids, w, ids2, w2 = (a.cpu().numpy() for a in (ids, w, ids2, w2))
    ref_ids, ref_w = oracle.topk_softmax(logits, K)
    np.testing.assert_array_equal(ids, ref_ids)
    tol = _weight_tol(logits, ref_ids)
    np.testing.assert_allclose(w, ref_w, rtol=tol, atol=0)
    np.testing.assert_array_equal(ids2, ids)          # reruns are bit-identical
    np.testing.assert_array_equal(w2, w)
    return ids, w


@pytest.mark.parametrize("T,E,K,seed", [
    (32, 256, 8, 0),          # one decode block
    (8192, 256, 8, 1),        # prefill-sized batch
    (4096, 256, 8, 2),
    (1, 1, 1, 3),             # one expert
    (9, 64, 64, 4),           # every expert selected
    (37, 100, 7, 5),          # ragged lanes (E not a multiple of 64)
    (130, 1024, 64, 6),       # largest E and K the router takes
    (5, 513, 3, 7),
    (3, 2, 2, 8),
])
def test_router_normal_logits(T, E, K, seed):
    rng = np.random.default_rng(seed)
    _check(rng.standard_normal((T, E)).astype(np.float32), K)


def test_router_zipf_logits():
    wl = WORKLOADS["zipf_w4a16"]
    _check(gen_router_logits(wl), wl.K)


def test_router_ties_and_signed_zero():
    rng = np.random.default_rng(11)
    l = rng.choice(np.array([-1.0, 0.0, 2.5], dtype=np.float32), size=(64, 200))
    l[::2][l[::2] == 0.0] = np.float32(-0.0)            # -0 and +0 are equal logits
    l[5, :] = 1.0                                       # all equal
    ids, w = _check(l, 8)
    assert list(ids[5]) == list(range(8))


def test_router_empty_batch():
    ids, w = qre.topk_softmax(torch.empty((0, 256), dtype=torch.float32, device=DEV), 8)
    assert ids.shape == (0, 8) and w.shape == (0, 8)


def test_router_feeds_forward():
    """Router output on the GPU, then the feed-forward on the GPU, against the
    oracle's router and feed-forward on the same logits."""
    wl = Workload("router_ffn", T=48, H=512, I=256, E=16, K=4, weight_bits=4, act_int8=False, seed=21)
    logits = gen_router_logits(wl)
    ids_ref, w_ref = oracle.topk_softmax(logits, wl.K)
    Wo = oracle_experts(wl, range(wl.E))
    x_bits = gen_x(wl)
    ref32, _, _, y_tok = oracle.moe_forward(x_bits, ids_ref, w_ref, Wo, E=wl.E, bits=wl.weight_bits, return_y=True)
    ids, w = qre.topk_softmax(torch.from_numpy(logits).to(DEV), wl.K)
    x = torch.from_numpy(x_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    out = qre.moe_forward(x, ids, w, to_gpu_experts(Wo, wl.weight_bits, DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    assert_forward_parity(bf16_np(out), ref32, y_tok, w_ref, what="router_ffn")


def test_router_non_finite_logits_keep_ids_valid():
    """NaN and infinite logits are unspecified input for the weights, but the
    ids must stay distinct and inside [0, E) (the header's guarantee)."""
    rng = np.random.default_rng(13)
    T, E, K = 16, 100, 8
    l = rng.standard_normal((T, E)).astype(np.float32)
    l[0, :] = np.nan                                    # every logit NaN
    l[1, : E - 3] = np.nan                              # fewer finite logits than K
    l[2, 5] = np.inf
    l[3, :] = -np.inf
    ids, _ = qre.topk_softmax(torch.from_numpy(l).to(DEV), K)
    ids = ids.cpu().numpy()
    assert ids.min() >= 0 and ids.max() < E
    for t in range(T):
        assert len(set(ids[t].tolist())) == K
    assert set(ids[1, :3].tolist()) == {E - 3, E - 2, E - 1}   # the finite ones first
    assert ids[2, 0] == 5
    assert list(ids[3]) == list(range(K))                # all equal (-inf): lowest ids
