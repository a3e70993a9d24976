"""The allocation-free entry point: qre_moe_forward_noalloc through the C ABI
gives bit for bit what qre_moe_forward gives (same kernels, the library's own
workspace), on two calls in a row, the second smaller than the first, and in
every weight/activation mode of a decode block."""
import numpy as np
import pytest
import torch

import quantized_routed_expert_top_amd as qre
from harness.inputs import WORKLOADS, Workload, gen_routing, gen_x
from harness.synthetic import gpu_experts, x_tensor

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(wl, T=None):
    x_bits = gen_x(wl)
    ids, w = gen_routing(wl)
    if T is not None:
        x_bits, ids, w = x_bits[:T], ids[:T], w[:T]
    return x_tensor(np.ascontiguousarray(x_bits), DEV), torch.from_numpy(np.ascontiguousarray(ids)).to(DEV), \
        torch.from_numpy(np.ascontiguousarray(w)).to(DEV)


@pytest.mark.parametrize("bits,a8", [(4, False), (8, False), (4, True), (8, True)])
def test_noalloc_matches_forward_two_calls(bits, a8):
    wl = WORKLOADS["decode_w4a16"].with_(weight_bits=bits, act_int8=a8)
    print(f"[no-alloc] W{bits}A{8 if a8 else 16} T=32 then T=7", flush=True)
    W = gpu_experts(wl, DEV)
    for T in (32, 7):                                   # the second call is smaller
        x, ids, w = _inputs(wl, T)
        ref = qre.moe_forward(x, ids, w, W, act_int8=a8)
        got = qre.moe_forward_noalloc(x, ids, w, W, act_int8=a8)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"T={T}"


def test_noalloc_batched_blocks_and_limit():
    """Sixteen 32-token blocks fit the library's workspace; an 8192-token
    prefill does not and is refused before anything is enqueued."""
    wl = WORKLOADS["cb_w4a16"]
    W = gpu_experts(wl, DEV)
    x, ids, w = _inputs(wl)
    ref = qre.moe_forward(x, ids, w, W)
    got = qre.moe_forward_noalloc(x, ids, w, W)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert qre.workspace_bytes(8192, 2048, 512, 256, 8, 8, True) > qre.NOALLOC_SCRATCH_BYTES
    big = Workload("big", T=8192, H=2048, I=512, E=256, K=8, weight_bits=4, act_int8=False)
    xb = torch.zeros((big.T, big.H), dtype=torch.bfloat16, device=DEV)
    ib = torch.zeros((big.T, big.K), dtype=torch.int32, device=DEV)
    wb = torch.zeros((big.T, big.K), dtype=torch.float32, device=DEV)
    with pytest.raises(qre.QreError) as ei:
        qre.moe_forward_noalloc(xb, ib, wb, W)
    assert ei.value.status == -9
