"""End-to-end GPU parity of qre_moe_forward against the CPU oracle.

* every weight/activation mode on small problems that span several row tiles
  and ragged tails (all outputs compared);
* every workload at its full size, through the same call and launch
  configuration the benchmark times, compared on a seeded sample of tokens
  that always includes the first and the last;
* edge cases: one expert, top-1, duplicate ids, out-of-range ids (dropped and
  counted), a single token, zero tokens;
* GPU self-invariants: bit-identical reruns, token permutation, expert
  relabelling.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_routed_expert_top_amd as qre
from harness.inputs import (WORKLOADS, Workload, gen_routing, gen_x, sample_tokens, topk_softmax,
                            f32_to_bf16_bits)
from harness.synthetic import gpu_experts, touched_experts, x_tensor
from gpu_helpers import assert_forward_parity, bf16_np, oracle_experts, to_gpu_experts

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_gpu(x_bits, ids, w, W, act_int8):
    return qre.moe_forward(x_tensor(x_bits, DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), W,
                           act_int8=act_int8)


def _check(wl: Workload, tokens=None, x_bits=None, ids=None, w=None, Wg=None, Wo=None):
    x_bits = gen_x(wl) if x_bits is None else x_bits
    if ids is None:
        ids, w = gen_routing(wl)
    toks = np.arange(wl.T) if tokens is None else tokens
    if Wo is None:
        Wo = oracle_experts(wl, touched_experts(ids[toks], wl.E))
    if Wg is None:
        Wg = to_gpu_experts(Wo, wl.weight_bits) if tokens is None else gpu_experts(wl, DEV)
    out = bf16_np(_run_gpu(x_bits, ids, w, Wg, wl.act_int8))
    ref32, _, _, y_tok = oracle.moe_forward(x_bits, ids, w, Wo, E=wl.E, bits=wl.weight_bits, act_int8=wl.act_int8,
                                            tokens=None if tokens is None else toks, return_y=True)
    return assert_forward_parity(out[toks], ref32, y_tok, w[toks], what=wl.name)


SMALL = [
    Workload("small_a", T=64, H=512, I=256, E=8, K=2, weight_bits=4, act_int8=False, seed=11),
    Workload("small_b", T=45, H=384, I=384, E=5, K=3, weight_bits=8, act_int8=False, seed=12),
    Workload("small_c", T=100, H=256, I=128, E=16, K=4, weight_bits=4, act_int8=True, seed=13),
    Workload("small_d", T=77, H=640, I=256, E=12, K=6, weight_bits=8, act_int8=True, seed=14,
             outlier_frac=0.02),
    # more than 2048 slots: the separate routing launch and the 8-row tile GEMMs
    Workload("small_e", T=300, H=256, I=128, E=16, K=8, weight_bits=4, act_int8=False, seed=15),
    Workload("small_f", T=260, H=384, I=256, E=20, K=8, weight_bits=8, act_int8=True, seed=16),
    # reductions that are multiples of 512 (permutation folded into gate/up;
    # several row tiles per expert; more than 2048 slots, after the routing
    # kernel)
    Workload("ks_a", T=40, H=512, I=512, E=8, K=2, weight_bits=4, act_int8=False, seed=17),
    Workload("ks_b", T=200, H=1024, I=512, E=8, K=2, weight_bits=8, act_int8=True, seed=18),
    Workload("ks_c", T=280, H=512, I=1536, E=64, K=8, weight_bits=4, act_int8=True, seed=19),
    Workload("ks_d", T=64, H=2048, I=512, E=16, K=4, weight_bits=8, act_int8=False, seed=20),
    Workload("ks_e", T=96, H=1536, I=1024, E=12, K=3, weight_bits=4, act_int8=False, seed=21),
    # more than 2048 slots and fewer than 64 per expert: 16-row tiles with two
    # column fragments per gate/up wave, INT8 weights with INT8 and with BF16
    # activations
    Workload("rt_a", T=300, H=512, I=256, E=48, K=8, weight_bits=8, act_int8=True, seed=29),
    Workload("rt_b", T=300, H=1024, I=256, E=48, K=8, weight_bits=8, act_int8=False, seed=30),
    # decode blocks (at most 4 rows per expert on average) in all four modes;
    # a Zipf-skewed top-1 routing puts more than 8 rows on one expert (several
    # row tiles)
    Workload("ksd_a", T=12, H=512, I=512, E=16, K=4, weight_bits=4, act_int8=False, seed=26),
    Workload("ksd_b", T=20, H=1024, I=1024, E=32, K=4, weight_bits=8, act_int8=True, seed=27),
    Workload("ksd_c", T=16, H=1536, I=512, E=24, K=6, weight_bits=4, act_int8=True, seed=28),
    Workload("ksd_d", T=10, H=2048, I=1536, E=12, K=4, weight_bits=8, act_int8=False, seed=29),
    Workload("ksd_e", T=48, H=512, I=512, E=12, K=1, weight_bits=4, act_int8=False, seed=30, router="zipf"),
    # decode-sized blocks (permutation inside the gate/up kernel) with
    # reductions of 8/16 groups (gate/up) and 1/2/4 groups (down); one
    # expert holding all 33 rows (several row tiles); Zipf routing
    Workload("st_a", T=24, H=1024, I=128, E=8, K=2, weight_bits=4, act_int8=False, seed=31),
    Workload("st_b", T=30, H=1024, I=256, E=40, K=6, weight_bits=8, act_int8=False, seed=32),
    Workload("st_c", T=33, H=512, I=128, E=1, K=1, weight_bits=8, act_int8=False, seed=33),
    Workload("st_d", T=7, H=2048, I=512, E=64, K=8, weight_bits=4, act_int8=False, seed=34, router="zipf"),
    # at least 64 rows per expert on average: the big-tile MFMA kernels
    # (64-row tiles with BF16 activations, 128-row with INT8; several tiles
    # per expert with ragged tails; a reduction of one group; H = 640: a
    # down column block of 256 that is half past the width)
    Workload("big_a", T=600, H=256, I=128, E=4, K=2, weight_bits=4, act_int8=False, seed=22),
    Workload("big_b", T=700, H=384, I=256, E=6, K=3, weight_bits=8, act_int8=True, seed=23),
    Workload("big_c", T=500, H=512, I=384, E=5, K=2, weight_bits=4, act_int8=True, seed=24),
    Workload("big_d", T=400, H=640, I=256, E=3, K=2, weight_bits=8, act_int8=False, seed=25),
    # more than 8192 slots with INT8 activations: the three routing kernels,
    # the last of which also quantizes x; 128-row tiles (INT8 weights: gate/up
    # quantizes h in its epilogue) and 8-row tiles (INT4 weights)
    Workload("big_e", T=1100, H=256, I=128, E=16, K=8, weight_bits=8, act_int8=True, seed=35),
    Workload("big_f", T=1040, H=256, I=128, E=160, K=8, weight_bits=4, act_int8=True, seed=36),
]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("act_int8", [False, True])
def test_tiny_workload_all_modes(bits, act_int8):
    wl = WORKLOADS["tiny_w8a16"].with_(weight_bits=bits, act_int8=act_int8)
    _check(wl)


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_small_workloads(wl):
    _check(wl)


@pytest.mark.parametrize("name", ["decode_w4a16", "cb_w4a16", "cb_w8a16", "prefill_w8a8", "zipf_w4a16"])
def test_full_size_workload_sampled(name):
    wl = WORKLOADS[name]
    print(f"[full-size parity] {name}", flush=True)
    tokens = sample_tokens(wl.T, 24 if wl.T > 32 else wl.T, seed=1)
    st = _check(wl, tokens=tokens)
    print(f"  {name}: {st}", flush=True)


@pytest.mark.parametrize("bits,a8", [(4, False), (8, False), (4, True), (8, True)])
def test_decode_block_wide_hidden(bits, a8):
    """A 32-token block at H = 4096, I = 1536: the decode gate/up kernel with
    a 32-group reduction (permutation folded in), every output compared."""
    wl = Workload("dec_h4096", T=32, H=4096, I=1536, E=64, K=8, weight_bits=bits, act_int8=a8, seed=41)
    _check(wl)


@pytest.mark.parametrize("bits,a8", [(4, False), (8, False), (4, True), (8, True)])
def test_batched_blocks_wide_hidden_sampled(bits, a8):
    """Sixteen 32-token blocks at H = 4096, I = 1536, E = 256: the gate/up
    row tiles (4096-wide reduction) run the split-reduction kernel; sampled
    tokens (first and last included)."""
    wl = Workload("cb_h4096", T=512, H=4096, I=1536, E=256, K=8, weight_bits=bits, act_int8=a8, seed=42)
    _check(wl, tokens=sample_tokens(wl.T, 8, seed=2))


def test_decode_modes_at_full_size():
    """The decode shape in the three other weight/activation modes."""
    for bits, a8 in ((8, False), (4, True), (8, True)):
        wl = WORKLOADS["decode_w4a16"].with_(weight_bits=bits, act_int8=a8)
        _check(wl, tokens=np.arange(wl.T))


def test_edge_cases():
    rng = np.random.default_rng(3)
    # one expert, top-1
    wl = Workload("e1", T=33, H=256, I=128, E=1, K=1, weight_bits=4, act_int8=False, seed=21)
    _check(wl)
    # single token, K = E
    wl = Workload("t1", T=1, H=256, I=256, E=4, K=4, weight_bits=8, act_int8=True, seed=22)
    _check(wl)
    # duplicate ids within a token and out-of-range ids (dropped, counted)
    wl = Workload("dup", T=40, H=256, I=128, E=6, K=3, weight_bits=4, act_int8=False, seed=23)
    x_bits = gen_x(wl)
    ids, w = gen_routing(wl)
    ids[0, 1] = ids[0, 0]
    ids[1, :] = ids[1, 0]
    ids[5, 2] = -1
    ids[9, 0] = wl.E
    ids[17, 1] = 1 << 30
    Wo = oracle_experts(wl, range(wl.E))
    Wg = to_gpu_experts(Wo, wl.weight_bits)
    _check(wl, x_bits=x_bits, ids=ids, w=w, Wg=Wg, Wo=Wo)
    ws = torch.empty(qre.workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.K, 4), dtype=torch.uint8, device=DEV)
    qre.moe_forward(x_tensor(x_bits, DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), Wg,
                    workspace=ws)
    assert qre.read_device_error(ws) == 3
    # the same at a reduction of 4 groups, INT8 weights
    wl_st = Workload("dup_st", T=40, H=512, I=256, E=6, K=3, weight_bits=8, act_int8=False, seed=24)
    ids_st, w_st = gen_routing(wl_st)
    ids_st[0, 1] = ids_st[0, 0]
    ids_st[1, :] = ids_st[1, 0]
    ids_st[5, 2] = -1
    ids_st[9, 0] = wl_st.E
    Wo_st = oracle_experts(wl_st, range(wl_st.E))
    _check(wl_st, ids=ids_st, w=w_st, Wg=to_gpu_experts(Wo_st, wl_st.weight_bits), Wo=Wo_st)
    # zero tokens: nothing to do, output untouched
    out = torch.full((0, 256), 1.0, dtype=torch.bfloat16, device=DEV)
    qre.moe_forward(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV),
                    torch.empty((0, 3), dtype=torch.int32, device=DEV),
                    torch.empty((0, 3), dtype=torch.float32, device=DEV), Wg, out=out)


def test_invariances_decode_shape():
    wl = WORKLOADS["decode_w4a16"]
    x_bits = gen_x(wl)
    ids, w = gen_routing(wl)
    Wg = gpu_experts(wl, DEV)
    a = bf16_np(_run_gpu(x_bits, ids, w, Wg, False))
    for _ in range(2):                                        # bit-identical reruns
        np.testing.assert_array_equal(bf16_np(_run_gpu(x_bits, ids, w, Wg, False)), a)
    perm = np.random.default_rng(0).permutation(wl.T)          # token permutation
    np.testing.assert_array_equal(bf16_np(_run_gpu(x_bits[perm], ids[perm], w[perm], Wg, False)), a[perm])
    relabel = np.random.default_rng(1).permutation(wl.E)       # expert e -> relabel[e]
    inv = torch.from_numpy(np.argsort(relabel)).to(DEV)
    W2 = qre.QuantizedExperts(*(t[inv].contiguous() for t in (Wg.gate_q, Wg.gate_s, Wg.up_q, Wg.up_s,
                                                              Wg.down_q, Wg.down_s)), Wg.bits)
    np.testing.assert_array_equal(bf16_np(_run_gpu(x_bits, relabel[ids].astype(np.int32), w, W2, False)), a)


@pytest.mark.parametrize("T,H,I,E,K,bits,a8", [
    (32, 2048, 512, 256, 8, 4, False),     # decode block: permutation computed inside the gate/up kernel
    (32, 2048, 512, 256, 8, 4, True),      # the same with INT8 activations
    (40, 256, 128, 6, 3, 8, True),
    (300, 256, 128, 16, 8, 4, False),      # > 2048 slots: separate routing launch
    (300, 512, 512, 64, 8, 4, True),       # > 2048 slots, 16-row tile kernels
])
def test_forward_permutation_matches_oracle(T, H, I, E, K, bits, a8):
    """The permutation a forward call leaves in its workspace equals the
    oracle's stable counting sort, bit for bit, including dropped and
    duplicate ids."""
    wl = Workload("perm", T=T, H=H, I=I, E=E, K=K, weight_bits=bits, act_int8=a8, seed=T + E)
    x_bits = gen_x(wl)
    ids, w = gen_routing(wl)
    ids[0, -1] = ids[0, 0]
    ids[1, 0] = -1
    ids[T - 1, K - 1] = E + 3
    Wg = to_gpu_experts(oracle_experts(wl, [0]), bits)
    ws = torch.empty(qre.workspace_bytes(T, H, I, E, K, bits, a8), dtype=torch.uint8, device=DEV)
    qre.moe_forward(x_tensor(x_bits, DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), Wg,
                    act_int8=a8, workspace=ws)
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in qre.workspace_permutation(T, H, I, E, K, bits, a8, ws)]
    ref = oracle.route(ids, E)
    for g, r in zip(got, ref[:4]):
        np.testing.assert_array_equal(g, r)
    assert qre.read_device_error(ws) == ref[4] == 2
