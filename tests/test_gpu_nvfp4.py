"""GPU parity of the NVFP4 (W4A4) path against the CPU oracle.

* the quantizers (inputs and weights): codes, E4M3 block scales and FP32 outer
  scales bit-exact against the oracle on the same inputs (ragged row counts,
  outlier channels, all-zero blocks and rows, blocks whose scale underflows);
* the two GEMM stages from the same quantized operands: every BF16 element at
  rounding level of the oracle's (one FP32 sum on the GPU, an exact sum on the
  oracle);
* the whole feed-forward at small sizes (all outputs) and at the decode
  block's full size (sampled tokens), in both row-tile heights, with the
  element-wise bar; edge cases (one token, dropped ids, all-zero weights);
  bit-identical reruns.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_routed_expert_top_amd as qre
from harness.inputs import WORKLOADS, Workload, f32_to_bf16_bits, gen_routing, gen_x, sample_tokens
from harness.synthetic import gpu_experts, touched_experts, x_tensor
from gpu_helpers import assert_forward_parity, assert_rounding_level, bf16_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def to_gpu(Wo: oracle.FP4Weights) -> qre.Nvfp4Experts:
    return qre.Nvfp4Experts(u8(Wo.gate_q), u8(Wo.gate_b), f32(Wo.gate_o), u8(Wo.up_q), u8(Wo.up_b), f32(Wo.up_o),
                            u8(Wo.down_q), u8(Wo.down_b), f32(Wo.down_o))


def np_all(t):
    return t.cpu().numpy()


# ---- quantizers ---------------------------------------------------------------------

def act_rows(rng, rows, cols):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[:, rng.integers(cols)] *= 40                                # an outlier channel
    x[1, :] = 0                                                   # an all-zero row
    x[2, 16:32] = 0                                               # an all-zero block
    x[3, 32:48] *= 1e-7                                           # a block whose scale underflows
    x[4] *= 1e-3
    return f32_to_bf16_bits(x)


@pytest.mark.parametrize("rows,cols", [(37, 256), (5, 16), (64, 2048), (130, 512)])
def test_quantize_act_bit_exact(rows, cols):
    rng = np.random.default_rng(100 + cols + rows)
    x = act_rows(rng, rows, cols)
    q, s, r = qre.nvfp4_quantize_act(x_tensor(x, DEV))
    oq, os_, orr = oracle.fp4_quantize_act(x)
    np.testing.assert_array_equal(np_all(r), orr)
    np.testing.assert_array_equal(np_all(s), os_)
    np.testing.assert_array_equal(np_all(q), oq)


def test_quantize_weights_bit_exact():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((3, 64, 256)) * 0.02).astype(np.float32)
    w[1, 5, 100] = 3.0                                            # one large weight sets matrix 1's outer scale
    w[2] = 0                                                      # an all-zero matrix
    q, s, o = qre.nvfp4_quantize_weights(f32(w))
    oq, os_, oo = oracle.fp4_quantize_weights(w)
    np.testing.assert_array_equal(np_all(o), oo)
    np.testing.assert_array_equal(np_all(s), os_)
    np.testing.assert_array_equal(np_all(q), oq)


def test_quantize_weights_full_expert_matrix():
    wl = WORKLOADS["decode_nvfp4"]
    from harness.inputs import GATE, DOWN, gen_expert_weight
    for m in (GATE, DOWN):
        w = gen_expert_weight(wl, 3, m)
        q, s, o = qre.nvfp4_quantize_weights(f32(w)[None])
        oq, os_, oo = oracle.fp4_quantize_weights(w[None])
        np.testing.assert_array_equal(np_all(o), oo)
        np.testing.assert_array_equal(np_all(s), os_)
        np.testing.assert_array_equal(np_all(q), oq)


# ---- GEMM stages ----------------------------------------------------------------------

STAGE = [
    Workload("f4_st_a", T=32, H=256, I=128, E=8, K=2, weight_bits=4, act_int8=False, fmt="nvfp4", seed=21),   # 16-row tiles
    Workload("f4_st_b", T=20, H=512, I=256, E=16, K=3, weight_bits=4, act_int8=False, fmt="nvfp4", seed=22),  # 8-row tiles
    Workload("f4_st_c", T=9, H=2048, I=512, E=64, K=8, weight_bits=4, act_int8=False, fmt="nvfp4", seed=23),  # decode shape
]


@pytest.mark.parametrize("wl", STAGE, ids=lambda w: w.name)
def test_stages_rounding_level(wl):
    x = gen_x(wl)
    ids, w = gen_routing(wl)
    Wo = oracle.fp4_workload_experts(wl, touched_experts(ids, wl.E))
    Wg = to_gpu(Wo)
    counts, offsets, sorted_slot, slot_row, _ = oracle.route(ids, wl.E)
    xq, xb, xr = oracle.fp4_quantize_act(x)
    shp = dict(T=wl.T, H=wl.H, I=wl.I, E=wl.E, K=wl.K)
    h_ref = oracle.fp4_gate_up(xq, xb, xr, sorted_slot, offsets, Wo, **shp)
    h = qre.nvfp4_gate_up(u8(xq), u8(xb), f32(xr), i32(sorted_slot), i32(offsets), Wg, wl.K)
    assert_rounding_level(bf16_np(h), h_ref, what=f"{wl.name} h")
    hq, hb, hr = oracle.fp4_quantize_act(h_ref)
    y_ref = oracle.fp4_down(hq, hb, hr, offsets, Wo, **shp)
    y = qre.nvfp4_down(u8(hq), u8(hb), f32(hr), i32(offsets), Wg, wl.T, wl.K)
    assert_rounding_level(bf16_np(y), y_ref, what=f"{wl.name} y")


# ---- the whole feed-forward ----------------------------------------------------------------

def run_forward(wl, x, ids, w, Wg):
    return bf16_np(qre.nvfp4_moe_forward(x_tensor(x, DEV), i32(ids), f32(w), Wg))


def check_forward(wl, tokens=None, x=None, ids=None, w=None, Wo=None, Wg=None):
    x = gen_x(wl) if x is None else x
    if ids is None:
        ids, w = gen_routing(wl)
    toks = np.arange(wl.T) if tokens is None else tokens
    if Wo is None:
        Wo = oracle.fp4_workload_experts(wl, touched_experts(ids[toks], wl.E))
    if Wg is None:
        Wg = to_gpu(Wo)
    out = run_forward(wl, x, ids, w, Wg)
    ref32, _, nbad, y_tok = oracle.fp4_moe_forward(x, ids, w, Wo, E=wl.E, tokens=None if tokens is None else toks,
                                                   return_y=True)
    assert_forward_parity(out[toks], ref32, y_tok, w[toks], what=wl.name)
    return out


SMALL = STAGE + [
    Workload("f4_sm_d", T=45, H=384, I=384, E=5, K=3, weight_bits=4, act_int8=False, fmt="nvfp4", seed=24),
    Workload("f4_sm_e", T=200, H=256, I=128, E=16, K=8, weight_bits=4, act_int8=False, fmt="nvfp4", seed=25,
             outlier_frac=0.02),
    # 512 slots: routing and the quantization of x share one launch; 513:
    # the routing kernel and the quantizer run as two launches
    Workload("f4_sm_f", T=64, H=256, I=128, E=32, K=8, weight_bits=4, act_int8=False, fmt="nvfp4", seed=29),
    Workload("f4_sm_g", T=57, H=256, I=128, E=32, K=9, weight_bits=4, act_int8=False, fmt="nvfp4", seed=30),
]


@pytest.mark.parametrize("wl", SMALL + [WORKLOADS["tiny_nvfp4"]], ids=lambda w: w.name)
def test_forward_small(wl):
    check_forward(wl)


def test_forward_decode_full_size_sampled():
    wl = WORKLOADS["decode_nvfp4"]
    Wg = gpu_experts(wl, DEV)                                     # the library's own weight quantizer
    ids, w = gen_routing(wl)
    toks = sample_tokens(wl.T, 12, seed=3)
    Wo = oracle.fp4_workload_experts(wl, touched_experts(ids[toks], wl.E))
    for name in ("gate", "up", "down"):                          # same bytes for every touched expert
        for e in touched_experts(ids[toks], wl.E):
            for part, dt in (("q", None), ("s", None), ("o", None)):
                g = getattr(Wg, f"{name}_{part}")[int(e)].cpu().numpy()
                o = getattr(Wo, f"{name}_{'b' if part == 's' else part}")[int(e)]
                np.testing.assert_array_equal(g, o)
    check_forward(wl, tokens=toks, ids=ids, w=w, Wo=Wo, Wg=Wg)


def test_forward_edges():
    base = Workload("f4_edge", T=6, H=256, I=128, E=4, K=2, weight_bits=4, act_int8=False, fmt="nvfp4", seed=26)
    x = gen_x(base)
    ids = np.array([[0, 1], [1, 7], [-1, 2], [3, 3], [2, 0], [1, 1]], np.int32)   # out of range, duplicates
    w = np.full((6, 2), 0.5, np.float32)
    Wo = oracle.fp4_workload_experts(base, range(4))
    out = check_forward(base, x=x, ids=ids, w=w, Wo=Wo)
    # one token
    one = base.with_(T=1, name="f4_one")
    check_forward(one, x=x[:1], ids=ids[:1], w=w[:1], Wo=Wo)
    # all-zero weights: exactly zero
    z = oracle.fp4_workload_experts(base, [])
    assert not run_forward(base, x, ids, w, to_gpu(z)).any()
    # bit-identical rerun
    np.testing.assert_array_equal(run_forward(base, x, ids, w, to_gpu(Wo)), out)


def test_argument_errors():
    wl = WORKLOADS["tiny_nvfp4"]
    with pytest.raises(qre.QreError):
        qre.nvfp4_workspace_bytes(wl.T, 100, wl.I, wl.E, wl.K)                # H not a multiple of 128
    with pytest.raises(qre.QreError):
        qre.nvfp4_workspace_bytes(64, 8192, 512, 8, 8)                          # x rows do not fit LDS


# ---- the forward against its own stages -----------------------------------------------

def stage_sequence(wl, x, ids, w, Wg):
    """The forward as separate launches: routing, quantization of x, gate/up,
    quantization of h, down, combine."""
    xt = x_tensor(x, DEV)
    counts, offsets, sorted_slot, slot_row, _ = qre.route(i32(ids), wl.E)
    xq, xs, xr = qre.nvfp4_quantize_act(xt)
    h = qre.nvfp4_gate_up(xq, xs, xr, sorted_slot, offsets, Wg, wl.K)
    hq, hs, hr = qre.nvfp4_quantize_act(h)
    y = qre.nvfp4_down(hq, hs, hr, offsets, Wg, wl.T, wl.K)
    return bf16_np(qre.combine(y, slot_row, f32(w)))


@pytest.mark.parametrize("name", ["decode_nvfp4", "f4_st_c"])
def test_forward_is_bit_identical_to_its_stages(name):
    wl = WORKLOADS[name] if name in WORKLOADS else next(w for w in STAGE if w.name == name)
    x = gen_x(wl)
    ids, w = gen_routing(wl)
    Wg = gpu_experts(wl, DEV)
    out = run_forward(wl, x, ids, w, Wg)
    np.testing.assert_array_equal(out, stage_sequence(wl, x, ids, w, Wg))


def test_forward_edges_8_row_tiles():
    """Decode-sized shapes with 8-row tiles and a 256-value step (reductions
    of 512): out-of-range and duplicate ids, one token, an expert with more
    rows than one tile; the forward equals its stages bit for bit."""
    base = Workload("f4_edge_fold", T=6, H=512, I=512, E=4, K=2, weight_bits=4, act_int8=False, fmt="nvfp4",
                    seed=27)
    x = gen_x(base)
    ids = np.array([[0, 1], [1, 7], [-1, 2], [3, 3], [2, 0], [1, 1]], np.int32)
    w = np.full((6, 2), 0.5, np.float32)
    Wo = oracle.fp4_workload_experts(base, range(4))
    Wg = to_gpu(Wo)
    check_forward(base, x=x, ids=ids, w=w, Wo=Wo, Wg=Wg)
    np.testing.assert_array_equal(run_forward(base, x, ids, w, Wg), stage_sequence(base, x, ids, w, Wg))
    check_forward(base.with_(T=1, name="f4_one_fold"), x=x[:1], ids=ids[:1], w=w[:1], Wo=Wo, Wg=Wg)
    # 32 slots over 16 experts (8-row tiles), expert 0 seeing 16 rows: two tiles
    many = base.with_(T=16, E=16, name="f4_many_rows", seed=28)
    xm = gen_x(many)
    idm = np.stack([np.zeros(16, np.int32), np.arange(16, dtype=np.int32) % 3 + 1], axis=1)
    wm = np.full((16, 2), 0.5, np.float32)
    Wm = oracle.fp4_workload_experts(many, range(4))
    Wmg = to_gpu(Wm)
    check_forward(many, x=xm, ids=idm, w=wm, Wo=Wm, Wg=Wmg)
    np.testing.assert_array_equal(run_forward(many, xm, idm, wm, Wmg), stage_sequence(many, xm, idm, wm, Wmg))
