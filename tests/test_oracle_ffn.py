"""Pins of the oracle's expert feed-forward, its INT8-activation mode and the
per-token combine.

What the pages fix (minnow README "Quantization"; model card "LLaDA2.2-flash for
minnow", "Checkpoints and precision"): routed experts are gate/up/down
projections with SiLU on the gate, fed BF16 activations and dequantized
weights; the INT8-activation mode uses INT32 group dot products whose scaled
groups are combined in FP32; expert outputs return to BF16.

Pins, chosen so that a dropped term, a swapped operand, a wrong index or a
wrong scale fails one of them:
  * one expert, top-1 reduces to a dense quantized SwiGLU MLP: checked against
    torch float64 matmul and F.silu on independently dequantized weights;
  * a closed-form case (exact integers, power-of-two scales, saturated SiLU);
  * INT8 activations on inputs that lie exactly on the INT8 grid give the same
    result as BF16 activations;
  * the combine: identity, exact doubling, one-hot selection, dropped slots;
  * brute force over tokens on tiny shapes, and token/expert relabelling.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from harness.inputs import bf16_bits_to_f32, f32_to_bf16_bits, topk_softmax
from np_ref import (np_bf16_bits, np_codes, np_dequant, np_quantize_act, np_round_bf16, np_scales)


# ---- independent helpers (numpy bit operations, numpy float16) -----------------

def half_ulp_bf16(v):
    v = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(np.where(v == 0, 1.0, v))       # v = m 2^e, m in [0.5,1)
    e = np.maximum(e - 1, -126)
    return np.ldexp(1.0, e - 8)


def quantize_experts(ws, bits):
    """ws: list over experts of [gate, up, down] float32 -> oracle.QWeights."""
    qs = [[oracle.quantize_weights(m, bits) for m in e] for e in ws]
    stack = lambda j, k: np.stack([qs[e][j][k] for e in range(len(ws))])
    return oracle.QWeights(stack(0, 0), stack(0, 1), stack(1, 0), stack(1, 1), stack(2, 0), stack(2, 1))


def rand_experts(rng, E, H, I, std=0.02):
    return [[(rng.standard_normal(sh) * std).astype(np.float32) for sh in ((I, H), (I, H), (H, I))]
            for _ in range(E)]


# ---- dense reduction: E = K = 1 is a quantized SwiGLU MLP -------------------------

@pytest.mark.parametrize("bits", [4, 8])
def test_single_expert_is_dense_swiglu(bits):
    rng = np.random.default_rng(20 + bits)
    T, H, I = 6, 384, 256
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    W = quantize_experts(rand_experts(rng, 1, H, I), bits)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    counts, offsets, sorted_slot, slot_row, _ = oracle.route(ids, 1)
    shp = dict(T=T, H=H, I=I, E=1, K=1, bits=bits)
    h = oracle.gate_up(x, sorted_slot, offsets, W, **shp)
    y = oracle.down(h, offsets, W, **shp)
    o32, o16, nbad = oracle.moe_forward(x, ids, w, W, E=1, bits=bits)

    xt = torch.from_numpy(bf16_bits_to_f32(x).astype(np.float64))
    Wg = torch.from_numpy(np_dequant(W.gate_q[0], W.gate_s[0], H, bits))
    Wu = torch.from_numpy(np_dequant(W.up_q[0], W.up_s[0], H, bits))
    Wd = torch.from_numpy(np_dequant(W.down_q[0], W.down_s[0], I, bits))
    h_exact = (F.silu(xt @ Wg.T) * (xt @ Wu.T)).numpy()
    hf = bf16_bits_to_f32(h).astype(np.float64)
    assert np.all(np.abs(hf - h_exact) <= half_ulp_bf16(h_exact) * (1 + 1e-9))
    y_exact = (torch.from_numpy(hf) @ Wd.T).numpy()
    yf = bf16_bits_to_f32(y).astype(np.float64)
    assert np.all(np.abs(yf - y_exact) <= half_ulp_bf16(y_exact) * (1 + 1e-9))
    # top-1 with weight 1: out = y exactly
    assert nbad == 0
    np.testing.assert_array_equal(o32, yf.astype(np.float32))
    np.testing.assert_array_equal(o16, y)
    # the gate really goes through SiLU and the up projection does not
    h_swapped = (F.silu(xt @ Wu.T) * (xt @ Wg.T)).numpy()
    assert np.abs(hf - h_swapped).max() > 10 * half_ulp_bf16(h_exact).max()


# ---- closed form: exact integers, power-of-two scales, saturated SiLU -------------

def test_closed_form_exact_case():
    H = I = 128
    a = 64.0
    # gate row i: 127/128 at input 0 -> g = a * 127/128 = 63.5 >= 17 (SiLU(g) = g to
    # far below BF16 precision); up row i: 2/128 at input 0 (u = 1) and a max
    # element 127/128 at input 1, where x is 0.  Every group max is 127/128 so
    # each FP16 scale is exactly 2^-7 and the codes are the integers below.
    gate = np.zeros((I, H), np.float32)
    gate[:, 0] = 127 / 128
    up = np.zeros((I, H), np.float32)
    up[:, 0] = 2 / 128
    up[:, 1] = 127 / 128
    down = np.zeros((H, I), np.float32)
    c = np.arange(H) % 5
    down[np.arange(H), np.arange(H) % I] = 127 / 128
    down[np.arange(H), (np.arange(H) + 1) % I] = c / 128
    W = quantize_experts([[gate, up, down]], 8)
    assert np.all(W.gate_s == np.float16(2 ** -7).view(np.uint16))
    x = np.zeros((2, H), np.float32)
    x[0, 0] = a
    x[1, 0] = -2 * a                               # g = -127, u = -2
    xb = f32_to_bf16_bits(x)
    ids = np.zeros((2, 1), np.int32)
    o32, o16, _ = oracle.moe_forward(xb, ids, np.ones((2, 1), np.float32), W, E=1, bits=8)
    # token 0: h_i = 63.5 for all i; y_j = 63.5 (127 + c_j) / 128, rounded to BF16
    expect = [oracle.round_bf16(float(Fraction(127, 2) * (127 + int(cj)) / 128)) for cj in c]
    np.testing.assert_array_equal(o32[0], np.array(expect, np.float32))
    # token 1: SiLU(-127) * -2 = 254 e^-127 ~ 1.8e-53, below half of BF16's smallest
    # subnormal 2^-133, so h rounds to zero and so does everything after it
    np.testing.assert_array_equal(np.abs(o32[1]), 0.0)


# ---- INT8 activations on grid inputs equal BF16 activations -----------------------

@pytest.mark.parametrize("bits", [4, 8])
def test_int8_activations_match_bf16_on_grid_inputs(bits):
    """If every x group is c * 2^k with integer |c| <= 127 and one |c| = 127,
    INT8 quantization of x is exact; with power-of-two weight scales every
    group partial is a multiple of 2^-15 far below 2^9, so the partials and
    their FP32 sums are exact and the INT32-group / FP32 combination must give
    the same g, u (and so the same BF16 h) as the BF16 path."""
    rng = np.random.default_rng(30 + bits)
    T, H, I = 8, 384, 128
    qmax = 7 if bits == 4 else 127
    xc = rng.integers(-127, 128, size=(T, H))
    xc[:, ::128] = 127
    x = (xc * 2.0 ** -6).astype(np.float32)
    xb = f32_to_bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(xb), x)            # 8-bit integers fit BF16
    def grid_w(rows, cols):
        wc = rng.integers(-qmax, qmax + 1, size=(rows, cols))
        wc[:, ::128] = qmax
        return (wc * 2.0 ** -9).astype(np.float32)
    W = quantize_experts([[grid_w(I, H), grid_w(I, H), grid_w(H, I)]], bits)
    ids = np.zeros((T, 1), np.int32)
    _, offsets, sorted_slot, _, _ = oracle.route(ids, 1)
    xq, xs = oracle.quantize_act(xb)
    assert np.all(xs == 2.0 ** -6)
    np.testing.assert_array_equal(xq, xc)
    shp = dict(T=T, H=H, I=I, E=1, K=1, bits=bits)
    h16 = oracle.gate_up(xb, sorted_slot, offsets, W, **shp)
    h8 = oracle.gate_up(None, sorted_slot, offsets, W, act_int8=True, xq=xq, xs=xs, **shp)
    np.testing.assert_array_equal(h8, h16)
    # down: feed an on-grid h to both modes
    hc = rng.integers(-127, 128, size=(T, I))
    hc[:, 0] = -127
    hb = f32_to_bf16_bits((hc * 2.0 ** -3).astype(np.float32))
    hq, hs = oracle.quantize_act(hb)
    y16 = oracle.down(hb, offsets, W, **shp)
    y8 = oracle.down(None, offsets, W, act_int8=True, hq=hq, hs=hs, **shp)
    np.testing.assert_array_equal(y8, y16)


def test_int8_group_sums_at_extremes():
    """Every product at its extreme: 128 * 127 * 127 = 2064512 < 2^24, so the
    INT32 group sum converts to FP32 exactly."""
    H = I = 128
    gate = np.full((I, H), 127 / 128, np.float32)
    up = np.full((I, H), -1 / 128, np.float32)
    up[:, 0] = -127 / 128
    down = np.full((H, I), 127 / 128, np.float32)
    W = quantize_experts([[gate, up, down]], 8)
    x = f32_to_bf16_bits(np.full((1, H), 127 * 2.0 ** -4, np.float32))
    xq, xs = oracle.quantize_act(x)
    assert np.all(xq == 127) and xs[0, 0] == 2.0 ** -4
    _, offsets, sorted_slot, _, _ = oracle.route(np.zeros((1, 1), np.int32), 1)
    h = oracle.gate_up(None, sorted_slot, offsets, W, T=1, H=H, I=I, E=1, K=1, bits=8, act_int8=True,
                       xq=xq, xs=xs)
    g = 128 * 127 * 127 * 2.0 ** -4 * 2.0 ** -7
    u = (127 * -127 + 127 * -1 * 127) * 2.0 ** -4 * 2.0 ** -7
    expect = oracle.round_bf16(g / (1 + np.exp(-g)) * u)
    np.testing.assert_array_equal(bf16_bits_to_f32(h)[0], np.float32(expect))


# ---- combine -------------------------------------------------------------------

def test_combine_identity_doubling_onehot_and_drops():
    rng = np.random.default_rng(40)
    T, K, H = 5, 3, 256
    S = T * K
    y = f32_to_bf16_bits(rng.standard_normal((S, H)).astype(np.float32))
    yf = bf16_bits_to_f32(y)
    ids = rng.integers(0, 4, size=(T, K)).astype(np.int32)
    _, _, _, slot_row, _ = oracle.route(ids, 4)
    w = rng.random((T, K)).astype(np.float32)
    o32, _ = oracle.combine(y, slot_row, w, T=T, K=K, H=H)
    o32x2, _ = oracle.combine(y, slot_row, w * 2, T=T, K=K, H=H)
    np.testing.assert_array_equal(o32x2, o32 * 2)               # scaling by 2 is exact
    onehot = np.zeros((T, K), np.float32)
    onehot[np.arange(T), np.arange(T) % K] = 1.0
    o1, o1b = oracle.combine(y, slot_row, onehot, T=T, K=K, H=H)
    pick = slot_row.reshape(T, K)[np.arange(T), np.arange(T) % K]
    np.testing.assert_array_equal(o1, yf[pick])
    np.testing.assert_array_equal(o1b, y[pick])
    # K = 1, w = 1: the identity
    o, ob = oracle.combine(y[:T], np.arange(T, dtype=np.int32), np.ones((T, 1), np.float32), T=T, K=1, H=H)
    np.testing.assert_array_equal(ob, y[:T])
    # a dropped slot contributes nothing
    sr = slot_row.copy()
    sr[0] = -1
    od, _ = oracle.combine(y, sr, w, T=T, K=K, H=H)
    w0 = w.copy()
    w0[0, 0] = 0.0
    oz, _ = oracle.combine(y, slot_row, w0, T=T, K=K, H=H)
    np.testing.assert_array_equal(od, oz)
    # the sum is a chain of single-rounding FMAs, k ascending (exact rational check)
    t, j = 2, 17
    acc = np.float32(0.0)
    for k in range(K):
        exact = Fraction(float(w[t, k])) * Fraction(float(yf[slot_row[t * K + k], j])) + Fraction(float(acc))
        acc = np.float32(oracle_round_f32(exact))
    assert o32[t, j] == acc


def oracle_round_f32(fr: Fraction) -> float:
    """Nearest-even float32 of an exact rational (test helper, no oracle code)."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    r = int(n)
    rem = n - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    return sign * float(r * quantum)


# ---- brute force over tokens and relabelling invariances -------------------------

def brute_force(x, ids, w, ws_deq, H, I):
    """Token-major float64 evaluation with the pipeline's BF16 rounding points."""
    T, K = ids.shape
    xf = bf16_bits_to_f32(x).astype(np.float64)
    rb = np.vectorize(oracle.round_bf16)
    out = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            g_, u_, d_ = ws_deq[ids[t, k]]
            g = g_ @ xf[t]
            u = u_ @ xf[t]
            h = rb(g / (1 + np.exp(-g)) * u)
            y = rb(d_ @ h)
            out[t] += float(w[t, k]) * y
    return out


@pytest.mark.parametrize("bits", [4, 8])
def test_brute_force_tiny(bits):
    rng = np.random.default_rng(50 + bits)
    T, H, I, E, K = 12, 256, 128, 5, 2
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ids, w = topk_softmax(rng.standard_normal((T, E)).astype(np.float32), K)
    W = quantize_experts(rand_experts(rng, E, H, I), bits)
    deq = [(np_dequant(W.gate_q[e], W.gate_s[e], H, bits), np_dequant(W.up_q[e], W.up_s[e], H, bits),
            np_dequant(W.down_q[e], W.down_s[e], I, bits)) for e in range(E)]
    o32, o16, nbad = oracle.moe_forward(x, ids, w, W, E=E, bits=bits)
    ref = brute_force(x, ids, w, deq, H, I)
    assert nbad == 0
    assert np.max(np.abs(o32 - ref)) <= 1e-6 * np.max(np.abs(ref))
    # sampled-token evaluation gives the same rows
    tok = np.array([0, 5, 11])
    s32, s16, _ = oracle.moe_forward(x, ids, w, W, E=E, bits=bits, tokens=tok)
    np.testing.assert_array_equal(s32, o32[tok])
    np.testing.assert_array_equal(s16, o16[tok])


@pytest.mark.parametrize("act_int8", [False, True])
def test_token_and_expert_relabelling(act_int8):
    rng = np.random.default_rng(60)
    T, H, I, E, K = 16, 256, 128, 6, 3
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ids, w = topk_softmax(rng.standard_normal((T, E)).astype(np.float32), K)
    ws = rand_experts(rng, E, H, I)
    W = quantize_experts(ws, 4)
    o32, o16, _ = oracle.moe_forward(x, ids, w, W, E=E, bits=4, act_int8=act_int8)
    perm = rng.permutation(T)
    p32, _, _ = oracle.moe_forward(x[perm], ids[perm], w[perm], W, E=E, bits=4, act_int8=act_int8)
    np.testing.assert_array_equal(p32, o32[perm])
    relabel = rng.permutation(E)                 # expert e becomes relabel[e]
    inv = np.argsort(relabel)
    W2 = quantize_experts([ws[inv[e]] for e in range(E)], 4)
    r32, _, _ = oracle.moe_forward(x, relabel[ids].astype(np.int32), w, W2, E=E, bits=4, act_int8=act_int8)
    np.testing.assert_array_equal(r32, o32)
    # dropping a slot (id out of range) equals giving it zero weight
    ids_bad = ids.copy()
    ids_bad[3, 1] = E + 7
    b32, _, nbad = oracle.moe_forward(x, ids_bad, w, W, E=E, bits=4, act_int8=act_int8)
    w0 = w.copy()
    w0[3, 1] = 0.0
    z32, _, _ = oracle.moe_forward(x, ids, w0, W, E=E, bits=4, act_int8=act_int8)
    assert nbad == 1
    np.testing.assert_array_equal(b32, z32)


# ---- INT8 activations: token-major brute force of the whole chain -----------------

def _np_group_dot_f32(xq, xs, codes, wsc):
    """FP32 combination of exact INT32 group dot products, groups ascending:
    acc = acc + float(isum_g) * (xs_g * ws_g), each operation rounded to FP32.
    xq [n] codes, xs [n/128]; codes [rows, n]; wsc [rows, n/128] FP32 scales."""
    rows, n = codes.shape
    G = n // 128
    isum = (codes.reshape(rows, G, 128) * np.asarray(xq, np.int64).reshape(1, G, 128)).sum(axis=2)
    assert np.abs(isum).max() < 2 ** 31
    acc = np.zeros(rows, np.float32)
    for g in range(G):
        sc = (np.float32(xs[g]) * wsc[:, g]).astype(np.float32)
        acc = (acc + (isum[:, g].astype(np.float32) * sc).astype(np.float32)).astype(np.float32)
    return acc


def a8_brute_force(x, ids, w, W, H, I, bits):
    """Per token, per routed expert: quantize x, INT32 group sums over dense
    unpacked codes, FP32 group combination, h = bf16(silu(g) u) in float64,
    quantize h, the same for down, y = bf16(acc); out by an FMA chain over k
    (w*y is exact in float64).  Returns (h [T,K,I], y [T,K,H], out [T,H]) as
    float64 values."""
    T, K = ids.shape
    xq, xs = np_quantize_act(x)
    hs_all = np.zeros((T, K, I))
    ys_all = np.zeros((T, K, H))
    out = np.zeros((T, H), np.float32)
    for t in range(T):
        acc = np.float32(0.0)
        acc = np.zeros(H, np.float32)
        for k in range(K):
            e = ids[t, k]
            cg, cu = np_codes(W.gate_q[e], H, bits), np_codes(W.up_q[e], H, bits)
            g = _np_group_dot_f32(xq[t], xs[t], cg, np_scales(W.gate_s[e])).astype(np.float64)
            u = _np_group_dot_f32(xq[t], xs[t], cu, np_scales(W.up_s[e])).astype(np.float64)
            h = np_round_bf16(g / (1.0 + np.exp(-g)) * u)
            hq, hsc = np_quantize_act(np_bf16_bits(h)[None, :])
            cd = np_codes(W.down_q[e], I, bits)
            y = np_round_bf16(_np_group_dot_f32(hq[0], hsc[0], cd, np_scales(W.down_s[e])).astype(np.float64))
            hs_all[t, k], ys_all[t, k] = h, y
            acc = (np.float64(w[t, k]) * y + acc.astype(np.float64)).astype(np.float32)
        out[t] = acc
    return hs_all, ys_all, out


@pytest.mark.parametrize("bits", [4, 8])
def test_int8_activation_chain_brute_force(bits):
    """The INT8-activation chain (quantize x, INT32 groups, FP32 combination,
    BF16 h, quantize h, down, BF16 y, combine) against a token-major numpy
    evaluation over dense unpacked codes: K = 3 experts per token, activation
    scales that differ per token and per group (outlier channels), weight
    scales that differ per row and group.  h, y and the FP32 output agree bit
    for bit."""
    rng = np.random.default_rng(70 + bits)
    T, H, I, E, K = 12, 384, 256, 5, 3
    xf = rng.standard_normal((T, H)).astype(np.float32)
    xf[:, rng.choice(H, 4, replace=False)] *= 20.0
    xf[3] *= 0.01
    x = f32_to_bf16_bits(xf)
    ids, w = topk_softmax(rng.standard_normal((T, E)).astype(np.float32), K)
    ws = rand_experts(rng, E, H, I)
    ws[2][0][:, :128] *= 8.0                     # one expert's gate: a group of much larger scale
    W = quantize_experts(ws, bits)
    h_bf, y_bf, out_bf = a8_brute_force(x, ids, w, W, H, I, bits)
    o32, _, nbad, y_tok = oracle.moe_forward(x, ids, w, W, E=E, bits=bits, act_int8=True, return_y=True)
    assert nbad == 0
    np.testing.assert_array_equal(bf16_bits_to_f32(y_tok).astype(np.float64), y_bf)
    np.testing.assert_array_equal(o32, out_bf)
    # h through the oracle's stage call on the oracle's own x quantization
    xq, xs = oracle.quantize_act(x)
    _, offsets, sorted_slot, slot_row, _ = oracle.route(ids, E)
    h = oracle.gate_up(None, sorted_slot, offsets, W, T=T, H=H, I=I, E=E, K=K, bits=bits, act_int8=True,
                       xq=xq, xs=xs)
    np.testing.assert_array_equal(bf16_bits_to_f32(h[slot_row]).astype(np.float64), h_bf.reshape(T * K, I))
    # the chain is not trivially exact: scales are not powers of two and
    # INT8 activations differ from the BF16-activation result
    o16a, _, _ = oracle.moe_forward(x, ids, w, W, E=E, bits=bits, act_int8=False)
    assert np.abs(o16a - o32).max() > 0
