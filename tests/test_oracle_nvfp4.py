"""Pins of the oracle's NVFP4 (W4A4) format and feed-forward.

What the pages fix (model card "LLaDA2.2-flash for minnow", precision table,
NVFP4 row; README "Quantization"): E2M1 weights and inputs, an E4M3 scale per 16
values, an FP32 outer scale per expert matrix (weights) or per input row
(inputs), FP32 accumulation; the printed NVFP4 checkpoint size.

Pins, chosen so that a wrong table entry, a wrong tie rule, a dropped scale, a
swapped outer scale or a wrong nibble order fails one of them:
  * the E2M1 value set of the OCP Microscaling (MX) formats specification, FP4
    E2M1 (a literal table), and E4M3 decoding/encoding against torch's
    float8_e4m3fn (round to nearest even);
  * E2M1 rounding against a brute-force nearest search with the even-code tie
    rule;
  * the block quantizer: its rounding decisions re-derived from the FP32
    quotients with the library E4M3 conversion and the brute-force E2M1 search;
    exact round trips of representable inputs; the largest element lands on
    the format maxima; power-of-two scaling moves only the outer scale;
  * the packed size reproduces the printed NVFP4 checkpoint sizes;
  * the whole feed-forward against a float64 torch computation on decoded
    operands (tiny shapes), and the all-zero case.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from harness.inputs import bf16_bits_to_f32, f32_to_bf16_bits, topk_softmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "checkpoint_sizes.txt")

# OCP Microscaling Formats (MX) v1.0, FP4 (E2M1): 1 sign, 2 exponent bits
# (bias 1), 1 mantissa bit; the positive codes 0..7 encode these values.
E2M1_POS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E2M1 = np.array(E2M1_POS + [-v for v in E2M1_POS])


def torch_e4m3_value(b):
    b = np.ascontiguousarray(b, dtype=np.uint8)
    return torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_e4m3_encode(v32):
    v = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32))
    return v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def brute_e2m1(v):
    """Nearest E2M1 code by exhaustive search; ties to the even code; beyond 6
    saturates; a result of magnitude 0 is code 0."""
    best, bd = 0, None
    for c in range(16):
        d = abs(v - E2M1[c])
        if bd is None or d < bd or (d == bd and (c & 1) == 0 and (best & 1) == 1):
            best, bd = c, d
    return 0 if E2M1[best] == 0 else best


def decode_codes(q, cols):
    q = np.asarray(q, np.uint8)
    c = np.empty(q.shape[:-1] + (cols,), np.int64)
    c[..., 0::2] = q & 0xF
    c[..., 1::2] = q >> 4
    return c


def decode(q, b, cols):
    """E2M1 * E4M3 per element (no outer scale), float64, from the literal table
    and torch's E4M3 decoding."""
    return E2M1[decode_codes(q, cols)] * np.repeat(torch_e4m3_value(b), 16, axis=-1)


# ---- number formats -------------------------------------------------------------

def test_e2m1_table():
    assert [oracle.e2m1_value(c) for c in range(16)] == list(E2M1)
    assert np.signbit(oracle.e2m1_value(8)) and oracle.e2m1_value(8) == 0.0


def test_e4m3_decode_all_bytes_matches_torch():
    ref = torch_e4m3_value(np.arange(256))
    ours = np.array([oracle.e4m3_value(b) for b in range(256)])
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])
    assert np.all(np.isnan(ours[~fin])) and (~fin).sum() == 2      # 0x7F and 0xFF only
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(1)
    vals = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    mids = (vals[1:] + vals[:-1]) / 2                               # every tie between neighbours
    v = np.concatenate([rng.uniform(0, 448, 3000), rng.uniform(0, 2.0 ** -5, 1000), mids, vals,
                        -rng.uniform(0, 448, 500)]).astype(np.float32)
    ours = np.array([oracle.e4m3_encode(float(a)) for a in v], np.uint8)
    np.testing.assert_array_equal(ours, torch_e4m3_encode(v))
    # past the largest finite value the reading saturates (torch's cast gives NaN there)
    for big in (448.5, 464.0, 500.0, 1e30):
        assert oracle.e4m3_encode(big) == 0x7E and oracle.e4m3_encode(-big) == 0xFE


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(2)
    ties = [(a + b) / 2 for a, b in zip(E2M1_POS[:-1], E2M1_POS[1:])]
    v = np.concatenate([rng.uniform(-8, 8, 4000), ties, [-t for t in ties], E2M1, [6.5, 7.0, 100.0, -7.0,
                        1e-30, -1e-30, -0.2]])
    for a in v:
        assert oracle.e2m1_encode(float(a)) == brute_e2m1(float(a)), a


# ---- the block quantizer ------------------------------------------------------------

def rederive(v32):
    """The quantizer's decisions for one float32 row, from its FP32 quotients:
    outer S = amax / 2688, block scale = E4M3 (torch) of amax_block / (S * 6),
    codes = brute-force E2M1 of v / (scale * S)."""
    v32 = np.asarray(v32, np.float32)
    S = np.float32(np.abs(v32).max()) / np.float32(2688.0)
    den = np.float32(S * np.float32(6.0))
    blocks = v32.reshape(-1, 16)
    amax = np.abs(blocks).max(axis=1).astype(np.float32)
    d = (amax / den).astype(np.float32) if den > 0 else np.zeros_like(amax)
    b = torch_e4m3_encode(np.minimum(d, np.float32(448.0)))
    den2 = (torch_e4m3_value(b).astype(np.float32) * S).astype(np.float32)
    codes = np.zeros(blocks.shape, np.int64)
    for i in range(blocks.shape[0]):
        if den2[i] > 0:
            q = (blocks[i] / den2[i]).astype(np.float32)
            codes[i] = [brute_e2m1(float(a)) for a in q]
    return S, b, codes.reshape(-1)


def test_act_quantizer_decisions():
    rng = np.random.default_rng(3)
    rows = [rng.standard_normal(256).astype(np.float32) for _ in range(6)]
    r = rng.standard_normal(256).astype(np.float32)
    r[37] *= 50                                                     # outlier channel
    r[64:80] = 0                                                    # an all-zero block
    r[96:112] *= 1e-6                                               # a block whose scale underflows
    rows += [r, np.zeros(256, np.float32)]
    x = f32_to_bf16_bits(np.stack(rows))
    q, b, rs = oracle.fp4_quantize_act(x)
    xf = bf16_bits_to_f32(x)
    for i in range(x.shape[0]):
        S, bb, cc = rederive(xf[i])
        assert rs[i] == S
        np.testing.assert_array_equal(b[i], bb)
        np.testing.assert_array_equal(decode_codes(q[i], 256), cc)
    assert np.all(b[6, 4] == 0) and np.all(decode_codes(q[6], 256)[64:80] == 0)
    assert rs[7] == 0 and not q[7].any() and not b[7].any()


def test_quantizer_maxima_and_error_bound():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((3, 32, 128)).astype(np.float32) * np.float32(0.02)
    q, b, o = oracle.fp4_quantize_weights(w)
    for m in range(3):
        amax = np.abs(w[m]).max()
        assert o[m] == np.float32(amax) / np.float32(2688.0)
        r, k = np.unravel_index(np.argmax(np.abs(w[m])), w[m].shape)
        assert b[m, r, k // 16] == 0x7E                                  # 448
        assert abs(E2M1[decode_codes(q[m, r], 128)[k]]) == 6.0
        # each code is a nearest E2M1 value of its quotient (within the FP32 rounding of the quotient)
        den = (torch_e4m3_value(b[m]).astype(np.float32) * o[m]).astype(np.float32)
        quo = w[m].reshape(32, 8, 16) / den[..., None]
        got = E2M1[decode_codes(q[m], 128)].reshape(32, 8, 16)
        dist = np.abs(quo[..., None] - E2M1[None, None, None, :]).min(axis=-1)
        assert np.all(np.abs(quo - got) <= dist + 1e-6 * np.abs(quo) + 1e-12)


def test_exact_round_trip_of_representable_values():
    rng = np.random.default_rng(5)
    # outer scale 1 (the row's max is 6 * 448); block k's scale is E4M3 value
    # s_k and its max 6 s_k, so every element c * s_k must come back exactly
    scales = [448.0, 0.5, 1.125, 2.0 ** -9, 13.0, 96.0, 0.0, 1.75]
    row = []
    for s in scales:
        c = E2M1[rng.integers(0, 16, 16)]
        c[rng.integers(16)] = 6.0 if s else 0.0
        row.append(c * s)
    w = np.array([np.concatenate(row)], np.float32)
    q, b, o = oracle.fp4_quantize_weights(w[None])
    assert o[0] == 1.0
    np.testing.assert_array_equal(torch_e4m3_value(b[0, 0]), scales)
    np.testing.assert_array_equal(decode(q[0], b[0], 128)[0], w[0])
    np.testing.assert_array_equal(oracle.fp4_dequantize(q[0], b[0], o, 128, 1)[0], w[0])


def test_power_of_two_scaling_moves_only_the_outer_scale():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((2, 16, 64)).astype(np.float32)
    w[1] = w[0] * np.float32(2.0 ** -7)
    q, b, o = oracle.fp4_quantize_weights(w)
    np.testing.assert_array_equal(q[0], q[1])
    np.testing.assert_array_equal(b[0], b[1])
    assert o[1] == o[0] * np.float32(2.0 ** -7)


def test_nibble_order():
    w = np.zeros((1, 1, 16), np.float32)
    w[0, 0, :4] = [6.0 * 448, -0.5 * 448, 1.5 * 448, 0.0]             # outer 1, block scale 448
    q, b, o = oracle.fp4_quantize_weights(w)
    assert o[0] == 1.0 and b[0, 0, 0] == 0x7E
    assert q[0, 0, 0] == (0x7 | (0x9 << 4)) and q[0, 0, 1] == 0x3


# ---- the packed size against the printed checkpoint sizes ---------------------------

def test_nvfp4_size_reproduces_checkpoint_sizes():
    w = np.random.default_rng(7).standard_normal((4, 16, 1024)).astype(np.float32)
    q, b, o = oracle.fp4_quantize_weights(w)
    per_w = (q.nbytes + b.nbytes) / w.size                         # the FP32 per matrix is negligible
    assert per_w == 0.5 + 1 / 16
    g = {}
    with open(GOLDEN) as f:
        for line in f:
            t = line.split("#")[0].split()
            if t:
                g[(t[0], t[1])] = float(t[2])
    for model, tol in (("flash", 0.01), ("mini", 0.1)):
        bf, i8 = g[(model, "bf16")], g[(model, "int8")]
        n = (bf - i8) / (2.0 - (1 + 2 / 128))
        rest = bf - 2.0 * n
        assert abs(rest + per_w * n - g[(model, "nvfp4")]) <= tol


# ---- the feed-forward ------------------------------------------------------------------

def quantize_experts(ws):
    mats = [oracle.fp4_quantize_weights(np.stack([e[m] for e in ws])) for m in range(3)]
    return oracle.FP4Weights(*mats[0], *mats[1], *mats[2])


def test_forward_against_float64_on_decoded_operands():
    rng = np.random.default_rng(8)
    T, H, I, E, K = 7, 64, 48, 3, 2
    ws = [[(rng.standard_normal(sh) * 0.05).astype(np.float32) for sh in ((I, H), (I, H), (H, I))]
          for _ in range(E)]
    W = quantize_experts(ws)
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ids, tw = topk_softmax(rng.standard_normal((T, E)).astype(np.float32), K)
    o32, o16, nbad, ytok = oracle.fp4_moe_forward(x, ids, tw, W, E=E, return_y=True)
    assert nbad == 0
    xq, xb, xr = oracle.fp4_quantize_act(x)
    xd = torch.from_numpy(decode(xq, xb, H) * xr[:, None].astype(np.float64))
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            wg = torch.from_numpy(decode(W.gate_q[e], W.gate_b[e], H) * np.float64(W.gate_o[e]))
            wu = torch.from_numpy(decode(W.up_q[e], W.up_b[e], H) * np.float64(W.up_o[e]))
            wd = torch.from_numpy(decode(W.down_q[e], W.down_b[e], I) * np.float64(W.down_o[e]))
            g, u = xd[t] @ wg.T, xd[t] @ wu.T
            h = (F.silu(g) * u).numpy()
            h16 = np.array([oracle.bf16_bits(float(a)) for a in h], np.uint16)
            hq, hb, hr = oracle.fp4_quantize_act(h16[None])
            hd = torch.from_numpy(decode(hq, hb, I)[0] * np.float64(hr[0]))
            y = (hd @ wd.T).numpy()
            y16 = np.array([oracle.bf16_bits(float(a)) for a in y], np.uint16)
            np.testing.assert_array_equal(ytok[t, k], y16)
    # the combine of those y (k ascending, FP32)
    yf = bf16_bits_to_f32(ytok).astype(np.float64)
    ref = (tw[:, :, None].astype(np.float64) * yf).sum(axis=1)
    assert np.all(np.abs(o32 - ref) <= 1e-6 * np.abs(yf).sum(axis=1) + 1e-30)


def test_forward_all_zero_weights_and_dropped_slots():
    T, H, I, E, K = 4, 32, 32, 2, 2
    z = [[np.zeros(sh, np.float32) for sh in ((I, H), (I, H), (H, I))] for _ in range(E)]
    W = quantize_experts(z)
    assert not W.gate_o.any() and not W.gate_q.any() and not W.gate_b.any()
    x = f32_to_bf16_bits(np.random.default_rng(9).standard_normal((T, H)).astype(np.float32))
    ids = np.array([[0, 1], [1, -1], [5, 0], [1, 0]], np.int32)
    o32, o16, nbad = oracle.fp4_moe_forward(x, ids, np.full((T, K), 0.5, np.float32), W, E=E)
    assert nbad == 2 and not o32.any() and not o16.any()
