"""Pins of the oracle's two quantizers.

Weights: signed INT4/INT8, one FP16 scale per 128 weights along the input
dimension (model card "LLaDA2.2-flash for minnow", precision table).  The pins
are the round-trip bound |w - s*q| <= s/2 against the stored scale, the code
range, the group maximum landing on +-qmax, FP16 scale encoding against numpy,
hand-worked ties, and per-group (not per-row) scaling.

Activations: signed INT8 with an FP32 scale per 128 values (same model card,
paragraph on --int8-expert-activations).  Same kind of pins.
"""
import numpy as np
import pytest

import oracle
from harness.inputs import f32_to_bf16_bits, bf16_bits_to_f32
from np_ref import np_quantize_act


def _scale_values(s_bits):
    return np.asarray(s_bits, dtype=np.uint16).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("bits", [4, 8])
def test_weight_quantizer_bound_range_and_max(bits):
    qmax = 7 if bits == 4 else 127
    rng = np.random.default_rng(10 + bits)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    w[3, 128:256] *= 50.0          # groups of very different magnitude in one row
    w[5, 0:128] = 0.0              # all-zero group
    q, s = oracle.quantize_weights(w, bits)
    codes = oracle.unpack_codes(q, 512, bits).astype(np.int64)
    sv = np.repeat(_scale_values(s), 128, axis=1)
    # FP16 scale = nearest-even FP16 of the FP32 quotient max|w| / qmax
    m = np.abs(w).reshape(64, 4, 128).max(axis=2)
    np.testing.assert_array_equal(s, (m / np.float32(qmax)).astype(np.float32).astype(np.float16).view(np.uint16))
    # round-trip bound against what is stored
    err = np.abs(w.astype(np.float64) - sv * codes)
    assert np.all(err <= sv / 2)
    assert codes.min() >= -qmax and codes.max() <= qmax
    # the largest |w| of each group lands on +-qmax (nonzero groups)
    wg = w.reshape(64, 4, 128)
    cg = codes.reshape(64, 4, 128)
    idx = np.abs(wg).argmax(axis=2)
    top = np.take_along_axis(cg, idx[..., None], axis=2)[..., 0]
    nz = m > 0
    assert np.all(np.abs(top[nz]) == qmax)
    # zero group: scale 0 and codes 0
    assert s[5, 0] == 0 and np.all(codes[5, :128] == 0)
    # per-group scaling: the small groups of row 3 are not crushed by the big one
    assert np.abs(codes[3, :128]).max() == qmax and np.abs(codes[3, 256:]).max() == qmax


def test_weight_quantizer_ties_to_even():
    # group max 7 * 2^-4 gives the exact scale 2^-4; w / s lands exactly on .5
    w = np.zeros((1, 128), np.float32)
    vals = [2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 7.0, -6.5]
    w[0, :len(vals)] = np.array(vals) * 2.0 ** -4
    q, s = oracle.quantize_weights(w, 4)
    assert _scale_values(s)[0, 0] == 2.0 ** -4
    codes = oracle.unpack_codes(q, 128, 4)[0, :len(vals)]
    np.testing.assert_array_equal(codes, [2, 4, -2, 0, 2, 0, 7, -6])


def test_weight_dequantize_is_exact():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    for bits in (4, 8):
        q, s = oracle.quantize_weights(w, bits)
        codes = oracle.unpack_codes(q, 256, bits).astype(np.float64)
        ref = np.repeat(_scale_values(s), 128, axis=1) * codes     # exact in float64
        np.testing.assert_array_equal(oracle.dequantize(q, s, 256, bits).astype(np.float64), ref)


def test_weight_quantizer_rejects_bad_shape():
    with pytest.raises(ValueError):
        oracle.quantize_weights(np.zeros((2, 100), np.float32), 4)


def test_act_quantizer_bound_range_and_max():
    rng = np.random.default_rng(13)
    v = rng.standard_normal((16, 512)).astype(np.float32)
    v[2, 128:256] *= 20.0           # outlier group
    v[4, 256:384] = 0.0             # zero group
    vb = f32_to_bf16_bits(v)
    vf = bf16_bits_to_f32(vb).astype(np.float64)
    q, s = oracle.quantize_act(vb)
    q = q.astype(np.int64)
    sv = np.repeat(s.astype(np.float64), 128, axis=1)
    m = np.abs(vf).reshape(16, 4, 128).max(axis=2)
    # the FP32 scale is max/127 to within FP32 rounding of the quotient
    assert np.all(np.abs(s.astype(np.float64) * 127 - m) <= m * 2.0 ** -23)
    # v/s is rounded once in FP32 before rint: allow that one rounding
    assert np.all(np.abs(vf - sv * q) <= sv * (0.5 + 2.0 ** -16))
    assert q.min() >= -127 and q.max() <= 127
    idx = np.abs(vf).reshape(16, 4, 128).argmax(axis=2)
    top = np.take_along_axis(q.reshape(16, 4, 128), idx[..., None], axis=2)[..., 0]
    assert np.all(np.abs(top[m > 0]) == 127)
    assert s[4, 2] == 0 and np.all(q[4, 256:384] == 0)
    assert np.abs(q[2, :128]).max() == 127      # the outlier group does not crush row 2


def test_act_quantizer_ties_scaling_and_sign():
    v = np.zeros((1, 128), np.float32)
    vals = [127.0, 2.5, 3.5, -0.5, 126.5, -2.5, 1.5]   # scale = 127*2^-3 / 127 = 2^-3
    v[0, :len(vals)] = np.array(vals) * 2.0 ** -3
    vb = f32_to_bf16_bits(v)
    q, s = oracle.quantize_act(vb)
    assert s[0, 0] == 2.0 ** -3
    np.testing.assert_array_equal(q[0, :len(vals)], [127, 2, 4, 0, 126, -2, 2])
    # power-of-two scaling is exact: scale doubles, codes unchanged; negation flips codes
    rng = np.random.default_rng(14)
    x = f32_to_bf16_bits(rng.standard_normal((4, 256)).astype(np.float32))
    xf = bf16_bits_to_f32(x)
    q1, s1 = oracle.quantize_act(x)
    q2, s2 = oracle.quantize_act(f32_to_bf16_bits(xf * 2))
    q3, s3 = oracle.quantize_act(f32_to_bf16_bits(-xf))
    np.testing.assert_array_equal(q2, q1)
    np.testing.assert_array_equal(s2, s1 * 2)
    np.testing.assert_array_equal(q3, -q1)
    np.testing.assert_array_equal(s3, s1)



def test_act_quantizer_bit_exact_vs_numpy():
    """Bit-exact against the numpy statement above on scales that are not
    powers of two (the quotient v / s is then rounded to FP32 before rint, so a
    reciprocal-multiply or a double-precision quotient would differ), with
    outlier groups, zero groups, and tiny and huge magnitudes (ties at exact
    power-of-two scales are pinned above)."""
    rng = np.random.default_rng(15)
    v = rng.standard_normal((64, 1024)).astype(np.float32)
    v[:, rng.choice(1024, 10, replace=False)] *= 20.0
    v[7, 256:384] = 0.0
    v[9, :128] *= 1e-30
    v[11, 128:256] *= 1e30
    vb = f32_to_bf16_bits(v)
    q, s = oracle.quantize_act(vb)
    nq, ns = np_quantize_act(vb)
    np.testing.assert_array_equal(s.view(np.uint32), ns.view(np.uint32))
    np.testing.assert_array_equal(q, nq)
    m64 = np.abs(bf16_bits_to_f32(vb)).reshape(64, 8, 128).max(axis=2).astype(np.float64)
    assert np.mean(ns.astype(np.float64) * 127 != m64) > 0.5          # most scales are inexact quotients
    # a reciprocal multiply is a plausible mistake this pin must see: on these
    # inputs it gives different codes somewhere
    vf = bf16_bits_to_f32(vb).reshape(64, 8, 128)
    recip = (np.float32(1.0) / np.where(ns == 0, np.float32(1), ns)).astype(np.float32)
    alt = np.clip(np.rint((vf * recip[..., None]).astype(np.float32)), -127, 127).reshape(64, 1024)
    alt[np.repeat(ns == 0, 128, axis=1)] = 0
    assert np.any(alt.astype(np.int8) != nq)
