"""Pins of the oracle's number formats and of the packed weight format.

The BF16/FP16 rounding helpers are checked against library conversions (torch's
float32->bfloat16 and numpy's float32->float16, both round-to-nearest-even) and
against hand-worked ties; the packed weight format is checked against the
checkpoint sizes the pages print.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "checkpoint_sizes.txt")


def _torch_bf16_bits(v32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_library_on_float32():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(3.0),
        rng.standard_normal(500).astype(np.float32) * np.float32(1e-39),   # subnormal range
        np.array([3.3895e38, 3.3896e38, 3.40e38, -3.40e38, 1e-45, -1e-45, 0.0, -0.0], np.float32),
        # exact ties of bf16 (the 16 dropped bits are exactly 0x8000)
        (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    ours = np.array([oracle.bf16_bits(float(a)) for a in v], dtype=np.uint16)
    np.testing.assert_array_equal(ours, _torch_bf16_bits(v))


def test_bf16_rounding_hand_ties_and_no_double_rounding():
    one = 1.0
    assert oracle.round_bf16(one + 2.0 ** -8) == 1.0                 # tie -> even (down)
    assert oracle.round_bf16(one + 3 * 2.0 ** -8) == one + 2.0 ** -6  # tie -> even (up)
    # just above a tie: a float32 intermediate would drop 2^-40 and round down
    assert oracle.round_bf16(one + 2.0 ** -8 + 2.0 ** -40) == one + 2.0 ** -7
    assert oracle.round_bf16(-(one + 2.0 ** -8 + 2.0 ** -40)) == -(one + 2.0 ** -7)
    assert np.isinf(oracle.round_bf16(3.5e38))


def test_fp16_rounding_matches_library():
    rng = np.random.default_rng(2)
    v = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(0.01),
        rng.uniform(0, 7e-5, 500).astype(np.float32),                     # subnormal fp16
        np.array([65504.0, 65519.0, 65520.0, 70000.0, 6.1035156e-05, 5.96e-8, 2.98e-8,
                  2.99e-8], np.float32),
        (np.arange(1, 300, dtype=np.uint32) << 13 | 0x1000 | 0x3C000000).view(np.float32),  # ties
    ])
    ours = np.array([oracle.fp16_bits(float(a)) for a in v], dtype=np.uint16)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_fp16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    ours = np.array([oracle.fp16_value(int(b)) for b in bits])
    finite = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[finite], ref[finite])
    assert np.all(np.isnan(ours[~finite]))


def _bytes_per_weight(bits: int) -> float:
    """Bytes per routed-expert weight of the oracle's packed format, measured on
    what the quantizer actually writes (codes + FP16 scales)."""
    w = np.random.default_rng(3).standard_normal((16, 1024)).astype(np.float32)
    q, s = oracle.quantize_weights(w, bits)
    return (q.nbytes + s.nbytes) / w.size


def _golden():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                rows[(line[0], line[1])] = float(line[2])
    return rows


def test_packed_format_reproduces_checkpoint_sizes():
    """Only the routed experts change between checkpoints, so with B bytes per
    weight: size = rest + n_expert_weights * B.  BF16 (2 B) and INT8 pin the two
    unknowns; the INT4 size is then a prediction of the INT4 format."""
    g = _golden()
    b8, b4 = _bytes_per_weight(8), _bytes_per_weight(4)
    assert b8 == 1 + 2 / 128 and b4 == 0.5 + 2 / 128
    for model, tol in (("flash", 0.01), ("mini", 0.15)):
        bf, i8, i4 = g[(model, "bf16")], g[(model, "int8")], g[(model, "int4")]
        n = (bf - i8) / (2.0 - b8)          # GiB per byte-per-weight
        rest = bf - 2.0 * n
        pred4 = rest + b4 * n
        assert abs(pred4 - i4) <= tol, (model, pred4, i4)
    # a zero-point per group (4.25 / 8.25 bits) would miss the printed flash size
    bf, i8, i4 = g[("flash", "bf16")], g[("flash", "int8")], g[("flash", "int4")]
    n = (bf - i8) / (2.0 - (1 + 4 / 128))
    assert abs(bf - 2.0 * n + (0.5 + 4 / 128) * n - i4) > 0.5


@pytest.mark.parametrize("bits", [4, 8])
def test_packing_round_trip_all_byte_patterns(bits):
    # the quantizer's own range is symmetric (-qmax..qmax); the extra INT4 code
    # -8 is decoded below from hand-packed bytes
    qmax = 7 if bits == 4 else 127
    codes = np.arange(-qmax, qmax + 1)
    # rows of 128: a group holding every code, scale forced to 2^-4 by the max
    n = 128
    rows = []
    rng = np.random.default_rng(4)
    for _ in range(40):
        c = rng.choice(codes, n)
        c[rng.integers(n)] = qmax
        rows.append(c)
    c = np.array(rows)
    w = (c * 2.0 ** -4).astype(np.float32)
    q, s = oracle.quantize_weights(w, bits)
    assert np.all(s == np.float16(2.0 ** -4).view(np.uint16))
    np.testing.assert_array_equal(oracle.unpack_codes(q, n, bits), c)
    if bits == 4:
        # element 2j -> low nibble, 2j+1 -> high nibble, two's complement
        lo = c[:, 0::2] & 0xF
        hi = c[:, 1::2] & 0xF
        np.testing.assert_array_equal(q, (lo | (hi << 4)).astype(np.uint8))
        w2 = np.zeros((1, 128), np.float32)
        w2[0, :4] = np.array([1, -1, -7, 7]) * 2.0 ** -4
        w2[0, 5] = 7 * 2.0 ** -4
        q2, _ = oracle.quantize_weights(w2, 4)
        assert q2[0, 0] == 0xF1 and q2[0, 1] == 0x79
        hand = {0x00: (0, 0), 0xF1: (1, -1), 0x78: (-8, 7), 0x87: (7, -8), 0xFF: (-1, -1),
                0x9A: (-6, -7), 0x80: (0, -8)}
        b = np.array([list(hand)], dtype=np.uint8)
        np.testing.assert_array_equal(oracle.unpack_codes(b, 2 * b.shape[1], 4)[0],
                                      np.array([v for k in hand for v in hand[k]]))
    else:
        np.testing.assert_array_equal(q.view(np.int8), c)
        b = np.array([[0x80, 0x7F, 0xFF, 0x01]], dtype=np.uint8)
        np.testing.assert_array_equal(oracle.unpack_codes(b, 4, 8)[0], [-128, 127, -1, 1])
