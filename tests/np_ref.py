"""Independent numpy statements of the format definitions the oracle's pins
use: INT4/INT8 code unpacking, exact dequantization, nearest-even rounding to
BF16 and the per-128 INT8 activation quantizer.  Written from the definitions
(signed two's-complement codes, element 2j in the low nibble; w = s * q;
round to 8 significant bits, ties to even; s = max|v| / 127 in FP32,
q = rint(v / s) in FP32), sharing nothing with the oracle's C code."""
import numpy as np

from harness.inputs import bf16_bits_to_f32


def np_codes(q, cols, bits):
    q = np.asarray(q, np.uint8)
    if bits == 8:
        return q.view(np.int8).astype(np.int64)
    lo = (q & 0xF).astype(np.int64)
    hi = (q >> 4).astype(np.int64)
    lo[lo >= 8] -= 16
    hi[hi >= 8] -= 16
    out = np.empty(q.shape[:-1] + (cols,), np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def np_scales(s):
    return np.asarray(s, np.uint16).view(np.float16).astype(np.float32)


def np_dequant(q, s, cols, bits):
    sc = np.asarray(s, np.uint16).view(np.float16).astype(np.float64)
    return np_codes(q, cols, bits) * np.repeat(sc, 128, axis=-1)


def np_round_bf16(v):
    """float64 -> the nearest BF16 value (ties to even), as float64."""
    v = np.asarray(v, np.float64)
    _, e = np.frexp(np.where(v == 0, 1.0, v))          # |v| in [2^(e-1), 2^e)
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)   # 8 significant bits; fixed below 2^-126
    return np.rint(v / quantum) * quantum


def np_bf16_bits(v):
    """BF16 bits of values that are already on the BF16 grid."""
    f = np.asarray(v, np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def np_quantize_act(vb):
    """bf16 bits [rows, cols] -> (codes int8 [rows, cols], scales fp32 [rows, cols/128])."""
    v = bf16_bits_to_f32(np.asarray(vb, np.uint16))
    rows, cols = v.shape
    g = v.reshape(rows, cols // 128, 128)
    m = np.abs(g).max(axis=2).astype(np.float32)
    s = (m / np.float32(127.0)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    quot = (g / safe[..., None]).astype(np.float32)
    q = np.clip(np.rint(quot), -127, 127)
    q[s == 0] = 0
    return q.reshape(rows, cols).astype(np.int8), s
