"""CPU oracle for the quantized routed-expert MoE feed-forward (test infrastructure).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The GPU library never uses it.  All arithmetic
lives in ``qre_oracle.c``; this module only marshals numpy arrays through
ctypes.  Every function cites, in the C source, the passage of the pages it
follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qre_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
GROUP = 128

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fopenmp", "-Wall"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, no intrinsics, no BLAS)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = C.CDLL(_LIB)
        P = C.c_void_p
        i64, i32 = C.c_int64, C.c_int32
        L.orc_round_bf16.restype = C.c_double
        L.orc_round_bf16.argtypes = [C.c_double]
        L.orc_round_fp16.restype = C.c_double
        L.orc_round_fp16.argtypes = [C.c_double]
        L.orc_bf16_from_double.restype = C.c_uint16
        L.orc_bf16_from_double.argtypes = [C.c_double]
        L.orc_fp16_from_double.restype = C.c_uint16
        L.orc_fp16_from_double.argtypes = [C.c_double]
        L.orc_fp16_to_double.restype = C.c_double
        L.orc_fp16_to_double.argtypes = [C.c_uint16]
        L.orc_quantize_weights.restype = C.c_int
        L.orc_quantize_weights.argtypes = [P, i64, i64, C.c_int, P, P]
        L.orc_unpack_codes.argtypes = [P, i64, i64, C.c_int, P]
        L.orc_dequantize.argtypes = [P, P, i64, i64, C.c_int, P]
        L.orc_topk_softmax.restype = C.c_int
        L.orc_topk_softmax.argtypes = [P, i32, i32, i32, P, P]
        L.orc_quantize_act.restype = C.c_int
        L.orc_quantize_act.argtypes = [P, i64, i64, P, P]
        L.orc_route.restype = C.c_int
        L.orc_route.argtypes = [P, i32, i32, i32, P, P, P, P]
        L.orc_gate_up.restype = C.c_int
        L.orc_gate_up.argtypes = [P, P, P, P, P, P, P, P, P]
        L.orc_down.restype = C.c_int
        L.orc_down.argtypes = [P, P, P, P, P, P, P, P]
        L.orc_combine.argtypes = [P, P, P, i32, i32, i32, P, i64, P, P]
        L.orc_moe_forward.restype = C.c_int
        L.orc_moe_forward.argtypes = [P, P, P, P, P, P, i64, P, P, P]
        L.orc_num_threads.restype = C.c_int
        L.orc_set_num_threads.argtypes = [C.c_int]
        L.orc_e2m1_value.restype = C.c_double
        L.orc_e2m1_value.argtypes = [C.c_int]
        L.orc_e4m3_value.restype = C.c_double
        L.orc_e4m3_value.argtypes = [C.c_uint8]
        L.orc_e4m3_encode.restype = C.c_uint8
        L.orc_e4m3_encode.argtypes = [C.c_double]
        L.orc_e2m1_encode.restype = C.c_int
        L.orc_e2m1_encode.argtypes = [C.c_double]
        L.orc_fp4_quantize_weights.restype = C.c_int
        L.orc_fp4_quantize_weights.argtypes = [P, i64, i64, i64, P, P, P]
        L.orc_fp4_quantize_act.restype = C.c_int
        L.orc_fp4_quantize_act.argtypes = [P, i64, i64, P, P, P]
        L.orc_fp4_dequantize.argtypes = [P, P, P, i64, i64, i64, P]
        L.orc_fp4_gate_up.restype = C.c_int
        L.orc_fp4_gate_up.argtypes = [P, P, P, P, P, P, P, P, P]
        L.orc_fp4_down.restype = C.c_int
        L.orc_fp4_down.argtypes = [P, P, P, P, P, P, P, P]
        L.orc_fp4_moe_forward.restype = C.c_int
        L.orc_fp4_moe_forward.argtypes = [P, P, P, P, P, P, i64, P, P, P]
        _lib = L
    return _lib


class _Shape(C.Structure):
    _fields_ = [("T", C.c_int32), ("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32),
                ("K", C.c_int32), ("bits", C.c_int32), ("act_int8", C.c_int32)]


class _Weights(C.Structure):
    _fields_ = [("gate_q", C.c_void_p), ("gate_s", C.c_void_p), ("up_q", C.c_void_p),
                ("up_s", C.c_void_p), ("down_q", C.c_void_p), ("down_s", C.c_void_p)]


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on."""
    lib().orc_set_num_threads(int(n))


# ---- number formats --------------------------------------------------------

def round_bf16(v: float) -> float:
    return lib().orc_round_bf16(float(v))


def round_fp16(v: float) -> float:
    return lib().orc_round_fp16(float(v))


def bf16_bits(v: float) -> int:
    return lib().orc_bf16_from_double(float(v))


def fp16_bits(v: float) -> int:
    return lib().orc_fp16_from_double(float(v))


def fp16_value(bits: int) -> float:
    return lib().orc_fp16_to_double(int(bits))


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- weight format -----------------------------------------------------------

def packed_cols(cols: int, bits: int) -> int:
    return cols // 2 if bits == 4 else cols


def quantize_weights(w: np.ndarray, bits: int):
    """w float32 [..., rows, cols] -> (q uint8 [..., rows, packed], s uint16 fp16 bits [..., rows, cols/128])."""
    w = _c(w, np.float32)
    lead, (rows, cols) = w.shape[:-2], w.shape[-2:]
    R = int(np.prod(lead, dtype=np.int64)) * rows
    q = np.zeros(lead + (rows, packed_cols(cols, bits)), dtype=np.uint8)
    s = np.zeros(lead + (rows, cols // GROUP), dtype=np.uint16)
    rc = lib().orc_quantize_weights(_p(w), R, cols, bits, _p(q), _p(s))
    if rc != 0:
        raise ValueError(f"orc_quantize_weights: {rc}")
    return q, s


def unpack_codes(q: np.ndarray, cols: int, bits: int) -> np.ndarray:
    q = _c(q, np.uint8)
    rows = int(np.prod(q.shape[:-1], dtype=np.int64))
    out = np.zeros(q.shape[:-1] + (cols,), dtype=np.int8)
    lib().orc_unpack_codes(_p(q), rows, cols, bits, _p(out))
    return out


def dequantize(q: np.ndarray, s: np.ndarray, cols: int, bits: int) -> np.ndarray:
    q, s = _c(q, np.uint8), _c(s, np.uint16)
    rows = int(np.prod(q.shape[:-1], dtype=np.int64))
    out = np.zeros(q.shape[:-1] + (cols,), dtype=np.float32)
    lib().orc_dequantize(_p(q), _p(s), rows, cols, bits, _p(out))
    return out


# ---- activation quantizer ----------------------------------------------------

def quantize_act(v_bf16: np.ndarray):
    """v bf16 bits [rows, cols] -> (q int8 [rows, cols], s float32 [rows, cols/128])."""
    v = _c(v_bf16, np.uint16)
    rows, cols = v.shape
    q = np.zeros((rows, cols), dtype=np.int8)
    s = np.zeros((rows, cols // GROUP), dtype=np.float32)
    rc = lib().orc_quantize_act(_p(v), rows, cols, _p(q), _p(s))
    if rc != 0:
        raise ValueError(f"orc_quantize_act: {rc}")
    return q, s


# ---- routing -------------------------------------------------------------------

def route(topk_ids: np.ndarray, E: int):
    ids = _c(topk_ids, np.int32)
    T, K = ids.shape
    S = T * K
    counts = np.zeros(E, dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    sorted_slot = np.zeros(S, dtype=np.int32)
    slot_row = np.zeros(S, dtype=np.int32)
    nbad = lib().orc_route(_p(ids), T, K, E, _p(counts), _p(offsets), _p(sorted_slot), _p(slot_row))
    return counts, offsets, sorted_slot, slot_row, nbad


def topk_softmax(logits: np.ndarray, K: int):
    """logits float32 [T, E] -> (ids int32 [T, K], w float32 [T, K]): the K
    largest logits per token in descending order, ties to the lower id, and a
    softmax over them (double inside, one rounding to float32)."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.zeros((T, K), dtype=np.int32)
    w = np.zeros((T, K), dtype=np.float32)
    rc = lib().orc_topk_softmax(_p(lg), T, E, K, _p(ids), _p(w))
    if rc != 0:
        raise ValueError(f"orc_topk_softmax: {rc}")
    return ids, w


# ---- expert feed-forward -------------------------------------------------------

class QWeights:
    """Packed weights of all experts: gate/up [E][I][H*bits/8] + fp16 scales
    [E][I][H/128]; down [E][H][I*bits/8] + [E][H][I/128]."""

    def __init__(self, gate_q, gate_s, up_q, up_s, down_q, down_s):
        self.gate_q, self.gate_s = _c(gate_q, np.uint8), _c(gate_s, np.uint16)
        self.up_q, self.up_s = _c(up_q, np.uint8), _c(up_s, np.uint16)
        self.down_q, self.down_s = _c(down_q, np.uint8), _c(down_s, np.uint16)

    def _struct(self):
        return _Weights(_p(self.gate_q), _p(self.gate_s), _p(self.up_q), _p(self.up_s),
                        _p(self.down_q), _p(self.down_s))


def _shape(T, H, I, E, K, bits, act_int8):
    return _Shape(T, H, I, E, K, bits, int(bool(act_int8)))


def gate_up(x_bf16, sorted_slot, offsets, W: QWeights, *, T, H, I, E, K, bits, act_int8=False,
            xq=None, xs=None, row_mask=None):
    """h bf16 bits [S, I] by sorted row (rows of experts not needed stay zero)."""
    S = T * K
    h = np.zeros((S, I), dtype=np.uint16)
    d = _shape(T, H, I, E, K, bits, act_int8)
    x = None if x_bf16 is None else _c(x_bf16, np.uint16)
    xq = None if xq is None else _c(xq, np.int8)
    xs = None if xs is None else _c(xs, np.float32)
    m = None if row_mask is None else _c(row_mask, np.uint8)
    rc = lib().orc_gate_up(C.byref(d), _p(x), _p(xq), _p(xs), _p(_c(sorted_slot, np.int32)),
                           _p(_c(offsets, np.int32)), C.byref(W._struct()), _p(m), _p(h))
    if rc != 0:
        raise ValueError(f"orc_gate_up: {rc}")
    return h


def down(h_bf16, offsets, W: QWeights, *, T, H, I, E, K, bits, act_int8=False, hq=None, hs=None,
         row_mask=None):
    """y bf16 bits [S, H] by sorted row."""
    S = T * K
    y = np.zeros((S, H), dtype=np.uint16)
    d = _shape(T, H, I, E, K, bits, act_int8)
    h = None if h_bf16 is None else _c(h_bf16, np.uint16)
    hq = None if hq is None else _c(hq, np.int8)
    hs = None if hs is None else _c(hs, np.float32)
    m = None if row_mask is None else _c(row_mask, np.uint8)
    rc = lib().orc_down(C.byref(d), _p(h), _p(hq), _p(hs), _p(_c(offsets, np.int32)),
                        C.byref(W._struct()), _p(m), _p(y))
    if rc != 0:
        raise ValueError(f"orc_down: {rc}")
    return y


def combine(y_bf16, slot_row, topk_w, *, T, K, H, tokens=None):
    """(out float32 before rounding, out bf16 bits), rows = tokens (or all T)."""
    y = _c(y_bf16, np.uint16)
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else len(tok)
    o32 = np.zeros((n, H), dtype=np.float32)
    o16 = np.zeros((n, H), dtype=np.uint16)
    lib().orc_combine(_p(y), _p(_c(slot_row, np.int32)), _p(_c(topk_w, np.float32)), T, K, H,
                      _p(tok), 0 if tok is None else len(tok), _p(o32), _p(o16))
    return o32, o16


def moe_forward(x_bf16, topk_ids, topk_w, W: QWeights, *, E, bits, act_int8=False, I=None,
                tokens=None, return_y=False):
    """Whole feed-forward. Returns (out float32 before final rounding, out bf16
    bits, number of dropped slots); rows follow `tokens` when given.  With
    return_y, a fourth item: the BF16 expert outputs each row combines,
    [n, K, H] bits in slot order (zeros for a dropped slot)."""
    x = _c(x_bf16, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, H = x.shape
    K = ids.shape[1]
    if I is None:
        I = W.gate_s.shape[-2]
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else len(tok)
    o32 = np.zeros((n, H), dtype=np.float32)
    o16 = np.zeros((n, H), dtype=np.uint16)
    d = _shape(T, H, I, E, K, bits, act_int8)
    y = np.zeros((n, K, H), dtype=np.uint16) if return_y else None
    rc = lib().orc_moe_forward(C.byref(d), _p(x), _p(ids), _p(_c(topk_w, np.float32)),
                               C.byref(W._struct()), _p(tok), 0 if tok is None else len(tok),
                               _p(o32), _p(o16), _p(y))
    if rc < 0:
        raise ValueError(f"orc_moe_forward: {rc}")
    return (o32, o16, rc, y) if return_y else (o32, o16, rc)


# ---- workload weights ------------------------------------------------------------

def workload_experts(wl, experts, threads=None) -> QWeights:
    """Oracle-quantized weights of the listed experts of a seeded workload
    (the float32 weights come from the shared input generators); the other
    experts are left zero."""
    from concurrent.futures import ThreadPoolExecutor
    from harness.inputs import GATE, UP, DOWN, default_threads, gen_expert_weight
    b = wl.weight_bits
    gq = np.zeros((wl.E, wl.I, packed_cols(wl.H, b)), np.uint8)
    gs = np.zeros((wl.E, wl.I, wl.H // GROUP), np.uint16)
    uq, us = np.zeros_like(gq), np.zeros_like(gs)
    dq = np.zeros((wl.E, wl.H, packed_cols(wl.I, b)), np.uint8)
    ds = np.zeros((wl.E, wl.H, wl.I // GROUP), np.uint16)

    def one(e):
        for m, (q, s) in ((GATE, (gq, gs)), (UP, (uq, us)), (DOWN, (dq, ds))):
            q[e], s[e] = quantize_weights(gen_expert_weight(wl, e, m), b)

    with ThreadPoolExecutor(threads or default_threads()) as ex:
        list(ex.map(one, [int(e) for e in experts]))
    return QWeights(gq, gs, uq, us, dq, ds)


# ---- NVFP4 (W4A4) ------------------------------------------------------------------

FP4_BLOCK = 16


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e4m3_value(b: int) -> float:
    return lib().orc_e4m3_value(int(b))


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def e2m1_encode(v: float) -> int:
    return lib().orc_e2m1_encode(float(v))


def fp4_quantize_weights(w: np.ndarray):
    """w float32 [..., rows, cols] -> (q uint8 [..., rows, cols/2], b uint8 E4M3
    [..., rows, cols/16], outer float32 [...]): one outer scale per matrix."""
    w = _c(w, np.float32)
    lead, (rows, cols) = w.shape[:-2], w.shape[-2:]
    mats = int(np.prod(lead, dtype=np.int64))
    q = np.zeros(lead + (rows, cols // 2), dtype=np.uint8)
    b = np.zeros(lead + (rows, cols // FP4_BLOCK), dtype=np.uint8)
    o = np.zeros(lead, dtype=np.float32)
    rc = lib().orc_fp4_quantize_weights(_p(w), mats, rows, cols, _p(q), _p(b), _p(o))
    if rc != 0:
        raise ValueError(f"orc_fp4_quantize_weights: {rc}")
    return q, b, o


def fp4_quantize_act(v_bf16: np.ndarray):
    """v bf16 bits [rows, cols] -> (q uint8 [rows, cols/2], b uint8 [rows, cols/16],
    row_scale float32 [rows])."""
    v = _c(v_bf16, np.uint16)
    rows, cols = v.shape
    q = np.zeros((rows, cols // 2), dtype=np.uint8)
    b = np.zeros((rows, cols // FP4_BLOCK), dtype=np.uint8)
    r = np.zeros(rows, dtype=np.float32)
    rc = lib().orc_fp4_quantize_act(_p(v), rows, cols, _p(q), _p(b), _p(r))
    if rc != 0:
        raise ValueError(f"orc_fp4_quantize_act: {rc}")
    return q, b, r


def fp4_dequantize(q, b, scale, cols: int, rows_per_scale: int) -> np.ndarray:
    """float64 [rows, cols] = E2M1 * E4M3 * scale[row // rows_per_scale]."""
    q, b, sc = _c(q, np.uint8), _c(b, np.uint8), _c(scale, np.float32)
    rows = int(np.prod(q.shape[:-1], dtype=np.int64))
    out = np.zeros((rows, cols), dtype=np.float64)
    lib().orc_fp4_dequantize(_p(q), _p(b), _p(sc), rows, cols, int(rows_per_scale), _p(out))
    return out


class _FP4Mat(C.Structure):
    _fields_ = [("q", C.c_void_p), ("b", C.c_void_p), ("o", C.c_void_p)]


class _FP4Weights(C.Structure):
    _fields_ = [("gate", _FP4Mat), ("up", _FP4Mat), ("down", _FP4Mat)]


class FP4Weights:
    """NVFP4 weights of all experts: codes gate/up [E][I][H/2], down [E][H][I/2];
    E4M3 block scales [E][rows][cols/16]; FP32 outer scales [E] per matrix."""

    def __init__(self, gate_q, gate_b, gate_o, up_q, up_b, up_o, down_q, down_b, down_o):
        self.gate_q, self.gate_b, self.gate_o = _c(gate_q, np.uint8), _c(gate_b, np.uint8), _c(gate_o, np.float32)
        self.up_q, self.up_b, self.up_o = _c(up_q, np.uint8), _c(up_b, np.uint8), _c(up_o, np.float32)
        self.down_q, self.down_b, self.down_o = _c(down_q, np.uint8), _c(down_b, np.uint8), _c(down_o, np.float32)

    def _struct(self):
        m = lambda q, b, o: _FP4Mat(_p(q), _p(b), _p(o))
        return _FP4Weights(m(self.gate_q, self.gate_b, self.gate_o), m(self.up_q, self.up_b, self.up_o),
                           m(self.down_q, self.down_b, self.down_o))


def fp4_gate_up(xq, xb, xr, sorted_slot, offsets, W: FP4Weights, *, T, H, I, E, K, row_mask=None):
    """h bf16 bits [S, I] by sorted row, from NVFP4-quantized x."""
    h = np.zeros((T * K, I), dtype=np.uint16)
    d = _shape(T, H, I, E, K, 4, False)
    m = None if row_mask is None else _c(row_mask, np.uint8)
    rc = lib().orc_fp4_gate_up(C.byref(d), _p(_c(xq, np.uint8)), _p(_c(xb, np.uint8)), _p(_c(xr, np.float32)),
                               _p(_c(sorted_slot, np.int32)), _p(_c(offsets, np.int32)), C.byref(W._struct()),
                               _p(m), _p(h))
    if rc != 0:
        raise ValueError(f"orc_fp4_gate_up: {rc}")
    return h


def fp4_down(hq, hb, hr, offsets, W: FP4Weights, *, T, H, I, E, K, row_mask=None):
    """y bf16 bits [S, H] by sorted row, from NVFP4-quantized h."""
    y = np.zeros((T * K, H), dtype=np.uint16)
    d = _shape(T, H, I, E, K, 4, False)
    m = None if row_mask is None else _c(row_mask, np.uint8)
    rc = lib().orc_fp4_down(C.byref(d), _p(_c(hq, np.uint8)), _p(_c(hb, np.uint8)), _p(_c(hr, np.float32)),
                            _p(_c(offsets, np.int32)), C.byref(W._struct()), _p(m), _p(y))
    if rc != 0:
        raise ValueError(f"orc_fp4_down: {rc}")
    return y


def fp4_moe_forward(x_bf16, topk_ids, topk_w, W: FP4Weights, *, E, I=None, tokens=None, return_y=False):
    """Whole NVFP4 feed-forward; same returns as moe_forward."""
    x = _c(x_bf16, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, H = x.shape
    K = ids.shape[1]
    if I is None:
        I = W.gate_b.shape[-2]
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else len(tok)
    o32 = np.zeros((n, H), dtype=np.float32)
    o16 = np.zeros((n, H), dtype=np.uint16)
    d = _shape(T, H, I, E, K, 4, False)
    y = np.zeros((n, K, H), dtype=np.uint16) if return_y else None
    rc = lib().orc_fp4_moe_forward(C.byref(d), _p(x), _p(ids), _p(_c(topk_w, np.float32)), C.byref(W._struct()),
                                   _p(tok), 0 if tok is None else len(tok), _p(o32), _p(o16), _p(y))
    if rc < 0:
        raise ValueError(f"orc_fp4_moe_forward: {rc}")
    return (o32, o16, rc, y) if return_y else (o32, o16, rc)


def fp4_workload_experts(wl, experts, threads=None) -> FP4Weights:
    """Oracle-quantized NVFP4 weights of the listed experts of a seeded
    workload (float32 weights from the shared input generators); the other
    experts are left zero."""
    from concurrent.futures import ThreadPoolExecutor
    from harness.inputs import GATE, UP, DOWN, default_threads, gen_expert_weight
    E, H, I = wl.E, wl.H, wl.I
    arrs = {}
    for m, (rows, cols) in ((GATE, (I, H)), (UP, (I, H)), (DOWN, (H, I))):
        arrs[m] = (np.zeros((E, rows, cols // 2), np.uint8), np.zeros((E, rows, cols // FP4_BLOCK), np.uint8),
                   np.zeros(E, np.float32))

    def one(e):
        for m, (q, b, o) in arrs.items():
            q[e], b[e], o[e] = fp4_quantize_weights(gen_expert_weight(wl, e, m))

    with ThreadPoolExecutor(threads or default_threads()) as ex:
        list(ex.map(one, [int(e) for e in experts]))
    return FP4Weights(*arrs[GATE], *arrs[UP], *arrs[DOWN])
