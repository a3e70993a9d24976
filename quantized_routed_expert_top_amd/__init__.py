"""Python binding of libqre.so, the MI355X (gfx950) routed-expert MoE
feed-forward with group-quantized expert weights.

Argument marshalling only: every function checks dtypes, devices, shapes and
contiguity of torch tensors, then calls the C entry point of the same name in
``libqre.so`` (declared in ``include/qre.h``) on the current torch stream.  Every
step of the computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and importing this module fails if the library is missing.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqre.so")
GROUP = 128

QRE_OK = 0
_STATUS = {0: "ok", -1: "null pointer", -2: "bad shape", -3: "bad weight_bits", -4: "bad group_size",
           -5: "misaligned pointer", -6: "workspace too small", -7: "HIP error", -8: "bad mode",
           -9: "size limit"}


class QreError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        extra = ""
        if status == -7:
            extra = f" (hipError {_lib().qre_last_hip_error()})"
        super().__init__(f"{fn}: {_lib().qre_status_string(status).decode()} [{status}]{extra}")


class _Desc(C.Structure):
    _fields_ = [("T", C.c_int32), ("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32), ("K", C.c_int32),
                ("weight_bits", C.c_int32), ("group_size", C.c_int32), ("act_int8", C.c_int32)]


class _Weights(C.Structure):
    _fields_ = [("gate_q", C.c_void_p), ("gate_s", C.c_void_p), ("up_q", C.c_void_p), ("up_s", C.c_void_p),
                ("down_q", C.c_void_p), ("down_s", C.c_void_p)]


_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m quantized_routed_expert_top_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.qre_status_string.restype = C.c_char_p
        L.qre_status_string.argtypes = [C.c_int]
        L.qre_last_hip_error.restype = C.c_int
        L.qre_workspace_bytes.argtypes = [P, P]
        L.qre_stage_workspace_bytes.argtypes = [P, P]
        L.qre_moe_forward.argtypes = [P, P, P, P, P, P, P, sz, P]
        L.qre_moe_forward_timed.argtypes = [P, P, P, P, P, P, P, sz, P, P]
        L.qre_read_device_error.argtypes = [P, P, P]
        L.qre_workspace_permutation.argtypes = [P, P, P, P, P, P]
        L.qre_route_workspace_bytes.argtypes = [i32, i32, i32, P]
        L.qre_route.argtypes = [P, i32, i32, i32, P, P, P, P, P, sz, P]
        L.qre_quantize_act.argtypes = [P, i32, i32, P, P, P]
        L.qre_gate_up.argtypes = [P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.qre_down.argtypes = [P, P, P, P, P, P, P, P, sz, P]
        L.qre_combine.argtypes = [P, P, P, i32, i32, i32, P, P]
        L.qre_topk_softmax.argtypes = [P, i32, i32, i32, P, P, P]
        L.qre_quantize_weights.argtypes = [P, i64, i64, i32, P, P, P]
        L.qre_hbm_read_probe.argtypes = [P, sz, P, P]
        L.qre_forward_plan.argtypes = [P, P]
        L.qre_moe_forward_noalloc.argtypes = [P, P, P, P, P, P, P]
        L.qre_nvfp4_quantize_weights.argtypes = [P, i64, i64, i64, P, P, P, P]
        L.qre_nvfp4_quantize_act.argtypes = [P, i32, i32, P, P, P, P]
        L.qre_nvfp4_workspace_bytes.argtypes = [P, P]
        L.qre_nvfp4_stage_workspace_bytes.argtypes = [P, P]
        L.qre_nvfp4_moe_forward.argtypes = [P, P, P, P, P, P, P, sz, P]
        L.qre_nvfp4_moe_forward_timed.argtypes = [P, P, P, P, P, P, P, sz, P, P]
        L.qre_nvfp4_workspace_permutation.argtypes = [P, P, P, P, P, P]
        L.qre_nvfp4_gate_up.argtypes = [P, P, P, P, P, P, P, P, P, sz, P]
        L.qre_nvfp4_down.argtypes = [P, P, P, P, P, P, P, P, sz, P]
        _L = L
    return _L


def library_path() -> str:
    return LIB_PATH


def status_string(status: int) -> str:
    return _lib().qre_status_string(status).decode()


def _check(fn: str, status: int):
    if status != QRE_OK:
        raise QreError(fn, status)


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def packed_cols(cols: int, bits: int) -> int:
    return cols // 2 if bits == 4 else cols


@dataclass
class QuantizedExperts:
    """Packed routed-expert weights on the GPU (layouts of include/qre.h)."""
    gate_q: torch.Tensor   # uint8 [E, I, H*bits/8]
    gate_s: torch.Tensor   # float16 [E, I, H/128]
    up_q: torch.Tensor
    up_s: torch.Tensor
    down_q: torch.Tensor   # uint8 [E, H, I*bits/8]
    down_s: torch.Tensor   # float16 [E, H, I/128]
    bits: int

    @property
    def E(self):
        return self.gate_q.shape[0]

    @property
    def I(self):
        return self.gate_q.shape[1]

    @property
    def H(self):
        return self.down_q.shape[1]

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.gate_q, self.gate_s, self.up_q, self.up_s, self.down_q, self.down_s))

    def expert_nbytes(self) -> int:
        return self.nbytes() // self.E

    def _struct(self):
        E, H, I, b = self.E, self.H, self.I, self.bits
        _need(self.gate_q, "gate_q", torch.uint8, (E, I, packed_cols(H, b)))
        _need(self.up_q, "up_q", torch.uint8, (E, I, packed_cols(H, b)))
        _need(self.down_q, "down_q", torch.uint8, (E, H, packed_cols(I, b)))
        _need(self.gate_s, "gate_s", torch.float16, (E, I, H // GROUP))
        _need(self.up_s, "up_s", torch.float16, (E, I, H // GROUP))
        _need(self.down_s, "down_s", torch.float16, (E, H, I // GROUP))
        return _Weights(self.gate_q.data_ptr(), self.gate_s.data_ptr(), self.up_q.data_ptr(),
                        self.up_s.data_ptr(), self.down_q.data_ptr(), self.down_s.data_ptr())

    def clone(self) -> "QuantizedExperts":
        return QuantizedExperts(*(t.clone() for t in (self.gate_q, self.gate_s, self.up_q, self.up_s,
                                                      self.down_q, self.down_s)), self.bits)

    @staticmethod
    def empty(E, H, I, bits, device="cuda"):
        u8, f16 = torch.uint8, torch.float16
        return QuantizedExperts(
            torch.empty((E, I, packed_cols(H, bits)), dtype=u8, device=device),
            torch.empty((E, I, H // GROUP), dtype=f16, device=device),
            torch.empty((E, I, packed_cols(H, bits)), dtype=u8, device=device),
            torch.empty((E, I, H // GROUP), dtype=f16, device=device),
            torch.empty((E, H, packed_cols(I, bits)), dtype=u8, device=device),
            torch.empty((E, H, I // GROUP), dtype=f16, device=device), bits)


def _desc(T, H, I, E, K, bits, act_int8):
    return _Desc(T, H, I, E, K, bits, GROUP, int(bool(act_int8)))


def workspace_bytes(T, H, I, E, K, bits, act_int8=False) -> int:
    n = C.c_size_t(0)
    _check("qre_workspace_bytes", _lib().qre_workspace_bytes(C.byref(_desc(T, H, I, E, K, bits, act_int8)),
                                                             C.byref(n)))
    return n.value


def stage_workspace_bytes(T, H, I, E, K, bits=4, act_int8=False) -> int:
    n = C.c_size_t(0)
    _check("qre_stage_workspace_bytes",
           _lib().qre_stage_workspace_bytes(C.byref(_desc(T, H, I, E, K, bits, act_int8)), C.byref(n)))
    return n.value


def _workspace(nbytes, device):
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def moe_forward(x, topk_ids, topk_w, W: QuantizedExperts, act_int8=False, out=None, workspace=None):
    """out[T,H] bf16 = routed-expert feed-forward of x[T,H] bf16."""
    T, H = x.shape
    K = topk_ids.shape[1]
    _need(x, "x", torch.bfloat16, (T, H))
    _need(topk_ids, "topk_ids", torch.int32, (T, K))
    _need(topk_w, "topk_w", torch.float32, (T, K))
    if W.H != H:
        raise ValueError("weights and x disagree on H")
    d = _desc(T, H, W.I, W.E, K, W.bits, act_int8)
    nb = workspace_bytes(T, H, W.I, W.E, K, W.bits, act_int8)
    if workspace is None:
        workspace = _workspace(nb, x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (T, H))
    _need(workspace, "workspace", torch.uint8)
    ws_struct = W._struct()
    _check("qre_moe_forward", _lib().qre_moe_forward(
        C.byref(d), _ptr(x), _ptr(topk_ids), _ptr(topk_w), C.byref(ws_struct), _ptr(out), _ptr(workspace),
        workspace.numel(), _stream()))
    return out


def moe_forward_timed(x, topk_ids, topk_w, W: QuantizedExperts, events, act_int8=False, out=None, workspace=None):
    """moe_forward that records eight caller-created hipEvent_t handles (ints,
    or None): six between its steps and the gate/up kernel's own begin and
    end; see qre_moe_forward_timed."""
    T, H = x.shape
    K = topk_ids.shape[1]
    _need(x, "x", torch.bfloat16, (T, H))
    _need(topk_ids, "topk_ids", torch.int32, (T, K))
    _need(topk_w, "topk_w", torch.float32, (T, K))
    if len(events) != 8:
        raise ValueError("eight events")
    d = _desc(T, H, W.I, W.E, K, W.bits, act_int8)
    if workspace is None:
        workspace = _workspace(workspace_bytes(T, H, W.I, W.E, K, W.bits, act_int8), x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    ev = (C.c_void_p * 8)(*[e if e else None for e in events])
    ws_struct = W._struct()
    _check("qre_moe_forward_timed", _lib().qre_moe_forward_timed(
        C.byref(d), _ptr(x), _ptr(topk_ids), _ptr(topk_w), C.byref(ws_struct), _ptr(out), _ptr(workspace),
        workspace.numel(), ev, _stream()))
    return out


def workspace_permutation(T, H, I, E, K, bits, act_int8, workspace):
    """(counts[E], offsets[E+1], sorted_slot[S], slot_row[S]) int32 views into a
    moe_forward workspace (valid once that call has finished)."""
    P = [C.c_void_p() for _ in range(4)]
    _check("qre_workspace_permutation", _lib().qre_workspace_permutation(
        C.byref(_desc(T, H, I, E, K, bits, act_int8)), _ptr(workspace), *[C.byref(p) for p in P]))
    base = workspace.data_ptr()
    S = T * K
    views = []
    for ptr, n in zip(P, (E, E + 1, S, S)):
        off = ptr.value - base
        views.append(workspace[off:off + 4 * n].view(torch.int32))
    return tuple(views)


def read_device_error(workspace) -> int:
    """Dropped-slot count (ids outside [0, E)) of the last routing that used
    `workspace` (a moe_forward or route workspace); synchronizes the stream."""
    _need(workspace, "workspace", torch.uint8)
    n = C.c_int32(0)
    _check("qre_read_device_error", _lib().qre_read_device_error(_ptr(workspace), C.byref(n), _stream()))
    return n.value


def stage_workspace(T, H, I, E, K, bits=4, act_int8=False, device="cuda"):
    """Workspace for the stage GEMM entry points (row-tile lists)."""
    return _workspace(stage_workspace_bytes(T, H, I, E, K, bits, act_int8), device)


def route(topk_ids, E, workspace=None):
    """(counts[E], offsets[E+1], sorted_slot[S], slot_row[S], workspace): the
    stable counting sort of the T*K slots by expert id."""
    T, K = topk_ids.shape
    _need(topk_ids, "topk_ids", torch.int32, (T, K))
    dev = topk_ids.device
    S = T * K
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_slot = torch.empty(max(S, 1), dtype=torch.int32, device=dev)[:S]
    slot_row = torch.empty(max(S, 1), dtype=torch.int32, device=dev)[:S]
    if workspace is None:
        n = C.c_size_t(0)
        _check("qre_route_workspace_bytes", _lib().qre_route_workspace_bytes(T, K, E, C.byref(n)))
        workspace = _workspace(n.value, dev)
    _need(workspace, "workspace", torch.uint8)
    _check("qre_route", _lib().qre_route(_ptr(topk_ids), T, K, E, _ptr(counts), _ptr(offsets), _ptr(sorted_slot),
                                         _ptr(slot_row), _ptr(workspace), workspace.numel(), _stream()))
    return counts, offsets, sorted_slot, slot_row, workspace


def quantize_act(v):
    """v[rows, cols] bf16 -> (q int8 [rows, cols], s fp32 [rows, cols/128])."""
    rows, cols = v.shape
    _need(v, "v", torch.bfloat16)
    q = torch.empty((rows, cols), dtype=torch.int8, device=v.device)
    s = torch.empty((rows, cols // GROUP), dtype=torch.float32, device=v.device)
    _check("qre_quantize_act", _lib().qre_quantize_act(_ptr(v), rows, cols, _ptr(q), _ptr(s), _stream()))
    return q, s


def quantize_weights(w, bits, out=None):
    """w[..., rows, cols] fp32 -> (q uint8 [..., rows, cols*bits/8], s fp16 [..., rows, cols/128]).
    `out` may give the (q, s) tensors to write."""
    _need(w, "w", torch.float32)
    lead, (rows, cols) = tuple(w.shape[:-2]), tuple(w.shape[-2:])
    R = rows
    for d in lead:
        R *= d
    if out is None:
        q = torch.empty(lead + (rows, packed_cols(cols, bits)), dtype=torch.uint8, device=w.device)
        s = torch.empty(lead + (rows, cols // GROUP), dtype=torch.float16, device=w.device)
    else:
        q, s = out
        _need(q, "q", torch.uint8, lead + (rows, packed_cols(cols, bits)))
        _need(s, "s", torch.float16, lead + (rows, cols // GROUP))
    _check("qre_quantize_weights", _lib().qre_quantize_weights(_ptr(w), R, cols, bits, _ptr(q), _ptr(s), _stream()))
    return q, s


def gate_up(x, sorted_slot, offsets, W: QuantizedExperts, K, act_int8=False, xq=None, xs=None, h=None,
            want_hq=False, h_out=True, workspace=None):
    """h[S, I] bf16 by sorted row.  INT8 mode with want_hq also returns the
    per-128 INT8 quantization of h: (h, hq int8 [S, I], hs fp32 [S, I/128]);
    h_out=False then skips h (returned as None)."""
    if act_int8:
        T, H = xq.shape
        _need(xq, "xq", torch.int8, (T, H))
        _need(xs, "xs", torch.float32, (T, H // GROUP))
        dev = xq.device
    else:
        T, H = x.shape
        _need(x, "x", torch.bfloat16, (T, H))
        dev = x.device
    S = T * K
    E = W.E
    _need(sorted_slot, "sorted_slot", torch.int32, (S,))
    _need(offsets, "offsets", torch.int32, (E + 1,))
    if h is None and (h_out or not want_hq):
        h = torch.empty((S, W.I), dtype=torch.bfloat16, device=dev)
    if h is not None:
        _need(h, "h", torch.bfloat16, (S, W.I))
    hq = hs = None
    if want_hq:
        hq = torch.empty((S, W.I), dtype=torch.int8, device=dev)
        hs = torch.empty((S, W.I // GROUP), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = stage_workspace(T, H, W.I, E, K, W.bits, act_int8, dev)
    _need(workspace, "workspace", torch.uint8)
    d = _desc(T, H, W.I, E, K, W.bits, act_int8)
    ws_struct = W._struct()
    _check("qre_gate_up", _lib().qre_gate_up(C.byref(d), _ptr(x), _ptr(xq), _ptr(xs), _ptr(sorted_slot),
                                             _ptr(offsets), C.byref(ws_struct), _ptr(h), _ptr(hq), _ptr(hs),
                                             _ptr(workspace), workspace.numel(), _stream()))
    return (h, hq, hs) if want_hq else h


def down(h, offsets, W: QuantizedExperts, T, K, act_int8=False, hq=None, hs=None, y=None, workspace=None):
    """y[S, H] bf16 by sorted row."""
    S = T * K
    I, H, E = W.I, W.H, W.E
    if act_int8:
        _need(hq, "hq", torch.int8, (S, I))
        _need(hs, "hs", torch.float32, (S, I // GROUP))
        dev = hq.device
    else:
        _need(h, "h", torch.bfloat16, (S, I))
        dev = h.device
    _need(offsets, "offsets", torch.int32, (E + 1,))
    if y is None:
        y = torch.empty((S, H), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (S, H))
    if workspace is None:
        workspace = stage_workspace(T, H, I, E, K, W.bits, act_int8, dev)
    _need(workspace, "workspace", torch.uint8)
    d = _desc(T, H, I, E, K, W.bits, act_int8)
    ws_struct = W._struct()
    _check("qre_down", _lib().qre_down(C.byref(d), _ptr(h), _ptr(hq), _ptr(hs), _ptr(offsets), C.byref(ws_struct),
                                       _ptr(y), _ptr(workspace), workspace.numel(), _stream()))
    return y


def topk_softmax(logits, K):
    """logits[T, E] fp32 -> (topk_ids int32 [T, K], topk_w fp32 [T, K]): the K
    largest logits per token (descending, ties to the lower id) and a softmax
    over them, computed by the library's router kernel."""
    T, E = logits.shape
    _need(logits, "logits", torch.float32, (T, E))
    ids = torch.empty((T, K), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    _check("qre_topk_softmax", _lib().qre_topk_softmax(_ptr(logits), T, E, K, _ptr(ids), _ptr(w), _stream()))
    return ids, w


def combine(y, slot_row, topk_w, out=None):
    """out[T, H] bf16 from y[S, H] bf16 (sorted rows), slot_row[S], topk_w[T, K]."""
    T, K = topk_w.shape
    S, H = y.shape
    _need(y, "y", torch.bfloat16, (T * K, H))
    _need(slot_row, "slot_row", torch.int32, (T * K,))
    _need(topk_w, "topk_w", torch.float32, (T, K))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _need(out, "out", torch.bfloat16, (T, H))
    _check("qre_combine", _lib().qre_combine(_ptr(y), _ptr(slot_row), _ptr(topk_w), T, K, H, _ptr(out), _stream()))
    return out


def hbm_read_probe(buf, sink):
    """Measurement aid: stream-read the bytes of `buf` (any contiguous GPU
    tensor, a multiple of 16 bytes) into `sink` (uint8, >= 4096 bytes)."""
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous GPU tensor")
    _need(sink, "sink", torch.uint8)
    if sink.numel() < 4096:
        raise ValueError("sink must hold 4096 bytes")
    _check("qre_hbm_read_probe", _lib().qre_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                           _stream()))


PLAN_ROUTE_IN_GATE_UP, PLAN_COMBINE_IN_DOWN, PLAN_BIG_TILES = 1, 2, 4


def forward_plan(T, H, I, E, K, bits, act_int8=False) -> int:
    """Bit mask of what moe_forward launches for this problem (PLAN_*)."""
    n = C.c_int32(0)
    _check("qre_forward_plan", _lib().qre_forward_plan(C.byref(_desc(T, H, I, E, K, bits, act_int8)), C.byref(n)))
    return n.value


NOALLOC_SCRATCH_BYTES = 32 << 20


def moe_forward_noalloc(x, topk_ids, topk_w, W: QuantizedExperts, act_int8=False, out=None):
    """moe_forward through the allocation-free entry point (the library's own
    per-GPU workspace; workspace sizes above NOALLOC_SCRATCH_BYTES raise)."""
    T, H = x.shape
    K = topk_ids.shape[1]
    _need(x, "x", torch.bfloat16, (T, H))
    _need(topk_ids, "topk_ids", torch.int32, (T, K))
    _need(topk_w, "topk_w", torch.float32, (T, K))
    if W.H != H:
        raise ValueError("weights and x disagree on H")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (T, H))
    d = _desc(T, H, W.I, W.E, K, W.bits, act_int8)
    ws_struct = W._struct()
    _check("qre_moe_forward_noalloc", _lib().qre_moe_forward_noalloc(
        C.byref(d), _ptr(x), _ptr(topk_ids), _ptr(topk_w), C.byref(ws_struct), _ptr(out), _stream()))
    return out


# ---- NVFP4 (W4A4) ------------------------------------------------------------------

NVFP4_BLOCK = 16


class _Fp4Mat(C.Structure):
    _fields_ = [("q", C.c_void_p), ("s", C.c_void_p), ("outer", C.c_void_p)]


class _Fp4Weights(C.Structure):
    _fields_ = [("gate", _Fp4Mat), ("up", _Fp4Mat), ("down", _Fp4Mat)]


@dataclass
class Nvfp4Experts:
    """NVFP4 routed-expert weights on the GPU (layouts of include/qre.h):
    codes uint8 [E, rows, cols/2], E4M3 block scales uint8 [E, rows, cols/16],
    FP32 outer scales [E]; gate/up rows I, cols H; down rows H, cols I."""
    gate_q: torch.Tensor
    gate_s: torch.Tensor
    gate_o: torch.Tensor
    up_q: torch.Tensor
    up_s: torch.Tensor
    up_o: torch.Tensor
    down_q: torch.Tensor
    down_s: torch.Tensor
    down_o: torch.Tensor

    @property
    def E(self):
        return self.gate_q.shape[0]

    @property
    def I(self):
        return self.gate_q.shape[1]

    @property
    def H(self):
        return self.down_q.shape[1]

    def tensors(self):
        return (self.gate_q, self.gate_s, self.gate_o, self.up_q, self.up_s, self.up_o,
                self.down_q, self.down_s, self.down_o)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tensors())

    def expert_nbytes(self) -> int:
        return self.nbytes() // self.E

    def clone(self) -> "Nvfp4Experts":
        return Nvfp4Experts(*(t.clone() for t in self.tensors()))

    def _struct(self):
        E, H, I = self.E, self.H, self.I
        for name, (rows, cols) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            _need(getattr(self, name + "_q"), name + "_q", torch.uint8, (E, rows, cols // 2))
            _need(getattr(self, name + "_s"), name + "_s", torch.uint8, (E, rows, cols // NVFP4_BLOCK))
            _need(getattr(self, name + "_o"), name + "_o", torch.float32, (E,))
        m = lambda n: _Fp4Mat(getattr(self, n + "_q").data_ptr(), getattr(self, n + "_s").data_ptr(),
                              getattr(self, n + "_o").data_ptr())
        return _Fp4Weights(m("gate"), m("up"), m("down"))

    @staticmethod
    def empty(E, H, I, device="cuda"):
        u8, f32 = torch.uint8, torch.float32
        mk = lambda rows, cols: (torch.empty((E, rows, cols // 2), dtype=u8, device=device),
                                 torch.empty((E, rows, cols // NVFP4_BLOCK), dtype=u8, device=device),
                                 torch.empty((E,), dtype=f32, device=device))
        return Nvfp4Experts(*mk(I, H), *mk(I, H), *mk(H, I))


def _fp4_desc(T, H, I, E, K):
    return _Desc(T, H, I, E, K, 4, NVFP4_BLOCK, 0)


def nvfp4_quantize_weights(w, out=None):
    """w[..., rows, cols] fp32 -> (q uint8 [..., rows, cols/2], s uint8 E4M3 [..., rows, cols/16],
    outer fp32 [...]): one outer scale per matrix.  `out` may give (q, s, outer)."""
    _need(w, "w", torch.float32)
    lead, (rows, cols) = tuple(w.shape[:-2]), tuple(w.shape[-2:])
    mats = 1
    for d in lead:
        mats *= d
    if out is None:
        q = torch.empty(lead + (rows, cols // 2), dtype=torch.uint8, device=w.device)
        s = torch.empty(lead + (rows, cols // NVFP4_BLOCK), dtype=torch.uint8, device=w.device)
        o = torch.empty(lead, dtype=torch.float32, device=w.device)
    else:
        q, s, o = out
        _need(q, "q", torch.uint8, lead + (rows, cols // 2))
        _need(s, "s", torch.uint8, lead + (rows, cols // NVFP4_BLOCK))
        _need(o, "outer", torch.float32, lead)
    _check("qre_nvfp4_quantize_weights", _lib().qre_nvfp4_quantize_weights(
        _ptr(w), mats, rows, cols, _ptr(q), _ptr(s), _ptr(o), _stream()))
    return q, s, o


def nvfp4_quantize_act(v):
    """v[rows, cols] bf16 -> (q uint8 [rows, cols/2], s uint8 [rows, cols/16], row_scale fp32 [rows])."""
    rows, cols = v.shape
    _need(v, "v", torch.bfloat16)
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=v.device)
    s = torch.empty((rows, cols // NVFP4_BLOCK), dtype=torch.uint8, device=v.device)
    r = torch.empty((rows,), dtype=torch.float32, device=v.device)
    _check("qre_nvfp4_quantize_act", _lib().qre_nvfp4_quantize_act(_ptr(v), rows, cols, _ptr(q), _ptr(s), _ptr(r),
                                                                   _stream()))
    return q, s, r


def nvfp4_workspace_bytes(T, H, I, E, K) -> int:
    n = C.c_size_t(0)
    _check("qre_nvfp4_workspace_bytes", _lib().qre_nvfp4_workspace_bytes(C.byref(_fp4_desc(T, H, I, E, K)),
                                                                         C.byref(n)))
    return n.value


def nvfp4_stage_workspace(T, H, I, E, K, device="cuda"):
    n = C.c_size_t(0)
    _check("qre_nvfp4_stage_workspace_bytes",
           _lib().qre_nvfp4_stage_workspace_bytes(C.byref(_fp4_desc(T, H, I, E, K)), C.byref(n)))
    return _workspace(n.value, device)


def nvfp4_moe_forward(x, topk_ids, topk_w, W: Nvfp4Experts, out=None, workspace=None):
    """out[T,H] bf16 = NVFP4 routed-expert feed-forward of x[T,H] bf16."""
    T, H = x.shape
    K = topk_ids.shape[1]
    _need(x, "x", torch.bfloat16, (T, H))
    _need(topk_ids, "topk_ids", torch.int32, (T, K))
    _need(topk_w, "topk_w", torch.float32, (T, K))
    if W.H != H:
        raise ValueError("weights and x disagree on H")
    d = _fp4_desc(T, H, W.I, W.E, K)
    if workspace is None:
        workspace = _workspace(nvfp4_workspace_bytes(T, H, W.I, W.E, K), x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (T, H))
    _need(workspace, "workspace", torch.uint8)
    ws_struct = W._struct()
    _check("qre_nvfp4_moe_forward", _lib().qre_nvfp4_moe_forward(
        C.byref(d), _ptr(x), _ptr(topk_ids), _ptr(topk_w), C.byref(ws_struct), _ptr(out), _ptr(workspace),
        workspace.numel(), _stream()))
    return out


def nvfp4_moe_forward_timed(x, topk_ids, topk_w, W: Nvfp4Experts, events, out=None, workspace=None):
    """nvfp4_moe_forward that records eight caller-created hipEvent_t handles
    (ints, or None): six between its steps and the gate/up kernel's own begin
    and end; see qre_nvfp4_moe_forward_timed."""
    T, H = x.shape
    K = topk_ids.shape[1]
    _need(x, "x", torch.bfloat16, (T, H))
    _need(topk_ids, "topk_ids", torch.int32, (T, K))
    _need(topk_w, "topk_w", torch.float32, (T, K))
    if len(events) != 8:
        raise ValueError("eight events")
    if workspace is None:
        workspace = _workspace(nvfp4_workspace_bytes(T, H, W.I, W.E, K), x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    ev = (C.c_void_p * 8)(*[e if e else None for e in events])
    ws_struct = W._struct()
    _check("qre_nvfp4_moe_forward_timed", _lib().qre_nvfp4_moe_forward_timed(
        C.byref(_fp4_desc(T, H, W.I, W.E, K)), _ptr(x), _ptr(topk_ids), _ptr(topk_w), C.byref(ws_struct), _ptr(out),
        _ptr(workspace), workspace.numel(), ev, _stream()))
    return out


def nvfp4_workspace_permutation(T, H, I, E, K, workspace):
    """(counts, offsets, sorted_slot, slot_row) int32 views into an NVFP4 forward workspace."""
    P = [C.c_void_p() for _ in range(4)]
    _check("qre_nvfp4_workspace_permutation", _lib().qre_nvfp4_workspace_permutation(
        C.byref(_fp4_desc(T, H, I, E, K)), _ptr(workspace), *[C.byref(p) for p in P]))
    base = workspace.data_ptr()
    S = T * K
    return tuple(workspace[p.value - base:p.value - base + 4 * n].view(torch.int32)
                 for p, n in zip(P, (E, E + 1, S, S)))


def nvfp4_gate_up(xq, xs, xr, sorted_slot, offsets, W: Nvfp4Experts, K, h=None, workspace=None):
    """h[T*K, I] bf16 by sorted row, from x quantized by nvfp4_quantize_act."""
    T = xr.shape[0]
    H, I, E = W.H, W.I, W.E
    _need(xq, "xq", torch.uint8, (T, H // 2))
    _need(xs, "xs", torch.uint8, (T, H // NVFP4_BLOCK))
    _need(xr, "xr", torch.float32, (T,))
    S = T * K
    _need(sorted_slot, "sorted_slot", torch.int32, (S,))
    _need(offsets, "offsets", torch.int32, (E + 1,))
    if h is None:
        h = torch.zeros((S, I), dtype=torch.bfloat16, device=xq.device)
    _need(h, "h", torch.bfloat16, (S, I))
    if workspace is None:
        workspace = nvfp4_stage_workspace(T, H, I, E, K, xq.device)
    ws_struct = W._struct()
    _check("qre_nvfp4_gate_up", _lib().qre_nvfp4_gate_up(
        C.byref(_fp4_desc(T, H, I, E, K)), _ptr(xq), _ptr(xs), _ptr(xr), _ptr(sorted_slot), _ptr(offsets),
        C.byref(ws_struct), _ptr(h), _ptr(workspace), workspace.numel(), _stream()))
    return h


def nvfp4_down(hq, hs, hr, offsets, W: Nvfp4Experts, T, K, y=None, workspace=None):
    """y[T*K, H] bf16 by sorted row, from h quantized per sorted row."""
    H, I, E = W.H, W.I, W.E
    S = T * K
    _need(hq, "hq", torch.uint8, (S, I // 2))
    _need(hs, "hs", torch.uint8, (S, I // NVFP4_BLOCK))
    _need(hr, "hr", torch.float32, (S,))
    _need(offsets, "offsets", torch.int32, (E + 1,))
    if y is None:
        y = torch.zeros((S, H), dtype=torch.bfloat16, device=hq.device)
    _need(y, "y", torch.bfloat16, (S, H))
    if workspace is None:
        workspace = nvfp4_stage_workspace(T, H, I, E, K, hq.device)
    ws_struct = W._struct()
    _check("qre_nvfp4_down", _lib().qre_nvfp4_down(
        C.byref(_fp4_desc(T, H, I, E, K)), _ptr(hq), _ptr(hs), _ptr(hr), _ptr(offsets), C.byref(ws_struct),
        _ptr(y), _ptr(workspace), workspace.numel(), _stream()))
    return y
