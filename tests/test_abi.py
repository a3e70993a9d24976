"""The C ABI without a GPU: libqre.so loads, exports every function that
include/qre.h declares, and rejects bad arguments on the host (validation runs
before any HIP call, so no device is needed)."""
import ctypes as C
import os
import re

import pytest

import quantized_routed_expert_top_amd as qre

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qre.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qre_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert "qre_moe_forward" in names and len(names) >= 12
    lib = C.CDLL(qre.library_path())
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    for code in range(0, -10, -1):
        assert qre.status_string(code) != "unknown status"
    assert qre.status_string(5) == "unknown status"


def _desc(**kw):
    d = dict(T=32, H=2048, I=512, E=256, K=8, weight_bits=4, group_size=128, act_int8=0)
    d.update(kw)
    return qre._Desc(*(d[k] for k, _ in qre._Desc._fields_))


@pytest.mark.parametrize("kw,code", [
    (dict(weight_bits=5), -3), (dict(group_size=64), -4), (dict(act_int8=2), -8),
    (dict(H=2000), -2), (dict(I=100), -2), (dict(T=-1), -2), (dict(K=0), -2), (dict(K=300), -2),
    (dict(E=0), -2), (dict(E=1024, K=8), -9), (dict(T=1 << 28, K=8), -9),
])
def test_descriptor_validation(kw, code):
    n = C.c_size_t(0)
    assert qre._lib().qre_workspace_bytes(C.byref(_desc(**kw)), C.byref(n)) == code


def test_workspace_sizes_grow_with_problem():
    small = qre.workspace_bytes(32, 2048, 512, 256, 8, 4)
    big = qre.workspace_bytes(512, 2048, 512, 256, 8, 4)
    a8 = qre.workspace_bytes(512, 2048, 512, 256, 8, 8, act_int8=True)
    assert 0 < small < big < a8
    # h (bf16 S x I) and y (bf16 S x H) dominate
    S = 512 * 8
    assert big >= S * 512 * 2 + S * 2048 * 2


def test_forward_argument_errors_need_no_gpu():
    L = qre._lib()
    d = _desc()
    w = qre._Weights(16, 16, 16, 16, 16, 16)
    ws = C.c_size_t(0)
    L.qre_workspace_bytes(C.byref(d), C.byref(ws))
    P = C.c_void_p
    # null x
    assert L.qre_moe_forward(C.byref(d), None, P(16), P(16), C.byref(w), P(16), P(16), ws.value, None) == -1
    # misaligned out
    assert L.qre_moe_forward(C.byref(d), P(16), P(16), P(16), C.byref(w), P(24), P(16), ws.value, None) == -5
    # workspace too small
    assert L.qre_moe_forward(C.byref(d), P(16), P(16), P(16), C.byref(w), P(32), P(16), ws.value - 1,
                             None) == -6
    # missing weight pointer
    w2 = qre._Weights(16, 16, 16, None, 16, 16)
    assert L.qre_moe_forward(C.byref(d), P(16), P(16), P(16), C.byref(w2), P(32), P(16), ws.value, None) == -1
    # zero tokens: valid, nothing enqueued (null pointers allowed)
    d0 = _desc(T=0)
    assert L.qre_moe_forward(C.byref(d0), None, None, None, None, None, None, 0, None) == 0
    # stage calls
    assert L.qre_quantize_act(P(16), 4, 100, P(16), P(16), None) == -2
    assert L.qre_quantize_weights(P(16), 4, 256, 3, P(16), P(16), None) == -3
    assert L.qre_combine(P(16), P(16), P(16), 4, 2, 100, P(16), None) == -2
    # INT8 mode without xq/xs; hq/hs in BF16 mode; only one of hq/hs
    assert L.qre_gate_up(C.byref(_desc(act_int8=1)), P(16), None, None, P(16), P(16), C.byref(w), P(16), None, None,
                         P(16), 1 << 30, None) == -8
    assert L.qre_gate_up(C.byref(_desc()), P(16), None, None, P(16), P(16), C.byref(w), P(16), P(16), P(16),
                         P(16), 1 << 30, None) == -8
    assert L.qre_gate_up(C.byref(_desc(act_int8=1)), None, P(16), P(16), P(16), P(16), C.byref(w), P(16), P(16), None,
                         P(16), 1 << 30, None) == -8
    # offsets are required; the workspace must hold the row tiles
    assert L.qre_gate_up(C.byref(_desc()), P(16), None, None, P(16), None, C.byref(w), P(16), None, None,
                         P(16), 1 << 30, None) == -1
    assert L.qre_down(C.byref(_desc()), P(16), None, None, None, C.byref(w), P(16), P(16), 1 << 30, None) == -1
    assert L.qre_down(C.byref(_desc()), P(16), None, None, P(16), C.byref(w), P(16), P(16), 16, None) == -6
    # router: K > E, limits, null, misaligned, empty
    assert L.qre_topk_softmax(P(16), 4, 8, 9, P(16), P(16), None) == -2
    assert L.qre_topk_softmax(P(16), 4, 8, 0, P(16), P(16), None) == -2
    assert L.qre_topk_softmax(P(16), 4, 2048, 8, P(16), P(16), None) == -9
    assert L.qre_topk_softmax(P(16), 4, 128, 65, P(16), P(16), None) == -9
    assert L.qre_topk_softmax(None, 4, 256, 8, P(16), P(16), None) == -1
    assert L.qre_topk_softmax(P(16), 4, 256, 8, P(20), P(16), None) == -5
    assert L.qre_topk_softmax(None, 0, 256, 8, None, None, None) == 0
    # routing: needs its workspace (large slot counts use routing scratch)
    assert L.qre_route(P(16), 8192, 8, 256, P(16), P(16), P(16), P(16), None, 0, None) == -1
    n = C.c_size_t(0)
    assert L.qre_route_workspace_bytes(8192, 8, 256, C.byref(n)) == 0 and n.value > 256
    assert L.qre_route(P(16), 8192, 8, 256, P(16), P(16), P(16), P(16), P(16), n.value - 1, None) == -6
    assert L.qre_route_workspace_bytes(4, 9, 8, C.byref(n)) == -2          # K > E
    assert L.qre_route_workspace_bytes(4, 8, 1024, C.byref(n)) == -9       # E > QRE_MAX_EXPERTS
    # the device-error read needs a workspace
    assert L.qre_read_device_error(None, P(16), None) == -1
    assert L.qre_read_device_error(P(20), P(16), None) == -5


def test_noalloc_rejects_oversized_problems_without_a_gpu():
    """The allocation-free entry point refuses a problem whose workspace
    exceeds the library's own before any HIP call."""
    L = qre._lib()
    w = qre._Weights(16, 16, 16, 16, 16, 16)
    P = C.c_void_p
    d = _desc(T=8192, weight_bits=8, act_int8=1)
    assert L.qre_moe_forward_noalloc(C.byref(d), P(16), P(16), P(16), C.byref(w), P(16), None) == -9
    assert L.qre_moe_forward_noalloc(C.byref(_desc(weight_bits=5)), P(16), P(16), P(16), C.byref(w), P(16),
                                     None) == -3
    n = C.c_size_t(0)
    assert L.qre_workspace_bytes(C.byref(_desc()), C.byref(n)) == 0 and n.value <= qre.NOALLOC_SCRATCH_BYTES


def _fp4_desc(**kw):
    return _desc(**{"group_size": 16, **kw})


@pytest.mark.parametrize("kw,code", [
    (dict(weight_bits=8), -3), (dict(group_size=128), -4), (dict(act_int8=1), -8), (dict(H=2000), -2),
    (dict(I=144), -2), (dict(K=300), -2), (dict(E=1024), -9),
    (dict(T=64, H=8192, E=8), -9),                     # 16 staged rows of x exceed the LDS
    (dict(T=4, H=8192, E=8, K=2), 0),                  # 8 rows fit
])
def test_nvfp4_descriptor_validation(kw, code):
    n = C.c_size_t(0)
    assert qre._lib().qre_nvfp4_workspace_bytes(C.byref(_fp4_desc(**kw)), C.byref(n)) == code


def test_nvfp4_argument_errors_need_no_gpu():
    L = qre._lib()
    P = C.c_void_p
    m = lambda o=16: qre._Fp4Mat(16, 16, o)
    w = qre._Fp4Weights(m(), m(), m())
    d = _fp4_desc()
    ws = C.c_size_t(0)
    assert L.qre_nvfp4_workspace_bytes(C.byref(d), C.byref(ws)) == 0
    args = lambda **k: [C.byref(k.get("d", d)), k.get("x", P(16)), P(16), P(16), C.byref(k.get("w", w)),
                        k.get("out", P(32)), P(16), k.get("n", ws.value), None]
    assert L.qre_nvfp4_moe_forward(*args(x=None)) == -1
    assert L.qre_nvfp4_moe_forward(*args(out=P(24))) == -5
    assert L.qre_nvfp4_moe_forward(*args(n=ws.value - 1)) == -6
    assert L.qre_nvfp4_moe_forward(*args(w=qre._Fp4Weights(m(), qre._Fp4Mat(16, None, 16), m()))) == -1
    assert L.qre_nvfp4_moe_forward(*args(w=qre._Fp4Weights(m(), m(), m(o=18)))) == -5     # outer: 4-byte alignment
    assert L.qre_nvfp4_moe_forward(*args(d=_desc())) == -4                              # an INT descriptor
    assert L.qre_nvfp4_moe_forward(C.byref(_fp4_desc(T=0)), None, None, None, None, None, None, 0, None) == 0
    # quantizers
    assert L.qre_nvfp4_quantize_act(P(16), 4, 100, P(16), P(16), P(16), None) == -2
    assert L.qre_nvfp4_quantize_act(P(16), 4, 64, P(16), P(16), None, None) == -1
    assert L.qre_nvfp4_quantize_weights(P(16), 2, 4, 24, P(16), P(16), P(16), None) == -2
    assert L.qre_nvfp4_quantize_weights(P(16), 2, 4, 32, P(16), P(16), P(18), None) == -5
    assert L.qre_nvfp4_quantize_weights(None, 0, 4, 32, None, None, None, None) == 0
    # stages: the workspace must hold the row tiles
    sw = C.c_size_t(0)
    assert L.qre_nvfp4_stage_workspace_bytes(C.byref(d), C.byref(sw)) == 0 and sw.value > 0
    assert L.qre_nvfp4_gate_up(C.byref(d), P(16), P(16), P(16), P(16), P(16), C.byref(w), P(16), P(16), 16,
                               None) == -6
    assert L.qre_nvfp4_down(C.byref(d), P(16), P(16), None, P(16), C.byref(w), P(16), P(16), sw.value, None) == -1
