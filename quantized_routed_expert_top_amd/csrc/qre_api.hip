// Host side of the C ABI declared in include/qre.h: argument validation,
// workspace layout and the launch sequence of the routed-expert feed-forward.
// No entry point allocates memory or synchronizes (except
// qre_read_device_error); all validation happens before the first launch.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "qre.h"
#include "qre_internal.h"

using namespace qre;

namespace qre {
KernelEvents& kernel_events() {
  static thread_local KernelEvents ke{nullptr, nullptr};
  return ke;
}
}  // namespace qre

namespace {

thread_local int g_last_hip_error = 0;

// Workspace of qre_moe_forward_noalloc: one array per GPU, held until the
// process ends.  In host code `scratch` is only a handle; its device address
// on the current GPU comes from hipGetSymbolAddress, taken once per device.
static __device__ __align__(256) uint8_t scratch[QRE_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return QRE_OK;
  g_last_hip_error = (int)e;
  return QRE_ERR_HIP;
}

// Carves a workspace into 256-byte aligned pieces (or only measures it).
struct Carver {
  uint8_t* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<uint8_t*>(b)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = align_up(off + count * sizeof(T));
    return p;
  }
};

// Every workspace (qre_moe_forward's and the stage entry points') starts with
// a 256-byte header; its first int32 is the number of dropped slots (ids
// outside [0, E)) of the last routing that used the workspace.
constexpr size_t kHeaderInts = kAlign / sizeof(int32_t);

// Scratch shared by qre_moe_forward and the stage entry points: the header,
// the two GEMM row-tile lists and the routing scratch (and, for the stage
// gate/up in INT8 mode, room for the BF16 h its quantizer reads when the
// caller asks for hq/hs only).  qre_moe_forward's workspace starts with the
// same block.
struct StageLayout {
  int32_t* header;
  int32_t* ntiles;            // [2]: gate/up, down
  Tile *tiles_gu, *tiles_dn;
  void* route_scratch;
  uint16_t* h_tmp;            // stage layout, INT8 mode only
  int bm_gu, bm_dn;
  int64_t mt_gu, mt_dn;
};

void carve_stage(const qre_desc& d, Carver& c, StageLayout& L, bool stage) {
  const int64_t S = (int64_t)d.T * d.K;
  L.bm_gu = gemm_tile_rows(S, d.E, 2 * d.I, d.H, d.act_int8);
  L.bm_dn = gemm_tile_rows(S, d.E, d.H, d.I, d.act_int8);
  L.mt_gu = max_tiles(S, d.E, L.bm_gu);
  L.mt_dn = max_tiles(S, d.E, L.bm_dn);
  L.header = c.take<int32_t>(kHeaderInts);
  L.ntiles = c.take<int32_t>(2);
  L.tiles_gu = c.take<Tile>(L.mt_gu);
  L.tiles_dn = c.take<Tile>(L.mt_dn);
  L.route_scratch = c.take<uint8_t>(route_scratch_bytes(S, d.E));
  L.h_tmp = (stage && d.act_int8) ? c.take<uint16_t>((size_t)S * d.I) : nullptr;
}

struct Layout {
  StageLayout st;
  int32_t *counts, *offsets, *sorted_slot, *slot_row;
  int8_t* xq; float* xs;      // INT8 activations of x
  uint16_t* h;                // bf16 [S][I]
  int8_t* hq; float* hs;      // INT8 activations of h
  uint16_t* y;                // bf16 [S][H]
  size_t bytes;
};

Layout make_layout(const qre_desc& d, void* ws) {
  Layout L;
  const int64_t S = (int64_t)d.T * d.K;
  Carver c(ws);
  carve_stage(d, c, L.st, false);
  L.counts = c.take<int32_t>(d.E);
  L.offsets = c.take<int32_t>(d.E + 1);
  L.sorted_slot = c.take<int32_t>(S);
  L.slot_row = c.take<int32_t>(S);
  L.xq = nullptr; L.xs = nullptr; L.hq = nullptr; L.hs = nullptr;
  if (d.act_int8) {
    L.xq = c.take<int8_t>((size_t)d.T * d.H);
    L.xs = c.take<float>((size_t)d.T * (d.H / kGroup));
    L.hq = c.take<int8_t>((size_t)S * d.I);
    L.hs = c.take<float>((size_t)S * (d.I / kGroup));
  }
  L.h = c.take<uint16_t>((size_t)S * d.I);
  L.y = c.take<uint16_t>((size_t)S * d.H);
  L.bytes = c.off;
  return L;
}

size_t stage_bytes(const qre_desc& d) {
  Carver c(nullptr);
  StageLayout L;
  carve_stage(d, c, L, true);
  return c.off;
}

StageLayout stage_layout(const qre_desc& d, const void* ws) {
  Carver c(const_cast<void*>(ws));
  StageLayout L;
  carve_stage(d, c, L, true);
  return L;
}

// Routing alone: the header, then the routing scratch.
size_t route_bytes(int64_t S, int E) { return kHeaderInts * sizeof(int32_t) + align_up(route_scratch_bytes(S, E)); }

int check_desc(const qre_desc* d) {
  if (!d) return QRE_ERR_NULL;
  if (d->weight_bits != 4 && d->weight_bits != 8) return QRE_ERR_BITS;
  if (d->group_size != QRE_GROUP) return QRE_ERR_GROUP;
  if (d->act_int8 != 0 && d->act_int8 != 1) return QRE_ERR_MODE;
  if (d->T < 0 || d->H <= 0 || d->I <= 0 || d->E <= 0 || d->K <= 0) return QRE_ERR_SHAPE;
  if (d->H % QRE_GROUP || d->I % QRE_GROUP) return QRE_ERR_SHAPE;
  if (d->K > d->E) return QRE_ERR_SHAPE;
  if (d->E > QRE_MAX_EXPERTS) return QRE_ERR_LIMIT;
  const int64_t S = (int64_t)d->T * d->K;
  if (S >= (1ll << 31)) return QRE_ERR_LIMIT;
  // the GEMMs address x, h and one expert's weights with 32-bit buffer offsets
  if ((int64_t)d->T * d->H * 2 >= (1ll << 31) || S * d->I * 2 >= (1ll << 31)) return QRE_ERR_LIMIT;
  if ((int64_t)d->H * d->I * 2 >= (1ll << 31)) return QRE_ERR_LIMIT;
  if (max_tiles(S, d->E, 1) >= (1ll << 31)) return QRE_ERR_LIMIT;
  // grid limit of the GEMM launch (row tiles along grid.y, rounded up to a multiple of 8)
  if (max_tiles(S, d->E, gemm_tile_rows(S, d->E, 2 * d->I, d->H, d->act_int8)) > 65528) return QRE_ERR_LIMIT;
  if (max_tiles(S, d->E, gemm_tile_rows(S, d->E, d->H, d->I, d->act_int8)) > 65528) return QRE_ERR_LIMIT;
  return QRE_OK;
}

int check_weights(const qre_weights* w, bool need_gate_up, bool need_down) {
  if (!w) return QRE_ERR_NULL;
  if (need_gate_up && (!w->gate_q || !w->gate_s || !w->up_q || !w->up_s)) return QRE_ERR_NULL;
  if (need_down && (!w->down_q || !w->down_s)) return QRE_ERR_NULL;
  if (need_gate_up && !(aligned16(w->gate_q) && aligned16(w->gate_s) && aligned16(w->up_q) && aligned16(w->up_s)))
    return QRE_ERR_ALIGN;
  if (need_down && !(aligned16(w->down_q) && aligned16(w->down_s))) return QRE_ERR_ALIGN;
  return QRE_OK;
}

GemmProblem gate_up_problem(const qre_desc& d, const void* x, const int8_t* xq, const float* xs,
                            const int32_t* sorted_slot, const qre_weights& w, const Tile* tiles,
                            const int32_t* ntiles, int64_t mt, int bm, void* h) {
  GemmProblem p;
  p.act_int8 = d.act_int8;
  p.bits = d.weight_bits;
  p.gather_k = d.K;
  p.sorted_slot = sorted_slot;
  p.a = d.act_int8 ? static_cast<const void*>(xq) : x;
  p.a_scale = xs;
  p.a_rows = d.T;
  p.w0q = static_cast<const uint8_t*>(w.gate_q);
  p.w0s = static_cast<const uint16_t*>(w.gate_s);
  p.w1q = static_cast<const uint8_t*>(w.up_q);
  p.w1s = static_cast<const uint16_t*>(w.up_s);
  p.tiles = tiles;
  p.ntiles = ntiles;
  p.max_tiles = mt;
  p.bm = bm;
  p.out = h;
  p.n = d.I;
  p.kdim = d.H;
  return p;
}

GemmProblem down_problem(const qre_desc& d, const void* h, const int8_t* hq, const float* hs, const qre_weights& w,
                         const Tile* tiles, const int32_t* ntiles, int64_t mt, int bm, void* y) {
  GemmProblem p;
  p.act_int8 = d.act_int8;
  p.bits = d.weight_bits;
  p.gather_k = 0;
  p.sorted_slot = nullptr;
  p.a = d.act_int8 ? static_cast<const void*>(hq) : h;
  p.a_scale = hs;
  p.a_rows = (int64_t)d.T * d.K;
  p.w0q = static_cast<const uint8_t*>(w.down_q);
  p.w0s = static_cast<const uint16_t*>(w.down_s);
  p.w1q = nullptr;
  p.w1s = nullptr;
  p.tiles = tiles;
  p.ntiles = ntiles;
  p.max_tiles = mt;
  p.bm = bm;
  p.out = y;
  p.n = d.H;
  p.kdim = d.I;
  return p;
}

// ---- NVFP4 (W4A4) ----

int check_nvfp4_desc(const qre_desc* d) {
  if (!d) return QRE_ERR_NULL;
  if (d->weight_bits != 4) return QRE_ERR_BITS;
  if (d->group_size != QRE_NVFP4_BLOCK) return QRE_ERR_GROUP;
  if (d->act_int8 != 0) return QRE_ERR_MODE;
  if (d->T < 0 || d->H <= 0 || d->I <= 0 || d->E <= 0 || d->K <= 0) return QRE_ERR_SHAPE;
  if (d->H % QRE_GROUP || d->I % QRE_GROUP) return QRE_ERR_SHAPE;   // the GEMMs step 128 values at a time
  if (d->K > d->E) return QRE_ERR_SHAPE;
  if (d->E > QRE_MAX_EXPERTS) return QRE_ERR_LIMIT;
  const int64_t S = (int64_t)d->T * d->K;
  if (S >= (1ll << 31)) return QRE_ERR_LIMIT;
  if (S * d->I * 2 >= (1ll << 31) || (int64_t)d->T * d->H >= (1ll << 31)) return QRE_ERR_LIMIT;
  if ((int64_t)d->H * d->I >= (1ll << 31)) return QRE_ERR_LIMIT;
  const int bm = fp4_tile_rows(S, d->E);
  if (fp4_gemm_lds_bytes(bm, d->H) > kFp4MaxLds) return QRE_ERR_LIMIT;   // the staged rows of x fit in LDS
  if (max_tiles(S, d->E, bm) > 65535) return QRE_ERR_LIMIT;              // grid.y
  return QRE_OK;
}

int check_nvfp4_weights(const qre_nvfp4_weights* w, bool gate_up, bool down) {
  if (!w) return QRE_ERR_NULL;
  auto ok = [](const qre_nvfp4_matrix& m) { return m.q && m.s && m.outer; };
  auto al = [](const qre_nvfp4_matrix& m) { return aligned16(m.q) && aligned16(m.s) && aligned4(m.outer); };
  if ((gate_up && (!ok(w->gate) || !ok(w->up))) || (down && !ok(w->down))) return QRE_ERR_NULL;
  if ((gate_up && (!al(w->gate) || !al(w->up))) || (down && !al(w->down))) return QRE_ERR_ALIGN;
  return QRE_OK;
}

// Stage scratch: the header, both tile lists and the routing scratch.
struct Fp4Stage {
  int32_t* header;
  int32_t* ntiles;            // [2]: gate/up, down
  Tile *tiles_gu, *tiles_dn;
  void* route_scratch;
  int bm;
  int64_t mt;
};

void carve_fp4_stage(const qre_desc& d, Carver& c, Fp4Stage& L) {
  const int64_t S = (int64_t)d.T * d.K;
  L.bm = fp4_tile_rows(S, d.E);
  L.mt = max_tiles(S, d.E, L.bm);
  L.header = c.take<int32_t>(kHeaderInts);
  L.ntiles = c.take<int32_t>(2);
  L.tiles_gu = c.take<Tile>(L.mt);
  L.tiles_dn = c.take<Tile>(L.mt);
  L.route_scratch = c.take<uint8_t>(route_scratch_bytes(S, d.E));
}

struct Fp4Layout {
  Fp4Stage st;
  int32_t *counts, *offsets, *sorted_slot, *slot_row;
  uint8_t *xq, *xb; float* xr;   // x quantized: codes, block scales, row scales
  uint16_t* h;                   // bf16 [S][I]
  uint8_t *hq, *hb; float* hr;   // h quantized
  uint16_t* y;                   // bf16 [S][H]
  size_t bytes;
};

Fp4Layout make_fp4_layout(const qre_desc& d, void* ws) {
  Fp4Layout L;
  const int64_t S = (int64_t)d.T * d.K;
  Carver c(ws);
  carve_fp4_stage(d, c, L.st);
  L.counts = c.take<int32_t>(d.E);
  L.offsets = c.take<int32_t>(d.E + 1);
  L.sorted_slot = c.take<int32_t>(S);
  L.slot_row = c.take<int32_t>(S);
  L.xq = c.take<uint8_t>((size_t)d.T * d.H / 2);
  L.xb = c.take<uint8_t>((size_t)d.T * d.H / QRE_NVFP4_BLOCK);
  L.xr = c.take<float>((size_t)d.T);
  L.h = c.take<uint16_t>((size_t)S * d.I);
  L.hq = c.take<uint8_t>((size_t)S * d.I / 2);
  L.hb = c.take<uint8_t>((size_t)S * d.I / QRE_NVFP4_BLOCK);
  L.hr = c.take<float>((size_t)S);
  L.y = c.take<uint16_t>((size_t)S * d.H);
  L.bytes = c.off;
  return L;
}

Fp4Problem fp4_gate_up_problem(const qre_desc& d, const void* xq, const void* xb, const float* xr,
                               const int32_t* sorted_slot, const qre_nvfp4_weights& w, const Fp4Stage& st, void* h) {
  Fp4Problem p;
  p.aq = static_cast<const uint8_t*>(xq);
  p.ab = static_cast<const uint8_t*>(xb);
  p.ar = xr;
  p.a_rows = d.T;
  p.gather_k = d.K;
  p.sorted_slot = sorted_slot;
  p.w0q = static_cast<const uint8_t*>(w.gate.q); p.w0b = static_cast<const uint8_t*>(w.gate.s); p.w0o = w.gate.outer;
  p.w1q = static_cast<const uint8_t*>(w.up.q);   p.w1b = static_cast<const uint8_t*>(w.up.s);   p.w1o = w.up.outer;
  p.tiles = st.tiles_gu; p.ntiles = st.ntiles; p.max_tiles = st.mt; p.bm = st.bm;
  p.out = static_cast<uint16_t*>(h);
  p.n = d.I;
  p.kdim = d.H;
  return p;
}

Fp4Problem fp4_down_problem(const qre_desc& d, const void* hq, const void* hb, const float* hr,
                            const qre_nvfp4_weights& w, const Fp4Stage& st, void* y) {
  Fp4Problem p;
  p.aq = static_cast<const uint8_t*>(hq);
  p.ab = static_cast<const uint8_t*>(hb);
  p.ar = hr;
  p.a_rows = (int64_t)d.T * d.K;
  p.gather_k = 0;
  p.sorted_slot = nullptr;
  p.w0q = static_cast<const uint8_t*>(w.down.q); p.w0b = static_cast<const uint8_t*>(w.down.s); p.w0o = w.down.outer;
  p.w1q = nullptr; p.w1b = nullptr; p.w1o = nullptr;
  p.tiles = st.tiles_dn; p.ntiles = st.ntiles + 1; p.max_tiles = st.mt; p.bm = st.bm;
  p.out = static_cast<uint16_t*>(y);
  p.n = d.H;
  p.kdim = d.I;
  return p;
}

}  // namespace

extern "C" {

const char* qre_status_string(int s) {
  switch (s) {
    case QRE_OK: return "ok";
    case QRE_ERR_NULL: return "null pointer";
    case QRE_ERR_SHAPE: return "bad shape";
    case QRE_ERR_BITS: return "weight_bits must be 4 or 8";
    case QRE_ERR_GROUP: return "group_size must be 128";
    case QRE_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case QRE_ERR_WORKSPACE: return "workspace too small";
    case QRE_ERR_HIP: return "HIP error";
    case QRE_ERR_MODE: return "bad act_int8 mode or missing mode argument";
    case QRE_ERR_LIMIT: return "size exceeds a library limit";
    default: return "unknown status";
  }
}

int qre_last_hip_error(void) { return g_last_hip_error; }

int qre_workspace_bytes(const qre_desc* desc, size_t* bytes) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!bytes) return QRE_ERR_NULL;
  *bytes = make_layout(*desc, nullptr).bytes;
  return QRE_OK;
}

int qre_stage_workspace_bytes(const qre_desc* desc, size_t* bytes) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!bytes) return QRE_ERR_NULL;
  *bytes = stage_bytes(*desc);
  return QRE_OK;
}

static int moe_forward_impl(const qre_desc* desc, const void* x, const int32_t* topk_ids, const float* topk_w,
                            const qre_weights* weights, void* out, void* workspace, size_t workspace_bytes,
                            hipEvent_t const* ev, hipStream_t s) {
  int rc = check_desc(desc);
  if (rc) return rc;
  const qre_desc& d = *desc;
  if (d.T == 0) return QRE_OK;
  if (!x || !topk_ids || !topk_w || !out || !workspace) return QRE_ERR_NULL;
  rc = check_weights(weights, true, true);
  if (rc) return rc;
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(out) || !aligned16(workspace))
    return QRE_ERR_ALIGN;
  const Layout L = make_layout(d, workspace);
  if (workspace_bytes < L.bytes) return QRE_ERR_WORKSPACE;
  const int64_t S = (int64_t)d.T * d.K;
  const StageLayout& st = L.st;
  auto mark = [&](int i) -> hipError_t { return (ev && ev[i]) ? hipEventRecord(ev[i], s) : hipSuccess; };

  GemmProblem gu = gate_up_problem(d, x, L.xq, L.xs, L.sorted_slot, *weights, st.tiles_gu, st.ntiles, st.mt_gu,
                                   st.bm_gu, L.h);
  // INT8 mode with 128-output gate/up workgroups: h leaves the gate/up kernel
  // already quantized (no BF16 h, no quantizer launch)
  const bool fused_hq = d.act_int8 && gate_up_quantizes_h(gu);
  if (fused_hq) {
    gu.hq = L.hq;
    gu.hs = L.hs;
    gu.out = nullptr;
  }
  const GemmProblem dn = down_problem(d, L.h, L.hq, L.hs, *weights, st.tiles_dn, st.ntiles + 1, st.mt_dn, st.bm_dn,
                                      L.y);
  // Decode-sized problems: the permutation is folded into the gate/up kernel;
  // otherwise the routing kernel builds it (and the row-tile lists).
  const bool routed = routed_applicable(S, d.E, d.H, d.I, d.act_int8);
  const RouteOut ro = {topk_ids, (int)S, d.E, L.counts, L.offsets, L.sorted_slot, L.slot_row, st.header};
  hipError_t e = mark(0);
  // INT8 mode: the quantization of x rides on the routing launches when there
  // are any (it shares the last of the three large-problem kernels)
  const QuantX qx = {static_cast<const uint16_t*>(x), d.T, d.H, L.xq, L.xs};
  if (e == hipSuccess && !routed)
    e = launch_route(topk_ids, d.T, d.K, d.E, L.counts, L.offsets, L.sorted_slot, L.slot_row, st.header,
                     st.route_scratch, st.tiles_gu, st.ntiles, st.bm_gu, st.tiles_dn, st.ntiles + 1, st.bm_dn, s,
                     d.act_int8 ? &qx : nullptr);
  if (e == hipSuccess && d.act_int8 && routed) e = launch_quantize_act(qx.v, qx.rows, qx.cols, qx.q, qx.s, s);
  if (e == hipSuccess) e = mark(1);
  if (ev) kernel_events() = KernelEvents{ev[6], ev[7]};   // the gate/up kernel's own begin and end
  if (e == hipSuccess) e = routed ? launch_gate_up_routed(gu, ro, s) : launch_gemm(gu, s);
  kernel_events() = KernelEvents{nullptr, nullptr};
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess && d.act_int8 && !fused_hq) e = launch_quantize_act(L.h, (int)S, d.I, L.hq, L.hs, s);
  if (e == hipSuccess) e = mark(3);
  if (e == hipSuccess) e = routed ? launch_down_routed(dn, ro, s) : launch_gemm(dn, s);
  if (e == hipSuccess) e = mark(4);
  if (e == hipSuccess) e = launch_combine(L.y, L.slot_row, topk_w, d.T, d.K, d.H, static_cast<uint16_t*>(out), s);
  if (e == hipSuccess) e = mark(5);
  return hip_status(e);
}

int qre_moe_forward(const qre_desc* desc, const void* x, const int32_t* topk_ids, const float* topk_w,
                    const qre_weights* weights, void* out, void* workspace, size_t workspace_bytes,
                    qre_stream_t stream) {
  return moe_forward_impl(desc, x, topk_ids, topk_w, weights, out, workspace, workspace_bytes, nullptr,
                          reinterpret_cast<hipStream_t>(stream));
}

int qre_moe_forward_noalloc(const qre_desc* desc, const void* x, const int32_t* topk_ids, const float* topk_w,
                            const qre_weights* weights, void* out, qre_stream_t stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (make_layout(*desc, nullptr).bytes > QRE_NOALLOC_SCRATCH_BYTES) return QRE_ERR_LIMIT;
  if (desc->T == 0) return QRE_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return QRE_ERR_LIMIT;
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  return moe_forward_impl(desc, x, topk_ids, topk_w, weights, out, ws, QRE_NOALLOC_SCRATCH_BYTES, nullptr,
                          reinterpret_cast<hipStream_t>(stream));
}

int qre_moe_forward_timed(const qre_desc* desc, const void* x, const int32_t* topk_ids, const float* topk_w,
                          const qre_weights* weights, void* out, void* workspace, size_t workspace_bytes,
                          void* const* events, qre_stream_t stream) {
  if (!events) return QRE_ERR_NULL;
  return moe_forward_impl(desc, x, topk_ids, topk_w, weights, out, workspace, workspace_bytes,
                          reinterpret_cast<hipEvent_t const*>(events), reinterpret_cast<hipStream_t>(stream));
}

int qre_workspace_permutation(const qre_desc* desc, void* workspace, int32_t** counts, int32_t** offsets,
                              int32_t** sorted_slot, int32_t** slot_row) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!workspace || !counts || !offsets || !sorted_slot || !slot_row) return QRE_ERR_NULL;
  const Layout L = make_layout(*desc, workspace);
  *counts = L.counts;
  *offsets = L.offsets;
  *sorted_slot = L.sorted_slot;
  *slot_row = L.slot_row;
  return QRE_OK;
}

int qre_read_device_error(const void* workspace, int32_t* n_bad_ids, qre_stream_t stream) {
  if (!workspace || !n_bad_ids) return QRE_ERR_NULL;
  if (!aligned16(workspace)) return QRE_ERR_ALIGN;
  int32_t n = 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&n, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e);
  *n_bad_ids = n;
  return QRE_OK;
}

static int check_stage_ws(const qre_desc& d, const void* workspace, size_t workspace_bytes) {
  if (!workspace) return QRE_ERR_NULL;
  if (!aligned16(workspace)) return QRE_ERR_ALIGN;
  if (workspace_bytes < stage_bytes(d)) return QRE_ERR_WORKSPACE;
  return QRE_OK;
}

int qre_route_workspace_bytes(int32_t T, int32_t K, int32_t E, size_t* bytes) {
  if (!bytes) return QRE_ERR_NULL;
  if (T < 0 || K <= 0 || E <= 0 || K > E) return QRE_ERR_SHAPE;
  if (E > QRE_MAX_EXPERTS || (int64_t)T * K >= (1ll << 31)) return QRE_ERR_LIMIT;
  *bytes = route_bytes((int64_t)T * K, E);
  return QRE_OK;
}

int qre_route(const int32_t* topk_ids, int32_t T, int32_t K, int32_t E, int32_t* counts, int32_t* offsets,
              int32_t* sorted_slot, int32_t* slot_row, void* workspace, size_t workspace_bytes,
              qre_stream_t stream) {
  size_t need = 0;
  int rc = qre_route_workspace_bytes(T, K, E, &need);
  if (rc) return rc;
  if (!counts || !offsets || !workspace) return QRE_ERR_NULL;
  if (!aligned16(counts) || !aligned16(offsets) || !aligned16(workspace)) return QRE_ERR_ALIGN;
  const int64_t S = (int64_t)T * K;
  if (S > 0) {
    if (!topk_ids || !sorted_slot || !slot_row) return QRE_ERR_NULL;
    if (!aligned16(topk_ids) || !aligned16(sorted_slot) || !aligned16(slot_row)) return QRE_ERR_ALIGN;
  }
  if (workspace_bytes < need) return QRE_ERR_WORKSPACE;
  int32_t* header = static_cast<int32_t*>(workspace);
  void* scratch = static_cast<uint8_t*>(workspace) + kHeaderInts * sizeof(int32_t);
  return hip_status(launch_route(topk_ids, T, K, E, counts, offsets, sorted_slot, slot_row, header, scratch,
                                 nullptr, nullptr, 0, nullptr, nullptr, 0, reinterpret_cast<hipStream_t>(stream)));
}

int qre_quantize_act(const void* v, int32_t rows, int32_t cols, int8_t* q, float* s, qre_stream_t stream) {
  if (rows < 0 || cols <= 0 || cols % QRE_GROUP) return QRE_ERR_SHAPE;
  if ((int64_t)rows * cols >= (1ll << 40)) return QRE_ERR_LIMIT;
  if (rows == 0) return QRE_OK;
  if (!v || !q || !s) return QRE_ERR_NULL;
  if (!aligned16(v) || !aligned16(q) || !aligned16(s)) return QRE_ERR_ALIGN;
  return hip_status(launch_quantize_act(static_cast<const uint16_t*>(v), rows, cols, q, s,
                                        reinterpret_cast<hipStream_t>(stream)));
}

int qre_quantize_weights(const float* w, int64_t rows, int64_t cols, int32_t bits, void* q, void* s,
                         qre_stream_t stream) {
  if (bits != 4 && bits != 8) return QRE_ERR_BITS;
  if (rows < 0 || cols <= 0 || cols % QRE_GROUP) return QRE_ERR_SHAPE;
  if (rows * (cols / QRE_GROUP) >= (1ll << 40)) return QRE_ERR_LIMIT;
  if (rows == 0) return QRE_OK;
  if (!w || !q || !s) return QRE_ERR_NULL;
  if (!aligned16(w) || !aligned16(q) || !aligned16(s)) return QRE_ERR_ALIGN;
  return hip_status(launch_quantize_weights(w, rows, cols, bits, static_cast<uint8_t*>(q),
                                            static_cast<uint16_t*>(s), reinterpret_cast<hipStream_t>(stream)));
}

int qre_gate_up(const qre_desc* desc, const void* x, const int8_t* xq, const float* xs, const int32_t* sorted_slot,
                const int32_t* offsets, const qre_weights* weights, void* h, int8_t* hq, float* hs, void* workspace,
                size_t workspace_bytes, qre_stream_t stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  const qre_desc& d = *desc;
  if (d.T == 0) return QRE_OK;
  rc = check_stage_ws(d, workspace, workspace_bytes);
  if (rc) return rc;
  if (d.act_int8 ? (!xq || !xs) : !x) return QRE_ERR_MODE;
  if (!d.act_int8 && (hq || hs)) return QRE_ERR_MODE;
  if (d.act_int8 && ((hq == nullptr) != (hs == nullptr))) return QRE_ERR_MODE;
  if (!sorted_slot || !offsets) return QRE_ERR_NULL;
  if (!h && !hq) return QRE_ERR_NULL;
  rc = check_weights(weights, true, false);
  if (rc) return rc;
  if (!aligned16(d.act_int8 ? (const void*)xq : x) || (d.act_int8 && !aligned16(xs)) || !aligned16(sorted_slot) ||
      !aligned16(offsets) || (h && !aligned16(h)) || (hq && (!aligned16(hq) || !aligned16(hs))))
    return QRE_ERR_ALIGN;
  const StageLayout st = stage_layout(d, workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  GemmProblem p = gate_up_problem(d, x, xq, xs, sorted_slot, *weights, st.tiles_gu, st.ntiles, st.mt_gu, st.bm_gu,
                                  h ? h : st.h_tmp);
  const bool fused_hq = hq && gate_up_quantizes_h(p);   // h quantized in the gate/up epilogue
  if (fused_hq) {
    p.hq = hq;
    p.hs = hs;
    p.out = h;
  }
  hipError_t e = launch_build_tiles(offsets, d.E, st.tiles_gu, st.ntiles, st.bm_gu, nullptr, nullptr, 0, s);
  if (e == hipSuccess) e = launch_gemm(p, s);
  if (e == hipSuccess && hq && !fused_hq)
    e = launch_quantize_act(static_cast<const uint16_t*>(p.out), (int)((int64_t)d.T * d.K), d.I, hq, hs, s);
  return hip_status(e);
}

int qre_down(const qre_desc* desc, const void* h, const int8_t* hq, const float* hs, const int32_t* offsets,
             const qre_weights* weights, void* y, void* workspace, size_t workspace_bytes, qre_stream_t stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  const qre_desc& d = *desc;
  if (d.T == 0) return QRE_OK;
  rc = check_stage_ws(d, workspace, workspace_bytes);
  if (rc) return rc;
  if (d.act_int8 ? (!hq || !hs) : !h) return QRE_ERR_MODE;
  if (!y || !offsets) return QRE_ERR_NULL;
  rc = check_weights(weights, false, true);
  if (rc) return rc;
  if (!aligned16(d.act_int8 ? (const void*)hq : h) || (d.act_int8 && !aligned16(hs)) || !aligned16(y) ||
      !aligned16(offsets))
    return QRE_ERR_ALIGN;
  const StageLayout st = stage_layout(d, workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_build_tiles(offsets, d.E, st.tiles_dn, st.ntiles + 1, st.bm_dn, nullptr, nullptr, 0, s);
  if (e == hipSuccess)
    e = launch_gemm(down_problem(d, h, hq, hs, *weights, st.tiles_dn, st.ntiles + 1, st.mt_dn, st.bm_dn, y), s);
  return hip_status(e);
}

int qre_combine(const void* y, const int32_t* slot_row, const float* topk_w, int32_t T, int32_t K, int32_t H,
                void* out, qre_stream_t stream) {
  if (T < 0 || K <= 0 || H <= 0 || H % QRE_GROUP) return QRE_ERR_SHAPE;
  if ((int64_t)T * K >= (1ll << 31)) return QRE_ERR_LIMIT;
  if (T == 0) return QRE_OK;
  if (!y || !slot_row || !topk_w || !out) return QRE_ERR_NULL;
  if (!aligned16(y) || !aligned16(slot_row) || !aligned16(topk_w) || !aligned16(out)) return QRE_ERR_ALIGN;
  return hip_status(launch_combine(static_cast<const uint16_t*>(y), slot_row, topk_w, T, K, H,
                                   static_cast<uint16_t*>(out), reinterpret_cast<hipStream_t>(stream)));
}

int qre_topk_softmax(const float* logits, int32_t T, int32_t E, int32_t K, int32_t* topk_ids, float* topk_w,
                     qre_stream_t stream) {
  if (T < 0 || E < 1 || K < 1 || K > E) return QRE_ERR_SHAPE;
  if (E > QRE_ROUTER_MAX_EXPERTS || K > QRE_ROUTER_MAX_K || (int64_t)T * E >= (1ll << 31)) return QRE_ERR_LIMIT;
  if (T == 0) return QRE_OK;
  if (!logits || !topk_ids || !topk_w) return QRE_ERR_NULL;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return QRE_ERR_ALIGN;
  return hip_status(launch_topk_softmax(logits, T, E, K, topk_ids, topk_w, reinterpret_cast<hipStream_t>(stream)));
}

int qre_forward_plan(const qre_desc* desc, int32_t* plan) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!plan) return QRE_ERR_NULL;
  const qre_desc& d = *desc;
  const int64_t S = (int64_t)d.T * d.K;
  int32_t f = 0;
  if (routed_applicable(S, d.E, d.H, d.I, d.act_int8)) f |= QRE_PLAN_ROUTE_IN_GATE_UP;
  if (big_applicable(S, d.E, d.H)) f |= QRE_PLAN_BIG_TILES;
  *plan = f;
  return QRE_OK;
}

int qre_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, qre_stream_t stream) {
  if (!buf || !sink) return QRE_ERR_NULL;
  if (!aligned16(buf) || !aligned16(sink)) return QRE_ERR_ALIGN;
  if (bytes == 0 || bytes % 16) return QRE_ERR_SHAPE;
  return hip_status(launch_hbm_read(buf, (int64_t)bytes, sink, reinterpret_cast<hipStream_t>(stream)));
}

int qre_nvfp4_quantize_weights(const float* w, int64_t mats, int64_t rows, int64_t cols, void* q, void* s,
                               float* outer, qre_stream_t stream) {
  if (mats < 0 || rows < 0 || cols <= 0 || cols % QRE_NVFP4_BLOCK) return QRE_ERR_SHAPE;
  if (mats * rows * (cols / QRE_NVFP4_BLOCK) >= (1ll << 40)) return QRE_ERR_LIMIT;
  if (mats == 0 || rows == 0) return QRE_OK;
  if (!w || !q || !s || !outer) return QRE_ERR_NULL;
  if (!aligned16(w) || !aligned16(q) || !aligned16(s) || !aligned4(outer)) return QRE_ERR_ALIGN;
  return hip_status(launch_fp4_quantize_weights(w, mats, rows, cols, static_cast<uint8_t*>(q),
                                                static_cast<uint8_t*>(s), outer, reinterpret_cast<hipStream_t>(stream)));
}

int qre_nvfp4_quantize_act(const void* v, int32_t rows, int32_t cols, void* q, void* s, float* row_scale,
                           qre_stream_t stream) {
  if (rows < 0 || cols <= 0 || cols % QRE_NVFP4_BLOCK) return QRE_ERR_SHAPE;
  if ((int64_t)rows * cols >= (1ll << 40)) return QRE_ERR_LIMIT;
  if (rows == 0) return QRE_OK;
  if (!v || !q || !s || !row_scale) return QRE_ERR_NULL;
  if (!aligned16(v) || !aligned16(q) || !aligned16(s) || !aligned16(row_scale)) return QRE_ERR_ALIGN;
  return hip_status(launch_fp4_quantize_act(static_cast<const uint16_t*>(v), rows, cols, static_cast<uint8_t*>(q),
                                            static_cast<uint8_t*>(s), row_scale,
                                            reinterpret_cast<hipStream_t>(stream)));
}

int qre_nvfp4_workspace_bytes(const qre_desc* desc, size_t* bytes) {
  int rc = check_nvfp4_desc(desc);
  if (rc) return rc;
  if (!bytes) return QRE_ERR_NULL;
  *bytes = make_fp4_layout(*desc, nullptr).bytes;
  return QRE_OK;
}

int qre_nvfp4_stage_workspace_bytes(const qre_desc* desc, size_t* bytes) {
  int rc = check_nvfp4_desc(desc);
  if (rc) return rc;
  if (!bytes) return QRE_ERR_NULL;
  Carver c(nullptr);
  Fp4Stage L;
  carve_fp4_stage(*desc, c, L);
  *bytes = c.off;
  return QRE_OK;
}

static int nvfp4_forward_impl(const qre_desc* desc, const void* x, const int32_t* topk_ids, const float* topk_w,
                              const qre_nvfp4_weights* weights, void* out, void* workspace, size_t workspace_bytes,
                              hipEvent_t const* ev, hipStream_t s) {
  int rc = check_nvfp4_desc(desc);
  if (rc) return rc;
  const qre_desc& d = *desc;
  if (d.T == 0) return QRE_OK;
  if (!x || !topk_ids || !topk_w || !out || !workspace) return QRE_ERR_NULL;
  rc = check_nvfp4_weights(weights, true, true);
  if (rc) return rc;
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(out) || !aligned16(workspace))
    return QRE_ERR_ALIGN;
  const Fp4Layout L = make_fp4_layout(d, workspace);
  if (workspace_bytes < L.bytes) return QRE_ERR_WORKSPACE;
  const int64_t S = (int64_t)d.T * d.K;
  const Fp4Stage& st = L.st;
  auto mark = [&](int i) -> hipError_t { return (ev && ev[i]) ? hipEventRecord(ev[i], s) : hipSuccess; };
  hipError_t e = mark(0);
  if (S <= kRouteQuantMaxSlots) {   // decode blocks: routing and the quantization of x in one launch
    const RouteArgs ra = {topk_ids, (int)S, d.E, 0, L.counts, L.offsets, L.sorted_slot, L.slot_row, st.header,
                          st.tiles_gu, st.ntiles, st.bm, st.tiles_dn, st.ntiles + 1, st.bm};
    if (e == hipSuccess)
      e = launch_fp4_route_quantize_x(ra, static_cast<const uint16_t*>(x), d.T, d.H, L.xq, L.xb, L.xr, s);
  } else {
    if (e == hipSuccess)
      e = launch_route(topk_ids, d.T, d.K, d.E, L.counts, L.offsets, L.sorted_slot, L.slot_row, st.header,
                       st.route_scratch, st.tiles_gu, st.ntiles, st.bm, st.tiles_dn, st.ntiles + 1, st.bm, s);
    if (e == hipSuccess) e = launch_fp4_quantize_act(static_cast<const uint16_t*>(x), d.T, d.H, L.xq, L.xb, L.xr, s);
  }
  if (e == hipSuccess) e = mark(1);
  if (ev) kernel_events() = KernelEvents{ev[6], ev[7]};   // the gate/up kernel's own begin and end
  if (e == hipSuccess)
    e = launch_fp4_gemm(fp4_gate_up_problem(d, L.xq, L.xb, L.xr, L.sorted_slot, *weights, st, L.h), s);
  kernel_events() = KernelEvents{nullptr, nullptr};
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess) e = launch_fp4_quantize_act(L.h, S, d.I, L.hq, L.hb, L.hr, s);
  if (e == hipSuccess) e = mark(3);
  if (e == hipSuccess) e = launch_fp4_gemm(fp4_down_problem(d, L.hq, L.hb, L.hr, *weights, st, L.y), s);
  if (e == hipSuccess) e = mark(4);
  if (e == hipSuccess) e = launch_combine(L.y, L.slot_row, topk_w, d.T, d.K, d.H, static_cast<uint16_t*>(out), s);
  if (e == hipSuccess) e = mark(5);
  return hip_status(e);
}

int qre_nvfp4_moe_forward(const qre_desc* desc, const void* x, const int32_t* topk_ids, const float* topk_w,
                          const qre_nvfp4_weights* weights, void* out, void* workspace, size_t workspace_bytes,
                          qre_stream_t stream) {
  return nvfp4_forward_impl(desc, x, topk_ids, topk_w, weights, out, workspace, workspace_bytes, nullptr,
                            reinterpret_cast<hipStream_t>(stream));
}

int qre_nvfp4_moe_forward_timed(const qre_desc* desc, const void* x, const int32_t* topk_ids, const float* topk_w,
                                const qre_nvfp4_weights* weights, void* out, void* workspace, size_t workspace_bytes,
                                void* const* events, qre_stream_t stream) {
  if (!events) return QRE_ERR_NULL;
  return nvfp4_forward_impl(desc, x, topk_ids, topk_w, weights, out, workspace, workspace_bytes,
                            reinterpret_cast<hipEvent_t const*>(events), reinterpret_cast<hipStream_t>(stream));
}

int qre_nvfp4_workspace_permutation(const qre_desc* desc, void* workspace, int32_t** counts, int32_t** offsets,
                                    int32_t** sorted_slot, int32_t** slot_row) {
  int rc = check_nvfp4_desc(desc);
  if (rc) return rc;
  if (!workspace || !counts || !offsets || !sorted_slot || !slot_row) return QRE_ERR_NULL;
  const Fp4Layout L = make_fp4_layout(*desc, workspace);
  *counts = L.counts;
  *offsets = L.offsets;
  *sorted_slot = L.sorted_slot;
  *slot_row = L.slot_row;
  return QRE_OK;
}

static int check_fp4_stage_ws(const qre_desc& d, const void* workspace, size_t workspace_bytes, Fp4Stage& st) {
  if (!workspace) return QRE_ERR_NULL;
  if (!aligned16(workspace)) return QRE_ERR_ALIGN;
  Carver c(const_cast<void*>(workspace));
  carve_fp4_stage(d, c, st);
  if (workspace_bytes < c.off) return QRE_ERR_WORKSPACE;
  return QRE_OK;
}

int qre_nvfp4_gate_up(const qre_desc* desc, const void* xq, const void* xs, const float* xr, const int32_t* sorted_slot,
                      const int32_t* offsets, const qre_nvfp4_weights* weights, void* h, void* workspace,
                      size_t workspace_bytes, qre_stream_t stream) {
  int rc = check_nvfp4_desc(desc);
  if (rc) return rc;
  const qre_desc& d = *desc;
  if (d.T == 0) return QRE_OK;
  Fp4Stage st;
  rc = check_fp4_stage_ws(d, workspace, workspace_bytes, st);
  if (rc) return rc;
  if (!xq || !xs || !xr || !sorted_slot || !offsets || !h) return QRE_ERR_NULL;
  rc = check_nvfp4_weights(weights, true, false);
  if (rc) return rc;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(xr) || !aligned16(sorted_slot) || !aligned16(offsets) ||
      !aligned16(h))
    return QRE_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_build_tiles(offsets, d.E, st.tiles_gu, st.ntiles, st.bm, nullptr, nullptr, 0, s);
  if (e == hipSuccess) e = launch_fp4_gemm(fp4_gate_up_problem(d, xq, xs, xr, sorted_slot, *weights, st, h), s);
  return hip_status(e);
}

int qre_nvfp4_down(const qre_desc* desc, const void* hq, const void* hs, const float* hr, const int32_t* offsets,
                   const qre_nvfp4_weights* weights, void* y, void* workspace, size_t workspace_bytes,
                   qre_stream_t stream) {
  int rc = check_nvfp4_desc(desc);
  if (rc) return rc;
  const qre_desc& d = *desc;
  if (d.T == 0) return QRE_OK;
  Fp4Stage st;
  rc = check_fp4_stage_ws(d, workspace, workspace_bytes, st);
  if (rc) return rc;
  if (!hq || !hs || !hr || !offsets || !y) return QRE_ERR_NULL;
  rc = check_nvfp4_weights(weights, false, true);
  if (rc) return rc;
  if (!aligned16(hq) || !aligned16(hs) || !aligned16(hr) || !aligned16(offsets) || !aligned16(y)) return QRE_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_build_tiles(offsets, d.E, st.tiles_dn, st.ntiles + 1, st.bm, nullptr, nullptr, 0, s);
  if (e == hipSuccess) e = launch_fp4_gemm(fp4_down_problem(d, hq, hs, hr, *weights, st, y), s);
  return hip_status(e);
}

}  // extern "C"
