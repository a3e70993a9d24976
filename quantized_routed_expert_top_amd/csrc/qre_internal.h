// Internal declarations of the gfx950 kernels behind include/qre.h.
//
// Device helpers and the launchers each kernel file exports to the host-side
// entry points (qre_api.hip).  Everything here is HIP C++ for CDNA4: wave64,
// MFMA, LDS.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qre {

constexpr int kGroup = 128;      // quantization group along the reduction dim
constexpr int kWave = 64;

// Tile of sorted rows processed by one GEMM workgroup: rows [row0, row0+nrows) of expert e.
struct Tile {
  int32_t e, row0, nrows, pad;
};

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Nearest-even rounding of an FP32 value to BF16 bits (quiet NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// v_perm_b32: byte i of the result is byte sel.byte[i] of the 8-byte value {hi, lo}.
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Maximum over the 16 lanes of an aligned 16-lane segment.
__device__ __forceinline__ float seg16_max(float m) {
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 16));
  return m;
}

// INT8 activation code of x for the group scale sc != 0 (r = 1 / sc, rounded
// to FP32): q = clamp(rint(x / sc), -127, 127) with x / sc rounded to FP32
// first, as defined (model card, paragraph on --int8-expert-activations).
// Fast form: y = x * r; both roundings keep |y - x / sc| <= 3 * 2^-24 *
// |x / sc| <= 2.3e-5 for |x / sc| <= 127, and the FP32 quotient is as close,
// so when y is more than 2^-14 from every half-integer rint(y) is the rint of
// the quotient.  Otherwise (rare), and for non-finite y (a subnormal scale
// whose reciprocal overflows), the quotient itself is taken.
__device__ __forceinline__ float act_code(float x, float sc, float r) {
  constexpr float kMargin = 0x1p-14f;
  const float y = x * r;
  float qf = rintf(y);
  if (!(fabsf(y - qf) <= 0.5f - kMargin)) qf = rintf(x / sc);
  return fminf(127.0f, fmaxf(-127.0f, qf));
}

// ---------------------------------------------------------------------------
// Launchers (all enqueue on `stream` and return the launch status)
// ---------------------------------------------------------------------------

// Routing.  The small variant runs in one workgroup and fuses the tile-list
// build for up to two GEMM row-tile heights; the large variant is three kernels.
// `ws` (route scratch) must hold route_scratch_bytes(S, E) bytes.
size_t route_scratch_bytes(int64_t S, int E);
// `dropped` (may be null) receives S - offsets[E], the slots whose id was
// outside [0, E).  Either tile list may be null.  With qx, the INT8
// quantization of x [rows][cols] is enqueued too (in the three-kernel path
// it shares the last routing launch).
struct QuantX {
  const uint16_t* v;
  int rows, cols;
  int8_t* q;
  float* s;
};
hipError_t launch_route(const int32_t* ids, int T, int K, int E, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_slot, int32_t* slot_row, int32_t* dropped, void* ws, Tile* tiles_a,
                        int32_t* ntiles_a, int bm_a, Tile* tiles_b, int32_t* ntiles_b, int bm_b, hipStream_t stream,
                        const QuantX* qx = nullptr);
// Tile list from offsets alone (used by the stage entry points); tiles_b may be null.
hipError_t launch_build_tiles(const int32_t* offsets, int E, Tile* tiles_a, int32_t* ntiles_a, int bm_a,
                              Tile* tiles_b, int32_t* ntiles_b, int bm_b, hipStream_t stream);
// Arguments of the one-workgroup routing when another kernel runs it.
struct RouteArgs {
  const int32_t* ids;
  int S, E, nbits;
  int32_t *counts, *offsets, *sorted_slot, *slot_row, *dropped;
  Tile* tiles_a;
  int32_t* ntiles_a;
  int bm_a;
  Tile* tiles_b;
  int32_t* ntiles_b;
  int bm_b;
};
// Upper bound on the number of row tiles of height bm over S sorted rows and E experts.
int64_t max_tiles(int64_t S, int E, int bm);

// INT8 quantizers.
hipError_t launch_quantize_act(const uint16_t* v, int rows, int cols, int8_t* q, float* s, hipStream_t stream);
hipError_t launch_quantize_weights(const float* w, int64_t rows, int64_t cols, int bits, uint8_t* q,
                                   uint16_t* s, hipStream_t stream);

// Grouped GEMMs.
struct GemmProblem {
  int act_int8;           // 0: bf16 activations, 1: int8 activations + fp32 scales
  int bits;               // 4 or 8
  int gather_k;           // >0: A row of sorted row r is token sorted_slot[r] / gather_k; 0: A row = r
  const int32_t* sorted_slot;
  const void* a;          // bf16 [a_rows][kdim] or int8 [a_rows][kdim]
  const float* a_scale;   // int8 mode: fp32 [a_rows][kdim/128]
  int64_t a_rows;         // rows of the A source (T for gathered x, S for h)
  const uint8_t* w0q; const uint16_t* w0s;   // [E][n][kdim*bits/8], [E][n][kdim/128]
  const uint8_t* w1q; const uint16_t* w1s;   // second matrix (gate/up: up), or null
  const Tile* tiles; const int32_t* ntiles; int64_t max_tiles; int bm;
  void* out;              // bf16 [S][n] (may be null when hq is given)
  int n, kdim;
  int8_t* hq = nullptr;   // fused gate/up, INT8 mode: h quantized per 128 values,
  float* hs = nullptr;    // int8 [S][n] and fp32 [S][n/128] (gate_up_quantizes_h)
};
// Fused gate/up + SiLU*mul (w1 = up) or plain projection (w1 = null).
hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream);
// Row-tile height the GEMM wants for a problem with S sorted rows over E experts.
int gemm_tile_rows(int64_t S, int E, int n, int kdim, int act_int8);
// Many rows per expert: the MFMA-bound kernels of gemm_big.hip, with tiles of
// big_tile_rows(act_int8) rows (64 with BF16 activations, 128 with INT8
// ones), used by launch_gemm for problems whose tile height is 64 or more.
bool big_applicable(int64_t S, int E, int kdim);
int big_tile_rows(int act_int8);
// Whether the 128-row gate/up kernel for p quantizes h itself (p.hq, p.hs):
// INT8 weights and activations, 128 outputs per workgroup.
bool gate_up_quantizes_h(const GemmProblem& p);
hipError_t launch_gemm_big(const GemmProblem& p, hipStream_t stream);

// Decode-sized problems (up to kRoutedMaxSlots slots): the gate/up kernel
// computes the permutation itself (writing counts, offsets, sorted_slot and
// slot_row) and the down kernel reads counts/offsets back; no tile list.
struct RouteOut {
  const int32_t* ids;
  int S, E;
  int32_t *counts, *offsets, *sorted_slot, *slot_row;
  int32_t* dropped;       // S - offsets[E]
};
constexpr int64_t kRoutedMaxSlots = 2048;
bool routed_applicable(int64_t S, int E, int H, int I, int act_int8);
hipError_t launch_gate_up_routed(const GemmProblem& p, const RouteOut& ro, hipStream_t stream);
hipError_t launch_down_routed(const GemmProblem& p, const RouteOut& ro, hipStream_t stream);



// NVFP4 (W4A4): E2M1 codes, E4M3 scale per 16 values, FP32 outer scale per
// expert matrix (weights) or per input row (activations).
struct Fp4Problem {
  const uint8_t* aq;      // activation codes [a_rows][kdim/2]
  const uint8_t* ab;      // activation E4M3 block scales [a_rows][kdim/16]
  const float* ar;        // activation outer scales [a_rows]
  int64_t a_rows;
  int gather_k;           // >0: A row of sorted row r is token sorted_slot[r] / gather_k; 0: A row = r
  const int32_t* sorted_slot;
  const uint8_t* w0q; const uint8_t* w0b; const float* w0o;   // [E][n][kdim/2], [E][n][kdim/16], [E]
  const uint8_t* w1q; const uint8_t* w1b; const float* w1o;   // up (fused gate/up) or null
  const Tile* tiles; const int32_t* ntiles; int64_t max_tiles; int bm;
  uint16_t* out;          // bf16 [S][n]
  int n, kdim;
};
constexpr size_t kFp4MaxLds = 160 * 1024;
constexpr int64_t kMaxQuantBlocks = 1 << 16;   // grid cap of the grid-stride quantizers
// Row-tile height of the NVFP4 GEMMs (8 or 16 rows).
int fp4_tile_rows(int64_t S, int E);
size_t fp4_gemm_lds_bytes(int bm, int kdim);
hipError_t launch_fp4_gemm(const Fp4Problem& p, hipStream_t stream);
hipError_t launch_fp4_quantize_act(const uint16_t* v, int64_t rows, int cols, uint8_t* q, uint8_t* b, float* rs,
                                   hipStream_t stream);
hipError_t launch_fp4_quantize_weights(const float* w, int64_t mats, int64_t rows, int64_t cols, uint8_t* q,
                                       uint8_t* b, float* outer, hipStream_t stream);
// The routing (one workgroup of four waves; ra.nbits is filled in) and the
// NVFP4 quantization of x [rows][cols] in one launch, for ra.S <=
// kRouteQuantMaxSlots.
constexpr int64_t kRouteQuantMaxSlots = 512;
hipError_t launch_fp4_route_quantize_x(RouteArgs ra, const uint16_t* v, int64_t rows, int cols, uint8_t* q,
                                       uint8_t* b, float* rs, hipStream_t stream);

// Combine.
hipError_t launch_combine(const uint16_t* y, const int32_t* slot_row, const float* topk_w, int T, int K,
                          int H, uint16_t* out, hipStream_t stream);

// Streaming-read probe over `bytes` (a multiple of 16) of `buf`; sink holds
// kProbeSinkWords words.
constexpr int kProbeSinkWords = 1024;
hipError_t launch_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);

// Router: top-K of E logits per token (one wave per token), softmax weights.
hipError_t launch_topk_softmax(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                               hipStream_t stream);

// Start and stop events for the next GEMM launch of this thread: the timed
// forward calls set them just before their gate/up step, and the first GEMM
// launch takes (and clears) them, so they hold that kernel's own dispatch
// begin and end (the interval a kernel trace reports).
struct KernelEvents {
  hipEvent_t start, stop;
};
KernelEvents& kernel_events();

// hipLaunchKernelGGL for the GEMM kernels, or hipExtLaunchKernelGGL with the
// pending events when there are any.
#define QRE_LAUNCH_GEMM(kernel, grid, block, shm, stream, ...)                                           \
  do {                                                                                                    \
    ::qre::KernelEvents& ke_ = ::qre::kernel_events();                                                    \
    if (ke_.start || ke_.stop) {                                                                          \
      const hipEvent_t a_ = ke_.start, z_ = ke_.stop;                                                     \
      ke_ = ::qre::KernelEvents{nullptr, nullptr};                                                        \
      hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)(shm), stream, a_, z_, 0u, __VA_ARGS__); \
    } else {                                                                                              \
      hipLaunchKernelGGL(kernel, grid, block, shm, stream, __VA_ARGS__);                                  \
    }                                                                                                     \
  } while (0)

}  // namespace qre
