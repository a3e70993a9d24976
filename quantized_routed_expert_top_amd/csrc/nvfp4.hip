// NVFP4 (W4A4) routed experts on CDNA4 (gfx950): the quantizers and the
// grouped GEMMs.
//
// The format (model card "LLaDA2.2-flash for minnow", precision table, NVFP4
// row): E2M1 codes, an E4M3 scale per 16 consecutive values of the reduction,
// and an FP32 outer scale per expert matrix (weights) or per input row
// (dynamically quantized inputs, W4A4); FP32 accumulation (README
// "Quantization").  Where NVIDIA's native FP4 tensor cores are absent, the
// pages' non-native path rebuilds the already quantized FP4 operands for
// 16-bit matrix cores (model card, paragraph after the precision table).
// gfx950's own FP4 matrix instructions take power-of-two (E8M0) scales per 32
// values, which cannot carry E4M3 scales per 16, so this file takes the
// rebuild path, on FP16 matrix cores:
//  * every E2M1 value times its E4M3 block scale has at most 6 significant
//    bits and a magnitude in [2^-10, 2688], so it is exact in FP16 (and the
//    product of two such values is exact in FP32): the rebuilt operands lose
//    nothing, and the MFMAs accumulate exact products in FP32;
//  * a pair of codes becomes a pair of FP16 values with one
//    v_cvt_scalef32_pk_f16_fp4 (scale 1) and one packed FP16 multiply by the
//    block scale (itself converted from E4M3 by v_cvt_scalef32_pk_f16_fp8);
//  * the FP32 outer scales (the input row's and the expert matrix's) multiply
//    the FP32 sums once, in the epilogue.
//
// Quantizer readings (the pages give the format, not the rounding recipe):
// outer S = max|v| / (6 * 448) (FP32); block scale = E4M3 of
// max|block| / (S * 6) (FP32 product, FP32 quotient, nearest-even, saturating
// at 448); code = E2M1 of v / (scale * S) (FP32 product, FP32 quotient,
// nearest-even, saturating at 6, a zero magnitude stored as code 0).
#include <type_traits>

#include "gemm_common.h"
#include "route_small.h"

namespace qre {
namespace {

using namespace gk;

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

constexpr int kBlk = 16;                    // values per E4M3 scale

// ---- the quantizer's roundings (FP32 decisions, as the oracle takes them) ----

// E4M3 byte of d >= 0 (finite): nearest, ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode(float d) {
  if (!(d < 448.0f)) return 0x7Eu;                                // 448 and beyond (RNE of [448, 464) is 448 too)
  if (d < 0x1p-6f) return (uint32_t)__builtin_rintf(d * 512.0f);  // subnormal: multiples of 2^-9 (8 -> 2^-6, code 0x08)
  const uint32_t u = __float_as_uint(d);
  const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) & ~0xFFFFFu;   // 3 mantissa bits, nearest even
  return (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);           // exponent bias 127 -> 7
}

// The value of an E4M3 byte < 0x7F (non-negative, finite), exact in FP32.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = b >> 3, m = b & 7u;
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 code of q: nearest, ties to even (the code with a zero low bit),
// saturating at 6; a magnitude that rounds to 0 gives code 0.
__device__ __forceinline__ uint32_t e2m1_encode(float q) {
  const float a = __builtin_fabsf(q);
  const uint32_t m = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return m == 0 ? 0u : (m | (q < 0.0f ? 8u : 0u));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, d));
  return v;
}

// One block of 16 values with outer scale S (den = S * 6): the 8 code bytes
// (two words) and the scale byte.
__device__ __forceinline__ void quantize_block(const float (&v)[kBlk], float S, float den, uint32_t& c0, uint32_t& c1,
                                               uint32_t& sb) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < kBlk; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
  sb = den > 0.f ? e4m3_encode(amax / den) : 0u;
  const float den2 = e4m3_value(sb) * S;
  c0 = 0; c1 = 0;
  if (den2 > 0.f) {
#pragma unroll
    for (int j = 0; j < kBlk; ++j) {
      const uint32_t c = e2m1_encode(v[j] / den2);
      if (j < 8) c0 |= c << (4 * j);
      else c1 |= c << (4 * (j - 8));
    }
  }
}

// Activations: one wave per row (grid-stride over rows).  Pass 1: the row's
// max; pass 2: each lane quantizes whole blocks (16 BF16 values, 32 bytes).
// Rows r = 4 blk0 + wave, stepping by 4 nblk (blk0 < nblk: this workgroup's
// index among the nblk that quantize).
__device__ void fp4_quantize_rows(const uint16_t* __restrict__ v, int64_t rows, int cols, uint8_t* __restrict__ q,
                                  uint8_t* __restrict__ b, float* __restrict__ rs, int blk0, int nblk) {
  const int lane = threadIdx.x & 63;
  const int nb = cols / kBlk;
  for (int64_t r = (int64_t)blk0 * 4 + (threadIdx.x >> 6); r < rows; r += (int64_t)nblk * 4) {
    const uint16_t* vr = v + r * cols;
    float amax = 0.f;
    for (int k = lane * 8; k < cols; k += 64 * 8) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(vr + k);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16_bits_to_f32(w[i] & 0xffffu)),
                                                     __builtin_fabsf(bf16_bits_to_f32(w[i] >> 16))));
    }
    amax = wave_max(amax);
    const float S = amax / (6.0f * 448.0f);
    const float den = S * 6.0f;
    if (lane == 0) rs[r] = S;
    for (int blk = lane; blk < nb; blk += 64) {
      const u32x4_t w0 = *reinterpret_cast<const u32x4_t*>(vr + blk * kBlk);
      const u32x4_t w1 = *reinterpret_cast<const u32x4_t*>(vr + blk * kBlk + 8);
      float x[kBlk];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_bits_to_f32(w0[i] & 0xffffu);
        x[2 * i + 1] = bf16_bits_to_f32(w0[i] >> 16);
        x[8 + 2 * i] = bf16_bits_to_f32(w1[i] & 0xffffu);
        x[8 + 2 * i + 1] = bf16_bits_to_f32(w1[i] >> 16);
      }
      uint32_t c0, c1, sb;
      quantize_block(x, S, den, c0, c1, sb);
      *reinterpret_cast<uint2*>(q + r * (cols / 2) + blk * 8) = uint2{c0, c1};
      b[r * nb + blk] = (uint8_t)sb;
    }
  }
}

__global__ __launch_bounds__(256) void k_fp4_quantize_act(const uint16_t* __restrict__ v, int64_t rows, int cols,
                                                          uint8_t* __restrict__ q, uint8_t* __restrict__ b,
                                                          float* __restrict__ rs) {
  fp4_quantize_rows(v, rows, cols, q, b, rs, blockIdx.x, gridDim.x);
}

// Decode blocks: the routing (workgroup 0, four waves) and the quantization
// of x (the other workgroups, one row per wave) in one launch, since neither
// reads what the other writes.
__global__ __launch_bounds__(256) void k_fp4_route_quantize_x(RouteArgs ra, const uint16_t* __restrict__ v,
                                                              int64_t rows, int cols, uint8_t* __restrict__ q,
                                                              uint8_t* __restrict__ b, float* __restrict__ rs) {
  extern __shared__ int route_lds[];
  if (blockIdx.x == 0) {
    route_small<4>(route_lds, ra.ids, ra.S, ra.E, ra.nbits, ra.counts, ra.offsets, ra.sorted_slot, ra.slot_row,
                   ra.dropped, ra.tiles_a, ra.ntiles_a, ra.bm_a, ra.tiles_b, ra.ntiles_b, ra.bm_b);
    return;
  }
  fp4_quantize_rows(v, rows, cols, q, b, rs, blockIdx.x - 1, gridDim.x - 1);
}

// Weights, pass 1: the largest magnitude of each matrix, as FP32 bits (the
// bits of non-negative floats order like the floats), into amax[mats]
// (cleared by the caller's launch sequence).
__global__ __launch_bounds__(256) void k_fp4_amax(const float* __restrict__ w, int64_t per_mat, int64_t mats,
                                                  uint32_t* __restrict__ amax) {
  for (int64_t m = blockIdx.y; m < mats; m += gridDim.y) {
    const float* wm = w + m * per_mat;
    float a = 0.f;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < per_mat; i += (int64_t)gridDim.x * blockDim.x)
      a = __builtin_fmaxf(a, __builtin_fabsf(wm[i]));
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0) atomicMax(amax + m, __float_as_uint(a));
  }
}

__global__ void k_fp4_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// Weights, pass 2: one thread per block of 16 (grid-stride); the outer scale
// of its matrix from amax.
__global__ __launch_bounds__(256) void k_fp4_quantize_w(const float* __restrict__ w, int64_t rows, int64_t cols,
                                                        int64_t nblocks, const uint32_t* __restrict__ amax,
                                                        uint8_t* __restrict__ q, uint8_t* __restrict__ b) {
  const int64_t bpm = rows * (cols / kBlk);                       // blocks per matrix
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nblocks; i += (int64_t)gridDim.x * blockDim.x) {
    const float S = __uint_as_float(amax[i / bpm]) / (6.0f * 448.0f);
    const float* src = w + i * kBlk;
    float x[kBlk];
#pragma unroll
    for (int j = 0; j < kBlk; j += 4) {
      const f32x4_t t = *reinterpret_cast<const f32x4_t*>(src + j);
      x[j] = t[0]; x[j + 1] = t[1]; x[j + 2] = t[2]; x[j + 3] = t[3];
    }
    uint32_t c0, c1, sb;
    quantize_block(x, S, S * 6.0f, c0, c1, sb);
    *reinterpret_cast<uint2*>(q + i * 8) = uint2{c0, c1};
    b[i] = (uint8_t)sb;
  }
}

// Weights, pass 3: amax bits -> outer scales (in place).
__global__ void k_fp4_outer(uint32_t* __restrict__ amax_then_outer, int64_t mats) {
  for (int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; m < mats; m += (int64_t)gridDim.x * blockDim.x)
    amax_then_outer[m] = __float_as_uint(__uint_as_float(amax_then_outer[m]) / (6.0f * 448.0f));
}

// ---- the grouped GEMM ----------------------------------------------------------

// A packed pair of codes (byte `sel` of w) times the block scale pair s2.
template <int sel>
__device__ __forceinline__ f16x2_t pair(uint32_t w, f16x2_t s2) {
  return __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, sel)) * s2;
}

// 8 codes (one word) with one scale -> the 8 FP16 values of an MFMA operand.
__device__ __forceinline__ f16x8_t rebuild8(uint32_t w, f16x2_t s2) {
  const f16x2_t p0 = pair<0>(w, s2), p1 = pair<1>(w, s2), p2 = pair<2>(w, s2), p3 = pair<3>(w, s2);
  return f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Row-tile kernel (decode blocks and batched blocks: weights stream once per
// tile of up to BMR sorted rows).  A workgroup's four waves each own 16 FN
// weight rows (columns of the output) over the whole reduction; the tile's
// activation rows are rebuilt into LDS once, as FP16 in natural order with
// the 16-byte chunk index XOR-swizzled by row.  The reduction is walked in
// steps of SW values (SW = 256 when its length is a known multiple of 256,
// else 128): per step a lane loads the codes of SW / 4 consecutive values
// (lanes kb = 0..3 of a row take consecutive quarters) and the SW / 64
// scale bytes of those blocks, DEPTH steps ahead.  MFMA t of the step takes
// code word t, matched by LDS chunk (SW / 32) kb + t of the row.  NS > 0 is
// the reduction length in 128s, known at compile time: the stream is then
// straight-line code and every wait covers exactly the step it needs; NS = 0
// takes the length at run time.
template <bool DUAL, int FN, int BMR, int DEPTH, int NS>
struct Fp4Gemm {
  static constexpr int NM = DUAL ? 2 : 1;
  static constexpr int BN = 4 * 16 * FN;                          // output columns per workgroup
  static constexpr int SW = (NS > 0 && NS % 2 == 0) ? 256 : 128;  // reduction values per step
  static constexpr int CW = SW / 128;                             // 16-byte code loads per lane per step
  static constexpr int NT = SW / 32;                              // MFMAs per fragment per step

  struct WBuf {
    u32x4_t c[FN][NM][CW];
    uint32_t s[FN][NM];        // the lane's SW / 64 scale bytes (low bytes first)
  };

  __device__ static int swz(int r) { return (r ^ ((r >> 3) & 1)) & 7; }
  __device__ static uint32_t lds_chunk(int row, int chunk, int kdim) {
    return (uint32_t)(row * kdim * 2 + ((chunk ^ swz(row)) << 4));
  }
  static size_t lds_bytes(int kdim) { return (size_t)BMR * kdim * 2 + 16 * 4; }

  template <class RowSrc>
  __device__ static void run(const Fp4Problem& p, int e, int row0, int nrows, RowSrc src_row, uint8_t* lds, int cb) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, kb = lane >> 4;
    const int K = NS > 0 ? NS * kGroup : p.kdim;
    const int nsteps = K / SW;
    const int col0 = min((cb * 4 + wave) * 16 * FN, p.n - 16 * FN);  // a surplus wave recomputes the last tile, stores nothing
    const int64_t cbytes = (int64_t)p.n * (K / 2), sbytes = (int64_t)p.n * (K / kBlk);
    rsrc_t rc[NM], rb[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      rc[m] = make_rsrc((m == 0 ? p.w0q : p.w1q) + e * cbytes, cbytes);
      rb[m] = make_rsrc((m == 0 ? p.w0b : p.w1b) + e * sbytes, sbytes);
    }
    uint32_t c_off[FN], s_off[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int n = col0 + f * 16 + li;
      c_off[f] = (uint32_t)(n * (K / 2) + kb * (SW / 8));
      s_off[f] = (uint32_t)(n * (K / kBlk) + kb * (SW / 64));
    }
    WBuf buf[DEPTH];
    auto load_step = [&](WBuf& bf, int g) {
      const bool in = NS > 0 || g < nsteps;
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
#pragma unroll
          for (int j = 0; j < CW; ++j)
            bf.c[f][m][j] = bload16(rc[m], in ? c_off[f] + (uint32_t)(g * (SW / 2) + 16 * j) : kOOB);
          const uint32_t so = in ? s_off[f] + (uint32_t)g * (SW / 16) : kOOB;
          bf.s[f][m] = SW == 256 ? __builtin_amdgcn_raw_buffer_load_b32(rb[m], so, 0, 0) : bload_u16(rb[m], so);
        }
    };
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      if (NS == 0 || j < NS * 128 / SW) load_step(buf[j], j);
      __builtin_amdgcn_sched_barrier(0);
    }

    // stage the tile's rows: chunk c of a row (8 values) from one code word
    // and the scale byte of its block; the row scales after the rows
    float* rs_lds = reinterpret_cast<float*>(lds + (size_t)BMR * K * 2);
    const int CPR = K / 8;
    for (int idx = tid; idx < nrows * CPR; idx += blockDim.x) {
      const int r = idx / CPR, c = idx - r * CPR;
      const int64_t src = src_row(r);
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p.aq + src * (K / 2) + c * 4);
      const uint32_t sb = p.ab[src * (K / kBlk) + c / 2];
      const f16x2_t s2 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb | (sb << 8), 1.0f, false));
      *reinterpret_cast<f16x8_t*>(lds + lds_chunk(r, c, K)) = rebuild8(w, s2);
    }
    if (tid < nrows) rs_lds[tid] = p.ar[src_row(tid)];
    __syncthreads();
    if ((cb * 4 + wave) * 16 * FN >= p.n) return;                 // wave-uniform, after the barrier

    // the lane's LDS row and the offsets of its NT chunks in step 0 (the
    // swizzle touches only the low 3 bits of a chunk index, and a step spans
    // a multiple of 8 chunks, so step g adds g * SW * 2 bytes)
    const int arow = (BMR == 16) ? li : (li & (BMR - 1));         // LDS row feeding MFMA row li
    uint32_t a_base[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) a_base[t] = lds_chunk(arow, kb * NT + t, K);
    f32x4_t acc[FN][NM];
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[f][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto step = [&](WBuf& bf, int g) {
      // the block scales as FP16 pairs: blocks 0, 1 (and 2, 3) of the lane's values
      f16x2_t sc[FN][NM][SW / 128];
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          sc[f][m][0] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bf.s[f][m], 1.0f, false));
          if constexpr (SW == 256)
            sc[f][m][1] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bf.s[f][m], 1.0f, true));
        }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f16x8_t a = *reinterpret_cast<const f16x8_t*>(lds + a_base[t] + g * SW * 2);
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const _Float16 s1 = sc[f][m][t / 4][(t / 2) % 2];       // block t / 2 of the lane's values
            const f16x8_t bv = rebuild8(bf.c[f][m][t / 4][t % 4], f16x2_t{s1, s1});
            acc[f][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bv, acc[f][m], 0, 0, 0);
          }
      }
    };
    if constexpr (NS > 0) {
      constexpr int NST = NS * 128 / SW;
#pragma unroll
      for (int g = 0; g < NST; ++g) {
        step(buf[g % DEPTH], g);
        if (g + DEPTH < NST) load_step(buf[g % DEPTH], g + DEPTH);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      for (int g0 = 0; g0 < nsteps; g0 += DEPTH) {
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {
          const int g = g0 + j;
          if (g < nsteps) {                                        // uniform
            step(buf[j], g);
            load_step(buf[j], g + DEPTH);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // epilogue: lane holds rows 4 kb + r of column li of each fragment
    const float o0 = p.w0o[e], o1 = DUAL ? p.w1o[e] : 0.f;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int col = col0 + f * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * kb + r;
        if (m < nrows) {
          const float xr = rs_lds[m];
          float o;
          if constexpr (DUAL) o = silu(acc[f][0][r] * (xr * o0)) * (acc[f][1][r] * (xr * o1));
          else o = acc[f][0][r] * (xr * o0);
          p.out[(int64_t)(row0 + m) * p.n + col] = (uint16_t)f32_to_bf16_bits(o);
        }
      }
    }
  }
};

template <bool DUAL, int FN, int BMR, int DEPTH, int NS>
__global__ __launch_bounds__(256) void k_fp4_gemm(Fp4Problem p) {
  using G = Fp4Gemm<DUAL, FN, BMR, DEPTH, NS>;
  extern __shared__ __attribute__((aligned(16))) uint8_t fp4_lds[];
  const int tile = blockIdx.y;
  if (tile >= *p.ntiles) return;
  const Tile td = p.tiles[tile];
  const int row0 = td.row0;
  if (p.gather_k)
    G::run(p, td.e, row0, td.nrows, [&](int r) { return (int64_t)(p.sorted_slot[row0 + r] / p.gather_k); }, fp4_lds,
           blockIdx.x);
  else
    G::run(p, td.e, row0, td.nrows, [&](int r) { return (int64_t)(row0 + r); }, fp4_lds, blockIdx.x);
}

template <bool DUAL, int FN, int BMR, int NS>
hipError_t launch_fp4_ns(const Fp4Problem& p, hipStream_t s) {
  // 1024 reduction values of weights in flight per lane (8 steps of 128 or 4
  // of 256), fewer when the reduction is shorter
  constexpr int SW = (NS > 0 && NS % 2 == 0) ? 256 : 128;
  constexpr int STEPS = NS > 0 ? NS * 128 / SW : 1 << 30;
  constexpr int DMAX = 1024 / SW;
  constexpr int DEPTH = STEPS < DMAX ? STEPS : DMAX;
  using G = Fp4Gemm<DUAL, FN, BMR, DEPTH, NS>;
  const size_t lds = G::lds_bytes(p.kdim);
  if (lds > kFp4MaxLds) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((p.n + G::BN - 1) / G::BN), (unsigned)p.max_tiles);
  QRE_LAUNCH_GEMM((k_fp4_gemm<DUAL, FN, BMR, DEPTH, NS>), grid, dim3(256), lds, s, p);
  return hipGetLastError();
}

template <bool DUAL, int FN, int BMR>
hipError_t launch_fp4_cfg(const Fp4Problem& p, hipStream_t s) {
  if (p.n % (16 * FN) != 0 || p.kdim % kGroup != 0) return hipErrorInvalidValue;
  switch (p.kdim / kGroup) {
    case 4: return launch_fp4_ns<DUAL, FN, BMR, 4>(p, s);
    case 8: return launch_fp4_ns<DUAL, FN, BMR, 8>(p, s);
    case 12: return launch_fp4_ns<DUAL, FN, BMR, 12>(p, s);
    case 16: return launch_fp4_ns<DUAL, FN, BMR, 16>(p, s);
    case 32: return launch_fp4_ns<DUAL, FN, BMR, 32>(p, s);
    default: return launch_fp4_ns<DUAL, FN, BMR, 0>(p, s);
  }
}

}  // namespace

int fp4_tile_rows(int64_t S, int E) { return S <= 4 * (int64_t)E ? 8 : 16; }

size_t fp4_gemm_lds_bytes(int bm, int kdim) { return (size_t)bm * kdim * 2 + 16 * 4; }

hipError_t launch_fp4_gemm(const Fp4Problem& p, hipStream_t s) {
  if (p.max_tiles == 0 || p.n == 0) return hipSuccess;
  const bool dual = p.w1q != nullptr;
  if (p.bm == 8) return dual ? launch_fp4_cfg<true, 1, 8>(p, s) : launch_fp4_cfg<false, 2, 8>(p, s);
  if (p.bm == 16) return dual ? launch_fp4_cfg<true, 1, 16>(p, s) : launch_fp4_cfg<false, 2, 16>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fp4_quantize_act(const uint16_t* v, int64_t rows, int cols, uint8_t* q, uint8_t* b, float* rs,
                                   hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t wgs = (rows + 3) / 4;
  const unsigned grid = (unsigned)(wgs < kMaxQuantBlocks ? wgs : kMaxQuantBlocks);
  hipLaunchKernelGGL(k_fp4_quantize_act, dim3(grid), dim3(256), 0, s, v, rows, cols, q, b, rs);
  return hipGetLastError();
}

hipError_t launch_fp4_route_quantize_x(RouteArgs ra, const uint16_t* v, int64_t rows, int cols, uint8_t* q,
                                       uint8_t* b, float* rs, hipStream_t s) {
  if ((int64_t)ra.S > kRouteQuantMaxSlots || rows == 0) return hipErrorInvalidValue;
  ra.nbits = bits_for(ra.E);
  const int64_t wgs = (rows + 3) / 4;
  const unsigned grid = 1 + (unsigned)(wgs < kMaxQuantBlocks ? wgs : kMaxQuantBlocks);
  hipLaunchKernelGGL(k_fp4_route_quantize_x, dim3(grid), dim3(256), sizeof(int) * route_small_lds_ints(4, ra.E), s,
                     ra, v, rows, cols, q, b, rs);
  return hipGetLastError();
}

hipError_t launch_fp4_quantize_weights(const float* w, int64_t mats, int64_t rows, int64_t cols, uint8_t* q,
                                       uint8_t* b, float* outer, hipStream_t s) {
  if (mats == 0 || rows == 0) return hipSuccess;
  uint32_t* amax = reinterpret_cast<uint32_t*>(outer);
  hipLaunchKernelGGL(k_fp4_fill_u32, dim3(1), dim3(256), 0, s, amax, mats, 0u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t per_mat = rows * cols;
  const int64_t gx64 = (per_mat + 256 * 16 - 1) / (256 * 16);
  const unsigned gx = (unsigned)(gx64 < 1024 ? gx64 : 1024), gy = (unsigned)(mats < 65535 ? mats : 65535);
  hipLaunchKernelGGL(k_fp4_amax, dim3(gx, gy), dim3(256), 0, s, w, per_mat, mats, amax);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nblocks = mats * per_mat / kBlk;
  const int64_t g64 = (nblocks + 255) / 256;
  hipLaunchKernelGGL(k_fp4_quantize_w, dim3((unsigned)(g64 < kMaxQuantBlocks ? g64 : kMaxQuantBlocks)), dim3(256), 0,
                     s, w, rows, cols, nblocks, amax, q, b);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_fp4_outer, dim3(1), dim3(256), 0, s, amax, mats);
  return hipGetLastError();
}

}  // namespace qre
