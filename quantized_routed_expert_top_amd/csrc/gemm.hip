// Grouped expert GEMMs with group-quantized weights, for CDNA4 (gfx950).
//
//   gate/up (fused):  h[r][i] = bf16( silu(g) * u ),  g = sum_k A[r][k] Wg[e][i][k],  u likewise
//   down:             y[r][j] = bf16( sum_k A[r][k] Wd[e][j][k] )
//
// for every sorted row r of a routed expert e (rows come from the routing
// permutation; A is x gathered by token for gate/up, h for down).  The pages
// (minnow README, section "Quantization"; model card "LLaDA2.2-flash for
// minnow", paragraphs after the precision table) fix what is computed:
// weights are signed INT4/INT8 with an FP16 scale per 128 inputs and are
// dequantized in registers, never expanded to a full copy; BF16 activations
// feed the matrix cores; with INT8 activations the group dot products are
// INT32 and the scaled groups are combined in FP32; outputs return to BF16.
//
// CDNA4 mapping (this is the kernel's own design, not the pages'):
//  * one wave computes a 16-row x 16*FN-column tile (both gate and up for the
//    fused kernel) over the whole reduction, so each weight byte is read from
//    HBM exactly once per 16-row tile, with 16-byte loads per lane (64
//    contiguous bytes per weight row per 128-group for INT4, 128 for INT8);
//  * a 128-group is four v_mfma_f32_16x16x32_bf16 steps (BF16 activations) or
//    two v_mfma_i32_16x16x64_i8 steps (INT8 activations); the group's partial
//    sums are scaled by the FP16 weight scale (and the FP32 activation scale)
//    in FP32 after the group, which keeps the in-register dequantization to a
//    few bit operations;
//  * INT4 codes become BF16 without arithmetic: XOR with 8 turns the nibble
//    into u = q + 8 in 0..15 and OR-ing it into the mantissa of BF16 128.0
//    gives exactly 136 + q; INT8 codes become 128 + q via the unsigned-byte
//    conversion.  The offset is removed per group with the row sums of A,
//    which one extra MFMA against a ones operand produces directly in the
//    accumulator layout (exact for INT8 activations, FP32 for BF16);
//  * nibble extraction pairs codes k and k+4 of each 32-bit word, so A is
//    permuted the same way with v_perm_b32 (a dot product is invariant under a
//    common permutation of the reduction index);
//  * loads of group g+PD are issued while group g is multiplied (a register
//    ring of PD groups) to keep enough bytes in flight for HBM;
//  * workgroups are (column block, row tile); tiles past the device-side tile
//    count exit at once, so no host readback is needed.
#include <hip/hip_fp16.h>

#include "qre_internal.h"

namespace qre {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  return __half2float(__ushort_as_half((unsigned short)h));
}

// Two BF16 values (exact small integers held in FP32) packed into one dword.
__device__ __forceinline__ uint32_t pack_bf16_hi(float lo, float hi) {
  return byte_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

template <int WB, bool A8, bool DUAL, int FN, int PD>
struct Gemm16 {
  static constexpr int NM = DUAL ? 2 : 1;                // weight matrices
  static constexpr int NA = A8 ? 2 : 4;                  // 16-byte A chunks per lane per group
  static constexpr int NB = (WB == 4) ? 1 : 2;           // 16-byte B chunks per lane per group
  static constexpr int BN = 4 * 16 * FN;                 // columns per workgroup

  struct Buf {
    u32x4_t a[NA];
    float xs[4];
    u32x4_t b[FN][NM][NB];
    uint32_t s[FN][NM];
  };

  const GemmProblem& p;
  int lane, li, kb, G, e, row0, nrows, n_wave;
  bool arow_ok;
  const uint8_t* a_row;          // this lane's A row (byte pointer)
  int64_t erow[4];               // A rows (for activation scales) of accumulator rows 4kb+r
  const uint8_t* wq[FN][NM];
  const uint16_t* wsp[FN][NM];

  __device__ Gemm16(const GemmProblem& prob, const Tile& td, int wave) : p(prob) {
    lane = threadIdx.x & 63;
    li = lane & 15;
    kb = lane >> 4;
    G = p.kdim / kGroup;
    e = td.e;
    row0 = td.row0;
    nrows = td.nrows;
    n_wave = (blockIdx.x * 4 + wave) * 16 * FN;
    const int a_elem = A8 ? 1 : 2;
    arow_ok = li < nrows;
    a_row = nullptr;
    if (arow_ok) {
      const int r = row0 + li;
      const int64_t ar = p.gather_k ? (int64_t)(p.sorted_slot[r] / p.gather_k) : (int64_t)r;
      a_row = static_cast<const uint8_t*>(p.a) + ar * p.kdim * a_elem;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * kb + r;
      erow[r] = -1;
      if (A8 && m < nrows) erow[r] = p.gather_k ? (int64_t)(p.sorted_slot[row0 + m] / p.gather_k) : (int64_t)(row0 + m);
    }
    const int64_t row_bytes = (int64_t)p.kdim * WB / 8;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int64_t n = (int64_t)e * p.n + n_wave + f * 16 + li;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        wq[f][m] = (m == 0 ? p.w0q : p.w1q) + n * row_bytes;
        wsp[f][m] = (m == 0 ? p.w0s : p.w1s) + n * G;
      }
    }
  }

  __device__ __forceinline__ void load(Buf& bf, int g) const {
    if (arow_ok) {
      const uint8_t* ap = a_row + (int64_t)(g * kGroup + kb * 32) * (A8 ? 1 : 2);
#pragma unroll
      for (int j = 0; j < NA; ++j) bf.a[j] = ld16(ap + 16 * j);
    } else {
#pragma unroll
      for (int j = 0; j < NA; ++j) bf.a[j] = u32x4_t{0u, 0u, 0u, 0u};
    }
    if constexpr (A8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) bf.xs[r] = erow[r] >= 0 ? p.a_scale[erow[r] * G + g] : 0.0f;
    }
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint8_t* bp = wq[f][m] + (int64_t)g * (kGroup * WB / 8) + kb * (WB == 4 ? 16 : 32);
#pragma unroll
        for (int j = 0; j < NB; ++j) bf.b[f][m][j] = ld16(bp + 16 * j);
        bf.s[f][m] = wsp[f][m][g];
      }
  }

  // BF16 activations: one 128-group, accumulated into acc[f][m] (FP32).
  __device__ __forceinline__ void group_bf16(const Buf& bf, f32x4_t (&acc)[FN][NM]) const {
    f32x4_t accg[FN][NM];
    f32x4_t accx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) accg[f][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4_t c = bf.a[t];
      u32x4_t av;
      if constexpr (WB == 4) {   // match the nibble pairing (k, k+4)
        av.x = byte_perm(c.z, c.x, 0x05040100u);
        av.y = byte_perm(c.z, c.x, 0x07060302u);
        av.z = byte_perm(c.w, c.y, 0x05040100u);
        av.w = byte_perm(c.w, c.y, 0x07060302u);
      } else {
        av = c;
      }
      const bf16x8_t a8 = __builtin_bit_cast(bf16x8_t, av);
      accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, __builtin_bit_cast(bf16x8_t, ones), accx, 0, 0, 0);
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          u32x4_t bv;
          if constexpr (WB == 4) {
            const uint32_t w = bf.b[f][m][0][t] ^ 0x88888888u;   // nibble -> q + 8
            bv.x = (w & 0x000f000fu) | 0x43004300u;              // bf16 (136+q_k, 136+q_{k+4})
            bv.y = ((w >> 4) & 0x000f000fu) | 0x43004300u;
            bv.z = ((w >> 8) & 0x000f000fu) | 0x43004300u;
            bv.w = ((w >> 12) & 0x000f000fu) | 0x43004300u;
          } else {
            const uint32_t w0 = bf.b[f][m][t >> 1][(t & 1) * 2] ^ 0x80808080u;       // byte -> q + 128
            const uint32_t w1 = bf.b[f][m][t >> 1][(t & 1) * 2 + 1] ^ 0x80808080u;
            bv.x = pack_bf16_hi((float)(w0 & 0xffu), (float)((w0 >> 8) & 0xffu));
            bv.y = pack_bf16_hi((float)((w0 >> 16) & 0xffu), (float)(w0 >> 24));
            bv.z = pack_bf16_hi((float)(w1 & 0xffu), (float)((w1 >> 8) & 0xffu));
            bv.w = pack_bf16_hi((float)((w1 >> 16) & 0xffu), (float)(w1 >> 24));
          }
          accg[f][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, __builtin_bit_cast(bf16x8_t, bv), accg[f][m],
                                                               0, 0, 0);
        }
    }
    constexpr float kOff = (WB == 4) ? 136.0f : 128.0f;
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const float sc = half_bits_to_f32(bf.s[f][m]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[f][m][r] = __builtin_fmaf(sc, accg[f][m][r] - kOff * accx[r], acc[f][m][r]);
      }
  }

  // INT8 activations: one 128-group as exact INT32 sums, combined in FP32.
  __device__ __forceinline__ void group_i8(const Buf& bf, f32x4_t (&acc)[FN][NM]) const {
    i32x4_t accg[FN][NM];
    i32x4_t accx = {0, 0, 0, 0};
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) accg[f][m] = i32x4_t{0, 0, 0, 0};
    const i32x4_t ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4_t c = bf.a[t];
      u32x4_t av;
      if constexpr (WB == 4) {   // match the nibble split (even codes, odd codes) of each word
        av.x = byte_perm(c.y, c.x, 0x06040200u);
        av.y = byte_perm(c.y, c.x, 0x07050301u);
        av.z = byte_perm(c.w, c.z, 0x06040200u);
        av.w = byte_perm(c.w, c.z, 0x07050301u);
      } else {
        av = c;
      }
      const i32x4_t ai = __builtin_bit_cast(i32x4_t, av);
      if constexpr (WB == 4) accx = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, ones, accx, 0, 0, 0);
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          u32x4_t bv;
          if constexpr (WB == 4) {
            const uint32_t w0 = bf.b[f][m][0][2 * t] ^ 0x88888888u;       // nibble -> q + 8
            const uint32_t w1 = bf.b[f][m][0][2 * t + 1] ^ 0x88888888u;
            bv.x = w0 & 0x0f0f0f0fu;
            bv.y = (w0 >> 4) & 0x0f0f0f0fu;
            bv.z = w1 & 0x0f0f0f0fu;
            bv.w = (w1 >> 4) & 0x0f0f0f0fu;
          } else {
            bv = bf.b[f][m][t];
          }
          accg[f][m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, __builtin_bit_cast(i32x4_t, bv), accg[f][m], 0, 0, 0);
        }
    }
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const float ws = half_bits_to_f32(bf.s[f][m]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int isum = (WB == 4) ? accg[f][m][r] - 8 * accx[r] : accg[f][m][r];
          acc[f][m][r] = __builtin_fmaf((float)isum, bf.xs[r] * ws, acc[f][m][r]);
        }
      }
  }

  __device__ void run() const {
    f32x4_t acc[FN][NM];
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[f][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    Buf buf[PD];
#pragma unroll
    for (int j = 0; j < PD; ++j)
      if (j < G) load(buf[j], j);
    for (int g0 = 0; g0 < G; g0 += PD) {
#pragma unroll
      for (int j = 0; j < PD; ++j) {
        const int g = g0 + j;
        if (g < G) {
          if constexpr (A8) group_i8(buf[j], acc);
          else group_bf16(buf[j], acc);
          if (g + PD < G) load(buf[j], g + PD);
        }
      }
    }
    // epilogue: lane holds rows 4kb+r of column li of each 16-column fragment
    uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int64_t col = n_wave + f * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * kb + r;
        if (m < nrows) {
          float v;
          if constexpr (DUAL) v = silu(acc[f][0][r]) * acc[f][1][r];
          else v = acc[f][0][r];
          out[(int64_t)(row0 + m) * p.n + col] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
  }
};

template <int WB, bool A8, bool DUAL, int FN, int PD>
__global__ __launch_bounds__(256) void k_gemm16(GemmProblem p) {
  if ((int)blockIdx.y >= *p.ntiles) return;                 // tile past the routed rows
  const Tile td = p.tiles[blockIdx.y];
  const int wave = threadIdx.x >> 6;
  if ((blockIdx.x * 4 + wave) * 16 * FN >= p.n) return;     // wave-uniform
  Gemm16<WB, A8, DUAL, FN, PD> g(p, td, wave);
  g.run();
}

template <int WB, bool A8, bool DUAL>
hipError_t launch_variant(const GemmProblem& p, hipStream_t stream) {
  constexpr int FN = 1, PD = 3;
  constexpr int BN = 4 * 16 * FN;
  const dim3 grid((p.n + BN - 1) / BN, (unsigned)p.max_tiles);
  hipLaunchKernelGGL((k_gemm16<WB, A8, DUAL, FN, PD>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int gemm_tile_rows(int64_t, int, int, int) { return 16; }

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream) {
  if (p.max_tiles == 0 || p.n == 0) return hipSuccess;
  const bool dual = p.w1q != nullptr;
  if (p.bits == 4) {
    if (p.act_int8) return dual ? launch_variant<4, true, true>(p, stream) : launch_variant<4, true, false>(p, stream);
    return dual ? launch_variant<4, false, true>(p, stream) : launch_variant<4, false, false>(p, stream);
  }
  if (p.act_int8) return dual ? launch_variant<8, true, true>(p, stream) : launch_variant<8, true, false>(p, stream);
  return dual ? launch_variant<8, false, true>(p, stream) : launch_variant<8, false, false>(p, stream);
}

}  // namespace qre
