// Decode-block grouped GEMMs with the reduction split over the four waves of
// a workgroup, CDNA4 (gfx950).
//
// Same arithmetic as the other GEMM kernels (gemm_common.h; the pages fix it:
// minnow README, section "Quantization"; model card "LLaDA2.2-flash for
// minnow", paragraphs after the precision table): weights dequantized in
// registers, BF16 activations on BF16 MFMAs or INT8 activations on INT8 MFMAs
// with exact INT32 group sums, each 128-group's sum scaled in FP32.  The work
// split is this kernel's own, made for the weight-streaming regime (a few
// rows per expert):
//  * a workgroup owns one expert and NBLK column blocks of 16*FN columns; its
//    rows' activations are staged once into LDS (permuted into the operand
//    order, with each row's per-group sums for the offset removal);
//  * within a block, wave w owns reduction groups [w*NGW, (w+1)*NGW), so the
//    four waves together request the block's whole weight slice (16*FN
//    contiguous rows, full length) at once, and the next block's slice is in
//    flight while the current one computes;
//  * the four partial sums meet in LDS (double-buffered, one barrier per
//    block) and are added in wave order 0..3 (deterministic); wave w
//    finishes accumulator element w of every lane (SiLU*mul for gate/up).
// The gate/up kernel computes its expert's rows from the ids itself
// (route_expert); the down kernel reads counts/offsets back.
#include "gemm_common.h"

namespace qre {
namespace {

using namespace gk;

// 16-byte chunk position within a staged row: 16 aligned consecutive rows put
// a given chunk in 16 distinct 16-byte bank groups of a 256-byte window
__device__ __forceinline__ int dswz(int r) { return (r ^ ((r >> 3) & 1)) & 7; }

template <int WB, bool A8, bool DUAL, int FN, int NGW, int NBLK, int BMR>
struct DecKS {
  static constexpr int NM = DUAL ? 2 : 1;                 // weight matrices
  static constexpr int NB = (WB == 4) ? 1 : 2;            // 16-byte weight loads per lane per (tile, group)
  static constexpr int NG = 4 * NGW;                      // groups of the reduction
  static constexpr int STEPS = A8 ? 2 : 4;                // MFMA steps per group
  static constexpr int CPG = A8 ? 8 : 16;                 // 16-byte A chunks per group
  static constexpr int WGB = kGroup * WB / 8;             // weight bytes per (column, group)
  static constexpr int ROWB = NG * kGroup * (A8 ? 1 : 2); // LDS bytes of a staged row
  static constexpr int CPR = ROWB / 16;
  static constexpr int BN = 16 * FN;                      // columns per block
  static constexpr int BCOLS = BN * NBLK;                 // columns per workgroup
  static constexpr bool RSUM = !A8 || WB == 4;            // per-row group sums remove the code offset
  static constexpr int XS_OFF = BMR * ROWB;               // A8: activation scales [NG][16]
  static constexpr int RS_OFF = XS_OFF + (A8 ? NG * 64 : 0);   // row sums [NG][16]
  static constexpr int RED_OFF = RS_OFF + (RSUM ? NG * 64 : 0);
  static constexpr int RED_BYTES = 4 * FN * NM * 64 * 16; // one buffer: every wave's partial sums
  static constexpr size_t lds_bytes() { return RED_OFF + 2 * (size_t)RED_BYTES; }
  static_assert(BMR == 8 || BMR == 16, "row tile of 8 or 16");
  static_assert(NBLK % 2 == 0, "blocks alternate between two weight buffers");

  struct W {
    u32x4_t b[NGW][FN][NM][NB];
    uint32_t s[NGW][FN][NM];
  };

  // Expert e, sorted rows [off, off + count); src(r) = A row of local row r.
  // The weight slice of the first block is issued by the caller-independent
  // prologue below before the rows are staged.
  template <class RowSrc>
  __device__ static void run(const GemmProblem& p, int e, int off, int count, RowSrc src, uint8_t* lds) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, kb = lane >> 4;
    const int col_base = blockIdx.x * BCOLS;
    const int64_t mat_bytes = (int64_t)p.n * NG * WGB;
    rsrc_t rw[NM], rs[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      rw[m] = make_rsrc((m == 0 ? p.w0q : p.w1q) + e * mat_bytes, mat_bytes);
      rs[m] = make_rsrc((m == 0 ? p.w0s : p.w1s) + e * (int64_t)p.n * NG, (int64_t)p.n * NG * 2);
    }
    const int g0 = wave * NGW;
    // block k of this workgroup's stream (k counts blocks over all row tiles)
    auto load_w = [&](W& w, int k) {
      const int blk = k % NBLK;
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const uint32_t n = (uint32_t)(col_base + blk * BN + f * 16 + li);
#pragma unroll
        for (int j = 0; j < NGW; ++j)
#pragma unroll
          for (int m = 0; m < NM; ++m) {
#pragma unroll
            for (int q = 0; q < NB; ++q)
              w.b[j][f][m][q] = bload16(rw[m], (n * NG + g0 + j) * WGB + kb * 16 * NB + 16 * q);
            w.s[j][f][m] = bload_u16(rs[m], (n * NG + g0 + j) * 2);
          }
      }
    };

    const int ntiles = (count + BMR - 1) / BMR;
    const int nk = ntiles * NBLK;
    W wb[2];
    load_w(wb[0], 0);

    const uint32_t mask_nib = vconst<0x000f000fu>(), magic = vconst<0x43004300u>();
    const int arow = li & (BMR - 1);                     // LDS row feeding MFMA row li
    uint32_t a_base[STEPS];
#pragma unroll
    for (int t = 0; t < STEPS; ++t)
      a_base[t] = (uint32_t)(arow * ROWB + ((((A8 ? kb * 2 : kb * 4) + t) ^ dswz(arow)) << 4));
    float* xs_lds = reinterpret_cast<float*>(lds + XS_OFF);
    float* rs_lds = reinterpret_cast<float*>(lds + RS_OFF);
    uint16_t* out = static_cast<uint16_t*>(p.out);

    int k = 0;
    for (int t0 = 0; t0 < count; t0 += BMR) {
      const int nrows = min(BMR, count - t0);
      // stage the tile's rows: permuted chunks and per-row group sums
      const uint8_t* a = static_cast<const uint8_t*>(p.a);
      for (int idx = tid; idx < nrows * CPR; idx += blockDim.x) {
        const int r = idx / CPR, c = idx % CPR;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a + src(t0 + r) * ROWB + c * 16);
        *reinterpret_cast<u32x4_t*>(lds + r * ROWB + (((c & ~7) | ((c & 7) ^ dswz(r))) << 4)) = a_operand<WB, A8>(v);
        if constexpr (RSUM) {
          // the CPG chunks of one (row, group) sit in CPG consecutive lanes
          float sum;
          if constexpr (A8) {
            int si = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) si = __builtin_amdgcn_sdot4((int)v[w], 0x01010101, si, false);
#pragma unroll
            for (int d = 1; d < CPG; d <<= 1) si += __shfl_xor(si, d);
            sum = __int_as_float(si);
          } else {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) t += bf16_bits_to_f32(v[w] & 0xffffu) + bf16_bits_to_f32(v[w] >> 16);
#pragma unroll
            for (int d = 1; d < CPG; d <<= 1) t += __shfl_xor(t, d);
            sum = t;
          }
          if (c % CPG == 0) {
            rs_lds[(c / CPG) * 16 + r] = sum;
            if (BMR == 8) rs_lds[(c / CPG) * 16 + r + 8] = sum;   // MFMA rows 8..15 repeat rows 0..7
          }
        }
      }
      if constexpr (A8) {
        for (int idx = tid; idx < nrows * NG; idx += blockDim.x) {
          const int r = idx / NG, g = idx % NG;
          const float x = p.a_scale[src(t0 + r) * NG + g];
          xs_lds[g * 16 + r] = x;
          if (BMR == 8) xs_lds[g * 16 + r + 8] = x;
        }
      }
      __syncthreads();

#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk, ++k) {        // k = tile * NBLK + blk, so k & 1 == blk & 1
        W& cur = wb[blk & 1];
        if (k + 1 < nk) load_w(wb[(blk + 1) & 1], k + 1);   // the next block's slice in flight
        f32x4_t acc[FN][NM];
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int m = 0; m < NM; ++m) acc[f][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NGW; ++j) {
          const int g = g0 + j;
          if constexpr (!A8) {
            f32x4_t part[FN][NM];
#pragma unroll
            for (int t = 0; t < STEPS; ++t) {
              const bf16x8_t av =
                  __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(lds + a_base[t] + g * CPG * 16));
#pragma unroll
              for (int f = 0; f < FN; ++f)
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                  const u32x4_t bv = b_operand_bf16<WB>(cur.b[j][f][m], t, mask_nib, magic);
                  part[f][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      av, __builtin_bit_cast(bf16x8_t, bv), t == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : part[f][m], 0, 0, 0);
                }
            }
            constexpr float kOff = (WB == 4) ? 136.0f : 128.0f;
            const f32x4_t rsum = *reinterpret_cast<const f32x4_t*>(rs_lds + g * 16 + 4 * kb);
#pragma unroll
            for (int f = 0; f < FN; ++f)
#pragma unroll
              for (int m = 0; m < NM; ++m) {
                const float s16 = half_bits_to_f32(cur.s[j][f][m]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  acc[f][m][r] = __builtin_fmaf(s16, __builtin_fmaf(-kOff, rsum[r], part[f][m][r]), acc[f][m][r]);
              }
          } else {
            i32x4_t part[FN][NM];
#pragma unroll
            for (int t = 0; t < STEPS; ++t) {
              const i32x4_t av =
                  __builtin_bit_cast(i32x4_t, *reinterpret_cast<const u32x4_t*>(lds + a_base[t] + g * CPG * 16));
#pragma unroll
              for (int f = 0; f < FN; ++f)
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                  const u32x4_t bv = b_operand_i8<WB>(cur.b[j][f][m], t);
                  part[f][m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                      av, __builtin_bit_cast(i32x4_t, bv), t == 0 ? i32x4_t{0, 0, 0, 0} : part[f][m], 0, 0, 0);
                }
            }
            const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(xs_lds + g * 16 + 4 * kb);
            i32x4_t rs8 = {0, 0, 0, 0};
            if constexpr (RSUM) rs8 = __builtin_bit_cast(i32x4_t, *reinterpret_cast<const f32x4_t*>(rs_lds + g * 16 + 4 * kb));
#pragma unroll
            for (int f = 0; f < FN; ++f)
#pragma unroll
              for (int m = 0; m < NM; ++m) {
                const float ws = half_bits_to_f32(cur.s[j][f][m]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const int isum = RSUM ? part[f][m][r] - 8 * rs8[r] : part[f][m][r];
                  acc[f][m][r] = __builtin_fmaf((float)isum, xs[r] * ws, acc[f][m][r]);
                }
              }
          }
        }
        // partial sums of the four waves; wave w finishes element w of each lane
        float* red = reinterpret_cast<float*>(lds + RED_OFF + (blk & 1) * RED_BYTES);
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int m = 0; m < NM; ++m)
            *reinterpret_cast<f32x4_t*>(red + (((wave * FN + f) * NM + m) * 64 + lane) * 4) = acc[f][m];
        __syncthreads();
        const int row = 4 * kb + wave;
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          float v[NM];
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) sum += red[(((w * FN + f) * NM + m) * 64 + lane) * 4 + wave];
            v[m] = sum;
          }
          if (row < nrows) {
            float o;
            if constexpr (DUAL) o = silu(v[0]) * v[1];
            else o = v[0];
            out[(int64_t)(off + t0 + row) * p.n + col_base + blk * BN + f * 16 + li] = (uint16_t)f32_to_bf16_bits(o);
          }
        }
      }
    }
  }
};

template <int WB, bool A8, int NGW, int BMR>
__global__ __launch_bounds__(256) void k_ks_gate_up(GemmProblem p, RouteOut ra) {
  using K = DecKS<WB, A8, true, 1, NGW, 4, BMR>;
  extern __shared__ __attribute__((aligned(16))) uint8_t ks_lds[];
  __shared__ int rows[kRoutedMaxSlots];                     // e's slots, ascending
  __shared__ int wcnt[2][4];
  const int e = blockIdx.y;
  const ExpertRows er = route_expert(ra, e, blockIdx.x == 0, rows, wcnt);
  if (er.count == 0) return;                                // uniform over the workgroup
  K::run(p, e, er.off, er.count, [&](int r) { return (int64_t)(rows[r] / p.gather_k); }, ks_lds);
}

template <int WB, bool A8, int NGW, int BMR>
__global__ __launch_bounds__(256) void k_ks_down(GemmProblem p, const int32_t* counts, const int32_t* offsets) {
  using K = DecKS<WB, A8, false, 4, NGW, 4, BMR>;
  extern __shared__ __attribute__((aligned(16))) uint8_t ks_lds[];
  const int e = blockIdx.y;
  const int count = counts[e], off = offsets[e];
  if (count == 0) return;
  K::run(p, e, off, count, [&](int r) { return (int64_t)(off + r); }, ks_lds);
}

template <int WB, bool A8, int NGW, int BMR>
hipError_t launch_ks_cfg(const GemmProblem& p, const RouteOut& ro, bool down, hipStream_t stream) {
  if (!down) {
    using K = DecKS<WB, A8, true, 1, NGW, 4, BMR>;
    if (p.n % K::BCOLS) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_ks_gate_up<WB, A8, NGW, BMR>), dim3(p.n / K::BCOLS, ro.E), dim3(256), K::lds_bytes(), stream,
                       p, ro);
  } else {
    using K = DecKS<WB, A8, false, 4, NGW, 4, BMR>;
    if (p.n % K::BCOLS) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_ks_down<WB, A8, NGW, BMR>), dim3(p.n / K::BCOLS, ro.E), dim3(256), K::lds_bytes(), stream,
                       p, ro.counts, ro.offsets);
  }
  return hipGetLastError();
}

template <int WB, bool A8, int BMR>
hipError_t launch_ks_ngw(const GemmProblem& p, const RouteOut& ro, bool down, hipStream_t stream) {
  switch (p.kdim / (4 * kGroup)) {
    case 1: return launch_ks_cfg<WB, A8, 1, BMR>(p, ro, down, stream);
    case 2: return launch_ks_cfg<WB, A8, 2, BMR>(p, ro, down, stream);
    case 3: return launch_ks_cfg<WB, A8, 3, BMR>(p, ro, down, stream);
    case 4: return launch_ks_cfg<WB, A8, 4, BMR>(p, ro, down, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int BMR>
hipError_t launch_ks_mode(const GemmProblem& p, const RouteOut& ro, bool down, hipStream_t stream) {
  if (p.bits == 4) return p.act_int8 ? launch_ks_ngw<4, true, BMR>(p, ro, down, stream)
                                     : launch_ks_ngw<4, false, BMR>(p, ro, down, stream);
  return p.act_int8 ? launch_ks_ngw<8, true, BMR>(p, ro, down, stream)
                    : launch_ks_ngw<8, false, BMR>(p, ro, down, stream);
}

bool ks_dim(int kdim, int n, int bcols) {
  return kdim % (4 * kGroup) == 0 && kdim / (4 * kGroup) <= 4 && n % bcols == 0;
}

}  // namespace

bool ks_applicable(int64_t S, int E, int H, int I) {
  // gate/up: reduction H, 64 columns per workgroup; down: reduction I, 256 columns
  return S <= kRoutedMaxSlots && S <= 4 * (int64_t)E && ks_dim(H, I, 64) && ks_dim(I, H, 256);
}

hipError_t launch_gate_up_ks(const GemmProblem& p, const RouteOut& ro, hipStream_t stream) {
  return launch_ks_mode<8>(p, ro, false, stream);
}

hipError_t launch_down_ks(const GemmProblem& p, const RouteOut& ro, hipStream_t stream) {
  return launch_ks_mode<8>(p, ro, true, stream);
}

}  // namespace qre
