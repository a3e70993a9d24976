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
//  * a workgroup computes a 16-row x 16*FN-column tile (both gate and up for
//    the fused kernel), so each weight byte is read from HBM once per 16-row
//    tile, with 16-byte loads per lane (64 contiguous bytes per weight row per
//    128-group for INT4, 128 for INT8).  Its four waves split the reduction:
//    each takes chunks of GW consecutive 128-groups, issues every load of a
//    chunk before its first MFMA (straight-line code, so the compiler waits
//    for exactly the group it needs next), and the four partial sums are
//    added through LDS in a fixed wave order (deterministic);
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
//  * all loads are raw buffer loads: a masked row or a group past the end of
//    the reduction uses an out-of-range offset, which returns zeros without
//    touching memory, so no load sits behind a branch;
//  * workgroups are (column block, row tile); tiles past the device-side tile
//    count exit at once, so no host readback is needed.
#include "gemm_common.h"

namespace qre {
namespace {

using namespace gk;

template <int WB, bool A8, bool DUAL, int FN, int GW>
struct Gemm16 {
  static constexpr int NM = DUAL ? 2 : 1;                // weight matrices
  static constexpr int NA = A8 ? 2 : 4;                  // 16-byte A chunks per lane per group
  static constexpr int NB = (WB == 4) ? 1 : 2;           // 16-byte B chunks per lane per group
  static constexpr int BN = 16 * FN;                     // columns per workgroup
  static constexpr int NW = 4;                           // waves per workgroup (split the reduction)
  static constexpr int A_GROUP_BYTES = A8 ? kGroup : 2 * kGroup;
  static constexpr int W_GROUP_BYTES = kGroup * WB / 8;

  struct Buf {
    u32x4_t a[NA];
    float xs[4];
    u32x4_t b[FN][NM][NB];
    uint32_t s[FN][NM];
  };

  const GemmProblem& p;
  int wave, lane, li, kb, G, e, row0, nrows, n_blk;
  rsrc_t ra, rxs, rw[NM], rs[NM];
  uint32_t a_off;              // byte offset of this lane's A row (+ k offset), or kOOB
  uint32_t xs_off[4];          // byte offsets of the activation scales of rows 4kb+r (INT8 mode)
  uint32_t w_off[FN];          // byte offset of this lane's weight row in the expert's matrix
  uint32_t s_off[FN];          // byte offset of this lane's scale row


  __device__ Gemm16(const GemmProblem& prob, const Tile& td, int col0) : p(prob) {
    wave = threadIdx.x >> 6;
    lane = threadIdx.x & 63;
    li = lane & 15;
    kb = lane >> 4;
    G = p.kdim / kGroup;
    e = td.e;
    row0 = td.row0;
    nrows = td.nrows;
    n_blk = col0;
    const int64_t a_rows = p.a_rows;
    ra = make_rsrc(p.a, a_rows * G * A_GROUP_BYTES);
    a_off = kOOB;
    if (li < nrows) {
      const int r = row0 + li;
      const int64_t ar = p.gather_k ? (int64_t)(p.sorted_slot[r] / p.gather_k) : (int64_t)r;
      a_off = (uint32_t)(ar * G * A_GROUP_BYTES + kb * 32 * (A8 ? 1 : 2));
    }
    if constexpr (A8) {
      rxs = make_rsrc(p.a_scale, a_rows * G * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * kb + r;
        xs_off[r] = kOOB;
        if (m < nrows) {
          const int64_t ar = p.gather_k ? (int64_t)(p.sorted_slot[row0 + m] / p.gather_k) : (int64_t)(row0 + m);
          xs_off[r] = (uint32_t)(ar * G * 4);
        }
      }
    }
    const int64_t mat_bytes = (int64_t)p.n * G * W_GROUP_BYTES;
    const int64_t smat_bytes = (int64_t)p.n * G * 2;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      rw[m] = make_rsrc((m == 0 ? p.w0q : p.w1q) + e * mat_bytes, mat_bytes);
      rs[m] = make_rsrc((m == 0 ? p.w0s : p.w1s) + e * (int64_t)p.n * G, smat_bytes);
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int n = n_blk + f * 16 + li;
      w_off[f] = (uint32_t)((int64_t)n * G * W_GROUP_BYTES + kb * (WB == 4 ? 16 : 32));
      s_off[f] = (uint32_t)((int64_t)n * G * 2);
    }
  }

  // Issue the loads of group g into bf.  With kCheck, g >= G loads nothing
  // (out-of-range offsets); without it the caller guarantees g < G, and every
  // per-group offset is a compile-time immediate on a per-lane base.  A masked
  // row's base is kOOB, and kOOB plus any in-row offset stays out of range.
  template <bool kCheck>
  __device__ __forceinline__ void load(Buf& bf, int g) const {
    const bool in = !kCheck || g < G;
    // issue order: scales, weights, activations (the MFMAs need the last two,
    // the scales come last in the group's arithmetic, so one wait covers all)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) bf.s[f][m] = bload_u16(rs[m], in ? s_off[f] + 2u * g : kOOB);
    if constexpr (A8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) bf.xs[r] = bload_f32(rxs, in ? xs_off[r] + 4u * g : kOOB);
    }
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint32_t wo = in ? w_off[f] + (uint32_t)g * W_GROUP_BYTES : kOOB;
#pragma unroll
        for (int j = 0; j < NB; ++j) bf.b[f][m][j] = bload16(rw[m], wo + 16 * j);
      }
    const uint32_t ao = in ? a_off + (uint32_t)g * A_GROUP_BYTES : kOOB;
#pragma unroll
    for (int j = 0; j < NA; ++j) bf.a[j] = bload16(ra, ao + 16 * j);
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
      const bf16x8_t a8 = __builtin_bit_cast(bf16x8_t, a_operand<WB, false>(bf.a[t]));
      accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, __builtin_bit_cast(bf16x8_t, ones), accx, 0, 0, 0);
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const u32x4_t bv = b_operand_bf16<WB>(bf.b[f][m], t);
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
      const i32x4_t ai = __builtin_bit_cast(i32x4_t, a_operand<WB, true>(bf.a[t]));
      if constexpr (WB == 4) accx = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, ones, accx, 0, 0, 0);
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const u32x4_t bv = b_operand_i8<WB>(bf.b[f][m], t);
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

  __device__ __forceinline__ void group(const Buf& bf, f32x4_t (&acc)[FN][NM]) const {
    if constexpr (A8) group_i8(bf, acc);
    else group_bf16(bf, acc);
  }

  // Store rows 4kb+r of column li of every fragment (lane layout of the MFMA
  // accumulator), applying SiLU*mul for the fused gate/up GEMM.
  __device__ __forceinline__ void store(const f32x4_t (&v)[FN][NM], int f) const {
    uint16_t* out = static_cast<uint16_t*>(p.out);
    const int64_t col = n_blk + f * 16 + li;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * kb + r;
      if (m < nrows) {
        float o;
        if constexpr (DUAL) o = silu(v[f][0][r]) * v[f][1][r];
        else o = v[f][0][r];
        out[(int64_t)(row0 + m) * p.n + col] = (uint16_t)f32_to_bf16_bits(o);
      }
    }
  }

  // red: LDS [NW][FN][NM][64] of f32x4 partial sums.
  __device__ void run_split(f32x4_t* red) const {
    f32x4_t acc[FN][NM];
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[f][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int c = wave; c * GW < G; c += NW) {        // chunks of GW groups, one per wave at a time
      Buf buf[GW];
#pragma unroll
      for (int j = 0; j < GW; ++j) load<true>(buf[j], c * GW + j);
      // keep every load of the chunk ahead of the first MFMA (the scheduler
      // would otherwise sink loads next to their uses and expose the latency
      // once per group)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < GW; ++j) group(buf[j], acc);
    }
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) red[((wave * FN + f) * NM + m) * 64 + lane] = acc[f][m];
    __syncthreads();
    // epilogue: wave w finishes fragments f = w, w + NW, ...
    for (int f = wave; f < FN; f += NW) {
      f32x4_t v[FN][NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        v[f][m] = red[((0 * FN + f) * NM + m) * 64 + lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) v[f][m] += red[((w * FN + f) * NM + m) * 64 + lane];
      }
      store(v, f);
    }
  }
};

// Row-tile kernel for short expert segments (decode blocks, batched blocks):
// the weights stream once per tile of up to BMR rows, so this path is bound by
// HBM.  The workgroup first copies its tile's activation rows into LDS
// (permuted for the INT4 code order; the 16-byte chunk index XOR-ed with the
// row so the 16 rows of an MFMA operand hit different banks), and every wave
// loads the FP16 scales of its columns once.  Afterwards the only vector-memory
// instructions are the weight loads (16 bytes per lane), DEPTH groups ahead.
// Rows past the tile's last (and, for BMR = 8, MFMA rows 8..15) read arbitrary
// LDS bytes; they only reach accumulator rows that are never stored.
template <int WB, bool A8, bool DUAL, int FN, int NG, int DEPTH, int BMR>
struct Dec16 {
  static constexpr int NM = DUAL ? 2 : 1;
  static constexpr int NB = (WB == 4) ? 1 : 2;
  static constexpr int ELEM = A8 ? 1 : 2;
  static constexpr int ROWB = NG * kGroup * ELEM;           // LDS bytes of one staged row
  static constexpr int CPR = ROWB / 16;                     // 16-byte chunks per row
  static constexpr int STEPS = A8 ? 2 : 4;                  // MFMA steps per 128-group
  static constexpr int W_GROUP_BYTES = kGroup * WB / 8;
  static constexpr int NSW = (NG + 1) / 2;                  // 32-bit words of one column's FP16 scales
  static constexpr int BN = 4 * 16 * FN;                    // columns per workgroup
  static_assert(CPR % 8 == 0, "row swizzle needs 8-chunk rows");

  static constexpr int NC = (NG + 3) / 4;                   // 4-group steps of the offset correction
  // LDS: rows [BMR][ROWB], then [NG][16] FP32: activation scales (INT8) or
  // row sums of each 128-group (BF16, for the 136 + q / 128 + q offset), then
  // the A-source row of each tile row [BMR]
  static constexpr size_t lds_bytes() { return (size_t)BMR * ROWB + (size_t)NG * 16 * 4 + (size_t)BMR * 4; }
  static constexpr int NCH = (BMR * CPR + 255) / 256;       // staged chunks per thread at most
  // chunk loads in flight together (8-row tiles: decode blocks, one or two
  // rows per tile, where registers go to the weight look-ahead)
  static constexpr int SBATCH = (BMR == 8) ? 1 : (NCH < 8 ? NCH : 8);

  struct WBuf {
    u32x4_t b[FN][NM][NB];
  };

  // chunk c of staged row r sits at c ^ swz(r): any 16 aligned consecutive
  // rows put a chunk in 16 distinct 16-byte bank groups of a 256-byte window
  __device__ static int swz(int r) { return (r ^ ((r >> 3) & 1)) & 7; }
  __device__ static uint32_t lds_chunk(int row, int chunk) { return (uint32_t)(row * ROWB + ((chunk ^ swz(row)) << 4)); }

  // Tile: rows [row0, row0 + nrows) (sorted order) of expert e; src(r) gives
  // the A-source row of local row r (a token for gate/up, a sorted row for
  // down); store(m, col, v) receives the FP32 result of local row m < nrows
  // (SiLU(gate) * up for the fused projection) before any rounding.
  // Column block cb: the workgroup's waves take columns (4 cb + wave) 16 FN.
  // With stage = false the rows staged by an earlier call (same tile) are
  // reused: no staging, no barrier.
  template <class RowSrc, class Store>
  __device__ static void run(const GemmProblem& p, int e, int row0, int nrows, RowSrc src_row, Store store,
                             uint8_t* lds, int cb, bool stage = true) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, kb = lane >> 4;
    int* s_src = reinterpret_cast<int*>(lds + (size_t)BMR * ROWB + (size_t)NG * 16 * 4);   // [BMR]
    // 0. the A-source rows of the tile, requested before the weights so that
    //    waiting for them does not wait for the weight stream
    if (stage && tid < BMR) s_src[tid] = tid < nrows ? (int)src_row(tid) : 0;
    // 1. per-wave descriptors, weight offsets, all scales of its columns and
    //    the first DEPTH groups of weights: issued before the activation rows
    //    are staged, so the weight stream starts at once
    const int col0 = min((cb * 4 + wave) * 16 * FN, p.n - 16 * FN);   // a surplus wave re-reads the last tile and stores nothing
    const int64_t mat_bytes = (int64_t)p.n * NG * W_GROUP_BYTES;
    const int64_t smat_bytes = (int64_t)p.n * NG * 2;
    rsrc_t rw[NM], rs[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      rw[m] = make_rsrc((m == 0 ? p.w0q : p.w1q) + e * mat_bytes, mat_bytes);
      rs[m] = make_rsrc((m == 0 ? p.w0s : p.w1s) + e * (int64_t)p.n * NG, smat_bytes);
    }
    uint32_t w_off[FN];
    uint32_t sc[FN][NM][NSW];   // FP16 scales of the lane's column, two per word
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int n = col0 + f * 16 + li;
      w_off[f] = (uint32_t)(n * NG * W_GROUP_BYTES + kb * (WB == 4 ? 16 : 32));
      const uint32_t so = (uint32_t)(n * NG * 2);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        // loads never cross the end of the column's scale row (a buffer load
        // that straddles the end of its descriptor returns zeros)
        if constexpr (NG % 8 == 0) {
#pragma unroll
          for (int q = 0; q < NG / 8; ++q) {
            const u32x4_t v = bload16(rs[m], so + 16 * q);
#pragma unroll
            for (int j = 0; j < 4; ++j) sc[f][m][4 * q + j] = v[j];
          }
        } else if constexpr (NG % 2 == 0) {
#pragma unroll
          for (int q = 0; q < NSW; ++q)
            sc[f][m][q] = __builtin_amdgcn_raw_buffer_load_b32(rs[m], so + 4 * q, 0, 0);
        } else {
#pragma unroll
          for (int q = 0; q < NSW; ++q) {
            const uint32_t lo = bload_u16(rs[m], so + 4 * q);
            const uint32_t hi = (2 * q + 1 < NG) ? bload_u16(rs[m], so + 4 * q + 2) : 0u;
            sc[f][m][q] = lo | (hi << 16);
          }
        }
      }
    }
    // BF16: FP32 scales of the lane's column for groups 4i + kb, the B operand
    // of the offset correction (an FP32 MFMA over groups after the stream)
    float csc[FN][NM][NC];
    if constexpr (!A8) {
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            const int g = 4 * i + kb;
            const uint32_t n = (uint32_t)(col0 + f * 16 + li);
            csc[f][m][i] = half_bits_to_f32(bload_u16(rs[m], g < NG ? (n * NG + g) * 2 : kOOB));
          }
    }
    const int arow = (BMR == 16) ? li : (li & (BMR - 1));   // LDS row feeding MFMA row li
    // the swizzle only touches the low 3 bits of a chunk index and a group
    // spans a multiple of 8 chunks, so every A read is a per-lane base plus a
    // compile-time group offset (folded into the LDS instruction)
    uint32_t a_base[STEPS];
#pragma unroll
    for (int t = 0; t < STEPS; ++t) a_base[t] = lds_chunk(arow, (A8 ? kb * 2 : kb * 4) + t);

    f32x4_t acc[FN][NM];
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[f][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    WBuf buf[DEPTH];
    auto load_group = [&](WBuf& bf, int g) {
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            bf.b[f][m][j] = bload16(rw[m], w_off[f] + (uint32_t)(g * W_GROUP_BYTES + 16 * j));
    };
#pragma unroll
    for (int j = 0; j < DEPTH && j < NG; ++j) {
      load_group(buf[j], j);
      __builtin_amdgcn_sched_barrier(0);
    }
    // 2. stage the tile's activation rows (and INT8 scales) into LDS.  The
    //    chunk loads go out SBATCH at a time, so staging waits for memory
    //    NCH / SBATCH times; the first wait also covers the weights in flight.
    float* xs_lds = reinterpret_cast<float*>(lds + (size_t)BMR * ROWB);   // [NG][16]
    if (stage) {
      __syncthreads();                                      // s_src
      const rsrc_t ra = make_rsrc(p.a, p.a_rows * (int64_t)ROWB);
      const int nch = nrows * CPR;
#pragma unroll 1
      for (int k0 = 0; k0 < NCH && k0 * 256 < nch; k0 += SBATCH) {   // uniform; only the batches holding rows
        u32x4_t v[SBATCH];
#pragma unroll
        for (int k = 0; k < SBATCH; ++k) {
          const int idx = tid + (k0 + k) * 256;
          const int r = idx / CPR, c = idx - r * CPR;
          const bool in = k0 + k < NCH && idx < nch;
          v[k] = bload16(ra, in ? (uint32_t)(s_src[in ? r : 0] * ROWB + c * 16) : kOOB);
        }
#pragma unroll
        for (int k = 0; k < SBATCH; ++k) {
          const int idx = tid + (k0 + k) * 256;
          const int r = idx / CPR, c = idx - r * CPR;
          const bool in = k0 + k < NCH && idx < nch;
          if constexpr (!A8) {
            // row sum of the 128-group: 8 values per lane, 16 consecutive
            // lanes (one DPP row; the xor-butterfly order)
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) t = add_bf16x2(v[k][w], t);
            t = row16_sum(t);
            if (in && (c & 15) == 0) {
              xs_lds[(c >> 4) * 16 + r] = t;
              if (BMR == 8) xs_lds[(c >> 4) * 16 + r + 8] = t;   // MFMA rows 8..15 repeat rows 0..7
            }
          }
          if (in) *reinterpret_cast<u32x4_t*>(lds + lds_chunk(r, c)) = a_operand<WB, A8>(v[k]);
        }
      }
      if constexpr (A8) {
        for (int idx = tid; idx < nrows * NG; idx += blockDim.x) {
          const int r = idx / NG, g = idx % NG;
          xs_lds[g * 16 + r] = p.a_scale[(int64_t)s_src[r] * NG + g];
        }
      }
      __syncthreads();
    }
    if ((cb * 4 + wave) * 16 * FN >= p.n) return;   // wave-uniform, after the barrier

    // 3. the weight stream

#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const WBuf& bf = buf[g % DEPTH];
      if constexpr (!A8) {
        f32x4_t accg[FN][NM];
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
          const u32x4_t av = *reinterpret_cast<const u32x4_t*>(lds + a_base[t] + g * 256);
          const bf16x8_t a8 = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
          for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
              const u32x4_t bv = b_operand_bf16<WB>(bf.b[f][m], t);
              accg[f][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  a8, __builtin_bit_cast(bf16x8_t, bv), t == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : accg[f][m], 0, 0, 0);
            }
        }
        // the offset (136 + q / 128 + q) is removed once, after the stream
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const uint32_t word = sc[f][m][g >> 1];
            const float s16 = half_bits_to_f32((g & 1) ? (word >> 16) : (word & 0xffffu));
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[f][m][r] = __builtin_fmaf(s16, accg[f][m][r], acc[f][m][r]);
          }
      } else {
        i32x4_t accg[FN][NM];
        i32x4_t accx = {0, 0, 0, 0};
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int m = 0; m < NM; ++m) accg[f][m] = i32x4_t{0, 0, 0, 0};
        const i32x4_t ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
          const u32x4_t av = *reinterpret_cast<const u32x4_t*>(lds + a_base[t] + g * 128);
          const i32x4_t ai = __builtin_bit_cast(i32x4_t, av);
          if constexpr (WB == 4) accx = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, ones, accx, 0, 0, 0);
#pragma unroll
          for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
              const u32x4_t bv = b_operand_i8<WB>(bf.b[f][m], t);
              accg[f][m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, __builtin_bit_cast(i32x4_t, bv), accg[f][m],
                                                                 0, 0, 0);
            }
        }
        const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(xs_lds + g * 16 + 4 * kb);
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const uint32_t word = sc[f][m][g >> 1];
            const float ws = half_bits_to_f32((g & 1) ? (word >> 16) : (word & 0xffffu));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int isum = (WB == 4) ? accg[f][m][r] - 8 * accx[r] : accg[f][m][r];
              acc[f][m][r] = __builtin_fmaf((float)isum, xs[r] * ws, acc[f][m][r]);
            }
          }
      }
      // finish this group's scaling now (otherwise the FMA chain is deferred
      // to the end and every group's partial sums stay live)
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < NM; ++m) asm volatile("" : "+v"(acc[f][m]));
      if (g + DEPTH < NG) load_group(buf[g % DEPTH], g + DEPTH);
      __builtin_amdgcn_sched_barrier(0);
    }
    // 4. BF16: subtract offset * sum_g s[col][g] * rowsum[row][g], an FP32
    //    MFMA over groups (lane (li, kb) feeds row li / column li, group 4i + kb)
    if constexpr (!A8) {
      constexpr float kOff = (WB == 4) ? 136.0f : 128.0f;
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          f32x4_t corr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            const int g = 4 * i + kb;
            const float ra = g < NG ? xs_lds[g * 16 + li] : 0.f;
            corr = __builtin_amdgcn_mfma_f32_16x16x4f32(ra, csc[f][m][i], corr, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[f][m][r] = __builtin_fmaf(-kOff, corr[r], acc[f][m][r]);
        }
    }
    // 5. epilogue: lane holds rows 4kb+r of column li of each fragment
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int col = col0 + f * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * kb + r;
        if (m < nrows) {
          float o;
          if constexpr (DUAL) o = silu(acc[f][0][r]) * acc[f][1][r];
          else o = acc[f][0][r];
          store(m, col, o);
        }
      }
    }
  }
};

// Store functor of the row-tile kernels: BF16 rows of p.out from row0.
struct GlobalRowStore {
  uint16_t* out;
  int64_t row0;
  int n;
  __device__ void operator()(int m, int col, float v) const {
    out[(row0 + m) * n + col] = (uint16_t)f32_to_bf16_bits(v);
  }
};

template <int WB, bool A8, bool DUAL, int FN, int NG, int DEPTH, int BMR>
__global__ __launch_bounds__(256) void k_gemm_dec(GemmProblem p) {
  using K = Dec16<WB, A8, DUAL, FN, NG, DEPTH, BMR>;
  extern __shared__ __attribute__((aligned(16))) uint8_t dec_lds[];
  int tile, cb;
  if (!xcd_tile(p, tile, cb)) return;   // an expert's tiles and a tile's column blocks share one L2
  const Tile td = p.tiles[tile];
  const int row0 = td.row0;
  const GlobalRowStore st{static_cast<uint16_t*>(p.out), row0, p.n};
  if (p.gather_k) {
    K::run(p, td.e, row0, td.nrows, [&](int r) { return (int64_t)(p.sorted_slot[row0 + r] / p.gather_k); }, st,
           dec_lds, cb);
  } else {
    K::run(p, td.e, row0, td.nrows, [&](int r) { return (int64_t)(row0 + r); }, st, dec_lds, cb);
  }
}

// Decode blocks with the permutation folded in.  Workgroup (column block, e):
// the gate/up kernel finds expert e's slots itself (per 64 slots, one ballot
// for id == e and one for 0 <= id < e, so its rows are e's slots in ascending
// order and its first sorted row is the number of valid slots with a smaller
// id: the stable counting sort), writes expert e's part of counts, offsets,
// sorted_slot and slot_row (column block 0 only), then runs the row tiles.
// The down kernel reads counts/offsets back.  Used for small slot counts,
// where every workgroup re-reading all ids is cheap.
template <int WB, bool A8, int NG, int DEPTH, int BMR>
__global__ __launch_bounds__(256) void k_gate_up_routed(GemmProblem p, RouteOut ra) {
  using K = Dec16<WB, A8, true, 1, NG, DEPTH, BMR>;
  extern __shared__ __attribute__((aligned(16))) uint8_t dec_lds[];
  __shared__ int rows[kRoutedMaxSlots];                     // e's slots, ascending
  __shared__ int wcnt[2][4];
  const int e = blockIdx.y;
  const ExpertRows er = route_expert(ra, e, blockIdx.x == 0, rows, wcnt);
  const int count = er.count, off = er.off;
  if (count == 0) return;                                   // uniform over the workgroup
  for (int t0 = 0; t0 < count; t0 += BMR) {
    // an opaque copy of e keeps the compiler from hoisting the weight loads
    // out of this loop (they would all stay live in registers)
    int ev = e;
    asm volatile("" : "+s"(ev));
    K::run(p, ev, off + t0, min(BMR, count - t0), [&](int r) { return (int64_t)(rows[t0 + r] / p.gather_k); },
           GlobalRowStore{static_cast<uint16_t*>(p.out), off + t0, p.n}, dec_lds, blockIdx.x);
    __syncthreads();                                        // the LDS tile is reused by the next row tile
  }
}

// Columns per wave of the routed down GEMM: one 16-column fragment.  With one
// or two rows per expert a workgroup streams 64 columns x the short
// reduction, and more, smaller workgroups keep more of the weight stream in
// flight than two fragments per wave did (about 1 us per decode step).
constexpr int kDownRoutedFn = 1;
template <int WB, bool A8, int NG, int DEPTH, int BMR>
__global__ __launch_bounds__(256) void k_down_routed(GemmProblem p, const int32_t* counts, const int32_t* offsets) {
  using K = Dec16<WB, A8, false, kDownRoutedFn, NG, DEPTH, BMR>;
  extern __shared__ __attribute__((aligned(16))) uint8_t dec_lds[];
  const int e = blockIdx.y;
  const int count = counts[e], off = offsets[e];
  for (int t0 = 0; t0 < count; t0 += BMR) {
    const int row0 = off + t0;
    int ev = e;                                             // opaque: no hoisting of weight loads
    asm volatile("" : "+s"(ev));
    K::run(p, ev, row0, min(BMR, count - t0), [&](int r) { return (int64_t)(row0 + r); },
           GlobalRowStore{static_cast<uint16_t*>(p.out), row0, p.n}, dec_lds, blockIdx.x);
    __syncthreads();
  }
}

template <int WB, bool A8, bool DUAL, int FN, int NG, int DEPTH, int BMR>
hipError_t launch_dec(const GemmProblem& p, hipStream_t stream) {
  using K = Dec16<WB, A8, DUAL, FN, NG, DEPTH, BMR>;
  const dim3 grid((p.n + K::BN - 1) / K::BN, (unsigned)((p.max_tiles + 7) / 8 * 8));
  QRE_LAUNCH_GEMM((k_gemm_dec<WB, A8, DUAL, FN, NG, DEPTH, BMR>), grid, dim3(256), K::lds_bytes(), stream, p);
  return hipGetLastError();
}

// Split-reduction kernel (any reduction length): workgroup = one 16 x 16*FN
// tile, four waves over the groups, LDS reduction.
template <int WB, bool A8, bool DUAL, int FN, int GW>
__global__ __launch_bounds__(256) void k_gemm16(GemmProblem p) {
  using K = Gemm16<WB, A8, DUAL, FN, GW>;
  __shared__ f32x4_t red[K::NW * FN * K::NM * 64];
  if ((int)blockIdx.y >= *p.ntiles) return;                 // tile past the routed rows
  const Tile td = p.tiles[blockIdx.y];
  K g(p, td, blockIdx.x * K::BN);
  g.run_split(red);
}

template <int WB, bool A8, bool DUAL, int FN, int GW>
hipError_t launch_split(const GemmProblem& p, hipStream_t stream) {
  constexpr int BN = 16 * FN;
  const dim3 grid((p.n + BN - 1) / BN, (unsigned)p.max_tiles);
  QRE_LAUNCH_GEMM((k_gemm16<WB, A8, DUAL, FN, GW>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Largest activation tile (rows x kdim x element bytes) the decode kernel stages in LDS.
constexpr int64_t kDecLdsMax = 64 * 1024;

template <int WB, bool A8, bool DUAL, int NG, int BMR>
hipError_t launch_dec_ng(const GemmProblem& p, hipStream_t stream) {
  // the fused gate/up GEMM streams two matrices per column, so one 16-column
  // fragment per wave; the down GEMM streams one, so two.  DEPTH groups of
  // weight loads in flight (64 VGPRs of INT4 / 128 of INT8 per wave).  With
  // 16-row tiles the staged rows already limit LDS to two workgroups per CU,
  // so the gate/up waves take two fragments each (twice the columns per
  // staged tile, more weight bytes in flight), with a shallower look-ahead
  // that keeps two waves per SIMD.
  constexpr int FN = DUAL ? (BMR == 16 ? 2 : 1) : 2;
  constexpr int DMAX = (DUAL && BMR == 16) ? (WB == 8 ? 3 : 6) : 8;
  constexpr int DEPTH = (NG < DMAX) ? NG : DMAX;
  return launch_dec<WB, A8, DUAL, FN, NG, DEPTH, BMR>(p, stream);
}

template <int WB, bool A8, bool DUAL, int BMR>
hipError_t launch_dec_shape(const GemmProblem& p, hipStream_t stream, bool* done) {
  *done = true;
  switch (p.kdim / kGroup) {
    case 1: return launch_dec_ng<WB, A8, DUAL, 1, BMR>(p, stream);
    case 2: return launch_dec_ng<WB, A8, DUAL, 2, BMR>(p, stream);
    case 3: return launch_dec_ng<WB, A8, DUAL, 3, BMR>(p, stream);
    case 4: return launch_dec_ng<WB, A8, DUAL, 4, BMR>(p, stream);
    case 5: return launch_dec_ng<WB, A8, DUAL, 5, BMR>(p, stream);
    case 8: return launch_dec_ng<WB, A8, DUAL, 8, BMR>(p, stream);
    case 12: return launch_dec_ng<WB, A8, DUAL, 12, BMR>(p, stream);
    case 16: return launch_dec_ng<WB, A8, DUAL, 16, BMR>(p, stream);
    case 32: return launch_dec_ng<WB, A8, DUAL, 32, BMR>(p, stream);
    default: *done = false; return hipSuccess;
  }
}

// Kernel choice: the LDS-staged decode kernel when the reduction length is one
// of the usual expert shapes and the activation tile fits in LDS; otherwise the
// split-reduction kernel (any reduction length).
template <int WB, bool A8, bool DUAL>
hipError_t launch_shape(const GemmProblem& p, hipStream_t stream) {
  // LDS of the decode kernel: staged rows (8 or 16) x kdim x element bytes,
  // plus the FP32 activation scales of 16 rows in INT8 mode
  const int64_t rows = (p.bm <= 8) ? 8 : 16;
  const int64_t tile_bytes = rows * p.kdim * (A8 ? 1 : 2) + (A8 ? (int64_t)(p.kdim / kGroup) * 16 * 4 : 0);
  if (tile_bytes <= kDecLdsMax) {
    bool done = false;
    hipError_t e = (p.bm <= 8) ? launch_dec_shape<WB, A8, DUAL, 8>(p, stream, &done)
                               : launch_dec_shape<WB, A8, DUAL, 16>(p, stream, &done);
    if (done) return e;
  }
  if constexpr (DUAL) return launch_split<WB, A8, DUAL, 1, 1>(p, stream);
  else return launch_split<WB, A8, DUAL, 4, 1>(p, stream);
}

template <int WB, bool A8, int NG, int BMR>
hipError_t launch_routed_ng(const GemmProblem& gu, const GemmProblem& dn, const RouteOut& ro, bool down,
                            hipStream_t stream) {
  constexpr int DEPTH = (NG < 8) ? NG : 8;
  if (!down) {
    using K = Dec16<WB, A8, true, 1, NG, DEPTH, BMR>;
    const dim3 grid((gu.n + K::BN - 1) / K::BN, ro.E);
    QRE_LAUNCH_GEMM((k_gate_up_routed<WB, A8, NG, DEPTH, BMR>), grid, dim3(256), K::lds_bytes(), stream, gu, ro);
  } else {
    using K = Dec16<WB, A8, false, kDownRoutedFn, NG, DEPTH, BMR>;
    const dim3 grid((dn.n + K::BN - 1) / K::BN, ro.E);
    QRE_LAUNCH_GEMM((k_down_routed<WB, A8, NG, DEPTH, BMR>), grid, dim3(256), K::lds_bytes(), stream, dn,
                       ro.counts, ro.offsets);
  }
  return hipGetLastError();
}

template <int WB, bool A8, int BMR>
hipError_t launch_routed_g(int G, const GemmProblem& gu, const GemmProblem& dn, const RouteOut& ro, bool down,
                           hipStream_t stream) {
  switch (G) {
    case 1: return launch_routed_ng<WB, A8, 1, BMR>(gu, dn, ro, down, stream);
    case 2: return launch_routed_ng<WB, A8, 2, BMR>(gu, dn, ro, down, stream);
    case 3: return launch_routed_ng<WB, A8, 3, BMR>(gu, dn, ro, down, stream);
    case 4: return launch_routed_ng<WB, A8, 4, BMR>(gu, dn, ro, down, stream);
    case 5: return launch_routed_ng<WB, A8, 5, BMR>(gu, dn, ro, down, stream);
    case 8: return launch_routed_ng<WB, A8, 8, BMR>(gu, dn, ro, down, stream);
    case 12: return launch_routed_ng<WB, A8, 12, BMR>(gu, dn, ro, down, stream);
    case 16: return launch_routed_ng<WB, A8, 16, BMR>(gu, dn, ro, down, stream);
    case 32: return launch_routed_ng<WB, A8, 32, BMR>(gu, dn, ro, down, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int WB, bool A8>
hipError_t launch_routed_mode(const GemmProblem& gu, const GemmProblem& dn, const RouteOut& ro, bool down,
                              hipStream_t stream) {
  const int G = (down ? dn.kdim : gu.kdim) / kGroup;
  return (gu.bm <= 8) ? launch_routed_g<WB, A8, 8>(G, gu, dn, ro, down, stream)
                      : launch_routed_g<WB, A8, 16>(G, gu, dn, ro, down, stream);
}

}  // namespace

// Row-tile height: 8 when experts see only a few rows each (decode blocks: the
// weights stream once per tile either way, and a smaller activation tile leaves
// LDS for more workgroups), 16 otherwise; the big-tile kernels' height (64 or
// 128) when experts average 64 rows or more.
int gemm_tile_rows(int64_t S, int E, int, int kdim, int act_int8) {
  return big_applicable(S, E, kdim) ? big_tile_rows(act_int8) : (S <= 4 * (int64_t)E) ? 8 : 16;
}

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream) {
  if (p.max_tiles == 0 || p.n == 0) return hipSuccess;
  if (p.bm >= 64) return launch_gemm_big(p, stream);
  const bool dual = p.w1q != nullptr;
  if (p.bits == 4) {
    if (p.act_int8) return dual ? launch_shape<4, true, true>(p, stream) : launch_shape<4, true, false>(p, stream);
    return dual ? launch_shape<4, false, true>(p, stream) : launch_shape<4, false, false>(p, stream);
  }
  if (p.act_int8) return dual ? launch_shape<8, true, true>(p, stream) : launch_shape<8, true, false>(p, stream);
  return dual ? launch_shape<8, false, true>(p, stream) : launch_shape<8, false, false>(p, stream);
}

bool routed_applicable(int64_t S, int E, int H, int I, int act_int8) {
  if (S > kRoutedMaxSlots || big_applicable(S, E, H) || big_applicable(S, E, I)) return false;
  auto ok_g = [](int G) { return (G >= 1 && G <= 5) || G == 8 || G == 12 || G == 16 || G == 32; };
  if (!ok_g(H / kGroup) || !ok_g(I / kGroup)) return false;
  const int64_t rows = (S <= 4 * (int64_t)E) ? 8 : 16;
  const int64_t elem = act_int8 ? 1 : 2;
  const int64_t extra_h = act_int8 ? (int64_t)(H / kGroup) * 64 : 0, extra_i = act_int8 ? (int64_t)(I / kGroup) * 64 : 0;
  return rows * H * elem + extra_h <= kDecLdsMax && rows * I * elem + extra_i <= kDecLdsMax;
}

hipError_t launch_gate_up_routed(const GemmProblem& p, const RouteOut& ro, hipStream_t stream) {
  const GemmProblem& dn = p;
  if (p.bits == 4) return p.act_int8 ? launch_routed_mode<4, true>(p, dn, ro, false, stream)
                                     : launch_routed_mode<4, false>(p, dn, ro, false, stream);
  return p.act_int8 ? launch_routed_mode<8, true>(p, dn, ro, false, stream)
                    : launch_routed_mode<8, false>(p, dn, ro, false, stream);
}

hipError_t launch_down_routed(const GemmProblem& p, const RouteOut& ro, hipStream_t stream) {
  if (p.bits == 4) return p.act_int8 ? launch_routed_mode<4, true>(p, p, ro, true, stream)
                                     : launch_routed_mode<4, false>(p, p, ro, true, stream);
  return p.act_int8 ? launch_routed_mode<8, true>(p, p, ro, true, stream)
                    : launch_routed_mode<8, false>(p, p, ro, true, stream);
}

}  // namespace qre
