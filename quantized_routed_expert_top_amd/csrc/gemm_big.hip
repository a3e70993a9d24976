// Grouped expert GEMMs for many rows per expert (prefill), CDNA4 (gfx950).
//
// Same arithmetic as the decode kernels (gemm.hip, gemm_common.h), which the
// pages fix (minnow README, section "Quantization"; model card "LLaDA2.2-flash
// for minnow", paragraphs after the precision table): weights dequantized in
// registers, BF16 activations on BF16 MFMAs (FP32 sums) or INT8 activations
// on INT8 MFMAs (exact INT32 sums per 128-group), each group's sum scaled in
// FP32 and the groups added in FP32.  The tiling is this kernel's own, made
// for tiles that the matrix cores, not HBM, bound:
//  * workgroup tile: four waves, each 64 sorted rows x 64 weight rows
//    (sixteen 16x16 MFMA tiles).  BF16 activations: the waves side by side
//    along the weight rows (64 sorted rows of one expert x 256 weight rows),
//    so each weight column is loaded and dequantized by one wave only and a
//    staged activation row serves 256 weight rows; INT8 activations: 2 x 2
//    (128 rows x 128 weight rows).  The fused gate/up kernel takes half its
//    weight rows from gate and the same columns from up;
//  * the reduction is walked one 128-group at a time: the group's activation
//    rows are staged into LDS (double-buffered, XOR-swizzled 16-byte chunks,
//    already permuted into the operand order), together with one FP32 per row
//    (the activation scale for INT8 activations; for BF16 activations the
//    row sum times -136 / -128, which removes the 136 + q / 128 + q offset);
//    each wave loads its own weight columns straight into registers (16-byte
//    buffer loads, next group in flight while the current one computes);
//  * per group: MFMAs into a per-group accumulator, then one FP32 update of
//    the running sums (INT8: acc += float(isum) * (xs * ws); BF16: the
//    group's MFMAs start from -offset * rowsum, then acc += ws * gsum), one
//    barrier per group;
//  * epilogue: SiLU(gate) * up (fused kernel) or the plain sum, rounded to
//    BF16, rows past the tile's end masked.
#include <type_traits>

#include "gemm_common.h"

namespace qre {
namespace {

using namespace gk;

// s_waitcnt immediates waiting for vmcnt <= n only (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
constexpr int vmcnt_enc(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kLgkmcnt0 = 15 | (3 << 14) | (7 << 4);   // lgkmcnt(0), vmcnt and expcnt at their maxima
constexpr int kVmcntEnc[17] = {vmcnt_enc(0),  vmcnt_enc(1),  vmcnt_enc(2),  vmcnt_enc(3),  vmcnt_enc(4),  vmcnt_enc(5),
                               vmcnt_enc(6),  vmcnt_enc(7),  vmcnt_enc(8),  vmcnt_enc(9),  vmcnt_enc(10), vmcnt_enc(11),
                               vmcnt_enc(12), vmcnt_enc(13), vmcnt_enc(14), vmcnt_enc(15), vmcnt_enc(16)};

// 16-byte chunk swizzle of a staged row: chunk c of row r sits at position
// c ^ swz(r).  Any 16 aligned consecutive rows then put a given chunk at 16
// distinct 16-byte bank groups of a 256-byte window, and any 8 at 8 distinct
// groups of a 128-byte window, so the MFMA operand reads (16 rows x one chunk
// per 16 lanes) are conflict-free.  swz depends on r mod 16 only, so row
// tiles 16 apart share read offsets up to a constant.
__device__ __forceinline__ int swz(int r) { return (r ^ ((r >> 3) & 1)) & 7; }

template <int WB, bool A8, bool DUAL, int WM = 2>
struct Big {
  static constexpr int WN = 4 / WM;                // waves along the weight rows (WM along the sorted rows)
  static constexpr int BM = 64 * WM;               // sorted rows per tile
  static constexpr int BNO = (DUAL ? 32 : 64) * WN;   // output columns per workgroup
  static constexpr int TM = 4, TN = 4;             // 16x16 tiles per wave (64 x 64)
  static constexpr int ELEM = A8 ? 1 : 2;
  static constexpr int GB = kGroup * ELEM;         // bytes of one row's 128-group
  static constexpr int CPG = GB / 16;              // 16-byte chunks per row-group
  static constexpr int STEPS = A8 ? 2 : 4;         // MFMA steps per group
  static constexpr int NB = (WB == 4) ? 1 : 2;     // 16-byte weight loads per lane per (tile, group)
  static constexpr int WGB = kGroup * WB / 8;      // weight bytes per (column, group)
  static constexpr int A_STAGE = BM * GB;          // LDS bytes of one staged A group
  static constexpr bool RS8 = A8 && WB == 4;       // INT4 codes with INT8 activations need INT8 row sums
  static constexpr int STAGE = A_STAGE + BM * 4 * (RS8 ? 2 : 1);   // + one FP32 per row (+ one INT32)
  static constexpr int CPT = BM * CPG / 256;       // staged chunks per thread
  static constexpr int RPI = 256 / CPG;            // rows covered per staging round
  static constexpr int NH = A8 ? 1 : 2;            // staging halves (BF16: half a group in flight at a time)
  static constexpr int QH = CPT / NH;              // staged chunks per thread per half
  static constexpr size_t lds_bytes() { return 2 * (size_t)STAGE; }
  static_assert(A8 || CPG == 16, "BF16 row-groups span one 16-lane DPP row");

  __device__ static uint32_t lds_chunk(int row, int chunk) { return (uint32_t)(row * GB + ((chunk ^ swz(row)) << 4)); }

  static constexpr float kOff = (WB == 4) ? 136.0f : 128.0f;   // BF16 operand offset of the codes

  // tile: rows [row0, row0 + nrows) of expert e; src(r) = A row of local row r
  template <class RowSrc>
  __device__ static void run(const GemmProblem& p, int cb, int e, int row0, int nrows, RowSrc src, uint8_t* lds) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, kb = lane >> 4;
    const int wm = wave % WM, wn = wave / WM;
    const int live = min(TM, max(0, (nrows - wm * 64 + 15) >> 4));   // 16-row blocks holding rows (uniform)
    const int NG = p.kdim / kGroup;
    const int n0 = cb * BNO;
    // a wave whose columns lie past n (the last column block of a width that
    // is not a multiple of BNO) reads zeros through the buffer bound and
    // stores nothing
    const bool wcols = n0 + wn * (DUAL ? 32 : 64) < p.n;

    // weights: column of each 16-wide tile this lane feeds
    const int64_t mat_bytes = (int64_t)p.n * NG * WGB;
    rsrc_t rw[DUAL ? 2 : 1], rs[DUAL ? 2 : 1];
#pragma unroll
    for (int m = 0; m < (DUAL ? 2 : 1); ++m) {
      rw[m] = make_rsrc((m == 0 ? p.w0q : p.w1q) + e * mat_bytes, mat_bytes);
      rs[m] = make_rsrc((m == 0 ? p.w0s : p.w1s) + e * (int64_t)p.n * NG, (int64_t)p.n * NG * 2);
    }
    uint32_t wcol[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j)
      wcol[j] = DUAL ? (uint32_t)(n0 + wn * 32 + (j & 1) * 16 + li) : (uint32_t)(n0 + wn * 64 + j * 16 + li);
    auto wsrc = [&](int j) -> const rsrc_t& { return rw[DUAL ? (j >> 1) : 0]; };
    auto ssrc = [&](int j) -> const rsrc_t& { return rs[DUAL ? (j >> 1) : 0]; };

    // activations: the rows this thread stages
    const rsrc_t ra = make_rsrc(p.a, p.a_rows * (int64_t)NG * GB);
    const rsrc_t rx = make_rsrc(p.a_scale, A8 ? p.a_rows * (int64_t)NG * 4 : 0);
    const int sc = tid % CPG;                        // chunk within the row-group
    uint32_t a_off[CPT];
    int aux_src[CPT];                                // A row (or -1) for the per-row FP32
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int r = tid / CPG + RPI * q;
      const int64_t s = r < nrows ? src(r) : -1;
      a_off[q] = s >= 0 ? (uint32_t)(s * NG * GB) + (uint32_t)(sc * 16) : kOOB;
      aux_src[q] = (int)s;
    }

    // staging of half h of a group: chunks q in [h*QH, (h+1)*QH) of this thread
    auto load_a = [&](u32x4_t* v, float* xs, int g, int h) {
#pragma unroll
      for (int k = 0; k < QH; ++k) v[k] = bload16(ra, a_off[h * QH + k] + (uint32_t)(g * GB));
      if constexpr (A8) {
#pragma unroll
        for (int k = 0; k < QH; ++k) {
          const int q = h * QH + k;
          xs[k] = (sc == 0) ? bload_f32(rx, aux_src[q] >= 0 ? (uint32_t)((aux_src[q] * NG + g) * 4) : kOOB) : 0.f;
        }
      }
    };
    // write a staged half to LDS buffer b: permuted chunks, plus the per-row FP32
    auto store_a = [&](const u32x4_t* v, const float* xs, int b, int h) {
      uint8_t* base = lds + b * STAGE;
      float* aux = reinterpret_cast<float*>(base + A_STAGE);
#pragma unroll
      for (int k = 0; k < QH; ++k) {
        const int q = h * QH + k;
        const int r = tid / CPG + RPI * q;
        *reinterpret_cast<u32x4_t*>(base + lds_chunk(r, sc)) = a_operand<WB, A8>(v[k]);
        if constexpr (A8) {
          if (sc == 0) aux[r] = xs[k];
          if constexpr (RS8) {
            // exact row sum of the group's 128 INT8 activations: 16 per lane, 8 lanes per row
            int t = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) t = __builtin_amdgcn_sdot4((int)v[k][w], 0x01010101, t, false);
#pragma unroll
            for (int d = 1; d < CPG; d <<= 1) t += __shfl_xor(t, d);
            if (sc == 0) reinterpret_cast<int*>(aux + BM)[r] = t;
          }
        } else {
          // row sum of the group's 128 BF16 values: 8 per lane, 16 lanes per row
          float t = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) t = add_bf16x2(v[k][w], t);
          t = row16_sum(t);                          // the 16 lanes of the row-group are one DPP row
          if (sc == 0) aux[r] = -kOff * t;           // the C operand of the group's first MFMA
        }
      }
    };

    struct WB_ {
      u32x4_t b[TN][NB];
      uint32_t s[TN];
    };
    auto load_w = [&](WB_& w, int g) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < NB; ++q)
          w.b[j][q] = bload16(wsrc(j), (wcol[j] * NG + g) * WGB + kb * 16 * NB + 16 * q);
        w.s[j] = bload_u16(ssrc(j), (wcol[j] * NG + g) * 2);
      }
    };

    // LDS read bases of this lane's A operand per step (row tile offsets are constants)
    uint32_t a_base[STEPS];
#pragma unroll
    for (int t = 0; t < STEPS; ++t) a_base[t] = lds_chunk(wm * 64 + li, (A8 ? kb * 2 : kb * 4) + t);

    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // prologue: group 0 staged, its weights in flight.  BF16 activations
    // with INT4 weights (registers to spare): the next group's weights are requested at the
    // start of each group, a whole group ahead; INT8 activations: after the
    // group's last MFMA.  The next group's activation rows are requested at
    // the start of each group too (BF16: both halves, 16 registers).
    constexpr bool kWAhead = !A8 && WB == 4;
    constexpr bool kAEarly = NH == 2;
    WB_ wcur, wnxt;
    load_w(wcur, 0);
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      u32x4_t v[QH];
      float xs[QH];
      load_a(v, xs, 0, h);
      store_a(v, xs, 0, h);
    }
    // BF16 activations with the weight look-ahead: the next group's loads go
    // out before the barrier that opens a group (not after it)
    constexpr bool kEarlyIssue = kAEarly && kWAhead;
    u32x4_t vn[QH], vn2[QH];
    float xsn[QH], xsn2[QH];
    if (kEarlyIssue && NG > 1) {
      load_a(vn, xsn, 1, 0);
      load_a(vn2, xsn2, 1, 1);
      load_w(wnxt, 1);
    }
    __syncthreads();

    for (int g = 0; g < NG; ++g) {
      const int b = g & 1;
      const bool more = g + 1 < NG;
      // the next group's activations are in flight during this whole group
      // (BF16: both halves requested here and staged after the last MFMA)
      if (!kEarlyIssue && more) load_a(vn, xsn, g + 1, 0);
      if (!kEarlyIssue && kAEarly && more) load_a(vn2, xsn2, g + 1, 1);
      if (!kEarlyIssue && kWAhead && more) load_w(wnxt, g + 1);
      const uint8_t* base = lds + b * STAGE;
      const float* aux = reinterpret_cast<const float*>(base + A_STAGE);
      float ws[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) ws[j] = half_bits_to_f32(wcur.s[j]);
      if constexpr (!A8) {
        // the group's sums start from -offset * (row sum) (staged that way),
        // so they leave the MFMAs without the 136 + q / 128 + q offset
        f32x4_t cinit[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (i >= live) continue;
          cinit[i] = *reinterpret_cast<const f32x4_t*>(aux + wm * 64 + i * 16 + 4 * kb);
        }
        f32x4_t part[TM][TN];
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
          u32x4_t bv[TN];
#pragma unroll
          for (int j = 0; j < TN; ++j) bv[j] = b_operand_bf16<WB>(wcur.b[j], t);
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            if (i >= live) continue;
            const bf16x8_t av =
                __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(base + a_base[t] + i * 16 * GB));
#pragma unroll
            for (int j = 0; j < TN; ++j)
              part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bv[j]),
                                                                   t == 0 ? cinit[i] : part[i][j], 0, 0, 0);
          }
          if (NH == 2 && !kAEarly && t == STEPS / 2 - 1 && more) {   // first half staged, second half in flight
            store_a(vn, xsn, b ^ 1, 0);
            load_a(vn, xsn, g + 1, NH - 1);
          }
        }
        // without look-ahead the weight registers are refilled once the last
        // MFMA has read them
        if (!kWAhead && more) load_w(wcur, g + 1);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (i >= live) continue;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(ws[j], part[i][j][v], acc[i][j][v]);
        }
      } else {
        i32x4_t part[TM][TN];
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
          u32x4_t bv[TN];
#pragma unroll
          for (int j = 0; j < TN; ++j) bv[j] = b_operand_i8<WB>(wcur.b[j], t);
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const i32x4_t av =
                __builtin_bit_cast(i32x4_t, *reinterpret_cast<const u32x4_t*>(base + a_base[t] + i * 16 * GB));
#pragma unroll
            for (int j = 0; j < TN; ++j)
              part[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                  av, __builtin_bit_cast(i32x4_t, bv[j]), t == 0 ? i32x4_t{0, 0, 0, 0} : part[i][j], 0, 0, 0);
          }
        }
        if (more) load_w(wcur, g + 1);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(aux + wm * 64 + i * 16 + 4 * kb);
          // INT4 codes entered as q + 8: remove 8 * (row sum of the INT8 activations)
          i32x4_t rs8 = {0, 0, 0, 0};
          if constexpr (RS8) rs8 = *reinterpret_cast<const i32x4_t*>(aux + BM + wm * 64 + i * 16 + 4 * kb);
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int isum = RS8 ? part[i][j][v] - 8 * rs8[v] : part[i][j][v];
              acc[i][j][v] = __builtin_fmaf((float)isum, xs[v] * ws[j], acc[i][j][v]);
            }
        }
      }
      if (kAEarly && more) {
        store_a(vn, xsn, b ^ 1, 0);
        store_a(vn2, xsn2, b ^ 1, 1);
      } else if (more) {
        store_a(vn, xsn, b ^ 1, NH - 1);
      }
      if (kWAhead && more) wcur = wnxt;
      if (kEarlyIssue && g + 2 < NG) {
        load_a(vn, xsn, g + 2, 0);
        load_a(vn2, xsn2, g + 2, 1);
        load_w(wnxt, g + 2);
      }
      __syncthreads();
    }

    // epilogue: lane holds rows 16i + 4kb + v of column 16j + li of its wave tile
    uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wm * 64 + i * 16 + 4 * kb + v;
        if (r < nrows && wcols) {
          uint16_t* orow = out + (int64_t)(row0 + r) * p.n;
          if constexpr (DUAL) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
              orow[n0 + wn * 32 + j * 16 + li] = (uint16_t)f32_to_bf16_bits(silu(acc[i][j][v]) * acc[i][j + 2][v]);
          } else {
#pragma unroll
            for (int j = 0; j < TN; ++j) orow[n0 + wn * 64 + j * 16 + li] = (uint16_t)f32_to_bf16_bits(acc[i][j][v]);
          }
        }
      }
  }
};

// INT8 weights with INT8 activations.  Both operands reach LDS through direct
// buffer->LDS loads (no staging registers), in stages of half a 128-group
// (64 reduction bytes of 128 rows and of 128 weight rows), four stages, loads
// issued three half-groups ahead.  A direct load writes lane L's 16 bytes at
// base + 16 L, so each lane fetches the chunk that belongs at its position:
// row r keeps its four chunks at positions c ^ ((r >> 1) & 3).  Rows are 64
// bytes apart, so any 8 consecutive rows then put a given chunk in 8 distinct
// 16-byte slots of a 128-byte window and the operand reads (16 rows x one
// chunk per 16 lanes) are free of bank conflicts.  Every stage issues the same
// four direct loads per thread and nothing else, so one static vmcnt fits all
// and no register waits on a load in flight.
//
// The weights are the MFMA's A operand and the activations its B operand, so
// the accumulator holds the tile transposed: a lane owns one activation row
// and four consecutive output columns, which leave as one 8-byte store after
// one packed BF16 conversion per pair.  The combination of a group's INT32
// sums needs the activation scale of the lane's row (one FP32) and the weight
// scales of its four columns (one 16-byte LDS read).  Both sets of scales of
// every group are placed in LDS once per workgroup: the activation scales by
// direct loads as [group][row] FP32; the weight scales, stored [row][group]
// FP16, are first copied into the LDS of the fourth stage (not loaded before
// the first round) and converted there into [group][row] FP32.
// WN: waves along the weight rows (two along the activation rows), so the
// workgroup has 2 WN waves and 64 WN weight rows.  WN = 2: 128 weight rows,
// two workgroups per CU; WN = 4: 256 weight rows, one workgroup per CU, which
// loads 24 KB per stage where two narrow workgroups load 32 KB for the same
// MFMA work.  CBW: consecutive column blocks of one row tile per workgroup,
// walked with one stage ring (the activation rows, their scales and the
// expert stay; the weight loads move by one column block), so the ring fills
// once per CBW blocks; each block ends with its own epilogue.
template <bool DUAL, int WN, int CBW = 1>
struct BigW8A8 {
  static constexpr int NWAVE = 2 * WN, NT = 64 * NWAVE;
  static constexpr int BM = 128, BNW = 64 * WN;
  static constexpr int HW = BNW / 2;               // DUAL: gate rows, then as many up rows
  static constexpr int BNO = DUAL ? HW : BNW;      // output columns per workgroup
  static constexpr int TM = 4, TN = 4;             // 16x16 tiles per wave (64 rows x 64 weight rows)
  static constexpr int HB = kGroup / 2;            // reduction bytes per stage (half a group)
  static constexpr int QA = BM * HB / 16 / NT;     // direct A loads per thread per stage
  static constexpr int QB = BNW * HB / 16 / NT;    // direct B loads per thread per stage (2)
  static_assert(QA >= 1 && QB == 2 && QA * NT * 16 == BM * HB, "stage split");
  static constexpr int B_OFF = BM * HB;
  static constexpr int STAGE = B_OFF + BNW * HB;
  static constexpr int NS = 4;                     // stages; loads run NS - 1 stages ahead
  static constexpr int VM = QA + QB;               // direct loads per thread per stage
  static constexpr int NHALF = DUAL ? 2 : 1;       // weight-scale sources (gate, up) or one
  static constexpr int kMaxGroups = 64;            // every group's scales sit in LDS
  // FP16 weight-scale copy in the fourth stage: NHALF parts of BNW / NHALF
  // rows, each padded to whole KB (the direct loads move 1 KB per wave)
  __host__ __device__ static int ws16_part(int ng) { return (BNW / NHALF) * ng * 2; }
  __host__ __device__ static int ws16_pad(int ng) { return (ws16_part(ng) + 1023) / 1024 * 1024; }
  // the stages, then the scales of every group: activations [group][row] and
  // weights [column block][group][weight row], both FP32; then the row maxima
  // of the h quantizer
  static constexpr int RED_BYTES = BM * WN * 4;
  __host__ __device__ static size_t lds_bytes(int ng) {
    return NS * (size_t)STAGE + (size_t)ng * (BM + CBW * BNW) * 4 + RED_BYTES;
  }

  __device__ static uint32_t chunk_pos(int row, int chunk) {
    return (uint32_t)(row * HB + ((chunk ^ ((row >> 1) & 3)) << 4));
  }
  // the FP16 weight-scale copy of ng groups fits the fourth stage and every
  // group's FP32 scales fit beside the stages
  __host__ __device__ static bool fits(int ng) {
    return ng <= kMaxGroups && CBW * NHALF * ws16_pad(ng) <= STAGE && lds_bytes(ng) <= 160 * 1024;
  }
  // first tile row of the wave's weight tile j (DUAL: j < 2 gate rows, j >= 2
  // the same columns' up rows, HW further on)
  __device__ static int wrow0(int wn, int j) { return DUAL ? (j >> 1) * HW + wn * 32 + (j & 1) * 16 : wn * 64 + j * 16; }

  template <class RowSrc>
  __device__ static void run(const GemmProblem& p, int cb, int e, int row0, int nrows, RowSrc src, uint8_t* lds) {
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, kb = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int NG = p.kdim / kGroup;
    const int NH = 2 * NG;                          // stages of one column block
    const int NHP = (NH + 3) & ~3;                  // ... in whole rounds of four
    const int n0 = cb * CBW * BNO;                  // first column block of the workgroup
    const int64_t mat_bytes = (int64_t)p.n * NG * kGroup;
    const rsrc_t rw0 = make_rsrc(p.w0q + e * mat_bytes, mat_bytes);
    const rsrc_t rw1 = DUAL ? make_rsrc(p.w1q + e * mat_bytes, mat_bytes) : rw0;
    const rsrc_t rs0 = make_rsrc(p.w0s + e * (int64_t)p.n * NG, (int64_t)p.n * NG * 2);
    const rsrc_t rs1 = DUAL ? make_rsrc(p.w1s + e * (int64_t)p.n * NG, (int64_t)p.n * NG * 2) : rs0;
    const rsrc_t ra = make_rsrc(p.a, p.a_rows * (int64_t)NG * kGroup);
    const rsrc_t rx = make_rsrc(p.a_scale, p.a_rows * (int64_t)NG * 4);

    // per-lane source offsets of the direct loads (the row's start plus the
    // chunk pair): stage h = 2g + t then reads the chunks 2c + t of group g,
    // at the scalar offset g * 128 + t * 16, which stays inside the row.
    // Rows past the tile's end carry an out-of-range offset (zeros).
    uint32_t a_off[QA], b_off[QB];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int P = (q * NWAVE + wave) * 64 + lane, row = P >> 2, c = (P & 3) ^ ((row >> 1) & 3);
      a_off[q] = row < nrows ? (uint32_t)(src(row) * NG * kGroup) + (uint32_t)(c * 32) : kOOB;
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int P = (q * NWAVE + wave) * 64 + lane, n = P >> 2, c = (P & 3) ^ ((n >> 1) & 3);
      const int wrow = DUAL ? n0 + (n & (HW - 1)) : n0 + n;   // DUAL: n < HW gate (q = 0), else up (q = 1)
      b_off[q] = (uint32_t)(wrow * NG * kGroup) + (uint32_t)(c * 32);
    }
    auto lds3 = [&](int off) { return (__attribute__((address_space(3))) void*)(lds + off); };

    const int XS_OFF = NS * STAGE, WS_OFF = XS_OFF + NG * BM * 4, WS16_OFF = (NS - 1) * STAGE;
    const int RED_OFF = WS_OFF + NG * CBW * BNW * 4;
    const int wpart = ws16_part(NG), wpad = ws16_pad(NG), nkb = wpad / 1024;
    // the tile's scales of every group, before the first stage's loads.
    // Activation scales: load q (of 2 NG, four bytes a lane) is group q / 2,
    // rows 64 (q % 2) + lane.  Weight scales: load q of a part copies its
    // bytes [1 KB q, 1 KB q + 1 KB), lanes past the part reading zeros into
    // the padding.  The waves share the loads; a wave's count varies, which
    // the static waits below tolerate (they only bound the newer loads).
    for (int q = wave; q < 2 * NG; q += NWAVE) {   // uniform
      const int r = (q & 1) * 64 + lane;
      const uint32_t off = r < nrows ? (uint32_t)((src(r) * NG + (q >> 1)) * 4) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, lds3(XS_OFF + ((q >> 1) * BM + (q & 1) * 64) * 4), 4, off, 0, 0, 0);
    }
    for (int q = wave; q < CBW * NHALF * nkb; q += NWAVE) {   // uniform
      const int cp = q / nkb, c = cp / NHALF, part = cp - c * NHALF, b = (q - cp * nkb) * 1024 + 16 * lane;
      const uint32_t off = b < wpart ? (uint32_t)((n0 + c * BNO) * NG * 2 + b) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(DUAL && part == 1 ? rs1 : rs0, lds3(WS16_OFF + cp * wpad + (q - cp * nkb) * 1024),
                                               16, off, 0, 0, 0);
    }
    // stage loads of ring stage hg (column block hg / NHP, half-group
    // hg % NHP) into stage st; past the reduction's end (the last round of a
    // block, or past the last block) the same loads with an out-of-range
    // offset, so that every stage keeps the same count.  The weights of
    // column block c sit c * BNO rows further on: a scalar offset, every
    // block's rows lying inside the matrix.
    auto issue = [&](int hg, auto stc) {
      constexpr int st = decltype(stc)::value;
      const int base = st * STAGE;
      const int c = CBW == 1 ? 0 : hg / NHP, h = hg - c * NHP;
      if (c < CBW && h < NH) {                       // uniform
        const uint32_t koff = (uint32_t)((h >> 1) * kGroup + (h & 1) * 16);
        const uint32_t kwoff = koff + (uint32_t)(c * BNO * NG * kGroup);
#pragma unroll
        for (int q = 0; q < QA; ++q)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds3(base + (q * NWAVE + wave) * 1024), 16, a_off[q], koff, 0, 0);
#pragma unroll
        for (int q = 0; q < QB; ++q)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(DUAL && q == 1 ? rw1 : rw0, lds3(base + B_OFF + (q * NWAVE + wave) * 1024),
                                                   16, b_off[q], kwoff, 0, 0);
      } else {
#pragma unroll
        for (int q = 0; q < QA; ++q)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds3(base + (q * NWAVE + wave) * 1024), 16, kOOB, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < QB; ++q)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(DUAL && q == 1 ? rw1 : rw0, lds3(base + B_OFF + (q * NWAVE + wave) * 1024),
                                                   16, kOOB, 0, 0, 0);
      }
    };
    issue(0, std::integral_constant<int, 0>{});
    issue(1, std::integral_constant<int, 1>{});
    issue(2, std::integral_constant<int, 2>{});

    // weight scales to FP32 [group][tile row] (the first round's barrier
    // publishes them and precedes the first load into the fourth stage)
    __builtin_amdgcn_s_waitcnt(vmcnt_enc((NS - 1) * VM));   // this thread's scale loads landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();                            // and every thread's
    asm volatile("" ::: "memory");
    for (int idx = tid; idx < CBW * BNW * NG; idx += NT) {
      const int c = idx / (BNW * NG), rem = idx - c * (BNW * NG);
      const int g = rem / BNW, n = rem - g * BNW;
      const int part = DUAL ? n / HW : 0, nr = DUAL ? n % HW : n;
      const uint16_t w =
          *reinterpret_cast<const uint16_t*>(lds + WS16_OFF + (c * NHALF + part) * wpad + (nr * NG + g) * 2);
      *reinterpret_cast<float*>(lds + WS_OFF + idx * 4) = half_bits_to_f32(w);
    }

    // LDS read bases (row tile and column tile offsets are compile-time constants)
    const uint32_t a_rd = chunk_pos(wm * 64 + li, kb);
    const uint32_t b_rd = chunk_pos((DUAL ? wn * 32 : wn * 64) + li, kb);

    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    i32x4_t part[TM][TN];
    float xsv[TM];
    f32x4_t wsv[TN];
    // a group's FP32 combination: acc += float(isum) * (xs * ws)
    auto combine = [&](int i, int j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf((float)part[i][j][v], xsv[i] * wsv[j][v], acc[i][j][v]);
    };

    // one stage: wait for it, refill the stage read last time, compute
    auto body = [&](int hg, auto stc) {
      constexpr int st = decltype(stc)::value;
      const int c = CBW == 1 ? 0 : hg / NHP, h = hg - c * NHP;
      constexpr int t = st & 1;                      // stage index and half agree (NS even)
      __builtin_amdgcn_s_waitcnt(vmcnt_enc((NS - 2) * VM));   // this thread's loads of stage h landed
      __builtin_amdgcn_s_waitcnt(kLgkmcnt0);                   // and its LDS reads of stage h - 1 completed
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();                  // every thread's; stage h - 1 may be refilled
      asm volatile("" ::: "memory");
      issue(hg + NS - 1, std::integral_constant<int, (st + NS - 1) % NS>{});
      const uint8_t* base = lds + st * STAGE;
      u32x4_t bv[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int nj = DUAL ? ((j >> 1) * HW + (j & 1) * 16) : j * 16;   // DUAL: up rows start at HW
        bv[j] = *reinterpret_cast<const u32x4_t*>(base + B_OFF + b_rd + nj * HB);
      }
      if constexpr (t == 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const i32x4_t av = __builtin_bit_cast(i32x4_t, *reinterpret_cast<const u32x4_t*>(base + a_rd + i * 16 * HB));
#pragma unroll
          for (int j = 0; j < TN; ++j)
            part[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, bv[j]), av,
                                                               i32x4_t{0, 0, 0, 0}, 0, 0, 0);
        }
        // this group's scales, for its combination after the second half (a
        // group past the reduction, the last round's: zero operands, zero
        // scales)
        const bool gin = (h >> 1) < NG;
        const int g = gin ? h >> 1 : NG - 1;
        const float* xsl = reinterpret_cast<const float*>(lds + XS_OFF) + g * BM + wm * 64 + li;
        const float* wsl = reinterpret_cast<const float*>(lds + WS_OFF) + (c * NG + g) * BNW + 4 * kb;
#pragma unroll
        for (int i = 0; i < TM; ++i) xsv[i] = gin ? xsl[i * 16] : 0.f;
#pragma unroll
        for (int j = 0; j < TN; ++j) wsv[j] = *reinterpret_cast<const f32x4_t*>(wsl + wrow0(wn, j));
      } else {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const i32x4_t av = __builtin_bit_cast(i32x4_t, *reinterpret_cast<const u32x4_t*>(base + a_rd + i * 16 * HB));
#pragma unroll
          for (int j = 0; j < TN; ++j)
            part[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, bv[j]), av, part[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) combine(i, j);
      }
    };

    // whole rounds of four stages: with an odd group count the last group is
    // a no-op one (zero operands, zero scales), which keeps every round the
    // same straight-line code and every wait count static.  A column block's
    // epilogue runs between its last round and the next block's first, with
    // the next block's first stages already in flight.
    uint16_t* out = static_cast<uint16_t*>(p.out);
    for (int c = 0; c < CBW; ++c) {
      for (int h = 0; h < NHP; h += 4) {
        const int hg = c * NHP + h;
        body(hg, std::integral_constant<int, 0>{});
        body(hg + 1, std::integral_constant<int, 1>{});
        body(hg + 2, std::integral_constant<int, 2>{});
        body(hg + 3, std::integral_constant<int, 3>{});
      }
      // lane: activation row wm*64 + 16 i + li, output columns 4 kb .. 4 kb + 3
      // of each 16-column tile
      const int cbc = cb * CBW + c, n0c = cbc * BNO;
      bool h_out = true;
      if constexpr (DUAL && BNO == kGroup) {
        if (p.hq) {
          quantize_h_epilogue(p, cbc, row0, nrows, acc, reinterpret_cast<float*>(lds + RED_OFF));
          h_out = out != nullptr;
        }
      }
      if (h_out) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int m = wm * 64 + i * 16 + li;
          if (m < nrows) {
            uint16_t* orow = out + (int64_t)(row0 + m) * p.n + n0c + 4 * kb;
            if constexpr (DUAL) {
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                float hv[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) hv[v] = silu(acc[i][j][v]) * acc[i][j + 2][v];
                *reinterpret_cast<uint2*>(orow + wn * 32 + j * 16) =
                    uint2{pack2_bf16(hv[0], hv[1]), pack2_bf16(hv[2], hv[3])};
              }
            } else {
#pragma unroll
              for (int j = 0; j < TN; ++j)
                *reinterpret_cast<uint2*>(orow + wn * 64 + j * 16) =
                    uint2{pack2_bf16(acc[i][j][0], acc[i][j][1]), pack2_bf16(acc[i][j][2], acc[i][j][3])};
            }
          }
        }
      }
      if (c + 1 < CBW) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));        // no load into LDS outlives the workgroup
  }

  // h quantized per 128 values, as the INT8 quantizer does it for the BF16 h
  // (the workgroup's 128 outputs are one group of each of its rows): the
  // group maximum of |h| over the lane's eight values, the four 16-lane
  // segments (xor 16, 32) and the four waves along the columns (LDS), then
  // s = max / 127 and the codes of the BF16 values.  hq int8 [rows][n],
  // hs fp32 [rows][n / 128].  red: LDS of BM * WN floats apart from the
  // stages (the ring may be filling them).
  __device__ static void quantize_h_epilogue(const GemmProblem& p, int cb, int row0, int nrows,
                                             const f32x4_t (&acc)[TM][TN], float* red) {
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, kb = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    float hb[TM][2][4];
    float mx[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t lo = pack2_bf16(silu(acc[i][j][0]) * acc[i][j + 2][0], silu(acc[i][j][1]) * acc[i][j + 2][1]);
        const uint32_t hi = pack2_bf16(silu(acc[i][j][2]) * acc[i][j + 2][2], silu(acc[i][j][3]) * acc[i][j + 2][3]);
        hb[i][j][0] = bf16_bits_to_f32(lo & 0xffffu);
        hb[i][j][1] = bf16_bits_to_f32(lo >> 16);
        hb[i][j][2] = bf16_bits_to_f32(hi & 0xffffu);
        hb[i][j][3] = bf16_bits_to_f32(hi >> 16);
#pragma unroll
        for (int v = 0; v < 4; ++v) m = fmaxf(m, fabsf(hb[i][j][v]));
      }
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      mx[i] = m;
    }
    __syncthreads();                                       // every wave's reads of red (previous block) are done
    if (kb == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i) red[(wm * 64 + i * 16 + li) * WN + wn] = mx[i];
    }
    __syncthreads();
    const int ng = p.n / kGroup;
    int8_t* hq = p.hq;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = wm * 64 + i * 16 + li;
      float M = red[m * WN];
#pragma unroll
      for (int w = 1; w < WN; ++w) M = fmaxf(M, red[m * WN + w]);
      const float sc = M / 127.0f;
      const bool zero = !(sc != 0.0f);
      const float r = 1.0f / (zero ? 1.0f : sc);
      if (m < nrows) {
        const int64_t row = row0 + m;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t packed = 0u;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int qv = zero ? 0 : (int)act_code(hb[i][j][v], sc, r);
            packed |= (uint32_t)(qv & 0xff) << (8 * v);
          }
          *reinterpret_cast<uint32_t*>(hq + row * p.n + cb * BNO + wn * 32 + j * 16 + 4 * kb) = packed;
        }
        if (wn == 0 && kb == 0) p.hs[row * ng + cb] = sc;
      }
    }
  }
};

template <bool DUAL, int WN, int CBW>
__global__ __launch_bounds__(128 * WN, (WN == 2) ? 2 : 1) void k_gemm_w8a8(GemmProblem p) {
  using K = BigW8A8<DUAL, WN, CBW>;
  extern __shared__ __attribute__((aligned(16))) uint8_t big_lds[];
  int tile, cb;
  if (!xcd_tile(p, tile, cb)) return;
  const Tile td = p.tiles[tile];
  const int row0 = td.row0;
  if (p.gather_k)
    K::run(p, cb, td.e, row0, td.nrows, [&](int r) { return (int64_t)(p.sorted_slot[row0 + r] / p.gather_k); },
           big_lds);
  else
    K::run(p, cb, td.e, row0, td.nrows, [&](int r) { return (int64_t)(row0 + r); }, big_lds);
}

template <int WB, bool A8, bool DUAL, int WM>
__global__ __launch_bounds__(256, 2) void k_gemm_big(GemmProblem p) {
  using K = Big<WB, A8, DUAL, WM>;
  extern __shared__ __attribute__((aligned(16))) uint8_t big_lds[];
  int tile, cb;
  if (!xcd_tile(p, tile, cb)) return;
  const Tile td = p.tiles[tile];
  const int row0 = td.row0;
  if (p.gather_k)
    K::run(p, cb, td.e, row0, td.nrows, [&](int r) { return (int64_t)(p.sorted_slot[row0 + r] / p.gather_k); },
           big_lds);
  else
    K::run(p, cb, td.e, row0, td.nrows, [&](int r) { return (int64_t)(row0 + r); }, big_lds);
}

template <bool DUAL, int WN, int CBW>
hipError_t launch_w8a8_wn(const GemmProblem& p, hipStream_t stream) {
  using K = BigW8A8<DUAL, WN, CBW>;
  const dim3 grid(p.n / (K::BNO * CBW), (unsigned)((p.max_tiles + 7) / 8 * 8));
  QRE_LAUNCH_GEMM((k_gemm_w8a8<DUAL, WN, CBW>), grid, dim3(K::NT), K::lds_bytes(p.kdim / kGroup), stream, p);
  return hipGetLastError();
}

// Column blocks per workgroup: as many as the width (whole groups of them)
// and the LDS allow, up to C.
template <bool DUAL, int WN, int C>
hipError_t launch_w8a8_cbw(const GemmProblem& p, hipStream_t stream) {
  using K = BigW8A8<DUAL, WN, C>;
  if constexpr (C > 1) {
    if (p.n % (K::BNO * C) != 0 || !K::fits(p.kdim / kGroup)) return launch_w8a8_cbw<DUAL, WN, C / 2>(p, stream);
  }
  return launch_w8a8_wn<DUAL, WN, C>(p, stream);
}

// Column blocks per workgroup: four for the down GEMM (its reduction is short,
// so the ring's fill is a large part of one block), two for gate/up.
constexpr int kGateUpCbw = 2, kDownCbw = 4;

// Gate/up: the wide workgroup (128 outputs, one quantization group of h)
// when the output width and the reduction allow it; it alone can quantize h
// in its epilogue.  Down: the narrow one (two workgroups per CU keep more
// loads in flight, which the down GEMM needs).
template <bool DUAL>
hipError_t launch_w8a8_cfg(const GemmProblem& p, hipStream_t stream) {
  using Nw = BigW8A8<DUAL, 2>;
  const int ng = p.kdim / kGroup;
  if constexpr (DUAL) {
    using Wd = BigW8A8<true, 4>;
    if (p.n % Wd::BNO == 0 && Wd::fits(ng)) return launch_w8a8_cbw<true, 4, kGateUpCbw>(p, stream);
  }
  if (p.hq || p.n % Nw::BNO != 0 || !Nw::fits(ng)) return hipErrorInvalidValue;
  return launch_w8a8_cbw<DUAL, 2, DUAL ? 1 : kDownCbw>(p, stream);
}

template <int WB, bool A8, bool DUAL, int WM>
hipError_t launch_big_cfg(const GemmProblem& p, hipStream_t stream) {
  using K = Big<WB, A8, DUAL, WM>;
  if (p.n % (DUAL ? 32 : 64) != 0 || p.bm != K::BM) return hipErrorInvalidValue;
  const dim3 grid((p.n + K::BNO - 1) / K::BNO, (unsigned)((p.max_tiles + 7) / 8 * 8));
  QRE_LAUNCH_GEMM((k_gemm_big<WB, A8, DUAL, WM>), grid, dim3(256), K::lds_bytes(), stream, p);
  return hipGetLastError();
}

}  // namespace

bool gate_up_quantizes_h(const GemmProblem& p) {
  using Wd = BigW8A8<true, 4>;
  return p.bm == 128 && p.act_int8 && p.bits == 8 && p.w1q != nullptr && p.n % Wd::BNO == 0 &&
         Wd::fits(p.kdim / kGroup);
}

bool big_applicable(int64_t S, int E, int kdim) {
  // many rows per expert: at least 64 on average; a reduction of at most 64
  // groups (the INT8-activation kernel keeps every group's scales in LDS)
  return S >= 64 * (int64_t)E && kdim <= BigW8A8<true, 2>::kMaxGroups * kGroup;
}

int big_tile_rows(int act_int8) { return act_int8 ? 128 : 64; }

hipError_t launch_gemm_big(const GemmProblem& p, hipStream_t stream) {
  const bool dual = p.w1q != nullptr;
  if (p.bm != big_tile_rows(p.act_int8)) return hipErrorInvalidValue;
  if (p.bits == 4) {
    if (p.act_int8)
      return dual ? launch_big_cfg<4, true, true, 2>(p, stream) : launch_big_cfg<4, true, false, 2>(p, stream);
    return dual ? launch_big_cfg<4, false, true, 1>(p, stream) : launch_big_cfg<4, false, false, 1>(p, stream);
  }
  if (p.act_int8) return dual ? launch_w8a8_cfg<true>(p, stream) : launch_w8a8_cfg<false>(p, stream);
  return dual ? launch_big_cfg<8, false, true, 1>(p, stream) : launch_big_cfg<8, false, false, 1>(p, stream);
}

}  // namespace qre
