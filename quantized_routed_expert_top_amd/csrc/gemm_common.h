// Device helpers shared by the grouped-GEMM kernel files (gfx950): raw buffer
// loads, the in-register INT4/INT8 -> MFMA operand conversions, and the
// per-expert routing pass of the decode gate/up kernels.
//
// Operand conversions (the kernels' own design):
//  * INT4 codes become BF16 without arithmetic: XOR with 8 turns the nibble
//    into u = q + 8 in 0..15 and OR-ing it into the mantissa of BF16 128.0
//    gives exactly 136 + q; INT8 codes become 128 + q via the unsigned-byte
//    conversion.  The offset is removed per group with the row sums of A,
//    which one extra MFMA against a ones operand produces in the accumulator
//    layout;
//  * nibble extraction pairs codes k and k+4 of each 32-bit word, so A is
//    permuted the same way with v_perm_b32 (a dot product is invariant under
//    a common permutation of the reduction index);
//  * all loads are raw buffer loads: a masked row or a group past the end of
//    the reduction uses an out-of-range offset, which returns zeros without
//    touching memory, so no load sits behind a branch.
#pragma once

#include <hip/hip_fp16.h>

#include "qre_internal.h"

namespace qre {
namespace gk {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr uint32_t kOOB = 0x80000000u;   // offset past every descriptor (all are < 2^31 bytes)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t bload_u16(rsrc_t r, uint32_t off) {
  return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ float bload_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// g * sigmoid(g) with the hardware reciprocal (1 ulp): g -> -inf gives
// g * rcp(inf) = -0, g -> +inf gives g * rcp(1) = g.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two FP32 values rounded to BF16 (round to nearest even, one v_cvt_pk_bf16_f32)
// and packed, lo in bits 15:0.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// v of lane + N within its row of 16 lanes (DPP row_shl; lanes whose source
// leaves the row read 0)
template <int N>
__device__ __forceinline__ float row_shl(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x100 + N, 0xf, 0xf,
                                                               true));
}

// Sum of t over the 16 lanes of each DPP row, in lane 16r: the pairwise tree
// ((t0 + t1) + (t2 + t3)) + ... that an xor butterfly over 16 lanes leaves in
// its lane 0 (the same additions in the same order).
__device__ __forceinline__ float row16_sum(float t) {
  t += row_shl<1>(t);
  t += row_shl<2>(t);
  t += row_shl<4>(t);
  t += row_shl<8>(t);
  return t;
}

// t plus the two BF16 values packed in w: one v_dot2c_f32_bf16 against (1, 1).
__device__ __forceinline__ float add_bf16x2(uint32_t w, float t) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, 0x3f803f80u), t,
                                         false);
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  return __half2float(__ushort_as_half((unsigned short)h));
}

// Two BF16 values (exact small integers held in FP32) packed into one dword.
__device__ __forceinline__ uint32_t pack_bf16_hi(float lo, float hi) {
  return byte_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// A operand of one MFMA step (16 bytes: 8 BF16 or 16 INT8 activations),
// permuted into the reduction order of the INT4 weight operand below.  INT8
// weights need no permutation.
template <int WB, bool A8>
__device__ __forceinline__ u32x4_t a_operand(u32x4_t c) {
  if constexpr (WB == 8) return c;
  u32x4_t av;
  if constexpr (!A8) {        // BF16: pair codes k and k+4 of each 32-bit word
    av.x = byte_perm(c.z, c.x, 0x05040100u);
    av.y = byte_perm(c.z, c.x, 0x07060302u);
    av.z = byte_perm(c.w, c.y, 0x05040100u);
    av.w = byte_perm(c.w, c.y, 0x07060302u);
  } else {                    // INT8: even codes then odd codes of each 32-bit word
    av.x = byte_perm(c.y, c.x, 0x06040200u);
    av.y = byte_perm(c.y, c.x, 0x07050301u);
    av.z = byte_perm(c.w, c.z, 0x06040200u);
    av.w = byte_perm(c.w, c.z, 0x07050301u);
  }
  return av;
}

// B operand for BF16 activations, MFMA step t (of 4), from the lane's slice of
// a 128-group of one weight row (16 bytes INT4 / 32 bytes INT8).  The values
// are 136 + q (INT4) or 128 + q (INT8), exact in BF16.  For INT4 each output
// word is one three-input logic op (v_bitop3) of the shifted codes: keep the
// two nibbles, flip their sign bits (q -> q + 8) and set BF16 128.0 around
// them.
template <int WB>
__device__ __forceinline__ u32x4_t b_operand_bf16(const u32x4_t* b, int t) {
  u32x4_t bv;
  if constexpr (WB == 4) {
    constexpr uint32_t kKeep = 0x000f000fu, kSet = 0x43084308u;   // 128.0 pair | nibble sign bits
    auto cvt = [](uint32_t v) { return ((v ^ kSet) & kKeep) | (kSet & ~kKeep); };
    const uint32_t w = b[0][t];
    bv.x = cvt(w);                                        // bf16 (136+q_k, 136+q_{k+4})
    bv.y = cvt(w >> 4);
    bv.z = cvt(w >> 8);
    bv.w = cvt(w >> 12);
  } else {
    const uint32_t w0 = b[t >> 1][(t & 1) * 2] ^ 0x80808080u;       // byte -> q + 128
    const uint32_t w1 = b[t >> 1][(t & 1) * 2 + 1] ^ 0x80808080u;
    bv.x = pack_bf16_hi((float)(w0 & 0xffu), (float)((w0 >> 8) & 0xffu));
    bv.y = pack_bf16_hi((float)((w0 >> 16) & 0xffu), (float)(w0 >> 24));
    bv.z = pack_bf16_hi((float)(w1 & 0xffu), (float)((w1 >> 8) & 0xffu));
    bv.w = pack_bf16_hi((float)((w1 >> 16) & 0xffu), (float)(w1 >> 24));
  }
  return bv;
}

// B operand for INT8 activations, MFMA step t (of 2): INT8 codes as they are,
// INT4 codes as q + 8 (even codes then odd codes of each word).
template <int WB>
__device__ __forceinline__ u32x4_t b_operand_i8(const u32x4_t* b, int t) {
  if constexpr (WB == 8) return b[t];
  const uint32_t w0 = b[0][2 * t] ^ 0x88888888u;
  const uint32_t w1 = b[0][2 * t + 1] ^ 0x88888888u;
  return u32x4_t{w0 & 0x0f0f0f0fu, (w0 >> 4) & 0x0f0f0f0fu, w1 & 0x0f0f0f0fu, (w1 >> 4) & 0x0f0f0f0fu};
}

// Workgroup -> (row tile, column block).  Workgroups are dispatched to the
// eight XCDs round-robin (linear id mod 8), and each XCD has its own L2.  The
// tile list is cut into eight contiguous ranges, one per XCD, walked tile by
// tile with all column blocks of a tile adjacent: the column blocks of a tile
// share its activation rows, and the consecutive tiles of an expert share its
// weights, in one L2.  Returns false for workgroups past the device-side tile
// count.  The grid's second dimension must be a multiple of 8 and at least
// the tile count.
__device__ __forceinline__ bool xcd_tile(const GemmProblem& p, int& tile, int& cb) {
  const int ncb = gridDim.x;
  const int lin = blockIdx.y * ncb + blockIdx.x;
  const int xcd = lin & 7, k = lin >> 3;
  const int nt = *p.ntiles;
  const int per = (nt + 7) >> 3;
  const int local = k / ncb;
  cb = k - local * ncb;
  tile = xcd * per + local;
  return local < per && tile < nt;
}

// One expert's share of the stable counting sort of the routed slots, computed
// by a workgroup of 256 threads from the ids alone (at most kRoutedMaxSlots
// slots).  Each wave takes a contiguous quarter of the slots and ballots, per
// 64 slots, id == e and 0 <= id < e: e's rows are its slots in ascending
// order, and its first sorted row is the number of valid slots with a smaller
// id.  Returns e's count and offset (uniform), fills rows[0..count) (LDS) with
// e's slots in order, and, if `writer`, stores e's part of counts, offsets,
// sorted_slot and slot_row (expert 0 also marks dropped slots, expert E-1
// also the end offset and the unused tail of sorted_slot).  Ends with a
// workgroup barrier.
struct ExpertRows {
  int count, off;
};
__device__ __forceinline__ ExpertRows route_expert(const RouteOut& ra, int e, bool writer, int* rows,
                                                   int (*wcnt)[4]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  constexpr int kSub = kRoutedMaxSlots / 256;              // 64-slot sub-chunks per wave
  const int nsub = (ra.S + 255) / 256;                      // 64-slot sub-chunks per wave (uniform)
  const int L = nsub * 64;                                  // slots per wave
  const int s0 = min(ra.S, wave * L), s1 = min(ra.S, s0 + L);
  // all loads first (out-of-range slots read nothing), then the ballots; the
  // ballot masks of e's slots stay in registers; the ballots of sub-chunks
  // past nsub are skipped by uniform branches
  const rsrc_t rid = make_rsrc(ra.ids, (int64_t)ra.S * 4);
  int ids[kSub];
  uint64_t eq[kSub];
#pragma unroll
  for (int c = 0; c < kSub; ++c) {
    const int s = s0 + c * 64 + lane;
    ids[c] = (int)__builtin_amdgcn_raw_buffer_load_b32(rid, s < s1 ? (uint32_t)s * 4u : kOOB, 0, 0);
    eq[c] = 0;
  }
  int n_eq = 0, n_lt = 0;
#pragma unroll
  for (int c = 0; c < kSub; ++c) {
    if (c < nsub) {
      const int s = s0 + c * 64 + lane;
      const int id = s < s1 ? ids[c] : -1;
      eq[c] = __ballot(id == e);
      n_eq += __popcll(eq[c]);
      n_lt += __popcll(__ballot(id >= 0 && id < e));
    }
  }
  if (writer && e == 0) {
#pragma unroll
    for (int c = 0; c < kSub; ++c) {
      const int s = s0 + c * 64 + lane;
      if (c < nsub && s < s1 && (ids[c] < 0 || ids[c] >= ra.E)) ra.slot_row[s] = -1;   // dropped slot
    }
  }
  if (lane == 0) {
    wcnt[0][wave] = n_eq;
    wcnt[1][wave] = n_lt;
  }
  __syncthreads();
  int count = 0, off = 0, wbase = 0;
  for (int w = 0; w < 4; ++w) {
    if (w < wave) wbase += wcnt[0][w];
    count += wcnt[0][w];
    off += wcnt[1][w];
  }
  // LDS reads land in vector registers: these values are uniform (per
  // workgroup, per wave for wbase), which keeps the callers' loops scalar
  count = __builtin_amdgcn_readfirstlane(count);
  off = __builtin_amdgcn_readfirstlane(off);
  wbase = __builtin_amdgcn_readfirstlane(wbase);
  if (writer && tid == 0) {
    ra.counts[e] = count;
    ra.offsets[e] = off;
    if (e == ra.E - 1) {
      ra.offsets[ra.E] = off + count;
      *ra.dropped = ra.S - (off + count);
    }
  }
  if (writer && e == ra.E - 1)
    for (int i = off + count + tid; i < ra.S; i += blockDim.x) ra.sorted_slot[i] = -1;
  if (count > 0) {
    int rank = wbase;
#pragma unroll
    for (int c = 0; c < kSub; ++c) {
      if (c >= nsub) break;
      if (eq[c] >> lane & 1ull) {
        const int s = s0 + c * 64 + lane;
        const int j = rank + __popcll(eq[c] & below);
        rows[j] = s;
        if (writer) {
          ra.sorted_slot[off + j] = s;
          ra.slot_row[s] = off + j;
        }
      }
      rank += __popcll(eq[c]);
    }
    __syncthreads();
  }
  return ExpertRows{count, off};
}

}  // namespace gk
}  // namespace qre
