// Router ahead of the permutation: per token, the K largest of E FP32 logits
// (descending, ties to the lower expert id) and their softmax weights.
//
// The pages put routing of decode blocks on the GPU (minnow README, section
// "Quantization") and keep routers in floating point (LLaDA2.2-flash model
// card, "Checkpoints and precision", paragraph on what quantization applies
// to).  The selection and weighting rule is the plain top-K softmax reading:
// top K by logit, weights = softmax over the K selected logits with the
// largest subtracted, in FP32.
//
// CDNA4 mapping: one wave per token.  Lane l holds logits l, l + 64, ... in
// registers (coalesced 256-byte rows); ids past E and taken experts hold a
// quiet NaN, which the maximum ignores and no comparison matches.  Each of
// the K rounds takes the wave maximum m of the remaining values with DPP
// steps (within rows of 16 lanes, then the row broadcasts; lane 63 ends with
// the maximum, read back as a uniform value), then one ballot per register
// slot for "value == m": the lowest slot with a hit and the lowest lane in
// it give the lowest id holding m (-0 and +0 compare equal).  That lane marks
// the value taken.  Lane k keeps round k's value and id; the weights are one
// expf per lane and a DPP sum (a fixed order, so reruns are bit-identical).
#include "qre_internal.h"

namespace qre {
namespace {

constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// Lanes of rows outside row_mask keep `x` (old value).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROWS, 0xF, false));
}

// Maximum over the wave (NaN lanes ignored), as a uniform value.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppXor1, 0xF>(x));
  x = fmaxf(x, dpp<kDppXor2, 0xF>(x));
  x = fmaxf(x, dpp<kDppHalfMirror, 0xF>(x));
  x = fmaxf(x, dpp<kDppMirror, 0xF>(x));
  x = fmaxf(x, dpp<kDppBcast15, 0xA>(x));
  x = fmaxf(x, dpp<kDppBcast31, 0xC>(x));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Sum over the wave in a fixed order, as a uniform value (lane 63's total;
// rows outside a broadcast's row_mask double their partial, which only lanes
// other than 63 see).
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kDppXor1, 0xF>(x);
  x += dpp<kDppXor2, 0xF>(x);
  x += dpp<kDppHalfMirror, 0xF>(x);
  x += dpp<kDppMirror, 0xF>(x);
  x += dpp<kDppBcast15, 0xA>(x);
  x += dpp<kDppBcast31, 0xC>(x);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

template <int NV>
__global__ __launch_bounds__(256) void k_topk_softmax(const float* __restrict__ logits, int T, int E, int K,
                                                       int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                                     // whole waves leave together
  const float* row = logits + (int64_t)t * E;
  const float kNaN = __int_as_float(0x7fc00000);
  float v[NV];
  uint32_t taken = 0;                                     // bit j: slot j taken or past E
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? row[e] : kNaN;
    taken |= e < E ? 0u : 1u << j;
  }
  float mv = 0.0f;                                        // lane k: round k's value and id
  int mid = 0;
  for (int k = 0; k < K; ++k) {
    float b = v[0];
#pragma unroll
    for (int j = 1; j < NV; ++j) b = fmaxf(b, v[j]);
    const float m = wave_max(b);
    int J = -1, L = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const uint64_t hit = __ballot(v[j] == m);
      if (J < 0 && hit) {
        J = j;
        L = __builtin_ctzll(hit);
      }
    }
    if (J < 0) {
      // every remaining value is NaN (unspecified input): take the lowest
      // id not yet taken, so the ids stay distinct and inside [0, E)
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const uint64_t free_ = __ballot(!((taken >> j) & 1u));
        if (J < 0 && free_) {
          J = j;
          L = __builtin_ctzll(free_);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (j == J && lane == L) {
        v[j] = kNaN;
        taken |= 1u << j;
      }
    if (lane == k) {
      mv = m;
      mid = 64 * J + L;
    }
  }
  // softmax over the selected: the first selection holds the largest logit
  const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mv), 0));
  const bool live = lane < K;
  const float z = live ? expf(mv - m0) : 0.0f;
  const float sum = wave_sum(z);
  if (live) {
    ids[(int64_t)t * K + lane] = mid;
    w[(int64_t)t * K + lane] = z / sum;
  }
}

}  // namespace

hipError_t launch_topk_softmax(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  const int nv = (E + 63) / 64;
  if (nv <= 1) hipLaunchKernelGGL(k_topk_softmax<1>, grid, block, 0, stream, logits, T, E, K, ids, w);
  else if (nv <= 2) hipLaunchKernelGGL(k_topk_softmax<2>, grid, block, 0, stream, logits, T, E, K, ids, w);
  else if (nv <= 4) hipLaunchKernelGGL(k_topk_softmax<4>, grid, block, 0, stream, logits, T, E, K, ids, w);
  else if (nv <= 8) hipLaunchKernelGGL(k_topk_softmax<8>, grid, block, 0, stream, logits, T, E, K, ids, w);
  else if (nv <= 16) hipLaunchKernelGGL(k_topk_softmax<16>, grid, block, 0, stream, logits, T, E, K, ids, w);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace qre
