// INT8 quantizers.
//
// Activations (model card "LLaDA2.2-flash for minnow", paragraph on
// --int8-expert-activations): expert inputs are quantized per 128 values to
// signed INT8 with an FP32 scale.  Here s = max|v| / 127 (IEEE division),
// q = clamp(rint(v / s), -127, 127) with ties to even, and a zero group gives
// s = 0, q = 0.
//
// Weights (minnow README, section "Quantization": convert --experts
// int4|int8; model card precision table: signed INT8/INT4, one FP16 scale per
// 128 weights): s = fp16(max|w| / qmax), q = clamp(rint(w / s), qmin, qmax)
// against the stored FP16 scale; INT4 codes are packed two per byte, element
// 2j in the low nibble.
//
// Layout of the work: one 16-lane segment of a wave per 128-group, 8 values
// per lane (one 16-byte load of bf16, two of fp32), the group max reduced with
// lane shuffles inside the segment.  Both are HBM-streaming passes.
#include <hip/hip_fp16.h>

#include <algorithm>

#include "quant_act.h"

namespace qre {
namespace {

// Grid-stride over (row, group) pairs, one 16-lane segment each; the grid is
// bounded, so any size the entry point accepts launches.

__global__ __launch_bounds__(256) void k_quantize_act(const uint16_t* __restrict__ v, int64_t ngroups, int G,
                                                      int8_t* __restrict__ q, float* __restrict__ s) {
  quantize_act_groups(v, ngroups, G, q, s, blockIdx.x, gridDim.x);
}

__global__ __launch_bounds__(256) void k_quantize_weights(const float* __restrict__ w, int64_t ngroups, int G,
                                                          int bits, uint8_t* __restrict__ q,
                                                          uint16_t* __restrict__ s) {
  const int sub = threadIdx.x & 15;
  for (int64_t gid = (int64_t)blockIdx.x * 16 + threadIdx.x / 16; gid < ngroups; gid += (int64_t)gridDim.x * 16) {
    const int64_t row = gid / G, g = gid % G;
    const int64_t off = row * (int64_t)G * kGroup + g * kGroup + sub * 8;
    const float4 a = *reinterpret_cast<const float4*>(w + off);
    const float4 b = *reinterpret_cast<const float4*>(w + off + 4);
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float m = 0.0f;
  #pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
    m = seg16_max(m);
    const float qmax = bits == 4 ? 7.0f : 127.0f;
    const float qmin = bits == 4 ? -8.0f : -127.0f;
    const __half s16 = __float2half_rn(m / qmax);
    const float sf = __half2float(s16);
    int codes[8];
  #pragma unroll
    for (int j = 0; j < 8; ++j) codes[j] = sf != 0.0f ? (int)fminf(qmax, fmaxf(qmin, rintf(x[j] / sf))) : 0;
    if (bits == 4) {
      uint32_t packed = 0;
  #pragma unroll
      for (int j = 0; j < 8; ++j) packed |= (uint32_t)(codes[j] & 0xf) << (4 * j);
      *reinterpret_cast<uint32_t*>(q + (off >> 1)) = packed;
    } else {
      uint32_t p0 = 0, p1 = 0;
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
        p0 |= (uint32_t)(codes[j] & 0xff) << (8 * j);
        p1 |= (uint32_t)(codes[j + 4] & 0xff) << (8 * j);
      }
      *reinterpret_cast<uint2*>(q + off) = make_uint2(p0, p1);
    }
    if (sub == 0) s[gid] = __half_as_ushort(s16);
  }
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t* v, int rows, int cols, int8_t* q, float* s, hipStream_t stream) {
  const int G = cols / kGroup;
  const int64_t ngroups = (int64_t)rows * G;
  if (ngroups == 0) return hipSuccess;
  const int64_t blocks = std::min((ngroups + 15) / 16, kMaxQuantBlocks);
  hipLaunchKernelGGL(k_quantize_act, dim3((unsigned)blocks), dim3(256), 0, stream, v, ngroups, G, q, s);
  return hipGetLastError();
}

hipError_t launch_quantize_weights(const float* w, int64_t rows, int64_t cols, int bits, uint8_t* q,
                                   uint16_t* s, hipStream_t stream) {
  const int G = (int)(cols / kGroup);
  const int64_t ngroups = rows * G;
  if (ngroups == 0) return hipSuccess;
  const int64_t blocks = std::min((ngroups + 15) / 16, kMaxQuantBlocks);
  hipLaunchKernelGGL(k_quantize_weights, dim3((unsigned)blocks), dim3(256), 0, stream, w, ngroups, G, bits, q, s);
  return hipGetLastError();
}

}  // namespace qre
