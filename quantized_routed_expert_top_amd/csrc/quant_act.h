// Per-128-group INT8 quantization of BF16 activations as device code, shared
// by the quantizer kernel and by kernels that run it in some of their
// workgroups.  Definition (model card "LLaDA2.2-flash for minnow", paragraph
// on --int8-expert-activations): s = max|v| / 127 (IEEE division),
// q = clamp(rint(v / s), -127, 127) with ties to even; a zero group gives
// s = 0, q = 0.  One 16-lane segment per group, 8 values per lane, the group
// maximum by lane shuffles inside the segment.
#pragma once

#include "qre_internal.h"

namespace qre {
namespace {

// Groups gid = 16 blk0 + threadIdx.x / 16, stepping by 16 nblk (blk0 < nblk:
// this workgroup's index among the nblk of 256 threads that quantize).
__device__ inline void quantize_act_groups(const uint16_t* __restrict__ v, int64_t ngroups, int G,
                                           int8_t* __restrict__ q, float* __restrict__ s, int blk0, int nblk) {
  const int sub = threadIdx.x & 15;
  for (int64_t gid = (int64_t)blk0 * 16 + threadIdx.x / 16; gid < ngroups; gid += (int64_t)nblk * 16) {
    // whole 16-lane segments take the same trips
    const int64_t row = gid / G, g = gid % G;
    const int64_t off = row * (int64_t)G * kGroup + g * kGroup + sub * 8;
    const uint4 raw = *reinterpret_cast<const uint4*>(v + off);
    float x[8];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_bits_to_f32(w[j] & 0xffffu);
      x[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
    m = seg16_max(m);
    const float sc = m / 127.0f;
    const bool zero = !(sc != 0.0f);
    const float r = 1.0f / (zero ? 1.0f : sc);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int qv = zero ? 0 : (int)act_code(x[j], sc, r);
      packed[j / 4] |= (uint32_t)(qv & 0xff) << (8 * (j % 4));
    }
    *reinterpret_cast<uint2*>(q + off) = make_uint2(packed[0], packed[1]);
    if (sub == 0) s[gid] = sc;
  }
}

}  // namespace
}  // namespace qre
