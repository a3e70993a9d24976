// Deterministic top-k weighted combine of the expert outputs.
//
// The expert outputs y return to BF16 (model card "LLaDA2.2-flash for
// minnow", paragraph on --int8-expert-activations); each token's output is
// the routing-weighted sum of its K expert outputs.  The order is fixed:
// FP32, k ascending, one fused multiply-add per term starting from 0, then one
// nearest-even rounding to BF16, so the result does not depend on scheduling.
//
// One workgroup per (token, 2048-column slab); each lane owns 8 consecutive
// columns (16-byte loads of y, one 16-byte store of out).
#include "qre_internal.h"

namespace qre {
namespace {

constexpr int kUnroll = 8;   // slots whose loads are in flight together

__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y, const int32_t* __restrict__ slot_row,
                                                 const float* __restrict__ topk_w, int K, int H,
                                                 uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int col = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (col >= H) return;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += kUnroll) {
    // issue every load of this batch of slots before the first FMA
    int32_t r[kUnroll];
    float wk[kUnroll];
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      r[u] = (k0 + u < K) ? slot_row[t * K + k0 + u] : -1;
      wk[u] = (k0 + u < K) ? topk_w[t * K + k0 + u] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = r[u] >= 0 ? *reinterpret_cast<const uint4*>(y + (int64_t)r[u] * H + col) : make_uint4(0, 0, 0, 0);
    // k ascending, one FMA per term; a dropped slot is skipped, not added as 0
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (r[u] < 0) continue;
      const uint32_t p[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = __builtin_fmaf(wk[u], bf16_bits_to_f32(p[j] & 0xffffu), acc[2 * j]);
        acc[2 * j + 1] = __builtin_fmaf(wk[u], bf16_bits_to_f32(p[j] >> 16), acc[2 * j + 1]);
      }
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = f32_to_bf16_bits(acc[2 * j]) | (f32_to_bf16_bits(acc[2 * j + 1]) << 16);
  *reinterpret_cast<uint4*>(out + t * H + col) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_combine(const uint16_t* y, const int32_t* slot_row, const float* topk_w, int T, int K, int H,
                          uint16_t* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int slabs = (H + 2047) / 2048;
  hipLaunchKernelGGL(k_combine, dim3(T, slabs), dim3(256), 0, stream, y, slot_row, topk_w, K, H, out);
  return hipGetLastError();
}

}  // namespace qre
