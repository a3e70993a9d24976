// HBM streaming-read probe: the measured ceiling the memory-bound kernels are
// compared against (next to the published 8 TB/s).  Every lane reads 16-byte
// words of the buffer in a grid-stride loop, four in flight, and folds them
// into one word; each workgroup stores one word, so the probe moves the
// buffer's bytes and almost nothing else.
#include "qre_internal.h"

namespace qre {
namespace {

constexpr int kProbeBlocks = 2048;   // 8 workgroups of 256 lanes per CU on 256 CUs

__global__ __launch_bounds__(256) void k_hbm_read(const uint4* __restrict__ buf, int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // one lane's word per workgroup (the loads cannot be dropped: it depends on all of them)
  for (int d = 1; d < 64; d <<= 1) acc ^= __shfl_xor(acc, d);
  if (threadIdx.x == 0) sink[blockIdx.x % kProbeSinkWords] = acc;
}

}  // namespace

hipError_t launch_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(k_hbm_read, dim3(kProbeBlocks), dim3(256), 0, stream, static_cast<const uint4*>(buf), bytes / 16,
                     sink);
  return hipGetLastError();
}

}  // namespace qre
