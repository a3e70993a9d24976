// Token->expert permutation for the routed-expert feed-forward: a stable
// counting sort of the slots s = t*K + k by expert id, plus the GEMM row-tile
// list.  The minnow README (section "Quantization") routes 32-token decode
// blocks on the GPU by default; this is that step for CDNA4.
//
// Method (no atomic decides any order, so the result is bit-exact and
// deterministic):
//  * every wave owns a contiguous chunk of slots and walks it 64 slots at a
//    time; lanes holding the same expert id find each other with one wave
//    ballot per id bit (a wave-level multi-split); the lowest such lane adds
//    the group's size to the wave's per-expert count, and a lane's rank inside
//    its group is the popcount of the group mask below it;
//  * an exclusive scan over (expert-major, wave-minor) counts gives every wave
//    its first output position per expert (in the three-kernel path: a prefix
//    over the waves per expert, parallel over experts, then each scatter
//    workgroup scans the E totals itself);
//  * the scatter pass re-walks the chunk in the same order, so equal ids keep
//    ascending slot order.
// Small problems (S <= kSmallMax) do all of it in one workgroup with the
// tables in LDS; larger ones use three kernels with the per-wave table in HBM.
#include <algorithm>

#include "quant_act.h"
#include "route_small.h"

namespace qre {
namespace {

constexpr int kLargeChunk = 256;  // slots per wave in the three-kernel path

// Count this wave's chunk [c0, c1) into hist_row[E] (LDS, zeroed by the caller).
// The ids of kBatch rows of 64 slots are loaded before the first is counted.
__device__ void wave_count(const int32_t* ids, int64_t c0, int64_t c1, int E, int nbits, int* hist_row) {
  const int lane = lane_id();
  for (int64_t base = c0; base < c1; base += kWave * kBatch) {
    uint32_t key[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) key[b] = slot_key(ids, base + b * kWave + lane, c1, E);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const uint64_t m = match_any(key[b], nbits);
      if (key[b] < (uint32_t)E && lane == __builtin_ctzll(m)) hist_row[key[b]] += __popcll(m);
    }
  }
}

// Scatter this wave's chunk; base_row[e] (LDS) holds the next output position
// of expert e for this wave and is advanced as the chunk is walked (in slot
// order, so equal ids keep ascending slot order).
__device__ void wave_scatter(const int32_t* ids, int64_t c0, int64_t c1, int E, int nbits, int* base_row,
                             int32_t* sorted_slot, int32_t* slot_row) {
  const int lane = lane_id();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int64_t base0 = c0; base0 < c1; base0 += kWave * kBatch) {
    uint32_t key[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) key[b] = slot_key(ids, base0 + b * kWave + lane, c1, E);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int64_t s = base0 + b * kWave + lane;
      const uint64_t m = match_any(key[b], nbits);
      if (s < c1) {
        if (key[b] < (uint32_t)E) {
          const int pos = base_row[key[b]] + __popcll(m & below);
          sorted_slot[pos] = (int32_t)s;
          slot_row[s] = pos;
        } else {
          slot_row[s] = -1;
        }
      }
      // every lane has read base_row[key] above; LDS ops of one wave stay in order
      if (key[b] < (uint32_t)E && lane == __builtin_ctzll(m)) base_row[key[b]] += __popcll(m);
    }
  }
}

template <int NW>
__global__ __launch_bounds__(NW * kWave) void k_route_small(const int32_t* __restrict__ ids, int S, int E,
                                                            int nbits, int32_t* counts, int32_t* offsets,
                                                            int32_t* sorted_slot, int32_t* slot_row,
                                                            int32_t* dropped, Tile* tiles_a, int32_t* ntiles_a, int bm_a,
                                                            Tile* tiles_b, int32_t* ntiles_b, int bm_b) {
  extern __shared__ int lds[];
  route_small<NW>(lds, ids, S, E, nbits, counts, offsets, sorted_slot, slot_row, dropped, tiles_a, ntiles_a, bm_a,
                  tiles_b, ntiles_b, bm_b);
}

// Rows [r0, r1) of the INT8 quantization of x by workgroup blk of nblk.
__device__ __forceinline__ void quantize_x_rows(const QuantX& qx, int r0, int r1, int blk, int nblk) {
  const int G = qx.cols / kGroup;
  quantize_act_groups(qx.v + (int64_t)r0 * qx.cols, (int64_t)(r1 - r0) * G, G, qx.q + (int64_t)r0 * qx.cols,
                      qx.s + (int64_t)r0 * G, blk, nblk);
}

// Three-kernel path.  ghist[gw][E]: per-wave counts, then per-wave bases.
// The workgroups past the first nroute of each launch quantize a third of
// the rows of x (qx.rows == 0: none), which no routing step reads.
__global__ __launch_bounds__(256) void k_route_count(const int32_t* __restrict__ ids, int S, int E, int nbits,
                                                     int32_t* ghist, int nroute, QuantX qx) {
  if ((int)blockIdx.x >= nroute) {
    quantize_x_rows(qx, 0, qx.rows / 3, (int)blockIdx.x - nroute, (int)gridDim.x - nroute);
    return;
  }
  extern __shared__ int lds[];
  const int w = threadIdx.x / kWave;
  int* row = lds + w * E;
  for (int i = threadIdx.x; i < 4 * E; i += blockDim.x) lds[i] = 0;
  __syncthreads();
  const int64_t gw = (int64_t)blockIdx.x * 4 + w;
  const int64_t c0 = min((int64_t)S, gw * kLargeChunk), c1 = min((int64_t)S, c0 + kLargeChunk);
  wave_count(ids, c0, c1, E, nbits, row);
  // the wave reads back its own LDS row (in-order within the wave)
  for (int e = lane_id(); e < E; e += kWave) ghist[gw * E + e] = row[e];
}

// Per-expert prefix over the waves' counts, relative to the expert's first
// sorted row, and the per-expert totals.  Experts are independent, so a
// workgroup takes kPxE of them: thread (el, q) walks partition q of the wave
// range for expert el (consecutive el read consecutive ints), pass 1 sums the
// partition, the partition sums are scanned in LDS, pass 2 rewrites the counts
// as bases.
constexpr int kPxE = 32, kPxP = 8;   // experts x partitions = 256 threads
__global__ __launch_bounds__(256) void k_route_prefix(int32_t* ghist, int nwaves, int E, int32_t* counts, int nroute,
                                                      QuantX qx) {
  if ((int)blockIdx.x >= nroute) {
    quantize_x_rows(qx, qx.rows / 3, 2 * (qx.rows / 3), (int)blockIdx.x - nroute, (int)gridDim.x - nroute);
    return;
  }
  __shared__ int part[kPxP][kPxE];
  const int el = threadIdx.x % kPxE, q = threadIdx.x / kPxE;
  const int e = blockIdx.x * kPxE + el;
  const int v0 = (int)((int64_t)q * nwaves / kPxP), v1 = (int)((int64_t)(q + 1) * nwaves / kPxP);
  constexpr int U = 16;            // loads in flight per thread
  int sum = 0;
  if (e < E) {
    int v = v0;
    for (; v + U <= v1; v += U) {
      int c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = ghist[(int64_t)(v + u) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) sum += c[u];
    }
    for (; v < v1; ++v) sum += ghist[(int64_t)v * E + e];
  }
  part[q][el] = sum;
  __syncthreads();
  int run = 0;
  for (int j = 0; j < q; ++j) run += part[j][el];
  if (e < E) {
    int v = v0;
    for (; v + U <= v1; v += U) {
      int c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = ghist[(int64_t)(v + u) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ghist[(int64_t)(v + u) * E + e] = run;
        run += c[u];
      }
    }
    for (; v < v1; ++v) {
      const int c = ghist[(int64_t)v * E + e];
      ghist[(int64_t)v * E + e] = run;
      run += c;
    }
    if (q == kPxP - 1) counts[e] = run;
  }
}

// Each workgroup scans the per-expert counts itself (E values); workgroup 0
// also writes offsets and the row-tile lists.  Then every wave scatters its
// chunk from its bases.  LDS: rows[4][E], cnt[E], offs[E+1], scratch[E],
// wave_tmp[4].
// Scatter pass of workgroup blk of nblk (LDS: 7E + 5 ints).
__device__ void route_scatter(int* lds, const int32_t* __restrict__ ids, int S, int E, int nbits, const int32_t* ghist,
                              const int32_t* counts, int32_t* offsets, int32_t* dropped, Tile* tiles_a,
                              int32_t* ntiles_a, int bm_a, Tile* tiles_b, int32_t* ntiles_b, int bm_b,
                              int32_t* sorted_slot, int32_t* slot_row, int blk, int nblk) {
  int* rows = lds;                 // [4][E]
  int* cnt = rows + 4 * E;         // [E]
  int* offs = cnt + E;             // [E+1]
  int* scratch = offs + E + 1;     // [E]
  int* wave_tmp = scratch + E;     // [4]
  const int tid = threadIdx.x, w = tid / kWave;
  for (int e = tid; e < E; e += blockDim.x) {
    const int c = counts[e];
    cnt[e] = c;
    offs[e] = c;
  }
  __syncthreads();
  const int total = block_exclusive_scan(offs, E, wave_tmp);
  if (tid == 0) offs[E] = total;
  __syncthreads();
  if (blk == 0) {                  // uniform over the workgroup
    for (int e = tid; e <= E; e += blockDim.x) offsets[e] = offs[e];
    if (tid == 0 && dropped) *dropped = S - total;
    if (tiles_a && tiles_b && bm_a == bm_b) {
      build_tiles(cnt, offs, E, bm_a, scratch, wave_tmp, tiles_a, ntiles_a, tiles_b, ntiles_b);
    } else {
      if (tiles_a) build_tiles(cnt, offs, E, bm_a, scratch, wave_tmp, tiles_a, ntiles_a);
      if (tiles_b) build_tiles(cnt, offs, E, bm_b, scratch, wave_tmp, tiles_b, ntiles_b);
    }
  }
  int* row = rows + w * E;
  const int64_t gw = (int64_t)blk * 4 + w;
  for (int e = lane_id(); e < E; e += kWave) row[e] = ghist[gw * E + e] + offs[e];
  const int64_t c0 = min((int64_t)S, gw * kLargeChunk), c1 = min((int64_t)S, c0 + kLargeChunk);
  wave_scatter(ids, c0, c1, E, nbits, row, sorted_slot, slot_row);
  for (int64_t i = total + (int64_t)blk * blockDim.x + threadIdx.x; i < S; i += (int64_t)nblk * blockDim.x)
    sorted_slot[i] = -1;
}

__global__ __launch_bounds__(256) void k_route_scatter(const int32_t* __restrict__ ids, int S, int E, int nbits,
                                                       const int32_t* ghist, const int32_t* counts, int32_t* offsets,
                                                       int32_t* dropped, Tile* tiles_a, int32_t* ntiles_a, int bm_a,
                                                       Tile* tiles_b, int32_t* ntiles_b, int bm_b, int32_t* sorted_slot,
                                                       int32_t* slot_row) {
  extern __shared__ int lds[];
  route_scatter(lds, ids, S, E, nbits, ghist, counts, offsets, dropped, tiles_a, ntiles_a, bm_a, tiles_b, ntiles_b,
                bm_b, sorted_slot, slot_row, blockIdx.x, gridDim.x);
}

// The scatter (the first nscatter workgroups) and the INT8 quantization of x
// (the others) in one launch: neither reads what the other writes.
__global__ __launch_bounds__(256) void k_route_scatter_qx(const int32_t* __restrict__ ids, int S, int E, int nbits,
                                                          const int32_t* ghist, const int32_t* counts,
                                                          int32_t* offsets, int32_t* dropped, Tile* tiles_a,
                                                          int32_t* ntiles_a, int bm_a, Tile* tiles_b,
                                                          int32_t* ntiles_b, int bm_b, int32_t* sorted_slot,
                                                          int32_t* slot_row, int nscatter, QuantX qx) {
  extern __shared__ int lds[];
  if ((int)blockIdx.x < nscatter) {
    route_scatter(lds, ids, S, E, nbits, ghist, counts, offsets, dropped, tiles_a, ntiles_a, bm_a, tiles_b, ntiles_b,
                  bm_b, sorted_slot, slot_row, blockIdx.x, nscatter);
    return;
  }
  quantize_x_rows(qx, 2 * (qx.rows / 3), qx.rows, (int)blockIdx.x - nscatter, (int)gridDim.x - nscatter);
}

__global__ __launch_bounds__(256) void k_build_tiles(const int32_t* offsets, int E, Tile* tiles_a,
                                                     int32_t* ntiles_a, int bm_a, Tile* tiles_b, int32_t* ntiles_b,
                                                     int bm_b) {
  extern __shared__ int lds[];
  int* cnt = lds;
  int* offs = cnt + E;
  int* scratch = offs + E + 1;
  int* wave_tmp = scratch + E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    offs[e] = offsets[e];
    cnt[e] = offsets[e + 1] - offsets[e];
  }
  __syncthreads();
  build_tiles(cnt, offs, E, bm_a, scratch, wave_tmp, tiles_a, ntiles_a);
  if (tiles_b) build_tiles(cnt, offs, E, bm_b, scratch, wave_tmp, tiles_b, ntiles_b);
}

}  // namespace

size_t route_scratch_bytes(int64_t S, int E) {
  if (S <= kSmallMax) return 0;
  const int64_t nwaves = (S + kLargeChunk - 1) / kLargeChunk;
  const int64_t nwaves4 = (nwaves + 3) / 4 * 4;
  return (size_t)nwaves4 * E * sizeof(int32_t);
}

int64_t max_tiles(int64_t S, int E, int bm) {
  // sum_e ceil(c_e / bm) <= (S + min(E, S) * (bm - 1)) / bm
  const int64_t touched = S < E ? S : E;
  return (S + touched * (bm - 1)) / bm;
}

hipError_t launch_route(const int32_t* ids, int T, int K, int E, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_slot, int32_t* slot_row, int32_t* dropped, void* ws, Tile* tiles_a,
                        int32_t* ntiles_a, int bm_a, Tile* tiles_b, int32_t* ntiles_b, int bm_b, hipStream_t stream,
                        const QuantX* qx) {
  const int64_t S = (int64_t)T * K;
  const int nbits = bits_for(E);
  if (S <= 512) {
    constexpr int NW = 4;
    const size_t lds = sizeof(int) * route_small_lds_ints(NW, E);
    hipLaunchKernelGGL(k_route_small<NW>, dim3(1), dim3(NW * kWave), lds, stream, ids, (int)S, E, nbits, counts,
                       offsets, sorted_slot, slot_row, dropped, tiles_a, ntiles_a, bm_a, tiles_b, ntiles_b, bm_b);
    const hipError_t err = hipGetLastError();
    return (err == hipSuccess && qx) ? launch_quantize_act(qx->v, qx->rows, qx->cols, qx->q, qx->s, stream) : err;
  }
  // the one-workgroup kernel holds at most kSmallRows rows of 64 slots per
  // wave in registers: 4 waves up to 512 slots, 16 waves up to kSmallMax
  static_assert(512 / 4 <= kSmallRows * kWave && kSmallMax / 16 <= kSmallRows * kWave, "chunk exceeds registers");
  if (S <= kSmallMax) {
    constexpr int NW = 16;
    const size_t lds = sizeof(int) * route_small_lds_ints(NW, E);
    hipLaunchKernelGGL(k_route_small<NW>, dim3(1), dim3(NW * kWave), lds, stream, ids, (int)S, E, nbits, counts,
                       offsets, sorted_slot, slot_row, dropped, tiles_a, ntiles_a, bm_a, tiles_b, ntiles_b, bm_b);
    const hipError_t err = hipGetLastError();
    return (err == hipSuccess && qx) ? launch_quantize_act(qx->v, qx->rows, qx->cols, qx->q, qx->s, stream) : err;
  }
  int32_t* ghist = static_cast<int32_t*>(ws);
  const int64_t nwaves = (S + kLargeChunk - 1) / kLargeChunk;
  const int nblocks = (int)((nwaves + 3) / 4);
  // the quantization of x, a third of its rows in each of the three launches
  const QuantX none = {nullptr, 0, kGroup, nullptr, nullptr};
  const QuantX q3 = (qx && qx->rows > 0) ? *qx : none;
  auto qblocks = [&](int r0, int r1) -> int64_t {
    const int64_t ngroups = (int64_t)(r1 - r0) * (q3.cols / kGroup);
    return std::min((ngroups + 15) / 16, kMaxQuantBlocks);
  };
  const int npx = (E + kPxE - 1) / kPxE;
  hipLaunchKernelGGL(k_route_count, dim3((unsigned)(nblocks + qblocks(0, q3.rows / 3))), dim3(256),
                     sizeof(int) * 4 * E, stream, ids, (int)S, E, nbits, ghist, nblocks, q3);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_route_prefix, dim3((unsigned)(npx + qblocks(q3.rows / 3, 2 * (q3.rows / 3)))), dim3(256), 0,
                     stream, ghist, nblocks * 4, E, counts, npx, q3);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t slds = sizeof(int) * (size_t)(7 * E + 5);
  if (q3.rows > 0) {
    hipLaunchKernelGGL(k_route_scatter_qx, dim3((unsigned)(nblocks + qblocks(2 * (q3.rows / 3), q3.rows))), dim3(256),
                       slds, stream, ids, (int)S, E, nbits, ghist, counts, offsets, dropped, tiles_a, ntiles_a, bm_a,
                       tiles_b, ntiles_b, bm_b, sorted_slot, slot_row, nblocks, q3);
  } else {
    hipLaunchKernelGGL(k_route_scatter, dim3(nblocks), dim3(256), slds, stream, ids, (int)S, E, nbits, ghist, counts,
                       offsets, dropped, tiles_a, ntiles_a, bm_a, tiles_b, ntiles_b, bm_b, sorted_slot, slot_row);
  }
  return hipGetLastError();
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, Tile* tiles_a, int32_t* ntiles_a, int bm_a,
                              Tile* tiles_b, int32_t* ntiles_b, int bm_b, hipStream_t stream) {
  hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(256), sizeof(int) * (size_t)(3 * E + 1 + 4), stream, offsets,
                     E, tiles_a, ntiles_a, bm_a, tiles_b, ntiles_b, bm_b);
  return hipGetLastError();
}

}  // namespace qre
