// One-workgroup routing as device code: the stable counting sort of the
// routed slots by expert id and the GEMM row-tile lists, shared by the
// routing kernels and by kernels that run it in one of their workgroups.
//
// Method (no atomic decides any order, so the result is bit-exact and
// deterministic): every wave owns a contiguous chunk of slots and walks it 64
// slots at a time; lanes holding the same expert id find each other with one
// wave ballot per id bit (a wave-level multi-split); the lowest such lane adds
// the group's size to the wave's per-expert count, and a lane's rank inside
// its group is the popcount of the group mask below it.  An exclusive scan
// over (expert-major, wave-minor) counts gives every wave its first output
// position per expert, and the scatter re-walks the chunk in the same order,
// so equal ids keep ascending slot order.
#pragma once

#include "qre_internal.h"

namespace qre {
namespace {

constexpr int kSmallMax = 8192;   // slots handled by the one-workgroup routing
constexpr int kBatch = 4;         // 64-slot rows whose id loads are issued together

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }


// Mask of the lanes whose key equals this lane's key (keys < 2^nbits).
// Must be called by all 64 lanes.
__device__ __forceinline__ uint64_t match_any(uint32_t key, int nbits) {
  uint64_t m = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

__device__ __forceinline__ uint32_t slot_key(const int32_t* ids, int64_t s, int64_t c1, int E) {
  if (s >= c1) return (uint32_t)E;
  const int32_t id = ids[s];
  return (id >= 0 && id < E) ? (uint32_t)id : (uint32_t)E;
}

// The one-workgroup kernel keeps its wave's chunk (at most kSmallRows rows of
// 64 slots) in registers between the count and the scatter: the keys and, per
// row, each lane's mask of equal keys.  Same order of work as wave_count and
// wave_scatter, so the same result.
constexpr int kSmallRows = kSmallMax / 16 / kWave;   // 16 waves cover kSmallMax slots
struct SmallChunk {
  uint32_t key[kSmallRows];
  uint64_t m[kSmallRows];
};

__device__ void small_load(const int32_t* ids, int64_t c0, int64_t c1, int E, int nbits, SmallChunk& ch) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < kSmallRows; ++r) ch.key[r] = slot_key(ids, c0 + r * kWave + lane, c1, E);
#pragma unroll
  for (int r = 0; r < kSmallRows; ++r) ch.m[r] = (c0 + r * kWave < c1) ? match_any(ch.key[r], nbits) : 0ull;   // uniform
}

__device__ void small_count(const SmallChunk& ch, int64_t c0, int64_t c1, int E, int* hist_row) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < kSmallRows; ++r)
    if (c0 + r * kWave < c1 && ch.key[r] < (uint32_t)E && lane == __builtin_ctzll(ch.m[r]))
      hist_row[ch.key[r]] += __popcll(ch.m[r]);
}

__device__ void small_scatter(const SmallChunk& ch, int64_t c0, int64_t c1, int E, int* base_row,
                              int32_t* sorted_slot, int32_t* slot_row) {
  const int lane = lane_id();
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < kSmallRows; ++r) {
    if (c0 + r * kWave >= c1) continue;                     // uniform
    const int64_t s = c0 + r * kWave + lane;
    const uint32_t key = ch.key[r];
    if (s < c1) {
      if (key < (uint32_t)E) {
        const int pos = base_row[key] + __popcll(ch.m[r] & below);
        sorted_slot[pos] = (int32_t)s;
        slot_row[s] = pos;
      } else {
        slot_row[s] = -1;
      }
    }
    // every lane has read base_row[key] above; LDS ops of one wave stay in order
    if (key < (uint32_t)E && lane == __builtin_ctzll(ch.m[r])) base_row[key] += __popcll(ch.m[r]);
  }
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then the
// row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Exclusive scan of data[0, n) (LDS) by the whole workgroup; returns the total.
__device__ int block_exclusive_scan(int* data, int n, int* wave_tmp) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = ceil_div(n, nt);
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += data[i];
  const int v = wave_incl_scan(local);
  if (lane_id() == kWave - 1) wave_tmp[tid / kWave] = v;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < nt / kWave; ++w) {
    if (w < tid / kWave) before += wave_tmp[w];
    total += wave_tmp[w];
  }
  int run = before + v - local;
  for (int i = lo; i < hi; ++i) {
    const int c = data[i];
    data[i] = run;
    run += c;
  }
  __syncthreads();
  return total;
}

// Write the row-tile list of height bm from cnt[e] and offs[e] (LDS), into
// tiles (and into tiles2 too, when given: two lists of the same height).
// scratch (LDS, E entries) is clobbered.  All threads must call.
__device__ void build_tiles(const int* cnt, const int* offs, int E, int bm, int* scratch, int* wave_tmp,
                            Tile* tiles, int32_t* ntiles, Tile* tiles2 = nullptr, int32_t* ntiles2 = nullptr) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) scratch[e] = ceil_div(cnt[e], bm);
  __syncthreads();
  const int total = block_exclusive_scan(scratch, E, wave_tmp);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int nt = ceil_div(cnt[e], bm);
    for (int j = 0; j < nt; ++j) {
      Tile t;
      t.e = e;
      t.row0 = offs[e] + j * bm;
      t.nrows = min(bm, cnt[e] - j * bm);
      t.pad = 0;
      tiles[scratch[e] + j] = t;
      if (tiles2) tiles2[scratch[e] + j] = t;
    }
  }
  if (threadIdx.x == 0) {
    *ntiles = total;
    if (ntiles2) *ntiles2 = total;
  }
  __syncthreads();
}

// The whole permutation and tile lists in one workgroup of NW waves (every
// thread of the workgroup calls).  lds: route_small_lds_ints(NW, E) ints:
// hist[NW][E], cnt[E], offs[E+1], scratch[E], wave_tmp[NW].
template <int NW>
__device__ void route_small(int* lds, const int32_t* __restrict__ ids, int S, int E, int nbits, int32_t* counts,
                            int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row, int32_t* dropped,
                            Tile* tiles_a, int32_t* ntiles_a, int bm_a, Tile* tiles_b, int32_t* ntiles_b, int bm_b) {
  int* hist = lds;                 // [NW][E]
  int* cnt = hist + NW * E;        // [E]
  int* offs = cnt + E;             // [E+1]
  int* scratch = offs + E + 1;     // [E]
  int* wave_tmp = scratch + E;     // [NW]
  const int tid = threadIdx.x, w = tid / kWave;
  for (int i = tid; i < NW * E; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int64_t L = (int64_t)ceil_div(ceil_div(S, NW), kWave) * kWave;
  const int64_t c0 = min((int64_t)S, w * L), c1 = min((int64_t)S, c0 + L);
  SmallChunk ch;
  small_load(ids, c0, c1, E, nbits, ch);
  small_count(ch, c0, c1, E, hist + w * E);
  __syncthreads();
  // per expert: prefix over waves, total count
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    for (int v = 0; v < NW; ++v) {
      const int c = hist[v * E + e];
      hist[v * E + e] = run;
      run += c;
    }
    cnt[e] = run;
    offs[e] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan(offs, E, wave_tmp);
  if (tid == 0) {
    offs[E] = total;
    if (dropped) *dropped = S - total;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += blockDim.x) {
    offsets[e] = offs[e];
    if (e < E) counts[e] = cnt[e];
  }
  for (int i = tid; i < NW * E; i += blockDim.x) hist[i] += offs[i % E];
  __syncthreads();
  small_scatter(ch, c0, c1, E, hist + w * E, sorted_slot, slot_row);
  for (int i = total + tid; i < S; i += blockDim.x) sorted_slot[i] = -1;
  if (tiles_a && tiles_b && bm_a == bm_b) {
    build_tiles(cnt, offs, E, bm_a, scratch, wave_tmp, tiles_a, ntiles_a, tiles_b, ntiles_b);
  } else {
    if (tiles_a) build_tiles(cnt, offs, E, bm_a, scratch, wave_tmp, tiles_a, ntiles_a);
    if (tiles_b) build_tiles(cnt, offs, E, bm_b, scratch, wave_tmp, tiles_b, ntiles_b);
  }
}


constexpr size_t route_small_lds_ints(int NW, int E) { return (size_t)NW * E + 3 * (size_t)E + 1 + NW; }

// Bits of an expert key (keys 0..E, E being the drop sentinel).
inline int bits_for(int E) {
  int b = 0;
  while ((1 << b) <= E) ++b;
  return b;
}

}  // namespace
}  // namespace qre
