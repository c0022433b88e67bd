// Device-side tile list shared by the grouped SwiGLU kernels.
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kMaxGroups = 256;

// Loads the group offsets into LDS and forms the inclusive prefix of tiles:
// tprefix[e+1] = sum_{g<=e} tiles(g), tiles(g) = row_tiles(count_g) * col_tiles.
// Row tiles of an empty group are 0, so empty experts never appear.  Must be
// called by every thread of the block (blockDim.x >= 256).
template <int ROWS_PER_TILE>
__device__ __forceinline__ int build_tile_list(const FfnArgs& p, int col_tiles, int* s_off, int* s_tp) {
  const int tid = threadIdx.x;
  if (p.fixed_rows > 0) {
    if (tid == 0) {
      s_off[0] = 0;
      s_off[1] = p.fixed_rows;
    }
  } else {
    for (int e = tid; e <= p.E; e += blockDim.x) s_off[e] = p.offsets[e];
  }
  __syncthreads();
  int tv = 0;
  if (tid < p.E) {
    const int cnt = s_off[tid + 1] - s_off[tid];
    tv = (ROWS_PER_TILE > 0 ? ceil_div(cnt, ROWS_PER_TILE) : (cnt > 0 ? 1 : 0)) * col_tiles;
  }
  if (tid < kMaxGroups) s_tp[tid + 1] = tv;   // groups beyond E contribute 0
  if (tid == 0) s_tp[0] = 0;
  __syncthreads();
  for (int off = 1; off < kMaxGroups; off <<= 1) {
    const int t = (tid < kMaxGroups && tid >= off) ? s_tp[tid + 1 - off] : 0;
    __syncthreads();
    if (tid < kMaxGroups) s_tp[tid + 1] += t;
    __syncthreads();
  }
  return s_tp[p.E];
}

// Group holding tile `t`: the largest e with s_tp[e] <= t.
__device__ __forceinline__ int find_group(const int* s_tp, int E, int t) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tp[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace moe
