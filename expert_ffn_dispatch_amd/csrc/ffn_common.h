// Device-side tile list shared by the grouped SwiGLU kernels.
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kMaxGroups = 256;

// Loads the group offsets into LDS and forms the inclusive prefix of tiles:
// s_tp[e+1] = sum_{g<=e} tiles(g), tiles(g) = row_tiles(count_g) * col_tiles
// (ROWS_PER_TILE = 0: one row tile per non-empty group).  Row tiles of an
// empty group are 0, so empty experts never appear.  The first wave does the
// work (each lane owns four consecutive groups, a shuffle scan joins them);
// every thread of the block must call it (one barrier).
template <int ROWS_PER_TILE>
__device__ __forceinline__ int build_tile_list(const FfnArgs& p, int col_tiles, int* s_off, int* s_tp) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    const int E = p.E;
    int off[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int e = lane * 4 + i;
      off[i] = 0;
      if (e <= E) off[i] = (p.fixed_rows > 0) ? (e == 0 ? 0 : p.fixed_rows) : p.offsets[e];
    }
    int t[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      int tv = 0;
      if (e < E) {
        const int cnt = off[i + 1] - off[i];
        tv = (ROWS_PER_TILE > 0 ? ceil_div(cnt, ROWS_PER_TILE) : (cnt > 0 ? 1 : 0)) * col_tiles;
      }
      sum += tv;
      t[i] = sum;                       // inclusive within the lane
    }
    int inc = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(inc, d);
      if (lane >= d) inc += o;
    }
    const int base = inc - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      if (e < E) {
        s_off[e] = off[i];
        s_tp[e + 1] = base + t[i];
      }
    }
    if (lane == ((E - 1) >> 2)) {          // this lane also holds offsets[E]
      const int j = E - 4 * lane;          // 1..4
      s_off[E] = j == 1 ? off[1] : j == 2 ? off[2] : j == 3 ? off[3] : off[4];
    }
    if (lane == 0) s_tp[0] = 0;
  }
  __syncthreads();
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
