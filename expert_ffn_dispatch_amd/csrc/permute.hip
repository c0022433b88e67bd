// Dispatch and permutation: per-expert counts, exclusive-scan offsets and a
// stable sort of the N*k assignments into expert order, plus the row gather.
//
// Page on MoE latency (wink.run), section "router 之后还有一串动作": top-k routing
// turns N tokens into N*k assignments; grouping them by expert is the
// dispatch, sorting the token rows by expert the permutation.  Order inside an
// expert group is by assignment index a = n*k + j (stable), which makes the
// permutation unique.
//
// Three launches, no atomics on anything that orders rows:
//   hist    - one block per tile of 256 assignments: LDS histogram (integer
//             atomics only count) -> tile_hist[e][t]
//   scan    - one block per expert: exclusive scan of tile_hist over the
//             tiles -> tile_off, and the expert's count
//   (the scatter blocks each scan the counts into the expert offsets; the
//   first one also stores them)
//   scatter - one block per tile: rank inside the tile from wave ballots
//             (lanes with the same expert and a lower lane id) plus the
//             counts of earlier waves, so sorted slot =
//             offsets[e] + tile_off[e][t] + rank.
// A batch of at most kSmallPermute assignments takes one launch instead:
// each of its blocks counts and scans all the assignments and places its own
// chunk of 1024 (the counts of the chunks before it give its expert bases).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int A, int E, int T,
                                                   int32_t* __restrict__ tile_hist) {
  __shared__ int h[256];
  const int tid = threadIdx.x, tile = blockIdx.x;
  if (tid < E) h[tid] = 0;
  __syncthreads();
  const int a = tile * kPermTile + tid;
  if (a < A) atomicAdd(&h[clamp_expert(ids[a], E)], 1);
  __syncthreads();
  if (tid < E) tile_hist[(size_t)tid * T + tile] = h[tid];
}

// One block per expert: exclusive scan of its tile counts over the tiles,
// 1024 tiles per pass (four consecutive per thread), and the expert's total.
__global__ __launch_bounds__(256) void scan_kernel(const int32_t* __restrict__ tile_hist, int T,
                                                   int32_t* __restrict__ tile_off, int32_t* __restrict__ counts) {
  __shared__ int wsum[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* h = tile_hist + (size_t)e * T;
  int32_t* o = tile_off + (size_t)e * T;
  int carry = 0;
  for (int t0 = 0; t0 < T; t0 += 1024) {
    int v[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + tid * 4 + i;
      v[i] = t < T ? h[t] : 0;
      s += v[i];
    }
    int inc = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int q = __shfl_up(inc, off);
      if (lane >= off) inc += q;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    int run = before + inc - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + tid * 4 + i;
      if (t < T) o[t] = run;
      run += v[i];
    }
    carry += total;
    __syncthreads();              // wsum is rewritten by the next pass
  }
  if (tid == 0) counts[e] = carry;
}

__global__ __launch_bounds__(256) void scatter_kernel(PermuteArgs p, int T, int nbits) {
  __shared__ int wc[4][256];
  __shared__ int s_base[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, tile = blockIdx.x;
  if (tile == 0 && tid < p.n_zero) p.zero[tid] = 0;
  for (int i = tid; i < 4 * 256; i += 256) (&wc[0][0])[i] = 0;
  // expert offsets: exclusive scan of the counts (every block; block 0 also
  // publishes them)
  if (wave == 0) {
    int v[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      v[i] = (e < p.E) ? p.counts[e] : 0;
      s += v[i];
    }
    int inc = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int q = __shfl_up(inc, off);
      if (lane >= off) inc += q;
    }
    int b = inc - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      if (e < p.E) {
        s_base[e] = b;
        if (tile == 0) p.offsets[e] = b;
      }
      b += v[i];
    }
    if (tile == 0 && lane == 63) p.offsets[p.E] = inc;
  }
  __syncthreads();
  const int a = tile * kPermTile + tid;
  const bool valid = a < p.A;
  const int e = valid ? clamp_expert(p.ids[a], p.E) : 0;
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(valid && bit);
    peers &= bit ? m : ~m;
  }
  const int rank = lanes_below(peers);
  if (valid && rank == 0) wc[wave][e] = __popcll(peers);
  __syncthreads();
  if (valid) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wc[w][e];
    const int pos = s_base[e] + p.tile_off[(size_t)e * T + tile] + before + rank;
    p.s2a[pos] = a;
    p.a2s[a] = pos;
    if (p.row_token) p.row_token[pos] = a / p.k;
    if (p.row_weight) p.row_weight[pos] = p.weights[a];
  }
}

// Up to 4096 assignments the single launch below; above, each of its blocks
// counting every assignment costs more than the three launches (Qwen3-235B-
// shaped batch, 65536 assignments: 29.0 against 15.5 us; DeepSeek-V2-shaped,
// 24576: 16.1 against 14.4 us).
constexpr int kSmallPermute = 4096;

// The same dispatch and stable permutation for a small batch, in one launch
// of ceil(A / 1024) blocks of 16 waves.  Every block counts all A
// assignments in LDS (and those of the chunks before its own), scans the
// counts with one wave, and then ranks and places its own chunk of 1024
// assignments like the scatter kernel's tiles: offset of the expert, plus
// the expert's assignments in earlier chunks, in earlier waves of the chunk
// and in lower lanes of the wave.  Counting 4096 ids again in each block is
// cheaper than one block placing all of them: the placements are scattered
// 4-byte stores, which one CU issues one address at a time (Qwen3-30B-shaped
// batch of 512 tokens, 4096 assignments: 12.4 us as one block).  Block 0
// also stores the counts and offsets and clears the tile queue words.
__global__ __launch_bounds__(1024) void permute_small_kernel(PermuteArgs p, int nbits) {
  __shared__ int cnt[256];
  __shared__ int base[256];     // assignments of each expert in the chunks before this block's
  __shared__ int off_s[256];
  __shared__ int wc[16][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E, A = p.A, chunk = blockIdx.x;
  if (chunk == 0 && tid < p.n_zero) p.zero[tid] = 0;
  if (tid < E) {
    cnt[tid] = 0;
    base[tid] = 0;
  }
  for (int i = tid; i < 16 * 256; i += 1024) (&wc[0][0])[i] = 0;
  const int a = chunk * 1024 + tid;
  const bool valid = a < A;
  const int e = valid ? clamp_expert(p.ids[a], E) : 0;
  const float wv = (valid && p.row_weight) ? p.weights[a] : 0.f;
  __syncthreads();
  // every assignment's expert, counted (and those of the earlier chunks)
  const int nch = (A + 1023) >> 10;
#pragma unroll 8
  for (int c = 0; c < nch; ++c) {
    const int ac = c * 1024 + tid;
    if (ac < A) {
      const int ec = clamp_expert(p.ids[ac], E);
      atomicAdd(&cnt[ec], 1);
      if (c < chunk) atomicAdd(&base[ec], 1);
    }
  }
  __syncthreads();
  if (wave == 0) {
    int v[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = lane * 4 + i;
      v[i] = (ee < E) ? cnt[ee] : 0;
      s += v[i];
    }
    int inc = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    int b = inc - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = lane * 4 + i;
      if (ee < E) {
        if (chunk == 0) {
          p.counts[ee] = v[i];
          p.offsets[ee] = b;
        }
        off_s[ee] = b;
      }
      b += v[i];
    }
    if (chunk == 0 && lane == 63) p.offsets[E] = inc;
  }
  // lanes of this wave with the same expert, and this lane's rank among them
  uint64_t peers = __ballot(valid);
  for (int bt = 0; bt < nbits; ++bt) {
    const bool bit = (e >> bt) & 1;
    const uint64_t m = __ballot(valid && bit);
    peers &= bit ? m : ~m;
  }
  const int rank = lanes_below(peers);
  if (valid && rank == 0) wc[wave][e] = __popcll(peers);
  __syncthreads();
  if (valid) {
    int before = base[e];
    for (int w = 0; w < wave; ++w) before += wc[w][e];
    const int pos = off_s[e] + before + rank;
    p.s2a[pos] = a;
    p.a2s[a] = pos;
    if (p.row_token) p.row_token[pos] = a / p.k;
    if (p.row_weight) p.row_weight[pos] = wv;
  }
}

// Row copy: one block moves `rows` rows of M bf16 in 16-byte chunks.
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* __restrict__ x,
                                                     const int32_t* __restrict__ s2a, int k, int A,
                                                     int M, uint16_t* __restrict__ xs) {
  const int chunks = M >> 3;
  const int rows_per_block = (256 / chunks) > 0 ? (256 / chunks) : 1;
  const int p0 = blockIdx.x * rows_per_block;
  for (int i = threadIdx.x; i < rows_per_block * chunks; i += 256) {
    const int r = i / chunks, c = i - r * chunks;
    const int p = p0 + r;
    if (p >= A) break;
    const int tok = s2a[p] / k;
    *reinterpret_cast<uint4*>(xs + (size_t)p * M + c * 8) =
        *reinterpret_cast<const uint4*>(x + (size_t)tok * M + c * 8);
  }
}

}  // namespace

__global__ __launch_bounds__(64) void zero_words_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0;
}

hipError_t launch_zero_words(int32_t* p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t st) {
  const int T = ceil_div(a.A, kPermTile);
  int nbits = 0;
  while ((1 << nbits) < a.E) ++nbits;
  if (a.A <= kSmallPermute) {
    const int blocks = a.A > 1024 ? ceil_div(a.A, 1024) : 1;
    hipLaunchKernelGGL(permute_small_kernel, dim3(blocks), dim3(1024), 0, st, a, nbits);
    return hipGetLastError();
  }
  if (T > 0) {
    hipLaunchKernelGGL(hist_kernel, dim3(T), dim3(256), 0, st, a.ids, a.A, a.E, T, a.tile_hist);
  }
  hipLaunchKernelGGL(scan_kernel, dim3(a.E), dim3(256), 0, st, a.tile_hist, T, a.tile_off, a.counts);
  if (T > 0) {
    hipLaunchKernelGGL(scatter_kernel, dim3(T), dim3(256), 0, st, a, T, nbits);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const uint16_t* x, const int32_t* s2a, int k, int A, int M, uint16_t* xs,
                         hipStream_t st) {
  if (A == 0) return hipSuccess;
  const int chunks = M >> 3;
  const int rpb = (256 / chunks) > 0 ? (256 / chunks) : 1;
  hipLaunchKernelGGL(gather_kernel, dim3(ceil_div(A, rpb)), dim3(256), 0, st, x, s2a, k, A, M, xs);
  return hipGetLastError();
}

}  // namespace moe
