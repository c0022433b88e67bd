// Single-launch MoE layer for decode-sized batches.
//
// Page on MoE latency (wink.run), "MoE 少算 FLOPs，延迟反而涨了：慢在搬 token 的路上":
// at decode the expert GEMMs are short, and the steps around them (router,
// dispatch, permutation, combine) are latency, not FLOPs.  Issued as one
// kernel each, every step also pays a launch and a wait for the previous one;
// for a one-token batch those waits are most of the layer.  Here one
// cooperative launch (every block resident at once) runs the whole layer for
// at most kDecodeTokens tokens and kDecodeAssign assignments, with three
// grid-wide barriers:
//   1. router partial scores: block g < G covers a slice of the hidden
//      dimension for every token and expert (fp32 FMAs; products of bf16
//      values are exact in fp32)
//   -- barrier --
//   2. every block sums the partial scores in slice order, keeps the k best
//      of each token (rank of 64-bit order keys, ties to the lower expert
//      id), renormalises them, and forms the stable permutation of the N*k
//      assignments in its own LDS.  All blocks compute the same result, which
//      costs less than another barrier; block 0 stores the ids and weights.
//   3. gate+up: split-contraction tiles dealt round-robin over the blocks -> h
//   -- barrier --
//   4. down tiles, routing weight applied in the epilogue -> y
//   -- barrier --
//   5. combine: each token's k rows of y summed in slot order (fp32) -> out
// The tiles are those of the split-contraction decode kernel (tile index =
// the block index that kernel would use), so h and y equal its results.
//
// Barrier: each block stores a tag in its own flag word; block 0 waits for
// all of them and then stores the tag in one word that the others wait on.
// A tag carries an epoch that the workspace holds: every block reads it
// before the first barrier and block 0 advances it after that barrier, so no
// call has to clear anything (graph replays included) and a tag left by an
// earlier call never matches.  Every wait is bounded in time: a block whose
// wait runs out fills the output with NaN and leaves, and so do the blocks
// waiting on it, so a failure shows in the result instead of hanging.
#include "common.h"
#include "kernels.h"
#include "ffn_stream.h"

namespace moe {

// Barrier words (in the workspace): the epoch, the release word and one flag
// per block, the first two on lines of their own.
struct DecodeSync {
  uint64_t epoch;
  uint64_t pad0[15];
  uint64_t go;
  uint64_t pad1[15];
  uint64_t flags[kDecodeMaxBlocks];
};

namespace {

static_assert(kDecodeMaxExperts == kMaxGroups, "the tile list holds every expert");
constexpr int kDT = kDecodeTokens;
constexpr int kRouteSlice = 512;     // hidden rows per router slice, at most
constexpr int kDecodeThreads = 256;

template <bool F8>
struct DecodeLds {
  union {
    KsLds<F8> ks;
    struct {
      float xs[kDT][kRouteSlice];          // token rows of the slice (fp32)
      float red[4][kDT][kDecodeMaxExperts];  // per-wave sums
    } route;
    struct {
      float sc[kDT * kDecodeMaxExperts];   // scores [n][e]
      f32x4_t red[kDecodeThreads];
      uint64_t key[4][kDecodeMaxExperts];
      float sx[4][16];
    } topk;
  } u;
  int s_off[kMaxGroups + 1];
  int s_tp[kMaxGroups + 1];
  int p_off[kMaxGroups + 1];               // expert offsets of the permutation
  int ids[kDecodeAssign];
  float wts[kDecodeAssign];
  int rowtok[kDecodeAssign];               // token of sorted row p
  float rowwt[kDecodeAssign];              // routing weight of sorted row p
  int a2s[kDecodeAssign];                  // sorted row of assignment a
  int fail;
  uint64_t epoch;
};

__device__ __forceinline__ uint64_t poll_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Order key of (score, expert): larger keys win; equal scores order by the
// lower id (negative zero is first made positive zero).
__device__ __forceinline__ uint64_t order_key(float v, int e) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  const uint32_t m = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)m << 32) | (uint32_t)~(uint32_t)e;
}

// Grid barrier.  Returns false in every thread of the block if a wait ran
// out (then the block must leave without touching shared results again).
__device__ bool grid_sync(DecodeSync* sy, uint64_t tag, uint64_t limit, int* s_fail) {
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(&sy->flags[blockIdx.x], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (blockIdx.x == 0) {
    for (int b = tid; b < (int)gridDim.x; b += kDecodeThreads) {
      const uint64_t t0 = (uint64_t)wall_clock64();
      while (poll_word(&sy->flags[b]) != tag) {
        if ((uint64_t)wall_clock64() - t0 > limit) {
          *s_fail = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
    if (tid == 0 && *s_fail == 0) {
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
      __hip_atomic_store(&sy->go, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (tid == 0) {
    const uint64_t t0 = (uint64_t)wall_clock64();
    while (poll_word(&sy->go) != tag) {
      if ((uint64_t)wall_clock64() - t0 > limit) {
        *s_fail = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  if (tid == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  return *s_fail == 0;
}

__device__ __forceinline__ void fill_nan(const DecodeArgs& d) {
  const int n = d.N * d.M;
  for (int i = threadIdx.x; i < n; i += kDecodeThreads) d.out[i] = 0x7fc0;
}

template <bool F8>
__global__ __launch_bounds__(kDecodeThreads, 2) void decode_layer_kernel(DecodeArgs d) {
  __shared__ __align__(16) DecodeLds<F8> lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = d.N, M = d.M, E = d.E, k = d.k, H = d.H, A = N * k;
  if (tid == 0) {
    lds.fail = 0;
    lds.epoch = poll_word(&d.sync->epoch);
  }
  __syncthreads();
  const uint64_t base = (lds.epoch + 1) << 4;

  // ---- 1. router partial scores: part[g][n][e] over hidden rows of slice g
  if ((int)blockIdx.x < d.G) {
    const int g = blockIdx.x;
    const int m0 = g * d.MS, m1 = min(M, m0 + d.MS);
    const int L = m1 - m0;                    // <= kRouteSlice (host-checked)
    for (int i = tid; i < N * L; i += kDecodeThreads) {
      const int n = i / L, j = i - n * L;
      lds.u.route.xs[n][j] = bf16_to_f32(d.x[(size_t)n * M + m0 + j]);
    }
    __syncthreads();
    // thread: 16-byte piece c (experts 8c..8c+7) of hidden row r, r + RPS, ...
    const int LPR = E >> 3, RPS = kDecodeThreads / LPR;
    const int c = tid % LPR, r = tid / LPR;
    float acc[kDT][8];
#pragma unroll
    for (int n = 0; n < kDT; ++n)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[n][q] = 0.f;
#pragma unroll 4
    for (int j = r; j < L; j += RPS) {
      const uint4 wv = *reinterpret_cast<const uint4*>(d.w_router + (size_t)(m0 + j) * E + c * 8);
      const uint32_t wq[4] = {wv.x, wv.y, wv.z, wv.w};
      float w[8];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        w[2 * h] = __uint_as_float(wq[h] << 16);
        w[2 * h + 1] = __uint_as_float(wq[h] & 0xffff0000u);
      }
#pragma unroll
      for (int n = 0; n < kDT; ++n)
        if (n < N) {
          const float xv = lds.u.route.xs[n][j];
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[n][q] = __fmaf_rn(xv, w[q], acc[n][q]);
        }
    }
    // rows of a wave (lanes with equal c) summed by an xor butterfly (LPR <= 32)
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
      for (int n = 0; n < kDT; ++n)
        if (n < N)
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[n][q] += __shfl_xor(acc[n][q], off);
    __syncthreads();                          // xs reads done before red (same union) is written
    if (lane < LPR) {
#pragma unroll
      for (int n = 0; n < kDT; ++n)
        if (n < N)
#pragma unroll
          for (int q = 0; q < 8; ++q) lds.u.route.red[wave][n][c * 8 + q] = acc[n][q];
    }
    __syncthreads();
    for (int i = tid; i < N * E; i += kDecodeThreads) {
      const int n = i / E, e = i - n * E;
      const float s = lds.u.route.red[0][n][e] + lds.u.route.red[1][n][e] + lds.u.route.red[2][n][e] +
                      lds.u.route.red[3][n][e];
      d.part[((size_t)g * N + n) * E + e] = s;
    }
  }
  if (!grid_sync(d.sync, base | 1, d.limit, &lds.fail)) {
    fill_nan(d);
    return;
  }
  // every block has read the epoch before arriving here: advance it
  if (blockIdx.x == 0 && tid == 0)
    __hip_atomic_store(&d.sync->epoch, lds.epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- 2. scores, top-k, weights, permutation (the same in every block)
  {
    const int items = (N * E) >> 2;           // float4 items (n, 4 experts)
    const int Q = items >= kDecodeThreads ? 1 : kDecodeThreads / items;
    const f32x4_t* part4 = reinterpret_cast<const f32x4_t*>(d.part);
    f32x4_t* sc4 = reinterpret_cast<f32x4_t*>(lds.u.topk.sc);
    if (Q == 1) {
      for (int i = tid; i < items; i += kDecodeThreads) {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
        for (int g = 0; g < d.G; ++g) s += part4[(size_t)g * items + i];
        sc4[i] = s;
      }
    } else {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
      if (tid < items * Q) {
        const int i = tid % items, q = tid / items;
        for (int g = q; g < d.G; g += Q) s += part4[(size_t)g * items + i];
      }
      lds.u.topk.red[tid] = s;
      __syncthreads();
      for (int i = tid; i < items; i += kDecodeThreads) {
        f32x4_t t = lds.u.topk.red[i];
        for (int q = 1; q < Q; ++q) t += lds.u.topk.red[q * items + i];
        sc4[i] = t;
      }
    }
    __syncthreads();
    // wave w ranks tokens w, w + 4 (lane l holds experts l + 64 i)
    for (int n = wave; n < N; n += 4) {
      float v[4];
      uint64_t key[4];
      int rank[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        v[i] = 0.f;
        key[i] = 0;
        rank[i] = 0;
        if (e < E) {
          v[i] = lds.u.topk.sc[n * E + e] + (d.bias ? d.bias[e] : 0.f);
          key[i] = order_key(v[i], e);
          lds.u.topk.key[wave][e] = key[i];
        }
      }
      __builtin_amdgcn_wave_barrier();
      for (int j = 0; j < E; ++j) {
        const uint64_t q = lds.u.topk.key[wave][j];
#pragma unroll
        for (int i = 0; i < 4; ++i) rank[i] += q > key[i] ? 1 : 0;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < E && rank[i] < k) lds.u.topk.sx[wave][rank[i]] = v[i];
      __builtin_amdgcn_wave_barrier();
      const float vmax = lds.u.topk.sx[wave][0];
      float ex[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ex[i] = __expf(v[i] - vmax);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < E && rank[i] < k) lds.u.topk.sx[wave][rank[i]] = ex[i];
      __builtin_amdgcn_wave_barrier();
      float sum = 0.f;
      for (int r = 0; r < k; ++r) sum += lds.u.topk.sx[wave][r];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < E && rank[i] < k) {
          lds.ids[n * k + rank[i]] = lane + 64 * i;
          lds.wts[n * k + rank[i]] = ex[i] / sum;
        }
      __builtin_amdgcn_wave_barrier();      // sx / key rows are rewritten for the next token
    }
    __syncthreads();
    // stable sort of the assignments by expert: sorted row of a = #(lower
    // experts) + #(same expert, lower assignment index)
    if (tid < A) {
      const int e = lds.ids[tid];
      int pos = 0;
      for (int a = 0; a < A; ++a) {
        const int e2 = lds.ids[a];
        pos += (e2 < e || (e2 == e && a < tid)) ? 1 : 0;
      }
      lds.a2s[tid] = pos;
      lds.rowtok[pos] = tid / k;
      lds.rowwt[pos] = lds.wts[tid];
    }
    if (tid < E) {
      int cnt = 0;
      for (int a = 0; a < A; ++a) cnt += lds.ids[a] < tid ? 1 : 0;
      lds.p_off[tid] = cnt;
    }
    if (tid == 0) lds.p_off[E] = A;
    __syncthreads();
    if (blockIdx.x == 0 && tid < A) {
      d.ids[tid] = lds.ids[tid];
      d.wts[tid] = lds.wts[tid];
    }
  }

  // ---- 3. gate+up -> h
  {
    FfnArgs g{};
    g.a = d.x;
    g.a_rows = lds.rowtok;
    g.offsets = lds.p_off;
    g.w0 = d.w_gate;
    g.w1 = d.w_up;
    g.q0 = d.q_gate;
    g.q1 = d.q_up;
    g.s0 = d.s_gate;
    g.s1 = d.s_up;
    g.out = d.h;
    g.E = E;
    g.rows_total = A;
    g.K = M;
    g.ncols = H;
    const int total = build_tile_list<16>(g, H / kSCols, lds.s_off, lds.s_tp);
    for (int t = blockIdx.x; t < total; t += gridDim.x) ks_tile<true, F8>(g, lds.s_off, lds.s_tp, t, (unsigned)t, lds.u.ks);
  }
  if (!grid_sync(d.sync, base | 2, d.limit, &lds.fail)) {
    fill_nan(d);
    return;
  }

  // ---- 4. down -> y (weighted)
  {
    FfnArgs dn{};
    dn.a = d.h;
    dn.offsets = lds.p_off;
    dn.w0 = d.w_down;
    dn.q0 = d.q_down;
    dn.s0 = d.s_down;
    dn.row_scale = lds.rowwt;
    dn.out = d.y;
    dn.E = E;
    dn.rows_total = A;
    dn.K = H;
    dn.ncols = M;
    const int total = build_tile_list<16>(dn, M / (2 * kSCols), lds.s_off, lds.s_tp);
    for (int t = blockIdx.x; t < total; t += gridDim.x) ks_tile<false, F8>(dn, lds.s_off, lds.s_tp, t, (unsigned)t, lds.u.ks);
  }
  if (!grid_sync(d.sync, base | 3, d.limit, &lds.fail)) {
    fill_nan(d);
    return;
  }

  // ---- 5. combine: slot order, fp32, one rounding
  {
    const int chunks = M >> 3;
    for (int i = blockIdx.x * kDecodeThreads + tid; i < N * chunks; i += gridDim.x * kDecodeThreads) {
      const int n = i / chunks, c = i - n * chunks;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < k; ++j) {
        const uint4 v = *reinterpret_cast<const uint4*>(d.y + (size_t)lds.a2s[n * k + j] * M + c * 8);
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] += 1.f * __uint_as_float(q[h] << 16);
          acc[2 * h + 1] += 1.f * __uint_as_float(q[h] & 0xffff0000u);
        }
      }
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(d.out + (size_t)n * M + c * 8) = o;
    }
  }
}

// Router slices: the router phase reads M*E/(2048 G) 16-byte pieces per
// thread and the score sums G*N*E/1024 floats-of-four, which meet near
// G = sqrt(M / 2N); slices stay within kRouteSlice rows.
int decode_slices(int N, int M) {
  int g = 1;
  while ((long)2 * N * g * g < M) ++g;
  const int lo = ceil_div(M, kRouteSlice);
  if (g < lo) g = lo;
  if (g > M / 32) g = M / 32 > lo ? M / 32 : lo;
  return g;
}

struct DecodeGrid {
  int grid[2] = {0, 0};   // per F8
};
DecodeGrid g_decode_grid[64];

template <bool F8>
int decode_grid(int dev, int num_cu) {
  int& v = g_decode_grid[dev].grid[F8 ? 1 : 0];
  if (v == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(&decode_layer_kernel<F8>),
                                                     kDecodeThreads, 0) != hipSuccess || nb <= 0)
      return -1;
    long g = (long)(nb < 2 ? nb : 2) * num_cu;
    if (g > kDecodeMaxBlocks) g = kDecodeMaxBlocks;
    v = (int)g;
  }
  return v;
}

}  // namespace

bool decode_fusable(int N, int M, int E, int k, int H, bool f8) {
  if (N < 1 || N > kDecodeTokens || N * k > kDecodeAssign || k < 1 || k > 16) return false;
  if (E != 8 && E != 16 && E != 32 && E != 64 && E != 128 && E != 256) return false;
  const int q = f8 ? 256 : 128;
  return M % q == 0 && H % q == 0 && M >= q && H >= q;
}

size_t decode_workspace_bytes(int N, int M, int E) {
  const size_t part = (size_t)decode_slices(N, M) * N * E * sizeof(float);
  return ((part + 255) & ~size_t(255)) + sizeof(DecodeSync);
}

hipError_t launch_decode_layer(DecodeArgs a, void* ws, int num_cu, hipStream_t st) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const bool f8 = a.q_gate != nullptr;
  const int grid = f8 ? decode_grid<true>(dev, num_cu) : decode_grid<false>(dev, num_cu);
  if (grid <= 0) return hipErrorLaunchFailure;
  a.G = decode_slices(a.N, a.M);
  if (a.G > grid) a.G = grid;
  a.MS = ceil_div(a.M, a.G);
  if (a.MS > kRouteSlice) return hipErrorInvalidValue;   // slices above are only for very wide M
  const size_t part = (size_t)decode_slices(a.N, a.M) * a.N * a.E * sizeof(float);
  a.part = static_cast<float*>(ws);
  a.sync = reinterpret_cast<DecodeSync*>(static_cast<char*>(ws) + ((part + 255) & ~size_t(255)));
  void* args[] = {&a};
  const void* fn = f8 ? reinterpret_cast<const void*>(&decode_layer_kernel<true>)
                      : reinterpret_cast<const void*>(&decode_layer_kernel<false>);
  return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kDecodeThreads), args, 0, st);
}

}  // namespace moe
