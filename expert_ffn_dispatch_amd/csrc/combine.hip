// Combine / unpermutation: each token gathers its k expert rows through the
// inverse mapping, weights them and sums them in slot order, then adds the
// shared experts' output.
//
// Page on MoE latency (wink.run), section "router 之后还有一串动作": results are
// restored to token order through the inverse mapping, multiplied by the
// routing weight and summed.  Shared experts (FinDEP review, 二、核心思想) see
// every token and add unweighted.  Sum in fp32, slots j = 0..k-1 then the
// shared term, one bf16 rounding at the store.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ void add8(float (&acc)[8], uint4 v, float w) {
  const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += w * __uint_as_float(q[i] << 16);
    acc[2 * i + 1] += w * __uint_as_float(q[i] & 0xffff0000u);
  }
}

// One block per token row; each thread owns 16-byte chunks of the row, U of
// them per trip.  The token's k positions and weights are read once; all k
// expert rows of the U chunks are loaded before the first is summed (KM >= k
// slots, unrolled).  y is read exactly once, so its loads carry the
// non-temporal hint.  Measured (flushed, one layer call): Qwen3-235B-shaped
// combine (65536 rows of 8 KB) 119 -> 102 us with two chunks per trip and
// the hint, DeepSeek-V2-shaped 67 -> 58 us; two chunks alone gave 2-3 us.
template <int KM, int U>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs p) {
  const int n = blockIdx.x;
  const int chunks = p.M >> 3;
  const int k = p.k;
  int pos[KM];
  float w[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    pos[j] = 0;
    w[j] = 0.f;
    if (j < k) {
      pos[j] = p.a2s[n * k + j];
      w[j] = p.weights ? p.weights[n * k + j] : 1.f;
    }
  }
  for (int c0 = threadIdx.x; c0 < chunks; c0 += 256 * U) {
    u32x4_t v[U][KM];
    uint4 sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 256 * u;
      sv[u] = make_uint4(0, 0, 0, 0);
      if (c >= chunks) continue;
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j < k)
          v[u][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.y + (size_t)pos[j] * p.M + c * 8));
      if (p.shared) sv[u] = *reinterpret_cast<const uint4*>(p.shared + (size_t)n * p.M + c * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 256 * u;
      if (c >= chunks) continue;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j < k) add8(acc, make_uint4(v[u][j].x, v[u][j].y, v[u][j].z, v[u][j].w), w[j]);
      if (p.shared) add8(acc, sv[u], 1.f);
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(p.out + (size_t)n * p.M + c * 8) = o;
    }
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  const dim3 g(a.N), b(256);
  if (a.k <= 1) hipLaunchKernelGGL((combine_kernel<1, 2>), g, b, 0, st, a);
  else if (a.k <= 2) hipLaunchKernelGGL((combine_kernel<2, 2>), g, b, 0, st, a);
  else if (a.k <= 4) hipLaunchKernelGGL((combine_kernel<4, 2>), g, b, 0, st, a);
  else if (a.k <= 8) hipLaunchKernelGGL((combine_kernel<8, 2>), g, b, 0, st, a);
  else hipLaunchKernelGGL((combine_kernel<16, 1>), g, b, 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
