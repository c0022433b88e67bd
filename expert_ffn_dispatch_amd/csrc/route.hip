// Router: scores (bf16 MFMA, fp32 accumulate), softmax top-k and renormalised
// routing weights for every token.
//
// Page on MoE latency (wink.run), section "dense 和 MoE 的差别": the router reads
// each token's hidden state, scores every available expert, keeps the top k
// and emits k routing weights.  Softmax -> top-k -> renormalise is the gating
// rule; the top k of the softmax are the top k of the logits (softmax is
// monotone), so selection runs on the logits and only the k winners are
// exponentiated: w_j = exp(l_j - l_max) / sum_sel exp(l_i - l_max), which is
// p_j / sum_sel p.  Ties go to the lower expert id; slot 0 holds the largest.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kTok = 64;              // tokens per block: 4 waves x 16 rows
constexpr int kBK = 64;               // contraction slab
constexpr int kLd = kBK + 8;          // LDS row pitch (bf16) with 16 B pad

// ncb = number of 16-expert column blocks held by each wave (E padded).
template <int NCB, bool VEC>
__global__ __launch_bounds__(256) void route_kernel(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ wr,
                                                    const float* __restrict__ bias, int N, int M,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ wts) {
  constexpr int EP = NCB * 16;
  extern __shared__ __align__(16) char smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);   // [kTok][kLd]
  uint16_t* wt = xs + kTok * kLd;                      // [EP][kLd]  (router transposed)
  float* lg = reinterpret_cast<float*>(smem);          // [kTok][EP] after the K loop

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tok0 = blockIdx.x * kTok;

  // padded expert rows stay zero
  for (int i = tid; i < (EP - E) * kLd; i += 256) wt[E * kLd + i] = 0;

  f32x4_t acc[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < M; k0 += kBK) {
    // x slab: 64 rows x 8 chunks of 16 B
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, ch = c & 7;
      const int n = tok0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < N) v = *reinterpret_cast<const uint4*>(x + (size_t)n * M + k0 + ch * 8);
      *reinterpret_cast<uint4*>(xs + r * kLd + ch * 8) = v;
    }
    // router slab [kBK][E] -> wt[e][kk]
    if (VEC) {
      const int e8n = E >> 3;
      for (int u = tid; u < kBK * e8n; u += 256) {
        const int kk = u / e8n, e8 = u - kk * e8n;
        const uint4 v = *reinterpret_cast<const uint4*>(wr + (size_t)(k0 + kk) * E + e8 * 8);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          wt[(e8 * 8 + 2 * q) * kLd + kk] = static_cast<uint16_t>(w4[q] & 0xffffu);
          wt[(e8 * 8 + 2 * q + 1) * kLd + kk] = static_cast<uint16_t>(w4[q] >> 16);
        }
      }
    } else {
      for (int u = tid; u < kBK * E; u += 256) {
        const int kk = u / E, e = u - kk * E;
        wt[e * kLd + kk] = wr[(size_t)(k0 + kk) * E + e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kc = ks * 32 + (lane >> 4) * 8;
      const uint4 a = *reinterpret_cast<const uint4*>(xs + (wave * 16 + (lane & 15)) * kLd + kc);
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const uint4 b = *reinterpret_cast<const uint4*>(wt + (c * 16 + (lane & 15)) * kLd + kc);
        acc[c] = mfma16(a, b, acc[c]);
      }
    }
    __syncthreads();
  }

  // logits (+ bias) to LDS: lane holds rows 4*(lane>>4)+r, expert c*16+(lane&15)
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const int e = c * 16 + (lane & 15);
    const float b = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) lg[(wave * 16 + (lane >> 4) * 4 + r) * EP + e] = acc[c][r] + b;
  }
  __syncthreads();

  constexpr int PER = (EP + 63) / 64;   // experts per lane
  for (int t = 0; t < 16; ++t) {
    const int row = wave * 16 + t;
    const int n = tok0 + row;
    if (n >= N) break;
    float v[PER];
    bool taken[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      v[i] = (e < E) ? lg[row * EP + e] : 0.f;
      taken[i] = !(e < E);
    }
    int my_e = 0;
    float my_v = 0.f;
    for (int j = 0; j < k; ++j) {
      float bv = 0.f;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        if (!taken[i] && (be == 0x7fffffff || v[i] > bv)) { bv = v[i]; be = e; }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        const bool better = (oe != 0x7fffffff) &&
                            (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
        if (better) { bv = ov; be = oe; }
      }
      if (lane == j) { my_e = be; my_v = bv; }
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (lane + 64 * i == be) taken[i] = true;
    }
    const float vmax = __shfl(my_v, 0);
    float ex = (lane < k) ? __expf(my_v - vmax) : 0.f;
    float s = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (lane < k) {
      ids[(size_t)n * k + lane] = my_e;
      wts[(size_t)n * k + lane] = ex / s;
    }
  }
}

template <int NCB, bool VEC>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
  constexpr int EP = NCB * 16;
  const size_t lds_k = (size_t)(kTok + EP) * kLd * 2;
  const size_t lds_l = (size_t)kTok * EP * 4;
  const size_t lds = lds_k > lds_l ? lds_k : lds_l;
  const int grid = ceil_div(a.N, kTok);
  hipLaunchKernelGGL((route_kernel<NCB, VEC>), dim3(grid), dim3(256), lds, st, a.x, a.w_router,
                     a.bias, a.N, a.M, a.E, a.k, a.ids, a.weights);
  return hipGetLastError();
}

template <bool VEC>
hipError_t launch_route_v(const RouteArgs& a, hipStream_t st) {
  const int ncb = ceil_div(a.E, 16);
  if (ncb <= 1) return launch_route_t<1, VEC>(a, st);
  if (ncb <= 2) return launch_route_t<2, VEC>(a, st);
  if (ncb <= 4) return launch_route_t<4, VEC>(a, st);
  if (ncb <= 8) return launch_route_t<8, VEC>(a, st);
  if (ncb <= 12) return launch_route_t<12, VEC>(a, st);
  return launch_route_t<16, VEC>(a, st);
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  return (a.E % 8 == 0) ? launch_route_v<true>(a, st) : launch_route_v<false>(a, st);
}

}  // namespace moe
