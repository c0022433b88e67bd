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
//
// Batches of up to 160 tokens over at most 32 experts take two launches:
// scores with fp32 FMAs straight from W_r (router_scores_small_kernel), then
// top-k; so do batches of one or two tokens over 64, 128 or 256 experts
// (router_scores_rows_kernel, 16-byte pieces of W_r rows per thread).  Other
// batches take three:
//   transpose - W_r [M][E] -> W_rT [EP][M] (E padded to 16), so that both MFMA
//               operands read 16 contiguous bytes of the contraction per lane
//   logits    - one block per (16-64 tokens, up to 80 experts, k slice),
//               its four waves splitting the slice: partial scores per slice;
//               the contraction is split into KS slices so that even a
//               decode batch spreads over many waves
//   topk      - one wave per token: sums the KS partials in slice order
//               (deterministic), adds the bias, ranks every score against
//               the others (ties to the lower id), renormalises the k best.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void router_transpose_kernel(const uint16_t* __restrict__ wr, int M, int E,
                                                               int EP, uint16_t* __restrict__ wt) {
  __shared__ uint16_t t[64][66];
  const int k0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  // all sixteen loads of a thread are issued before the first LDS store
  uint16_t v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = tid + 256 * j;
    const int e = e0 + (i & 63);
    v[j] = (e < E) ? wr[(size_t)(k0 + (i >> 6)) * E + e] : (uint16_t)0;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = tid + 256 * j;
    t[i >> 6][i & 63] = v[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = tid + 256 * j;
    const int ee = i >> 6, kk = i & 63;
    const int e = e0 + ee;
    if (e < EP) wt[(size_t)e * M + k0 + kk] = t[kk][ee];
  }
}

// part[ks][n][e] = sum over the slice's k of x[n,k] * W_r[k,e].  A block
// covers RW x 16 tokens (blockIdx.x) and NCBW x 16 experts (expert group
// blockIdx.z) for one k slice (blockIdx.y); its four waves take consecutive
// quarters of the slice, and their partial tiles are added in wave order
// through LDS, so the slice's partials leave the block once.  Each router
// fragment a wave loads serves RW token blocks and each token fragment NCBW
// expert blocks; the next 32-wide step is loaded while the current one is
// multiplied (two register sets).
template <int NCBW, int RW>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wt, int N, int M, int EP,
                                                            int steps_per_slice, float* __restrict__ part) {
  constexpr int NV = RW * NCBW * 4;             // accumulator values per lane
  __shared__ float red[4][NV][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * 16 * RW;
  const int ks = blockIdx.y;
  const int eb0 = blockIdx.z * NCBW;             // first 16-expert block
  const int b0 = ks * steps_per_slice;
  const int b1 = min(M / 32, b0 + steps_per_slice);
  const int s0 = b0 + ((b1 - b0) * wave) / 4, s1 = b0 + ((b1 - b0) * (wave + 1)) / 4;
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* xa[RW];
#pragma unroll
  for (int t = 0; t < RW; ++t) xa[t] = x + (size_t)min(tok0 + 16 * t + r, N - 1) * M + g * 8;
  const uint16_t* wb = wt + (size_t)(eb0 * 16 + r) * M + g * 8;

  f32x4_t acc[RW][NCBW];
#pragma unroll
  for (int t = 0; t < RW; ++t)
#pragma unroll
    for (int c = 0; c < NCBW; ++c) acc[t][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t pa[RW], pb[NCBW], qa[RW], qb[NCBW];
#define MOE_RLOAD(A_, B_, S_)                                                                       \
  {                                                                                                 \
    _Pragma("unroll") for (int t = 0; t < RW; ++t)                                                  \
        A_[t] = *reinterpret_cast<const u32x4_t*>(xa[t] + (S_) * 32);                               \
    _Pragma("unroll") for (int c = 0; c < NCBW; ++c)                                                \
        B_[c] = *reinterpret_cast<const u32x4_t*>(wb + (size_t)c * 16 * M + (S_) * 32);             \
  }
#define MOE_RMMA(A_, B_)                                                                            \
  _Pragma("unroll") for (int t = 0; t < RW; ++t)                                                    \
      _Pragma("unroll") for (int c = 0; c < NCBW; ++c) acc[t][c] = mfma16(A_[t], B_[c], acc[t][c]);
  if (s0 < s1) {
    MOE_RLOAD(pa, pb, s0)
    int st = s0;
    for (; st + 1 < s1; st += 2) {
      MOE_RLOAD(qa, qb, st + 1)
      MOE_RMMA(pa, pb)
      MOE_RLOAD(pa, pb, min(st + 2, s1 - 1))   // the last step re-reads itself
      MOE_RMMA(qa, qb)
    }
    if (st < s1) { MOE_RMMA(pa, pb) }
  }
#undef MOE_RLOAD
#undef MOE_RMMA
#pragma unroll
  for (int t = 0; t < RW; ++t)
#pragma unroll
    for (int c = 0; c < NCBW; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) red[wave][(t * NCBW + c) * 4 + q][lane] = acc[t][c][q];
  __syncthreads();
  // value v of lane l: token tok0 + 16t + 4(l >> 4) + q, expert (eb0 + c)*16 + (l & 15)
  float* out = part + (size_t)ks * N * EP;
  for (int i = threadIdx.x; i < NV * 64; i += 256) {
    const int v = i >> 6, l = i & 63;
    const int q = v & 3, c = (v >> 2) % NCBW, t = (v >> 2) / NCBW;
    const int n = tok0 + 16 * t + 4 * (l >> 4) + q;
    if (n >= N) continue;
    const float s = red[0][v][l] + red[1][v][l] + red[2][v][l] + red[3][v][l];
    out[(size_t)n * EP + (eb0 + c) * 16 + (l & 15)] = s;
  }
}

// Order key of (score, expert): larger keys win.  The score's bits are made
// monotone as an unsigned integer (negative zero first becomes positive zero,
// so that equal scores stay equal) and the expert id, inverted, breaks ties
// in favour of the lower id.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  const uint32_t m = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)m << 32) | (uint32_t)~(uint32_t)e;
}

// One wave per token.  Each lane holds PER scores (experts lane + 64 i); the
// token's order keys are also written to this wave's LDS row, and every lane
// counts the keys above each of its own: that count is the score's rank, and
// ranks 0..k-1 are the k slots.  No cross-lane reduction chains: the
// broadcast LDS reads and 64-bit compares of all lanes run side by side.
// The weights are exp(l - l_max) of the k winners over their sum (in slot
// order).
template <int PER>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ part, const float* __restrict__ bias,
                                                          int N, int E, int EP, int KS, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ wts) {
  __shared__ __align__(16) uint64_t sk[4][64 * PER];
  __shared__ float sx[4][16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = blockIdx.x * 4 + w;
  if (n >= N) return;                    // whole waves; no block barrier below
  float v[PER];
  uint64_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    float s = 0.f;
    if (e < E) {
#pragma unroll 8
      for (int ks = 0; ks < KS; ++ks) s += part[((size_t)ks * N + n) * EP + e];
      if (bias) s += bias[e];
    }
    v[i] = s;
    key[i] = topk_key(s, e);
    sk[w][e] = e < E ? key[i] : 0;       // padding loses to every expert
  }
  // LDS operations of a wave complete in order; the barrier only keeps the
  // compiler from moving the reads above the writes
  __builtin_amdgcn_wave_barrier();
  int rank[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) rank[i] = 0;
  // E rounded up to pairs: a padding key (0) never counts
  for (int j = 0; j < E; j += 4) {
    const uint4 a = *reinterpret_cast<const uint4*>(&sk[w][j]);
    const uint4 b = *reinterpret_cast<const uint4*>(&sk[w][j + 2]);
    const uint64_t q[4] = {((uint64_t)a.y << 32) | a.x, ((uint64_t)a.w << 32) | a.z,
                           ((uint64_t)b.y << 32) | b.x, ((uint64_t)b.w << 32) | b.z};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < PER; ++i) rank[i] += q[u] > key[i] ? 1 : 0;
  }
  // slot r of the winners: the largest score first
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (lane + 64 * i < E && rank[i] < k) sx[w][rank[i]] = v[i];
  __builtin_amdgcn_wave_barrier();
  const float vmax = sx[w][0];
  float ex[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) ex[i] = __expf(v[i] - vmax);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (lane + 64 * i < E && rank[i] < k) sx[w][rank[i]] = ex[i];
  __builtin_amdgcn_wave_barrier();
  float sum = 0.f;
  for (int r = 0; r < k; ++r) sum += sx[w][r];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    if (e < E && rank[i] < k) {
      ids[(size_t)n * k + rank[i]] = e;
      wts[(size_t)n * k + rank[i]] = ex[i] / sum;
    }
  }
}

// Small batches (small_route): scores without the transpose.
// Block (t, ks) covers tokens [16t, 16t+16) and contraction slice ks; thread
// i accumulates expert i % E over the (i / E)-th of P sub-slices for the
// block's 16 tokens with fp32 FMAs (products of bf16 values are exact in
// fp32), reading each router weight once and the token rows from LDS.  The
// P partials are added in sub-slice order and written as part[ks][n][e]
// (row stride E) for router_topk_kernel.
constexpr int kSmallRouteTokens = 160;
constexpr int kSmallRouteExperts = 32;
constexpr int kSRT = 16;          // tokens per block
constexpr int kSmallRouteLoads = 8;   // 16-byte token-row pieces per thread: slice <= 1024

__global__ __launch_bounds__(256) void router_scores_small_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wr, int N, int M,
                                                                  int E, int slice, float* __restrict__ part) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * kSRT, ks = blockIdx.y;
  const int k0 = ks * slice, k1 = min(M, k0 + slice);
  const int L = k1 - k0;
  float* xs = smem;                       // [kSRT][slice] token rows of the slice (fp32)
  float* red = smem + kSRT * slice;       // [256][kSRT] partials
  {
    // 16-byte pieces of the token rows (slice and L are multiples of 32);
    // all of a thread's loads are issued before the first store
    const int pr = L >> 3, np = kSRT * pr;
    uint4 v[kSmallRouteLoads];
#pragma unroll
    for (int j = 0; j < kSmallRouteLoads; ++j) {
      const int c = tid + 256 * j;
      v[j] = make_uint4(0, 0, 0, 0);
      if (c < np) {
        const int t = c / pr, kc = c - t * pr;
        const int n = min(n0 + t, N - 1);
        v[j] = *reinterpret_cast<const uint4*>(x + (size_t)n * M + k0 + kc * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < kSmallRouteLoads; ++j) {
      const int c = tid + 256 * j;
      if (c < np) {
        const int t = c / pr, kc = c - t * pr;
        float* d = xs + t * slice + kc * 8;
        const uint32_t q[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          d[2 * h] = __uint_as_float(q[h] << 16);
          d[2 * h + 1] = __uint_as_float(q[h] & 0xffff0000u);
        }
      }
    }
  }
  __syncthreads();
  const int P = 256 / E;
  const int e = tid % E, sub = tid / E;
  float acc[kSRT];
#pragma unroll
  for (int t = 0; t < kSRT; ++t) acc[t] = 0.f;
  if (sub < P) {
    const int sl = ceil_div(L, P);
    const int a0 = sub * sl, a1 = min(L, a0 + sl);
    // eight weights in flight before the first is used
    int kk = a0;
    for (; kk + 8 <= a1; kk += 8) {
      float w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = bf16_to_f32(wr[(size_t)(k0 + kk + u) * E + e]);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int t = 0; t < kSRT; ++t) acc[t] = __fmaf_rn(xs[t * slice + kk + u], w[u], acc[t]);
    }
    for (; kk < a1; ++kk) {
      const float w = bf16_to_f32(wr[(size_t)(k0 + kk) * E + e]);
#pragma unroll
      for (int t = 0; t < kSRT; ++t) acc[t] = __fmaf_rn(xs[t * slice + kk], w, acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < kSRT; ++t) red[tid * kSRT + t] = acc[t];
  __syncthreads();
  for (int i = tid; i < kSRT * E; i += 256) {
    const int t = i / E, ee = i - t * E;
    const int n = n0 + t;
    if (n >= N) continue;
    float s = 0.f;
    for (int q = 0; q < P; ++q) s += red[(q * E + ee) * kSRT + t];
    part[((size_t)ks * N + n) * E + ee] = s;
  }
}

// Decode batches over 64, 128 or 256 experts: scores with fp32 FMAs
// straight from W_r, so the transpose the MFMA path needs is not launched.
// Block (g, t) covers hidden rows [g*slice, (g+1)*slice) and tokens
// [T t, T t + T) (T = 1, 2, 4 or 8 by batch size).  Thread (c, r) reads the
// 16-byte piece c (experts 8c..8c+7) of rows r, r + RPS, ... (RPS = 2048 / E
// rows side by side), all of its rows in flight at once, and accumulates them
// for the block's tokens, whose rows of the slice wait in LDS as fp32 laid
// out [row][token] (absent tokens are zeros, so the loop has no branches).
// The rows of a wave are summed by an xor butterfly over the lanes that hold
// the same piece, the four waves through LDS in wave order, and the block
// writes part[g][n][e] (row stride E) for router_topk_kernel.
constexpr int kRowRouteTokens = 2;
constexpr int kRowSliceMax = 1024; // hidden rows per block, at most
constexpr int kRowLoads = 16;      // W_r pieces a thread has in flight

template <int T>
__global__ __launch_bounds__(256) void router_scores_rows_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wr, int N, int M,
                                                                 int E, int slice, float* __restrict__ part) {
  __shared__ __align__(16) float xs[kRowSliceMax][T];
  __shared__ float red[4][T][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x, n0 = blockIdx.y * T;
  const int nt = min(T, N - n0);
  const int m0 = g * slice, L = min(M, m0 + slice) - m0;
  for (int i = tid; i < T * L; i += 256) {
    const int t = i / L, j = i - t * L;
    xs[j][t] = t < nt ? bf16_to_f32(x[(size_t)(n0 + t) * M + m0 + j]) : 0.f;
  }
  __syncthreads();
  const int LPR = E >> 3, RPS = 256 / LPR;   // LPR divides 64
  const int c = tid % LPR, r = tid / LPR;
  float acc[T][8];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[t][q] = 0.f;
  for (int j0 = r; j0 < L; j0 += kRowLoads * RPS) {
    u32x4_t wv[kRowLoads];
#pragma unroll
    for (int u = 0; u < kRowLoads; ++u) {
      const int j = j0 + u * RPS;
      wv[u] = u32x4_t{0u, 0u, 0u, 0u};
      if (j < L) wv[u] = *reinterpret_cast<const u32x4_t*>(wr + (size_t)(m0 + j) * E + c * 8);
    }
#pragma unroll
    for (int u = 0; u < kRowLoads; ++u) {
      const int j = min(j0 + u * RPS, L - 1);   // rows past the slice carry zero weights
      float w[8];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        w[2 * h] = __uint_as_float(wv[u][h] << 16);
        w[2 * h + 1] = __uint_as_float(wv[u][h] & 0xffff0000u);
      }
      float xv[T];
#pragma unroll
      for (int t = 0; t < T; ++t) xv[t] = xs[j][t];
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[t][q] = __fmaf_rn(xv[t], w[q], acc[t][q]);
    }
  }
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[t][q] += __shfl_xor(acc[t][q], off);
  if (lane < LPR) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int q = 0; q < 8; ++q) red[wave][t][c * 8 + q] = acc[t][q];
  }
  __syncthreads();
  for (int i = tid; i < nt * E; i += 256) {
    const int t = i / E, e = i - t * E;
    part[((size_t)g * N + n0 + t) * E + e] = red[0][t][e] + red[1][t][e] + red[2][t][e] + red[3][t][e];
  }
}

// hidden-dimension slices of the rows path: about 8 of at least 256 rows
void rows_route_plan(int M, int& slice, int& KS) {
  int ks = M / 256;
  if (ks > 8) ks = 8;
  if (ks < 1) ks = 1;
  slice = ceil_div(M, ks);
  if (slice > kRowSliceMax) slice = kRowSliceMax;
  KS = ceil_div(M, slice);
}

// slices (multiples of 32 wide) so that the launch has about 256 blocks
void small_route_plan(int N, int M, int& slice, int& KS) {
  const int tb = ceil_div(N, kSRT);
  int ks = ceil_div(256, tb);
  if (ks > M / 32) ks = M / 32;
  if (ks < 1) ks = 1;
  slice = ceil_div(ceil_div(M, ks), 32) * 32;
  KS = ceil_div(M, slice);
}

struct RoutePlan {
  int NCB, EP, NCBW, EG, RW, KS, steps;
};

RoutePlan plan(int N, int M, int E) {
  RoutePlan p;
  const int ncb = ceil_div(E, 16);
  p.NCB = ncb <= 1 ? 1 : ncb <= 2 ? 2 : ncb <= 4 ? 4 : ncb <= 8 ? 8 : ncb <= 10 ? 10 : ncb <= 12 ? 12 : 16;
  p.EP = p.NCB * 16;
  // expert blocks per wave: at most five, so that two register sets of
  // operands and the accumulators fit; the rest go to more blocks
  p.NCBW = p.NCB <= 4 ? p.NCB : p.NCB == 10 ? 5 : 4;
  p.EG = p.NCB / p.NCBW;
  // tokens per wave: more rows reuse each router fragment, fewer rows spread
  // a small batch over more waves
  p.RW = N >= 2048 ? 4 : (N >= 512 ? 2 : 1);
  const int blocks = ceil_div(N, 16 * p.RW) * p.EG;
  const int total_steps = M / 32;
  int ks = ceil_div(1024, blocks);
  const int max_ks = ceil_div(total_steps, 16);     // slices of at least 512 k (128 per wave)
  if (ks > max_ks) ks = max_ks;
  // partial scores are written and re-read once: keep them under 32 MB
  // (16 MB cost the DeepSeek-V2-shaped router 2 us of its 64)
  while (ks > 1 && (size_t)ks * N * p.EP * 4 > ((size_t)32 << 20)) --ks;
  if (ks < 1) ks = 1;
  p.steps = ceil_div(total_steps, ks);
  p.KS = ceil_div(total_steps, p.steps);
  return p;
}

template <int NCBW, int RW>
void launch_logits_rw(const RouteArgs& a, const RoutePlan& pl, const uint16_t* wt, float* part, hipStream_t st) {
  hipLaunchKernelGGL((router_logits_kernel<NCBW, RW>), dim3(ceil_div(a.N, 16 * RW), pl.KS, pl.EG), dim3(256), 0,
                     st, a.x, wt, a.N, a.M, pl.EP, pl.steps, part);
}

template <int NCBW>
void launch_logits(const RouteArgs& a, const RoutePlan& pl, const uint16_t* wt, float* part, hipStream_t st) {
  if (pl.RW == 4) launch_logits_rw<NCBW, 4>(a, pl, wt, part, st);
  else if (pl.RW == 2) launch_logits_rw<NCBW, 2>(a, pl, wt, part, st);
  else launch_logits_rw<NCBW, 1>(a, pl, wt, part, st);
}

}  // namespace

// The FMA path wins for few tokens and few experts (measured: 12.5 against
// 15.9 us for 156 tokens x 8 experts); with 128 experts a 1-token batch is
// faster on the MFMA path, whose top-k sums fewer partial slices.
bool small_route(int N, int E) { return N <= kSmallRouteTokens && E <= kSmallRouteExperts; }

// The smallest decode batches over 64, 128 or 256 experts.  Measured on the
// Qwen3-30B-shaped router (128 experts, hidden 2048): at one token the scores
// kernel takes 5.0 us and the layer 44.0 us against 48.5 us with the
// transpose and MFMA launches; at 8 and 32 tokens (12.9 us, eight tokens per
// block) the layer is 2 us slower than with them.
bool rows_route(int N, int E) {
  return !small_route(N, E) && N <= kRowRouteTokens && (E == 64 || E == 128 || E == 256);
}

size_t route_workspace_bytes(int N, int M, int E) {
  if (rows_route(N, E)) {
    int slice, KS;
    rows_route_plan(M, slice, KS);
    return ((size_t)KS * N * E * 4 + 255) & ~size_t(255);
  }
  if (small_route(N, E)) {
    int slice, KS;
    small_route_plan(N, M, slice, KS);
    return ((size_t)KS * N * E * 4 + 255) & ~size_t(255);
  }
  const RoutePlan pl = plan(N, M, E);
  const size_t wt = ((size_t)pl.EP * M * 2 + 255) & ~size_t(255);
  const size_t part = ((size_t)pl.KS * N * pl.EP * 4 + 255) & ~size_t(255);
  return wt + part;
}

hipError_t launch_route(const RouteArgs& a, void* ws, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  if (rows_route(a.N, a.E)) {
    int slice, KS;
    rows_route_plan(a.M, slice, KS);
    float* part = static_cast<float*>(ws);
    const int T = a.N >= 8 ? 8 : a.N >= 4 ? 4 : a.N >= 2 ? 2 : 1;
    const dim3 gr(KS, ceil_div(a.N, T));
    if (T == 8)
      hipLaunchKernelGGL(router_scores_rows_kernel<8>, gr, dim3(256), 0, st, a.x, a.w_router, a.N, a.M, a.E, slice, part);
    else if (T == 4)
      hipLaunchKernelGGL(router_scores_rows_kernel<4>, gr, dim3(256), 0, st, a.x, a.w_router, a.N, a.M, a.E, slice, part);
    else if (T == 2)
      hipLaunchKernelGGL(router_scores_rows_kernel<2>, gr, dim3(256), 0, st, a.x, a.w_router, a.N, a.M, a.E, slice, part);
    else
      hipLaunchKernelGGL(router_scores_rows_kernel<1>, gr, dim3(256), 0, st, a.x, a.w_router, a.N, a.M, a.E, slice, part);
    const dim3 g(ceil_div(a.N, 4));
    if (a.E <= 64)
      hipLaunchKernelGGL(router_topk_kernel<1>, g, dim3(256), 0, st, part, a.bias, a.N, a.E, a.E, KS, a.k, a.ids, a.weights);
    else if (a.E <= 128)
      hipLaunchKernelGGL(router_topk_kernel<2>, g, dim3(256), 0, st, part, a.bias, a.N, a.E, a.E, KS, a.k, a.ids, a.weights);
    else
      hipLaunchKernelGGL(router_topk_kernel<4>, g, dim3(256), 0, st, part, a.bias, a.N, a.E, a.E, KS, a.k, a.ids, a.weights);
    return hipGetLastError();
  }
  if (small_route(a.N, a.E)) {
    int slice, KS;
    small_route_plan(a.N, a.M, slice, KS);
    float* part = static_cast<float*>(ws);
    const size_t lds = ((size_t)kSRT * slice + 256 * kSRT) * sizeof(float);
    hipLaunchKernelGGL(router_scores_small_kernel, dim3(ceil_div(a.N, kSRT), KS), dim3(256), lds, st, a.x,
                       a.w_router, a.N, a.M, a.E, slice, part);
    const int per = ceil_div(a.E, 64);
    const dim3 g(ceil_div(a.N, 4));
    if (per <= 1)
      hipLaunchKernelGGL(router_topk_kernel<1>, g, dim3(256), 0, st, part, a.bias, a.N, a.E, a.E, KS, a.k, a.ids, a.weights);
    else if (per <= 2)
      hipLaunchKernelGGL(router_topk_kernel<2>, g, dim3(256), 0, st, part, a.bias, a.N, a.E, a.E, KS, a.k, a.ids, a.weights);
    else
      hipLaunchKernelGGL(router_topk_kernel<4>, g, dim3(256), 0, st, part, a.bias, a.N, a.E, a.E, KS, a.k, a.ids, a.weights);
    return hipGetLastError();
  }
  const RoutePlan pl = plan(a.N, a.M, a.E);
  uint16_t* wt = static_cast<uint16_t*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + (((size_t)pl.EP * a.M * 2 + 255) & ~size_t(255)));
  hipLaunchKernelGGL(router_transpose_kernel, dim3(a.M / 64, ceil_div(pl.EP, 64)), dim3(256), 0, st, a.w_router,
                     a.M, a.E, pl.EP, wt);
  switch (pl.NCBW) {
    case 1: launch_logits<1>(a, pl, wt, part, st); break;
    case 2: launch_logits<2>(a, pl, wt, part, st); break;
    case 5: launch_logits<5>(a, pl, wt, part, st); break;
    default: launch_logits<4>(a, pl, wt, part, st); break;
  }
  const int per = ceil_div(pl.EP, 64);
  const dim3 g(ceil_div(a.N, 4));
  if (per <= 1)
    hipLaunchKernelGGL(router_topk_kernel<1>, g, dim3(256), 0, st, part, a.bias, a.N, a.E, pl.EP, pl.KS, a.k, a.ids, a.weights);
  else if (per <= 2)
    hipLaunchKernelGGL(router_topk_kernel<2>, g, dim3(256), 0, st, part, a.bias, a.N, a.E, pl.EP, pl.KS, a.k, a.ids, a.weights);
  else if (per <= 3)
    hipLaunchKernelGGL(router_topk_kernel<3>, g, dim3(256), 0, st, part, a.bias, a.N, a.E, pl.EP, pl.KS, a.k, a.ids, a.weights);
  else
    hipLaunchKernelGGL(router_topk_kernel<4>, g, dim3(256), 0, st, part, a.bias, a.N, a.E, pl.EP, pl.KS, a.k, a.ids, a.weights);
  return hipGetLastError();
}

}  // namespace moe
