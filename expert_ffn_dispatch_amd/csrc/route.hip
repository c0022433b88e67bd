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
// batches take two launches below 2048 tokens where E is a multiple of 8,
// else three:
//   logits    - one block per (16-64 tokens, up to 80 experts, k slice),
//               its four waves splitting the slice: partial scores per slice;
//               the contraction is split into KS slices so that even a
//               decode batch spreads over many waves.  Below 2048 tokens
//               the router operand reads W_r as stored and turns each
//               32-wide step around in LDS (router_logits_wr_kernel); larger
//               batches and E % 8 != 0 read W_rT [EP][M] (E padded to 16)
//               written by a transpose launch, so that both MFMA operands
//               hold 8 contraction elements per lane
//   topk      - one wave per token: sums the KS partials in slice order
//               (deterministic), adds the bias, takes the k best by k
//               wave-wide maxima of order keys (ties to the lower id) and
//               renormalises them.
// Batches of 8192 tokens and more take the transpose and one fused launch
// (router_fused_kernel, below).
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

// The same partial scores with the router fragments taken from W_r as
// stored ([M][E], experts fastest), so that no transpose is launched (E a
// multiple of 8).  For each 32-wide step a wave loads the 32 x 16 NCBW block
// of W_r it needs as 16-byte pieces (eight experts of one row), writes them
// to a wave-private LDS tile, and reads back each lane's eight consecutive
// contraction elements of its expert as 16-bit reads.  The next step's
// pieces and token fragments load while the current step is multiplied.
// Partial tiles of the four waves are added in wave order, as above.
template <int NCBW, int RW>
__global__ __launch_bounds__(256) void router_logits_wr_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ wr, int N, int M, int E,
                                                               int EP, int steps_per_slice, float* __restrict__ part) {
  constexpr int NV = RW * NCBW * 4;             // accumulator values per lane
  constexpr int WC = NCBW * 16;                 // experts of the block
  constexpr int PR = WC / 8;                    // 16-byte pieces per W_r row
  constexpr int TS = WC + 8;                    // LDS tile pitch (bf16), rows 16-byte aligned
  static_assert(32 * PR == 64 * NCBW, "NCBW pieces per lane per step");
  union Lds {
    float red[4][NV][64];
    uint16_t tile[4][32 * TS];
  };
  __shared__ __align__(16) Lds lds;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * 16 * RW;
  const int ks = blockIdx.y;
  const int eb0 = blockIdx.z * NCBW;
  const int b0 = ks * steps_per_slice;
  const int b1 = min(M / 32, b0 + steps_per_slice);
  const int s0 = b0 + ((b1 - b0) * wave) / 4, s1 = b0 + ((b1 - b0) * (wave + 1)) / 4;
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* xa[RW];
#pragma unroll
  for (int t = 0; t < RW; ++t) xa[t] = x + (size_t)min(tok0 + 16 * t + r, N - 1) * M + g * 8;
  // piece i of this lane: row q / PR of the step, experts 8 (q % PR) .. +7, q = 64 i + lane
  const uint16_t* wp[NCBW];
  int wdst[NCBW];
  bool wok[NCBW];
#pragma unroll
  for (int i = 0; i < NCBW; ++i) {
    const int q = 64 * i + lane, row = q / PR, pc = q - row * PR;
    const int e = eb0 * 16 + 8 * pc;
    wok[i] = e < E;
    wp[i] = wr + (size_t)row * E + (wok[i] ? e : 0);
    wdst[i] = row * TS + 8 * pc;
  }
  uint16_t* tile = lds.tile[wave];

  f32x4_t acc[RW][NCBW];
#pragma unroll
  for (int t = 0; t < RW; ++t)
#pragma unroll
    for (int c = 0; c < NCBW; ++c) acc[t][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t pa[RW], pw[NCBW], qa[RW], qw[NCBW], bf[NCBW];
#define MOE_WLOAD(A_, W_, S_)                                                                       \
  {                                                                                                 \
    _Pragma("unroll") for (int t = 0; t < RW; ++t)                                                  \
        A_[t] = *reinterpret_cast<const u32x4_t*>(xa[t] + (S_) * 32);                               \
    _Pragma("unroll") for (int i = 0; i < NCBW; ++i)                                                \
        W_[i] = wok[i] ? *reinterpret_cast<const u32x4_t*>(wp[i] + (size_t)(S_) * 32 * E)           \
                       : u32x4_t{0u, 0u, 0u, 0u};                                                   \
  }
  // the step's W_r block into the tile, then each lane's fragments out of it
  // (a wave's LDS operations complete in order; the wave barriers keep the
  // compiler from moving reads above writes or the next writes above reads)
#define MOE_WTURN(W_)                                                                               \
  {                                                                                                 \
    _Pragma("unroll") for (int i = 0; i < NCBW; ++i)                                                \
        *reinterpret_cast<u32x4_t*>(tile + wdst[i]) = W_[i];                                        \
    __builtin_amdgcn_wave_barrier();                                                                \
    _Pragma("unroll") for (int c = 0; c < NCBW; ++c) {                                              \
      const uint16_t* col = tile + (8 * g) * TS + 16 * c + r;                                       \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                 \
          bf[c][j] = (uint32_t)col[(2 * j) * TS] | ((uint32_t)col[(2 * j + 1) * TS] << 16);         \
    }                                                                                               \
    __builtin_amdgcn_wave_barrier();                                                                \
  }
#define MOE_WMMA(A_)                                                                                \
  _Pragma("unroll") for (int t = 0; t < RW; ++t)                                                    \
      _Pragma("unroll") for (int c = 0; c < NCBW; ++c) acc[t][c] = mfma16(A_[t], bf[c], acc[t][c]);
  if (s0 < s1) {
    MOE_WLOAD(pa, pw, s0)
    int st = s0;
    for (; st + 1 < s1; st += 2) {
      MOE_WLOAD(qa, qw, st + 1)
      MOE_WTURN(pw)
      MOE_WMMA(pa)
      MOE_WLOAD(pa, pw, min(st + 2, s1 - 1))   // the last step re-reads itself
      MOE_WTURN(qw)
      MOE_WMMA(qa)
    }
    if (st < s1) {
      MOE_WTURN(pw)
      MOE_WMMA(pa)
    }
  }
#undef MOE_WLOAD
#undef MOE_WTURN
#undef MOE_WMMA
  __syncthreads();                               // the tiles and the partial sums share the LDS
#pragma unroll
  for (int t = 0; t < RW; ++t)
#pragma unroll
    for (int c = 0; c < NCBW; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) lds.red[wave][(t * NCBW + c) * 4 + q][lane] = acc[t][c][q];
  __syncthreads();
  float* out = part + (size_t)ks * N * EP;
  for (int i = threadIdx.x; i < NV * 64; i += 256) {
    const int v = i >> 6, l = i & 63;
    const int q = v & 3, c = (v >> 2) % NCBW, t = (v >> 2) / NCBW;
    const int n = tok0 + 16 * t + 4 * (l >> 4) + q;
    if (n >= N) continue;
    const float sum = lds.red[0][v][l] + lds.red[1][v][l] + lds.red[2][v][l] + lds.red[3][v][l];
    out[(size_t)n * EP + (eb0 + c) * 16 + (l & 15)] = sum;
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

// One lane's 64-bit value from another lane of its row of 16 (DPP pattern CTRL).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// The largest of the wave's 64 values, in every lane: within each row of 16
// by DPP (swap within pairs, then pairs within quads, then the half-row and
// row mirrors), then across rows by exchanges with lanes 16 and 32 away.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0xB1>(v));      // quad_perm [1,0,3,2]
  v = max_u64(v, dpp_u64<0x4E>(v));      // quad_perm [2,3,0,1]
  v = max_u64(v, dpp_u64<0x141>(v));     // row_half_mirror
  v = max_u64(v, dpp_u64<0x140>(v));     // row_mirror
#pragma unroll
  for (int d = 16; d <= 32; d *= 2) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, d);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), d);
    v = max_u64(v, ((uint64_t)hi << 32) | lo);
  }
  return v;
}

// The score an order key was made from (topk_key without the id; -0 comes
// back as +0, which changes no difference of scores below).
__device__ __forceinline__ float key_score(uint64_t key) {
  const uint32_t m = (uint32_t)(key >> 32);
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m);
}

// Ranks NT tokens' scores side by side, one wave for all of them (lane l
// holds experts l + 64 i of token t in v[t]) and writes each token's k
// slots: ids in descending score order (ties to the lower id) and the
// weights exp(l_r - l_0) over their sum in slot order.  The order keys are
// unique (their low word is the complemented expert id), so k rounds of a
// wave-wide maximum give the slots in turn: round r's maximum is slot r's
// winner, which is then removed, and its expert and score are read back from
// the key.  Lane r keeps slot r.  Token t is stored only where ok[t]; the
// interleaved tokens overlap each other's reduction chains.  No LDS; about
// k * (PER + 30) VALU operations per token, where counting every expert's
// rank takes E * PER 64-bit compares.  Called by every lane of one wave.
template <int PER, int NT>
__device__ __forceinline__ void rank_tokens(const float (&v)[NT][PER], const bool (&ok)[NT], int lane, int E,
                                                int k, int32_t* const (&ids_n)[NT], float* const (&wts_n)[NT]) {
  uint64_t key[NT][PER];
  float vmax[NT], sum[NT], my_ex[NT];
  int my_e[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      key[t][i] = e < E ? topk_key(v[t][i], e) : 0;   // 0 is below every expert's key
    }
    vmax[t] = 0.f;
    sum[t] = 0.f;
    my_ex[t] = 0.f;
    my_e[t] = 0;
  }
  for (int r = 0; r < k; ++r) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint64_t m = key[t][0];
#pragma unroll
      for (int i = 1; i < PER; ++i) m = max_u64(m, key[t][i]);
      m = wave_max_u64(m);
#pragma unroll
      for (int i = 0; i < PER; ++i) key[t][i] = key[t][i] == m ? 0 : key[t][i];
      const float s = key_score(m);
      if (r == 0) vmax[t] = s;
      const float ex = __expf(s - vmax[t]);
      sum[t] += ex;
      if (lane == r) {
        my_e[t] = (int)~(uint32_t)m;
        my_ex[t] = ex;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (ok[t] && lane < k) {
      ids_n[t][lane] = my_e[t];
      wts_n[t][lane] = my_ex[t] / sum[t];
    }
}

template <int PER>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ part, const float* __restrict__ bias,
                                                          int N, int E, int EP, int KS, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = blockIdx.x * 4 + w;
  if (n >= N) return;                    // whole waves; no block barrier below
  float v[PER];
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
  }
  const float(&vt)[1][PER] = reinterpret_cast<const float(&)[1][PER]>(v);
  int32_t* const idp[1] = {ids + (size_t)n * k};
  float* const wtp[1] = {wts + (size_t)n * k};
  rank_tokens<PER, 1>(vt, {true}, lane, E, k, idp, wtp);
}

// At most four tokens (one block): top-k, then the dispatch and stable
// permutation of the N*k <= 64 assignments in the same block, so the
// decode path skips the permutation launch.  Each wave ranks one token as
// router_topk_kernel does, its slots into LDS; the block then stores the ids and
// weights, counts the assignments per expert, scans the counts (one wave)
// and places assignment a at offsets[e] plus the number of earlier
// assignments of its expert (the order the permutation launches give).
template <int PER>
__global__ __launch_bounds__(256) void router_topk_tiny_kernel(const float* __restrict__ part,
                                                               const float* __restrict__ bias, int N, int E,
                                                               int EP, int KS, int k, int32_t* __restrict__ ids,
                                                               float* __restrict__ wts, PermuteArgs pa) {
  __shared__ int s_ids[4 * 16];
  __shared__ float s_wts[4 * 16];
  __shared__ int cnt[256];
  __shared__ int off[256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (w < N) {
    float v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      float s = 0.f;
      if (e < E) {
#pragma unroll 8
        for (int ks = 0; ks < KS; ++ks) s += part[((size_t)ks * N + w) * EP + e];
        if (bias) s += bias[e];
      }
      v[i] = s;
    }
    const float(&vt)[1][PER] = reinterpret_cast<const float(&)[1][PER]>(v);
    int32_t* const idp[1] = {s_ids + w * k};
    float* const wtp[1] = {s_wts + w * k};
    rank_tokens<PER, 1>(vt, {true}, lane, E, k, idp, wtp);
  }
  if (tid < pa.n_zero) pa.zero[tid] = 0;
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  const int A = N * k;
  int e = 0;
  if (tid < A) {
    e = s_ids[tid];
    ids[tid] = e;
    wts[tid] = s_wts[tid];
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (w == 0) {
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = lane * 4 + i;
      c[i] = ee < E ? cnt[ee] : 0;
      sum += c[i];
    }
    int inc = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(inc, d);
      if (lane >= d) inc += o;
    }
    int b = inc - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = lane * 4 + i;
      if (ee < E) {
        pa.counts[ee] = c[i];
        pa.offsets[ee] = b;
        off[ee] = b;
      }
      b += c[i];
    }
    if (lane == 63) pa.offsets[E] = inc;
  }
  __syncthreads();
  if (tid < A) {
    int r = 0;
    for (int a2 = 0; a2 < tid; ++a2) r += s_ids[a2] == e ? 1 : 0;
    const int pos = off[e] + r;
    pa.s2a[pos] = tid;
    pa.a2s[tid] = pos;
    if (pa.row_token) pa.row_token[pos] = tid / k;
    if (pa.row_weight) pa.row_weight[pos] = s_wts[tid];
  }
}

// Large batches (fused_route): scores and top-k in one launch.  A block takes
// 32 tokens and every expert (E padded to 64 * NEBW rows of the transposed
// router) over the whole hidden dimension.  Token rows and router rows are
// loaded straight into a ring of kFusedStages LDS stages of 64 contraction
// elements, kFusedStages - 1 stages ahead (16-byte chunks XOR-swizzled by row
// on the source side, so the 16-row fragment reads are free of bank
// conflicts); each of the four waves multiplies every fourth 16-expert block
// against both 16-token blocks (16x16x32 MFMAs).  The scores then pass
// through LDS to rank_tokens, four tokens at a time per wave: no partial scores
// leave the block and no second launch follows.  Against the split path
// only the fp32 summation order of the scores differs.
// Measured (route stage, flushed medians): Qwen3-235B-shaped router (8192
// tokens, 128 experts) 73 -> 57 us against transpose + split scores + top-k;
// DeepSeek-V2-shaped (4096 tokens, 160 experts) 63 -> 84 us, where the 128
// blocks leave half the GPU idle, so smaller batches keep the split path.
constexpr int kFusedStages = 4;
constexpr int kFusedMinTokens = 8192;

__device__ __forceinline__ int rsw(int row) { return ((row >> 1) ^ ((row & 1) << 2)) & 7; }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t route_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// 16 bytes per lane straight into LDS (lane l writes lds + 16 l); bytes past
// the resource read as zeros.  A plain function: kernel templates call no
// target builtin directly.
__device__ __forceinline__ void route_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 0);
}
#define MOE_RWAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | 0x0F70)

template <int NEBW>
__global__ __launch_bounds__(256, 1) void router_fused_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ wt,
                                                              const float* __restrict__ bias, int N, int M, int E,
                                                              int EP, int k, int32_t* __restrict__ ids,
                                                              float* __restrict__ wts) {
  constexpr int TR = 32;                       // tokens per block
  constexpr int ER = 64 * NEBW;                // router rows per stage (>= EP; the rest read zeros)
  constexpr int R = TR + ER;                   // rows per stage: tokens, then experts
  constexpr int ST = R * 64;                   // bf16 elements of a stage
  constexpr int LPW = R / 32;                  // direct loads per wave per stage, 8 rows each
  static_assert(kFusedStages == 4, "the ring below names four buffers");
  __shared__ __align__(16) uint16_t s0[ST];
  __shared__ __align__(16) uint16_t s1[ST];
  __shared__ __align__(16) uint16_t s2[ST];
  __shared__ __align__(16) uint16_t s3[ST];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * TR;
  const int nvalid = min(TR, N - n0);
  const int KT = M / 64;
  const __amdgpu_buffer_rsrc_t xr = route_rsrc(x + (size_t)n0 * M, (uint32_t)nvalid * (uint32_t)M * 2u);
  const __amdgpu_buffer_rsrc_t wr = route_rsrc(wt, (uint32_t)EP * (uint32_t)M * 2u);
  // load i of this wave fills rows 8 (wave + 4 i) .. + 7, slot lane & 7; load
  // 0 holds token rows, the others router rows
  uint32_t voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = 8 * (wave + 4 * i) + (lane >> 3);
    const int ch = (lane & 7) ^ rsw(r);
    voff[i] = (uint32_t)(i == 0 ? r : r - TR) * (uint32_t)(2 * M) + (uint32_t)(ch * 16);
  }
#define MOE_RLOAD(BUF, KT_)                                                                        \
  _Pragma("unroll") for (int i = 0; i < LPW; ++i)                                                  \
      route_dma16(i == 0 ? xr : wr, voff[i], (uint32_t)((KT_) * 128), (BUF) + 8 * (wave + 4 * i) * 64);

  // fragment offsets: token block tb, expert block j, 32-wide half h
  const int fr = lane & 15, fg = lane >> 4;
  int aoff[2][2], boff[NEBW][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int r = 16 * tb + fr;
      aoff[tb][h] = r * 64 + (((4 * h + fg) ^ rsw(r)) << 3);
    }
#pragma unroll
    for (int j = 0; j < NEBW; ++j) {
      const int r = TR + 16 * (wave + 4 * j) + fr;
      boff[j][h] = r * 64 + (((4 * h + fg) ^ rsw(r)) << 3);
    }
  }
  f32x4_t acc[2][NEBW];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int j = 0; j < NEBW; ++j) acc[tb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  MOE_RLOAD(s0, 0)
  MOE_RLOAD(s1, min(1, KT - 1))
  MOE_RLOAD(s2, min(2, KT - 1))
  // stage KT_: wait for this wave's loads of it, publish them, load stage
  // KT_ + 3 into the buffer every wave finished reading before the barrier,
  // multiply stage KT_ (past the last stage the loads repeat it)
#define MOE_RSTEP(BUF, NBUF, KT_)                                                                  \
  {                                                                                                \
    MOE_RWAIT_VM(2 * LPW);                                                                         \
    __builtin_amdgcn_s_barrier();                                                                  \
    MOE_RLOAD(NBUF, min((KT_) + 3, KT - 1))                                                        \
    __builtin_amdgcn_sched_barrier(0);                                                             \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                                \
      u32x4_t af[2], bf[NEBW];                                                                     \
      _Pragma("unroll") for (int tb = 0; tb < 2; ++tb)                                             \
          af[tb] = *reinterpret_cast<const u32x4_t*>((BUF) + aoff[tb][h]);                         \
      _Pragma("unroll") for (int j = 0; j < NEBW; ++j)                                             \
          bf[j] = *reinterpret_cast<const u32x4_t*>((BUF) + boff[j][h]);                           \
      _Pragma("unroll") for (int tb = 0; tb < 2; ++tb)                                             \
          _Pragma("unroll") for (int j = 0; j < NEBW; ++j) acc[tb][j] = mfma16(af[tb], bf[j], acc[tb][j]); \
    }                                                                                              \
    __builtin_amdgcn_s_waitcnt(0xC07F);                                                            \
  }
  int kt = 0;
  for (; kt + 3 < KT; kt += 4) {
    MOE_RSTEP(s0, s3, kt)
    MOE_RSTEP(s1, s0, kt + 1)
    MOE_RSTEP(s2, s1, kt + 2)
    MOE_RSTEP(s3, s2, kt + 3)
  }
  if (kt < KT) MOE_RSTEP(s0, s3, kt)
  if (kt + 1 < KT) MOE_RSTEP(s1, s0, kt + 1)
  if (kt + 2 < KT) MOE_RSTEP(s2, s1, kt + 2)
#undef MOE_RSTEP
#undef MOE_RLOAD
  MOE_RWAIT_VM(0);
  __syncthreads();

  // scores [32][ER] in s0; lane l of the accumulators holds tokens
  // 16 tb + 4 (l >> 4) + q of expert 16 (wave + 4 j) + (l & 15)
  float* lg = reinterpret_cast<float*>(s0);
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int j = 0; j < NEBW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) lg[(16 * tb + 4 * fg + q) * ER + 16 * (wave + 4 * j) + fr] = acc[tb][j][q];
  __syncthreads();
  // RT tokens per wave at a time: t, t + 4, ...
  constexpr int RT = 4;
  for (int t = wave; t < nvalid; t += 4 * RT) {
    bool ok[RT];
    float v[RT][NEBW];
    int32_t* idp[RT];
    float* wtp[RT];
#pragma unroll
    for (int h = 0; h < RT; ++h) {
      ok[h] = t + 4 * h < nvalid;
      const size_t n = (size_t)(n0 + (ok[h] ? t + 4 * h : t));
      idp[h] = ids + n * k;
      wtp[h] = wts + n * k;
#pragma unroll
      for (int i = 0; i < NEBW; ++i) {
        const int e = lane + 64 * i;
        v[h][i] = 0.f;
        if (e < E && ok[h]) v[h][i] = lg[(t + 4 * h) * ER + e] + (bias ? bias[e] : 0.f);
      }
    }
    rank_tokens<NEBW, RT>(v, ok, lane, E, k, idp, wtp);
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
  // a small batch over more waves.  Below 8192 tokens at most two, so that
  // the scores can read W_r as stored: DeepSeek-V2-shaped route (4096 tokens)
  // 59.0 -> 55.3 us against four with the transpose launch.
  p.RW = N >= 8192 ? 4 : (N >= 512 ? 2 : 1);
  const int blocks = ceil_div(N, 16 * p.RW) * p.EG;
  const int total_steps = M / 32;
  // about 1024 blocks; from 2048 tokens about 512, as fewer slices write
  // and re-read fewer partial scores (DeepSeek-V2-shaped route at 4096
  // tokens: 56.3 us with four slices, 51.4 with two, 64.6 with eight)
  int ks = ceil_div(N >= 2048 ? 512 : 1024, blocks);
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
  const dim3 grid(ceil_div(a.N, 16 * RW), pl.KS, pl.EG);
  if constexpr (RW <= 2) {   // W_r as stored: batches below 8192 tokens only
    if (wt == nullptr) {
      hipLaunchKernelGGL((router_logits_wr_kernel<NCBW, RW>), grid, dim3(256), 0, st, a.x, a.w_router, a.N, a.M,
                         a.E, pl.EP, pl.steps, part);
      return;
    }
  }
  hipLaunchKernelGGL((router_logits_kernel<NCBW, RW>), grid, dim3(256), 0, st, a.x, wt, a.N, a.M, pl.EP, pl.steps,
                     part);
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

// Batches of at least kFusedMinTokens tokens over at most 256 experts take
// the fused scores-and-top-k launch after the transpose.
bool fused_route(int N, int E) {
  return !small_route(N, E) && !rows_route(N, E) && N >= kFusedMinTokens && E <= 256;
}

namespace {

// Top-k over KS partial score slices of row stride EP; with a.perm (at most
// four tokens), the permutation in the same launch.
template <int PER>
hipError_t launch_topk_per(const RouteArgs& a, const float* part, int EP, int KS, hipStream_t st) {
  if (a.perm != nullptr)
    hipLaunchKernelGGL(router_topk_tiny_kernel<PER>, dim3(1), dim3(256), 0, st, part, a.bias, a.N, a.E, EP, KS, a.k,
                       a.ids, a.weights, *a.perm);
  else
    hipLaunchKernelGGL(router_topk_kernel<PER>, dim3(ceil_div(a.N, 4)), dim3(256), 0, st, part, a.bias, a.N, a.E,
                       EP, KS, a.k, a.ids, a.weights);
  return hipGetLastError();
}
hipError_t launch_topk(const RouteArgs& a, const float* part, int EP, int KS, hipStream_t st) {
  const int per = ceil_div(EP, 64);
  if (per <= 1) return launch_topk_per<1>(a, part, EP, KS, st);
  if (per <= 2) return launch_topk_per<2>(a, part, EP, KS, st);
  if (per <= 3) return launch_topk_per<3>(a, part, EP, KS, st);
  return launch_topk_per<4>(a, part, EP, KS, st);
}

}  // namespace

bool route_permutes(int N) { return N >= 1 && N <= 4; }

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
  if (a.perm != nullptr && (!route_permutes(a.N) || a.k > 16 || a.E > 256)) return hipErrorInvalidValue;
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
    if (hipError_t e = hipGetLastError()) return e;
    return launch_topk(a, part, a.E, KS, st);
  }
  if (small_route(a.N, a.E)) {
    int slice, KS;
    small_route_plan(a.N, a.M, slice, KS);
    float* part = static_cast<float*>(ws);
    const size_t lds = ((size_t)kSRT * slice + 256 * kSRT) * sizeof(float);
    hipLaunchKernelGGL(router_scores_small_kernel, dim3(ceil_div(a.N, kSRT), KS), dim3(256), lds, st, a.x,
                       a.w_router, a.N, a.M, a.E, slice, part);
    if (hipError_t e = hipGetLastError()) return e;
    return launch_topk(a, part, a.E, KS, st);
  }
  const RoutePlan pl = plan(a.N, a.M, a.E);
  uint16_t* wt = static_cast<uint16_t*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + (((size_t)pl.EP * a.M * 2 + 255) & ~size_t(255)));
  // Below 8192 tokens the split scores read W_r as stored where its rows
  // hold whole 16-byte pieces of experts (E % 8 == 0): Qwen3-30B-shaped route
  // at 8-512 tokens 17.6-19.0 -> 15.7-16.6 us, the transpose launch gone;
  // DeepSeek-V2-shaped at 4096 tokens, two token blocks per wave, 59.0 ->
  // 55.3 us (with four per wave, each block turning the same router rows
  // around, it had been 64 -> 73 us).  The fused launch and other E take
  // the transpose.
  const bool fused = fused_route(a.N, a.E);
  if (!fused && a.E % 8 == 0 && pl.RW <= 2) {
    wt = nullptr;
  } else {
    hipLaunchKernelGGL(router_transpose_kernel, dim3(a.M / 64, ceil_div(pl.EP, 64)), dim3(256), 0, st, a.w_router,
                       a.M, a.E, pl.EP, wt);
  }
  if (fused) {
    const dim3 g(ceil_div(a.N, 32));
    const int nebw = ceil_div(pl.EP, 64);
    if (nebw <= 2)
      hipLaunchKernelGGL(router_fused_kernel<2>, g, dim3(256), 0, st, a.x, wt, a.bias, a.N, a.M, a.E, pl.EP, a.k,
                         a.ids, a.weights);
    else if (nebw == 3)
      hipLaunchKernelGGL(router_fused_kernel<3>, g, dim3(256), 0, st, a.x, wt, a.bias, a.N, a.M, a.E, pl.EP, a.k,
                         a.ids, a.weights);
    else
      hipLaunchKernelGGL(router_fused_kernel<4>, g, dim3(256), 0, st, a.x, wt, a.bias, a.N, a.M, a.E, pl.EP, a.k,
                         a.ids, a.weights);
    return hipGetLastError();
  }
  switch (pl.NCBW) {
    case 1: launch_logits<1>(a, pl, wt, part, st); break;
    case 2: launch_logits<2>(a, pl, wt, part, st); break;
    case 5: launch_logits<5>(a, pl, wt, part, st); break;
    default: launch_logits<4>(a, pl, wt, part, st); break;
  }
  if (hipError_t e = hipGetLastError()) return e;
  return launch_topk(a, part, pl.EP, pl.KS, st);
}

}  // namespace moe
