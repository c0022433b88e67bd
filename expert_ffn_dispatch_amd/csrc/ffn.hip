// Grouped SwiGLU expert GEMMs on bf16 MFMA (gfx950, 16x16x32, fp32 accumulate).
//
// FinDEP review, section 核心公式: one expert costs three GEMMs of m_e x M x H
// (gate, up, down).  Page on MoE latency (wink.run), section
// "router 之后还有一串动作": every expert's matrix runs in one grouped launch,
// an expert with no assignments creates no work and no padded row is
// computed into the result.
//
// Phase 1 (gate+up): a tile holds BM rows of one expert and BN columns of h;
//   its B operand is BN rows of W_gate and the same BN rows of W_up, so the
//   epilogue forms h = silu(g) * u in registers and stores bf16.
// Phase 2 (down): y = (h W_down^T) * row_scale, stored bf16.
//
// Scheduling: a persistent grid walks the tile list (expert, row tile, column
// tile) built in LDS from the device-side expert offsets, so the host never
// needs the counts.  Row tiles vary fastest so that blocks running at the
// same time share one column tile of weights.  Operands are staged through
// LDS (register double buffering, 16-byte chunks XOR-swizzled by row to keep
// the MFMA fragment reads free of bank conflicts).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBK = 64;     // contraction slab (8 chunks of 16 B per row)

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

template <int BM, int BN, int WM, int WN, bool GATEUP>
__global__ __launch_bounds__(256) void ffn_kernel(FfnArgs p) {
  constexpr int NB = GATEUP ? 2 * BN : BN;   // weight rows per tile
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile (output)
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int NACC = GATEUP ? 2 : 1;
  constexpr int A_LD = BM * 8 / 256;
  constexpr int B_LD = NB * 8 / 256;
  static_assert(BM % 32 == 0 && NB % 32 == 0 && TM % 16 == 0 && TN % 16 == 0, "tile shape");
  static_assert(WM * WN == 4, "four waves");

  __shared__ __align__(16) uint16_t lds[2][(BM + NB) * kBK];
  __shared__ int s_off[257];
  __shared__ int s_tp[257];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int E = p.E, K = p.K, ncols = p.ncols;
  const int NT = ncols / BN;

  // ---- tile list: per-expert tile counts, inclusive prefix in LDS ----
  if (p.fixed_rows > 0) {
    if (tid == 0) { s_off[0] = 0; s_off[1] = p.fixed_rows; }
  } else {
    for (int e = tid; e <= E; e += 256) s_off[e] = p.offsets[e];
  }
  __syncthreads();
  {
    int tv = 0;
    if (tid < E) tv = ceil_div(s_off[tid + 1] - s_off[tid], BM) * NT;
    s_tp[tid + 1] = tv;
    if (tid == 0) s_tp[0] = 0;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int t = (tid >= off) ? s_tp[tid + 1 - off] : 0;
      __syncthreads();
      s_tp[tid + 1] += t;
      __syncthreads();
    }
  }
  const int total = s_tp[E];

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tp[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int cnt = s_off[e + 1] - s_off[e];
    const int RT = ceil_div(cnt, BM);
    const int local = tile - s_tp[e];
    const int ct = local / RT, rt = local - ct * RT;
    const int row0 = s_off[e] + rt * BM;
    const int nrows = min(BM, cnt - rt * BM);
    const int col0 = ct * BN;

    const uint16_t* a_src[A_LD];
    int a_dst[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int c = tid + 256 * i, r = c >> 3, ch = c & 7;
      const int rr = (r < nrows) ? r : 0;
      const int grow = p.a_rows ? p.a_rows[row0 + rr] : (row0 + rr);
      a_src[i] = p.a + (size_t)grow * K + ch * 8;
      a_dst[i] = swz(r, ch);
    }
    const uint16_t* b_src[B_LD];
    int b_dst[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int c = tid + 256 * i, r = c >> 3, ch = c & 7;
      const uint16_t* wrow;
      if (GATEUP) {
        wrow = (r < BN) ? p.w0 + ((size_t)e * ncols + col0 + r) * K
                        : p.w1 + ((size_t)e * ncols + col0 + r - BN) * K;
      } else {
        wrow = p.w0 + ((size_t)e * ncols + col0 + r) * K;
      }
      b_src[i] = wrow + ch * 8;
      b_dst[i] = swz(BM + r, ch);
    }

    f32x4_t acc[NACC][FM][FN];
#pragma unroll
    for (int g = 0; g < NACC; ++g)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[g][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 ra[A_LD], rb[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i]);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i]);
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *reinterpret_cast<uint4*>(&lds[0][a_dst[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) *reinterpret_cast<uint4*>(&lds[0][b_dst[i]]) = rb[i];
    __syncthreads();

    const int KT = K / kBK;
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < KT;
      if (more) {
        const int ko = (kt + 1) * kBK;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + ko);
#pragma unroll
        for (int i = 0; i < B_LD; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + ko);
      }
      const uint16_t* L = lds[cur];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int ch = ks * 4 + (lane >> 4);
        uint4 af[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * TM + i * 16 + (lane & 15);
          af[i] = *reinterpret_cast<const uint4*>(&L[swz(r, ch)]);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int rb0 = BM + wn * TN + j * 16 + (lane & 15);
          const uint4 b0 = *reinterpret_cast<const uint4*>(&L[swz(rb0, ch)]);
#pragma unroll
          for (int i = 0; i < FM; ++i) acc[0][i][j] = mfma16(af[i], b0, acc[0][i][j]);
          if (GATEUP) {
            const uint4 b1 = *reinterpret_cast<const uint4*>(&L[swz(rb0 + BN, ch)]);
#pragma unroll
            for (int i = 0; i < FM; ++i) acc[NACC - 1][i][j] = mfma16(af[i], b1, acc[NACC - 1][i][j]);
          }
        }
      }
      if (more) {
        uint16_t* Ln = lds[cur ^ 1];
#pragma unroll
        for (int i = 0; i < A_LD; ++i) *reinterpret_cast<uint4*>(&Ln[a_dst[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i) *reinterpret_cast<uint4*>(&Ln[b_dst[i]]) = rb[i];
      }
      __syncthreads();
    }

    // ---- epilogue ----
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * TM + i * 16 + (lane >> 4) * 4 + r;
        if (row >= nrows) continue;
        const size_t orow = (size_t)(row0 + row) * ncols;
        const float s = (!GATEUP && p.row_scale) ? p.row_scale[row0 + row] : 1.f;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = col0 + wn * TN + j * 16 + (lane & 15);
          float v;
          if (GATEUP) {
            const float g = acc[0][i][j][r], u = acc[NACC - 1][i][j][r];
            v = g / (1.f + __expf(-g)) * u;
          } else {
            v = acc[0][i][j][r] * s;
          }
          p.out[orow + col] = f32_to_bf16(v);
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, bool GATEUP>
hipError_t launch_t(const FfnArgs& a, int num_cu, hipStream_t st) {
  const int NT = a.ncols / BN;
  const long ub_rows = a.rows_total / BM + (a.E < a.rows_total ? a.E : a.rows_total);
  long ub = ub_rows * NT;
  long grid = (long)num_cu * 2;
  if (ub < grid) grid = ub;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((ffn_kernel<BM, BN, WM, WN, GATEUP>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_gateup(const FfnArgs& a, int num_cu, hipStream_t st) {
  if (a.rows_total == 0) return hipSuccess;
  return launch_t<64, 64, 2, 2, true>(a, num_cu, st);
}

hipError_t launch_ffn_down(const FfnArgs& a, int num_cu, hipStream_t st) {
  if (a.rows_total == 0) return hipSuccess;
  if (a.ncols % 128 == 0) return launch_t<64, 128, 2, 2, false>(a, num_cu, st);
  return launch_t<64, 64, 2, 2, false>(a, num_cu, st);
}

}  // namespace moe
