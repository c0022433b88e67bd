// Grouped SwiGLU expert GEMMs on bf16 MFMA (gfx950, 16x16x32, fp32 accumulate).
//
// FinDEP review, section 核心公式: one expert costs three GEMMs of m_e x M x H
// (gate, up, down), and the per-expert batch m_e decides whether they are
// bound by compute or by weight reads (MegaScale-Infer summary, 核心问题).
// Page on MoE latency (wink.run), section "router 之后还有一串动作": all
// experts run in one grouped launch, an expert without assignments creates no
// work, and no padded row is computed into the result.
//
// Phase 1 (gate+up): h = silu(x W_g^T) * (x W_u^T), the gate and up rows of
//   the same h columns live in one tile so the epilogue forms h in registers.
// Phase 2 (down): y = (h W_d^T) * row_scale.
//
// Two kernels, chosen on the host from the mean rows per expert (N*k/E):
//  * stream (decode-sized groups, <= 64 mean rows): every wave owns 16 output
//    columns and streams its weight rows from HBM straight into MFMA
//    registers, one 128-wide k chunk ahead; the group's token rows (at most
//    64 per pass) are staged in LDS and shared by the four waves.  Weights
//    are read once per pass; the kernel is bound by HBM bandwidth.
//  * tile (large groups): 256-row x 256-column tiles, both operands staged
//    through LDS (register double buffering, 16-byte chunks XOR-swizzled by
//    row so MFMA fragment reads are free of bank conflicts), four waves of
//    128 x 128.  Tiles are ordered row-tile-fastest and dealt to the eight
//    XCDs in contiguous runs so that tiles sharing weights or rows share an
//    L2.
// Both walk a tile list built in LDS from the device-side group offsets, so
// the host never reads the counts.
#include "ffn_common.h"

namespace moe {

namespace {

// =========================== streaming kernel ==============================

constexpr int kSK = 128;   // k per chunk
constexpr int kSCols = 16; // output columns per wave

template <int FM, bool GATEUP>
__global__ __launch_bounds__(256, (FM <= 3 ? 3 : 2)) void ffn_stream_kernel(FfnArgs p) {
  constexpr int RB = FM * 16;
  constexpr int NMAT = GATEUP ? 2 : 1;
  constexpr int BNC = 4 * kSCols;
  __shared__ __align__(16) uint16_t sa[2][RB * kSK];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tp[kMaxGroups + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, ncols = p.ncols;
  const int NT = ncols / BNC;
  const int NC = K / kSK;                     // the host sends only K % 128 == 0 here
  const int total = build_tile_list<0>(p, NT, s_off, s_tp);

  // one tile per block; blocks past the end of the list exit
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int e = find_group(s_tp, p.E, tile);
    const int ct = tile - s_tp[e];
    const int base = s_off[e];
    const int cnt = s_off[e + 1] - base;
    const int col0 = ct * BNC + wave * kSCols;
    const uint16_t* wb[NMAT];
    wb[0] = p.w0 + ((size_t)e * ncols + col0 + (lane & 15)) * K + (lane >> 4) * 8;
    if (GATEUP) wb[NMAT - 1] = p.w1 + ((size_t)e * ncols + col0 + (lane & 15)) * K + (lane >> 4) * 8;

    for (int r0 = 0; r0 < cnt; r0 += RB) {
      const int nrows = min(RB, cnt - r0);
      uint32_t aoff[FM];
      int adst[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = (tid >> 4) + 16 * i, ch = tid & 15;
        const int rr = (r < nrows) ? r : 0;
        const int grow = p.a_rows ? p.a_rows[base + r0 + rr] : (base + r0 + rr);
        aoff[i] = (uint32_t)grow * (uint32_t)K + ch * 8;
        adst[i] = r * kSK + ((ch ^ (r & 15)) << 3);
      }
      f32x4_t acc[NMAT][FM];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[m][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      // B fragments for chunk c live in bc; chunk c+1 is in flight in bn
      // while chunk c is multiplied.
      uint4 bc[NMAT][4], bn[NMAT][4];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        *reinterpret_cast<uint4*>(&sa[0][adst[i]]) = *reinterpret_cast<const uint4*>(p.a + aoff[i]);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int s = 0; s < 4; ++s) bc[m][s] = *reinterpret_cast<const uint4*>(wb[m] + 32 * s);
      __syncthreads();

      for (int c = 0; c < NC; ++c) {
        // the last chunk re-reads itself so that loads and stores stay
        // unconditional (keeps the staging arrays in registers)
        const int ko = (c + 1 < NC ? c + 1 : c) * kSK;
        uint4 ra[FM];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int s = 0; s < 4; ++s) bn[m][s] = *reinterpret_cast<const uint4*>(wb[m] + ko + 32 * s);
#pragma unroll
        for (int i = 0; i < FM; ++i) ra[i] = *reinterpret_cast<const uint4*>(p.a + aoff[i] + ko);
        const uint16_t* L = sa[c & 1];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int ch = s * 4 + (lane >> 4);
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int r = i * 16 + (lane & 15);
            const uint4 af = *reinterpret_cast<const uint4*>(&L[r * kSK + ((ch ^ (r & 15)) << 3)]);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) acc[m][i] = mfma16(af, bc[m][s], acc[m][i]);
          }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) *reinterpret_cast<uint4*>(&sa[(c + 1) & 1][adst[i]]) = ra[i];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int s = 0; s < 4; ++s) bc[m][s] = bn[m][s];
        __syncthreads();
      }

      const int col = col0 + (lane & 15);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = i * 16 + (lane >> 4) * 4 + q;
          if (r >= nrows) continue;
          const int orow = base + r0 + r;
          float v;
          if (GATEUP) {
            const float g = acc[0][i][q], u = acc[NMAT - 1][i][q];
            v = g / (1.f + __expf(-g)) * u;
          } else {
            v = acc[0][i][q] * (p.row_scale ? p.row_scale[orow] : 1.f);
          }
          p.out[(size_t)orow * ncols + col] = f32_to_bf16(v);
        }
      }
    }
  }
}

// ============================== tiled kernel ===============================

constexpr int kBK = 64;   // contraction slab: 8 chunks of 16 B per row

__device__ __forceinline__ int swz8(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

template <int BM, int BN, int WM, int WN, bool GATEUP>
__global__ __launch_bounds__(256) void ffn_tile_kernel(FfnArgs p) {
  constexpr int NB = GATEUP ? 2 * BN : BN;   // weight rows per tile
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile (output)
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int NACC = GATEUP ? 2 : 1;
  constexpr int A_LD = BM * 8 / 256;
  constexpr int B_LD = NB * 8 / 256;
  static_assert(BM % 32 == 0 && NB % 32 == 0 && TM % 16 == 0 && TN % 16 == 0, "tile shape");
  static_assert(WM * WN == 4, "four waves");

  extern __shared__ __align__(16) uint16_t lds[];   // [2][(BM + NB) * kBK]
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tp[kMaxGroups + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int K = p.K, ncols = p.ncols;
  const int NT = ncols / BN;
  const int total = build_tile_list<BM>(p, NT, s_off, s_tp);
  const int G = gridDim.x;
  const int per_xcd = G >> 3;              // G is a multiple of 8
  const int slot = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  constexpr int STAGE = (BM + NB) * kBK;

  for (int round = 0;; ++round) {
    const int tile = round * G + slot;
    if (round * G >= total) break;
    if (tile >= total) continue;
    const int e = find_group(s_tp, p.E, tile);
    const int cnt = s_off[e + 1] - s_off[e];
    const int RT = ceil_div(cnt, BM);
    const int local = tile - s_tp[e];
    const int ct = local / RT, rt = local - ct * RT;
    const int row0 = s_off[e] + rt * BM;
    const int nrows = min(BM, cnt - rt * BM);
    const int col0 = ct * BN;

    uint32_t a_off[A_LD];
    int a_dst[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int c = tid + 256 * i, r = c >> 3, ch = c & 7;
      const int rr = (r < nrows) ? r : 0;
      const int grow = p.a_rows ? p.a_rows[row0 + rr] : (row0 + rr);
      a_off[i] = (uint32_t)grow * (uint32_t)K + ch * 8;
      a_dst[i] = swz8(r, ch);
    }
    const uint16_t* w0 = p.w0 + ((size_t)e * ncols + col0) * K;
    const uint16_t* w1 = GATEUP ? p.w1 + ((size_t)e * ncols + col0) * K : nullptr;
    uint32_t b_off[B_LD];
    int b_dst[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int c = tid + 256 * i, r = c >> 3, ch = c & 7;
      const int wr = (GATEUP && r >= BN) ? r - BN : r;
      b_off[i] = (uint32_t)wr * (uint32_t)K + ch * 8;
      b_dst[i] = swz8(BM + r, ch);
    }
    auto bsrc = [&](int i) -> const uint16_t* {
      const int r = (tid + 256 * i) >> 3;
      return ((GATEUP && r >= BN) ? w1 : w0) + b_off[i];
    };

    f32x4_t acc[NACC][FM][FN];
#pragma unroll
    for (int g = 0; g < NACC; ++g)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[g][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      *reinterpret_cast<uint4*>(&lds[a_dst[i]]) = *reinterpret_cast<const uint4*>(p.a + a_off[i]);
#pragma unroll
    for (int i = 0; i < B_LD; ++i)
      *reinterpret_cast<uint4*>(&lds[b_dst[i]]) = *reinterpret_cast<const uint4*>(bsrc(i));
    __syncthreads();

    const int KT = K / kBK;
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      // the last slab re-reads itself so loads/stores stay unconditional
      const int ko = (kt + 1 < KT ? kt + 1 : kt) * kBK;
      uint4 ra[A_LD], rb[B_LD];
#pragma unroll
      for (int i = 0; i < A_LD; ++i) ra[i] = *reinterpret_cast<const uint4*>(p.a + a_off[i] + ko);
#pragma unroll
      for (int i = 0; i < B_LD; ++i) rb[i] = *reinterpret_cast<const uint4*>(bsrc(i) + ko);
      const uint16_t* L = lds + cur * STAGE;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int ch = ks * 4 + (lane >> 4);
        uint4 af[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const uint4*>(&L[swz8(wm * TM + i * 16 + (lane & 15), ch)]);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int rb0 = BM + wn * TN + j * 16 + (lane & 15);
          const uint4 b0 = *reinterpret_cast<const uint4*>(&L[swz8(rb0, ch)]);
#pragma unroll
          for (int i = 0; i < FM; ++i) acc[0][i][j] = mfma16(af[i], b0, acc[0][i][j]);
          if (GATEUP) {
            const uint4 b1 = *reinterpret_cast<const uint4*>(&L[swz8(rb0 + BN, ch)]);
#pragma unroll
            for (int i = 0; i < FM; ++i) acc[NACC - 1][i][j] = mfma16(af[i], b1, acc[NACC - 1][i][j]);
          }
        }
      }
      uint16_t* Ln = lds + (cur ^ 1) * STAGE;
#pragma unroll
      for (int i = 0; i < A_LD; ++i) *reinterpret_cast<uint4*>(&Ln[a_dst[i]]) = ra[i];
#pragma unroll
      for (int i = 0; i < B_LD; ++i) *reinterpret_cast<uint4*>(&Ln[b_dst[i]]) = rb[i];
      __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wm * TM + i * 16 + (lane >> 4) * 4 + q;
        if (row >= nrows) continue;
        const size_t orow = (size_t)(row0 + row) * ncols;
        const float s = (!GATEUP && p.row_scale) ? p.row_scale[row0 + row] : 1.f;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = col0 + wn * TN + j * 16 + (lane & 15);
          float v;
          if (GATEUP) {
            const float g = acc[0][i][j][q], u = acc[NACC - 1][i][j][q];
            v = g / (1.f + __expf(-g)) * u;
          } else {
            v = acc[0][i][j][q] * s;
          }
          p.out[orow + col] = f32_to_bf16(v);
        }
      }
    }
  }
}

// ================================ launchers =================================

template <int FM, bool GATEUP>
hipError_t launch_stream(const FfnArgs& a, int num_cu, hipStream_t st) {
  (void)num_cu;
  const int NT = a.ncols / (4 * kSCols);
  const long groups = a.E < a.rows_total ? a.E : a.rows_total;   // non-empty groups, at most
  const long grid = groups * NT;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((ffn_stream_kernel<FM, GATEUP>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool GATEUP>
hipError_t launch_tile(const FfnArgs& a, int num_cu, hipStream_t st) {
  constexpr int NB = GATEUP ? 2 * BN : BN;
  const size_t lds = (size_t)2 * (BM + NB) * kBK * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_tile_kernel<BM, BN, WM, WN, GATEUP>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int NT = a.ncols / BN;
  const long ub_rows = a.rows_total / BM + (a.E < a.rows_total ? a.E : a.rows_total);
  const long ub = ub_rows * NT;
  long grid = num_cu;
  if (ub < grid) grid = ((ub + 7) / 8) * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((ffn_tile_kernel<BM, BN, WM, WN, GATEUP>), dim3((unsigned)grid), dim3(256), lds, st, a);
  return hipGetLastError();
}

// Mean rows per group decides the kernel; the streaming kernel's pass height
// covers ~1.5x the mean so that typical groups take one pass.
int stream_fm(const FfnArgs& a) {
  if (a.K % kSK != 0 || a.ncols % (4 * kSCols) != 0) return 0;
  const double mean = (double)a.rows_total / (a.E > 0 ? a.E : 1);
  if (mean > 56.0) return 0;
  const double need = mean * 1.2;
  if (need <= 16.0) return 1;
  if (need <= 32.0) return 2;
  if (need <= 48.0) return 3;
  return 4;
}

}  // namespace

hipError_t launch_ffn_gateup(const FfnArgs& a, int num_cu, hipStream_t st) {
  if (a.rows_total == 0) return hipSuccess;
  switch (stream_fm(a)) {
    case 1: return launch_stream<1, true>(a, num_cu, st);
    case 2: return launch_stream<2, true>(a, num_cu, st);
    case 3: return launch_stream<3, true>(a, num_cu, st);
    case 4: return launch_stream<4, true>(a, num_cu, st);
    default: break;
  }
  if (a.ncols % 128 == 0) return launch_tile<256, 128, 2, 2, true>(a, num_cu, st);
  return launch_tile<128, 64, 2, 2, true>(a, num_cu, st);
}

hipError_t launch_ffn_down(const FfnArgs& a, int num_cu, hipStream_t st) {
  if (a.rows_total == 0) return hipSuccess;
  switch (stream_fm(a)) {
    case 1: return launch_stream<1, false>(a, num_cu, st);
    case 2: return launch_stream<2, false>(a, num_cu, st);
    case 3: return launch_stream<3, false>(a, num_cu, st);
    case 4: return launch_stream<4, false>(a, num_cu, st);
    default: break;
  }
  if (a.ncols % 256 == 0) return launch_tile<256, 256, 2, 2, false>(a, num_cu, st);
  return launch_tile<128, 64, 2, 2, false>(a, num_cu, st);
}

}  // namespace moe
