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
//  * stream (decode-sized groups, <= 56 mean rows): every wave owns 16 output
//    columns and streams its weight rows from HBM (row-contiguous loads two
//    chunks ahead, staged through a wave-private LDS slot); the group's token
//    rows (at most 64 per pass) are staged in LDS and shared by the four
//    waves.  Weights are read once per pass; the kernel is bound by HBM
//    bandwidth.  Blocks start their walk over the contraction at different
//    chunks so that concurrent loads spread over DRAM channels.
//  * tile (large groups): 256-row x 256-column tiles, both operands loaded
//    straight into LDS in 64-wide stages (16-byte chunks XOR-swizzled by row
//    so MFMA fragment reads are free of bank conflicts), eight waves of
//    128 x 64.  Tiles are ordered row-tile-fastest and dealt to the eight
//    XCDs in contiguous runs so that tiles sharing weights or rows share an
//    L2.
// Both walk a tile list built in LDS from the device-side group offsets, so
// the host never reads the counts.
#include "ffn_common.h"

namespace moe {

namespace {

// =========================== streaming kernel ==============================
//
// Weights are read row-contiguously: one load instruction covers 4 weight
// rows x 256 contiguous bytes (16 lanes per row), which keeps the DRAM and L2
// request stream dense (an MFMA-fragment-shaped load touches 16 rows x 64 B
// and streams markedly slower).  Each wave owns 16 output columns; its
// weight chunks are prefetched LA = 2 chunks ahead into registers, then
// staged through a wave-private LDS slot (16-byte chunks XOR-swizzled by row)
// from which the MFMA fragments are read.  Only the token rows (A) are shared
// by the block's four waves: double-buffered in LDS, one barrier per chunk.

constexpr int kSK = 128;   // k per chunk: 256 B of every weight row
constexpr int kSCols = 16; // output columns per wave
// LA: weight chunks in flight per wave (registers).  NMD: 16-row groups per
// wave for down (2 or 3).
template <int FM, bool GATEUP, int LA, int NMD>
__global__ __launch_bounds__(256, 2) void ffn_stream_kernel(FfnArgs p) {
  constexpr int RB = FM * 16;
  // every wave streams groups of 16 weight rows: gate and up rows of the
  // same 16 h columns, or (down) NMD x 16 consecutive rows of W_down, i.e.
  // 16 * NMD output columns (measured on the Mixtral-shaped down: 48 columns
  // per wave, 256 blocks, ran 9% faster than 32 columns per wave)
  constexpr int NMAT = GATEUP ? 2 : NMD;
  constexpr int WCOLS = GATEUP ? kSCols : NMD * kSCols;   // output columns per wave
  constexpr int BNC = 4 * WCOLS;
  constexpr int AL = RB * 16 / 256;          // A uint4 per thread per chunk
  __shared__ __align__(16) uint16_t sa[2][RB * kSK];
  __shared__ __align__(16) uint16_t sb[4][NMAT][kSCols * kSK];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tp[kMaxGroups + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, ncols = p.ncols;
  const int NT = ncols / BNC;
  const int NC = K / kSK;                     // the host sends only K % 128 == 0 here
  // one tile = (group, pass of RB rows, 64 output columns); one tile per block
  const int total = build_tile_list<RB>(p, NT, s_off, s_tp);
  // Tiles follow the block index.  (Dealing one expert's tiles to a single
  // XCD keeps its token rows in one L2 but measured ~20% slower: eight
  // XCDs each streaming one contiguous weight region.)
  const int tile = blockIdx.x;
  if (tile >= total) return;
  const int e = find_group(s_tp, p.E, tile);
  const int cnt = s_off[e + 1] - s_off[e];
  const int RT = ceil_div(cnt, RB);
  const int local = tile - s_tp[e];
  const int ct = local / RT, rt = local - ct * RT;
  const int row0 = s_off[e] + rt * RB;
  const int nrows = min(RB, cnt - rt * RB);
  const int col0 = ct * BNC + wave * WCOLS;
  // element offset of the block's c-th chunk: each block starts its k walk
  // at a different chunk (wrapping), so the blocks running together spread
  // over the offsets within the weight rows.  Measured: with every block at
  // the same offset, gate+up streamed ~10% slower whenever the gate and up
  // tensors sat at unfavourable relative addresses.
  const int rot = (int)(blockIdx.x % (unsigned)NC);
  auto kof = [rot, NC](int c) {
    const int cc = c + rot;
    return (cc >= NC ? cc - NC : cc) * kSK;
  };

  // weight load mapping: instruction i covers rows 4i + (lane >> 4), 16-byte chunk lane & 15
  const int brow = lane >> 4, bch = lane & 15;
  const size_t wrow = ((size_t)e * ncols + col0 + brow) * K + bch * 8;
  const uint16_t* wb0 = p.w0 + wrow;
  const uint16_t* wb1 = GATEUP ? p.w1 + wrow : p.w0 + wrow + (size_t)kSCols * K;
  // weight group m: gate / up rows, or down rows 16m.. of the wave's columns
  auto wsrc = [&](int m) -> const uint16_t* {
    return GATEUP ? (m == 0 ? wb0 : wb1) : wb0 + (size_t)m * kSCols * K;
  };
  int bdst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + brow;
    bdst[i] = r * kSK + ((bch ^ r) << 3);
  }
  const int fr = lane & 15;                   // MFMA fragment row / column

  uint32_t aoff[AL];
  int adst[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int r = (tid >> 4) + 16 * i, ch = tid & 15;
    const int rr = (r < nrows) ? r : 0;
    const int grow = p.a_rows ? p.a_rows[row0 + rr] : (row0 + rr);
    aoff[i] = (uint32_t)grow * (uint32_t)K + ch * 8;
    adst[i] = r * kSK + ((ch ^ (r & 15)) << 3);
  }
  f32x4_t acc[NMAT][FM];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[m][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // prologue: chunk 0 straight into LDS, chunks 1..LA into registers
  uint4 bq[LA][NMAT][4];
  {
    const int k0 = kof(0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
        *reinterpret_cast<uint4*>(&sb[wave][m][bdst[i]]) = *reinterpret_cast<const uint4*>(wsrc(m) + (size_t)4 * i * K + k0);
  }
#pragma unroll
  for (int l = 0; l < LA; ++l) {
    const int ko = kof(1 + l < NC ? 1 + l : NC - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
        bq[l][m][i] = *reinterpret_cast<const uint4*>(wsrc(m) + (size_t)4 * i * K + ko);
  }
#pragma unroll
  for (int i = 0; i < AL; ++i)
    *reinterpret_cast<uint4*>(&sa[0][adst[i]]) = *reinterpret_cast<const uint4*>(p.a + aoff[i] + kof(0));
  __syncthreads();

  for (int c = 0; c < NC; ++c) {
    // the last chunk re-reads itself so loads and stores stay unconditional
    const int ka = kof(c + 1 < NC ? c + 1 : c);
    uint4 ra[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) ra[i] = *reinterpret_cast<const uint4*>(p.a + aoff[i] + ka);
    const uint16_t* L = sa[c & 1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = s * 4 + (lane >> 4);
      uint4 bf[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
        bf[m] = *reinterpret_cast<const uint4*>(&sb[wave][m][fr * kSK + ((ch ^ fr) << 3)]);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = i * 16 + fr;
        const uint4 af = *reinterpret_cast<const uint4*>(&L[r * kSK + ((ch ^ (r & 15)) << 3)]);
#pragma unroll
        for (int m = 0; m < NMAT; ++m) acc[m][i] = mfma16(af, bf[m], acc[m][i]);
      }
    }
    // chunk c+1 (oldest registers) into this wave's LDS slot, after this
    // wave's reads of chunk c; rotate; fetch chunk c+1+LA
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&sb[wave][m][bdst[i]]) = bq[0][m][i];
#pragma unroll
    for (int l = 0; l + 1 < LA; ++l)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) bq[l][m][i] = bq[l + 1][m][i];
    {
      const int cn = c + 1 + LA;
      const int ko = kof(cn < NC ? cn : NC - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
          bq[LA - 1][m][i] = *reinterpret_cast<const uint4*>(wsrc(m) + (size_t)4 * i * K + ko);
    }
#pragma unroll
    for (int i = 0; i < AL; ++i) *reinterpret_cast<uint4*>(&sa[(c + 1) & 1][adst[i]]) = ra[i];
    __syncthreads();
  }

  const int col = col0 + fr;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = i * 16 + (lane >> 4) * 4 + q;
      if (r >= nrows) continue;
      const int orow = row0 + r;
      if (GATEUP) {
        const float g = acc[0][i][q], u = acc[1][i][q];
        p.out[(size_t)orow * ncols + col] = f32_to_bf16(g / (1.f + __expf(-g)) * u);
      } else {
        const float sc = p.row_scale ? p.row_scale[orow] : 1.f;
        const size_t dst = (size_t)(p.out_rows ? p.out_rows[orow] : orow) * ncols + col;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) p.out[dst + m * kSCols] = f32_to_bf16(acc[m][i][q] * sc);
      }
    }
  }
}

// Decode variant (at most 16 rows per pass): the four waves of a block share
// one 16-row x WCOLS output tile and split the contraction four ways, so a
// batch of a few tokens still spreads over hundreds of blocks.  Each wave
// stages its own token rows and weight rows in private LDS slots, so the k
// loop has no block barrier; the four partial tiles are summed in wave order
// through LDS at the end (deterministic).
template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void ffn_stream_ks_kernel(FfnArgs p) {
  constexpr int RB = 16;
  constexpr int WCOLS = GATEUP ? kSCols : 2 * kSCols;   // output columns per block
  constexpr int LA = 2;
  __shared__ __align__(16) uint16_t sa[4][RB * kSK];
  __shared__ __align__(16) uint16_t sb[4][2][kSCols * kSK];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tp[kMaxGroups + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, ncols = p.ncols;
  const int NT = ncols / WCOLS;
  const int NC = K / kSK;                     // the host sends only K % 128 == 0 here
  const int c0 = (wave * NC) / 4, c1 = ((wave + 1) * NC) / 4;   // this wave's chunks
  const int total = build_tile_list<RB>(p, NT, s_off, s_tp);
  const int tile = blockIdx.x;
  if (tile >= total) return;
  const int e = find_group(s_tp, p.E, tile);
  const int cnt = s_off[e + 1] - s_off[e];
  const int RT = ceil_div(cnt, RB);
  const int local = tile - s_tp[e];
  const int ct = local / RT, rt = local - ct * RT;
  const int row0 = s_off[e] + rt * RB;
  const int nrows = min(RB, cnt - rt * RB);
  const int col0 = ct * WCOLS;

  const int brow = lane >> 4, bch = lane & 15, fr = lane & 15;
  const size_t wrow = ((size_t)e * ncols + col0 + brow) * K + bch * 8;
  const uint16_t* wb0 = p.w0 + wrow;
  const uint16_t* wb1 = GATEUP ? p.w1 + wrow : p.w0 + wrow + (size_t)kSCols * K;
  int bdst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + brow;
    bdst[i] = r * kSK + ((bch ^ r) << 3);
  }
  // token rows: lane loads rows 4i + (lane >> 4), chunk lane & 15 (like the weights)
  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + brow;
    const int rr = (r < nrows) ? r : 0;
    const int grow = p.a_rows ? p.a_rows[row0 + rr] : (row0 + rr);
    aoff[i] = (uint32_t)grow * (uint32_t)K + bch * 8;
  }
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

  if (c0 < c1) {
    // the wave walks its chunks starting at a block-dependent one (wrapping),
    // so that concurrent blocks spread over the weight rows' offsets
    const int L = c1 - c0;
    const int rot = (int)(blockIdx.x % (unsigned)L);
    auto kof = [c0, L, rot](int j) {
      const int jj = j + rot;
      return (c0 + (jj >= L ? jj - L : jj)) * kSK;
    };
    // prologue: chunk 0 of the walk into LDS, chunks 1..LA into registers
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ko = kof(0);
      *reinterpret_cast<uint4*>(&sa[wave][bdst[i]]) = *reinterpret_cast<const uint4*>(p.a + aoff[i] + ko);
      *reinterpret_cast<uint4*>(&sb[wave][0][bdst[i]]) = *reinterpret_cast<const uint4*>(wb0 + (size_t)4 * i * K + ko);
      *reinterpret_cast<uint4*>(&sb[wave][1][bdst[i]]) = *reinterpret_cast<const uint4*>(wb1 + (size_t)4 * i * K + ko);
    }
    uint4 qa[LA][4], qb[LA][2][4];
#pragma unroll
    for (int l = 0; l < LA; ++l) {
      const int ko = kof(min(1 + l, L - 1));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qa[l][i] = *reinterpret_cast<const uint4*>(p.a + aoff[i] + ko);
        qb[l][0][i] = *reinterpret_cast<const uint4*>(wb0 + (size_t)4 * i * K + ko);
        qb[l][1][i] = *reinterpret_cast<const uint4*>(wb1 + (size_t)4 * i * K + ko);
      }
    }
    for (int c = 0; c < L; ++c) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ch = s * 4 + (lane >> 4);
        const int off = fr * kSK + ((ch ^ fr) << 3);
        const uint4 af = *reinterpret_cast<const uint4*>(&sa[wave][off]);
        acc0 = mfma16(af, *reinterpret_cast<const uint4*>(&sb[wave][0][off]), acc0);
        acc1 = mfma16(af, *reinterpret_cast<const uint4*>(&sb[wave][1][off]), acc1);
      }
      // same wave: LDS operations complete in order, so the slot can be
      // overwritten right after this wave's reads
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4*>(&sa[wave][bdst[i]]) = qa[0][i];
        *reinterpret_cast<uint4*>(&sb[wave][0][bdst[i]]) = qb[0][0][i];
        *reinterpret_cast<uint4*>(&sb[wave][1][bdst[i]]) = qb[0][1][i];
      }
#pragma unroll
      for (int l = 0; l + 1 < LA; ++l)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qa[l][i] = qa[l + 1][i];
          qb[l][0][i] = qb[l + 1][0][i];
          qb[l][1][i] = qb[l + 1][1][i];
        }
      const int ko = kof(min(c + 1 + LA, L - 1));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qa[LA - 1][i] = *reinterpret_cast<const uint4*>(p.a + aoff[i] + ko);
        qb[LA - 1][0][i] = *reinterpret_cast<const uint4*>(wb0 + (size_t)4 * i * K + ko);
        qb[LA - 1][1][i] = *reinterpret_cast<const uint4*>(wb1 + (size_t)4 * i * K + ko);
      }
    }
  }

  // partial tiles -> LDS (reusing the weight slots), summed in wave order
  __syncthreads();
  float* red = reinterpret_cast<float*>(&sb[0][0][0]);   // [4 waves][64 lanes][8]
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    red[(wave * 64 + lane) * 8 + q] = acc0[q];
    red[(wave * 64 + lane) * 8 + 4 + q] = acc1[q];
  }
  __syncthreads();
  if (wave == 0) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = red[lane * 8 + q];
#pragma unroll
    for (int w = 1; w < 4; ++w)
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] += red[(w * 64 + lane) * 8 + q];
    const int col = col0 + fr;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = (lane >> 4) * 4 + q;
      if (r >= nrows) continue;
      const int orow = row0 + r;
      if (GATEUP) {
        const float g = v[q], u = v[4 + q];
        p.out[(size_t)orow * ncols + col] = f32_to_bf16(g / (1.f + __expf(-g)) * u);
      } else {
        const float sc = p.row_scale ? p.row_scale[orow] : 1.f;
        const size_t dst = (size_t)(p.out_rows ? p.out_rows[orow] : orow) * ncols + col;
        p.out[dst] = f32_to_bf16(v[q] * sc);
        p.out[dst + kSCols] = f32_to_bf16(v[4 + q] * sc);
      }
    }
  }
}

// ============================== tiled kernel ===============================
//
// 256 rows x 256 weight rows per tile (gate+up: 128 gate and the same 128 up
// rows, i.e. 128 h columns; down: 256 output columns), eight waves in a 2 x 4
// grid, each 128 rows x 64 weight rows, bf16 MFMA 32x32x16 (fp32 accumulate).
// The k loop walks 64-wide stages (128 contiguous bytes of every row, one L2
// line) through two LDS stage buffers of 64 KB: stage kt+1 is loaded while
// stage kt is multiplied.  Stages are loaded straight into LDS (16 bytes per
// lane, no staging registers).  Each buffer is its own LDS array and the
// loop is unrolled over the two, so the compiler can tell which buffer a load
// writes and does not wait for it before reading the other; each wave waits
// for its own loads of a stage before the barrier that publishes the stage to
// the other waves.  A direct LDS load writes 16 bytes per lane at consecutive
// addresses, so the row swizzle is applied on the source side: the lane that
// fills slot p of row r fetches chunk p ^ g(r), g(r) = ((r >> 1) ^ ((r & 1)
// << 2)) & 7, which makes the 32-row fragment reads conflict-free for 32- and
// 64-bank LDS.  Tiles are ordered row-tile-fastest and dealt to the eight XCDs
// in contiguous runs, so tiles sharing weights or token rows share an L2.
//
// Measured on 16 experts x 2048 rows (M=4096, H=1536): ~1.0 PFLOP/s gate+up,
// ~0.8 down; the same loop without its loads reaches 1.6 / 1.1 and the loads
// alone take 75% of the full time, so the operand feed from L2 bounds it.
// (Four waves of 128 x 128, register-staged 32-wide stages and a four-deep
// ring of 32-wide stages all measured equal or slower.)

constexpr int kTBK = 64;                        // k per stage: 128-byte row segments
constexpr int kTN = 256;                        // weight rows per tile

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// 8 chunks of 16 B per row: chunk c of row r lives at slot c ^ g(r)
__device__ __forceinline__ int tsw(int row) { return ((row >> 1) ^ ((row & 1) << 2)) & 7; }

// 16 bytes per lane from global memory straight into LDS: lane l writes
// lds + 16 l (the LDS address must be the same in every lane).  A plain
// function, so that kernel templates call no target builtin directly.
__device__ __forceinline__ void dma16(const uint16_t* g, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// s_waitcnt for vector-memory count N only (expcnt and lgkmcnt left at their maxima)
#define MOE_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | 0x0F70)
// s_waitcnt lgkmcnt(0) only: the fragments of a stage are known complete at
// the end of its step
#define MOE_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)


// BM token rows per tile (256, 192 or 128): each wave covers BM/2 rows,
// FMW = BM/64 blocks of 32.
template <bool GATEUP, int BM>
__global__ __launch_bounds__(512, 1) void ffn_tile_kernel(FfnArgs p) {
  constexpr int HC = GATEUP ? kTN / 2 : kTN;     // output columns per tile
  constexpr int FMW = BM / 64;                   // 32-row MFMA blocks per wave
  constexpr int AI = BM / 64;                    // direct loads of token rows per wave per stage
  constexpr int STA = BM * kTBK;                 // bf16 elements of the token-row part
  __shared__ __align__(16) uint16_t sr0[(BM + kTN) * kTBK];
  __shared__ __align__(16) uint16_t sr1[(BM + kTN) * kTBK];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tp[kMaxGroups + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;       // 2 x 4 waves
  const int K = p.K, ncols = p.ncols;
  const int NT = ceil_div(ncols, HC);            // the last column tile may be partial
  const int KT = K / kTBK;
  const int total = build_tile_list<BM>(p, NT, s_off, s_tp);
  const int G = gridDim.x;                       // a multiple of 8
  const int slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int fr = lane & 31, fg = lane >> 5;

  const int swf = tsw(fr);
  int aoff0[4], boff0[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    aoff0[s] = (wm * (BM / 2) + fr) * kTBK + (((2 * s + fg) ^ swf) << 3);
    boff0[s] = STA + fr * kTBK + (((2 * s + fg) ^ swf) << 3);
  }
  int brow0[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) brow0[j] = GATEUP ? (j == 0 ? wn * 32 : HC + wn * 32) : wn * 64 + 32 * j;

  // direct LDS loads: instruction i of this wave fills token rows
  // (BM/8)*wave + 8*i + (lane >> 3) and weight rows 32*wave + 8*i + (lane >> 3),
  // slot lane & 7
  const int lrow = lane >> 3, lslot = lane & 7;

  for (int round = 0; round * G < total; ++round) {
    const int tile = round * G + slot;
    if (tile >= total) continue;
    const int e = find_group(s_tp, p.E, tile);
    const int cnt = s_off[e + 1] - s_off[e];
    const int RT = ceil_div(cnt, BM);
    const int local = tile - s_tp[e];
    const int ct = local / RT, rt = local - ct * RT;
    const int row0 = s_off[e] + rt * BM;
    const int nrows = min(BM, cnt - rt * BM);
    const int col0 = ct * HC;
    const uint16_t* wexp0 = p.w0 + (size_t)e * ncols * K;
    const uint16_t* wexp1 = GATEUP ? p.w1 + (size_t)e * ncols * K : wexp0;

    const uint16_t* asrc[AI];
    const uint16_t* bsrc[4];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int r = (BM / 8) * wave + 8 * i + lrow;
      const int ch = lslot ^ tsw(r);
      const int rr = (r < nrows) ? r : 0;
      const int grow = p.a_rows ? p.a_rows[row0 + rr] : (row0 + rr);
      asrc[i] = p.a + (size_t)grow * K + ch * 8;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * wave + 8 * i + lrow;
      const int ch = lslot ^ tsw(r);
      int wc = col0 + ((GATEUP && r >= HC) ? r - HC : r);
      if (wc >= ncols) wc = col0;                // partial column tile: any valid row
      bsrc[i] = ((GATEUP && r >= HC) ? wexp1 : wexp0) + (size_t)wc * K + ch * 8;
    }
    const int ldsA = ((BM / 8) * wave) * kTBK;
    const int ldsB = STA + (32 * wave) * kTBK;

#define MOE_DMA(BUF, KT_)                                                                          \
  {                                                                                                \
    const int ko_ = ((KT_) < KT ? (KT_) : KT - 1) * kTBK;                                         \
    _Pragma("unroll") for (int i = 0; i < AI; ++i)                                                 \
        dma16(asrc[i] + ko_, (BUF) + ldsA + 8 * i * kTBK);                                         \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                  \
        dma16(bsrc[i] + ko_, (BUF) + ldsB + 8 * i * kTBK);                                         \
  }

    f32x16_t acc[FMW][2];
#pragma unroll
    for (int i = 0; i < FMW; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // the previous tile's last reads of the buffers are done
    __syncthreads();
    MOE_DMA(sr0, 0)

    // one stage: wait for this wave's loads of stage KT_, publish it with the
    // barrier, start stage KT_+1 into the other buffer (every wave finished
    // reading it before the barrier), multiply stage KT_
#define MOE_TSTEP(BUF, NBUF, KT_)                                                                  \
  {                                                                                                \
    MOE_WAIT_VM(0);                                                                                \
    __builtin_amdgcn_s_barrier();                                                                  \
    MOE_DMA(NBUF, (KT_) + 1)                                                                       \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                                \
      u32x4_t af[FMW], bf[2];                                                                      \
      _Pragma("unroll") for (int i = 0; i < FMW; ++i)                                              \
          af[i] = *reinterpret_cast<const u32x4_t*>((BUF) + aoff0[s] + 32 * i * kTBK);            \
      _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                \
          bf[j] = *reinterpret_cast<const u32x4_t*>((BUF) + boff0[s] + brow0[j] * kTBK);          \
      _Pragma("unroll") for (int i = 0; i < FMW; ++i)                                              \
          _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]); \
    }                                                                                              \
    MOE_WAIT_LGKM0();                                                                              \
  }

    // the loop names each buffer explicitly (see above); an odd stage count
    // ends with one more step on the first buffer
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
      MOE_TSTEP(sr0, sr1, kt)
      MOE_TSTEP(sr1, sr0, kt + 1)
    }
    if (kt < KT) MOE_TSTEP(sr0, sr1, kt)
#undef MOE_TSTEP
#undef MOE_DMA
    MOE_WAIT_VM(0);
    // down: the tile's row scales through LDS (the first buffer is free once
    // every wave has finished its last stage)
    float* s_scale = reinterpret_cast<float*>(sr0);
    int* s_orow = reinterpret_cast<int*>(sr0) + BM;
    if (!GATEUP) {
      __syncthreads();
      if (tid < BM) {
        s_scale[tid] = (p.row_scale && tid < nrows) ? p.row_scale[row0 + tid] : 1.f;
        s_orow[tid] = (p.out_rows && tid < nrows) ? p.out_rows[row0 + tid] : row0 + tid;
      }
      __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < FMW; ++i) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wm * (BM / 2) + 32 * i + 8 * b + 4 * fg + q;
          if (row >= nrows) continue;
          uint16_t* orow = p.out + (size_t)(GATEUP ? row0 + row : s_orow[row]) * ncols;
          if (GATEUP) {
            const int col = col0 + wn * 32 + fr;
            const float g = acc[i][0][4 * b + q], u = acc[i][1][4 * b + q];
            if (col < ncols) orow[col] = f32_to_bf16(g / (1.f + __expf(-g)) * u);
          } else {
            const float sc = s_scale[row];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int col = col0 + wn * 64 + 32 * j + fr;
              if (col < ncols) orow[col] = f32_to_bf16(acc[i][j][4 * b + q] * sc);
            }
          }
        }
      }
    }
  }
}
#undef MOE_WAIT_VM
#undef MOE_WAIT_LGKM0

// ================================ launchers =================================

template <int FM, bool GATEUP, int LA = 2>
hipError_t launch_stream(const FfnArgs& a, int num_cu, hipStream_t st) {
  (void)num_cu;
  // down: three 16-row groups per wave where the columns divide evenly and
  // two blocks still fit a CU's LDS (at most 48 rows per pass)
  const bool nm3 = !GATEUP && FM <= 3 && a.ncols % (4 * 3 * kSCols) == 0;
  const int NT = a.ncols / (4 * kSCols * (GATEUP ? 1 : (nm3 ? 3 : 2)));
  const long groups = a.E < a.rows_total ? a.E : a.rows_total;   // non-empty groups, at most
  const long passes = a.rows_total / (FM * 16) + groups;          // >= sum of ceil(count / rows per pass)
  const long grid = passes * NT;
  if (grid <= 0) return hipSuccess;
  if constexpr (!GATEUP && FM <= 3) {
    if (nm3) {
      hipLaunchKernelGGL((ffn_stream_kernel<FM, GATEUP, LA, 3>), dim3((unsigned)grid), dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((ffn_stream_kernel<FM, GATEUP, LA, 2>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <bool GATEUP, int BM>
hipError_t launch_tile_bm(const FfnArgs& a, int num_cu, hipStream_t st) {
  constexpr int HC = GATEUP ? kTN / 2 : kTN;
  const int NT = ceil_div(a.ncols, HC);
  const long ub_rows = a.rows_total / BM + (a.E < a.rows_total ? a.E : a.rows_total);
  const long ub = ub_rows * NT;
  long grid = (num_cu / 8) * 8;
  if (ub < grid) grid = ((ub + 7) / 8) * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((ffn_tile_kernel<GATEUP, BM>), dim3((unsigned)grid), dim3(512), 0, st, a);
  return hipGetLastError();
}

// Tile height from the mean rows per group: the smallest of 128 / 192 / 256
// that holds 1.25x the mean, so that typical groups fill one row tile (a
// 256-row tile over 154-row groups wastes 40% of its MFMA work).
template <bool GATEUP>
hipError_t launch_tile(const FfnArgs& a, int num_cu, hipStream_t st) {
  const double need = 1.25 * (double)a.rows_total / (a.E > 0 ? a.E : 1);
  if (need <= 128.0) return launch_tile_bm<GATEUP, 128>(a, num_cu, st);
  if (need <= 192.0) return launch_tile_bm<GATEUP, 192>(a, num_cu, st);
  return launch_tile_bm<GATEUP, 256>(a, num_cu, st);
}

// The split-contraction decode kernel pays off only when the plain streaming
// launch would have too few blocks to keep every CU streaming (measured: it
// helps a 1-token batch, and loses at 32 tokens).
bool use_split_waves(const FfnArgs& a, bool gateup) {
  const long groups = a.E < a.rows_total ? a.E : a.rows_total;
  const long blocks = groups * (a.ncols / (4 * kSCols * (gateup ? 1 : 2)));
  return blocks < 1024;
}

template <bool GATEUP>
hipError_t launch_stream_ks(const FfnArgs& a, hipStream_t st) {
  const int NT = a.ncols / (GATEUP ? kSCols : 2 * kSCols);
  const long groups = a.E < a.rows_total ? a.E : a.rows_total;
  const long grid = (a.rows_total / 16 + groups) * NT;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((ffn_stream_ks_kernel<GATEUP>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Mean rows per group decides the kernel; the streaming kernel's pass height
// covers ~1.5x the mean so that typical groups take one pass.
int stream_fm(const FfnArgs& a, bool gateup) {
  if (a.K % kSK != 0 || a.ncols % (4 * kSCols * (gateup ? 1 : 2)) != 0) return 0;
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
  switch (stream_fm(a, true)) {
    case 1: return use_split_waves(a, true) ? launch_stream_ks<true>(a, st) : launch_stream<1, true>(a, num_cu, st);
    case 2: return launch_stream<2, true>(a, num_cu, st);
    case 3: return launch_stream<3, true>(a, num_cu, st);
    case 4: return launch_stream<4, true>(a, num_cu, st);
    default: break;
  }
  return launch_tile<true>(a, num_cu, st);
}

hipError_t launch_ffn_down(const FfnArgs& a, int num_cu, hipStream_t st) {
  if (a.rows_total == 0) return hipSuccess;
  switch (stream_fm(a, false)) {
    case 1: return use_split_waves(a, false) ? launch_stream_ks<false>(a, st) : launch_stream<1, false>(a, num_cu, st);
    case 2: return launch_stream<2, false>(a, num_cu, st);
    case 3: return launch_stream<3, false>(a, num_cu, st);
    case 4: return launch_stream<4, false>(a, num_cu, st);
    default: break;
  }
  return launch_tile<false>(a, num_cu, st);
}

}  // namespace moe
