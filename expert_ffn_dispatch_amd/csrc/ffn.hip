// Grouped SwiGLU expert GEMMs on bf16 MFMA (gfx950, fp32 accumulate): 16x16x32
// in the streaming kernels, 32x32x16 in the tile kernel.
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
//  * stream (decode-sized groups, <= 56 mean rows): every wave owns 16 (or
//    48) output columns and streams its weight rows from HBM (row-contiguous
//    loads two chunks ahead, staged through a wave-private LDS slot); the
//    group's token rows (at most 64 per pass) are staged in LDS and shared
//    by the block's waves.  Weights are read once per pass, with the
//    non-temporal hint (always for gate+up, from 8 KB rows on for down); the
//    kernel is bound by HBM bandwidth.  Blocks start their walk over the
//    contraction at different chunks so that concurrent loads spread over
//    DRAM channels.
//  * tile (large groups): 128/192/256-row x 256-column tiles, both operands
//    loaded straight into LDS in 64-wide stages (16-byte chunks XOR-swizzled
//    by row so MFMA fragment reads are free of bank conflicts), eight waves
//    of (rows/2) x 64.  Tiles are ordered row-tile-fastest and taken from
//    eight per-XCD queues of contiguous runs, so that tiles sharing weights
//    or rows share an L2.
// Both walk a tile list built on the device from the group offsets (the
// stream kernel's in LDS, the tile kernel's in registers), so the host never
// reads the counts.  Both also take FP8 (OCP E4M3) weights
// with one scale per output channel: the codes are widened to bf16 exactly
// as MFMA fragments are read from LDS, and the scale multiplies the fp32 sum.
#include <type_traits>

#include "ffn_common.h"
#include "ffn_stream.h"

namespace moe {

namespace {

// =========================== streaming kernel ==============================
//
// Weights are read row-contiguously: one load instruction covers 4 weight
// rows x 256 contiguous bytes (16 lanes per row), which keeps the DRAM and L2
// request stream dense (an MFMA-fragment-shaped load touches 16 rows x 64 B
// and streams markedly slower).  Each wave owns 16 output columns; its
// weight chunks are prefetched LA = 2 chunks ahead into registers, then
// staged through a wave-private LDS slot (16-byte pieces XOR-swizzled by row)
// from which the MFMA fragments are read.  Only the token rows (A) are shared
// by the block's four waves: double-buffered in LDS, one barrier per chunk.
//
// A chunk is 256 bytes of every weight row: 128 bf16 weights, or 256 FP8
// (OCP E4M3) codes.  FP8 codes are widened to bf16 as the MFMA fragments are
// read from LDS (exactly: every E4M3 value is a bf16 value), the products
// run on the bf16 MFMA, and the per-output-channel scale multiplies the fp32
// sum in the epilogue, so a weight row costs half the HBM bytes.

// LA: weight chunks in flight per wave (registers).  NMD: 16-row groups per
// wave for down (2 or 3).  F8: E4M3 weights with per-channel scales.  NW:
// waves per block (4 or 8); the token rows a block stages serve all of its
// waves, so 8 waves halve the token-row reads per weight byte.  NTL:
// non-temporal weight loads.
template <int FM, bool GATEUP, int LA, int NMD, bool F8, int NW, bool NTL>
__global__ __launch_bounds__(64 * NW, 8 / NW) void ffn_stream_kernel(FfnArgs p) {
  constexpr int RB = FM * 16;
  constexpr int KC = F8 ? 2 * kSK : kSK;     // contraction elements per chunk
  constexpr int ACH = KC / 8;                // 16-byte pieces of a token row per chunk
  constexpr int NSUB = KC / 32;              // MFMA sub-steps per chunk
  // Token rows: bf16 weights double-buffer them (one barrier per chunk);
  // FP8 chunks are twice as long in k, so one buffer (two barriers per
  // chunk) keeps the LDS at two blocks per CU.  Either way the wait for the
  // next chunk's token rows, issued before this chunk's weight prefetch,
  // leaves the prefetch a whole chunk to land (vector loads complete in
  // order, so waiting for a load waits for every older one).
  constexpr int NABUF = F8 ? 1 : 2;
  using ARow = typename std::conditional<F8, u32x4_t, uint4>::type;
  // every wave streams groups of 16 weight rows: gate and up rows of the
  // same 16 h columns, or (down) NMD x 16 consecutive rows of W_down, i.e.
  // 16 * NMD output columns (measured on the Mixtral-shaped down: 48 columns
  // per wave, 256 blocks, ran 9% faster than 32 columns per wave)
  constexpr int NMAT = GATEUP ? 2 : NMD;
  constexpr int WCOLS = GATEUP ? kSCols : NMD * kSCols;   // output columns per wave
  constexpr int BNC = NW * WCOLS;
  constexpr int NTH = 64 * NW;
  constexpr int AL = (RB * ACH + NTH - 1) / NTH;   // A pieces per thread per chunk (the last may be partial)
  constexpr bool AFULL = RB * ACH % NTH == 0;
  __shared__ __align__(16) uint16_t sa[NABUF][RB * KC];
  __shared__ __align__(16) uint16_t sb[NW][NMAT][kSCols * kSK];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tp[kMaxGroups + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, ncols = p.ncols;
  const int NT = ncols / BNC;
  const int NC = K / KC;                      // the host sends only K % KC == 0 here
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
  // the block's c-th chunk: each block starts its k walk at a different
  // chunk (wrapping), so the blocks running together spread over the
  // offsets within the weight rows.  Measured: with every block at the same
  // offset, gate+up streamed ~10% slower whenever the gate and up tensors
  // sat at unfavourable relative addresses.
  // Down: blocks are dealt to the eight XCDs round-robin by index, and the
  // blocks of one expert on one XCD share their starting chunk, so they read
  // each chunk of the expert's h rows at about the same time and that XCD's
  // L2 serves all but the first read (measured on the Mixtral-shaped batch:
  // FP8 down 175 -> 150 us, bf16 down 260 -> 258 us; the same start for
  // gate+up made the bf16 launch 3% slower there).
  const int rot = GATEUP ? (int)(blockIdx.x % (unsigned)NC)
                         : (int)((((unsigned)e * 8u + (blockIdx.x & 7u)) * 5u) % (unsigned)NC);
  auto kc = [rot, NC](int c) {
    const int cc = c + rot;
    return cc >= NC ? cc - NC : cc;
  };

  // weight load mapping: instruction i covers rows 4i + (lane >> 4), 16-byte piece lane & 15
  const int brow = lane >> 4, bch = lane & 15;
  const size_t RP = (size_t)K * (F8 ? 1 : 2);                 // weight row pitch in bytes
  const uint8_t* w0b = F8 ? p.q0 : reinterpret_cast<const uint8_t*>(p.w0);
  const uint8_t* w1b = F8 ? p.q1 : reinterpret_cast<const uint8_t*>(p.w1);
  const size_t wrow = ((size_t)e * ncols + col0 + brow) * RP + bch * 16;
  const uint8_t* wb0 = w0b + wrow;
  const uint8_t* wb1 = GATEUP ? w1b + wrow : wb0 + (size_t)kSCols * RP;
  // weight group m: gate / up rows, or down rows 16m.. of the wave's columns
  auto wsrc = [&](int m) -> const uint8_t* {
    return GATEUP ? (m == 0 ? wb0 : wb1) : wb0 + (size_t)m * kSCols * RP;
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
    const int r = tid / ACH + (NTH / ACH) * i, ch = tid % ACH;
    const int rr = (r < nrows) ? r : 0;
    const int grow = p.a_rows ? p.a_rows[row0 + rr] : (row0 + rr);
    aoff[i] = (uint32_t)grow * (uint32_t)K + ch * 8;
    adst[i] = r * KC + ((ch ^ (r & 15)) << 3);
  }
  f32x4_t acc[NMAT][FM];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[m][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // prologue: chunk 0 straight into LDS, chunks 1..LA into registers.
  // FP8 walks the chunks LA at a time with set u of bq holding chunk c+1 at
  // chunk c = c0 + u (no register copies); bf16 shifts the sets down by one
  // each chunk (measured: the copies cost FP8 ~6% and save bf16 ~4%).
  using WRow = typename std::conditional<F8, u32x4_t, uint4>::type;
  constexpr int UN = F8 ? LA : 1;            // chunks per trip of the loop
  WRow bq[LA][NMAT][4];
  {
    const int k0 = kc(0) * kRowBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
        *reinterpret_cast<uint4*>(&sb[wave][m][bdst[i]]) = load_weight<NTL, uint4>(wsrc(m) + 4 * i * RP + k0);
  }
#pragma unroll
  for (int l = 0; l < LA; ++l) {
    const int ko = kc(1 + l < NC ? 1 + l : NC - 1) * kRowBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
        bq[l][m][i] = load_weight<NTL, WRow>(wsrc(m) + 4 * i * RP + ko);
  }
#pragma unroll
  for (int i = 0; i < AL; ++i)
    if (AFULL || tid + NTH * i < RB * ACH)
      *reinterpret_cast<uint4*>(&sa[0][adst[i]]) = *reinterpret_cast<const uint4*>(p.a + aoff[i] + kc(0) * KC);
  __syncthreads();

  for (int c0 = 0; c0 < NC; c0 += UN) {
#pragma unroll
  for (int u = 0; u < UN; ++u) {
    const int c = c0 + u;
    if (UN > 1 && c >= NC) break;
    // the last chunk re-reads itself so loads and stores stay unconditional
    const int ka = kc(c + 1 < NC ? c + 1 : c) * KC;
    // (FP8's longer chunks need up to 8 of these per thread: kept as native
    // vectors, which stay in registers where a uint4 array would be copied
    // through scratch memory)
    ARow ra[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i)
      if (AFULL || tid + NTH * i < RB * ACH) ra[i] = *reinterpret_cast<const ARow*>(p.a + aoff[i] + ka);
    const uint16_t* L = sa[NABUF == 1 ? 0 : (c & 1)];
#pragma unroll
    for (int s = 0; s < (F8 ? NSUB / 2 : NSUB); ++s) {
      // FP8: s counts pairs of sub-steps (weight_pair_f8)
      u32x4_t bf[NMAT][F8 ? 2 : 1];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        if constexpr (F8) weight_pair_f8(&sb[wave][m][0], s, lane, bf[m][0], bf[m][F8 ? 1 : 0]);
        else bf[m][0] = weight_fragment<F8>(&sb[wave][m][0], s, lane);
      }
#pragma unroll
      for (int h = 0; h < (F8 ? 2 : 1); ++h) {
        const int ch = F8 ? 8 * s + 2 * (lane >> 4) + h : s * 4 + (lane >> 4);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = i * 16 + fr;
          const u32x4_t af = *reinterpret_cast<const u32x4_t*>(&L[r * KC + ((ch ^ (r & 15)) << 3)]);
#pragma unroll
          for (int m = 0; m < NMAT; ++m) acc[m][i] = mfma16(af, bf[m][h], acc[m][i]);
        }
      }
    }
    // chunk c+1 (oldest registers) into this wave's LDS slot, after this
    // wave's reads of chunk c; fetch chunk c+1+LA into the freed set
    const int su = F8 ? u : 0;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<WRow*>(&sb[wave][m][bdst[i]]) = bq[su][m][i];
    if (!F8) {
#pragma unroll
      for (int l = 0; l + 1 < LA; ++l)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) bq[l][m][i] = bq[l + 1][m][i];
    }
    {
      const int cn = c + 1 + LA;
      const int ko = kc(cn < NC ? cn : NC - 1) * kRowBytes;
      const int sl = F8 ? u : LA - 1;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
          bq[sl][m][i] = load_weight<NTL, WRow>(wsrc(m) + 4 * i * RP + ko);
    }
    if (NABUF == 1) __syncthreads();          // every wave is done with this chunk's token rows
#pragma unroll
    for (int i = 0; i < AL; ++i)
      if (AFULL || tid + NTH * i < RB * ACH)
        *reinterpret_cast<ARow*>(&sa[NABUF == 1 ? 0 : ((c + 1) & 1)][adst[i]]) = ra[i];
    __syncthreads();
  }
  }

  const int col = col0 + fr;
  // FP8: per-output-channel scales of this lane's columns
  float wsc[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    wsc[m] = 1.f;
    if constexpr (F8) {
      const size_t ch = (size_t)e * ncols + col;
      wsc[m] = GATEUP ? (m == 0 ? p.s0[ch] : p.s1[ch]) : p.s0[ch + m * kSCols];
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = i * 16 + (lane >> 4) * 4 + q;
      if (r >= nrows) continue;
      const int orow = row0 + r;
      if (GATEUP) {
        const float g = acc[0][i][q] * wsc[0], u = acc[1][i][q] * wsc[1];
        p.out[(size_t)orow * ncols + col] = f32_to_bf16(silu_mul(g, u));
      } else {
        const float sc = p.row_scale ? p.row_scale[orow] : 1.f;
        const size_t dst = (size_t)(p.out_rows ? p.out_rows[orow] : orow) * ncols + col;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) p.out[dst + m * kSCols] = f32_to_bf16(acc[m][i][q] * wsc[m] * sc);
      }
    }
  }
}

// Decode variant of the streaming kernel: one split-contraction tile per block.
template <bool GATEUP, bool F8>
__global__ __launch_bounds__(256, 2) void ffn_stream_ks_kernel(FfnArgs p) {
  constexpr int WCOLS = GATEUP ? kSCols : 2 * kSCols;
  __shared__ __align__(16) KsLds<F8> lds;
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tp[kMaxGroups + 1];
  const int total = build_tile_list<16>(p, p.ncols / WCOLS, s_off, s_tp);
  const int tile = blockIdx.x;
  if (tile >= total) return;
  ks_tile<GATEUP, F8>(p, s_off, s_tp, tile, blockIdx.x, lds);
}

// ============================== tiled kernel ===============================
//
// BM rows (128, 192 or 256) x 256 weight rows per tile (gate+up: 128 gate
// and the same 128 up rows, i.e. 128 h columns; down: 256 output columns),
// eight waves in a 2 x 4 grid, each BM/2 rows x 64 weight rows, bf16 MFMA
// 32x32x16 (fp32 accumulate).  The k loop walks 64-wide stages (128
// contiguous bytes of every row, one L2 line): token rows one stage ahead in
// two LDS buffers, weight rows two stages ahead in three (two for 256-row FP8
// tiles).  Stages are loaded straight into LDS (16 bytes per lane, no
// staging registers).  Each buffer is its own LDS array and the loop is
// unrolled over their period, so the compiler can tell which buffer a load
// writes and does not wait for it before reading another; each wave waits
// for its own loads of a stage before the barrier that publishes the stage to
// the other waves.  A direct LDS load writes 16 bytes per lane at consecutive
// addresses, so the row swizzle is applied on the source side: the lane that
// fills slot p of row r fetches chunk p ^ g(r), g(r) = ((r >> 1) ^ ((r & 1)
// << 2)) & 7, which makes the 32-row fragment reads conflict-free for 32- and
// 64-bank LDS.  Tiles are ordered row-tile-fastest (a group's row tiles
// balanced to within one 32-row block) and taken from per-XCD queues of
// contiguous runs, so tiles sharing weights or token rows share an L2.
//
// (Four waves of 128 x 128, register-staged 32-wide stages and a four-deep
// ring of 32-wide stages all measured equal or slower than eight waves.)

constexpr int kTBK = 64;                        // k per stage: 128-byte row segments
// A buffer offset past every token matrix that takes 32-bit offsets (those
// are below kA32Limit bytes, and a stage adds at most 128 KB): loads from it
// return zeros without a memory access.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr unsigned long long kA32Limit = 0x7FFF0000ull;
constexpr int kTN = 256;                        // weight rows per tile

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// 8 chunks of 16 B per row: chunk c of row r lives at slot c ^ g(r)
__device__ __forceinline__ int tsw(int row) { return ((row >> 1) ^ ((row & 1) << 2)) & 7; }

// Swizzle of the down epilogue's 32 x 64 staging block (row r, 16-byte chunk
// c, 8-byte half h at chunk c ^ stg_chunk(r), half h ^ stg_half(r)).  A
// ds_write_b64 of 32 lanes (rows 0..31, one chunk and half) covers 256 bytes:
// with 64 four-byte banks a row's 128 bytes take the bank half given by r & 1,
// and (r & 1, chunk, half) must be distinct for all 32 rows, which this
// mapping makes a bijection of r; with 32 banks, 16 lanes (rows 0..15) must be
// distinct in (chunk, half), which it also is.  Plain c ^ (r & 7) left rows r,
// r+8, r+16, r+24 on one bank pair.
__device__ __forceinline__ int stg_chunk(int r) { return (r & 7) ^ ((r >> 4) & 1); }
__device__ __forceinline__ int stg_half(int r) { return (r >> 3) & 1; }

// The routed groups' tile list, held in registers so that the stage buffers
// can take the whole LDS: lane l of every wave owns groups 4l .. 4l+3 (at most
// 256 groups), with their row offsets and the inclusive prefix of their tile
// counts; a tile's group is found with one ballot and a few lane reads.
struct RegTiles {
  int off[5];     // offsets of groups 4l .. 4l+4
  int tp[4];      // tiles of groups 0 .. 4l+i, inclusive
  int total;
};

template <int BM>
__device__ __forceinline__ RegTiles reg_tile_list(const FfnArgs& p, int col_tiles, int lane) {
  RegTiles r;
  const int E = p.E;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int e = 4 * lane + i;
    r.off[i] = e <= E ? (p.fixed_rows > 0 ? (e == 0 ? 0 : p.fixed_rows) : p.offsets[e]) : 0;
  }
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    if (e < E) sum += ceil_div(r.off[i + 1] - r.off[i], BM) * col_tiles;
    r.tp[i] = sum;
  }
  int inc = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) r.tp[i] += inc - sum;
  r.total = __shfl(inc, 63);
  return r;
}

// Row tile rt of a group of cnt rows cut into RT tiles of at most BM rows
// (RT = ceil(cnt / BM)): the group's 32-row blocks are dealt out evenly, so
// tiles of one group differ by one block at most and a group's padding is
// under 32 rows.  off: the tile's first row (a multiple of 32); nrows: its
// live rows.
__device__ __forceinline__ void row_tile(int cnt, int RT, int rt, int& off, int& nrows) {
  const int nb = (cnt + 31) >> 5;
  const int q = nb / RT, r = nb - q * RT;
  const int b0 = rt * q + min(rt, r);
  off = 32 * b0;
  nrows = min(32 * (q + (rt < r ? 1 : 0)), cnt - off);
}

// Group of routed tile t (t < total): its index, the first tile of the group,
// its first row and its row count (wave-uniform results).
__device__ __forceinline__ void reg_find(const RegTiles& r, int t, int& e, int& first, int& base, int& cnt) {
  const int L = (int)__builtin_ctzll(__ballot(r.tp[3] > t));
  int tp[4], off[5];
#pragma unroll
  for (int i = 0; i < 4; ++i) tp[i] = __builtin_amdgcn_readlane(r.tp[i], L);
#pragma unroll
  for (int i = 0; i < 5; ++i) off[i] = __builtin_amdgcn_readlane(r.off[i], L);
  const int prev = L > 0 ? __builtin_amdgcn_readlane(r.tp[3], L > 0 ? L - 1 : 0) : 0;
  const int i = (tp[0] <= t) + (tp[1] <= t) + (tp[2] <= t);
  e = 4 * L + i;
  first = i == 0 ? prev : i == 1 ? tp[0] : i == 2 ? tp[1] : tp[2];
  base = i == 0 ? off[0] : i == 1 ? off[1] : i == 2 ? off[2] : off[3];
  cnt = (i == 0 ? off[1] : i == 1 ? off[2] : i == 2 ? off[3] : off[4]) - base;
}

// 16 bytes per lane from global memory straight into LDS: lane l writes
// lds + 16 l (the LDS address must be the same in every lane).  A plain
// function, so that kernel templates call no target builtin directly.
__device__ __forceinline__ void dma16(const uint16_t* g, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}
__device__ __forceinline__ void dma16(const uint8_t* g, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}
// A block barrier for the block's LDS reads and writes (not its direct
// loads into LDS, which the stage barriers publish after each wave's own
// vmcnt wait): each wave's LDS operations complete (lgkmcnt), then the
// barrier; the empty asm statements keep the compiler from moving memory
// accesses across it.  __syncthreads would also wait for every vector-memory
// operation in flight (its fence covers global memory, and a release fence
// for LDS alone still waits for the direct loads into LDS), which in the
// tile kernel are the next tile's first loads and the last tile's stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// 4 bytes per lane: lane l writes lds + 4 l.
__device__ __forceinline__ void dma4(const int32_t* g, int32_t* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
}
// The same through a buffer resource: byte `voff + soff` of the buffer
// (per-lane and scalar parts kept apart, so that the compiler cannot turn them
// into 64-bit per-lane pointers; reads past `bytes` return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 0);
}
// The same with the non-temporal hint, for weight rows that no later tile
// reads again.
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 2);
}

// s_waitcnt for vector-memory count N only (expcnt and lgkmcnt left at their maxima)
#define MOE_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | 0x0F70)
// s_waitcnt lgkmcnt(0) only: the fragments of a stage are known complete at
// the end of its step
#define MOE_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)


// BM token rows per tile (256, 192 or 128): each wave covers BM/2 rows,
// FMW = BM/64 blocks of 32.
// F8: FP8 (E4M3) weights.  A stage then holds 64 bytes of every weight row
// (four 16-byte pieces, piece c of row r at c ^ ((r >> 2) & 3)); each lane
// reads its eight codes of a B fragment and widens them to bf16 exactly, and
// the per-channel scales multiply the sums in the epilogue.
// A32: the token matrix of every segment spans less than kA32Limit bytes
// (just under 2 GiB), so token rows are addressed by 32-bit offsets through a
// buffer resource, and padding rows by an offset past it; otherwise by 64-bit
// pointers (more registers, used with 128-row tiles only).
// PF: down tiles whose stage count divides by six (every segment's) load
// the next tile's first stages in their own last two (see the stage loop).
template <bool GATEUP, int BM, bool F8, bool A32, bool PF, bool NTW = false>
__global__ __launch_bounds__(512, 1) void ffn_tile_kernel(FfnArgs p, FfnArgs p2) {
  constexpr int HC = GATEUP ? kTN / 2 : kTN;     // output columns per tile
  constexpr int FMW = BM / 64;                   // 32-row MFMA blocks per wave
  constexpr int AI = BM / 64;                    // direct loads of token rows per wave per stage
  constexpr int BI = F8 ? 2 : 4;                 // direct loads of weight rows per wave per stage
  constexpr int STA = BM * kTBK;                 // bf16 elements of a token-row stage
  constexpr int WRB = F8 ? kTBK : 2 * kTBK;      // bytes of a weight row per stage
  constexpr int STB = kTN * WRB / 2;             // 16-bit elements of a weight stage
  // Token rows are loaded one stage ahead into two buffers.  Weight rows,
  // which mostly come from HBM, are loaded two stages ahead into three below
  // 256-row tiles (DeepSeek-V2-shaped layer 2.36 -> 2.18 ms, Qwen3-235B-shaped
  // 3.12 -> 3.00 ms); 256-row tiles keep two (bf16: three would not fit in
  // LDS; FP8: no faster).
  // Every buffer is an array of its own: the compiler then knows that loads
  // into one buffer do not touch the reads of another (as parts of one array
  // it waits for the loads before every read).
  constexpr int NB = (BM == 256 && F8) ? 2 : 3;
  // (three token buffers, with two or three weight buffers: 5% slower with
  // bf16 weights, within 1% with FP8)
  constexpr int NA = 2;
  // The MFMA takes the weight fragment as its first operand, so the
  // accumulators hold D[weight row][token row]: each lane ends with one
  // token row and four consecutive output columns per 32 x 32 block.  The
  // epilogue then stores four columns per lane (gate+up) or stages down's
  // output through LDS as whole row segments (FP8 Qwen3-235B-shaped layer
  // 3.37 -> 3.19 ms for the swap, 2.92 -> 2.72 ms for the staging; with
  // D[token row][weight row] lanes would hold columns and store 2 bytes).
  // (256-row bf16 tiles: five 32 KB buffers, the whole 160 KB of LDS)
  __shared__ __align__(16) uint16_t sa0[STA];
  __shared__ __align__(16) uint16_t sa1[STA];
  __shared__ __align__(16) uint16_t sb0[STB];
  __shared__ __align__(16) uint16_t sb1[STB];
  __shared__ __align__(16) uint16_t sb2[NB == 3 ? STB : 8];
  static_assert(NA == 2, "token rows are double-buffered");
  // Down (where the LDS has room): the row scales and output rows of the
  // tile, loaded straight into LDS at the tile start and read by the
  // epilogue.  Loaded by the epilogue itself, their latency stood between
  // the last multiplication and the first store of every tile.  (The whole
  // epilogue costs about 7 us per tile: timed without it, down on a
  // Qwen3-235B-shaped batch took 718 instead of 915 us.)
  constexpr bool RLDS = !GATEUP && !(BM == 256 && !F8);
  // (one array: each array loaded straight into LDS takes a slot of the
  // compiler's tracking of those loads, and past six it lost track and
  // waited for every load in flight before the epilogue's LDS writes)
  __shared__ __align__(16) int32_t s_rows[RLDS ? 2 * BM : 1];   // scale bits, then output rows

  // the wave index as a scalar: the weight rows a wave loads come from one
  // matrix, so their base address stays in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;       // 2 x 4 waves
  // p2 (if p2.E == 1): one group of p2.fixed_rows rows, the shared experts,
  // whose tiles are dealt first; then the routed groups of p.  One launch for
  // both spreads the shared tiles over the routed rounds instead of ending
  // each launch on a partly empty round.
  const int NT = ceil_div(p.ncols, HC);          // the last column tile may be partial
  const int RT2 = p2.E > 0 ? ceil_div(p2.fixed_rows, BM) : 0;
  const int T2 = RT2 * ceil_div(p2.ncols, HC);
  // The tile list: in registers, or (PF, whose registers are tighter and
  // whose LDS has room) in LDS.
  constexpr bool TLDS = PF;
  __shared__ int s_off[TLDS ? kMaxGroups + 1 : 1];
  __shared__ int s_tp[TLDS ? kMaxGroups + 1 : 1];
  RegTiles tl;
  int ltotal;
  if constexpr (TLDS) {
    ltotal = build_tile_list<BM>(p, NT, s_off, s_tp);
  } else {
    tl = reg_tile_list<BM>(p, NT, lane);
    ltotal = tl.total;
  }
  // group of routed tile t1: index, first tile, first row, row count
  auto find = [&](int t1, int& e, int& first, int& base, int& cnt) {
    if constexpr (TLDS) {
      e = find_group(s_tp, p.E, t1);
      first = s_tp[e];
      base = s_off[e];
      cnt = s_off[e + 1] - base;
    } else {
      reg_find(tl, t1, e, first, base, cnt);
    }
  };
  const int total = T2 + ltotal;
  const int G = gridDim.x;                       // a multiple of 8
  const int slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  // Tiles come from a queue per XCD (p.queue: eight counters, zero at
  // launch) wherever the LDS has room for the ticket (all but 256-row bf16
  // tiles, whose buffers take all of it): XCD x (blocks are
  // dealt to the XCDs round-robin by index) takes tiles of the x-th eighth
  // of the list in order, then those of the other eighths.  Tiles taken in
  // order start in order, so the tiles that share a weight tile (adjacent in
  // the list) run side by side and read it once into their XCD's L2, however
  // uneven the tiles before them were; dealt statically, blocks drifted apart
  // (a group's last row tile is cheaper) and the launch fetched up to twice
  // its bytes.  Otherwise tiles are dealt statically: tile round * G + slot,
  // contiguous runs per XCD.
  constexpr bool QCAP = !(BM == 256 && !F8);
  int* s_ticket = nullptr;
  int* s_next = nullptr;
  if constexpr (QCAP) {
    __shared__ int s_ticket_lds[2];
    s_ticket = &s_ticket_lds[0];
    s_next = &s_ticket_lds[1];
  }
  constexpr bool dyn = QCAP;           // (a runtime choice of the two costs ~20 registers)
  // A ticket of this XCD's queue (one thread of the block).  Its value is
  // first needed by claim(), stages later, so the atomic's latency is not
  // spent at the tile start, where every wave waits at the first barrier.
  auto take = [&]() -> int { return atomicAdd(&p.queue[blockIdx.x & 7], 1); };
  // The tile of ticket t of this XCD's queue; past its end, a tile of the
  // other queues in turn; -1 when every queue is exhausted.
  auto claim = [&](int t) -> int {
    const int tot = total;
    const int x = blockIdx.x & 7;
    const int lo = (int)(((long long)tot * x) >> 3), hi = (int)(((long long)tot * (x + 1)) >> 3);
    if (t < hi - lo) return lo + t;
#pragma nounroll
    for (int i = 1; i < 8; ++i) {
      const int y = (x + i) & 7;
      const int lo2 = (int)(((long long)tot * y) >> 3), hi2 = (int)(((long long)tot * (y + 1)) >> 3);
      if (lo2 >= hi2) continue;
      const int u = atomicAdd(&p.queue[y], 1);
      if (u < hi2 - lo2) return lo2 + u;
    }
    return -1;
  };
  const int fr = lane & 31, fg = lane >> 5;

  const int swf = tsw(fr);
  // boff0: 16-bit elements (bf16 weights) or bytes (FP8 codes) from the stage start
  int aoff0[4], boff0[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    aoff0[s] = (wm * (BM / 2) + fr) * kTBK + (((2 * s + fg) ^ swf) << 3);
    boff0[s] = F8 ? fr * WRB + ((s ^ ((fr >> 2) & 3)) << 4) + (fg << 3)
                  : fr * kTBK + (((2 * s + fg) ^ swf) << 3);
  }
  int brow0[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) brow0[j] = GATEUP ? (j == 0 ? wn * 32 : HC + wn * 32) : wn * 64 + 32 * j;

  // direct LDS loads: instruction i of this wave fills token rows
  // (BM/8)*wave + 8*i + (lane >> 3), slot lane & 7, and weight rows
  // 32*wave + 8*i + (lane >> 3), slot lane & 7 (FP8: 32*wave + 16*i + (lane >> 2),
  // slot lane & 3)
  const int lrow = lane >> 3, lslot = lane & 7;
  const int qrow = lane >> 2, qslot = lane & 3;

  // Tile t's expert, first token row, live rows, first output column and
  // the row tiles of its group.
  auto tile_geom = [&](int t, int& e, int& row0, int& nrows, int& col0, int& RT) {
    int cnt, local, base;
    e = 0;
    if (t < T2) {
      cnt = p2.fixed_rows;
      RT = RT2;
      local = t;
      base = 0;
    } else {
      const int t1 = t - T2;
      int first;
      find(t1, e, first, base, cnt);
      RT = ceil_div(cnt, BM);
      local = t1 - first;
    }
    const int ct = local / RT, rt = local - ct * RT;
    int off;
    row_tile(cnt, RT, rt, off, nrows);
    row0 = base + off;
    col0 = ct * HC;
  };
  // The direct loads of a tile of segment q: buffer resources (the weight
  // rows of a wave, rows 32 wave .. 32 wave + 31, lie all in the gate or all
  // in the up half of the tile, so one base per wave) and per-lane offsets,
  // or token-row pointers where !A32.
  auto tile_loads = [&](const FfnArgs& q, int e, int row0, int nrows, int col0, __amdgpu_buffer_rsrc_t& ar,
                        __amdgpu_buffer_rsrc_t& wr, uint32_t (&ao)[AI], const uint16_t* (&as)[A32 ? 1 : AI],
                        uint32_t (&bo)[BI]) {
    const int K = q.K, ncols = q.ncols;
    // weight rows as bytes (bf16: 2 per element, FP8: 1)
    constexpr int WB = F8 ? 1 : 2;
    const uint8_t* wexp0 = (F8 ? q.q0 : reinterpret_cast<const uint8_t*>(q.w0)) + (size_t)e * ncols * K * WB;
    const uint8_t* wexp1 =
        GATEUP ? (F8 ? q.q1 : reinterpret_cast<const uint8_t*>(q.w1)) + (size_t)e * ncols * K * WB : wexp0;
    ar = buffer_rsrc(q.a, A32 ? q.a_bytes : 0u);
    wr = buffer_rsrc((GATEUP && 32 * wave >= HC) ? wexp1 : wexp0, (uint32_t)ncols * (uint32_t)(K * WB));
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int r = (BM / 8) * wave + 8 * i + lrow;
      const int ch = lslot ^ tsw(r);
      const int rr = (r < nrows) ? r : 0;
      // (down reads h in sorted order: a_rows is for gate+up only, and a load
      // here that down never makes still cost it a wait for every load in flight)
      const int grow = (GATEUP && q.a_rows) ? q.a_rows[row0 + rr] : (row0 + rr);
      // padding rows (past the group's count) take an offset beyond the
      // buffer: the load writes zeros and reads no memory
      if constexpr (A32) ao[i] = r < nrows ? (uint32_t)grow * (uint32_t)(2 * K) + (uint32_t)(ch * 16) : kOutOfRange;
      else as[i] = q.a + (size_t)grow * K + ch * 8;
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int r = F8 ? 32 * wave + 16 * i + qrow : 32 * wave + 8 * i + lrow;
      const int ch = F8 ? qslot ^ ((r >> 2) & 3) : lslot ^ tsw(r);
      int wc = col0 + ((GATEUP && r >= HC) ? r - HC : r);
      if (wc >= ncols) wc = col0;                // partial column tile: any valid row
      bo[i] = (uint32_t)wc * (uint32_t)(K * WB) + (uint32_t)(ch * 16);
    }
  };

  // PF: every tile's stage count divides by six (the period of the stage
  // loop's buffer pattern), and each tile loads the next tile's first stages
  // in its own last two, into the buffers the next tile starts from, so
  // that they are in flight during this tile's epilogue (pre: this tile's
  // first stages were loaded so).  Down, with balanced row tiles:
  // DeepSeek-V2-shaped 773 -> 721 us, Qwen3-235B-shaped 911 -> 885 us.  (A
  // runtime choice between the two endings of the stage loop took the down
  // kernel past its registers, hence a kernel of its own.)
  static_assert(!PF || (!GATEUP && NB == 3 && A32 && BM < 256 && QCAP), "next-tile loads: down, three weight buffers");
  constexpr bool PFC = PF;
  bool pre = false;

  int tile = slot < total ? slot : -1;
  if (dyn) {
    if (tid == 0) *s_ticket = claim(take());
    __syncthreads();
    tile = __builtin_amdgcn_readfirstlane(*s_ticket);   // the same in every lane
  }
  for (int round = 0; tile >= 0; ++round) {
    // the next tile: its ticket is taken now and claimed later (after this
    // tile, or in its last stages where they load the next tile's first)
    int next = (round + 1) * G + slot;
    if (next >= total) next = -1;
    int tk = 0;
    if (dyn && tid == 0) tk = take();
    bool claimed = false, pre_next = false;    // set in the last stages (PFC)
    int nx = -1;
    const bool seg2 = tile < T2;
    const FfnArgs& pa = seg2 ? p2 : p;
    const int K = pa.K, ncols = pa.ncols, KT = K / kTBK;
    int e = 0, cnt, RT, local, base;
    if (seg2) {
      cnt = p2.fixed_rows;
      RT = RT2;
      local = tile;
      base = 0;
    } else {
      const int t1 = tile - T2;
      int first;
      find(t1, e, first, base, cnt);
      RT = ceil_div(cnt, BM);
      local = t1 - first;
    }
    const int ct = local / RT, rt = local - ct * RT;
    int roff, nrows;
    row_tile(cnt, RT, rt, roff, nrows);
    const int row0 = base + roff;
    const int col0 = ct * HC;
    // weight rows as bytes (bf16: 2 per element, FP8: 1)
    constexpr int WB = F8 ? 1 : 2;
    const uint8_t* wexp0 = (F8 ? pa.q0 : reinterpret_cast<const uint8_t*>(pa.w0)) + (size_t)e * ncols * K * WB;
    const uint8_t* wexp1 =
        GATEUP ? (F8 ? pa.q1 : reinterpret_cast<const uint8_t*>(pa.w1)) + (size_t)e * ncols * K * WB : wexp0;

    // token rows: 32-bit byte offsets into the token matrix (A32), else pointers
    const __amdgpu_buffer_rsrc_t arsrc = buffer_rsrc(pa.a, A32 ? pa.a_bytes : 0u);
    uint32_t aoffg[AI];
    const uint16_t* asrc[A32 ? 1 : AI];
    // weight rows: one base per wave (rows 32 wave .. 32 wave + 31 lie all in
    // the gate or all in the up half of the tile) and 32-bit offsets per lane
    const __amdgpu_buffer_rsrc_t wrsrc =
        buffer_rsrc((GATEUP && 32 * wave >= HC) ? wexp1 : wexp0, (uint32_t)ncols * (uint32_t)(K * WB));
    uint32_t boffg[BI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int r = (BM / 8) * wave + 8 * i + lrow;
      const int ch = lslot ^ tsw(r);
      const int rr = (r < nrows) ? r : 0;
      const int grow = (GATEUP && pa.a_rows) ? pa.a_rows[row0 + rr] : (row0 + rr);
      // padding rows (past the group's count) take an offset beyond the
      // buffer: the load writes zeros and reads no memory
      if constexpr (A32) aoffg[i] = r < nrows ? (uint32_t)grow * (uint32_t)(2 * K) + (uint32_t)(ch * 16) : kOutOfRange;
      else asrc[i] = pa.a + (size_t)grow * K + ch * 8;
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int r = F8 ? 32 * wave + 16 * i + qrow : 32 * wave + 8 * i + lrow;
      const int ch = F8 ? qslot ^ ((r >> 2) & 3) : lslot ^ tsw(r);
      int wc = col0 + ((GATEUP && r >= HC) ? r - HC : r);
      if (wc >= ncols) wc = col0;                // partial column tile: any valid row
      boffg[i] = (uint32_t)wc * (uint32_t)(K * WB) + (uint32_t)(ch * 16);
    }
    const int ldsA = ((BM / 8) * wave) * kTBK;
    const int ldsB = (32 * wave) * (WRB / 2);

#define MOE_DMA_A(BUF, KT_)                                                                        \
  _Pragma("unroll") for (int i = 0; i < AI; ++i) {                                                 \
    if constexpr (A32) dma16(arsrc, aoffg[i], (uint32_t)((KT_) * 2 * kTBK), (BUF) + ldsA + 8 * i * kTBK); \
    else dma16(asrc[i] + (KT_) * kTBK, (BUF) + ldsA + 8 * i * kTBK);                              \
  }
#define MOE_DMA_B(BUF, KT_)                                                                        \
  _Pragma("unroll") for (int i = 0; i < BI; ++i) {                                                 \
    if constexpr (NTW) dma16_nt(wrsrc, boffg[i], (uint32_t)((KT_) * WRB), (BUF) + ldsB + (F8 ? 16 : 8) * i * (WRB / 2)); \
    else dma16(wrsrc, boffg[i], (uint32_t)((KT_) * WRB), (BUF) + ldsB + (F8 ? 16 : 8) * i * (WRB / 2)); \
  }
#define MOE_DMA_B1(BUF, KT_, I_)                                                                   \
  if constexpr ((I_) < BI) {                                                                       \
    if constexpr (NTW) dma16_nt(wrsrc, boffg[I_], (uint32_t)((KT_) * WRB), (BUF) + ldsB + (F8 ? 16 : 8) * (I_) * (WRB / 2)); \
    else dma16(wrsrc, boffg[I_], (uint32_t)((KT_) * WRB), (BUF) + ldsB + (F8 ? 16 : 8) * (I_) * (WRB / 2)); \
  }

    // NBLK: this wave's 32-row blocks that hold rows of the group; the
    // others (in the group's last row tile only) are padding, whose
    // multiplications and stores are skipped.  Every wave still issues its
    // loads and meets every barrier.
    auto tile_body = [&](auto nblk_c) __attribute__((always_inline)) {
    constexpr int NBLK = decltype(nblk_c)::value;
    f32x16_t acc[NBLK > 0 ? NBLK : 1][2];
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // the previous tile's last reads of the buffers are done
    lds_barrier();
    if constexpr (RLDS) {
      // BM / 64 waves, one row per lane (padding rows load a live one)
      if (wave < BM / 64) {
        const int r = 64 * wave + lane;
        const int rr = r < nrows ? r : 0;
        if (pa.row_scale) dma4(reinterpret_cast<const int32_t*>(pa.row_scale) + row0 + rr, s_rows + 64 * wave);
        if (pa.out_rows) dma4(pa.out_rows + row0 + rr, s_rows + BM + 64 * wave);
      }
    }
    // issue order: weights of stage 0, tokens of stage 0, then (three weight
    // buffers) the weights of stage 1; none where the previous tile loaded them
    if (!pre) {
      MOE_DMA_B(sb0, 0)
      MOE_DMA_A(sa0, 0)
      if constexpr (NB == 3) { MOE_DMA_B(sb1, min(1, KT - 1)) }
    }

    // Fragments of one 16-wide step of a stage (FA: this wave's live token
    // blocks, FB: its two weight blocks), and the multiplications of a step.
#define MOE_FRAG(FA, FB, ABUF, BBUF, S_)                                                           \
  {                                                                                                \
    _Pragma("unroll") for (int i = 0; i < NBLK; ++i)                                               \
        FA[i] = *reinterpret_cast<const u32x4_t*>((ABUF) + aoff0[S_] + 32 * i * kTBK);            \
    _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                                \
      if constexpr (F8) {                                                                          \
        const uint2 raw_ = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(BBUF) + boff0[S_] + brow0[j] * WRB); \
        FB[j] = e4m3x8_to_bf16x8(raw_.x, raw_.y);                                                  \
      } else {                                                                                     \
        FB[j] = *reinterpret_cast<const u32x4_t*>((BBUF) + boff0[S_] + brow0[j] * kTBK);          \
      }                                                                                            \
    }                                                                                              \
  }
#define MOE_MMA(FA, FB)                                                                            \
  _Pragma("unroll") for (int i = 0; i < NBLK; ++i)                                                 \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(FB[j], FA[i], acc[i][j]);

    // One stage: wait for this wave's reads of the previous stage and its
    // loads of stage KT_ (with three weight buffers the weights of stage
    // KT_+1, issued last, may stay in flight), publish the loads with the
    // barrier, start the tokens of stage KT_+1 into a buffer every wave
    // finished reading before the barrier, then the four 16-wide steps of
    // stage KT_, each followed by one of the wave's loads of the weights of
    // stage KT_+NB-1.  (All seven loads at once after the barrier backed up
    // in the vector L1, whose pending-miss stalls took about half the
    // kernel's time, and the waves' MFMAs waited behind them; one weight load
    // per step: Qwen3-235B-shaped gate+up 1575 -> 1498 us, down 930 -> 887,
    // DeepSeek-V2-shaped gate+up 1209 -> 1170.  Spreading the token loads
    // too was slower, and the non-temporal hint on these loads much slower.)  The steps are pipelined by
    // one across the barrier: the fragments of the last step of a stage are
    // read before the next stage's barrier and multiplied after it, while the
    // fragments of the next stage's first step load, so each wave has
    // multiplications to issue while it waits for its reads; scheduling
    // barriers keep each step's reads beside the previous step's
    // multiplications (left alone, the compiler moved multiplications past
    // the stage barrier and waited there for reads it had just issued).  Past the last
    // stage the loads repeat it (into buffers nobody reads): every step then
    // issues the same loads, without branches, whose merging costs the
    // compiler its knowledge of which buffer a load writes.  The scheduling
    // barrier keeps the loads ahead of the multiplications (left to itself
    // the compiler sinks them to the end of the step, where they overlap
    // nothing).
// Order of one group of a stage: the fragment reads of the next step first,
// then the multiplications of this one (MMA_: the group has them), then its
// weight load (VM_), and nothing moves across the group's end.
#define MOE_ORDER(MMA_, VM_)                                                                       \
  if constexpr (NBLK > 0) {                                                                        \
    __builtin_amdgcn_sched_group_barrier(0x100, NBLK + 2, 0);                                      \
    if constexpr (MMA_) __builtin_amdgcn_sched_group_barrier(0x008, 2 * NBLK, 0);                 \
  }                                                                                                \
  if constexpr (VM_) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                            \
  __builtin_amdgcn_sched_barrier(0);
// DA_ / DB_: the loads of a step (token rows of stage S, weight rows of
// stage S, load I): this tile's, clamped to its last stage (C), or, for
// stages past it, the next tile's first (N).
#define MOE_DMA_AC(BUF, S) MOE_DMA_A(BUF, min((S), KT - 1))
#define MOE_DMA_B1C(BUF, S, I_) MOE_DMA_B1(BUF, min((S), KT - 1), I_)
#define MOE_PSTEPX(ABUF, NABUF, BBUF, NBBUF, KT_, FIRST, DA_, DB_)                                 \
  {                                                                                                \
    MOE_WAIT_LGKM0();                                                                              \
    MOE_WAIT_VM(NB == 3 ? BI : 0);                                                                 \
    __builtin_amdgcn_s_barrier();                                                                  \
    DA_(NABUF, (KT_) + 1)                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                             \
    MOE_FRAG(ga, gb, ABUF, BBUF, 0)                                                                \
    if constexpr (!(FIRST)) { MOE_MMA(fa, fb) }                                                   \
    DB_(NBBUF, (KT_) + NB - 1, 0)                                                                  \
    MOE_ORDER(!(FIRST), BI > 0)                                                                    \
    MOE_FRAG(fa, fb, ABUF, BBUF, 1)                                                                \
    MOE_MMA(ga, gb)                                                                                \
    DB_(NBBUF, (KT_) + NB - 1, 1)                                                                  \
    MOE_ORDER(true, BI > 1)                                                                        \
    MOE_FRAG(ga, gb, ABUF, BBUF, 2)                                                                \
    MOE_MMA(fa, fb)                                                                                \
    DB_(NBBUF, (KT_) + NB - 1, 2)                                                                  \
    MOE_ORDER(true, BI > 2)                                                                        \
    MOE_FRAG(fa, fb, ABUF, BBUF, 3)                                                                \
    MOE_MMA(ga, gb)                                                                                \
    DB_(NBBUF, (KT_) + NB - 1, 3)                                                                  \
    MOE_ORDER(true, BI > 3)                                                                        \
  }
#define MOE_PSTEP(ABUF, NABUF, BBUF, NBBUF, KT_, FIRST) \
  MOE_PSTEPX(ABUF, NABUF, BBUF, NBBUF, KT_, FIRST, MOE_DMA_AC, MOE_DMA_B1C)

    // the loop names each buffer explicitly (see above): stage kt reads token
    // buffer kt % 2 and weight buffer kt % NB, a pattern of period 2 or 6;
    // the remainder continues it step by step
#define MOE_A(I) ((I) % 2 == 0 ? sa0 : sa1)
#define MOE_B(I) ((I) % NB == 0 ? sb0 : (I) % NB == 1 ? sb1 : sb2)
#define MOE_USTEP(U, KT_, FIRST) MOE_PSTEP(MOE_A(U), MOE_A((U) + 1), MOE_B(U), MOE_B((U) + NB - 1), KT_, FIRST)
#define MOE_USTEPX(U, KT_, DA_, DB_) \
  MOE_PSTEPX(MOE_A(U), MOE_A((U) + 1), MOE_B(U), MOE_B((U) + NB - 1), KT_, false, DA_, DB_)
    u32x4_t fa[NBLK > 0 ? NBLK : 1], fb[2], ga[NBLK > 0 ? NBLK : 1], gb[2];
    MOE_USTEP(0, 0, true)
    int kt = 1;
    for (; kt + 5 < KT; kt += 6) {
      MOE_USTEP(1, kt, false)
      MOE_USTEP(2, kt + 1, false)
      MOE_USTEP(3, kt + 2, false)
      MOE_USTEP(4, kt + 3, false)
      MOE_USTEP(5, kt + 4, false)
      MOE_USTEP(6, kt + 5, false)
    }
    constexpr bool pf = PF;
    if constexpr (pf) {
      // The loop ended at stage KT - 5 (phase 1): five stages remain, and
      // stage KT falls on the buffers of a tile's stage 0.  Claim the next
      // tile (published by the next stage's barrier), then load its tokens of
      // stage 0 and weights of stages 0 and 1 where this tile's loads past
      // its end would go.  Without a next tile those loads repeat this
      // tile's first stages, into buffers nobody reads.
      if (tid == 0) *s_next = claim(tk);
      MOE_USTEP(1, kt, false)
      MOE_USTEP(2, kt + 1, false)
      MOE_USTEP(3, kt + 2, false)
      nx = __builtin_amdgcn_readfirstlane(*s_next);
      claimed = true;
      pre_next = nx >= 0;
      __amdgpu_buffer_rsrc_t arN = arsrc, wrN = wrsrc;
      uint32_t aoN[AI], boN[BI];
      const uint16_t* asN[A32 ? 1 : AI];
#pragma unroll
      for (int i = 0; i < AI; ++i) aoN[i] = aoffg[i];
#pragma unroll
      for (int i = 0; i < BI; ++i) boN[i] = boffg[i];
      int ktN = KT;
      if (nx >= 0) {
        int en, r0n, nrn, c0n, rtn;
        tile_geom(nx, en, r0n, nrn, c0n, rtn);
        const FfnArgs& qn = nx < T2 ? p2 : p;
        tile_loads(qn, en, r0n, nrn, c0n, arN, wrN, aoN, asN, boN);
        ktN = qn.K / kTBK;
      }
#define MOE_DMA_AN(BUF, S)                                                                         \
  _Pragma("unroll") for (int i = 0; i < AI; ++i)                                                   \
      dma16(arN, aoN[i], (uint32_t)(min((S) - KT, ktN - 1) * 2 * kTBK), (BUF) + ldsA + 8 * i * kTBK);
#define MOE_DMA_B1N(BUF, S, I_)                                                                    \
  if constexpr ((I_) < BI) {                                                                       \
    if constexpr (NTW) dma16_nt(wrN, boN[I_], (uint32_t)(min((S) - KT, ktN - 1) * WRB), (BUF) + ldsB + (F8 ? 16 : 8) * (I_) * (WRB / 2)); \
    else dma16(wrN, boN[I_], (uint32_t)(min((S) - KT, ktN - 1) * WRB), (BUF) + ldsB + (F8 ? 16 : 8) * (I_) * (WRB / 2)); \
  }
      MOE_USTEPX(4, kt + 3, MOE_DMA_AC, MOE_DMA_B1N)
      MOE_USTEPX(5, kt + 4, MOE_DMA_AN, MOE_DMA_B1N)
#undef MOE_DMA_AN
#undef MOE_DMA_B1N
    } else {
      if (kt < KT) MOE_USTEP(1, kt, false)
      if (kt + 1 < KT) MOE_USTEP(2, kt + 1, false)
      if (kt + 2 < KT) MOE_USTEP(3, kt + 2, false)
      if (kt + 3 < KT) MOE_USTEP(4, kt + 3, false)
      if (kt + 4 < KT) MOE_USTEP(5, kt + 4, false)
    }
    MOE_MMA(fa, fb)                                // the last stage's last step
#undef MOE_USTEP
#undef MOE_USTEPX
#undef MOE_A
#undef MOE_B
#undef MOE_PSTEP
#undef MOE_PSTEPX
#undef MOE_DMA_AC
#undef MOE_DMA_B1C
#undef MOE_ORDER
#undef MOE_FRAG
#undef MOE_MMA
#undef MOE_DMA_A
#undef MOE_DMA_B
    // (after the next tile's loads nothing in flight targets sa1 or sb2,
    // where down stages its output)
    if (!pf) MOE_WAIT_VM(0);

    if constexpr (!GATEUP) {
      // Down: the output goes through LDS so that the stores write whole
      // 128-byte row segments, eight rows per instruction.  Stored straight
      // from the accumulators (16 bytes per row per instruction, over 32
      // rows) it reached HBM as about 1.8x its bytes.  Each wave stages one
      // 32 x 64 block at a time in a 4 KB slot of the token buffers, which
      // every wave has finished reading; 16-byte chunk c of row r sits at
      // c ^ stg_chunk(r) with its 8-byte halves swapped where stg_half(r), so
      // neither the 8-byte writes nor the 16-byte reads conflict.  The rows
      // are read once, after the launch (by the combine), so the stores carry
      // the non-temporal hint and do not displace the weights and h rows
      // that later tiles read again: DeepSeek-V2-shaped down 698 -> 653 us,
      // Qwen3-235B-shaped 829 -> 822 us (flushed, one layer call).  FP8: the
      // per-channel scales of this lane's columns, four at a time.
      constexpr int RB = BM / 2;
      // the scale and output row of this lane's token rows (one per live
      // 32-row block), loaded after the contraction so that they hold no
      // registers during it
      float rsc[NBLK > 0 ? NBLK : 1];
      int orow_i[NBLK > 0 ? NBLK : 1];
#pragma unroll
      for (int i = 0; i < NBLK; ++i) {
        const int row = wm * RB + 32 * i + fr;
        const bool in = row < nrows;
        if constexpr (RLDS) {
          rsc[i] = (pa.row_scale && in) ? __builtin_bit_cast(float, s_rows[row]) : 1.f;
          orow_i[i] = (pa.out_rows && in) ? s_rows[BM + row] : row0 + row;
        } else {
          rsc[i] = (pa.row_scale && in) ? pa.row_scale[row0 + row] : 1.f;
          orow_i[i] = (pa.out_rows && in) ? pa.out_rows[row0 + row] : row0 + row;
        }
      }
      lds_barrier();
      // Staging slots of 32 x 64 bf16 (4 KB) per wave.  PF: the next tile's
      // first stages are in flight into sa0, sb0 and sb1, so the slots are in
      // sb2 (free once the last stage is read) where its bf16 weight stages
      // hold all eight (32 KB); FP8 weight stages hold four (16 KB), and the
      // other four waves use sa1.  (A choice of two buffers leaves the
      // compiler waiting for every load in flight before the first staging
      // write, so bf16 keeps to one.)
      constexpr int kSlot = 32 * 64;
      constexpr bool STAGE_B2 = PFC && STB >= 8 * kSlot;
      static_assert(STA >= 4 * kSlot && (NB != 3 || STB >= 4 * kSlot), "four staging slots per buffer");
      uint16_t* blk = STAGE_B2 ? sb2 + wave * kSlot
                    : PFC      ? (wave < 4 ? sa1 : sb2) + (wave & 3) * kSlot
                               : (wave < 4 ? sa0 : sa1) + (wave & 3) * kSlot;
      const int c = col0 + wn * 64;
      float4 sc4[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          sc4[j][b] = (F8 && c < ncols) ? *reinterpret_cast<const float4*>(pa.s0 + (size_t)e * ncols + c + 32 * j + 8 * b + 4 * fg)
                                : make_float4(1.f, 1.f, 1.f, 1.f);
      const int ch = lane & 7;
#pragma unroll
      for (int i = 0; i < FMW; ++i) {
        if (i >= NBLK) break;                  // padding rows only
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const f32x16_t& a0 = acc[i][j];
            const float4 g = sc4[j][b];
            const uint2 v = make_uint2(pack_bf16x2(a0[4 * b] * g.x * rsc[i], a0[4 * b + 1] * g.y * rsc[i]),
                                       pack_bf16x2(a0[4 * b + 2] * g.z * rsc[i], a0[4 * b + 3] * g.w * rsc[i]));
            *reinterpret_cast<uint2*>(blk + fr * 64 + (((4 * j + b) ^ stg_chunk(fr)) << 3) +
                                      4 * (fg ^ stg_half(fr))) = v;
          }
        __builtin_amdgcn_wave_barrier();       // a wave's LDS operations complete in order
        if (c < ncols) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int r = 8 * t + (lane >> 3);
            uint4 v = *reinterpret_cast<const uint4*>(blk + r * 64 + ((ch ^ stg_chunk(r)) << 3));
            if (stg_half(r)) v = make_uint4(v.z, v.w, v.x, v.y);    // (t & 1: known at compile time)
            const int orow = __shfl(orow_i[i], r);
            if (wm * RB + 32 * i + r < nrows)
              __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w},
                                          reinterpret_cast<u32x4_t*>(pa.out + (size_t)orow * ncols + c + ch * 8));
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
      return;
    }

    // Gate+up.  acc[i][0] and acc[i][1] hold the gate and up sums of the same
    // 32 h columns: this lane's token row is 32 i + (lane & 31) of the wave's
    // half, and element 4 b + q is column 8 b + 4 (lane >> 5) + q, so every
    // lane stores four consecutive h columns (8 bytes) at a time.  Column
    // groups of four lie wholly inside or outside ncols (a multiple of 64).
    // FP8: the per-channel scales of those columns, four at a time.
    if constexpr (GATEUP) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int c = col0 + wn * 32 + 8 * b + 4 * fg;
        if (c >= ncols) continue;
        float4 sg = make_float4(1.f, 1.f, 1.f, 1.f), su = sg;
        if constexpr (F8) {
          sg = *reinterpret_cast<const float4*>(pa.s0 + (size_t)e * ncols + c);
          su = *reinterpret_cast<const float4*>(pa.s1 + (size_t)e * ncols + c);
        }
        const float gs[4] = {sg.x, sg.y, sg.z, sg.w}, us[4] = {su.x, su.y, su.z, su.w};
#pragma unroll
        for (int i = 0; i < NBLK; ++i) {
          const int row = wm * (BM / 2) + 32 * i + fr;
          if (row >= nrows) continue;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g = acc[i][0][4 * b + q] * gs[q], u = acc[i][1][4 * b + q] * us[q];
            v[q] = silu_mul(g, u);
          }
          *reinterpret_cast<uint2*>(pa.out + (size_t)(row0 + row) * ncols + c) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
    }
    };
    // one instance of the contraction and epilogue per count of live blocks,
    // so that no accumulator is merged across them
    // Padding blocks are skipped in every tile.  A group's row tiles differ
    // by one 32-row block at most (row_tile), so the tiles that share its
    // weights stay in step; with full tiles and one short last tile, the
    // short one ran ahead of them, each fetched the weights again, and
    // gate+up skipped padding in one-tile groups only.  Balanced tiles with
    // the skip: Qwen3-235B-shaped gate+up 1541 -> 1462 us (padding MFMA work
    // 1.18x -> about 1.03x of the algorithmic), DeepSeek-V2-shaped down
    // 751 -> 723 us.
    const int live = nrows - wm * (BM / 2);
    const int nblk = live <= 0 ? 0 : min(FMW, ceil_div(live, 32));
    if (nblk == FMW) {
      tile_body(std::integral_constant<int, FMW>{});
    } else if (nblk == 0) {
      tile_body(std::integral_constant<int, 0>{});
    } else if (nblk == 1) {
      tile_body(std::integral_constant<int, 1>{});
    } else if constexpr (FMW >= 3) {
      if (nblk == 2) tile_body(std::integral_constant<int, 2>{});
      else if constexpr (FMW >= 4) tile_body(std::integral_constant<int, 3>{});
    }
    if (dyn) {
      // every wave read this tile's ticket before the tile's barriers
      if (claimed) {
        next = nx;                             // claimed in the last stages
      } else {
        if (tid == 0) *s_ticket = claim(tk);
        lds_barrier();
        next = *s_ticket;
      }
    }
    tile = __builtin_amdgcn_readfirstlane(next);
    pre = pre_next;
  }
  MOE_WAIT_VM(0);                                // loads past the last tile land before the block ends
}
#undef MOE_WAIT_VM
#undef MOE_WAIT_LGKM0

// ================================ launchers =================================

template <int FM, bool GATEUP, bool F8, bool NTL, int LA = 2>
hipError_t launch_stream_nt(const FfnArgs& a, hipStream_t st) {
  // down: four 16-row groups per wave at 16 rows per pass, else three, where
  // the columns divide evenly and two blocks still fit a CU's LDS.  Fewer,
  // longer blocks pay off on short weight rows: Qwen3-30B-shaped down (1.5 KB
  // rows) at 8 / 32 / 128 tokens took 40.0 / 74.6 / 85.0 us with two groups
  // per wave and 39.0 / 73.0 / 81.1 us with four.
  const bool nm4 = !GATEUP && FM == 1 && a.ncols % (4 * 4 * kSCols) == 0;
  const bool nm3 = !GATEUP && FM <= 3 && a.ncols % (4 * 3 * kSCols) == 0;
  // FP8 gate+up: eight waves per block where the columns divide evenly
  constexpr int NWG = (GATEUP && F8) ? 8 : 4;
  const bool w8 = NWG == 8 && a.ncols % (8 * kSCols) == 0;
  const int NT = a.ncols / ((w8 ? 8 : 4) * kSCols * (GATEUP ? 1 : (nm4 ? 4 : nm3 ? 3 : 2)));
  const long groups = a.E < a.rows_total ? a.E : a.rows_total;   // non-empty groups, at most
  const long passes = a.rows_total / (FM * 16) + groups;          // >= sum of ceil(count / rows per pass)
  const long grid = passes * NT;
  if (grid <= 0) return hipSuccess;
  if constexpr (!GATEUP && FM == 1) {
    if (nm4) {
      hipLaunchKernelGGL((ffn_stream_kernel<FM, GATEUP, LA, 4, F8, 4, NTL>), dim3((unsigned)grid), dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
  if constexpr (!GATEUP && FM <= 3) {
    if (nm3) {
      hipLaunchKernelGGL((ffn_stream_kernel<FM, GATEUP, LA, 3, F8, 4, NTL>), dim3((unsigned)grid), dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
  if constexpr (NWG == 8) {
    if (w8) {
      hipLaunchKernelGGL((ffn_stream_kernel<FM, GATEUP, LA, 2, F8, 8, NTL>), dim3((unsigned)grid), dim3(512), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((ffn_stream_kernel<FM, GATEUP, LA, 2, F8, 4, NTL>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Non-temporal weight loads for gate+up always, for down from 8 KB rows on
// (where the measurements favour them).
template <int FM, bool GATEUP, bool F8>
hipError_t launch_stream(const FfnArgs& a, hipStream_t st) {
  if constexpr (GATEUP) {
    return launch_stream_nt<FM, GATEUP, F8, true>(a, st);
  } else {
    const long row_bytes = (long)a.K * (F8 ? 1 : 2);
    return row_bytes >= 8192 ? launch_stream_nt<FM, GATEUP, F8, true>(a, st)
                             : launch_stream_nt<FM, GATEUP, F8, false>(a, st);
  }
}

template <bool GATEUP, int BM, bool F8, bool A32 = true>
hipError_t launch_tile_bm(const FfnArgs& a, const FfnArgs& a2, int num_cu, hipStream_t st) {
  constexpr int HC = GATEUP ? kTN / 2 : kTN;
  const int NT = ceil_div(a.ncols, HC);
  const long ub_rows = a.rows_total / BM + (a.E < a.rows_total ? a.E : a.rows_total);
  const long ub = ub_rows * NT + (a2.E > 0 ? (long)ceil_div(a2.fixed_rows, BM) * ceil_div(a2.ncols, HC) : 0);
  long grid = (num_cu / 8) * 8;
  if (ub < grid) grid = ((ub + 7) / 8) * 8;
  if (grid <= 0) return hipSuccess;
  // every tile launch but 256-row bf16 tiles takes its tiles from a queue
  if (!(BM == 256 && !F8)) {
    if (a.queue == nullptr) return hipErrorInvalidValue;
    if (!a.queue_zeroed) {
      if (hipError_t e = launch_zero_words(a.queue, kQueueWords, st)) return e;
    }
  }
  // down with every segment's contraction a multiple of six 64-wide stages
  // (expert widths of 384 m, as 1536): the next-tile loads
  // Where a typical group fits one row tile (mean rows per group <= BM), no
  // later tile reads its bf16 weight rows again, and they are loaded with the
  // non-temporal hint, which leaves L2 to the h rows that every column tile
  // reads: DeepSeek-V2-shaped down (mean 154 rows, 192-row tiles) 654 ->
  // 628 us.  Groups several tiles deep lose by it (Qwen3-235B-shaped down
  // 830 -> 862 us), as their row tiles share each weight tile through L2,
  // and so do FP8 weights (DeepSeek-V2-shaped FP8 down 545 -> 605 us).
  if constexpr (!GATEUP && A32 && BM < 256) {
    constexpr int kStages6 = 6 * kTBK;
    if (a.K % kStages6 == 0 && (a2.E == 0 || a2.K % kStages6 == 0)) {
      if constexpr (!F8) {
        if (a.rows_total <= (long)BM * a.E) {
          hipLaunchKernelGGL((ffn_tile_kernel<GATEUP, BM, F8, A32, true, true>), dim3((unsigned)grid), dim3(512), 0, st, a, a2);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((ffn_tile_kernel<GATEUP, BM, F8, A32, true>), dim3((unsigned)grid), dim3(512), 0, st, a, a2);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((ffn_tile_kernel<GATEUP, BM, F8, A32, false>), dim3((unsigned)grid), dim3(512), 0, st, a, a2);
  return hipGetLastError();
}

// Bytes of a segment's token matrix, or ~0 where its row count is not known.
unsigned long long token_bytes(const FfnArgs& a) {
  if (a.a_rows != nullptr && a.a_nrows <= 0) return ~0ull;
  const long long rows = a.a_rows != nullptr ? a.a_nrows : a.rows_total;
  return (unsigned long long)rows * (unsigned long long)a.K * 2ull;
}

// Tile height from the mean rows per group.  128 rows where 1.25x the mean
// fits one such tile, 192 where it fits that, and 192 also up to a mean of
// 640: a group pads about half a tile on average (96 rows against 128),
// which outweighs the shorter tile's lower efficiency per row until the
// groups are several tiles deep (and 192-row tiles keep their weight rows
// two stages ahead, which 256-row tiles have no LDS for).  Measured: a
// 256-row tile over 154-row groups wastes 40% of its MFMA work (DeepSeek-V2-
// shaped layer 2.91 -> 2.63 ms with 192); Qwen3-235B-shaped groups (mean 512)
// 3.47 -> 3.30 ms with 192 (FP8 weights 3.15 -> 2.95 ms); the expert-node
// share (mean 2048) is 1-2% faster with 256.
// a2: an optional single-group segment (a2.E == 1, a2.fixed_rows rows) run
// in the same launch, with the tile height chosen for a.
template <bool GATEUP, bool F8>
hipError_t launch_tile(const FfnArgs& a_in, const FfnArgs& a2_in, int num_cu, hipStream_t st) {
  FfnArgs a = a_in, a2 = a2_in;
  const unsigned long long tb = token_bytes(a), tb2 = a2.E > 0 ? token_bytes(a2) : 0;
  if (tb > kA32Limit || tb2 > kA32Limit) return launch_tile_bm<GATEUP, 128, F8, false>(a, a2, num_cu, st);
  a.a_bytes = (uint32_t)tb;
  a2.a_bytes = (uint32_t)tb2;
  const double mean = (double)a.rows_total / (a.E > 0 ? a.E : 1);
  if (1.25 * mean <= 128.0) return launch_tile_bm<GATEUP, 128, F8>(a, a2, num_cu, st);
  if (1.25 * mean <= 192.0 || mean <= 640.0) return launch_tile_bm<GATEUP, 192, F8>(a, a2, num_cu, st);
  return launch_tile_bm<GATEUP, 256, F8>(a, a2, num_cu, st);
}

// The split-contraction decode kernel pays off only when the plain streaming
// launch would have too few blocks to keep every CU streaming.  Gate+up:
// below 1024 blocks (measured: it helps at 1 and 8 tokens, 65 against 71 us
// on the Qwen3-30B shape at 8, and loses at 32 tokens).  Down: below 256, one
// per CU (Qwen3-30B shape: at 4 tokens the plain down launch takes 25.4
// against 31.4 us, at 2 tokens 19.9 against 20.5, at 1 token 18.6 against
// 12.2 us for the split one).
bool use_split_waves(const FfnArgs& a, bool gateup) {
  const long groups = a.E < a.rows_total ? a.E : a.rows_total;
  const long blocks = groups * (a.ncols / (4 * kSCols * (gateup ? 1 : 2)));
  return blocks < (gateup ? 1024 : 256);
}

template <bool GATEUP, bool F8>
hipError_t launch_stream_ks(const FfnArgs& a, hipStream_t st) {
  const int NT = a.ncols / (GATEUP ? kSCols : 2 * kSCols);
  const long groups = a.E < a.rows_total ? a.E : a.rows_total;
  const long grid = (a.rows_total / 16 + groups) * NT;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((ffn_stream_ks_kernel<GATEUP, F8>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Mean rows per group decides the kernel; the streaming kernel's pass height
// covers ~1.2x the mean so that typical groups take one pass; above 56 mean
// rows the tile kernel takes over (bf16 and FP8 weights alike).
int stream_fm(const FfnArgs& a, bool gateup) {
  const bool f8 = a.q0 != nullptr;
  if (a.K % (f8 ? 2 * kSK : kSK) != 0 || a.ncols % (4 * kSCols * (gateup ? 1 : 2)) != 0) return 0;
  const double mean = (double)a.rows_total / (a.E > 0 ? a.E : 1);
  if (mean > 56.0) return 0;
  const double need = mean * 1.2;
  if (need <= 16.0) return 1;
  if (need <= 32.0) return 2;
  if (need <= 48.0) return 3;
  return 4;
}

template <bool GATEUP, bool F8>
hipError_t launch_ffn(const FfnArgs& a, int num_cu, hipStream_t st) {
  switch (stream_fm(a, GATEUP)) {
    case 1:
      return use_split_waves(a, GATEUP) ? launch_stream_ks<GATEUP, F8>(a, st) : launch_stream<1, GATEUP, F8>(a, st);
    case 2: return launch_stream<2, GATEUP, F8>(a, st);
    case 3: return launch_stream<3, GATEUP, F8>(a, st);
    case 4: return launch_stream<4, GATEUP, F8>(a, st);
    default: break;
  }
  return launch_tile<GATEUP, F8>(a, FfnArgs{}, num_cu, st);
}

// Routed groups and the shared experts (one group of all rows): one tile
// launch when both take the tile kernel with the same weight type, else the
// shared launch and then the routed one.
template <bool GATEUP>
hipError_t launch_ffn_with_shared(const FfnArgs& routed, const FfnArgs& shared, int num_cu, hipStream_t st) {
  const bool f8 = routed.q0 != nullptr;
  if (routed.rows_total > 0 && f8 == (shared.q0 != nullptr) && stream_fm(routed, GATEUP) == 0 &&
      stream_fm(shared, GATEUP) == 0) {
    return f8 ? launch_tile<GATEUP, true>(routed, shared, num_cu, st)
              : launch_tile<GATEUP, false>(routed, shared, num_cu, st);
  }
  if (shared.rows_total > 0) {
    const hipError_t e = shared.q0 ? launch_ffn<GATEUP, true>(shared, num_cu, st)
                                   : launch_ffn<GATEUP, false>(shared, num_cu, st);
    if (e != hipSuccess) return e;
  }
  if (routed.rows_total == 0) return hipSuccess;
  return f8 ? launch_ffn<GATEUP, true>(routed, num_cu, st) : launch_ffn<GATEUP, false>(routed, num_cu, st);
}

}  // namespace

hipError_t launch_ffn_gateup(const FfnArgs& a, int num_cu, hipStream_t st) {
  if (a.rows_total == 0) return hipSuccess;
  return a.q0 ? launch_ffn<true, true>(a, num_cu, st) : launch_ffn<true, false>(a, num_cu, st);
}

hipError_t launch_ffn_down(const FfnArgs& a, int num_cu, hipStream_t st) {
  if (a.rows_total == 0) return hipSuccess;
  return a.q0 ? launch_ffn<false, true>(a, num_cu, st) : launch_ffn<false, false>(a, num_cu, st);
}

hipError_t launch_ffn_gateup_shared(const FfnArgs& routed, const FfnArgs& shared, int num_cu, hipStream_t st) {
  return launch_ffn_with_shared<true>(routed, shared, num_cu, st);
}

hipError_t launch_ffn_down_shared(const FfnArgs& routed, const FfnArgs& shared, int num_cu, hipStream_t st) {
  return launch_ffn_with_shared<false>(routed, shared, num_cu, st);
}

}  // namespace moe
