// Streaming pieces shared by the grouped SwiGLU kernels and the
// single-launch decode layer: weight-row chunk constants, FP8 widening, MFMA
// weight fragments from a wave's LDS slot, weight loads, and the
// split-contraction tile.
#pragma once
#include "ffn_common.h"

namespace moe {

constexpr int kSK = 128;     // 16-bit elements per 256-byte weight-row chunk
constexpr int kSCols = 16;   // output columns per wave
constexpr int kRowBytes = 256;

// Eight E4M3 codes (the bytes of lo, then hi, in k order) -> eight bf16.
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return r;
}

// B fragment of MFMA sub-step s from a wave's 16-row weight slot (256 bytes
// per row, 16-byte piece c of row r at piece c ^ r): lane l supplies row
// l & 15 and the eight contraction elements 8 (l >> 4) .. +7 of the step.
template <bool F8>
__device__ __forceinline__ u32x4_t weight_fragment(const uint16_t* slot, int s, int lane) {
  const int fr = lane & 15, g = lane >> 4;
  if constexpr (F8) {
    const int piece = 2 * s + (g >> 1);          // bytes 32 s + 8 g of the row
    const uint8_t* p = reinterpret_cast<const uint8_t*>(slot) + fr * kRowBytes + ((piece ^ fr) << 4) + ((g & 1) << 3);
    const uint2 raw = *reinterpret_cast<const uint2*>(p);
    return e4m3x8_to_bf16x8(raw.x, raw.y);
  } else {
    const int piece = 4 * s + g;
    return *reinterpret_cast<const u32x4_t*>(slot + fr * kSK + ((piece ^ fr) << 3));
  }
}

// FP8 weights, two MFMA sub-steps at a time.  Within a chunk the order in
// which contraction elements meet the MFMA is free as long as the token-row
// fragments follow it, so sub-steps 2 s2 and 2 s2 + 1 give lane group g the
// 16 contraction elements 64 s2 + 16 g .. +15: its codes are one 16-byte
// piece of the slot row (piece 4 s2 + g, read at (4 s2 + g) ^ row), the low
// eight for the first sub-step and the high eight for the second, and its
// token-row pieces (8 bf16 each) are 8 s2 + 2 g and 8 s2 + 2 g + 1.  One
// 128-bit LDS read serves two sub-steps, and a 16-lane group of it touches 16
// different pieces of 16 rows, like the bf16 fragments (the 64-bit reads of
// one sub-step at a time hit LDS bank conflicts: measured 65% of the
// LDS-active cycles of the FP8 gate+up launch).
__device__ __forceinline__ void weight_pair_f8(const uint16_t* slot, int s2, int lane, u32x4_t& lo, u32x4_t& hi) {
  const int fr = lane & 15, q = 4 * s2 + (lane >> 4);
  const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(slot) + fr * kRowBytes +
                                                    ((q ^ fr) << 4));
  lo = e4m3x8_to_bf16x8(raw.x, raw.y);
  hi = e4m3x8_to_bf16x8(raw.z, raw.w);
}

// 16 bytes of a weight row.  NTL marks the load non-temporal: every weight
// byte is read once per launch, and the hint keeps it from pushing the token
// rows and h out of the caches.  Measured: gate+up streams 4-6% faster with
// it at every shape tried; down gains 6-9% once a row is 8 KB or longer and
// loses up to 18% on short rows (1.5 KB).
template <bool NTL, class T>
__device__ __forceinline__ T load_weight(const uint8_t* q) {
  if constexpr (NTL) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(q));
    T r;
    __builtin_memcpy(&r, &v, sizeof(T));
    return r;
  } else {
    return *reinterpret_cast<const T*>(q);
  }
}

// Split-contraction tile (at most 16 rows per pass): the four waves of a
// block share one 16-row x WCOLS output tile and split the contraction four
// ways, so a batch of a few tokens still spreads over hundreds of blocks.
// Each wave stages its own token rows and weight rows in private LDS slots,
// so the k loop has no block barrier; the four partial tiles are summed in
// wave order through LDS at the end (deterministic).  `tile` indexes the
// tile list s_off / s_tp (build_tile_list with 16 rows per tile); rot_key
// picks the chunk each wave's walk starts at.  Every thread of the block
// calls it with the same tile.
template <bool F8>
struct KsLds {
  static constexpr int KC = F8 ? 2 * kSK : kSK;
  uint16_t sa[4][16 * KC];
  uint16_t sb[4][2][kSCols * kSK];
};

template <bool GATEUP, bool F8>
__device__ __forceinline__ void ks_tile(const FfnArgs& p, const int* s_off, const int* s_tp, int tile,
                                        unsigned rot_key, KsLds<F8>& lds) {
  constexpr int RB = 16;
  constexpr int KC = F8 ? 2 * kSK : kSK;     // contraction elements per chunk
  constexpr int ACH = KC / 8;                // 16-byte pieces of a token row per chunk
  constexpr int AI = RB * ACH / 64;          // token-row loads per lane per chunk
  constexpr int NSUB = KC / 32;
  constexpr int WCOLS = GATEUP ? kSCols : 2 * kSCols;   // output columns per block
  constexpr int LA = 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, ncols = p.ncols;
  const int NC = K / KC;                      // the host sends only K % KC == 0 here
  const int c0 = (wave * NC) / 4, c1 = ((wave + 1) * NC) / 4;   // this wave's chunks
  const int e = find_group(s_tp, p.E, tile);
  const int cnt = s_off[e + 1] - s_off[e];
  const int RT = ceil_div(cnt, RB);
  const int local = tile - s_tp[e];
  const int ct = local / RT, rt = local - ct * RT;
  const int row0 = s_off[e] + rt * RB;
  const int nrows = min(RB, cnt - rt * RB);
  const int col0 = ct * WCOLS;

  const int brow = lane >> 4, bch = lane & 15, fr = lane & 15;
  const size_t RP = (size_t)K * (F8 ? 1 : 2);                 // weight row pitch in bytes
  const uint8_t* w0b = F8 ? p.q0 : reinterpret_cast<const uint8_t*>(p.w0);
  const uint8_t* w1b = F8 ? p.q1 : reinterpret_cast<const uint8_t*>(p.w1);
  const size_t wrow = ((size_t)e * ncols + col0 + brow) * RP + bch * 16;
  const uint8_t* wb0 = w0b + wrow;
  const uint8_t* wb1 = GATEUP ? w1b + wrow : wb0 + (size_t)kSCols * RP;
  int bdst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + brow;
    bdst[i] = r * kSK + ((bch ^ r) << 3);
  }
  // token rows: load i of a lane covers row (64 / ACH) i + lane / ACH, piece lane % ACH
  uint32_t aoff[AI];
  int adst[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = (64 / ACH) * i + lane / ACH, ch = lane % ACH;
    const int rr = (r < nrows) ? r : 0;
    const int grow = p.a_rows ? p.a_rows[row0 + rr] : (row0 + rr);
    aoff[i] = (uint32_t)grow * (uint32_t)K + ch * 8;
    adst[i] = r * KC + ((ch ^ (r & 15)) << 3);
  }
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

  if (c0 < c1) {
    // the wave walks its chunks starting at a block-dependent one (wrapping),
    // so that concurrent blocks spread over the weight rows' offsets
    const int L = c1 - c0;
    const int rot = (int)(rot_key % (unsigned)L);
    auto kc = [c0, L, rot](int j) {
      const int jj = j + rot;
      return c0 + (jj >= L ? jj - L : jj);
    };
    // prologue: chunk 0 of the walk into LDS, chunks 1..LA into registers
    {
      const int k0 = kc(0);
#pragma unroll
      for (int i = 0; i < AI; ++i)
        *reinterpret_cast<uint4*>(&lds.sa[wave][adst[i]]) = *reinterpret_cast<const uint4*>(p.a + aoff[i] + k0 * KC);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4*>(&lds.sb[wave][0][bdst[i]]) = *reinterpret_cast<const uint4*>(wb0 + 4 * i * RP + k0 * kRowBytes);
        *reinterpret_cast<uint4*>(&lds.sb[wave][1][bdst[i]]) = *reinterpret_cast<const uint4*>(wb1 + 4 * i * RP + k0 * kRowBytes);
      }
    }
    uint4 qa[LA][AI], qb[LA][2][4];
#pragma unroll
    for (int l = 0; l < LA; ++l) {
      const int kk = kc(min(1 + l, L - 1));
#pragma unroll
      for (int i = 0; i < AI; ++i) qa[l][i] = *reinterpret_cast<const uint4*>(p.a + aoff[i] + kk * KC);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qb[l][0][i] = *reinterpret_cast<const uint4*>(wb0 + 4 * i * RP + kk * kRowBytes);
        qb[l][1][i] = *reinterpret_cast<const uint4*>(wb1 + 4 * i * RP + kk * kRowBytes);
      }
    }
    for (int c = 0; c < L; ++c) {
      if constexpr (F8) {
#pragma unroll
        for (int s2 = 0; s2 < NSUB / 2; ++s2) {
          u32x4_t b0[2], b1[2];
          weight_pair_f8(&lds.sb[wave][0][0], s2, lane, b0[0], b0[1]);
          weight_pair_f8(&lds.sb[wave][1][0], s2, lane, b1[0], b1[1]);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int ch = 8 * s2 + 2 * (lane >> 4) + h;
            const u32x4_t af = *reinterpret_cast<const u32x4_t*>(&lds.sa[wave][fr * KC + ((ch ^ fr) << 3)]);
            acc0 = mfma16(af, b0[h], acc0);
            acc1 = mfma16(af, b1[h], acc1);
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          const int ch = s * 4 + (lane >> 4);
          const u32x4_t af = *reinterpret_cast<const u32x4_t*>(&lds.sa[wave][fr * KC + ((ch ^ fr) << 3)]);
          acc0 = mfma16(af, weight_fragment<F8>(&lds.sb[wave][0][0], s, lane), acc0);
          acc1 = mfma16(af, weight_fragment<F8>(&lds.sb[wave][1][0], s, lane), acc1);
        }
      }
      // same wave: LDS operations complete in order, so the slot can be
      // overwritten right after this wave's reads
#pragma unroll
      for (int i = 0; i < AI; ++i) *reinterpret_cast<uint4*>(&lds.sa[wave][adst[i]]) = qa[0][i];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4*>(&lds.sb[wave][0][bdst[i]]) = qb[0][0][i];
        *reinterpret_cast<uint4*>(&lds.sb[wave][1][bdst[i]]) = qb[0][1][i];
      }
#pragma unroll
      for (int l = 0; l + 1 < LA; ++l) {
#pragma unroll
        for (int i = 0; i < AI; ++i) qa[l][i] = qa[l + 1][i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qb[l][0][i] = qb[l + 1][0][i];
          qb[l][1][i] = qb[l + 1][1][i];
        }
      }
      const int kk = kc(min(c + 1 + LA, L - 1));
#pragma unroll
      for (int i = 0; i < AI; ++i) qa[LA - 1][i] = *reinterpret_cast<const uint4*>(p.a + aoff[i] + kk * KC);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qb[LA - 1][0][i] = *reinterpret_cast<const uint4*>(wb0 + 4 * i * RP + kk * kRowBytes);
        qb[LA - 1][1][i] = *reinterpret_cast<const uint4*>(wb1 + 4 * i * RP + kk * kRowBytes);
      }
    }
  }

  // partial tiles -> LDS (reusing the weight slots), summed in wave order
  __syncthreads();
  float* red = reinterpret_cast<float*>(&lds.sb[0][0][0]);   // [4 waves][64 lanes][8]
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
    float w0s = 1.f, w1s = 1.f;
    if constexpr (F8) {
      const size_t ch = (size_t)e * ncols + col;
      w0s = p.s0[ch];
      w1s = GATEUP ? p.s1[ch] : p.s0[ch + kSCols];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = (lane >> 4) * 4 + q;
      if (r >= nrows) continue;
      const int orow = row0 + r;
      if (GATEUP) {
        const float g = v[q] * w0s, u = v[4 + q] * w1s;
        p.out[(size_t)orow * ncols + col] = f32_to_bf16(silu_mul(g, u));
      } else {
        const float sc = p.row_scale ? p.row_scale[orow] : 1.f;
        const size_t dst = (size_t)(p.out_rows ? p.out_rows[orow] : orow) * ncols + col;
        p.out[dst] = f32_to_bf16(v[q] * w0s * sc);
        p.out[dst + kSCols] = f32_to_bf16(v[4 + q] * w1s * sc);
      }
    }
  }
  // the slots (and the partial tiles in them) are free again for the next tile
  __syncthreads();
}

}  // namespace moe
