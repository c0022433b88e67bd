// Internal launchers of the MoE FFN layer's kernels (not part of the C ABI).
// Every launcher enqueues on `st` and returns the launch status; shapes have
// been validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct PermuteArgs;
struct RouteArgs {
  const uint16_t* x;         // [N][M]
  const uint16_t* w_router;  // [M][E]
  const float* bias;         // [E] or null
  int N, M, E, k;
  int32_t* ids;              // [N][k]
  float* weights;            // [N][k]
  // optional, where route_permutes(N): the dispatch and permutation of the
  // routed ids (perm->ids and perm->weights are ids and weights), done by
  // the top-k launch
  const PermuteArgs* perm = nullptr;
};
size_t route_workspace_bytes(int N, int M, int E);
// Batches of at most four tokens: the top-k launch (one block) also permutes.
bool route_permutes(int N);
hipError_t launch_route(const RouteArgs& a, void* ws, hipStream_t st);

// Dispatch + stable permutation.  Tiles of kPermTile assignments.
constexpr int kPermTile = 256;
struct PermuteArgs {
  const int32_t* ids;        // [A] expert of assignment a
  int A, E, k;
  int32_t* counts;           // [E]
  int32_t* offsets;          // [E+1]
  int32_t* s2a;              // [A]
  int32_t* a2s;              // [A]
  int32_t* row_token;        // [A] token of sorted row p (= s2a[p] / k), or null
  const float* weights;      // [A] routing weight per assignment, or null
  float* row_weight;         // [A] weight in sorted order, or null
  int32_t* tile_hist;        // [E][T] workspace
  int32_t* tile_off;         // [E][T] workspace
  int32_t* zero = nullptr;   // n_zero ints set to zero on the way (the expert GEMMs' tile queues)
  int n_zero = 0;
};
// n ints of device memory set to zero (one small launch)
hipError_t launch_zero_words(int32_t* p, int n, hipStream_t st);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t st);

// x_sorted[p] = x[row_token[p]] or x[s2a[p] / k]
hipError_t launch_gather(const uint16_t* x, const int32_t* s2a, int k, int A, int M, uint16_t* xs,
                         hipStream_t st);

// One phase of the grouped SwiGLU.  Rows of group e are
// [offsets[e], offsets[e+1]) (or [0, fixed_rows) with E = 1 if fixed_rows > 0).
struct FfnArgs {
  // phase 1 (gate+up): A rows from `a` ([rows][K]); if a_rows is set, row p
  // of the group reads a[a_rows[p]].  phase 2 (down): A = h, in sorted order
  // (a_rows is ignored).
  const uint16_t* a;
  const int32_t* a_rows;
  const int32_t* offsets;    // [E+1] device, or null with fixed_rows > 0
  int fixed_rows;
  const uint16_t* w0;        // gate [E][H][M] | down [E][M][H]
  const uint16_t* w1;        // up   [E][H][M] | unused
  const float* row_scale;    // phase 2: [rows] fp32 or null
  uint16_t* out;             // phase 1: h [rows][H]; phase 2: y [rows][M]
  int E;                     // groups
  int rows_total;            // upper bound on rows (N*k)
  int K;                     // contraction: M (phase 1) | H (phase 2)
  int ncols;                 // output columns: H (phase 1) | M (phase 2)
  // phase 2: if set, sorted row p is stored as row out_rows[p] of `out` (a
  // token row of the layer output: top-1 routing without shared experts
  // needs no combine)
  const int32_t* out_rows = nullptr;
  // rows of `a` where a_rows is set (0: not known); a launcher sets a_bytes
  // to the bytes of `a` when they fit 32-bit offsets
  int a_nrows = 0;
  uint32_t a_bytes = 0;
  // FP8 weights: if q0 is set, w0/w1 are unused and q0/q1 hold OCP E4M3
  // codes laid out like them; s0/s1 [E][ncols] are the float32 scales of
  // each output channel (weight = value(code) * scale)
  const uint8_t* q0 = nullptr;
  const uint8_t* q1 = nullptr;
  const float* s0 = nullptr;
  const float* s1 = nullptr;
  // eight tile counters of the tile kernel's queues (device, kQueueWords
  // ints), or null for static dealing; queue_zeroed: they are zero when the
  // launch starts (else the launcher clears them first)
  int32_t* queue = nullptr;
  bool queue_zeroed = false;
};
constexpr int kQueueWords = 8;
hipError_t launch_ffn_gateup(const FfnArgs& a, int num_cu, hipStream_t st);
hipError_t launch_ffn_down(const FfnArgs& a, int num_cu, hipStream_t st);
// The routed groups together with the shared experts (shared: E = 1,
// fixed_rows = N): one launch where both take the tile kernel, else two.
hipError_t launch_ffn_gateup_shared(const FfnArgs& routed, const FfnArgs& shared, int num_cu, hipStream_t st);
hipError_t launch_ffn_down_shared(const FfnArgs& routed, const FfnArgs& shared, int num_cu, hipStream_t st);

// Per-row OCP E4M3 quantisation: scale[r] = max_k |w[r][k]| / 448 (1 for a
// zero row), q[r][k] = E4M3 nearest to w[r][k] / scale[r], ties to even,
// saturating.  cols % 8 == 0.
hipError_t launch_quantize_fp8(const uint16_t* w, long long rows, int cols, uint8_t* q, float* scale,
                               hipStream_t st);

// Single-launch layer for decode-sized batches (decode.hip): router, top-k,
// permutation, grouped SwiGLU and combine in one cooperative launch with
// grid-wide barriers.  Weights are bf16 (w_*) or FP8 codes with scales
// (q_*, s_*).  ws holds decode_workspace_bytes(N, M, E) bytes; h and y are
// [N*k][H] and [N*k][M].
constexpr int kDecodeTokens = 8;
constexpr int kDecodeAssign = 64;
constexpr int kDecodeMaxBlocks = 1024;
constexpr int kDecodeMaxExperts = 256;
struct DecodeSync;
struct DecodeArgs {
  const uint16_t* x;         // [N][M]
  const uint16_t* w_router;  // [M][E]
  const float* bias;         // [E] or null
  int N, M, E, k, H;
  const uint16_t* w_gate;
  const uint16_t* w_up;
  const uint16_t* w_down;
  const uint8_t* q_gate;
  const uint8_t* q_up;
  const uint8_t* q_down;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
  int32_t* ids;              // [N][k] out
  float* wts;                // [N][k] out
  uint16_t* out;             // [N][M] out
  uint16_t* h;
  uint16_t* y;
  uint64_t limit;            // longest barrier wait, in wall-clock ticks
  // set by the launcher
  float* part;
  DecodeSync* sync;
  int G, MS;
};
bool decode_fusable(int N, int M, int E, int k, int H, bool f8);
size_t decode_workspace_bytes(int N, int M, int E);
hipError_t launch_decode_layer(DecodeArgs a, void* ws, int num_cu, hipStream_t st);

struct CombineArgs {
  const uint16_t* y;         // [A][M] bf16
  const int32_t* a2s;        // [A]
  const float* weights;      // [N][k] or null
  const uint16_t* shared;    // [N][M] or null
  uint16_t* out;             // [N][M]
  int N, M, k;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

}  // namespace moe
