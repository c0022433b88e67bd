// C ABI of the MoE FFN layer: argument checks, workspace carving and the
// launch sequence.  Every check runs on the host before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "../../include/moe_ffn.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_stage_ev[MOE_STAGE_EVENTS];
thread_local bool g_stage_on = false;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MOE_OK;
}

int device_error(const char* where, hipError_t e) {
  return fail(MOE_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQ_PTR(p)                                                                        \
  do {                                                                                    \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID, "%s: %s is NULL", fn, #p);          \
    if (!aligned(p)) return fail(MOE_ERR_INVALID, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)
#define OPT_PTR(p)                                                                        \
  do {                                                                                    \
    if ((p) != nullptr && !aligned(p))                                                    \
      return fail(MOE_ERR_INVALID, "%s: %s is not 16-byte aligned", fn, #p);             \
  } while (0)

constexpr int kMaxE = 256;
constexpr int kMaxK = 16;

// Shape limits shared by every entry point.  `need_k`: top_k must be valid.
int check_dims(const char* fn, const moe_dims* d, bool need_router_shape) {
  if (d == nullptr) return fail(MOE_ERR_INVALID, "%s: dims is NULL", fn);
  if (d->n_tokens < 1 || d->n_tokens > (1 << 20))
    return fail(MOE_ERR_INVALID, "%s: n_tokens=%d outside [1, 2^20]", fn, d->n_tokens);
  if (d->hidden < 64 || d->hidden > 16384 || d->hidden % 64 != 0)
    return fail(MOE_ERR_INVALID, "%s: hidden=%d must be a multiple of 64 in [64, 16384]", fn, d->hidden);
  if (d->n_experts < 1)
    return fail(MOE_ERR_INVALID, "%s: n_experts=%d must be >= 1", fn, d->n_experts);
  if (d->n_experts > kMaxE)
    return fail(MOE_ERR_UNSUPPORTED, "%s: n_experts=%d above the supported %d", fn, d->n_experts, kMaxE);
  if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > kMaxK)
    return fail(MOE_ERR_INVALID, "%s: top_k=%d must be in [1, min(n_experts, %d)]", fn, d->top_k, kMaxK);
  if ((long long)d->n_tokens * d->top_k > (1 << 24))
    return fail(MOE_ERR_INVALID, "%s: n_tokens*top_k above 2^24", fn);
  if (need_router_shape) {
    if (d->expert_width < 64 || d->expert_width > 65536 || d->expert_width % 64 != 0)
      return fail(MOE_ERR_INVALID, "%s: expert_width=%d must be a multiple of 64 in [64, 65536]", fn,
                  d->expert_width);
    if (d->n_shared < 0) return fail(MOE_ERR_INVALID, "%s: n_shared=%d < 0", fn, d->n_shared);
    if (d->n_shared > 0) {
      const long long sh = (long long)d->n_shared * d->shared_width;
      if (d->shared_width < 1 || sh > 65536 || sh % 64 != 0)
        return fail(MOE_ERR_INVALID,
                    "%s: n_shared*shared_width=%lld must be a positive multiple of 64 <= 65536", fn, sh);
    }
  }
  return MOE_OK;
}

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t n) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(n * sizeof(T));
    return p;
  }
};

struct PermuteWs {
  int32_t* tile_hist;
  int32_t* tile_off;
};
PermuteWs carve_permute(Carver& c, int A, int E) {
  const size_t T = (size_t)moe::ceil_div(A, moe::kPermTile);
  PermuteWs w;
  w.tile_hist = c.take<int32_t>((size_t)E * T);
  w.tile_off = c.take<int32_t>((size_t)E * T);
  return w;
}

struct LayerWs {
  void* route;
  int32_t* ids;
  float* wts;
  int32_t* counts;
  int32_t* offsets;
  int32_t* s2a;
  int32_t* a2s;
  int32_t* row_token;
  float* row_weight;
  int32_t* queue;        // tile queues of the routed and shared gate+up and down launches (zeroed by the permutation)
  PermuteWs perm;
  uint16_t* h;
  uint16_t* y;
  uint16_t* hs;
  uint16_t* ys;
  void* decode;          // single-launch decode path (router partials, barrier words)
  bool has_decode;
};
// The single-launch decode path (decode.hip) is switched off: its first run
// ended the calling process with a segmentation fault inside the layer call,
// before any of its kernels had completed, and the fault has not been traced
// to a cause.  Until it is, decode-sized batches run as separate kernels.
constexpr bool kSingleLaunchDecode = false;

// Shapes the single-launch decode path can take (bf16 weights; FP8 weights
// need a subset of them).
bool decode_shape(const moe_dims& d) {
  return kSingleLaunchDecode && d.n_shared == 0 &&
         moe::decode_fusable(d.n_tokens, d.hidden, d.n_experts, d.top_k, d.expert_width, false);
}
LayerWs carve_layer(Carver& c, const moe_dims& d) {
  const size_t N = d.n_tokens, A = (size_t)d.n_tokens * d.top_k, E = d.n_experts;
  const size_t SH = (size_t)d.n_shared * (d.n_shared > 0 ? d.shared_width : 0);
  LayerWs w;
  w.route = c.take<char>(moe::route_workspace_bytes(d.n_tokens, d.hidden, d.n_experts));
  w.ids = c.take<int32_t>(A);
  w.wts = c.take<float>(A);
  w.counts = c.take<int32_t>(E);
  w.offsets = c.take<int32_t>(E + 1);
  w.s2a = c.take<int32_t>(A);
  w.a2s = c.take<int32_t>(A);
  w.row_token = c.take<int32_t>(A);
  w.row_weight = c.take<float>(A);
  w.queue = c.take<int32_t>(4 * moe::kQueueWords);
  w.perm = carve_permute(c, (int)A, (int)E);
  w.h = c.take<uint16_t>(A * d.expert_width);
  w.y = c.take<uint16_t>(A * d.hidden);
  w.hs = SH ? c.take<uint16_t>(N * SH) : nullptr;
  w.ys = SH ? c.take<uint16_t>(N * d.hidden) : nullptr;
  w.has_decode = decode_shape(d);
  w.decode = w.has_decode ? c.take<char>(moe::decode_workspace_bytes(d.n_tokens, d.hidden, d.n_experts)) : nullptr;
  return w;
}

// Ticks of the device's constant-rate clock in half a second: the longest
// wait of a grid barrier in the single-launch decode path.
uint64_t barrier_limit_ticks() {
  static uint64_t cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) return 0;
    cache[dev] = (uint64_t)khz * 500;
  }
  return cache[dev];
}

int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      return -1;
    cache[dev] = v;
  }
  return cache[dev];
}

int check_ws(const char* fn, void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MOE_OK;
  if (ws == nullptr) return fail(MOE_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, need);
  return MOE_OK;
}

// Expert weights of one call: bf16 matrices, or FP8 codes with per-channel
// scales (then the bf16 pointers are NULL).
struct ExpertWeights {
  const uint16_t* gate = nullptr;
  const uint16_t* up = nullptr;
  const uint16_t* down = nullptr;
  const uint8_t* qgate = nullptr;
  const uint8_t* qup = nullptr;
  const uint8_t* qdown = nullptr;
  const float* sgate = nullptr;
  const float* sup = nullptr;
  const float* sdown = nullptr;
};

ExpertWeights bf16_weights(const moe_bf16* g, const moe_bf16* u, const moe_bf16* d) {
  ExpertWeights w;
  w.gate = g;
  w.up = u;
  w.down = d;
  return w;
}

ExpertWeights fp8_weights(const moe_fp8_ffn* f) {
  ExpertWeights w;
  if (f == nullptr) return w;
  w.qgate = f->gate;
  w.qup = f->up;
  w.qdown = f->down;
  w.sgate = f->gate_scale;
  w.sup = f->up_scale;
  w.sdown = f->down_scale;
  return w;
}

moe::FfnArgs gateup_args(const ExpertWeights& w) {
  moe::FfnArgs a{};
  a.w0 = w.gate;
  a.w1 = w.up;
  a.q0 = w.qgate;
  a.q1 = w.qup;
  a.s0 = w.sgate;
  a.s1 = w.sup;
  return a;
}

moe::FfnArgs down_args(const ExpertWeights& w) {
  moe::FfnArgs a{};
  a.w0 = w.down;
  a.q0 = w.qdown;
  a.s0 = w.sdown;
  return a;
}

// An FP8 weight set: every pointer present and aligned.
int check_fp8_ffn(const char* fn, const char* which, const moe_fp8_ffn* f) {
  if (f == nullptr) return fail(MOE_ERR_INVALID, "%s: %s is NULL", fn, which);
  const void* ptrs[6] = {f->gate, f->up, f->down, f->gate_scale, f->up_scale, f->down_scale};
  const char* names[6] = {"gate", "up", "down", "gate_scale", "up_scale", "down_scale"};
  for (int i = 0; i < 6; ++i) {
    if (ptrs[i] == nullptr) return fail(MOE_ERR_INVALID, "%s: %s->%s is NULL", fn, which, names[i]);
    if (!aligned(ptrs[i])) return fail(MOE_ERR_INVALID, "%s: %s->%s is not 16-byte aligned", fn, which, names[i]);
  }
  return MOE_OK;
}

// The FP8 kernels walk the contraction in 256-element chunks.
int check_fp8_dims(const char* fn, const moe_dims* d) {
  if (d->hidden % 256 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: FP8 weights need hidden %% 256 == 0 (hidden=%d)", fn, d->hidden);
  if (d->expert_width % 256 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: FP8 weights need expert_width %% 256 == 0 (expert_width=%d)", fn,
                d->expert_width);
  if (d->n_shared > 0 && (d->n_shared * d->shared_width) % 256 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: FP8 weights need n_shared*shared_width %% 256 == 0", fn);
  return MOE_OK;
}

// Both grouped GEMM phases; the arguments have been checked.
int run_grouped_ffn(const char* fn, const moe_dims* dims, const moe_bf16* x_sorted, const int32_t* expert_offsets,
                    const ExpertWeights& wt, const float* row_scale, moe_bf16* y_sorted, void* ws,
                    hipStream_t st) {
  const int ncu = num_cus();
  if (ncu <= 0) return fail(MOE_ERR_DEVICE, "%s: cannot query the device", fn);
  const int A = dims->n_tokens * dims->top_k;
  Carver c(ws);
  uint16_t* h = c.take<uint16_t>((size_t)A * dims->expert_width);
  int32_t* queue = c.take<int32_t>(2 * moe::kQueueWords);
  moe::FfnArgs g = gateup_args(wt);
  g.queue = queue;
  g.a = x_sorted;
  g.offsets = expert_offsets;
  g.out = h;
  g.E = dims->n_experts;
  g.rows_total = A;
  g.K = dims->hidden;
  g.ncols = dims->expert_width;
  if (hipError_t e = moe::launch_ffn_gateup(g, ncu, st)) return device_error(fn, e);
  moe::FfnArgs dn = down_args(wt);
  dn.queue = queue + moe::kQueueWords;
  dn.a = h;
  dn.offsets = expert_offsets;
  dn.row_scale = row_scale;
  dn.out = y_sorted;
  dn.E = dims->n_experts;
  dn.rows_total = A;
  dn.K = dims->expert_width;
  dn.ncols = dims->hidden;
  if (hipError_t e = moe::launch_ffn_down(dn, ncu, st)) return device_error(fn, e);
  return ok();
}

// Argument rules of the layer entry points other than the weights (checked
// by each caller) and the workspace.
int check_layer_args(const char* fn, uint32_t flags, const moe_bf16* x, const moe_bf16* w_router,
                     const float* router_bias, const int32_t* topk_ids, const float* topk_weights,
                     const moe_bf16* out) {
  if (flags & ~uint32_t(MOE_FLAG_IDS_IN)) return fail(MOE_ERR_INVALID, "%s: unknown flags 0x%x", fn, flags);
  const bool ids_in = (flags & MOE_FLAG_IDS_IN) != 0;
  REQ_PTR(x);
  if (ids_in) {
    if (w_router != nullptr || router_bias != nullptr)
      return fail(MOE_ERR_INVALID, "%s: w_router/router_bias must be NULL with MOE_FLAG_IDS_IN", fn);
    REQ_PTR(topk_ids);
    REQ_PTR(topk_weights);
  } else {
    REQ_PTR(w_router);
    OPT_PTR(router_bias);
    OPT_PTR(topk_ids);
    OPT_PTR(topk_weights);
  }
  REQ_PTR(out);
  return MOE_OK;
}

// Optional cross-stream ordering of a layer's expert GEMMs (shared and
// routed): wait for `before` ahead of the first, record `after` behind the
// last.  Used by the micro-batched layer so that one micro-batch's GEMMs run
// at a time while the small kernels around them overlap.
struct GemmOrder {
  hipEvent_t before = nullptr;
  hipEvent_t after = nullptr;
};

// Enqueue the whole layer on `st`; every argument has been checked and `ws`
// holds carve_layer(dims).  `rec`: record the stage events.
// True while `st` records into a graph (or its state cannot be read).
bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return true;
  return cs != hipStreamCaptureStatusNone;
}

int enqueue_layer(const char* fn, const moe_dims* dims, bool ids_in, const moe_bf16* x, const moe_bf16* w_router,
                  const float* router_bias, const ExpertWeights& routed, const ExpertWeights& shared,
                  int32_t* topk_ids, float* topk_weights, moe_bf16* out, void* ws, hipStream_t st, int ncu,
                  bool rec, const GemmOrder& order) {
  Carver c(ws);
  LayerWs w = carve_layer(c, *dims);
  const int N = dims->n_tokens, M = dims->hidden, E = dims->n_experts, k = dims->top_k, H = dims->expert_width;
  const int A = N * k;
  int32_t* ids = topk_ids ? topk_ids : w.ids;
  float* wts = topk_weights ? topk_weights : w.wts;
  auto mark = [&](int i) -> hipError_t { return rec ? hipEventRecord(g_stage_ev[i], st) : hipSuccess; };

  // Decode-sized batches: the whole layer in one launch (not while per-stage
  // events are wanted, not between the micro-batch streams, and not under
  // stream capture, where the kernels below are recorded instead).
  const bool f8 = routed.qgate != nullptr;
  if (!ids_in && !rec && w.has_decode && order.before == nullptr && order.after == nullptr &&
      moe::decode_fusable(N, M, E, k, H, f8) && !capturing(st)) {
    const uint64_t limit = barrier_limit_ticks();
    if (limit == 0) return fail(MOE_ERR_DEVICE, "%s: cannot query the device clock", fn);
    moe::DecodeArgs da{};
    da.x = x;
    da.w_router = w_router;
    da.bias = router_bias;
    da.N = N;
    da.M = M;
    da.E = E;
    da.k = k;
    da.H = H;
    da.w_gate = routed.gate;
    da.w_up = routed.up;
    da.w_down = routed.down;
    da.q_gate = routed.qgate;
    da.q_up = routed.qup;
    da.q_down = routed.qdown;
    da.s_gate = routed.sgate;
    da.s_up = routed.sup;
    da.s_down = routed.sdown;
    da.ids = ids;
    da.wts = wts;
    da.out = out;
    da.h = w.h;
    da.y = w.y;
    da.limit = limit;
    if (hipError_t e = moe::launch_decode_layer(da, w.decode, ncu, st)) return device_error(fn, e);
    return ok();
  }
  if (hipError_t e = mark(0)) return device_error(fn, e);

  moe::PermuteArgs p{ids, A, E, k, w.counts, w.offsets, w.s2a, w.a2s, w.row_token, wts, w.row_weight,
                     w.perm.tile_hist, w.perm.tile_off, w.queue, 4 * moe::kQueueWords};
  // up to four tokens: the route's top-k launch (one block) also permutes
  const bool route_perm = !ids_in && moe::route_permutes(N);
  if (!ids_in) {
    moe::RouteArgs r{x, w_router, router_bias, N, M, E, k, ids, wts};
    if (route_perm) r.perm = &p;
    if (hipError_t e = moe::launch_route(r, w.route, st)) return device_error(fn, e);
  }
  if (hipError_t e = mark(1)) return device_error(fn, e);
  if (!route_perm) {
    if (hipError_t e = moe::launch_permute(p, st)) return device_error(fn, e);
  }
  if (hipError_t e = mark(2)) return device_error(fn, e);
  if (order.before != nullptr) {
    if (hipError_t e = hipStreamWaitEvent(st, order.before, 0)) return device_error(fn, e);
  }

  // Shared experts: one group of all N rows, gate+up then down.  They go
  // into the routed experts' launches (moe::launch_ffn_*_shared), so the
  // "shared" stage between marks 2 and 3 is empty and its time counts in
  // the gate+up and down stages.
  const bool has_shared = dims->n_shared > 0;
  moe::FfnArgs sg{}, sd{};
  if (has_shared) {
    const int SH = dims->n_shared * dims->shared_width;
    sg = gateup_args(shared);
    sg.a = x;
    sg.fixed_rows = N;
    sg.out = w.hs;
    sg.E = 1;
    sg.rows_total = N;
    sg.K = M;
    sg.ncols = SH;
    sd = down_args(shared);
    sd.a = w.hs;
    sd.fixed_rows = N;
    sd.out = w.ys;
    sd.E = 1;
    sd.rows_total = N;
    sd.K = SH;
    sd.ncols = M;
    sg.queue = w.queue + 2 * moe::kQueueWords;
    sd.queue = w.queue + 3 * moe::kQueueWords;
    sg.queue_zeroed = sd.queue_zeroed = true;
  }
  if (hipError_t e = mark(3)) return device_error(fn, e);
  moe::FfnArgs g = gateup_args(routed);
  g.a = x;
  g.a_rows = w.row_token;
  g.a_nrows = N;
  g.offsets = w.offsets;
  g.out = w.h;
  g.E = E;
  g.rows_total = A;
  g.K = M;
  g.ncols = H;
  g.queue = w.queue;
  g.queue_zeroed = true;
  if (hipError_t e = has_shared ? moe::launch_ffn_gateup_shared(g, sg, ncu, st) : moe::launch_ffn_gateup(g, ncu, st))
    return device_error(fn, e);
  if (hipError_t e = mark(4)) return device_error(fn, e);
  // top-1 routing without shared experts: every token has exactly one row,
  // so the down GEMM stores it straight into the output (the combine would
  // only copy it)
  const bool direct = (k == 1 && dims->n_shared == 0);
  moe::FfnArgs dn = down_args(routed);
  dn.a = w.h;
  dn.offsets = w.offsets;
  dn.row_scale = w.row_weight;
  dn.out = direct ? out : w.y;
  dn.E = E;
  dn.rows_total = A;
  dn.K = H;
  dn.ncols = M;
  dn.out_rows = direct ? w.row_token : nullptr;
  dn.queue = w.queue + moe::kQueueWords;
  dn.queue_zeroed = true;
  if (hipError_t e = has_shared ? moe::launch_ffn_down_shared(dn, sd, ncu, st) : moe::launch_ffn_down(dn, ncu, st))
    return device_error(fn, e);
  if (order.after != nullptr) {
    if (hipError_t e = hipEventRecord(order.after, st)) return device_error(fn, e);
  }
  if (hipError_t e = mark(5)) return device_error(fn, e);

  if (!direct) {
    moe::CombineArgs cb{w.y, w.a2s, nullptr, w.ys, out, N, M, k};
    if (hipError_t e = moe::launch_combine(cb, st)) return device_error(fn, e);
  }
  if (hipError_t e = mark(6)) return device_error(fn, e);
  return ok();
}

// The whole layer; the weight pointers have been checked by the caller.
int run_layer(const char* fn, const moe_dims* dims, uint32_t flags, const moe_bf16* x, const moe_bf16* w_router,
              const float* router_bias, const ExpertWeights& routed, const ExpertWeights& shared,
              int32_t* topk_ids, float* topk_weights, moe_bf16* out, void* ws, size_t ws_bytes,
              moe_stream stream) {
  if (int r = check_layer_args(fn, flags, x, w_router, router_bias, topk_ids, topk_weights, out)) return r;
  Carver sz(nullptr);
  carve_layer(sz, *dims);
  if (int r = check_ws(fn, ws, ws_bytes, sz.off)) return r;
  const int ncu = num_cus();
  if (ncu <= 0) return fail(MOE_ERR_DEVICE, "%s: cannot query the device", fn);
  const bool rec = g_stage_on;
  g_stage_on = false;
  return enqueue_layer(fn, dims, (flags & MOE_FLAG_IDS_IN) != 0, x, w_router, router_bias, routed, shared,
                       topk_ids, topk_weights, out, ws, static_cast<hipStream_t>(stream), ncu, rec, GemmOrder{});
}

// ---------------------------------------------------------------------------
// Micro-batched layer: a second stream per calling thread and device, held
// until the process ends (created on first use, default priority), and the
// events that order work across the two streams.

constexpr int kMaxDevices = 64;
constexpr int kMaxMicro = 64;

struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr;       // caller's stream -> side stream
  hipEvent_t join = nullptr;       // side stream -> caller's stream
  hipEvent_t gemm[2] = {nullptr, nullptr};   // end of a micro-batch's GEMMs, per stream
};
thread_local SideStream g_side[kMaxDevices];

int side_stream(const char* fn, SideStream** out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return device_error(fn, e);
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  SideStream& s = g_side[dev];
  if (s.stream == nullptr) {
    SideStream n;
    if (hipError_t e = hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking)) return device_error(fn, e);
    hipEvent_t* evs[4] = {&n.fork, &n.join, &n.gemm[0], &n.gemm[1]};
    for (hipEvent_t* ev : evs)
      if (hipError_t e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) return device_error(fn, e);
    s = n;
  }
  *out = &s;
  return MOE_OK;
}

// Token range of micro-batch i of n over N tokens (sizes differ by at most one).
void micro_range(int N, int n, int i, int* start, int* count) {
  const int base = N / n, extra = N % n;
  *start = i * base + (i < extra ? i : extra);
  *count = base + (i < extra ? 1 : 0);
}

moe_dims micro_dims(const moe_dims& d, int n_micro) {
  moe_dims m = d;
  m.n_tokens = (d.n_tokens + n_micro - 1) / n_micro;
  return m;
}

size_t pipelined_ws_bytes(const moe_dims& d, int n_micro) {
  const moe_dims m = micro_dims(d, n_micro);
  Carver c(nullptr);
  carve_layer(c, m);
  return n_micro > 1 ? 2 * c.off : c.off;
}

int run_layer_pipelined(const char* fn, const moe_dims* dims, uint32_t flags, int32_t n_micro, const moe_bf16* x,
                        const moe_bf16* w_router, const float* router_bias, const ExpertWeights& routed,
                        const ExpertWeights& shared, int32_t* topk_ids, float* topk_weights, moe_bf16* out,
                        void* ws, size_t ws_bytes, moe_stream stream) {
  if (n_micro < 1 || n_micro > kMaxMicro || n_micro > dims->n_tokens)
    return fail(MOE_ERR_INVALID, "%s: n_micro=%d must be in [1, min(%d, n_tokens)]", fn, n_micro, kMaxMicro);
  if (int r = check_layer_args(fn, flags, x, w_router, router_bias, topk_ids, topk_weights, out)) return r;
  if (int r = check_ws(fn, ws, ws_bytes, pipelined_ws_bytes(*dims, n_micro))) return r;
  const int ncu = num_cus();
  if (ncu <= 0) return fail(MOE_ERR_DEVICE, "%s: cannot query the device", fn);
  g_stage_on = false;
  const bool ids_in = (flags & MOE_FLAG_IDS_IN) != 0;
  hipStream_t main_st = static_cast<hipStream_t>(stream);
  if (n_micro == 1)
    return enqueue_layer(fn, dims, ids_in, x, w_router, router_bias, routed, shared, topk_ids, topk_weights, out,
                         ws, main_st, ncu, false, GemmOrder{});
  SideStream* side = nullptr;
  if (int r = side_stream(fn, &side)) return r;
  const size_t slot = pipelined_ws_bytes(*dims, n_micro) / 2;
  const int M = dims->hidden, k = dims->top_k;
  if (hipError_t e = hipEventRecord(side->fork, main_st)) return device_error(fn, e);
  if (hipError_t e = hipStreamWaitEvent(side->stream, side->fork, 0)) return device_error(fn, e);
  for (int i = 0; i < n_micro; ++i) {
    int t0 = 0, nt = 0;
    micro_range(dims->n_tokens, n_micro, i, &t0, &nt);
    moe_dims d = *dims;
    d.n_tokens = nt;
    hipStream_t st = (i & 1) ? side->stream : main_st;
    GemmOrder order;
    order.before = i > 0 ? side->gemm[(i - 1) & 1] : nullptr;
    order.after = side->gemm[i & 1];
    void* wsi = static_cast<char*>(ws) + (i & 1) * slot;
    if (int r = enqueue_layer(fn, &d, ids_in, x + (size_t)t0 * M, w_router, router_bias, routed, shared,
                              topk_ids ? topk_ids + (size_t)t0 * k : nullptr,
                              topk_weights ? topk_weights + (size_t)t0 * k : nullptr, out + (size_t)t0 * M, wsi,
                              st, ncu, false, order))
      return r;
  }
  if (hipError_t e = hipEventRecord(side->join, side->stream)) return device_error(fn, e);
  if (hipError_t e = hipStreamWaitEvent(main_st, side->join, 0)) return device_error(fn, e);
  return ok();
}

// Workspace of moe_layer_noalloc: one array per GPU, in the code object's
// device memory.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address comes from hipGetSymbolAddress, once per
// device (with that device current), and only that address is used.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

int scratch_address(const char* fn, void** ptr) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return device_error(fn, e);
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return device_error(fn, e);
    if (p == nullptr) return fail(MOE_ERR_DEVICE, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_FFN_ABI_VERSION; }

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_set_stage_events(void* const* events, int n) {
  const char* fn = "moe_set_stage_events";
  if (events == nullptr) {
    g_stage_on = false;
    return ok();
  }
  if (n != MOE_STAGE_EVENTS) return fail(MOE_ERR_INVALID, "%s: n=%d, expected %d", fn, n, MOE_STAGE_EVENTS);
  for (int i = 0; i < n; ++i) {
    if (events[i] == nullptr) return fail(MOE_ERR_INVALID, "%s: events[%d] is NULL", fn, i);
    g_stage_ev[i] = static_cast<hipEvent_t>(events[i]);
  }
  g_stage_on = true;
  return ok();
}

int moe_layer_workspace_bytes(const moe_dims* dims, uint32_t flags, size_t* bytes) {
  const char* fn = "moe_layer_workspace_bytes";
  if (int r = check_dims(fn, dims, true)) return r;
  if (flags & ~uint32_t(MOE_FLAG_IDS_IN)) return fail(MOE_ERR_INVALID, "%s: unknown flags 0x%x", fn, flags);
  if (bytes == nullptr) return fail(MOE_ERR_INVALID, "%s: bytes is NULL", fn);
  Carver c(nullptr);
  carve_layer(c, *dims);
  *bytes = c.off;
  return ok();
}

int moe_layer_single_launch(const moe_dims* dims, uint32_t flags, int fp8, int* single) {
  const char* fn = "moe_layer_single_launch";
  if (int r = check_dims(fn, dims, true)) return r;
  if (flags & ~uint32_t(MOE_FLAG_IDS_IN)) return fail(MOE_ERR_INVALID, "%s: unknown flags 0x%x", fn, flags);
  if (single == nullptr) return fail(MOE_ERR_INVALID, "%s: single is NULL", fn);
  *single = ((flags & MOE_FLAG_IDS_IN) == 0 && decode_shape(*dims) &&
             moe::decode_fusable(dims->n_tokens, dims->hidden, dims->n_experts, dims->top_k, dims->expert_width,
                                 fp8 != 0))
                ? 1
                : 0;
  return ok();
}

int moe_route_workspace_bytes(const moe_dims* dims, size_t* bytes) {
  const char* fn = "moe_route_workspace_bytes";
  if (int r = check_dims(fn, dims, false)) return r;
  if (bytes == nullptr) return fail(MOE_ERR_INVALID, "%s: bytes is NULL", fn);
  *bytes = moe::route_workspace_bytes(dims->n_tokens, dims->hidden, dims->n_experts);
  return ok();
}

int moe_permute_workspace_bytes(const moe_dims* dims, size_t* bytes) {
  const char* fn = "moe_permute_workspace_bytes";
  if (int r = check_dims(fn, dims, false)) return r;
  if (bytes == nullptr) return fail(MOE_ERR_INVALID, "%s: bytes is NULL", fn);
  Carver c(nullptr);
  carve_permute(c, dims->n_tokens * dims->top_k, dims->n_experts);
  *bytes = c.off;
  return ok();
}

int moe_grouped_ffn_workspace_bytes(const moe_dims* dims, size_t* bytes) {
  const char* fn = "moe_grouped_ffn_workspace_bytes";
  if (int r = check_dims(fn, dims, true)) return r;
  if (bytes == nullptr) return fail(MOE_ERR_INVALID, "%s: bytes is NULL", fn);
  Carver c(nullptr);
  c.take<uint16_t>((size_t)dims->n_tokens * dims->top_k * dims->expert_width);
  c.take<int32_t>(2 * moe::kQueueWords);
  *bytes = c.off;
  return ok();
}

int moe_route(const moe_dims* dims, const moe_bf16* x, const moe_bf16* w_router,
              const float* router_bias, int32_t* topk_ids, float* topk_weights, void* ws, size_t ws_bytes,
              moe_stream stream) {
  const char* fn = "moe_route";
  if (int r = check_dims(fn, dims, false)) return r;
  REQ_PTR(x);
  REQ_PTR(w_router);
  OPT_PTR(router_bias);
  REQ_PTR(topk_ids);
  REQ_PTR(topk_weights);
  if (int r = check_ws(fn, ws, ws_bytes, moe::route_workspace_bytes(dims->n_tokens, dims->hidden, dims->n_experts)))
    return r;
  moe::RouteArgs a{x, w_router, router_bias, dims->n_tokens, dims->hidden, dims->n_experts, dims->top_k,
                   topk_ids, topk_weights};
  if (hipError_t e = moe::launch_route(a, ws, static_cast<hipStream_t>(stream))) return device_error(fn, e);
  return ok();
}

int moe_permute(const moe_dims* dims, const int32_t* topk_ids, const moe_bf16* x, int32_t* expert_counts,
                int32_t* expert_offsets, int32_t* sorted_to_assign, int32_t* assign_to_sorted,
                moe_bf16* x_sorted, void* ws, size_t ws_bytes, moe_stream stream) {
  const char* fn = "moe_permute";
  if (int r = check_dims(fn, dims, false)) return r;
  REQ_PTR(topk_ids);
  REQ_PTR(expert_counts);
  REQ_PTR(expert_offsets);
  REQ_PTR(sorted_to_assign);
  REQ_PTR(assign_to_sorted);
  OPT_PTR(x_sorted);
  if (x_sorted != nullptr) REQ_PTR(x);
  const int A = dims->n_tokens * dims->top_k;
  Carver sz(nullptr);
  carve_permute(sz, A, dims->n_experts);
  if (int r = check_ws(fn, ws, ws_bytes, sz.off)) return r;
  Carver c(ws);
  PermuteWs w = carve_permute(c, A, dims->n_experts);
  hipStream_t st = static_cast<hipStream_t>(stream);
  moe::PermuteArgs p{topk_ids, A, dims->n_experts, dims->top_k, expert_counts, expert_offsets,
                     sorted_to_assign, assign_to_sorted, nullptr, nullptr, nullptr, w.tile_hist, w.tile_off};
  if (hipError_t e = moe::launch_permute(p, st)) return device_error(fn, e);
  if (x_sorted != nullptr) {
    if (hipError_t e = moe::launch_gather(x, sorted_to_assign, dims->top_k, A, dims->hidden, x_sorted, st))
      return device_error(fn, e);
  }
  return ok();
}

int moe_grouped_ffn(const moe_dims* dims, const moe_bf16* x_sorted, const int32_t* expert_offsets,
                    const moe_bf16* w_gate, const moe_bf16* w_up, const moe_bf16* w_down,
                    const float* row_scale, moe_bf16* y_sorted, void* ws, size_t ws_bytes, moe_stream stream) {
  const char* fn = "moe_grouped_ffn";
  if (int r = check_dims(fn, dims, true)) return r;
  REQ_PTR(x_sorted);
  REQ_PTR(expert_offsets);
  REQ_PTR(w_gate);
  REQ_PTR(w_up);
  REQ_PTR(w_down);
  OPT_PTR(row_scale);
  REQ_PTR(y_sorted);
  size_t need = 0;
  moe_grouped_ffn_workspace_bytes(dims, &need);
  if (int r = check_ws(fn, ws, ws_bytes, need)) return r;
  return run_grouped_ffn(fn, dims, x_sorted, expert_offsets, bf16_weights(w_gate, w_up, w_down), row_scale,
                         y_sorted, ws, static_cast<hipStream_t>(stream));
}

int moe_grouped_ffn_fp8(const moe_dims* dims, const moe_bf16* x_sorted, const int32_t* expert_offsets,
                        const moe_fp8_ffn* experts, const float* row_scale, moe_bf16* y_sorted, void* ws,
                        size_t ws_bytes, moe_stream stream) {
  const char* fn = "moe_grouped_ffn_fp8";
  if (int r = check_dims(fn, dims, true)) return r;
  if (int r = check_fp8_dims(fn, dims)) return r;
  REQ_PTR(x_sorted);
  REQ_PTR(expert_offsets);
  if (int r = check_fp8_ffn(fn, "experts", experts)) return r;
  OPT_PTR(row_scale);
  REQ_PTR(y_sorted);
  size_t need = 0;
  moe_grouped_ffn_workspace_bytes(dims, &need);
  if (int r = check_ws(fn, ws, ws_bytes, need)) return r;
  return run_grouped_ffn(fn, dims, x_sorted, expert_offsets, fp8_weights(experts), row_scale, y_sorted, ws,
                         static_cast<hipStream_t>(stream));
}

int moe_quantize_fp8(const moe_bf16* w, int64_t rows, int32_t cols, moe_fp8* q, float* scale,
                     moe_stream stream) {
  const char* fn = "moe_quantize_fp8";
  if (rows < 1 || rows > (int64_t(1) << 26))
    return fail(MOE_ERR_INVALID, "%s: rows=%lld outside [1, 2^26]", fn, (long long)rows);
  if (cols < 64 || cols > 65536 || cols % 64 != 0)
    return fail(MOE_ERR_INVALID, "%s: cols=%d must be a multiple of 64 in [64, 65536]", fn, cols);
  REQ_PTR(w);
  REQ_PTR(q);
  REQ_PTR(scale);
  if (hipError_t e = moe::launch_quantize_fp8(w, rows, cols, q, scale, static_cast<hipStream_t>(stream)))
    return device_error(fn, e);
  return ok();
}

int moe_combine(const moe_dims* dims, const moe_bf16* y_sorted, const int32_t* assign_to_sorted,
                const float* topk_weights, const moe_bf16* shared_out, moe_bf16* out, moe_stream stream) {
  const char* fn = "moe_combine";
  if (int r = check_dims(fn, dims, false)) return r;
  REQ_PTR(y_sorted);
  REQ_PTR(assign_to_sorted);
  OPT_PTR(topk_weights);
  OPT_PTR(shared_out);
  REQ_PTR(out);
  moe::CombineArgs a{y_sorted, assign_to_sorted, topk_weights, shared_out, out, dims->n_tokens,
                     dims->hidden, dims->top_k};
  if (hipError_t e = moe::launch_combine(a, static_cast<hipStream_t>(stream))) return device_error(fn, e);
  return ok();
}

int moe_layer(const moe_dims* dims, uint32_t flags, const moe_bf16* x, const moe_bf16* w_router,
              const float* router_bias, const moe_bf16* w_gate, const moe_bf16* w_up, const moe_bf16* w_down,
              const moe_bf16* ws_gate, const moe_bf16* ws_up, const moe_bf16* ws_down, int32_t* topk_ids,
              float* topk_weights, moe_bf16* out, void* ws, size_t ws_bytes, moe_stream stream) {
  const char* fn = "moe_layer";
  if (int r = check_dims(fn, dims, true)) return r;
  REQ_PTR(w_gate);
  REQ_PTR(w_up);
  REQ_PTR(w_down);
  if (dims->n_shared > 0) {
    REQ_PTR(ws_gate);
    REQ_PTR(ws_up);
    REQ_PTR(ws_down);
  } else if (ws_gate || ws_up || ws_down) {
    return fail(MOE_ERR_INVALID, "%s: shared-expert weights given with n_shared = 0", fn);
  }
  return run_layer(fn, dims, flags, x, w_router, router_bias, bf16_weights(w_gate, w_up, w_down),
                   bf16_weights(ws_gate, ws_up, ws_down), topk_ids, topk_weights, out, ws, ws_bytes, stream);
}

int moe_layer_noalloc(const moe_dims* dims, uint32_t flags, const moe_bf16* x, const moe_bf16* w_router,
                      const float* router_bias, const moe_bf16* w_gate, const moe_bf16* w_up,
                      const moe_bf16* w_down, const moe_bf16* ws_gate, const moe_bf16* ws_up,
                      const moe_bf16* ws_down, int32_t* topk_ids, float* topk_weights, moe_bf16* out,
                      moe_stream stream) {
  const char* fn = "moe_layer_noalloc";
  if (int r = check_dims(fn, dims, true)) return r;
  REQ_PTR(w_gate);
  REQ_PTR(w_up);
  REQ_PTR(w_down);
  if (dims->n_shared > 0) {
    REQ_PTR(ws_gate);
    REQ_PTR(ws_up);
    REQ_PTR(ws_down);
  } else if (ws_gate || ws_up || ws_down) {
    return fail(MOE_ERR_INVALID, "%s: shared-expert weights given with n_shared = 0", fn);
  }
  if (int r = check_layer_args(fn, flags, x, w_router, router_bias, topk_ids, topk_weights, out)) return r;
  Carver sz(nullptr);
  carve_layer(sz, *dims);
  if (sz.off > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE, "%s: this shape needs %zu bytes of workspace, above the %zu of the library's "
                "scratch array (use moe_layer with a workspace)", fn, sz.off, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  if (int r = scratch_address(fn, &ptr)) return r;
  return run_layer(fn, dims, flags, x, w_router, router_bias, bf16_weights(w_gate, w_up, w_down),
                   bf16_weights(ws_gate, ws_up, ws_down), topk_ids, topk_weights, out, ptr,
                   MOE_NOALLOC_SCRATCH_BYTES, stream);
}

int moe_layer_fp8(const moe_dims* dims, uint32_t flags, const moe_bf16* x, const moe_bf16* w_router,
                  const float* router_bias, const moe_fp8_ffn* experts, const moe_fp8_ffn* shared,
                  int32_t* topk_ids, float* topk_weights, moe_bf16* out, void* ws, size_t ws_bytes,
                  moe_stream stream) {
  const char* fn = "moe_layer_fp8";
  if (int r = check_dims(fn, dims, true)) return r;
  if (int r = check_fp8_dims(fn, dims)) return r;
  if (int r = check_fp8_ffn(fn, "experts", experts)) return r;
  if (dims->n_shared > 0) {
    if (int r = check_fp8_ffn(fn, "shared", shared)) return r;
  } else if (shared != nullptr) {
    return fail(MOE_ERR_INVALID, "%s: shared-expert weights given with n_shared = 0", fn);
  }
  return run_layer(fn, dims, flags, x, w_router, router_bias, fp8_weights(experts), fp8_weights(shared),
                   topk_ids, topk_weights, out, ws, ws_bytes, stream);
}

int moe_layer_pipelined_workspace_bytes(const moe_dims* dims, uint32_t flags, int32_t n_micro, size_t* bytes) {
  const char* fn = "moe_layer_pipelined_workspace_bytes";
  if (int r = check_dims(fn, dims, true)) return r;
  if (flags & ~uint32_t(MOE_FLAG_IDS_IN)) return fail(MOE_ERR_INVALID, "%s: unknown flags 0x%x", fn, flags);
  if (n_micro < 1 || n_micro > kMaxMicro || n_micro > dims->n_tokens)
    return fail(MOE_ERR_INVALID, "%s: n_micro=%d must be in [1, min(%d, n_tokens)]", fn, n_micro, kMaxMicro);
  if (bytes == nullptr) return fail(MOE_ERR_INVALID, "%s: bytes is NULL", fn);
  *bytes = pipelined_ws_bytes(*dims, n_micro);
  return ok();
}

int moe_layer_pipelined(const moe_dims* dims, uint32_t flags, int32_t n_micro, const moe_bf16* x,
                        const moe_bf16* w_router, const float* router_bias, const moe_bf16* w_gate,
                        const moe_bf16* w_up, const moe_bf16* w_down, const moe_bf16* ws_gate,
                        const moe_bf16* ws_up, const moe_bf16* ws_down, int32_t* topk_ids, float* topk_weights,
                        moe_bf16* out, void* ws, size_t ws_bytes, moe_stream stream) {
  const char* fn = "moe_layer_pipelined";
  if (int r = check_dims(fn, dims, true)) return r;
  REQ_PTR(w_gate);
  REQ_PTR(w_up);
  REQ_PTR(w_down);
  if (dims->n_shared > 0) {
    REQ_PTR(ws_gate);
    REQ_PTR(ws_up);
    REQ_PTR(ws_down);
  } else if (ws_gate || ws_up || ws_down) {
    return fail(MOE_ERR_INVALID, "%s: shared-expert weights given with n_shared = 0", fn);
  }
  return run_layer_pipelined(fn, dims, flags, n_micro, x, w_router, router_bias, bf16_weights(w_gate, w_up, w_down),
                             bf16_weights(ws_gate, ws_up, ws_down), topk_ids, topk_weights, out, ws, ws_bytes,
                             stream);
}

}  // extern "C"
