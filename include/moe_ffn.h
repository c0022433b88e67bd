/*
 * moe_ffn.h - C ABI of one Mixture-of-Experts FFN layer on an AMD Instinct
 * MI355X (gfx950): router -> softmax -> top-k -> dispatch / permutation ->
 * grouped SwiGLU expert GEMM (+ shared experts) -> combine / unpermutation.
 *
 * Sources.  The steps are those the page "MoE 少算 FLOPs，延迟反而涨了：慢在搬
 * token 的路上" (wink.run) lays out in its sections "dense 和 MoE 的差别" (the router
 * scores every expert, keeps the top two and emits two routing weights) and
 * "router 之后还有一串动作" (N*k assignments grouped by expert = dispatch, token
 * rows sorted by expert = permutation, one grouped GEMM over all experts,
 * inverse mapping x weight + sum = combine).  Argument names follow the FinDEP
 * review page ("FinDEP: Efficient MoE Inference with Fine-Grained Scheduling of
 * Disaggregated Expert Parallelism", section 核心公式 and Algorithm 1's inputs):
 * N tokens, hidden size M, E experts, top_k, expert width H, shared experts.
 * Each expert is three GEMMs of m_e x M x H (FinDEP, 核心公式), read here as
 * SwiGLU: y = W_d (silu(W_g x) * (W_u x)), silu(z) = z / (1 + exp(-z)).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked host.  The caller owns every
 *    buffer; the library allocates and frees nothing.  All pointers must be
 *    16-byte aligned.
 *  - bf16 arrays are raw bfloat16 bit patterns (moe_bf16).  Matrices are
 *    row-major.  Expert weights are [out, in] (the contraction dimension is
 *    contiguous): w_gate/w_up [E][H][M], w_down [E][M][H].  The router is
 *    w_router [M][E].
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *    the null stream).  Outputs are valid after the caller synchronises it.
 *    No call synchronises the device or copies to the host.
 *  - Errors: every argument is checked on the host before anything is
 *    enqueued; a bad argument returns MOE_ERR_INVALID / MOE_ERR_UNSUPPORTED /
 *    MOE_ERR_WORKSPACE and enqueues nothing.  A failed launch returns
 *    MOE_ERR_DEVICE.  moe_last_error() gives the message of the last failure on
 *    the calling thread.  No C++ exception crosses this boundary.
 *  - Determinism: the same inputs give bitwise-identical outputs; floating-
 *    point sums are never ordered by atomics.
 *  - Numerics: bf16 operands, fp32 accumulation.  The SwiGLU intermediate h,
 *    the per-row expert outputs and `out` are stored in bf16.
 *  - Limits: 1 <= N <= 2^20; 64 <= M <= 16384 and M % 64 == 0;
 *    1 <= E <= 256; 1 <= top_k <= min(E, 16); 64 <= H <= 65536 and
 *    H % 64 == 0; shared: n_shared >= 0, n_shared * shared_width <= 65536 and
 *    a multiple of 64; N * top_k <= 2^24.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FFN_ABI_VERSION 1

typedef uint16_t moe_bf16;   /* raw bfloat16 bits */
typedef uint8_t moe_fp8;     /* raw OCP FP8 E4M3 bits */
typedef void* moe_stream;    /* a hipStream_t */

typedef struct moe_dims {
  int32_t n_tokens;      /* N: tokens (rows of x)                                 */
  int32_t hidden;        /* M: hidden size                                         */
  int32_t n_experts;     /* E: routed experts held by this GPU                     */
  int32_t top_k;         /* k: experts per token                                   */
  int32_t expert_width;  /* H: SwiGLU width of a routed expert                     */
  int32_t n_shared;      /* S: always-on shared experts (0 = none)                 */
  int32_t shared_width;  /* Hs: width of each shared expert                        */
} moe_dims;

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,      /* a NULL/misaligned pointer or out-of-range size      */
  MOE_ERR_UNSUPPORTED = 2,  /* a valid request this build does not implement       */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required          */
  MOE_ERR_DEVICE = 4        /* HIP reported an error (launch or device query)      */
};

enum {
  /* moe_layer: topk_ids / topk_weights are inputs (pre-routed rows, e.g. the
   * expert-node share fed by attention replicas); the router is skipped and
   * w_router / router_bias must be NULL.  Ids must lie in [0, E); rows of one
   * token need not be distinct.  An id outside [0, E) is clamped into range
   * on the device (no fault; the result is that of the clamped id). */
  MOE_FLAG_IDS_IN = 1u
};

/*
 * FP8 expert weights: OCP 8-bit floating point E4M3 codes (sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent 0 = subnormals m * 2^-9;
 * S.1111.111 = NaN; no infinity; largest finite 448) with one float32 scale
 * per output channel: weight[e][c][j] = value(code[e][c][j]) * scale[e][c].
 * Codes are laid out like the bf16 matrices; NaN codes must not occur (the
 * quantiser never writes them).  All six pointers are device pointers.
 */
typedef struct moe_fp8_ffn {
  const moe_fp8* gate;       /* [E][H][M] codes                                  */
  const moe_fp8* up;         /* [E][H][M] codes                                  */
  const moe_fp8* down;       /* [E][M][H] codes                                  */
  const float* gate_scale;   /* [E][H]                                           */
  const float* up_scale;     /* [E][H]                                           */
  const float* down_scale;   /* [E][M]                                           */
} moe_fp8_ffn;

/* Stage boundaries recorded by moe_set_stage_events. */
#define MOE_STAGE_EVENTS 7

/* ABI version of the loaded library (MOE_FFN_ABI_VERSION). */
int moe_abi_version(void);

/* Message of the last failed call on this thread ("" if none).  Valid until
 * the next call on the same thread. */
const char* moe_last_error(void);

/* Workspace moe_layer needs for `dims` and `flags`, in bytes (host). */
int moe_layer_workspace_bytes(const moe_dims* dims, uint32_t flags, size_t* bytes);

/*
 * moe_layer_single_launch - whether moe_layer (fp8 = 0) or moe_layer_fp8
 * (fp8 != 0) runs the whole layer as one launch for these dims and flags
 * (host only; *single = 1 or 0).  Page on MoE latency ("MoE 少算 FLOPs，延迟
 * 反而涨了"): at decode the steps around the expert GEMMs cost latency, not
 * FLOPs, and each kernel launch and wait adds to it.
 *
 * The single launch needs at most 8 tokens and 64 assignments (N*k), E in
 * {8, 16, 32, 64, 128, 256}, M and H multiples of 128 (256 with FP8 weights),
 * no shared experts and the router (no MOE_FLAG_IDS_IN).  It routes with fp32
 * FMAs whose summation order differs from moe_route's, so routing weights may
 * differ in the last bits and ids only where scores tie within rounding.
 * It is not taken while the stream is being captured into a graph or while
 * stage events are set; the layer then runs as separate kernels.
 *
 * In this build the single launch is switched off (its first run ended the
 * calling process with a fault not yet traced): *single is always 0.
 */
int moe_layer_single_launch(const moe_dims* dims, uint32_t flags, int fp8, int* single);

/* Workspace moe_route / moe_permute / moe_grouped_ffn need, in bytes (host).
 * For moe_grouped_ffn the dims are those of the call (E groups, N*k rows). */
int moe_route_workspace_bytes(const moe_dims* dims, size_t* bytes);
int moe_permute_workspace_bytes(const moe_dims* dims, size_t* bytes);
int moe_grouped_ffn_workspace_bytes(const moe_dims* dims, size_t* bytes);

/*
 * moe_route - router scores, softmax, top-k and renormalised routing weights.
 * Page on MoE latency, section "dense 和 MoE 的差别": the router reads each
 * token's hidden state, scores every expert and keeps the top k with k
 * routing weights.
 *
 *   logits[n,e]      = sum_m x[n,m] * w_router[m,e] (+ router_bias[e]),  fp32
 *   topk_ids[n,j]    = the k experts with the largest softmax probability,
 *                      slot 0 the largest, ties to the lower expert id
 *   topk_weights[n,j]= p[n,ids[n,j]] / sum_j' p[n,ids[n,j']]  (fp32)
 *
 * x [N][M] bf16; w_router [M][E] bf16; router_bias [E] fp32 or NULL;
 * topk_ids [N][k] int32 (out); topk_weights [N][k] fp32 (out).
 * ws: moe_route_workspace_bytes (the transposed router and partial scores).
 */
int moe_route(const moe_dims* dims, const moe_bf16* x, const moe_bf16* w_router,
              const float* router_bias, int32_t* topk_ids, float* topk_weights,
              void* ws, size_t ws_bytes, moe_stream stream);

/*
 * moe_permute - dispatch (per-expert counts and offsets) and the permutation
 * of assignments into expert order, plus the optional row gather.  Page on MoE
 * latency, section "router 之后还有一串动作".
 *
 * Assignment a = n*k + j goes to expert topk_ids[n][j] (must be in [0, E)).
 *   expert_counts[e]   = number of assignments to e                 [E] int32
 *   expert_offsets[e]  = sum of counts below e; [E] = N*k          [E+1] int32
 *   sorted_to_assign[p]= assignment in sorted slot p; slots of one expert are
 *                        contiguous and in increasing a (stable)    [N*k] int32
 *   assign_to_sorted[a]= inverse of sorted_to_assign               [N*k] int32
 *   x_sorted[p]        = x[sorted_to_assign[p] / k]   [N*k][M] bf16, optional
 * x may be NULL only if x_sorted is NULL.  ws: moe_permute_workspace_bytes.
 */
int moe_permute(const moe_dims* dims, const int32_t* topk_ids, const moe_bf16* x,
                int32_t* expert_counts, int32_t* expert_offsets,
                int32_t* sorted_to_assign, int32_t* assign_to_sorted,
                moe_bf16* x_sorted, void* ws, size_t ws_bytes, moe_stream stream);

/*
 * moe_grouped_ffn - every expert's SwiGLU over its contiguous block of sorted
 * rows, all experts in one launch per GEMM phase.  Experts with no rows cost
 * nothing and no row is padded into the result (page on MoE latency, section
 * "router 之后还有一串动作": a grouped GEMM cannot create work for an expert
 * without assignments, and fixed-shape padding computes empty rows).
 *
 * Rows p in [expert_offsets[e], expert_offsets[e+1]) belong to expert e;
 * expert_offsets [E+1] int32 on the device, non-decreasing, [0] = 0 and
 * [E] = N*k (N*k rows in total).
 *   h[p]        = silu(x_sorted[p] . w_gate[e]^T) * (x_sorted[p] . w_up[e]^T)
 *   y_sorted[p] = row_scale[p] * (h[p] . w_down[e]^T)     (row_scale NULL = 1)
 * x_sorted [N*k][M] bf16; w_gate/w_up [E][H][M]; w_down [E][M][H];
 * row_scale [N*k] fp32 or NULL; y_sorted [N*k][M] bf16 (out).
 * Shared experts are this call with E = 1, offsets {0, N} and H = S*Hs, the
 * S experts' weights concatenated along the width.
 */
int moe_grouped_ffn(const moe_dims* dims, const moe_bf16* x_sorted, const int32_t* expert_offsets,
                    const moe_bf16* w_gate, const moe_bf16* w_up, const moe_bf16* w_down,
                    const float* row_scale, moe_bf16* y_sorted,
                    void* ws, size_t ws_bytes, moe_stream stream);

/*
 * moe_quantize_fp8 - per-output-channel FP8 quantisation of a weight matrix.
 * The page on MoE latency, in its section on what to do about the cost, names
 * quantising weights as a way to move fewer bytes and asks that the numerical
 * error be measured; the format and scale rule are this library's reading:
 *   scale[r]  = max_j |w[r][j]| / 448 in float32 (1 for an all-zero row)
 *   q[r][j]   = the E4M3 code nearest to w[r][j] / scale[r] (float32
 *               quotient), ties to the even code, magnitudes >= 448
 *               saturated to 448, the sign kept (-0 for small negatives)
 * w [rows][cols] bf16 (rows = output channels: E*H for gate/up, E*M for
 * down; cols = the contraction); q [rows][cols] (out); scale [rows] (out).
 * 1 <= rows <= 2^26; 64 <= cols <= 65536, cols % 64 == 0.  A one-off weight
 * conversion, not part of the layer's path.
 */
int moe_quantize_fp8(const moe_bf16* w, int64_t rows, int32_t cols, moe_fp8* q, float* scale,
                     moe_stream stream);

/*
 * moe_grouped_ffn_fp8 - moe_grouped_ffn with FP8 expert weights.  The same
 * computation with each weight read as value(code) * scale: the codes are
 * widened to bf16 exactly, products are summed in fp32 and the channel's
 * scale multiplies the sum.  Every weight costs one byte of HBM traffic
 * instead of two, which is what bounds decode-sized batches (page on MoE
 * latency, section "router 之后还有一串动作": the grouped GEMM's cost in decode
 * is reading weights).  experts: a host pointer to the weight set.  Needs
 * hidden % 256 == 0 and expert_width % 256 == 0 (else MOE_ERR_UNSUPPORTED).
 * Workspace: moe_grouped_ffn_workspace_bytes.  Kernels are chosen by the
 * mean rows per expert as for bf16 weights (weight streaming for small
 * groups, MFMA tiles for large ones).
 */
int moe_grouped_ffn_fp8(const moe_dims* dims, const moe_bf16* x_sorted, const int32_t* expert_offsets,
                        const moe_fp8_ffn* experts, const float* row_scale, moe_bf16* y_sorted,
                        void* ws, size_t ws_bytes, moe_stream stream);

/*
 * moe_combine - unpermute and sum.  Page on MoE latency, section
 * "router 之后还有一串动作": results go back to token order through the inverse
 * mapping, are multiplied by the routing weight and summed.
 *   out[n] = sum_{j<k} w[n,j] * y_sorted[assign_to_sorted[n*k+j]] + shared_out[n]
 * summed in fp32 in slot order j = 0..k-1, then the shared term; stored bf16.
 * topk_weights [N][k] fp32, or NULL when y_sorted is already weighted (w = 1);
 * shared_out [N][M] bf16 or NULL.
 */
int moe_combine(const moe_dims* dims, const moe_bf16* y_sorted, const int32_t* assign_to_sorted,
                const float* topk_weights, const moe_bf16* shared_out, moe_bf16* out,
                moe_stream stream);

/*
 * moe_layer - the whole layer in one call, with no host synchronisation:
 * route (unless MOE_FLAG_IDS_IN) -> permute -> grouped SwiGLU with the routing
 * weight applied to each row -> shared experts -> combine.  Equal to the
 * chain of the four calls above up to bf16 rounding of where the weight is
 * applied.  The token-row gather is folded into the first GEMM's operand
 * loads, so x_sorted is never written.
 *
 * With MOE_FLAG_IDS_IN and k = 1 this is the expert-node share of
 * disaggregated expert parallelism (MegaScale-Infer summary, 核心贡献 1; FinDEP
 * review, 二、核心思想): rows aggregated from attention replicas, each pre-routed
 * to one local expert, run through it, scaled by their weight and returned in
 * arrival order.
 *
 * x [N][M]; w_router [M][E] (NULL iff IDS_IN); router_bias [E] or NULL;
 * w_gate/w_up [E][H][M]; w_down [E][M][H]; ws_gate/ws_up [S*Hs][M] and
 * ws_down [M][S*Hs] (NULL iff S = 0); topk_ids [N][k] int32 and topk_weights
 * [N][k] fp32: outputs (may be NULL) or, with IDS_IN, inputs (required);
 * out [N][M] bf16.  ws: moe_layer_workspace_bytes.
 *
 * Decode-sized batches (moe_layer_single_launch) run as one cooperative
 * launch instead of one kernel per step.  The workspace then also keeps a few
 * barrier words from call to call: like every other use of a workspace,
 * calls that share one must not overlap.
 */
int moe_layer(const moe_dims* dims, uint32_t flags, const moe_bf16* x,
              const moe_bf16* w_router, const float* router_bias,
              const moe_bf16* w_gate, const moe_bf16* w_up, const moe_bf16* w_down,
              const moe_bf16* ws_gate, const moe_bf16* ws_up, const moe_bf16* ws_down,
              int32_t* topk_ids, float* topk_weights, moe_bf16* out,
              void* ws, size_t ws_bytes, moe_stream stream);

/*
 * moe_layer_noalloc - moe_layer without a workspace argument, for callers that
 * cannot allocate device memory: code recorded under HIP graph capture, tight
 * serving loops, and harnesses that forbid hipMalloc.  The workspace is an
 * array inside the library, MOE_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU it
 * runs on, held until the process ends; its address is looked up once per
 * device, on the first call with that device current.  The call allocates
 * nothing (no hipMalloc, no hipFree).
 *
 * Arguments and results as for moe_layer.  Shapes whose
 * moe_layer_workspace_bytes exceed MOE_NOALLOC_SCRATCH_BYTES are rejected
 * with MOE_ERR_WORKSPACE before anything is enqueued (decode-sized batches
 * fit: e.g. N = 512 tokens of M = 2048, E = 128, k = 8, H = 768 need 29 MiB).
 * Every call on one GPU shares that GPU's array and nothing in it has to
 * start at zero, but calls that overlap on one GPU (two streams, two
 * threads) race on it: the caller must order them.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_layer_noalloc(const moe_dims* dims, uint32_t flags, const moe_bf16* x,
                      const moe_bf16* w_router, const float* router_bias,
                      const moe_bf16* w_gate, const moe_bf16* w_up, const moe_bf16* w_down,
                      const moe_bf16* ws_gate, const moe_bf16* ws_up, const moe_bf16* ws_down,
                      int32_t* topk_ids, float* topk_weights, moe_bf16* out, moe_stream stream);

/*
 * moe_layer_fp8 - moe_layer with FP8 weights for the routed experts and, if
 * n_shared > 0, the shared experts (their concatenation [S*Hs][M] and
 * [M][S*Hs] quantised as one matrix each, one scale per output channel).
 * The router stays bf16.  experts / shared: host pointers to the weight sets
 * (shared NULL iff n_shared = 0).  Needs hidden, expert_width and
 * n_shared*shared_width to be multiples of 256 (else MOE_ERR_UNSUPPORTED).
 * Workspace: moe_layer_workspace_bytes.  Stage events as for moe_layer.
 */
int moe_layer_fp8(const moe_dims* dims, uint32_t flags, const moe_bf16* x, const moe_bf16* w_router,
                  const float* router_bias, const moe_fp8_ffn* experts, const moe_fp8_ffn* shared,
                  int32_t* topk_ids, float* topk_weights, moe_bf16* out, void* ws, size_t ws_bytes,
                  moe_stream stream);

/*
 * moe_layer_pipelined - moe_layer over n_micro micro-batches of consecutive
 * tokens (sizes differ by at most one), overlapped on two streams: the
 * single-GPU form of the ping-pong pipeline of the MegaScale-Infer summary
 * (核心贡献 2: m micro-batches keep the attention and expert stages busy at the
 * same time).  Micro-batches alternate between `stream` and a second stream
 * that the library creates on first use per calling thread and device (default
 * priority, held until the process ends); the expert GEMMs of micro-batch i
 * start after those of micro-batch i-1 end, while routing, permutation and
 * combine of the neighbouring micro-batches run beside them.  The call
 * returns with all work ordered before later work on `stream`.  Each token's
 * result equals moe_layer's up to the summation order of its expert GEMMs
 * (the kernels are chosen per micro-batch size).  Arguments as for moe_layer;
 * 1 <= n_micro <= min(64, n_tokens); n_micro = 1 is moe_layer on `stream`.
 * Workspace: moe_layer_pipelined_workspace_bytes (two micro-batch slots).
 * Stage events are not recorded (a pending moe_set_stage_events is dropped).
 */
int moe_layer_pipelined_workspace_bytes(const moe_dims* dims, uint32_t flags, int32_t n_micro, size_t* bytes);
int moe_layer_pipelined(const moe_dims* dims, uint32_t flags, int32_t n_micro, const moe_bf16* x,
                        const moe_bf16* w_router, const float* router_bias, const moe_bf16* w_gate,
                        const moe_bf16* w_up, const moe_bf16* w_down, const moe_bf16* ws_gate,
                        const moe_bf16* ws_up, const moe_bf16* ws_down, int32_t* topk_ids, float* topk_weights,
                        moe_bf16* out, void* ws, size_t ws_bytes, moe_stream stream);

/*
 * moe_set_stage_events - per-stage timing of the next moe_layer call on the
 * calling thread.  The page on MoE latency, section "最慢的 GPU 决定这一步",
 * asks for per-step records of dispatch, expert and combine times; this hook
 * provides them without a host synchronisation.  `events` holds
 * MOE_STAGE_EVENTS hipEvent_t handles created by the caller; the next
 * moe_layer call on this thread records them on its stream at:
 *   [0] start  [1] after routing  [2] after dispatch/permutation
 *   [3] after the shared experts  [4] after the gate+up GEMM
 *   [5] after the down GEMM  [6] after the combine (end).
 * The setting is consumed by that one call (moe_layer or moe_layer_fp8).  events = NULL clears it.
 * n must equal MOE_STAGE_EVENTS.
 */
int moe_set_stage_events(void* const* events, int n);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FFN_H */
