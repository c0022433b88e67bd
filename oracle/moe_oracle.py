"""Oracle for one Mixture-of-Experts FFN layer: a plain, slow, CPU implementation.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests, the smoke check
and the bench's CPU-baseline leg may import or run anything under oracle/.  It
shares no code with the HIP path; both are fed by the seeded generators in
datagen/, which hold none of the layer's arithmetic.

What is computed (sources are the web pages the method is described on):

* The page "MoE 少算 FLOPs，延迟反而涨了：慢在搬 token 的路上" (wink.run), sections
  "dense 和 MoE 的差别" and "router 之后还有一串动作": a router scores every expert
  from the token's hidden state, keeps the top k and emits k routing weights;
  the N*k assignments are grouped by expert (dispatch), the token rows are
  sorted into expert order (permutation), each expert runs its own matrix
  (grouped GEMM), and the results are mapped back through the inverse mapping,
  multiplied by the routing weight and summed (combine / unpermutation).
* The FinDEP review page ("FinDEP: Efficient MoE Inference with Fine-Grained
  Scheduling of Disaggregated Expert Parallelism"), section 核心公式: one expert
  is three GEMMs of size m_e x M x H; section 二、核心思想 and Algorithm 1's input
  list: shared experts exist and are always on.

Readings where the pages are silent (each also listed in the design notes):
  gating is softmax -> top-k -> renormalise; ties go to the lower expert id and
  slots are in descending probability; the expert is SwiGLU,
  y = W_d (silu(W_g x) * (W_u x)), silu(z) = z / (1 + e^-z), no biases; shared
  experts apply to every token, unweighted, and add to the routed sum; no
  capacity limit, nothing dropped; the order inside an expert group is stable
  by assignment index a = n*k + j; the combine sums slots j = 0..k-1 in order
  and then adds the shared output.

Precision: the routing decision (logits, softmax, top-k, renormalised weights)
is taken in float32, the precision the kernel decides in: each logit is the
float64 dot product of the bf16 inputs (exact products) rounded once to
float32, and the optional router bias is added in float32.  Expert GEMMs, the
activation and the combine are float64.

Pinned by tests/test_oracle.py: brute force on tiny inputs, closed forms,
invariants, a library dense SwiGLU, the shared-expert concatenation identity and
the pages' worked numbers (156 tokens top-2 of 8 -> 39 rows per expert).
"""
from typing import Dict, Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# bf16 handling (inputs arrive as uint16 bit patterns)
# ----------------------------------------------------------------------------

def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    return bf16_to_f32(u16).astype(np.float64)


# ----------------------------------------------------------------------------
# Router: scores -> softmax -> top-k -> renormalised weights
# ----------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """logits[n, e] = sum_m x[n, m] * W_r[m, e] (+ b[e]).  W_r is [M, E].

    The router reads each token's hidden state and scores every expert (MoE
    latency page, section "dense 和 MoE 的差别")."""
    l = (bf16_to_f64(x) @ bf16_to_f64(w_router)).astype(np.float32)
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float32)[None, :]
    return l


def softmax32(logits: np.ndarray) -> np.ndarray:
    l = np.asarray(logits, dtype=np.float32)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True, dtype=np.float32)


def topk(p: np.ndarray, k: int):
    """Top-k by descending probability, ties to the lower expert id.

    Returns ids [N, k] (slot 0 = most probable), renormalised weights [N, k]
    (float32) and the tie margin per token: the smallest gap between
    consecutive probabilities among the k+1 largest (among the k largest when
    k = E), which bounds both the selected set and the slot order."""
    N, E = p.shape
    eid = np.broadcast_to(np.arange(E), (N, E))
    order = np.lexsort((eid, -p), axis=1)          # primary key -p, then id
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(p, ids, axis=1)
    weights = (sel / sel.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    kk = min(k + 1, E)
    ps = np.take_along_axis(p, order[:, :kk], axis=1).astype(np.float64)
    if kk >= 2:
        margin = (ps[:, :-1] - ps[:, 1:]).min(axis=1)
    else:
        margin = np.full(N, np.inf)
    return ids, weights, margin


def route(x, w_router, k: int, bias=None) -> Dict[str, np.ndarray]:
    logits = router_logits(x, w_router, bias)
    p = softmax32(logits)
    ids, weights, margin = topk(p, k)
    return {"logits": logits, "probs": p, "topk_ids": ids, "topk_weights": weights, "margin": margin}


# ----------------------------------------------------------------------------
# Dispatch and permutation
# ----------------------------------------------------------------------------

def dispatch(topk_ids: np.ndarray, E: int) -> Dict[str, np.ndarray]:
    """Group the N*k assignments by expert (MoE latency page, section
    "router 之后还有一串动作": dispatch, then permutation).

    Assignment a = n*k + j goes to expert ids[n, j].  counts[e] rows per
    expert, offsets = exclusive prefix sum, sorted_to_assign = stable sort of
    assignments by expert, assign_to_sorted its inverse."""
    e_a = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    A = e_a.size
    counts = np.bincount(e_a, minlength=E).astype(np.int32) if A else np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    s2a = np.argsort(e_a, kind="stable").astype(np.int32)
    a2s = np.empty(A, np.int32)
    a2s[s2a] = np.arange(A, dtype=np.int32)
    return {"expert_counts": counts, "expert_offsets": offsets,
            "sorted_to_assign": s2a, "assign_to_sorted": a2s}


def gather(x: np.ndarray, sorted_to_assign: np.ndarray, k: int) -> np.ndarray:
    """x_sorted[p] = x[token of the assignment in sorted slot p]; a byte copy."""
    return np.asarray(x)[np.asarray(sorted_to_assign) // k]


# ----------------------------------------------------------------------------
# Experts
# ----------------------------------------------------------------------------

def weights_f64(w) -> np.ndarray:
    """Expert weights as float64: bf16 bit patterns (uint16) are widened;
    anything else (e.g. dequantised FP8 weights) is taken as its values."""
    w = np.asarray(w)
    return bf16_to_f64(w) if w.dtype == np.uint16 else w.astype(np.float64)


def swiglu(X: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray):
    """One expert, three GEMMs (FinDEP review, 核心公式: t_e uses 3 GEMMs of
    m_e x M x H): G = X W_g^T, U = X W_u^T, h = silu(G) * U, Y = h W_d^T.
    X float64 [m, M]; weights bf16 bits or float64, W_g/W_u [H, M], W_d [M, H]."""
    G = X @ weights_f64(wg).T
    U = X @ weights_f64(wu).T
    h = G / (1.0 + np.exp(-G)) * U
    return h @ weights_f64(wd).T, h


def grouped_ffn(x_sorted: np.ndarray, offsets: np.ndarray, w_gate, w_up, w_down,
                row_scale: Optional[np.ndarray] = None, keep_h: bool = False):
    """Each expert runs its own block of sorted rows; experts with no rows do
    no work (MoE latency page, section "router 之后还有一串动作")."""
    A, M = np.asarray(x_sorted).shape
    E = len(offsets) - 1
    H = w_gate.shape[1] if E else 0
    y = np.zeros((A, M), np.float64)
    h_all = np.zeros((A, H), np.float64) if keep_h else None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        Y, h = swiglu(bf16_to_f64(x_sorted[lo:hi]), w_gate[e], w_up[e], w_down[e])
        y[lo:hi] = Y
        if keep_h:
            h_all[lo:hi] = h
    if row_scale is not None:
        y *= np.asarray(row_scale, np.float64)[:, None]
    return (y, h_all) if keep_h else y


def shared_experts(x: np.ndarray, ws_gate, ws_up, ws_down, S: int, Hs: int) -> np.ndarray:
    """Sum of S always-on experts applied to every token, unweighted (FinDEP
    review, 二、核心思想: shared experts live with attention and see every
    token).  Computed expert by expert from the slices of the concatenated
    arrays, so that a test can pin the concatenated form against it."""
    X = bf16_to_f64(x)
    out = np.zeros((X.shape[0], X.shape[1]), np.float64)
    for s in range(S):
        sl = slice(s * Hs, (s + 1) * Hs)
        Y, _ = swiglu(X, ws_gate[sl], ws_up[sl], ws_down[:, sl])
        out += Y
    return out


# ----------------------------------------------------------------------------
# Combine
# ----------------------------------------------------------------------------

def combine(y_sorted: np.ndarray, assign_to_sorted: np.ndarray, topk_weights: Optional[np.ndarray],
            k: int, shared: Optional[np.ndarray] = None) -> np.ndarray:
    """out[n] = sum_{j<k} w[n, j] * y_sorted[assign_to_sorted[n*k + j]] (+ shared[n]):
    inverse mapping, times routing weight, sum (MoE latency page, section
    "router 之后还有一串动作").  topk_weights=None means y is already weighted."""
    a2s = np.asarray(assign_to_sorted).reshape(-1)
    A = a2s.size
    N = A // k if k else 0
    M = y_sorted.shape[1]
    out = np.zeros((N, M), np.float64)
    w = None if topk_weights is None else np.asarray(topk_weights, np.float64).reshape(N, k)
    for j in range(k):
        rows = y_sorted[a2s[np.arange(N) * k + j]]
        out += rows if w is None else w[:, j:j + 1] * rows
    if shared is not None:
        out += shared
    return out


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------

def moe_layer(inp: Dict[str, np.ndarray], k: int, S: int = 0, Hs: int = 0,
              topk_ids: Optional[np.ndarray] = None, topk_weights: Optional[np.ndarray] = None,
              keep_h: bool = False) -> Dict[str, np.ndarray]:
    """Router -> top-k -> dispatch -> permutation -> grouped SwiGLU -> shared
    experts -> combine, returning every intermediate.  If topk_ids/weights are
    given, routing is skipped and they are used as is (pre-routed rows)."""
    x = inp["x"]
    E = inp["w_gate"].shape[0]
    res: Dict[str, np.ndarray] = {}
    if topk_ids is None:
        res.update(route(x, inp["w_router"], k, inp.get("router_bias")))
        topk_ids, topk_weights = res["topk_ids"], res["topk_weights"]
    res["topk_ids"], res["topk_weights"] = np.asarray(topk_ids, np.int32), np.asarray(topk_weights, np.float32)
    res.update(dispatch(topk_ids, E))
    xs = gather(x, res["sorted_to_assign"], k)
    res["x_sorted"] = xs
    r = grouped_ffn(xs, res["expert_offsets"], inp["w_gate"], inp["w_up"], inp["w_down"], keep_h=keep_h)
    y, h = r if keep_h else (r, None)
    if keep_h:
        res["h"] = h
    res["y_sorted"] = y
    sh = shared_experts(x, inp["ws_gate"], inp["ws_up"], inp["ws_down"], S, Hs) if S > 0 else None
    if sh is not None:
        res["shared_out"] = sh
    res["out"] = combine(y, res["assign_to_sorted"], res["topk_weights"], k, sh)
    return res


def token_outputs(inp: Dict[str, np.ndarray], topk_ids: np.ndarray, topk_weights: np.ndarray,
                  tokens: Sequence[int], S: int = 0, Hs: int = 0) -> np.ndarray:
    """The layer's output for selected tokens only, straight from the
    definition: out[n] = sum_j w[n, j] * FFN_{ids[n, j]}(x[n]) + shared(x[n]).
    Used to check full-size runs on sampled rows."""
    tokens = np.asarray(tokens, dtype=np.int64)
    x = inp["x"][tokens]
    X = bf16_to_f64(x)
    ids_all = np.asarray(topk_ids)
    ids = ids_all.reshape(ids_all.shape[0], -1)[tokens]
    w = np.asarray(topk_weights, np.float64).reshape(ids_all.shape[0], -1)[tokens]
    out = np.zeros((len(tokens), X.shape[1]), np.float64)
    # slot by slot, then expert by expert: inside one slot a token appears
    # once, so the row updates below never collide
    for j in range(ids.shape[1]):
        for e in np.unique(ids[:, j]):
            rows = np.nonzero(ids[:, j] == e)[0]
            Y, _ = swiglu(X[rows], inp["w_gate"][e], inp["w_up"][e], inp["w_down"][e])
            out[rows] += w[rows, j][:, None] * Y
    if S > 0:
        out += shared_experts(x, inp["ws_gate"], inp["ws_up"], inp["ws_down"], S, Hs)
    return out


def expert_node(x, topk_ids, topk_weights, w_gate, w_up, w_down) -> Dict[str, np.ndarray]:
    """Expert-node share of disaggregated expert parallelism (MegaScale-Infer
    summary, 核心贡献 1; FinDEP review, 二、核心思想: the expert group holds the
    non-shared experts and serves rows aggregated from attention replicas).
    Rows arrive pre-routed to one local expert each (k = 1); they are
    dispatched, run through their expert, scaled by their routing weight and
    scattered back to arrival order.  The sum over a token's experts happens
    after the return trip and is not part of this step."""
    E = w_gate.shape[0]
    d = dispatch(topk_ids, E)
    xs = gather(x, d["sorted_to_assign"], 1)
    y = grouped_ffn(xs, d["expert_offsets"], w_gate, w_up, w_down)
    out = combine(y, d["assign_to_sorted"], topk_weights, 1, None)
    d.update({"x_sorted": xs, "y_sorted": y, "out": out})
    return d

