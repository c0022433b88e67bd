"""Brute force for tiny MoE layers: one token at a time, pure Python loops.

It is written independently of oracle/ (no shared helpers): the bf16 widening,
the dot products (math.fsum of exact products), the selection (Python sorted
on (-p, id)), the per-expert grouping (a scan over assignments) and the SwiGLU
are all spelled out here.  Used only to pin the oracle on small shapes.
"""
import math
import struct

import numpy as np


def bf16(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(u) & 0xFFFF) << 16))[0]


def f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def dot(a, b) -> float:
    return math.fsum(x * y for x, y in zip(a, b))


def route_token(xrow, wr_cols, bias, k):
    """Scores in float32 (fsum of exact products, rounded once), softmax with
    float32 rounding of each step, top-k by (-p, id), renormalise."""
    E = len(wr_cols)
    logits = [f32(dot(xrow, wr_cols[e])) for e in range(E)]
    if bias is not None:
        logits = [f32(logits[e] + float(bias[e])) for e in range(E)]
    mx = max(logits)
    z = [f32(math.exp(f32(l - mx))) for l in logits]
    s = f32(math.fsum(z))
    p = [f32(v / s) for v in z]
    order = sorted(range(E), key=lambda e: (-p[e], e))
    ids = order[:k]
    ssel = math.fsum(p[e] for e in ids)
    w = [p[e] / ssel for e in ids]
    return ids, w, p


def swiglu_row(xrow, wg, wu, wd):
    H = len(wg)
    h = []
    for j in range(H):
        g = dot(xrow, wg[j])
        u = dot(xrow, wu[j])
        h.append(g * (1.0 / (1.0 + math.exp(-g))) * u)
    return [dot(h, wd[m]) for m in range(len(wd))]


def layer(inp, k, S=0, Hs=0, ids_in=None, w_in=None):
    """Returns dict with ids, weights, counts, sorted_to_assign, out (lists)."""
    x = [[bf16(v) for v in row] for row in inp["x"]]
    N, M = len(x), (len(x[0]) if len(x) else 0)
    E = inp["w_gate"].shape[0]
    Wg = [[[bf16(v) for v in r] for r in inp["w_gate"][e]] for e in range(E)]
    Wu = [[[bf16(v) for v in r] for r in inp["w_up"][e]] for e in range(E)]
    Wd = [[[bf16(v) for v in r] for r in inp["w_down"][e]] for e in range(E)]
    bias = inp.get("router_bias")
    ids_all, w_all = [], []
    for n in range(N):
        if ids_in is None:
            wr_cols = [[bf16(inp["w_router"][m][e]) for m in range(M)] for e in range(E)]
            ids, w, _ = route_token(x[n], wr_cols, bias, k)
        else:
            ids, w = [int(v) for v in ids_in[n]], [float(v) for v in w_in[n]]
        ids_all.append(ids)
        w_all.append(w)
    # dispatch: scan assignments in order for each expert
    assigns = [(n * k + j, ids_all[n][j]) for n in range(N) for j in range(k)]
    counts = [sum(1 for _, e in assigns if e == ee) for ee in range(E)]
    s2a = [a for ee in range(E) for a, e in assigns if e == ee]
    out = []
    for n in range(N):
        acc = [0.0] * M
        for j in range(k):
            e = ids_all[n][j]
            y = swiglu_row(x[n], Wg[e], Wu[e], Wd[e])
            for m in range(M):
                acc[m] += w_all[n][j] * y[m]
        for s in range(S):
            gs = [[bf16(v) for v in r] for r in inp["ws_gate"][s * Hs:(s + 1) * Hs]]
            us = [[bf16(v) for v in r] for r in inp["ws_up"][s * Hs:(s + 1) * Hs]]
            ds = [[bf16(v) for v in r[s * Hs:(s + 1) * Hs]] for r in inp["ws_down"]]
            y = swiglu_row(x[n], gs, us, ds)
            for m in range(M):
                acc[m] += y[m]
        out.append(acc)
    return {"topk_ids": ids_all, "topk_weights": w_all, "counts": counts,
            "sorted_to_assign": s2a, "out": np.array(out, dtype=np.float64).reshape(N, M)}
