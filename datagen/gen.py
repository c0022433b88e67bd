"""Seeded synthetic inputs for the MoE FFN layer.

Both the oracle and the HIP path are fed from here; the module holds none of
the layer's arithmetic (no routing, no GEMM, no activation).  Every array is a
pure function of (workload, seed):

  * values: x ~ N(0, 1); every weight ~ N(0, 0.02^2) (0.02 is the standard
    deviation); drawn in float32 and rounded to bfloat16 with round-to-nearest-
    even on the bit pattern.  bf16 arrays are returned as uint16 bit patterns.
  * streams: numpy SeedSequence([cfg_id, stream, sub, seed]) with
    stream 0 x, 1 router, 2/3/4 gate/up/down (sub = expert), 5 shared
    (sub = 3*s + {0,1,2}), 6 popularity permutation, 7 pre-routed ids,
    8 pre-routed weights.
  * the skewed workload's per-expert router bias is b_e = -beta * s * ln(r_e),
    r a seeded permutation of 1..E and s = 1.2 the Zipf exponent; beta is the
    calibrated scale stored in skew_qwen235.json (written by
    oracle/calibrate_skew.py, which routes with the oracle only).
  * the pre-routed expert-node share draws local expert ids iid from
    p_e proportional to (pi(e)+1)^(-a), pi a seeded permutation, with a solved
    so that the hottest expert's expected load is 4x the mean; its routing
    weights are U(0, 1) float32.
"""
import json
import os
import concurrent.futures as cf
from typing import Dict, Optional

import numpy as np

from .configs import Workload

WEIGHT_STD = 0.02
ZIPF_S = 1.2
HOT_RATIO = 4.0
_HERE = os.path.dirname(os.path.abspath(__file__))
SKEW_FILE = os.path.join(_HERE, "skew_qwen235.json")


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.
    Inputs here are finite normals, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def _rng(cfg_id: int, stream: int, sub: int, seed: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, stream, sub, seed]))


def _normal_bf16_into(out: np.ndarray, cfg_id: int, stream: int, sub: int, seed: int, std: float) -> None:
    rng = _rng(cfg_id, stream, sub, seed)
    flat = out.reshape(-1)
    chunk = 1 << 22
    buf = np.empty(min(chunk, flat.size), np.float32)
    for s in range(0, flat.size, chunk):
        n = min(chunk, flat.size - s)
        b = buf[:n]
        rng.standard_normal(out=b, dtype=np.float32)
        if std != 1.0:
            b *= np.float32(std)
        flat[s:s + n] = f32_to_bf16_bits(b)


def normal_bf16(shape, cfg_id: int, stream: int, sub: int, seed: int = 0, std: float = 1.0) -> np.ndarray:
    out = np.empty(shape, np.uint16)
    _normal_bf16_into(out, cfg_id, stream, sub, seed, std)
    return out


def _stacked(n_sub: int, shape, cfg_id: int, stream: int, seed: int, std: float) -> np.ndarray:
    out = np.empty((n_sub,) + tuple(shape), np.uint16)
    with cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda e: _normal_bf16_into(out[e], cfg_id, stream, e, seed, std), range(n_sub)))
    return out


def popularity_permutation(E: int, cfg_id: int, seed: int = 0) -> np.ndarray:
    """Seeded permutation r of 1..E: expert e has popularity rank r[e]."""
    return _rng(cfg_id, 6, 0, seed).permutation(E) + 1


def zipf_bias(E: int, beta: float, cfg_id: int, seed: int = 0) -> np.ndarray:
    r = popularity_permutation(E, cfg_id, seed).astype(np.float64)
    return (-beta * ZIPF_S * np.log(r)).astype(np.float32)


def load_skew_beta() -> float:
    with open(SKEW_FILE) as f:
        return float(json.load(f)["beta"])


def solve_hot_exponent(E: int, ratio: float = HOT_RATIO) -> float:
    """a with max_e p_e = ratio / E for p_e proportional to r^(-a), r = 1..E
    (sum_r r^-a = E / ratio).  Bisection; the sum falls monotonically in a."""
    target = E / ratio
    r = np.arange(1, E + 1, dtype=np.float64)
    lo, hi = 0.0, 16.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.sum(r ** -mid) > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def pre_routed(N: int, E: int, cfg_id: int, seed: int = 0):
    """Expert-node share: local ids (int32 [N,1]) and weights (float32 [N,1])."""
    a = solve_hot_exponent(E)
    pi = _rng(cfg_id, 7, 1, seed).permutation(E)
    p = (pi + 1.0) ** -a
    p /= p.sum()
    ids = _rng(cfg_id, 7, 0, seed).choice(E, size=N, p=p).astype(np.int32)
    w = _rng(cfg_id, 8, 0, seed).random(N, dtype=np.float32)
    return ids.reshape(N, 1), w.reshape(N, 1), a


def generate(w: Workload, seed: int = 0, beta: Optional[float] = None) -> Dict[str, np.ndarray]:
    """All inputs of one layer call, as host arrays (bf16 as uint16 bits)."""
    rows = max(w.x_rows, w.N)
    x = normal_bf16((rows, w.M), w.cfg_id, 0, 0, seed)[: w.N]
    d: Dict[str, np.ndarray] = {"x": x}
    if w.pre_routed:
        ids, wts, a = pre_routed(w.N, w.E, w.cfg_id, seed)
        d["topk_ids"] = ids
        d["topk_weights"] = wts
        d["hot_exponent"] = np.float64(a)
    else:
        d["w_router"] = normal_bf16((w.M, w.E), w.cfg_id, 1, 0, seed, WEIGHT_STD)
        if w.skewed_bias:
            b = load_skew_beta() if beta is None else beta
            d["router_bias"] = zipf_bias(w.E, b, w.cfg_id, seed)
            d["beta"] = np.float64(b)
    d["w_gate"] = _stacked(w.E, (w.H, w.M), w.cfg_id, 2, seed, WEIGHT_STD)
    d["w_up"] = _stacked(w.E, (w.H, w.M), w.cfg_id, 3, seed, WEIGHT_STD)
    d["w_down"] = _stacked(w.E, (w.M, w.H), w.cfg_id, 4, seed, WEIGHT_STD)
    if w.S > 0:
        SH = w.S * w.Hs
        wg = np.empty((SH, w.M), np.uint16)
        wu = np.empty((SH, w.M), np.uint16)
        wd = np.empty((w.M, SH), np.uint16)
        for s in range(w.S):
            wg[s * w.Hs:(s + 1) * w.Hs] = normal_bf16((w.Hs, w.M), w.cfg_id, 5, 3 * s + 0, seed, WEIGHT_STD)
            wu[s * w.Hs:(s + 1) * w.Hs] = normal_bf16((w.Hs, w.M), w.cfg_id, 5, 3 * s + 1, seed, WEIGHT_STD)
            wd[:, s * w.Hs:(s + 1) * w.Hs] = normal_bf16((w.M, w.Hs), w.cfg_id, 5, 3 * s + 2, seed, WEIGHT_STD)
        d["ws_gate"], d["ws_up"], d["ws_down"] = wg, wu, wd
    return d


def random_small(N: int, M: int, E: int, k: int, H: int, S: int = 0, Hs: int = 0,
                 seed: int = 0, bias: bool = False, std: float = WEIGHT_STD) -> Dict[str, np.ndarray]:
    """Arbitrary small shapes for pins and ragged GPU cases (cfg_id 100)."""
    cid = 100
    sub = seed * 7919 + N * 31 + E
    d = {
        "x": normal_bf16((N, M), cid, 0, sub),
        "w_router": normal_bf16((M, E), cid, 1, sub, std=std),
        "w_gate": np.stack([normal_bf16((H, M), cid, 2, sub * 1024 + e, std=std) for e in range(E)]) if E else np.zeros((0, H, M), np.uint16),
        "w_up": np.stack([normal_bf16((H, M), cid, 3, sub * 1024 + e, std=std) for e in range(E)]) if E else np.zeros((0, H, M), np.uint16),
        "w_down": np.stack([normal_bf16((M, H), cid, 4, sub * 1024 + e, std=std) for e in range(E)]) if E else np.zeros((0, M, H), np.uint16),
    }
    if bias:
        d["router_bias"] = _rng(cid, 6, sub, 0).standard_normal(E).astype(np.float32)
    if S > 0:
        d["ws_gate"] = normal_bf16((S * Hs, M), cid, 5, sub * 3 + 0, std=std)
        d["ws_up"] = normal_bf16((S * Hs, M), cid, 5, sub * 3 + 1, std=std)
        d["ws_down"] = normal_bf16((M, S * Hs), cid, 5, sub * 3 + 2, std=std)
    return d
