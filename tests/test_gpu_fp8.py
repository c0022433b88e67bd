"""GPU parity of the FP8 (OCP E4M3, per-output-channel scale) entry points.

moe_quantize_fp8 must write the oracle's codes and scales bit for bit.  The
FP8 grouped FFN and layer are compared with the oracle's layer run on the
oracle's own dequantised weights (value(code) * scale in float64), to the
same bars as the bf16 path (max_rel <= 2e-2, rel_L2 <= 5e-3): both sides
multiply the same E4M3 values, only the summation order and the bf16
rounding of h and the output differ.  The cost of FP8 itself (FP8 layer
against the bf16 layer) is printed and bounded loosely; it is a measurement,
not a parity bar.
"""
import numpy as np
import pytest
import torch

from datagen import configs, gen
from oracle import fp8 as F
from oracle import moe_oracle as O
import expert_ffn_dispatch_amd as moe
from gpu_util import (TIE_MARGIN, assert_close, assert_rows_close, bf, errors, f32, host64, i32, note, upload)

pytestmark = pytest.mark.gpu


def _codes(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def _check_quant(bits: np.ndarray, what: str):
    q, s = moe.moe_quantize_fp8(bf(bits))
    torch.cuda.synchronize()
    oq, os_ = F.quantize_rows(bits)
    gq, gs = _codes(q), s.cpu().numpy()
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), f"{what}: scales differ"
    bad = np.count_nonzero(gq != oq)
    assert bad == 0, f"{what}: {bad} codes differ"
    return q, s, oq, os_


def _special_rows(cols: int) -> np.ndarray:
    """Rows that exercise the encoder: zeros, a lone value, exact ties (a row
    whose amax is 448 * 2^-8 has scale 2^-8 exactly, so midpoints between
    E4M3 values land exactly), subnormals and saturation neighbours."""
    rng = np.random.default_rng(5)
    t = F.e4m3_table()
    pos = t[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    rows = np.zeros((6, cols), np.float32)
    rows[1, 7] = -0.75
    r = rng.choice(np.concatenate([mids, -mids, pos, -pos]), size=cols) * 2.0 ** -8
    r[0] = 448 * 2.0 ** -8
    rows[2] = r
    rows[3] = rng.standard_normal(cols) * 1e-3
    rows[3, 0] = 3.0                         # most of the row becomes subnormal codes
    rows[4] = rng.standard_normal(cols).astype(np.float32) * 0.02
    rows[5] = -rows[4]
    return gen.f32_to_bf16_bits(rows)


@pytest.mark.parametrize("rows,cols", [(1, 64), (37, 192), (256, 768), (64, 16384)])
def test_quantize_bit_exact(rows, cols):
    note(f"quantize {rows}x{cols}")
    bits = gen.normal_bf16((rows, cols), 100, 9, rows * 131 + cols, std=0.02)
    _check_quant(bits, f"random {rows}x{cols}")
    _check_quant(_special_rows(cols), f"special rows x{cols}")


def _quant_set(t, d, names=("w_gate", "w_up", "w_down")):
    """GPU codes for the product path, oracle codes for the oracle (each from
    the same bf16 weights, and required to agree bit for bit)."""
    gq, oq = [], {}
    for n in names:
        q, s, oqq, oss = _check_quant(d[n], n)
        gq += [q, s]
        oq[n] = F.DequantizedExperts(oqq, oss)
    return moe.Fp8Weights(gq[0], gq[2], gq[4], gq[1], gq[3], gq[5]), oq


# N, M, E, k, H: the launches each one reaches are named
FFN_SHAPES = [
    (1, 256, 8, 2, 256),      # two rows: split-contraction kernels
    (37, 512, 5, 2, 768),     # ragged groups, 32-row passes
    (64, 256, 64, 8, 1024),   # 1-row groups: plain 16-row gate+up, split down
    (60, 768, 4, 2, 512),     # 48-row passes, down with 48 columns per wave
    (100, 768, 4, 2, 512),    # 64-row passes
    (300, 256, 3, 1, 256),    # 100-row groups: the tile kernel, 128-row tiles
    (50, 256, 6, 6, 256),     # k = E
    (40, 512, 16, 2, 256),    # empty experts
    (600, 512, 4, 1, 512),    # 150-row groups: the tile kernel, 192-row tiles
    (1200, 256, 4, 1, 256),   # 300-row groups: 192-row tiles, two row tiles per group
    (3000, 256, 4, 1, 256),   # 750-row groups: 256-row tiles, three row tiles per group
]


@pytest.mark.parametrize("shape", FFN_SHAPES, ids=[str(s) for s in FFN_SHAPES])
def test_grouped_ffn_fp8(shape):
    N, M, E, k, H = shape
    note(f"grouped ffn fp8 {shape}")
    d = gen.random_small(N, M, E, k, H, seed=3, std=0.05)
    r = O.route(d["x"], d["w_router"], k)
    o = O.dispatch(r["topk_ids"], E)
    xs = O.gather(d["x"], o["sorted_to_assign"], k)
    rs = np.random.default_rng(7).uniform(0.1, 1.0, N * k).astype(np.float32)
    t = upload(d)
    gw, ow = _quant_set(t, d)
    dm = moe.dims(N, M, E, k, H)
    y = moe.moe_grouped_ffn_fp8(dm, bf(xs), i32(o["expert_offsets"]), gw, row_scale=f32(rs))
    torch.cuda.synchronize()
    ref = O.grouped_ffn(xs, o["expert_offsets"], ow["w_gate"], ow["w_up"], ow["w_down"], row_scale=rs)
    assert_close(host64(y), ref, "y_sorted")


# N, M, E, k, H, S, Hs, bias
LAYER_SHAPES = [
    (64, 256, 8, 2, 512, 0, 0, False),
    (130, 512, 20, 1, 256, 0, 0, True),     # k = 1: the down GEMM writes the output rows
    (200, 256, 16, 2, 256, 2, 128, False),  # shared experts (concatenated width 256)
    (1, 512, 32, 4, 768, 1, 256, False),    # one token
    (512, 256, 8, 2, 256, 2, 128, False),   # tile kernel with the shared experts in the same launch
]


def _layer_ref(d, k, S, Hs, ow, osh, ids, wts, toks=None):
    inp = {**d, **ow, **osh}
    if toks is None:
        return O.moe_layer(inp, k, S, Hs, topk_ids=ids, topk_weights=wts)["out"]
    return O.token_outputs(inp, ids, wts, toks, S, Hs)


@pytest.mark.parametrize("shape", LAYER_SHAPES, ids=[str(s[:7]) for s in LAYER_SHAPES])
def test_layer_fp8(shape):
    N, M, E, k, H, S, Hs, bias = shape
    note(f"layer fp8 {shape}")
    d = gen.random_small(N, M, E, k, H, S, Hs, seed=4, bias=bias, std=0.05)
    t = upload(d)
    gw, ow = _quant_set(t, d)
    gsh, osh = (None, {})
    if S > 0:
        gsh, osh_ = _quant_set(t, d, ("ws_gate", "ws_up", "ws_down"))
        osh = {n: F.dequantize_rows(v.q, v.scale) for n, v in osh_.items()}
    dm = moe.dims(N, M, E, k, H, S, Hs)
    ids = torch.empty((N, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((N, k), dtype=torch.float32, device="cuda")
    out = moe.moe_layer_fp8(dm, t["x"], gw, gsh, w_router=t["w_router"], router_bias=t.get("router_bias"),
                            topk_ids=ids, topk_weights=wts)
    torch.cuda.synchronize()
    r = O.route(d["x"], d["w_router"], k, d.get("router_bias"))
    ok = r["margin"] >= TIE_MARGIN
    assert np.array_equal(ids.cpu().numpy()[ok], r["topk_ids"][ok])
    ref = _layer_ref(d, k, S, Hs, ow, osh, r["topk_ids"], r["topk_weights"])
    assert_close(host64(out)[ok], ref[ok], "out")


def test_layer_fp8_deterministic():
    N, M, E, k, H = 96, 512, 8, 2, 512
    d = gen.random_small(N, M, E, k, H, seed=6, std=0.05)
    t = upload(d)
    gw, _ = _quant_set(t, d)
    dm = moe.dims(N, M, E, k, H)
    a = moe.moe_layer_fp8(dm, t["x"], gw, w_router=t["w_router"])
    b = moe.moe_layer_fp8(dm, t["x"], gw, w_router=t["w_router"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------
# full-size decode workloads, launched as the bench launches them
# ---------------------------------------------------------------------------

_cache = {}


def _workload(name):
    if name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        w = configs.get(name)
        note(f"generate {w.title}")
        d = gen.generate(w)
        t = upload(d)
        gw = moe.quantize_ffn_fp8(t["w_gate"], t["w_up"], t["w_down"])
        torch.cuda.synchronize()
        _cache[name] = (w, d, t, gw)
    return _cache[name]


# workload, tokens (None = the workload's own)
FULL = [
    ("mixtral", None),
    ("qwen30", 1),
    ("qwen30", 32),
    ("qwen30", 512),
    ("dsv2", None),
    ("qwen235", None),
]


def _oracle_all(d, gw, names=("w_gate", "w_up", "w_down")):
    """The oracle's FP8 weights for every expert, checked bit for bit against
    the GPU's codes and scales."""
    ow = {}
    gpu = {"w_gate": (gw.gate, gw.gate_scale), "w_up": (gw.up, gw.up_scale), "w_down": (gw.down, gw.down_scale),
           "ws_gate": (gw.gate, gw.gate_scale), "ws_up": (gw.up, gw.up_scale), "ws_down": (gw.down, gw.down_scale)}
    for n in names:
        q, s = F.quantize_rows(d[n])
        gq, gs = gpu[n]
        assert np.array_equal(gq.cpu().numpy(), q), f"{n} codes"
        assert np.array_equal(gs.cpu().numpy().view(np.uint32), s.view(np.uint32)), f"{n} scales"
        ow[n] = F.DequantizedExperts(q, s) if q.ndim == 3 else F.dequantize_rows(q, s)
    return ow


@pytest.mark.parametrize("name,n_tokens", FULL, ids=[f"{c[0]}-{c[1]}" for c in FULL])
def test_layer_fp8_workload(name, n_tokens):
    w0, d, t, gw = _workload(name)
    w = w0 if n_tokens is None else w0.with_tokens(n_tokens)
    N = w.N
    x = t["x"][:N].contiguous()
    dm = moe.dims(N, w.M, w.E, w.k, w.H, w.S, w.Hs)
    note(f"layer fp8 {w.title} N={N}")
    gsh = None
    if w.S > 0:
        gsh = moe.quantize_ffn_fp8(t["ws_gate"], t["ws_up"], t["ws_down"])
    ids = torch.empty((N, w.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((N, w.k), dtype=torch.float32, device="cuda")
    out = moe.moe_layer_fp8(dm, x, gw, gsh, w_router=t["w_router"], router_bias=t.get("router_bias"),
                            topk_ids=ids, topk_weights=wts)
    torch.cuda.synchronize()
    xs = d["x"][:N]
    r = O.route(xs, d["w_router"], w.k, d.get("router_bias"))
    ok = r["margin"] >= TIE_MARGIN
    assert np.array_equal(ids.cpu().numpy()[ok], r["topk_ids"][ok])
    note(f"  near-tie tokens: {(~ok).sum()} of {N}")
    note("  oracle quantisation of every expert")
    ow = _oracle_all(d, gw)
    inp = {"x": xs, **ow}
    if gsh is not None:
        inp.update(_oracle_all(d, gsh, ("ws_gate", "ws_up", "ws_down")))
    note("  oracle layer (every token)")
    ref = O.moe_layer(inp, w.k, w.S, w.Hs, topk_ids=r["topk_ids"], topk_weights=r["topk_weights"])["out"]
    got = host64(out)
    assert_rows_close(got[ok], ref[ok], f"out ({ok.sum()} tokens)")
    if (~ok).any():
        out2 = moe.moe_layer_fp8(dm, x, gw, gsh, topk_ids=i32(r["topk_ids"]), topk_weights=f32(r["topk_weights"]),
                                 ids_in=True)
        torch.cuda.synchronize()
        assert_rows_close(host64(out2), ref, f"oracle routing fed, every token ({N})")
    # the cost of FP8 weights: the bf16 layer's oracle on the same routing
    if w.S == 0 and N <= 512:
        refb = O.moe_layer({"x": xs, "w_gate": d["w_gate"], "w_up": d["w_up"], "w_down": d["w_down"]}, w.k,
                           topk_ids=r["topk_ids"], topk_weights=r["topk_weights"])["out"]
        mx, l2 = errors(ref, refb)
        note(f"  FP8 vs bf16 weights: oracle rel_l2={l2:.3e} max_rel={mx:.3e}")
        assert l2 < 0.08


def test_expert_node_share_fp8():
    """16 local experts fed 32768 pre-routed rows (k = 1) with FP8 weights:
    the tile kernel at full size, every row against the oracle."""
    w, d, t, gw = _workload("qwen235_node")
    dm = moe.dims(w.N, w.M, w.E, w.k, w.H)
    note(f"layer fp8 {w.title}")
    out = moe.moe_layer_fp8(dm, t["x"], gw, topk_ids=t["topk_ids"], topk_weights=t["topk_weights"], ids_in=True)
    torch.cuda.synchronize()
    ow = _oracle_all(d, gw)
    ref = O.expert_node(d["x"], d["topk_ids"], d["topk_weights"], ow["w_gate"], ow["w_up"], ow["w_down"])["out"]
    assert_rows_close(host64(out), ref, f"expert-node rows ({w.N})")
