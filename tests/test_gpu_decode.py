"""GPU parity of the single-launch decode layer.

moe_layer (and moe_layer_fp8) run batches of at most 8 tokens and 64
assignments as one cooperative launch: router, top-k, permutation, grouped
SwiGLU and combine with grid-wide barriers in between.  Each case checks that
the shape really takes that path, that the ids equal the oracle's outside the
tie margin, that the output meets the parity bars against the oracle, and that
the same layer run as separate kernels (forced by per-stage events) agrees.
The barrier keeps its state in the workspace: workspaces filled with zeros,
with random bytes, and shared with calls of other shapes must all work.
"""
import numpy as np
import pytest
import torch

from datagen import configs, gen
from oracle import fp8 as F
from oracle import moe_oracle as O
import expert_ffn_dispatch_amd as moe
from gpu_util import TIE_MARGIN, assert_close, host64, note, upload

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="the single-launch decode path is switched off in the library: its first run ended "
                            "the process with a segmentation fault inside the layer call, cause not yet found"),
]

# N, M, E, k, H, bias
SHAPES = [
    (1, 256, 8, 2, 256, False),
    (3, 512, 16, 2, 384, False),     # six assignments over 16 experts: empty experts
    (8, 1024, 64, 6, 256, True),     # 48 assignments, router bias
    (5, 256, 128, 8, 128, False),    # 40 assignments over 128 experts, one chunk of H per split
    (2, 128, 256, 8, 128, False),    # the most experts, the smallest hidden size
    (8, 384, 32, 8, 512, False),     # 64 assignments: the limit
    (1, 640, 8, 1, 256, True),       # k = 1
    (7, 2048, 128, 8, 768, False),   # Qwen3-30B-shaped, 7 tokens
]


def _events():
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(moe._lib.MOE_STAGE_EVENTS)]
    for e in evs:
        e.record()
    return evs


def _run(dm, t, ids, wts, out=None, ws=None, split=False):
    if split:
        moe.moe_set_stage_events(_events())
    return moe.moe_layer(dm, t["x"], t["w_gate"], t["w_up"], t["w_down"], w_router=t["w_router"],
                         router_bias=t.get("router_bias"), topk_ids=ids, topk_weights=wts, out=out, ws=ws)


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_decode_layer(shape):
    N, M, E, k, H, bias = shape
    note(f"decode layer {shape}")
    dm = moe.dims(N, M, E, k, H)
    assert moe.moe_layer_single_launch(dm)
    d = gen.random_small(N, M, E, k, H, seed=31, bias=bias, std=0.05)
    t = upload(d)
    ids = torch.empty((N, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((N, k), dtype=torch.float32, device="cuda")
    out = _run(dm, t, ids, wts)
    out2 = _run(dm, t, None, None)
    ids_s = torch.empty_like(ids)
    wts_s = torch.empty_like(wts)
    out_s = _run(dm, t, ids_s, wts_s, split=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "repeated calls differ"
    r = O.route(d["x"], d["w_router"], k, d.get("router_bias"))
    ok = r["margin"] >= TIE_MARGIN
    assert ok.any()
    assert np.array_equal(ids.cpu().numpy()[ok], r["topk_ids"][ok])
    np.testing.assert_allclose(wts.cpu().numpy()[ok], r["topk_weights"][ok], rtol=1e-5, atol=1e-6)
    ref = O.moe_layer(d, k, topk_ids=r["topk_ids"], topk_weights=r["topk_weights"])["out"]
    assert_close(host64(out)[ok], ref[ok], "out")
    # the separate-kernel path: same ids, outputs within the parity bars of each other
    assert np.array_equal(ids_s.cpu().numpy()[ok], ids.cpu().numpy()[ok])
    assert_close(host64(out)[ok], host64(out_s)[ok], "single launch vs separate kernels")


def test_decode_layer_fp8():
    N, M, E, k, H = 4, 512, 32, 4, 512
    note(f"decode layer fp8 {(N, M, E, k, H)}")
    dm = moe.dims(N, M, E, k, H)
    assert moe.moe_layer_single_launch(dm, fp8=True)
    d = gen.random_small(N, M, E, k, H, seed=32, std=0.05)
    t = upload(d)
    gw = moe.quantize_ffn_fp8(t["w_gate"], t["w_up"], t["w_down"])
    ids = torch.empty((N, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((N, k), dtype=torch.float32, device="cuda")
    out = moe.moe_layer_fp8(dm, t["x"], gw, w_router=t["w_router"], topk_ids=ids, topk_weights=wts)
    torch.cuda.synchronize()
    r = O.route(d["x"], d["w_router"], k)
    ok = r["margin"] >= TIE_MARGIN
    assert np.array_equal(ids.cpu().numpy()[ok], r["topk_ids"][ok])
    ow = {}
    for n, q, s in (("w_gate", gw.gate, gw.gate_scale), ("w_up", gw.up, gw.up_scale),
                    ("w_down", gw.down, gw.down_scale)):
        oq, os_ = F.quantize_rows(d[n])
        assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_), n
        ow[n] = F.DequantizedExperts(oq, os_)
    ref = O.moe_layer({**d, **ow}, k, topk_ids=r["topk_ids"], topk_weights=r["topk_weights"])["out"]
    assert_close(host64(out)[ok], ref[ok], "out")


@pytest.mark.parametrize("fill", ["zeros", "random", "shared"])
def test_decode_workspace_state(fill):
    """The barrier's words live in the caller's workspace and are never
    cleared: any prior content must do, including that of calls of another
    shape (separate kernels) on the same workspace between decode calls."""
    N, M, E, k, H = 2, 512, 16, 4, 256
    note(f"decode workspace {fill}")
    dm = moe.dims(N, M, E, k, H)
    big = moe.dims(64, M, E, k, H)
    nbytes = max(moe.moe_layer_workspace_bytes(dm), moe.moe_layer_workspace_bytes(big))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    if fill == "zeros":
        ws.zero_()
    else:
        g = torch.Generator(device="cuda").manual_seed(5)
        ws.copy_(torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g))
    d = gen.random_small(N, M, E, k, H, seed=33, std=0.05)
    t = upload(d)
    db = gen.random_small(64, M, E, k, H, seed=34, std=0.05)
    tb = upload(db)
    r = O.route(d["x"], d["w_router"], k)
    ok = r["margin"] >= TIE_MARGIN
    ref = O.moe_layer(d, k, topk_ids=r["topk_ids"], topk_weights=r["topk_weights"])["out"]
    first = None
    for i in range(4):
        out = _run(dm, t, None, None, ws=ws)
        if fill == "shared":
            _run(big, tb, None, None, ws=ws)          # 64 tokens: separate kernels, same workspace
        torch.cuda.synchronize()
        assert_close(host64(out)[ok], ref[ok], f"out, call {i}")
        if first is None:
            first = out.clone()
        assert torch.equal(out.view(torch.int16), first.view(torch.int16)), f"call {i} differs"


def test_decode_workload_qwen30():
    """Qwen3-30B-shaped decode at 1 and 8 tokens (the bench's launch)."""
    w0 = configs.get("qwen30")
    d = gen.generate(w0)
    t = upload(d)
    for n in (1, 8):
        w = w0.with_tokens(n)
        note(f"decode {w.title} N={n}")
        dm = moe.dims(n, w.M, w.E, w.k, w.H)
        assert moe.moe_layer_single_launch(dm)
        x = t["x"][:n].contiguous()
        ids = torch.empty((n, w.k), dtype=torch.int32, device="cuda")
        wts = torch.empty((n, w.k), dtype=torch.float32, device="cuda")
        out = moe.moe_layer(dm, x, t["w_gate"], t["w_up"], t["w_down"], w_router=t["w_router"],
                            topk_ids=ids, topk_weights=wts)
        torch.cuda.synchronize()
        xs = d["x"][:n]
        r = O.route(xs, d["w_router"], w.k)
        ok = r["margin"] >= TIE_MARGIN
        assert np.array_equal(ids.cpu().numpy()[ok], r["topk_ids"][ok])
        toks = np.nonzero(ok)[0]
        ref = O.token_outputs({"x": xs, "w_gate": d["w_gate"], "w_up": d["w_up"], "w_down": d["w_down"]},
                              r["topk_ids"], r["topk_weights"], toks)
        assert_close(host64(out)[toks], ref, f"out ({len(toks)} tokens)")
