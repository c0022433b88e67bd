"""GPU parity of moe_layer_pipelined (micro-batches overlapped on two streams).

Each token's output must meet the parity bars against the oracle, its ids
must equal the oracle's outside the tie margin, and repeated calls must give
identical bits.  Shapes cover ragged micro-batch sizes, shared experts,
pre-routed rows, one token per micro-batch and full-size prefill workloads.
"""
import numpy as np
import pytest
import torch

from datagen import configs, gen
from oracle import moe_oracle as O
import expert_ffn_dispatch_amd as moe
from gpu_util import TIE_MARGIN, assert_close, host64, i32, f32, note, upload

pytestmark = pytest.mark.gpu

# N, M, E, k, H, S, Hs, bias, n_micro
SMALL = [
    (64, 256, 8, 2, 512, 0, 0, False, 2),
    (37, 192, 5, 2, 320, 0, 0, False, 5),      # ragged micro-batches (8, 8, 7, 7, 7)
    (200, 256, 16, 2, 256, 2, 128, False, 4),  # shared experts
    (130, 320, 20, 1, 192, 0, 0, True, 3),     # k = 1: rows stored straight into the output
    (6, 128, 4, 2, 128, 0, 0, False, 6),       # one token per micro-batch
]


@pytest.mark.parametrize("shape", SMALL, ids=[str(s) for s in SMALL])
def test_pipelined_small(shape):
    N, M, E, k, H, S, Hs, bias, nm = shape
    note(f"pipelined {shape}")
    d = gen.random_small(N, M, E, k, H, S, Hs, seed=8, bias=bias, std=0.05)
    t = upload(d)
    dm = moe.dims(N, M, E, k, H, S, Hs)
    ids = torch.empty((N, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((N, k), dtype=torch.float32, device="cuda")
    out = moe.moe_layer_pipelined(dm, nm, t["x"], t["w_gate"], t["w_up"], t["w_down"], w_router=t["w_router"],
                                  router_bias=t.get("router_bias"), ws_gate=t.get("ws_gate"), ws_up=t.get("ws_up"),
                                  ws_down=t.get("ws_down"), topk_ids=ids, topk_weights=wts)
    out2 = moe.moe_layer_pipelined(dm, nm, t["x"], t["w_gate"], t["w_up"], t["w_down"], w_router=t["w_router"],
                                   router_bias=t.get("router_bias"), ws_gate=t.get("ws_gate"),
                                   ws_up=t.get("ws_up"), ws_down=t.get("ws_down"))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    r = O.route(d["x"], d["w_router"], k, d.get("router_bias"))
    ok = r["margin"] >= TIE_MARGIN
    assert np.array_equal(ids.cpu().numpy()[ok], r["topk_ids"][ok])
    ref = O.moe_layer(d, k, S, Hs, topk_ids=r["topk_ids"], topk_weights=r["topk_weights"])["out"]
    assert_close(host64(out)[ok], ref[ok], "out")


def test_pipelined_ids_in():
    """Pre-routed rows (the expert-node share's form), three micro-batches."""
    N, M, E, H = 300, 256, 16, 256
    d = gen.random_small(N, M, E, 1, H, seed=9, std=0.05)
    rng = np.random.default_rng(9)
    ids = rng.integers(0, E, (N, 1)).astype(np.int32)
    wts = rng.uniform(0, 1, (N, 1)).astype(np.float32)
    t = upload(d)
    dm = moe.dims(N, M, E, 1, H)
    out = moe.moe_layer_pipelined(dm, 3, t["x"], t["w_gate"], t["w_up"], t["w_down"], topk_ids=i32(ids),
                                  topk_weights=f32(wts), ids_in=True)
    torch.cuda.synchronize()
    ref = O.expert_node(d["x"], ids, wts, d["w_gate"], d["w_up"], d["w_down"])["out"]
    assert_close(host64(out), ref, "pre-routed rows")


FULL = [("dsv2", 2, 24), ("qwen235", 2, 24), ("qwen235", 4, 16)]


@pytest.mark.parametrize("name,nm,sample", FULL, ids=[f"{c[0]}-{c[1]}" for c in FULL])
def test_pipelined_workload(name, nm, sample):
    torch.cuda.empty_cache()
    w = configs.get(name)
    note(f"generate {w.title}")
    d = gen.generate(w)
    t = upload(d)
    dm = moe.dims(w.N, w.M, w.E, w.k, w.H, w.S, w.Hs)
    note(f"pipelined {w.title} n_micro={nm}")
    ids = torch.empty((w.N, w.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.N, w.k), dtype=torch.float32, device="cuda")
    out = moe.moe_layer_pipelined(dm, nm, t["x"], t["w_gate"], t["w_up"], t["w_down"], w_router=t["w_router"],
                                  router_bias=t.get("router_bias"), ws_gate=t.get("ws_gate"), ws_up=t.get("ws_up"),
                                  ws_down=t.get("ws_down"), topk_ids=ids, topk_weights=wts)
    torch.cuda.synchronize()
    r = O.route(d["x"], d["w_router"], w.k, d.get("router_bias"))
    ok = r["margin"] >= TIE_MARGIN
    assert np.array_equal(ids.cpu().numpy()[ok], r["topk_ids"][ok])
    good = np.nonzero(ok)[0]
    # sample across every micro-batch
    rng = np.random.default_rng(21)
    toks = np.sort(rng.choice(good, size=min(sample, good.size), replace=False))
    ref = O.token_outputs(d, r["topk_ids"], r["topk_weights"], toks, w.S, w.Hs)
    assert_close(host64(out)[toks], ref, f"out ({len(toks)} tokens)")
    del t
