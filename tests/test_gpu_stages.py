"""GPU parity of each C-ABI entry point against the oracle on small and ragged
shapes, plus the edge cases of the method (N = 1, k = 1, k = E, E = 1, empty
experts, every token on one expert, exact score ties, determinism)."""
import numpy as np
import pytest
import torch

from datagen import gen
from oracle import moe_oracle as O
import expert_ffn_dispatch_amd as moe
from gpu_util import (TIE_MARGIN, assert_close, bf, f32, host64, host_bits, i32, note, upload)

pytestmark = pytest.mark.gpu

# N, M, E, k, H, S, Hs, bias
SHAPES = [
    (64, 256, 8, 2, 512, 0, 0, False),      # the tiny workload's shape
    (37, 192, 5, 2, 320, 0, 0, False),      # ragged everything
    (1, 128, 16, 4, 128, 0, 0, False),      # one token
    # up to four tokens: the layer's top-k launch also permutes (one block)
    (3, 256, 256, 16, 128, 0, 0, True),     # 256 experts, top-16 (48 assignments), bias
    (7, 256, 64, 8, 128, 0, 0, False),      # seven tokens: router scores from W_r as stored, 64 experts
    (8, 128, 160, 16, 128, 0, 0, True),     # the same over 160 experts (five 16-expert blocks per wave), top-16
    (4, 128, 20, 3, 192, 1, 64, False),     # four tokens with a shared expert
    (2, 256, 64, 8, 128, 0, 0, False),      # two tokens on the row-wise router
    (130, 320, 20, 1, 192, 0, 0, True),     # k = 1, bias
    (50, 128, 6, 6, 256, 0, 0, False),      # k = E
    (77, 256, 1, 1, 384, 0, 0, False),      # E = 1
    (200, 256, 160, 6, 128, 2, 64, False),  # many experts (some empty), shared
    (300, 512, 128, 8, 256, 1, 128, True),  # several permutation tiles, > 64 experts
    (333, 256, 8, 2, 256, 2, 128, False),   # tile kernel with the shared experts in the same launch, ragged
    (600, 256, 6, 3, 384, 1, 256, True),    # the same with 192-row tiles, 300-row groups
    (1800, 256, 6, 3, 384, 1, 256, True),   # the same with 256-row tiles, 900-row groups
    # down contraction of six stages (H = 384): each down tile loads the next
    # tile's first stages; more tiles than blocks, so blocks run several
    (2304, 4096, 8, 2, 384, 0, 0, False),
    (2304, 4096, 8, 2, 384, 1, 384, True),  # the shared segment too (contraction 384)
]


def _case(shape, seed=0):
    N, M, E, k, H, S, Hs, bias = shape
    d = gen.random_small(N, M, E, k, H, S, Hs, seed=seed, bias=bias, std=0.05)
    return d, moe.dims(N, M, E, k, H, S, Hs)


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s[:5]) for s in SHAPES])
def test_route(shape):
    d, dm = _case(shape)
    note(f"route {shape}")
    t = upload(d)
    ids, w = moe.moe_route(dm, t["x"], t["w_router"], t.get("router_bias"))
    torch.cuda.synchronize()
    r = O.route(d["x"], d["w_router"], dm.top_k, d.get("router_bias"))
    ok = r["margin"] >= TIE_MARGIN
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    assert np.array_equal(gi[ok], r["topk_ids"][ok])
    np.testing.assert_allclose(gw[ok], r["topk_weights"][ok], rtol=1e-5, atol=1e-6)
    assert np.abs(gw.astype(np.float64).sum(1) - 1).max() < 1e-5


# one- and two-token batches over 64 / 128 / 256 experts: scores from W_r rows
# with fp32 FMAs (no transpose); the larger batches check the MFMA path's
# boundary next to it; N, M, E, k, bias
ROW_ROUTE = [
    (1, 2048, 128, 8, False),     # the Qwen3-30B-shaped router, one token
    (2, 512, 64, 6, True),        # two tokens per block, bias
    (1, 1024, 256, 8, False),     # the most experts
    (2, 4096, 128, 8, True),      # eight slices of 512 rows
    (1, 768, 64, 2, False),       # three slices of 256 rows
    (1, 16384, 128, 4, False),    # slices capped at 1024 rows: 16 of them
    (3, 2048, 128, 8, False),     # three tokens: the MFMA path
    (32, 1024, 256, 8, True),     # the MFMA path at the most experts
]


@pytest.mark.parametrize("shape", ROW_ROUTE, ids=[str(s) for s in ROW_ROUTE])
def test_route_rows(shape):
    N, M, E, k, bias = shape
    note(f"route rows {shape}")
    d = gen.random_small(N, M, E, k, 128, seed=12, bias=bias, std=0.05)
    dm = moe.dims(N, M, E, k, 128)
    t = upload(d)
    ids, w = moe.moe_route(dm, t["x"], t["w_router"], t.get("router_bias"))
    ids2, w2 = moe.moe_route(dm, t["x"], t["w_router"], t.get("router_bias"))
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w.view(torch.int32), w2.view(torch.int32))
    r = O.route(d["x"], d["w_router"], k, d.get("router_bias"))
    ok = r["margin"] >= TIE_MARGIN
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    assert ok.any()
    assert np.array_equal(gi[ok], r["topk_ids"][ok])
    np.testing.assert_allclose(gw[ok], r["topk_weights"][ok], rtol=1e-5, atol=1e-6)


# batches of 8192 tokens or more over more than 32 experts: scores and top-k
# in one launch (32 tokens per block, 4-stage LDS ring over the hidden
# dimension); ragged last blocks, hidden sizes of 1..5 and 16 stages, 48 /
# 160 / 256 padded experts (the three kernel widths)
FUSED_ROUTE = [
    (8204, 256, 40, 4, True),     # last block of 12 tokens, 48 padded experts
    (8192, 320, 160, 6, False),   # five stages: the ring's remainder steps
    (8192, 128, 256, 8, True),    # two stages (fewer than the ring's depth), most experts
    (8224, 64, 64, 2, False),     # one stage
    (8200, 1024, 128, 8, True),   # sixteen stages: the ring's loop four times
]


@pytest.mark.parametrize("shape", FUSED_ROUTE, ids=[str(s) for s in FUSED_ROUTE])
def test_route_fused(shape):
    _route_twice(shape)


def _route_twice(shape):
    N, M, E, k, bias = shape
    note(f"route fused {shape}")
    d = gen.random_small(N, M, E, k, 128, seed=13, bias=bias, std=0.05)
    dm = moe.dims(N, M, E, k, 128)
    t = upload(d)
    ids, w = moe.moe_route(dm, t["x"], t["w_router"], t.get("router_bias"))
    ids2, w2 = moe.moe_route(dm, t["x"], t["w_router"], t.get("router_bias"))
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w.view(torch.int32), w2.view(torch.int32))
    r = O.route(d["x"], d["w_router"], k, d.get("router_bias"))
    ok = r["margin"] >= TIE_MARGIN
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    note(f"  near-tie tokens: {(~ok).sum()} of {N}")
    assert ok.sum() > N // 2
    assert np.array_equal(gi[ok], r["topk_ids"][ok])
    np.testing.assert_allclose(gw[ok], r["topk_weights"][ok], rtol=1e-5, atol=1e-6)
    assert np.abs(gw.astype(np.float64).sum(1) - 1).max() < 1e-5
    # every token's ids are k distinct experts in range, including near ties
    assert (gi >= 0).all() and (gi < E).all()
    assert all(len(set(row)) == k for row in gi.tolist())


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s[:5]) for s in SHAPES])
def test_permute_bit_exact(shape):
    d, dm = _case(shape)
    note(f"permute {shape}")
    r = O.route(d["x"], d["w_router"], dm.top_k, d.get("router_bias"))
    o = O.dispatch(r["topk_ids"], dm.n_experts)
    t = upload(d)
    g = moe.moe_permute(dm, i32(r["topk_ids"]), t["x"], want_x_sorted=True)
    torch.cuda.synchronize()
    for key in ("expert_counts", "expert_offsets", "sorted_to_assign", "assign_to_sorted"):
        assert np.array_equal(g[key].cpu().numpy(), o[key]), key
    assert np.array_equal(host_bits(g["x_sorted"]), O.gather(d["x"], o["sorted_to_assign"], dm.top_k))


# Both launch shapes of the permutation: one block up to 4096 assignments,
# tiles of 256 beyond; ragged last tile, more experts than a tile holds.
PERMUTE_SIZES = [(1024, 64, 4), (4097, 16, 1), (2500, 256, 8), (3000, 3, 2), (1, 1, 1)]


@pytest.mark.parametrize("size", PERMUTE_SIZES, ids=[str(s) for s in PERMUTE_SIZES])
def test_permute_launch_shapes(size):
    N, E, k = size
    note(f"permute sizes N={N} E={E} k={k}")
    rng = np.random.default_rng(N * 1000 + E)
    # skewed expert choice: a few hot experts and empty ones
    pop = rng.zipf(1.5, size=(N, k)) % E
    ids = pop.astype(np.int32)
    dm = moe.dims(N, 64, E, k, 64)
    g = moe.moe_permute(dm, i32(ids))
    torch.cuda.synchronize()
    o = O.dispatch(ids, E)
    for key in ("expert_counts", "expert_offsets", "sorted_to_assign", "assign_to_sorted"):
        assert np.array_equal(g[key].cpu().numpy(), o[key]), key


def test_permute_forced_and_empty():
    """All assignments on one expert except the k-1 others forced per token."""
    N, E, k = 1000, 32, 3
    ids = np.stack([np.full(N, 7), np.arange(N) % 5, 20 + np.arange(N) % 3], 1).astype(np.int32)
    dm = moe.dims(N, 64, E, k, 64)
    g = moe.moe_permute(dm, i32(ids))
    torch.cuda.synchronize()
    o = O.dispatch(ids, E)
    for key in ("expert_counts", "expert_offsets", "sorted_to_assign", "assign_to_sorted"):
        assert np.array_equal(g[key].cpu().numpy(), o[key]), key
    assert (o["expert_counts"] == 0).sum() > 0


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s[:5]) for s in SHAPES])
def test_grouped_ffn(shape):
    d, dm = _case(shape)
    note(f"grouped_ffn {shape}")
    r = O.route(d["x"], d["w_router"], dm.top_k, d.get("router_bias"))
    o = O.dispatch(r["topk_ids"], dm.n_experts)
    xs = O.gather(d["x"], o["sorted_to_assign"], dm.top_k)
    rng = np.random.default_rng(3)
    scale = rng.random(xs.shape[0]).astype(np.float32)
    t = upload(d)
    y = moe.moe_grouped_ffn(dm, bf(xs), i32(o["expert_offsets"]), t["w_gate"], t["w_up"], t["w_down"],
                            row_scale=f32(scale))
    torch.cuda.synchronize()
    ref = O.grouped_ffn(xs, o["expert_offsets"], d["w_gate"], d["w_up"], d["w_down"], row_scale=scale)
    assert_close(host64(y), ref, "y_sorted")


def test_grouped_ffn_shared_as_one_group():
    """Shared experts through moe_grouped_ffn: E = 1, offsets {0, N}, the S
    experts concatenated along the width."""
    N, M, S, Hs = 96, 256, 2, 192
    d = gen.random_small(N, M, 1, 1, 64, S, Hs, std=0.05)
    dm = moe.dims(N, M, 1, 1, S * Hs)
    y = moe.moe_grouped_ffn(dm, bf(d["x"]), i32([0, N]), bf(d["ws_gate"][None]), bf(d["ws_up"][None]),
                            bf(d["ws_down"][None]))
    torch.cuda.synchronize()
    ref = O.shared_experts(d["x"], d["ws_gate"], d["ws_up"], d["ws_down"], S, Hs)
    assert_close(host64(y), ref, "shared")


@pytest.mark.parametrize("weighted", [False, True])
def test_combine(weighted):
    N, M, k = 123, 320, 3
    rng = np.random.default_rng(5)
    ids = np.stack([rng.permutation(10)[:k] for _ in range(N)]).astype(np.int32)
    o = O.dispatch(ids, 10)
    y = gen.f32_to_bf16_bits(rng.standard_normal((N * k, M)).astype(np.float32))
    sh = gen.f32_to_bf16_bits(rng.standard_normal((N, M)).astype(np.float32))
    w = rng.random((N, k)).astype(np.float32) if weighted else None
    dm = moe.dims(N, M, 10, k)
    out = moe.moe_combine(dm, bf(y), i32(o["assign_to_sorted"]), f32(w) if weighted else None, bf(sh))
    torch.cuda.synchronize()
    ref = O.combine(O.bf16_to_f64(y), o["assign_to_sorted"], w, k, O.bf16_to_f64(sh))
    # only the final bf16 rounding separates them
    assert_close(host64(out), ref, "combine", tol_max=2 ** -8, tol_l2=2 ** -8)


def _layer_vs_oracle(d, dm, S=0, Hs=0, tag=""):
    t = upload(d)
    k = dm.top_k
    r = O.route(d["x"], d["w_router"], k, d.get("router_bias"))
    ids = torch.empty((dm.n_tokens, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((dm.n_tokens, k), dtype=torch.float32, device="cuda")
    out = moe.moe_layer(dm, t["x"], t["w_gate"], t["w_up"], t["w_down"], w_router=t["w_router"],
                        router_bias=t.get("router_bias"), ws_gate=t.get("ws_gate"), ws_up=t.get("ws_up"),
                        ws_down=t.get("ws_down"), topk_ids=ids, topk_weights=wts)
    torch.cuda.synchronize()
    ok = r["margin"] >= TIE_MARGIN
    gi = ids.cpu().numpy()
    assert np.array_equal(gi[ok], r["topk_ids"][ok])
    full = O.moe_layer(d, k, S, Hs)
    assert ok.sum() >= len(ok) // 2, "too few tokens above the tie margin for a useful check"
    assert_close(host64(out)[ok], full["out"][ok], f"layer out {tag}")
    # fed ids: the GPU's, with the oracle's where the margin is below 1e-6
    fi = np.where(ok[:, None], gi, r["topk_ids"]).astype(np.int32)
    fw = np.where(ok[:, None], wts.cpu().numpy(), r["topk_weights"]).astype(np.float32)
    out2 = moe.moe_layer(dm, t["x"], t["w_gate"], t["w_up"], t["w_down"], ws_gate=t.get("ws_gate"),
                         ws_up=t.get("ws_up"), ws_down=t.get("ws_down"), topk_ids=i32(fi),
                         topk_weights=f32(fw), ids_in=True)
    torch.cuda.synchronize()
    ref2 = O.moe_layer(d, k, S, Hs, topk_ids=fi, topk_weights=fw)
    assert_close(host64(out2), ref2["out"], f"layer out fed {tag}")
    return out


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s[:5]) for s in SHAPES])
def test_layer_small(shape):
    d, dm = _case(shape)
    note(f"layer {shape}")
    _layer_vs_oracle(d, dm, shape[5], shape[6], str(shape[:5]))


def test_layer_exact_ties():
    """Duplicated router columns: bit-identical scores, lower id first."""
    N, M, E, k, H = 96, 256, 8, 2, 128
    d = gen.random_small(N, M, E, k, H, std=0.05)
    d["w_router"][:, 6] = d["w_router"][:, 1]
    d["w_router"][:, 3] = d["w_router"][:, 1]
    dm = moe.dims(N, M, E, k, H)
    t = upload(d)
    ids, _ = moe.moe_route(dm, t["x"], t["w_router"])
    torch.cuda.synchronize()
    gi = ids.cpu().numpy()
    r = O.route(d["x"], d["w_router"], k)
    assert np.array_equal(gi, r["topk_ids"])     # ties resolved identically
    assert ((gi == 1).sum() > 0) and (gi == 6).sum() == 0 and (gi[:, 0] == 3).sum() == 0


def test_layer_all_on_one_expert():
    """A router bias puts every token's slot 0 on one expert."""
    N, M, E, k, H = 100, 128, 12, 2, 128
    d = gen.random_small(N, M, E, k, H, std=0.05)
    d["router_bias"] = np.zeros(E, np.float32)
    d["router_bias"][9] = 6.0      # large enough to win every token, small enough to keep margins
    dm = moe.dims(N, M, E, k, H)
    out = _layer_vs_oracle(d, dm, tag="forced")
    r = O.route(d["x"], d["w_router"], k, d["router_bias"])
    assert (r["topk_ids"][:, 0] == 9).all()


def test_layer_deterministic():
    shape = (300, 512, 128, 8, 256, 1, 128, True)
    d, dm = _case(shape)
    t = upload(d)
    outs = []
    for _ in range(2):
        o = moe.moe_layer(dm, t["x"], t["w_gate"], t["w_up"], t["w_down"], w_router=t["w_router"],
                          router_bias=t["router_bias"], ws_gate=t["ws_gate"], ws_up=t["ws_up"],
                          ws_down=t["ws_down"])
        torch.cuda.synchronize()
        outs.append(host_bits(o))
    assert np.array_equal(outs[0], outs[1])


def test_ids_out_of_range_no_fault():
    """Pre-routed ids outside [0, E) are clamped into range on the device
    (documented); the call must complete and equal the clamped ids' result."""
    N, M, E, H = 40, 128, 4, 64
    d = gen.random_small(N, M, E, 1, H, std=0.05)
    ids = (np.arange(N) % 7 - 1).astype(np.int32).reshape(N, 1)     # -1 .. 5
    w = np.ones((N, 1), np.float32)
    dm = moe.dims(N, M, E, 1, H)
    t = upload(d)
    out = moe.moe_layer(dm, t["x"], t["w_gate"], t["w_up"], t["w_down"], topk_ids=i32(ids),
                        topk_weights=f32(w), ids_in=True)
    torch.cuda.synchronize()
    ref = O.moe_layer(d, 1, topk_ids=np.clip(ids, 0, E - 1), topk_weights=w)
    assert_close(host64(out), ref["out"], "clamped ids")
