"""Pins for the oracle (CPU only).

Each check compares the oracle with something other than itself: a per-token
brute force, closed forms, invariants, a library dense SwiGLU (torch CPU), the
shared-expert concatenation identity, and the numbers the pages print.  The
mutation tests at the end plant plausible mistakes in the oracle and show that
some pin fails for each.
"""
import json
import os

import numpy as np
import pytest
import torch

import brute
from datagen import configs, gen
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

SMALL_CASES = [
    # N, M, E, k, H, S, Hs, bias
    (1, 16, 1, 1, 8, 0, 0, False),
    (5, 16, 4, 2, 8, 0, 0, False),
    (7, 8, 8, 3, 16, 2, 4, True),
    (9, 24, 6, 6, 8, 0, 0, False),
    (12, 16, 5, 1, 12, 1, 8, True),
]


def _small(case, seed=0, std=0.3):
    N, M, E, k, H, S, Hs, bias = case
    return gen.random_small(N, M, E, k, H, S, Hs, seed=seed, bias=bias, std=std)


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------

def check_brute_force(case, seed=0):
    N, M, E, k, H, S, Hs, _ = case
    inp = _small(case, seed)
    o = O.moe_layer(inp, k, S, Hs)
    b = brute.layer(inp, k, S, Hs)
    safe = o["margin"] > 1e-5
    assert np.array_equal(np.asarray(b["topk_ids"])[safe], o["topk_ids"][safe])
    np.testing.assert_allclose(np.asarray(b["topk_weights"])[safe], o["topk_weights"][safe], rtol=2e-6, atol=1e-7)
    if safe.all():
        assert np.array_equal(np.asarray(b["counts"]), o["expert_counts"])
        assert np.array_equal(np.asarray(b["sorted_to_assign"]), o["sorted_to_assign"])
        np.testing.assert_allclose(o["out"], b["out"], rtol=1e-5, atol=1e-6 * np.abs(b["out"]).max())
    # with the oracle's routing fed in, the expert math must agree to rounding
    bf = brute.layer(inp, k, S, Hs, ids_in=o["topk_ids"], w_in=o["topk_weights"])
    np.testing.assert_allclose(o["out"], bf["out"], rtol=1e-11, atol=1e-12 * max(1.0, np.abs(bf["out"]).max()))
    assert np.array_equal(np.asarray(bf["sorted_to_assign"]), o["sorted_to_assign"])


@pytest.mark.parametrize("case", SMALL_CASES)
def test_brute_force(case):
    check_brute_force(case)


# --------------------------------------------------------------------------
# the per-token form and the expert-node share
# --------------------------------------------------------------------------

def check_token_outputs(case, seed=1):
    """token_outputs (the per-token definition that full-size GPU runs are
    checked against) equals brute force fed the same routing, on every token
    and on a scrambled subset with a repeated token; and equals the batched
    layer's combine on every token."""
    N, M, E, k, H, S, Hs, _ = case
    inp = _small(case, seed)
    o = O.moe_layer(inp, k, S, Hs)
    ids, w = o["topk_ids"], o["topk_weights"]
    b = brute.layer(inp, k, S, Hs, ids_in=ids, w_in=w)
    scale = max(1.0, np.abs(b["out"]).max())
    t = O.token_outputs(inp, ids, w, np.arange(N), S, Hs)
    np.testing.assert_allclose(t, b["out"], rtol=1e-11, atol=1e-12 * scale)
    np.testing.assert_allclose(t, o["out"], rtol=1e-11, atol=1e-12 * scale)
    sub = np.array([N - 1, 0, N // 2, N - 1])
    t2 = O.token_outputs(inp, ids, w, sub, S, Hs)
    np.testing.assert_allclose(t2, b["out"][sub], rtol=1e-11, atol=1e-12 * scale)
    # arbitrary routing (not the router's): distinct random experts per
    # token, weights of either sign that do not sum to one
    rng = np.random.default_rng(seed + 17)
    ids_r = np.stack([rng.permutation(E)[:k] for _ in range(N)]).astype(np.int32)
    w_r = rng.uniform(-1.5, 2.0, size=(N, k)).astype(np.float32)
    br = brute.layer(inp, k, S, Hs, ids_in=ids_r, w_in=w_r)
    tr = O.token_outputs(inp, ids_r, w_r, np.arange(N), S, Hs)
    np.testing.assert_allclose(tr, br["out"], rtol=1e-11, atol=1e-12 * max(1.0, np.abs(br["out"]).max()))


def check_expert_node(N=23, M=16, E=6, H=8, seed=3):
    """expert_node: pre-routed rows (k = 1) with arbitrary weights, some
    experts empty; equals brute force with k = 1 (which scatters each row's
    weighted output back to its arrival position), counts and permutation
    included."""
    inp = gen.random_small(N, M, E, 1, H, seed=seed, std=0.3)
    rng = np.random.default_rng(seed)
    used = np.array([1, 2, 4])                     # the other experts get no rows
    ids = rng.choice(used, size=(N, 1)).astype(np.int32)
    ids[0, 0] = 4
    w = rng.uniform(-2.0, 3.0, size=(N, 1)).astype(np.float32)
    r = O.expert_node(inp["x"], ids, w, inp["w_gate"], inp["w_up"], inp["w_down"])
    b = brute.layer(inp, 1, ids_in=ids, w_in=w)
    assert np.array_equal(r["expert_counts"], np.asarray(b["counts"]))
    empty = np.setdiff1d(np.arange(E), used)
    assert empty.size > 0 and r["expert_counts"][empty].sum() == 0
    assert np.array_equal(r["sorted_to_assign"], np.asarray(b["sorted_to_assign"]))
    np.testing.assert_allclose(r["out"], b["out"], rtol=1e-11, atol=1e-12 * max(1.0, np.abs(b["out"]).max()))
    # and the per-token form agrees with it (k = 1)
    t = O.token_outputs(inp, ids, w, np.arange(N))
    np.testing.assert_allclose(t, b["out"], rtol=1e-11, atol=1e-12 * max(1.0, np.abs(b["out"]).max()))


@pytest.mark.parametrize("case", SMALL_CASES)
def test_token_outputs(case):
    check_token_outputs(case)


def test_expert_node():
    check_expert_node()
    check_expert_node(N=1, E=5, seed=4)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def check_zero_router(N=6, E=5, k=3, M=16, H=8):
    """W_r = 0: all scores tie, so ids = [0..k), weights = 1/k, counts =
    [N]*k + [0]*(E-k), and slot group j holds tokens in order."""
    inp = gen.random_small(N, M, E, k, H)
    inp["w_router"][:] = 0
    o = O.moe_layer(inp, k)
    assert np.array_equal(o["topk_ids"], np.tile(np.arange(k, dtype=np.int32), (N, 1)))
    np.testing.assert_allclose(o["topk_weights"], np.full((N, k), 1.0 / k), rtol=3e-7)   # float32 rounding
    assert list(o["expert_counts"]) == [N] * k + [0] * (E - k)
    exp = np.array([n * k + j for j in range(k) for n in range(N)])
    assert np.array_equal(o["sorted_to_assign"], exp)


def check_k_equals_E(N=7, E=4, M=16, H=8):
    """k = E: weights are the full softmax; sorted slot e*N + n holds
    assignment n*E + slot_of(e)."""
    inp = gen.random_small(N, M, E, E, H, std=0.3)
    o = O.moe_layer(inp, E)
    p = o["probs"]
    w_by_expert = np.zeros_like(p)
    np.put_along_axis(w_by_expert, o["topk_ids"].astype(np.int64), o["topk_weights"], axis=1)
    np.testing.assert_allclose(w_by_expert, p, rtol=1e-6)
    assert list(o["expert_counts"]) == [N] * E
    slot_of = np.argsort(o["topk_ids"], axis=1)          # slot holding expert e
    exp = np.array([n * E + slot_of[n, e] for e in range(E) for n in range(N)])
    assert np.array_equal(o["sorted_to_assign"], exp)


def check_bias_forces_expert(N=9, E=6, k=2, M=16, H=8, hot=4):
    inp = gen.random_small(N, M, E, k, H)
    inp["router_bias"] = np.zeros(E, np.float32)
    inp["router_bias"][hot] = 50.0
    o = O.moe_layer(inp, k)
    assert (o["topk_ids"][:, 0] == hot).all()
    assert o["expert_counts"][hot] == N


def check_duplicate_columns_tie(N=40, E=8, k=2, M=32, H=8):
    """Two identical router columns give bit-identical probabilities; the
    lower id must come first whenever either is chosen."""
    inp = gen.random_small(N, M, E, k, H, std=0.3)
    inp["w_router"][:, 5] = inp["w_router"][:, 2]
    o = O.moe_layer(inp, k)
    ids = o["topk_ids"]
    has5 = (ids == 5).any(axis=1)
    assert has5.sum() == 0 or ((ids == 2).any(axis=1)[has5]).all()
    both = (ids == 2).any(axis=1) & has5
    for n in np.nonzero(both)[0]:
        assert list(ids[n]).index(2) < list(ids[n]).index(5)
    assert ((ids == 2).any(axis=1)).sum() > 0   # the tie was exercised


def test_closed_forms():
    check_zero_router()
    check_k_equals_E()
    check_bias_forces_expert()
    check_duplicate_columns_tie()


def check_dense_swiglu(N=6, M=24, H=40):
    """E = 1, k = 1: the layer is one dense SwiGLU FFN; compare with torch's
    F.silu and matmul on the CPU in float64."""
    inp = gen.random_small(N, M, 1, 1, H, std=0.2)
    o = O.moe_layer(inp, 1)
    t = lambda u: torch.from_numpy(O.bf16_to_f32(u).astype(np.float64))
    x, wg, wu, wd = t(inp["x"]), t(inp["w_gate"][0]), t(inp["w_up"][0]), t(inp["w_down"][0])
    ref = (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)) @ wd.T
    np.testing.assert_allclose(o["out"], ref.numpy(), rtol=1e-12, atol=1e-14)


def check_shared_concat(N=5, M=16, Hs=12, S=2):
    """S shared experts of width Hs = one SwiGLU of width S*Hs (down is linear
    in the intermediate dimension)."""
    inp = gen.random_small(N, M, 1, 1, 8, S=S, Hs=Hs, std=0.2)
    sh = O.shared_experts(inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"], S, Hs)
    t = lambda u: torch.from_numpy(O.bf16_to_f32(u).astype(np.float64))
    x = t(inp["x"])
    ref = (torch.nn.functional.silu(x @ t(inp["ws_gate"]).T) * (x @ t(inp["ws_up"]).T)) @ t(inp["ws_down"]).T
    np.testing.assert_allclose(sh, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_library_swiglu():
    check_dense_swiglu()
    check_shared_concat()


# --------------------------------------------------------------------------
# invariants on a real workload shape
# --------------------------------------------------------------------------

def check_invariants(o, N, E, k):
    ids, w = o["topk_ids"], o["topk_weights"].astype(np.float64)
    assert ids.shape == (N, k)
    assert all(len(set(r)) == k for r in ids.tolist())
    assert np.abs(w.sum(axis=1) - 1.0).max() <= 1e-6
    assert (np.diff(w, axis=1) <= 1e-7).all()            # descending slots
    c, off, s2a, a2s = o["expert_counts"], o["expert_offsets"], o["sorted_to_assign"], o["assign_to_sorted"]
    assert c.sum() == N * k and off[0] == 0 and off[-1] == N * k
    assert np.array_equal(np.diff(off), c)
    assert np.array_equal(s2a[a2s], np.arange(N * k)) and np.array_equal(a2s[s2a], np.arange(N * k))
    flat = ids.reshape(-1)
    for e in range(E):
        grp = s2a[off[e]:off[e + 1]]
        assert (flat[grp] == e).all()
        assert (np.diff(grp) > 0).all()                   # stable


def test_invariants_tiny_workload():
    w = configs.TINY
    d = gen.generate(w)
    o = O.moe_layer(d, w.k)
    check_invariants(o, w.N, w.E, w.k)
    xs = O.gather(d["x"], o["sorted_to_assign"], w.k)
    assert np.array_equal(xs, d["x"][o["sorted_to_assign"] // w.k])


# --------------------------------------------------------------------------
# the pages' printed numbers
# --------------------------------------------------------------------------

def test_pages_numbers():
    g = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))
    mx = g["mixtral_decode_batch"]
    N, k, E = mx["tokens"], mx["top_k"], mx["experts"]
    # the Mixtral-shaped workload is exactly the printed decode batch
    assert (configs.MIXTRAL.N, configs.MIXTRAL.k, configs.MIXTRAL.E) == (N, k, E)
    # route a batch of that size (small hidden size keeps it cheap; the
    # identity holds for any scores)
    inp = gen.random_small(N, 64, E, k, 8, std=0.3)
    o = O.moe_layer(inp, k)
    assert o["expert_counts"].sum() == N * g["top2_assignments"]["assignments_per_token"]
    assert o["expert_counts"].mean() == mx["mean_rows_per_expert"]
    assert o["expert_counts"].mean() / N == mx["ffn_mfu_topk_over_experts"]
    q = g["qwen3_30b_a3b"]
    w = configs.QWEN30
    assert (w.E, w.k) == (q["routed_experts"], q["top_k"])
    # expert parameters of the Qwen3-30B-A3B-shaped layer over 48 layers
    # stay below the printed total and the active ones below the active count
    per_expert = 3 * w.M * w.H
    assert per_expert * w.E * q["layers"] < q["total_params_billion"] * 1e9
    assert per_expert * w.k * q["layers"] < q["active_params_billion"] * 1e9
    assert g["findep_expert_cost"]["gemms_per_expert"] == 3


# --------------------------------------------------------------------------
# mutation tests: plant a mistake in the oracle, some pin must fail
# --------------------------------------------------------------------------

def _all_pins():
    for case in SMALL_CASES[1:3]:
        check_brute_force(case)
    check_zero_router()
    check_k_equals_E()
    check_bias_forces_expert()
    check_duplicate_columns_tie()
    check_dense_swiglu()
    check_shared_concat()
    w = configs.TINY
    d = gen.generate(w)
    check_invariants(O.moe_layer(d, w.k), w.N, w.E, w.k)
    check_token_outputs(SMALL_CASES[2])
    check_expert_node()


def _mut_tie_high(p, k):
    N, E = p.shape
    eid = np.broadcast_to(-np.arange(E), (N, E))
    order = np.lexsort((eid, -p), axis=1)
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(p, ids, axis=1)
    return ids, (sel / sel.sum(axis=1, keepdims=True)).astype(np.float32), np.full(N, 1.0)


def _mut_no_renorm(p, k):
    ids, _, m = ORIG["topk"](p, k)
    return ids, np.take_along_axis(p, ids, axis=1).astype(np.float32), m


def _mut_silu_sign(X, wg, wu, wd):
    G = X @ O.bf16_to_f64(wg).T
    U = X @ O.bf16_to_f64(wu).T
    h = G / (1.0 + np.exp(G)) * U
    return h @ O.bf16_to_f64(wd).T, h


def _mut_gate_up_swapped(X, wg, wu, wd):
    return ORIG["swiglu"](X, wu, wg, wd)


def _mut_unstable(topk_ids, E):
    d = ORIG["dispatch"](topk_ids, E)
    s2a = d["sorted_to_assign"].copy()
    off = d["expert_offsets"]
    for e in range(E):
        s2a[off[e]:off[e + 1]] = s2a[off[e]:off[e + 1]][::-1]
    a2s = np.empty_like(s2a)
    a2s[s2a] = np.arange(s2a.size, dtype=np.int32)
    d["sorted_to_assign"], d["assign_to_sorted"] = s2a, a2s
    return d


def _mut_combine_wrong_map(y, a2s, w, k, shared=None):
    s2a = np.argsort(np.asarray(a2s))
    return ORIG["combine"](y, s2a, w, k, shared)


def _mut_drop_shared(y, a2s, w, k, shared=None):
    return ORIG["combine"](y, a2s, w, k, None)


def _mut_gather_mod(x, s2a, k):
    return np.asarray(x)[np.asarray(s2a) % max(1, x.shape[0])]


def _mut_no_softmax_max(logits):
    l = np.asarray(logits, dtype=np.float32)
    z = np.exp(l)
    return z / z.sum(axis=1, keepdims=True) * np.float32(1.0 + 1e-3)


def _mut_token_outputs_slot0_weight(inp, topk_ids, topk_weights, tokens, S=0, Hs=0):
    w = np.array(topk_weights, np.float32, copy=True)
    w[:] = w[:, :1]
    return ORIG["token_outputs"](inp, topk_ids, w, tokens, S, Hs)


def _mut_expert_node_no_weight(x, topk_ids, topk_weights, w_gate, w_up, w_down):
    return ORIG["expert_node"](x, topk_ids, np.ones_like(np.asarray(topk_weights)), w_gate, w_up, w_down)


ORIG = {name: getattr(O, name) for name in ("topk", "swiglu", "dispatch", "combine", "gather", "softmax32",
                                            "token_outputs", "expert_node")}

MUTANTS = [
    ("topk", _mut_tie_high),
    ("topk", _mut_no_renorm),
    ("swiglu", _mut_silu_sign),
    ("swiglu", _mut_gate_up_swapped),
    ("dispatch", _mut_unstable),
    ("combine", _mut_combine_wrong_map),
    ("combine", _mut_drop_shared),
    ("gather", _mut_gather_mod),
    ("softmax32", _mut_no_softmax_max),
    ("token_outputs", _mut_token_outputs_slot0_weight),
    ("expert_node", _mut_expert_node_no_weight),
]


def test_pins_pass_unmutated():
    _all_pins()


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    with pytest.raises(AssertionError):
        _all_pins()
