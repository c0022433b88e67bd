"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad arguments on the host before anything is enqueued
(no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import expert_ffn_dispatch_amd as moe
from expert_ffn_dispatch_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")

FAKE = 1 << 20          # an aligned address that is never dereferenced
MIS = FAKE + 4          # a misaligned one


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from expert_ffn_dispatch_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)
    assert lib.moe_abi_version() == 1


def _err(lib):
    return lib.moe_last_error().decode()


def D(N=8, M=128, E=4, k=2, H=128, S=0, Hs=0):
    return moe.dims(N, M, E, k, H, S, Hs)


BAD_DIMS = [
    (D(N=0), 1, "n_tokens"),
    (D(M=100), 1, "hidden"),
    (D(M=32), 1, "hidden"),
    (D(E=0), 1, "n_experts"),
    (D(E=300, k=2), 2, "n_experts"),
    (D(k=5), 1, "top_k"),
    (D(E=32, k=17), 1, "top_k"),
    (D(H=96), 1, "expert_width"),
    (D(S=1, Hs=100), 1, "n_shared*shared_width"),
    (D(S=-1), 1, "n_shared"),
]


@pytest.mark.parametrize("d,code,word", BAD_DIMS, ids=[b[2] + str(i) for i, b in enumerate(BAD_DIMS)])
def test_bad_dims(lib, d, code, word):
    n = ctypes.c_size_t(0)
    r = lib.moe_layer_workspace_bytes(ctypes.byref(d), 0, ctypes.byref(n))
    assert r == code and word in _err(lib)
    r = lib.moe_layer(ctypes.byref(d), 0, *([FAKE] * 13), 1 << 40, None)
    assert r == code and word in _err(lib)


def test_route_pointer_checks(lib):
    d = D()
    assert lib.moe_route(ctypes.byref(d), None, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == _lib.MOE_ERR_INVALID
    assert "x is NULL" in _err(lib)
    assert lib.moe_route(ctypes.byref(d), MIS, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == _lib.MOE_ERR_INVALID
    assert "aligned" in _err(lib)
    assert lib.moe_route(ctypes.byref(d), FAKE, FAKE, MIS, FAKE, FAKE, FAKE, 1 << 30, None) == _lib.MOE_ERR_INVALID
    assert lib.moe_route(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, 0, None) == _lib.MOE_ERR_WORKSPACE
    # small batches keep fp32 partial scores per contraction slice; larger
    # ones also hold the transposed router (E padded to 16)
    small = moe.moe_route_workspace_bytes(D(N=156, M=6144, E=8))
    assert small >= 156 * 8 * 4 and small % 256 == 0
    assert moe.moe_route_workspace_bytes(D(N=4096, M=6144, E=8)) >= 16 * 6144 * 2 + 4096 * 16 * 4


def _layer(lib, d, flags=0, ws_bytes=None, **over):
    args = dict(x=FAKE, w_router=FAKE, router_bias=None, w_gate=FAKE, w_up=FAKE, w_down=FAKE,
                ws_gate=None, ws_up=None, ws_down=None, topk_ids=None, topk_weights=None, out=FAKE, ws=FAKE)
    args.update(over)
    return lib.moe_layer(ctypes.byref(d), flags, args["x"], args["w_router"], args["router_bias"],
                         args["w_gate"], args["w_up"], args["w_down"], args["ws_gate"], args["ws_up"],
                         args["ws_down"], args["topk_ids"], args["topk_weights"], args["out"], args["ws"],
                         0 if ws_bytes is None else ws_bytes, None)


def test_layer_argument_rules(lib):
    d = D()
    assert _layer(lib, d, flags=8) == _lib.MOE_ERR_INVALID and "flags" in _err(lib)
    # IDS_IN: router must be absent, ids/weights present
    assert _layer(lib, d, flags=1) == _lib.MOE_ERR_INVALID and "w_router" in _err(lib)
    assert _layer(lib, d, flags=1, w_router=None) == _lib.MOE_ERR_INVALID and "topk_ids" in _err(lib)
    # router required without IDS_IN
    assert _layer(lib, d, w_router=None) == _lib.MOE_ERR_INVALID and "w_router" in _err(lib)
    # shared weights iff n_shared > 0
    assert _layer(lib, d, ws_gate=FAKE) == _lib.MOE_ERR_INVALID and "n_shared" in _err(lib)
    ds = D(S=2, Hs=64)
    assert _layer(lib, ds) == _lib.MOE_ERR_INVALID and "ws_gate" in _err(lib)
    # workspace
    assert _layer(lib, d, ws=None) == _lib.MOE_ERR_WORKSPACE and "NULL" in _err(lib)
    assert _layer(lib, d, ws_bytes=16) == _lib.MOE_ERR_WORKSPACE and "needed" in _err(lib)
    assert _layer(lib, d, ws=FAKE + 16, ws_bytes=1 << 30) == _lib.MOE_ERR_WORKSPACE


def test_noalloc_argument_rules(lib):
    """moe_layer_noalloc: the moe_layer rules, and shapes whose workspace
    exceeds the library's array are refused before any device call."""
    def call(d, flags=0, **over):
        a = dict(x=FAKE, w_router=FAKE, router_bias=None, w_gate=FAKE, w_up=FAKE, w_down=FAKE, ws_gate=None,
                 ws_up=None, ws_down=None, topk_ids=None, topk_weights=None, out=FAKE)
        a.update(over)
        return lib.moe_layer_noalloc(ctypes.byref(d), flags, a["x"], a["w_router"], a["router_bias"], a["w_gate"],
                                     a["w_up"], a["w_down"], a["ws_gate"], a["ws_up"], a["ws_down"], a["topk_ids"],
                                     a["topk_weights"], a["out"], None)
    assert call(D(N=0)) == _lib.MOE_ERR_INVALID and "n_tokens" in _err(lib)
    assert call(D(), flags=8) == _lib.MOE_ERR_INVALID and "flags" in _err(lib)
    assert call(D(), w_gate=None) == _lib.MOE_ERR_INVALID and "w_gate" in _err(lib)
    assert call(D(), x=MIS) == _lib.MOE_ERR_INVALID and "aligned" in _err(lib)
    big = D(N=8192, M=4096, E=128, k=8, H=1536)
    assert moe.moe_layer_workspace_bytes(big, 0) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    assert call(big) == _lib.MOE_ERR_WORKSPACE and "scratch" in _err(lib)
    fits = D(N=512, M=2048, E=128, k=8, H=768)
    assert moe.moe_layer_workspace_bytes(fits, 0) <= _lib.MOE_NOALLOC_SCRATCH_BYTES


def test_other_entry_points_reject(lib):
    d = D()
    assert lib.moe_permute(ctypes.byref(d), None, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30,
                           None) == _lib.MOE_ERR_INVALID
    assert lib.moe_permute(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                           None) == _lib.MOE_ERR_INVALID and "x is NULL" in _err(lib)
    assert lib.moe_permute(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, 0,
                           None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_grouped_ffn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 0,
                               None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_grouped_ffn(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 30,
                               None) == _lib.MOE_ERR_INVALID
    assert lib.moe_combine(ctypes.byref(d), FAKE, FAKE, MIS, None, FAKE, None) == _lib.MOE_ERR_INVALID


def _f8(**over):
    f = dict(gate=FAKE, up=FAKE, down=FAKE, gate_scale=FAKE, up_scale=FAKE, down_scale=FAKE)
    f.update(over)
    return _lib.MoeFp8Ffn(**f)


def test_fp8_entry_points_reject(lib):
    q = lib.moe_quantize_fp8
    assert q(FAKE, 0, 128, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID and "rows" in _err(lib)
    assert q(FAKE, 4, 100, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID and "cols" in _err(lib)
    assert q(None, 4, 128, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID and "w is NULL" in _err(lib)
    assert q(FAKE, 4, 128, MIS, FAKE, None) == _lib.MOE_ERR_INVALID and "aligned" in _err(lib)
    assert q(FAKE, 4, 128, FAKE, None, None) == _lib.MOE_ERR_INVALID and "scale" in _err(lib)

    g = lib.moe_grouped_ffn_fp8
    d = D(M=256, H=256)
    ok = _f8()
    assert g(ctypes.byref(D(M=192, H=256)), FAKE, FAKE, ctypes.byref(ok), None, FAKE, FAKE, 1 << 30,
             None) == _lib.MOE_ERR_UNSUPPORTED and "hidden" in _err(lib)
    assert g(ctypes.byref(D(M=256, H=192)), FAKE, FAKE, ctypes.byref(ok), None, FAKE, FAKE, 1 << 30,
             None) == _lib.MOE_ERR_UNSUPPORTED and "expert_width" in _err(lib)
    assert g(ctypes.byref(d), FAKE, FAKE, None, None, FAKE, FAKE, 1 << 30, None) == _lib.MOE_ERR_INVALID
    assert "experts is NULL" in _err(lib)
    bad = _f8(down_scale=None)
    assert g(ctypes.byref(d), FAKE, FAKE, ctypes.byref(bad), None, FAKE, FAKE, 1 << 30,
             None) == _lib.MOE_ERR_INVALID and "experts->down_scale" in _err(lib)
    bad = _f8(up=MIS)
    assert g(ctypes.byref(d), FAKE, FAKE, ctypes.byref(bad), None, FAKE, FAKE, 1 << 30,
             None) == _lib.MOE_ERR_INVALID and "experts->up" in _err(lib)
    assert g(ctypes.byref(d), FAKE, FAKE, ctypes.byref(ok), None, FAKE, FAKE, 0, None) == _lib.MOE_ERR_WORKSPACE

    L = lib.moe_layer_fp8

    def layer(dd, shared=None, flags=0, ws_bytes=1 << 40):
        return L(ctypes.byref(dd), flags, FAKE, FAKE, None, ctypes.byref(ok),
                 None if shared is None else ctypes.byref(shared), None, None, FAKE, FAKE, ws_bytes, None)

    assert layer(d, shared=ok) == _lib.MOE_ERR_INVALID and "n_shared" in _err(lib)
    ds = D(M=256, H=256, S=2, Hs=128)
    assert layer(ds) == _lib.MOE_ERR_INVALID and "shared is NULL" in _err(lib)
    assert layer(D(M=256, H=256, S=1, Hs=64), shared=ok) == _lib.MOE_ERR_UNSUPPORTED
    assert layer(d, flags=4) == _lib.MOE_ERR_INVALID and "flags" in _err(lib)
    assert layer(d, ws_bytes=16) == _lib.MOE_ERR_WORKSPACE


def test_pipelined_rejects(lib):
    d = D(N=8)
    n = ctypes.c_size_t(0)

    def call(dd, n_micro, flags=0, ws_bytes=1 << 40, **over):
        a = dict(x=FAKE, w_router=FAKE, w_gate=FAKE, w_up=FAKE, w_down=FAKE, out=FAKE)
        a.update(over)
        return lib.moe_layer_pipelined(ctypes.byref(dd), flags, n_micro, a["x"], a["w_router"], None, a["w_gate"],
                                       a["w_up"], a["w_down"], None, None, None, None, None, a["out"], FAKE,
                                       ws_bytes, None)

    assert call(d, 0) == _lib.MOE_ERR_INVALID and "n_micro" in _err(lib)
    assert call(d, 9) == _lib.MOE_ERR_INVALID and "n_micro" in _err(lib)
    assert call(D(N=100), 65) == _lib.MOE_ERR_INVALID
    assert call(d, 2, w_gate=None) == _lib.MOE_ERR_INVALID and "w_gate" in _err(lib)
    assert call(d, 2, flags=1) == _lib.MOE_ERR_INVALID and "w_router" in _err(lib)
    assert call(d, 2, ws_bytes=16) == _lib.MOE_ERR_WORKSPACE
    r = lib.moe_layer_pipelined_workspace_bytes(ctypes.byref(d), 0, 0, ctypes.byref(n))
    assert r == _lib.MOE_ERR_INVALID
    # two slots of the larger micro-batch's layer workspace
    big = moe.moe_layer_pipelined_workspace_bytes(D(N=1000), 4)
    one = moe.moe_layer_workspace_bytes(D(N=250))
    assert big == 2 * one
    assert moe.moe_layer_pipelined_workspace_bytes(D(N=1000), 1) == moe.moe_layer_workspace_bytes(D(N=1000))


def test_workspace_sizes(lib):
    def ws(d):
        return moe.moe_layer_workspace_bytes(d)
    small, big = ws(D(N=8)), ws(D(N=800))
    assert big > small
    d = D(N=4096, M=5120, E=160, k=6, H=1536, S=2, Hs=1536)
    A = 4096 * 6
    assert ws(d) >= A * 1536 * 2 + A * 5120 * 2 + 4096 * 3072 * 2 + 4096 * 5120 * 2
    assert moe.moe_grouped_ffn_workspace_bytes(D(N=10, k=2, H=256)) >= 20 * 256 * 2
    assert moe.moe_permute_workspace_bytes(D(N=1000, E=8, k=2)) >= 2 * 8 * 8 * 4


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libmoe_ffn.so")
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def test_single_launch_query(lib):
    """moe_layer_single_launch checks its arguments like the others and, with
    the single-launch path switched off in this build, reports 0 for every
    shape, decode-sized ones included."""
    v = ctypes.c_int(7)
    for n in (1, 8, 64):
        d = _lib.MoeDims(n, 2048, 128, 8, 768, 0, 0)
        assert lib.moe_layer_single_launch(ctypes.byref(d), 0, 0, ctypes.byref(v)) == _lib.MOE_OK
        assert v.value == 0
        assert lib.moe_layer_single_launch(ctypes.byref(d), 0, 1, ctypes.byref(v)) == _lib.MOE_OK
        assert v.value == 0
    d = _lib.MoeDims(1, 2048, 128, 8, 768, 0, 0)
    assert lib.moe_layer_single_launch(ctypes.byref(d), 0, 0, None) == _lib.MOE_ERR_INVALID
    assert lib.moe_layer_single_launch(ctypes.byref(d), 6, 0, ctypes.byref(v)) == _lib.MOE_ERR_INVALID
    assert "flags" in _err(lib)
    bad = _lib.MoeDims(1, 100, 128, 8, 768, 0, 0)
    assert lib.moe_layer_single_launch(ctypes.byref(bad), 0, 0, ctypes.byref(v)) == _lib.MOE_ERR_INVALID


def test_bench_refuses_several_gpus():
    """bench.py runs one GPU; --gpus 2 exits with a message before touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""
