"""moe_layer_noalloc (the layer with the library's own workspace array) against
moe_layer with a caller workspace: the same kernels on the same inputs, so the
outputs, ids and weights must be identical bit for bit.  Two calls in a row,
the second on a smaller batch, so that the second finds the first's contents
in the shared array; then a shape whose workspace exceeds the array must be
refused before anything is enqueued."""
import numpy as np
import pytest
import torch

from datagen import configs, gen
import expert_ffn_dispatch_amd as moe
from expert_ffn_dispatch_amd import _lib
from gpu_util import note, upload

pytestmark = pytest.mark.gpu


def _call_both(w, t, N):
    dm = moe.dims(N, w.M, w.E, w.k, w.H, w.S, w.Hs)
    x = t["x"][:N].contiguous()
    outs = []
    for fn in (moe.moe_layer, moe.moe_layer_noalloc):
        ids = torch.full((N, w.k), -1, dtype=torch.int32, device="cuda")
        wts = torch.full((N, w.k), -1.0, dtype=torch.float32, device="cuda")
        out = fn(dm, x, t["w_gate"], t["w_up"], t["w_down"], w_router=t["w_router"], topk_ids=ids,
                 topk_weights=wts)
        torch.cuda.synchronize()
        outs.append((out, ids, wts))
    (o1, i1, w1), (o2, i2, w2) = outs
    note(f"  N={N}: workspace {moe.moe_layer_workspace_bytes(dm, 0) / 2**20:.1f} MiB of "
         f"{_lib.MOE_NOALLOC_SCRATCH_BYTES / 2**20:.0f}")
    assert torch.equal(i1, i2), "routing ids differ"
    assert torch.equal(w1.view(torch.int32), w2.view(torch.int32)), "routing weights differ"
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "layer outputs differ"
    assert torch.isfinite(o2.float()).all()


@pytest.mark.parametrize("name,sizes", [("qwen30", (512, 37)), ("mixtral", (156, 5))])
def test_noalloc_matches_layer(name, sizes):
    w = configs.get(name)
    note(f"no-alloc layer, {w.title}")
    d = gen.generate(w)
    t = upload(d)
    for N in sizes:
        _call_both(w, t, N)


def test_noalloc_refuses_large_shapes():
    # the Qwen3-235B-shaped layer needs about 0.7 GiB of workspace
    w = configs.QWEN235
    dm = moe.dims(w.N, w.M, w.E, w.k, w.H)
    assert moe.moe_layer_workspace_bytes(dm, 0) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    fake = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_noalloc(dm, fake, fake, fake, fake, w_router=fake, out=fake)
    assert ei.value.code == _lib.MOE_ERR_WORKSPACE
    assert "moe_layer_noalloc" in str(ei.value)
