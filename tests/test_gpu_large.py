"""GPU parity of the grouped SwiGLU GEMMs when a token matrix spans more than
4 GiB.  Below that size the tile kernel addresses token rows by 32-bit byte
offsets; above it, by 64-bit pointers (with 128-row tiles).  Here both the
sorted input rows (530000 x 4096 bf16, 4.34 GB) and the intermediate h
(530000 x 4096) are past the limit, so gate+up and down both take the 64-bit
form.  Rows repeat a seeded random block of 4099 rows (the kernels do not
depend on the values), and the oracle checks sampled rows, among them rows
whose byte offsets exceed 2^32."""
import numpy as np
import pytest
import torch

from datagen import gen
from oracle import moe_oracle as O
import expert_ffn_dispatch_amd as moe
from gpu_util import assert_close, bf, host64, i32, note

pytestmark = pytest.mark.gpu

BLOCK = 4099


def test_grouped_ffn_token_matrix_over_4gib():
    M, H = 4096, 4096
    counts = np.array([131101, 0, 398899], np.int64)      # ragged, one empty expert
    E = len(counts)
    A = int(counts.sum())
    N, k = A // 2, 2
    assert A * M * 2 > 2 ** 32 and A * H * 2 > 2 ** 32
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    note(f"grouped_ffn over 4 GiB: A={A} M={M} H={H} E={E}")
    block = gen.normal_bf16((BLOCK, M), 91, 0, 0, std=0.5)
    wg = gen.normal_bf16((E, H, M), 91, 1, 0, std=0.02)
    wu = gen.normal_bf16((E, H, M), 91, 2, 0, std=0.02)
    wd = gen.normal_bf16((E, M, H), 91, 3, 0, std=0.02)
    x_sorted = bf(block).repeat((A + BLOCK - 1) // BLOCK, 1)[:A].contiguous()
    dm = moe.dims(N, M, E, k, H)
    y = moe.moe_grouped_ffn(dm, x_sorted, i32(offsets), bf(wg), bf(wu), bf(wd))
    torch.cuda.synchronize()
    del x_sorted
    rng = np.random.default_rng(7)
    rows = {0, int(offsets[1]) - 1, int(offsets[2]), A - 1, 2 ** 31 // (2 * M), 2 ** 32 // (2 * M),
            2 ** 32 // (2 * M) - 1, 2 ** 32 // (2 * H) + 17}
    rows |= set(int(r) for r in rng.integers(0, A, 24))
    rows |= set(int(r) for r in rng.integers(2 ** 32 // (2 * M), A, 8))
    rows = np.array(sorted(rows), np.int64)
    got = host64(y[torch.from_numpy(rows).to(y.device)])
    ref = np.zeros((len(rows), M), np.float64)
    for e in range(E):
        sel = np.nonzero((rows >= offsets[e]) & (rows < offsets[e + 1]))[0]
        if len(sel) == 0:
            continue
        X = O.bf16_to_f64(block[rows[sel] % BLOCK])
        ref[sel] = O.swiglu(X, wg[e], wu[e], wd[e])[0]
    assert_close(got, ref, f"y_sorted ({len(rows)} sampled rows)")
