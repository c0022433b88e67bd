"""Helpers for the GPU parity tests: upload seeded inputs, read results back,
and the error metrics of the parity bar.

Parity bar (floating point): normwise max relative error
max|got - ref| / max|ref| <= 2e-2 and relative L2 error
||got - ref||_2 / ||ref||_2 <= 5e-3, got upcast from bf16/fp32 to float64.
Beside the tensor-wide bar, every token row of a layer output must meet the
same normwise max bar and a relative L2 of at most 1e-2 on its own, so that
one wrong row cannot hide in the tensor's norm: the expected per-row error is
that of two bf16 roundings (h and the output, each at most 2^-9 relative,
about 1.1e-3 RMS) plus fp32 summation order, so 1e-2 leaves a margin of three
or more, while a row with a wrong expert, weight or token is off by O(1).
Integer and byte outputs (ids, counts, offsets, permutation, gathered rows)
must match bit for bit.  Routing ids are compared on tokens whose top-k
probability margin is at least 1e-6; below that the oracle's ids are fed in.
"""
import sys

import numpy as np
import torch

from datagen import gen
from oracle import moe_oracle as O

TOL_MAX = 2e-2
TOL_L2 = 5e-3
TIE_MARGIN = 1e-6
DEV = "cuda"


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def errors(got: np.ndarray, ref: np.ndarray):
    d = np.asarray(got, np.float64) - np.asarray(ref, np.float64)
    mref = np.abs(ref).max()
    nref = np.linalg.norm(ref)
    return float(np.abs(d).max() / mref), float(np.linalg.norm(d) / nref)


def assert_close(got, ref, what: str, tol_max=TOL_MAX, tol_l2=TOL_L2):
    mx, l2 = errors(got, ref)
    note(f"  {what}: max_rel={mx:.3e} rel_l2={l2:.3e}")
    assert mx <= tol_max and l2 <= tol_l2, f"{what}: max_rel={mx:.3e} (<= {tol_max}), rel_l2={l2:.3e} (<= {tol_l2})"


ROW_TOL_MAX = 2e-2
ROW_TOL_L2 = 1e-2


def assert_rows_close(got, ref, what: str, tol_max=ROW_TOL_MAX, tol_l2=ROW_TOL_L2):
    """The tensor-wide bar, then the per-row bar on every row."""
    assert_close(got, ref, what)
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    rmax = np.abs(ref).max(axis=1)
    rl2 = np.linalg.norm(ref, axis=1)
    live = rl2 > 0
    row_max = np.abs(d).max(axis=1)[live] / rmax[live]
    row_l2 = np.linalg.norm(d, axis=1)[live] / rl2[live]
    worst = int(np.argmax(row_l2)) if row_l2.size else -1
    note(f"  {what}: per row, worst max_rel={row_max.max() if row_max.size else 0:.3e} "
         f"worst rel_l2={row_l2.max() if row_l2.size else 0:.3e} (row {worst} of {live.sum()} live)")
    # a row whose reference is exactly zero must be exactly zero
    assert np.all(d[~live] == 0), f"{what}: rows with a zero reference are not zero"
    bad = np.nonzero((row_max > tol_max) | (row_l2 > tol_l2))[0]
    assert bad.size == 0, (f"{what}: {bad.size} rows above the per-row bar (max_rel <= {tol_max}, "
                           f"rel_l2 <= {tol_l2}); first {bad[:8].tolist()}")


def upload(d: dict) -> dict:
    out = {}
    for k, v in d.items():
        if not isinstance(v, np.ndarray) or v.ndim == 0:
            continue
        if v.dtype == np.uint16:
            out[k] = bf(v)
        elif v.dtype == np.float32:
            out[k] = f32(v)
        elif v.dtype == np.int32:
            out[k] = i32(v)
    return out
