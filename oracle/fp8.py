"""Oracle for FP8 (OCP E4M3) expert weights with one scale per output channel.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT (same rules as moe_oracle.py:
only the tests, the smoke check and the bench's CPU-baseline leg use it).

Source: the page "MoE 少算 FLOPs，延迟反而涨了：慢在搬 token 的路上" (wink.run),
section on what to do about the cost, lists quantising weights and
activations as a way to move fewer bytes, and says its numerical error must be
measured.  The pages fix no format, so the reading taken here is:

  * format: OCP 8-bit floating point E4M3 (1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits).  Exponent field 0 holds the subnormals
    m * 2^-9; S.1111.111 is NaN; there is no infinity; the largest finite
    magnitude is 448 (S.1111.110).
  * quantisation of a weight matrix [rows][K] (rows = output channels, K the
    contraction): per row, amax = max |w| and scale = amax / 448 in float32
    (scale = 1 for an all-zero row); each weight becomes the E4M3 value
    nearest to the float32 quotient w / scale, ties to the even code,
    magnitudes at or above 448 saturate to 448, the sign is kept (a negative
    weight that rounds to zero is -0).
  * dequantised weight = value(code) * scale.  The layer is the bf16 layer's
    definition with these dequantised weights (moe_oracle, unchanged).

Pinned by tests/test_oracle_fp8.py against torch's float8_e4m3fn conversion
(a library routine), a brute-force nearest-value search over all 256 codes,
the format's own bounds, and a layer whose weights are exactly representable.
"""
import concurrent.futures as cf
import os
from typing import Tuple

import numpy as np

E4M3_MAX = 448.0


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code, from its bit fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9           # subnormal: m/8 * 2^(1-7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3_table() -> np.ndarray:
    """float64 value of every code 0..255 (NaN at 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3_table()
_POS = _TABLE[:0x7F]          # codes 0..0x7E: 0 .. 448, strictly increasing


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to each float32 value, ties to the even code,
    saturating at +-448.

    Within [2^e, 2^(e+1)) (e >= -6) the representable values are the
    multiples of 2^(e-3); below 2^-6 they are the multiples of 2^-9.  So the
    nearest value is rint(a / step) * step with rint rounding half to even,
    and an even multiple is an even code (codes are consecutive multiples
    within a binade, and a binade starts at an even code)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v.astype(np.float64)), E4M3_MAX)
    _, ex = np.frexp(a)                        # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                 # binade exponent, subnormals share -6
    step = np.ldexp(1.0, e - 3)
    val = np.rint(a / step) * step             # exact: step is a power of two
    code = np.searchsorted(_POS, val).astype(np.uint8)
    assert np.array_equal(_POS[code], val)
    return code | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(code, dtype=np.uint8)]


def quantize_rows(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-output-channel quantisation of bf16 weights [..., K] (uint16 bits).
    Returns codes (uint8, same shape) and scales (float32, shape[:-1]).
    Rows are independent; they are taken in blocks of about 2^20 weights, on
    a few threads, only to keep the temporaries small and the wait short."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    K = w_bits.shape[-1]
    flat = w_bits.reshape(-1, K)
    q = np.empty(flat.shape, np.uint8)
    scale = np.empty(flat.shape[0], np.float32)
    step = max(1, (1 << 20) // K)

    def block(r0):
        w = (flat[r0:r0 + step].astype(np.uint32) << np.uint32(16)).view(np.float32)
        amax = np.abs(w).max(axis=-1)
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        q[r0:r0 + step] = e4m3_encode((w / s[:, None]).astype(np.float32))
        scale[r0:r0 + step] = s

    starts = range(0, flat.shape[0], step)
    if len(starts) > 1:
        with cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(block, starts))
    else:
        for r0 in starts:
            block(r0)
    return q.reshape(w_bits.shape), scale.reshape(w_bits.shape[:-1])


def dequantize_rows(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """value(code) * scale, float64."""
    out = e4m3_decode(q)
    out *= np.asarray(scale, np.float64)[..., None]
    return out


class DequantizedExperts:
    """Expert weights [E][rows][K] held as codes + scales, dequantised one
    expert at a time on indexing (float64 [rows][K]), so that the layer oracle
    can read full-size models expert by expert."""

    def __init__(self, q: np.ndarray, scale: np.ndarray):
        self.q, self.scale = q, scale
        self.shape = q.shape

    def __len__(self):
        return self.shape[0]

    def __getitem__(self, e):
        return dequantize_rows(self.q[e], self.scale[e])


def quantize_experts(w_bits: np.ndarray) -> DequantizedExperts:
    q, s = quantize_rows(w_bits)
    return DequantizedExperts(q, s)
