"""Pins for the FP8 (OCP E4M3, per-output-channel scale) part of the oracle.

Each check compares oracle/fp8.py with something other than itself: torch's
float8_e4m3fn conversion (a library routine), a brute-force nearest-value
search over all 256 codes, the format's bounds, and a layer whose weights are
exactly representable (there the FP8 layer must equal the bf16 layer).  The
mutation tests plant plausible mistakes and show that some pin fails.
"""
import numpy as np
import pytest
import torch

from datagen import gen
from oracle import fp8 as F
from oracle import moe_oracle as O


def _torch_codes(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _tricky_values(seed=0, n=200_000) -> np.ndarray:
    """Every finite value, the midpoints between neighbours (the ties), one
    float32 ulp either side of them, and log-uniform magnitudes, all with
    both signs, inside [-448, 448]."""
    pos = F.e4m3_table()[:0x7F]
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    rng = np.random.default_rng(seed)
    r = np.exp2(rng.uniform(-12, np.log2(448), n)).astype(np.float32)
    v = np.concatenate([pos.astype(np.float32), mid, up, dn, r, np.float32([0.0, 2.0 ** -10, 3 * 2.0 ** -11])])
    v = np.minimum(v, np.float32(448))
    return np.concatenate([v, -v])


# --------------------------------------------------------------------------
# the pins
# --------------------------------------------------------------------------

def check_decode():
    t = F.e4m3_table()
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(t), np.isnan(lib))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], lib[ok])
    assert np.array_equal(np.signbit(t[ok]), np.signbit(lib[ok]))
    # the format's own landmarks
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isfinite(t).sum() == 254
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.all(np.diff(t[:0x7F]) > 0)


def check_encode_library():
    v = _tricky_values()
    assert np.array_equal(F.e4m3_encode(v), _torch_codes(v))


def check_encode_brute_force(seed=1, n=3000):
    rng = np.random.default_rng(seed)
    v = np.concatenate([_tricky_values(seed)[rng.integers(0, 400_000, n)],
                        (rng.standard_normal(n) * 50).astype(np.float32)])
    v = np.clip(v, -448, 448).astype(np.float32)
    t = F.e4m3_table()
    codes = np.array([c for c in range(256) if np.isfinite(t[c])])
    vals = t[codes]
    got = F.e4m3_encode(v)
    for x, g in zip(v.astype(np.float64), got):
        d = np.abs(vals - x)
        best = codes[d == d.min()]
        same_sign = best[np.signbit(t[best]) == np.signbit(x)] if x == 0 or d.min() == 0 else best
        cand = same_sign if len(same_sign) else best
        if len(cand) > 1:                     # a tie between two values: the even code
            cand = cand[(cand & 1) == 0]
        if x == 0 or np.abs(t[cand[0]]) == 0:  # zero keeps the input's sign
            cand = np.array([0x80 if np.signbit(x) else 0x00])
        assert int(g) == int(cand[0]), (x, g, cand)


def check_encode_saturates():
    v = np.float32([448, 449, 463.9, 464, 470, 500, 1e4, 3e38])
    assert np.all(F.e4m3_encode(v) == 0x7E)
    assert np.all(F.e4m3_encode(-v) == 0xFE)


def check_quantize_bounds(seed=2):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((48, 320)) * 0.02).astype(np.float32)
    w[3] = 0.0                                # an all-zero row
    w[5] = 0.0
    w[5, 17] = -0.5                           # a single non-zero
    w[7, :160] *= 1e-4                        # a wide range inside one row
    bits = gen.f32_to_bf16_bits(w)
    wf = O.bf16_to_f64(bits)
    q, s = F.quantize_rows(bits)
    assert q.dtype == np.uint8 and s.dtype == np.float32 and s.shape == (48,)
    amax = np.abs(wf).max(axis=1)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz].astype(np.float32) / np.float32(448)))
    assert np.all(s[~nz] == 1.0) and np.all(q[~nz] == 0)
    dq = F.dequantize_rows(q, s)
    assert np.all(np.abs(dq[nz]).max(axis=1) == 448.0 * s[nz].astype(np.float64))
    assert q[5, 17] == 0xFE and np.all(q[5, np.arange(320) != 17] == 0)
    # rounding error: half the local spacing, 2^-4 relative in the normal
    # range and 2^-10 * scale among the subnormals (+ the float32 quotient)
    err = np.abs(dq - wf)
    a = np.abs(wf) / s[:, None].astype(np.float64)
    bound = np.where(a >= 2.0 ** -6, a * 2.0 ** -4, 2.0 ** -10) * s[:, None] * (1 + 1e-6)
    assert np.all(err <= bound)
    assert np.array_equal(np.signbit(dq[wf != 0]), np.signbit(wf[wf != 0]))


def check_exact_layer(seed=3):
    """Weights that are E4M3 values times 2^-12, each row holding +-448 * 2^-12:
    the scale is exactly 2^-12, the codes are the chosen ones and the FP8
    layer equals the bf16 layer bit for bit."""
    N, M, E, k, H = 9, 32, 4, 2, 16
    inp = gen.random_small(N, M, E, k, H, 0, 0, seed=seed)
    rng = np.random.default_rng(seed)
    t = F.e4m3_table()
    finite = np.array([c for c in range(256) if np.isfinite(t[c]) and c not in (0x80,)], dtype=np.uint8)
    fp8 = {}
    for name, shape in (("w_gate", (E, H, M)), ("w_up", (E, H, M)), ("w_down", (E, M, H))):
        codes = rng.choice(finite, size=shape)
        codes[..., 0] = rng.choice(np.uint8([0x7E, 0xFE]), size=shape[:-1])
        vals = (t[codes] * 2.0 ** -12).astype(np.float32)
        inp[name] = gen.f32_to_bf16_bits(vals)
        q, s = F.quantize_rows(inp[name])
        assert np.all(s == np.float32(2.0 ** -12))
        assert np.array_equal(q, codes)
        fp8[name] = F.DequantizedExperts(q, s)
    ref = O.moe_layer(inp, k)
    got = O.moe_layer({**inp, **fp8}, k, topk_ids=ref["topk_ids"], topk_weights=ref["topk_weights"])
    assert np.array_equal(got["out"], ref["out"])


def _all_pins():
    check_decode()
    check_encode_library()
    check_encode_brute_force()
    check_encode_saturates()
    check_quantize_bounds()
    check_exact_layer()


def test_decode():
    check_decode()


def test_encode_matches_library():
    check_encode_library()


def test_encode_brute_force():
    check_encode_brute_force()


def test_encode_saturates():
    check_encode_saturates()


def test_quantize_bounds():
    check_quantize_bounds()


def test_exact_layer():
    check_exact_layer()


# --------------------------------------------------------------------------
# mutation tests
# --------------------------------------------------------------------------

ORIG = {n: getattr(F, n) for n in ("e4m3_encode", "e4m3_value", "quantize_rows")}


def _mut_ties_away(v):
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v.astype(np.float64)), F.E4M3_MAX)
    _, ex = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    val = np.floor(a / step + 0.5) * step
    code = np.searchsorted(F._POS, val).astype(np.uint8)
    return code | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))


def _mut_no_subnormals(v):
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v.astype(np.float64)), F.E4M3_MAX)
    a = np.where(a < 2.0 ** -6, np.where(a < 2.0 ** -7, 0.0, 2.0 ** -6), a)   # flush to zero / min normal
    return ORIG["e4m3_encode"](np.where(np.signbit(v), -a, a).astype(np.float32))


def _mut_bias8(code):
    x = ORIG["e4m3_value"](code)
    return x / 2.0 if np.isfinite(x) else x


def _mut_scale_447(w_bits):
    w = (np.asarray(w_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    amax = np.abs(w).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(447), np.float32(1)).astype(np.float32)
    return F.e4m3_encode((w / scale[..., None]).astype(np.float32)), scale


def _mut_row_block_mixup(w_bits):
    """One scale per block of rows instead of per row."""
    q, s = ORIG["quantize_rows"](w_bits)
    w = (np.asarray(w_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    amax = np.abs(w).max()
    s = np.full_like(s, amax / np.float32(448) if amax > 0 else 1)
    return F.e4m3_encode((w / s[..., None]).astype(np.float32)), s


def _mut_drop_sign(v):
    return ORIG["e4m3_encode"](np.abs(np.asarray(v, dtype=np.float32)))


MUTANTS = [
    ("e4m3_encode", _mut_ties_away),
    ("e4m3_encode", _mut_no_subnormals),
    ("e4m3_encode", _mut_drop_sign),
    ("e4m3_value", _mut_bias8),
    ("quantize_rows", _mut_scale_447),
    ("quantize_rows", _mut_row_block_mixup),
]


def test_pins_pass_unmutated():
    _all_pins()


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(F, name, mutant)
    if name == "e4m3_value":
        monkeypatch.setattr(F, "_TABLE", F.e4m3_table())
        monkeypatch.setattr(F, "_POS", F._TABLE[:0x7F])
    with pytest.raises(AssertionError):
        _all_pins()
