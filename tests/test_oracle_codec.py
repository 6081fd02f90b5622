"""Pins for the oracle's e4m3 codec and the quantiser's f32 division (CPU only).

Each check ties the oracle to something other than itself: torch's own
float8_e4m3fn codec (a library routine), a brute-force nearest-value encoder
over the enumerated value set, exact rational arithmetic for the division, the
format facts printed on the pages (tests/golden/e4m3_format.txt), and hand
values from the OCP E4M3 definition.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


ALL_CODES = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _all_bf16_f32():
    bits = np.arange(65536, dtype=np.uint32) << 16
    return bits.view(np.float32)


def _brute_encode(y):
    """Nearest e4m3 code by enumeration: 127 non-negative finite magnitudes, ties to the
    even code, saturation above 448, sign kept, NaN to 0x7F|sign."""
    mags = _torch_decode(np.arange(0x7F, dtype=np.uint8))  # codes 0x00..0x7E, increasing
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    sign = np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    idx = np.searchsorted(mags, a)               # first mag >= a
    idx = np.clip(idx, 1, 126)
    lo, hi = mags[idx - 1], mags[idx]
    dlo, dhi = a - lo, hi - a
    pick = np.where(dlo < dhi, idx - 1, np.where(dhi < dlo, idx, np.where((idx - 1) % 2 == 0, idx - 1, idx)))
    pick = np.where(a <= mags[0], 0, pick)
    pick = np.where(a >= 448.0, 0x7E, pick)
    code = (pick.astype(np.uint8) | sign)
    code = np.where(np.isnan(y), 0x7F | sign, code).astype(np.uint8)
    return code


# ------------------------------------------------------------ decode ----

def test_decode_matches_torch_e4m3fn(oracle_mod):
    ours = oracle_mod.e4m3_decode(ALL_CODES)
    ref = _torch_decode(ALL_CODES)
    nan_o, nan_r = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_o, nan_r)
    assert set(np.nonzero(nan_o)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan_o], ref[~nan_r])
    assert np.array_equal(np.signbit(ours[~nan_o]), np.signbit(ref[~nan_r]))


def test_decode_format_facts_from_pages(oracle_mod):
    g = _golden("e4m3_format.txt")
    vals = oracle_mod.e4m3_decode(ALL_CODES)
    finite = vals[np.isfinite(vals)]
    assert finite.max() == g["max_normal"] == 448.0
    assert finite.min() == -448.0
    # 3 mantissa bits: the spacing of codes in [1, 2) is 2^-3
    ones = np.sort(finite[(finite >= 1.0) & (finite < 2.0)])
    assert len(ones) == 2 ** int(g["mantissa_bits"])
    assert np.allclose(np.diff(ones), 2.0 ** -g["mantissa_bits"])


def test_decode_hand_values(oracle_mod):
    d = lambda c: float(oracle_mod.e4m3_decode(np.array([c], np.uint8))[0])
    assert d(0x38) == 1.0
    assert d(0x08) == 2.0 ** -6          # smallest normal
    assert d(0x01) == 2.0 ** -9          # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert d(0x7E) == 448.0
    assert d(0x3A) == 1.25
    assert d(0xB8) == -1.0
    assert d(0x00) == 0.0 and not math.copysign(1.0, d(0x00)) < 0
    assert d(0x80) == 0.0 and math.copysign(1.0, d(0x80)) < 0


def test_decode_monotone_and_counts(oracle_mod):
    vals = oracle_mod.e4m3_decode(ALL_CODES)
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(vals[0x80:0xFF], -pos)
    assert np.isfinite(vals).sum() == 254 and np.isnan(vals).sum() == 2


def test_roundtrip_all_codes(oracle_mod):
    vals = oracle_mod.e4m3_decode(ALL_CODES)
    back = oracle_mod.e4m3_encode(vals)
    assert np.array_equal(back, ALL_CODES)   # NaN codes keep their sign, -0 -> 0x80


# ------------------------------------------------------------ encode ----

def test_encode_hand_values(oracle_mod):
    e = lambda y: int(oracle_mod.e4m3_encode(np.array([y]))[0])
    assert e(1.0) == 0x38
    assert e(1.0625) == 0x38          # halfway 1 and 1.125 -> even mantissa
    assert e(1.1875) == 0x3A          # halfway 1.125 and 1.25 -> even mantissa (1.25)
    assert e(470.0) == 0x7E           # above the max: saturate
    assert e(464.0) == 0x7E
    assert e(447.99) == 0x7E
    assert e(1e30) == 0x7E and e(-1e30) == 0xFE
    assert e(math.inf) == 0x7E and e(-math.inf) == 0xFE
    assert e(-0.0) == 0x80 and e(0.0) == 0x00
    assert e(2.0 ** -10) == 0x00      # tie between 0 and the smallest subnormal -> 0
    assert e(1.5 * 2.0 ** -9) == 0x02  # tie between 1 and 2 subnormal steps -> even
    assert e(2.5 * 2.0 ** -9) == 0x02
    assert e(-2.0 ** -6) == 0x88
    assert e(7.5 * 2.0 ** -9) == 0x08  # rounds up into the smallest normal
    assert e(math.nan) == 0x7F and e(-math.nan) == 0xFF


def test_encode_matches_torch_in_range(oracle_mod):
    """torch's f32 -> float8_e4m3fn rounds to nearest even; it does not saturate, so
    compare only where |y| <= 448."""
    y = _all_bf16_f32()
    y = y[np.isfinite(y) & (np.abs(y) <= 448.0)]
    rng = np.random.default_rng(0)
    extra = (rng.standard_normal(200000) * rng.choice([1e-3, 1e-1, 1.0, 30.0, 200.0], 200000)).astype(np.float32)
    extra = extra[np.abs(extra) <= 448.0]
    y = np.concatenate([y, extra])
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle_mod.e4m3_encode(y.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_encode_matches_brute_force_every_bf16(oracle_mod):
    y = _all_bf16_f32().astype(np.float64)
    assert np.array_equal(oracle_mod.e4m3_encode(y), _brute_encode(y))


SCALES = [1.0, 0.125, 3.0, 0.1, 36.5 / 448.0, 4.40625 / 448.0, 0.0078125, 1e-3, 7.0]


@pytest.mark.parametrize("scale", SCALES)
def test_quantize_every_bf16_matches_brute_force(oracle_mod, scale):
    """Quantiser = one f32 division then one e4m3 rounding, over all 65536 bf16 inputs."""
    bits = np.arange(65536, dtype=np.uint16)
    x = _all_bf16_f32()
    with np.errstate(all="ignore"):
        y = (x / np.float32(scale)).astype(np.float32)
    assert np.array_equal(oracle_mod.quantize(bits, scale), _brute_encode(y.astype(np.float64)))


# ---------------------------------------------------------- division ----

def _round_fraction_to_f32(r: Fraction) -> float:
    """Round a rational to the nearest binary32 (ties to even) with integer arithmetic only."""
    if r == 0:
        return 0.0
    neg = r < 0
    r = -r if neg else r
    n, d = r.numerator, r.denominator
    e = n.bit_length() - d.bit_length()          # 2^e <= r < 2^(e+2)
    if Fraction(n, d) < Fraction(2) ** e:
        e -= 1
    if Fraction(n, d) >= Fraction(2) ** (e + 1):
        e += 1
    e = max(e, -126)                              # subnormals share the smallest exponent
    scaled = Fraction(n, d) / (Fraction(2) ** (e - 23))
    q, rem = divmod(scaled.numerator, scaled.denominator)
    twice = 2 * rem
    if twice > scaled.denominator or (twice == scaled.denominator and q % 2 == 1):
        q += 1
    if e > 127 or (e == 127 and q >= 2 ** 24):
        val = math.inf
    else:
        val = math.ldexp(q, e - 23)
    return -val if neg else val


@pytest.mark.parametrize("scale", [0.1, 3.0, 36.5 / 448.0, 1.0 / 3.0, 0.0078125])
def test_division_is_correctly_rounded_f32(oracle_mod, scale):
    s32 = float(np.float32(scale))
    rng = np.random.default_rng(7)
    bits = np.concatenate([rng.integers(0, 65536, 3000, dtype=np.uint32),
                           np.arange(0, 65536, 97, dtype=np.uint32)]).astype(np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x)]
    got = oracle_mod.div_f32(x, s32)
    for xi, gi in zip(x.tolist(), got.tolist()):
        want = _round_fraction_to_f32(Fraction(xi) / Fraction(s32))
        assert want == gi or (want == 0.0 and gi == 0.0), (xi, s32, gi, want)
