"""Pins of the oracle's UE5M3 block scale.

The Finer-is-Better page (key findings; significance) compares a custom
unsigned wide-exponent scale, UE5M3, with E4M3 + hierarchical scaling +
4-over-6, without giving its encoding.  Reading: 5 exponent bits, bias 15,
3 mantissa bits, subnormals, no infinities, 0xFF NaN.  The bias has nothing
on the pages to pin it ("parity unpinned" for the bias); everything built on
the reading is pinned here: the encoder against round-half-even computed
from the binade spacing in exact rationals (a different algorithm from the
oracle's nearest-of-255 search), exactly representable blocks, brute force
against the exact argmin, and the wide range that makes prevent-zero moot.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import exact_ref as X

UE5M3 = 2
ABSMAX, PZ, FOS, BF, GIVEN = 0, 1, 2, 3, 4
NONE, TAMAX, USER, SEARCH = 0, 1, 2, 3
TOP = Fraction(7, 4) * Fraction(2) ** 16
MIN_NORMAL = Fraction(2) ** -14
SUB_STEP = Fraction(2) ** -17


def reading_value(code):
    e, m = code >> 3, code & 7
    return m * SUB_STEP if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 15)


VALUES = {c: reading_value(c) for c in range(0xFF)}
CODE_OF = {v: c for c, v in VALUES.items()}


def rne_by_spacing(v: Fraction) -> Fraction:
    """Round v >= 0 half-to-even onto the UE5M3 grid from the spacing of its
    binade (Python's round() of a Fraction rounds half to even)."""
    if v >= TOP:
        return TOP
    if v < MIN_NORMAL:
        return round(v / SUB_STEP) * SUB_STEP
    e = math.floor(math.log2(v))
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    step = Fraction(2) ** (e - 3)
    return min(round(v / step) * step, TOP)


def from_bits(u):
    return np.uint32(u).view(np.float32)


def test_decode_all_codes(O):
    prev = -1.0
    for c in range(0xFF):
        v = O.ue5m3_decode(c)
        assert Fraction(v) == VALUES[c]
        assert v > prev
        prev = v
    assert math.isnan(O.ue5m3_decode(0xFF))
    assert O.ue5m3_decode(0xFE) == 114688.0 and O.ue5m3_decode(1) == 2.0 ** -17


def test_encode_all_bf16_patterns(O):
    lib = O.lib()
    for h in range(0, 0x7F80):                        # every non-negative finite bf16
        v = from_bits(h << 16)
        want = CODE_OF[rne_by_spacing(Fraction(float(v)))]
        assert lib.oracle_ue5m3_encode(float(v)) == want, float(v)


def test_encode_midpoints(O):
    vals = [VALUES[c] for c in range(0xFF)]
    pts = []
    for a, b in zip(vals[:-1], vals[1:]):
        mid = np.float32(float((a + b) / 2))
        x = mid
        for _ in range(3):
            x = np.nextafter(x, np.float32(0))
        for _ in range(7):
            pts.append(x)
            x = np.nextafter(x, np.float32(np.inf))
    pts += [np.float32(114688.0), np.float32(120000.0), np.float32(1e30)]
    for v in pts:
        assert O.ue5m3_encode(v) == CODE_OF[rne_by_spacing(Fraction(float(v)))], float(v)
    assert O.ue5m3_encode(float("inf")) == 0xFE
    assert O.ue5m3_encode(float("nan")) == 0xFF
    assert O.ue5m3_encode(2.0 ** -18) == 0             # tie between 0 and 2^-17 goes to even 0


def exact_blocks(rng, codes, B):
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    mags = rng.integers(0, 8, (len(codes), B))
    mags[:, 0] = 7
    sign = np.where(rng.integers(0, 2, (len(codes), B)) == 1, -1.0, 1.0).astype(np.float32)
    S = np.array([float(VALUES[int(c)]) for c in codes], np.float32)
    return (grid[mags] * sign * S[:, None]).astype(np.float32)


@pytest.mark.parametrize("B", [4, 16, 32])
def test_roundtrip_exact(O, B):
    rng = np.random.default_rng(B)
    codes = rng.integers(1, 0xFF, 64)
    codes[:4] = [1, 7, 0x80, 0xFE]                      # subnormal, largest subnormal, 2.0, top
    y = exact_blocks(rng, codes, B).reshape(8, -1)
    for st in (ABSMAX, FOS, BF):
        r = O.quantize(y, fmt=UE5M3, block=B, strategy=st)
        assert np.array_equal(r["dequant"].view(np.uint32), y.view(np.uint32)), st
        assert np.all(r["mse"] == 0)
        if st != FOS:
            # a smaller scale saturates the |q| = 6 element, so the block's own code is the
            # smallest one without error: abs-max finds it and brute force ties to it
            assert r["scales"].reshape(-1).tolist() == codes.tolist(), st


def ue5m3_sse_exact(block, code, g=Fraction(1)):
    return X.block_sse_exact(block, VALUES[code] * g)


@pytest.mark.parametrize("B", [4, 8])
@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_matches_exact_argmin(O, B, seed):
    rng = np.random.default_rng(100 + seed)
    x = (rng.standard_normal((2, 8 * B)) * np.exp(rng.uniform(-6, 6, (2, 1)))).astype(np.float32)
    r = O.quantize(x, fmt=UE5M3, block=B, strategy=BF)
    blocks = x.reshape(-1, B)
    for b, blk in enumerate(blocks):
        sse = {c: ue5m3_sse_exact(blk, c) for c in range(1, 0xFF)}
        best = min(sse, key=lambda c: (sse[c], c))
        got = int(r["scales"].reshape(-1)[b])
        if got != best:                                   # only at a near-tie of the exact errors
            assert float(sse[got] - sse[best]) <= 1e-6 * float(sse[best]), (b, got, best)


def test_brute_force_never_worse(O):
    rng = np.random.default_rng(9)
    x = rng.laplace(0, 1, (16, 256)).astype(np.float32)
    rb = O.quantize(x, fmt=UE5M3, block=16, strategy=BF)
    for st in (ABSMAX, PZ, FOS):
        r = O.quantize(x, fmt=UE5M3, block=16, strategy=st)
        assert np.all(rb["sse"] <= r["sse"]), st


def test_abs_max_candidates_restated(O):
    """s6 = RNE_UE5M3(fl(a / fl(6 g))) and s4 likewise; 4-over-6 takes s4 only
    when its fp32 error is strictly smaller."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((8, 128)) * 3.0).astype(np.float32)
    g = np.float32(0.37)
    a = np.abs(x).reshape(-1, 16).max(axis=1)
    s6 = [CODE_OF[rne_by_spacing(Fraction(float(np.float32(v / (np.float32(6.0) * g)))))] for v in a]
    s4 = [CODE_OF[rne_by_spacing(Fraction(float(np.float32(v / (np.float32(4.0) * g)))))] for v in a]
    ra = O.quantize(x, fmt=UE5M3, block=16, strategy=ABSMAX, global_mode=USER, user_g=g)
    assert ra["scales"].reshape(-1).tolist() == s6
    rf = O.quantize(x, fmt=UE5M3, block=16, strategy=FOS, global_mode=USER, user_g=g)
    picks = rf["scales"].reshape(-1)
    assert all(p in (c6, c4) for p, c6, c4 in zip(picks, s6, s4))


def test_wide_range_needs_no_prevent_zero(O):
    """At 1e-4 the E4M3 abs-max scale underflows to 0 (region A of the page);
    UE5M3's smallest scale 2^-17 keeps every block with a value above
    0.25 * 2^-17 non-zero, so prevent-zero changes nothing."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((16, 256)) * np.float32(1e-4)).astype(np.float32)
    ra = O.quantize(x, fmt=UE5M3, block=16, strategy=ABSMAX)
    rp = O.quantize(x, fmt=UE5M3, block=16, strategy=PZ)
    assert np.array_equal(ra["scales"], rp["scales"])
    assert np.all(ra["scales"] > 0)
    nonzero = (ra["codes"] & 0x77).reshape(-1, 8).any(axis=1)
    assert np.all(nonzero)


def test_given_codes_use_all_eight_bits(O):
    x = np.full((1, 16), 2.0, np.float32)
    scales = np.array([[0x80]], np.uint8)                   # 2^(16-15) = 2.0
    r = O.quantize(x, fmt=UE5M3, block=16, strategy=GIVEN, scales_in=scales)
    assert np.all(r["dequant"] == 2.0)                       # |x| / 2 = 1 -> code 2 -> 1 * 2
    assert np.all((r["codes"] & 0x77) == 0x22)


def test_global_modes(O):
    x = np.ones((2, 32), np.float32)
    for gm in (TAMAX, SEARCH):
        with pytest.raises(ValueError):
            O.quantize(x, fmt=UE5M3, block=16, strategy=ABSMAX, global_mode=gm)
    r = O.quantize(x, fmt=UE5M3, block=16, strategy=ABSMAX, global_mode=USER, user_g=0.5)
    assert r["g"] == np.float32(0.5)
