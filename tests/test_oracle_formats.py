"""Pins of the oracle's number formats against things other than itself.

E2M1 ("OCP E2M1" in "Finer is Better (with the Right Scaling)", method
part 1): exact rational nearest-value search and Python's banker's round().
E4M3 / E8M0 scales: torch's float8_e4m3fn / float8_e8m0fnu decoders and
torch's round-half-to-even e4m3 cast (which does not saturate, so values are
clamped to 448 first).  bf16 / fp16 narrowing: torch / numpy casts.
MXFP4 power-of-two abs-max scale (MR-GPTQ page, section 1): closed form over
every fp32 exponent.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def f32(x):
    return np.float32(x)


def bits(x):
    return struct.unpack("<I", struct.pack("<f", float(np.float32(x))))[0]


def from_bits(b):
    return np.float32(struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0])


def e2m1_exact(u):
    """Nearest E2M1 magnitude by exact rationals, ties to the even code."""
    if math.isnan(u):
        return 0
    if math.isinf(u):
        return 7
    a = abs(Fraction(float(u)))
    best, best_d = None, None
    for m, g in enumerate(GRID):
        d = abs(a - g)
        if best is None or d < best_d or (d == best_d and m % 2 == 0):
            best, best_d = m, d
    return best


def e2m1_banker(u):
    """Same rounding written as Python round() on the binade's spacing."""
    a = abs(float(u))
    if a >= 4:
        v = 2 * round(a / 2)
    elif a >= 2:
        v = round(a)
    else:
        v = round(2 * a) / 2
    v = min(v, 6)
    return [0, 0.5, 1, 1.5, 2, 3, 4, 6].index(v)


def neighbourhood(x, k=4):
    b = bits(x)
    out = []
    for d in range(-k, k + 1):
        nb = b + d
        if 0 <= nb < 0x7F800000:
            out.append(from_bits(nb))
    return out


def test_e2m1_midpoints_exhaustive(O):
    pts = [0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 8.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]
    for p in pts:
        for u in neighbourhood(p, 4):
            for s in (1.0, -1.0):
                uu = np.float32(s * u)
                want = e2m1_exact(float(uu))
                assert O.e2m1_mag(uu) == want, (float(uu), want)
                assert e2m1_banker(uu) == want


def test_e2m1_all_bf16_patterns(O):
    lib = O.lib()
    for h in range(0, 1 << 16, 1):
        u = from_bits(h << 16)
        want = e2m1_exact(float(u))
        got = lib.oracle_e2m1_mag(float(u))
        assert got == want, (h, float(u), got, want)


def test_e2m1_special_values(O):
    assert O.e2m1_mag(float("nan")) == 0
    assert O.e2m1_mag(float("inf")) == 7
    assert O.e2m1_mag(-float("inf")) == 7
    assert O.e2m1_mag(3.0e38) == 7
    assert O.e2m1_mag(1e30) == 7
    assert O.e2m1_mag(1e-45) == 0
    for m in range(8):
        assert O.lib().oracle_e2m1_value(m) == float(GRID[m])


def test_e4m3_decode_all_codes(O):
    ref = torch.arange(128, dtype=torch.uint8).view(torch.float8_e4m3fn).double()
    for c in range(128):
        want = ref[c].item()
        got = O.e4m3_decode(c)
        if c == 0x7F:
            assert math.isnan(got) and math.isnan(want)
        else:
            assert got == want, c
        # bit 7 is ignored for an unsigned scale
        got_hi = O.e4m3_decode(c | 0x80)
        assert (math.isnan(got_hi) and math.isnan(got)) or got_hi == got
    assert O.e4m3_decode(0x7E) == 448.0
    assert O.e4m3_decode(0x01) == 2.0 ** -9


def torch_e4m3(vals):
    t = torch.tensor(np.asarray(vals, dtype=np.float32))
    return t.clamp(max=448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_all_bf16_patterns(O):
    vals = [from_bits(h << 16) for h in range(0, 0x7F80)]   # every non-negative finite bf16
    want = torch_e4m3(vals)
    lib = O.lib()
    for v, w in zip(vals, want):
        assert lib.oracle_e4m3_encode(float(v)) == int(w), float(v)


def test_e4m3_encode_midpoints(O):
    codes = np.arange(0, 0x7F)
    vals = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    pts = []
    for a, b in zip(vals[:-1], vals[1:]):
        mid = (a + b) / 2
        pts += neighbourhood(np.float32(mid), 2)
    pts += neighbourhood(np.float32(448.0), 3) + [np.float32(464.0), np.float32(1e30)]
    want = torch_e4m3(pts)
    for v, w in zip(pts, want):
        assert O.e4m3_encode(v) == int(w), float(v)
    assert O.e4m3_encode(float("inf")) == 0x7E
    assert O.e4m3_encode(float("nan")) == 0x7F
    assert O.e4m3_encode(2.0 ** -10) == 0          # tie between 0 and 2^-9 goes to even 0
    assert O.e4m3_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 1


def test_e8m0_decode_all_codes(O):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double()
    for c in range(255):
        assert O.e8m0_decode(c) == ref[c].item() == 2.0 ** (c - 127)
    assert math.isnan(O.e8m0_decode(255))


def test_e8m0_absmax_closed_form(O):
    """code = floor(log2 a) - 2 + 127, clamped at 0, for every exponent."""
    for e in range(-149, 128):
        for frac in (1.0, 1.5, 1.9999999):
            a = np.float32(math.ldexp(frac, e))
            if a == 0 or math.isinf(a):
                continue
            m, ex = math.frexp(float(a))
            want = max(ex - 1 - 2 + 127, 0)
            if float(a) < 2.0 ** -124:
                want = 0
            assert O.e8m0_absmax_code(a) == want, (e, frac)
    assert O.e8m0_absmax_code(0.0) == 0
    # the block maximum lands in [4, 8) after division by the scale
    rng = np.random.default_rng(0)
    for a in rng.uniform(1e-30, 1e30, 500).astype(np.float32):
        s = O.e8m0_decode(O.e8m0_absmax_code(a))
        assert 4.0 <= float(a) / s < 8.0


def test_bf16_narrowing_vs_torch(O):
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(3000).astype(np.float32))
    vals += list((rng.standard_normal(2000) * 1e-39).astype(np.float32))     # subnormals
    for h in range(0x3F80, 0x3F90):                                           # exact ties
        vals.append(from_bits((h << 16) | 0x8000))
        vals.append(from_bits((h << 16) | 0x8001))
        vals.append(from_bits((h << 16) | 0x7FFF))
    vals += [np.float32(3.4028235e38), np.float32(-3.39e38), np.float32(0.0), np.float32(-0.0)]
    want = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, w in zip(vals, want):
        assert O.bf16_from_f32(v) == int(w), float(v)
    assert O.bf16_from_f32(float("nan")) & 0x7FC0 == 0x7FC0
    for h in range(0, 1 << 16, 7):
        f = O.bf16_to_f32(h)
        ref = torch.tensor([h], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float().item()
        assert (math.isnan(f) and math.isnan(ref)) or f == ref


def test_f16_narrowing_vs_numpy(O):
    rng = np.random.default_rng(2)
    vals = list(rng.standard_normal(3000).astype(np.float32) * 100)
    vals += list((rng.standard_normal(2000) * 1e-6).astype(np.float32))      # fp16 subnormals
    vals += [np.float32(65504.0), np.float32(65519.0), np.float32(65520.0), np.float32(1e6),
             np.float32(2.0 ** -25), np.float32(2.0 ** -24 * 1.5), np.float32(-0.0)]
    want = np.asarray(vals, np.float32).astype(np.float16).view(np.uint16)
    for v, w in zip(vals, want):
        assert O.f16_from_f32(v) == int(w), float(v)
    for h in range(0, 1 << 16, 5):
        f = O.f16_to_f32(h)
        ref = np.array([h], np.uint16).view(np.float16).astype(np.float32)[0]
        assert (math.isnan(f) and math.isnan(ref)) or f == ref
