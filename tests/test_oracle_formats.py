"""Pins for the oracle's number formats and fp32 FMA emulation.

Each check ties the oracle to something other than itself: torch's CPU
float8_e4m3fn cast (a library routine), exact rational arithmetic
(fractions.Fraction), or closed-form values of the OCP formats.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def torch_e4m3(x):
    t = torch.tensor(np.asarray(x, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_known_values():
    # 1.0 is byte 56 (the "+56" of 8*log2(p)+56); 448 the largest finite value
    assert F.e4m3_decode(0x38) == 1.0 and F.e4m3_encode(1.0) == 0x38 == 56
    assert F.e4m3_decode(0x7E) == 448.0 and F.e4m3_encode(448.0) == 0x7E
    assert F.e4m3_decode(0x01) == 2.0 ** -9 and F.e4m3_encode(2.0 ** -9) == 0x01
    assert F.e4m3_decode(0x08) == 2.0 ** -6
    assert np.isnan(F.e4m3_decode(0x7F)) and np.isnan(F.e4m3_decode(0xFF))
    assert F.e4m3_decode(0xB8) == -1.0


def test_e4m3_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_e4m3_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-448, 448, 200000),
        rng.uniform(-0.02, 0.02, 100000),
        np.exp2(rng.uniform(-12, 8.8, 100000)) * rng.choice([-1, 1], 100000),
    ]).astype(np.float32)
    assert np.array_equal(F.e4m3_encode(x.astype(np.float64)), torch_e4m3(x))


def test_e4m3_ties_to_even_at_every_midpoint():
    vals = F.e4m3_decode(np.arange(0, 0x7E + 1))
    mids = (vals[:-1] + vals[1:]) / 2.0          # exact in fp64 and fp32
    got = F.e4m3_encode(mids)
    assert np.array_equal(got, torch_e4m3(mids))
    # the even code (mantissa lsb 0) wins each tie
    assert np.all(got % 2 == 0)


def test_e4m3_saturates():
    for v in (448.0, 449.0, 463.9, 464.0, 480.0, 1e6, np.inf):
        assert F.e4m3_encode(v) == 0x7E
        assert F.e4m3_encode(-v) == 0xFE


def test_e2m1_grid_and_rounding():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(F.e2m1_decode(np.arange(8))) == grid
    assert list(F.e2m1_decode(np.arange(8, 16))) == [-g for g in grid]
    assert np.array_equal(F.e2m1_encode(F.e2m1_decode(np.arange(16))), np.arange(16))
    # nearest on the grid by brute force, ties to the code with mantissa bit 0
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.uniform(-7, 7, 20000), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0]])
    for x in xs:
        a = min(abs(x), 6.0)
        dist = [abs(a - g) for g in grid]
        best = min(dist)
        cands = [i for i, dd in enumerate(dist) if dd == best]
        i = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        want = i | (8 if np.signbit(x) else 0)
        assert F.e2m1_encode(x) == want, x


def test_mx_shared_exponent():
    # X = 2^(floor(log2 amax) - 2): the block maximum lands in [4, 8) before
    # element rounding, the OCP MX v1.0 rule for E2M1
    for amax, e in [(6.0, 0), (1.0, -2), (0.75, -3), (8.0, 1), (7.99, 0), (2.0 ** -130, -127), (0.0, 0)]:
        assert F.mx_shared_exponent(amax) == e, amax
    assert F.e8m0_decode(127) == 1.0 and F.e8m0_decode(0) == 2.0 ** -127


def _round_f32_exact(q: Fraction) -> float:
    """Correct RNE of an exact rational to binary32, by bracketing."""
    f = float(q)                                  # correctly rounded to fp64
    lo = np.float32(f)
    cand = [np.nextafter(lo, np.float32(-np.inf)), lo, np.nextafter(lo, np.float32(np.inf))]
    best = min(cand, key=lambda c: (abs(Fraction(float(c)) - q),
                                    int(np.array(c, np.float32).view(np.uint32)) & 1))
    return float(best)


def test_fma_f32_matches_exact_rounding():
    rng = np.random.default_rng(2)
    n = 4000
    a = rng.standard_normal(n).astype(np.float32) * np.float32(1000)
    b = rng.standard_normal(n).astype(np.float32)
    c = rng.standard_normal(n).astype(np.float32) * np.float32(50)
    # crafted near-ties: c chosen so a*b + c sits on / next to a binary32 midpoint
    a2 = np.float32(1.0) + np.arange(1, 200, dtype=np.float32) * np.float32(2 ** -23)
    b2 = np.float32(1.0) + np.float32(2 ** -23) * np.float32(3)
    c2 = np.full(a2.shape, np.float32(-1.0))
    A = np.concatenate([a, a2, np.float32([1.5, 3.0, -2.0])])
    B = np.concatenate([b, np.full(a2.shape, b2), np.float32([2 ** -24 + 2 ** -47, 1.0, 2 ** -25])])
    C = np.concatenate([c, c2, np.float32([1.0, 2 ** -23, 1.0])])
    got = F.fma_f32(A, B, C)
    for i in range(A.size):
        q = Fraction(float(A[i])) * Fraction(float(B[i])) + Fraction(float(C[i]))
        assert got[i] == _round_f32_exact(q), (A[i], B[i], C[i])


def test_fma_f32_double_rounding_case():
    # a*b + c = 1 + 2^-23 + 2^-24 - 2^-70.  The fp64 sum drops the 2^-70 and
    # lands exactly on the binary32 midpoint 1 + 2^-23 + 2^-24, which a second
    # rounding sends to the even neighbour 1 + 2^-22; the exact value is just
    # below the midpoint, so the single rounding is 1 + 2^-23.
    a = np.float32(1.0 + 2 ** -23)
    b = np.float32(2 ** -24 - 2 ** -47)
    c = np.float32(1.0 + 2 ** -23)
    naive = float(np.float32(float(a) * float(b) + float(c)))
    assert naive == 1.0 + 2 ** -22
    got = F.fma_f32(a, b, c)
    q = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    assert got == _round_f32_exact(q) == 1.0 + 2 ** -23
