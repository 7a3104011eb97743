"""Pins for the oracle's ExpCast-FP8 bytes.

Ties the oracle's ExpCast to (a) the byte/probability relation the pages print
(golden fixture, integer z), (b) the exact E4M3 encoding of 2^z computed by
torch's CPU float8 cast, over a dense grid of z, and (c) its own defining
clamp and ordering properties.
"""
import math
import os

import numpy as np
import torch

from oracle import formats as F
from oracle.attention import expcast_bytes, DEFAULT_BETA

GOLD = os.path.join(os.path.dirname(__file__), "golden", "expcast_integer_z.txt")


def bytes_for_z(z, beta=DEFAULT_BETA):
    """ExpCast of log2-domain z via the oracle's single FMA, with S=z, A=8,
    B=56+beta-8*0 (row max 0)."""
    z = np.asarray(z, np.float32)
    B = np.float32(F.f32(56.0 + beta))
    return expcast_bytes(z.astype(np.float64), 8.0, np.full(z.shape, B, np.float64))


def exact_e4m3_of_exp2(z):
    p = np.exp2(np.asarray(z, np.float64)).astype(np.float32)
    return torch.tensor(p).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)


def test_golden_integer_z():
    rows = [l.split() for l in open(GOLD) if l.strip() and not l.startswith("#")]
    for z, byte, val in rows:
        z, byte, val = int(z), int(byte), float(val)
        for beta in (DEFAULT_BETA, 0.0, -0.49, 0.3):
            assert bytes_for_z(np.float32(z), beta) == byte
        assert F.e4m3_decode(byte) == val == 2.0 ** z
        assert exact_e4m3_of_exp2(z) == byte


def test_below_normal_range_is_zero():
    # ExpCast is linear in log p; E4M3 codes 1..7 are linear in p, so the
    # formula stops matching: exact E4M3(2^z) is 4, 2, 1 at z=-7,-8,-9 while
    # the ExpCast byte 8z+56+beta rounds to 0 there (expected, not a bug).
    assert list(exact_e4m3_of_exp2([-7, -8, -9])) == [4, 2, 1]
    assert list(bytes_for_z(np.float32([-7, -8, -9, -10, -40]))) == [0, 0, 0, 0, 0]


def test_dense_grid_against_exact_exp2_cast():
    z = -np.arange(0, 12 * 4096 + 1, dtype=np.float64) / 4096.0     # [-12, 0], step 2^-12
    got = bytes_for_z(z).astype(np.int64)
    ref = exact_e4m3_of_exp2(z)
    d = got - ref
    normal = z >= -6
    assert np.abs(d[normal]).max() == 1
    assert np.abs(d).max() <= 4
    # the default beta centres the pre-rounding offset: mean code error ~ 0
    assert abs(d[normal].mean()) < 0.05
    # and the decoded probabilities agree with 2^z on average in the normal range
    rel = F.e4m3_decode(got[normal]) / np.exp2(z[normal]) - 1.0
    assert abs(rel.mean()) < 0.01 and np.abs(rel).max() < 0.09


def test_monotone_and_clamped():
    z = np.sort(np.random.default_rng(3).uniform(-20, 0, 100000)).astype(np.float32)
    b = bytes_for_z(z).astype(np.int64)
    assert np.all(np.diff(b) >= 0)
    assert b.min() >= 0 and b.max() <= 56
    # clamp at both ends of [0, 56]; -inf (masked key) and NaN give 0
    S = np.array([10.0, -np.inf, np.nan, -1e30], np.float64)
    out = expcast_bytes(S, 8.0, np.full(4, 56.0))
    assert list(out) == [56, 0, 0, 0]


# ---- range-shifted ExpCast: the same FMA with the addend 120 + beta ----

def shifted_bytes_for_z(z, beta=DEFAULT_BETA):
    z = np.asarray(z, np.float32)
    B = np.float32(F.f32(120.0 + beta))
    return expcast_bytes(z.astype(np.float64), 8.0, np.full(z.shape, B, np.float64), 120.0)


def test_shifted_bytes_are_exact_powers_down_to_z_minus_14():
    # byte 8z + 120 has exponent field z + 15 and mantissa 0: the E4M3 value
    # 2^(z+8), normal for z >= -14 (torch's float8 cast gives the same code)
    z = np.arange(-14, 1)
    for beta in (DEFAULT_BETA, 0.0, -0.49, 0.3):
        got = shifted_bytes_for_z(z.astype(np.float32), beta).astype(np.int64)
        assert list(got) == list(8 * z + 120)
    assert list(exact_e4m3_of_exp2(z + 8)) == list(8 * z + 120)
    assert np.array_equal(F.e4m3_decode(8 * z + 120), np.exp2(z + 8.0))
    # the literal mode loses these below z = -6
    assert list(bytes_for_z(np.float32([-7, -10, -14]))) == [0, 0, 0]


def test_shifted_is_literal_plus_64_codes_in_the_normal_range():
    # on z in [-6, 0] the two FMAs differ by 64 before rounding, so the bytes
    # differ by 64 except where x lies within an fp32 ulp (2^-17 above 64) of
    # a rounding midpoint; no point of this grid (step 2^-12) does
    z = -np.arange(0, 6 * 4096 + 1, dtype=np.float64) / 4096.0
    lit = bytes_for_z(z).astype(np.int64)
    sh = shifted_bytes_for_z(z).astype(np.int64)
    ok = lit > 0
    assert np.array_equal(sh[ok], lit[ok] + 64)


def test_shifted_dense_grid_against_exact_exp2_cast():
    # against the exact E4M3 byte of 2^(z+8): within one code for z >= -14
    z = -np.arange(0, 14 * 4096 + 1, dtype=np.float64) / 4096.0
    got = shifted_bytes_for_z(z).astype(np.int64)
    ref = exact_e4m3_of_exp2(z + 8.0)
    assert np.abs(got - ref).max() == 1
    assert got.max() <= 120 and got.min() >= 8


def test_shifted_clamps_at_120():
    S = np.array([10.0, -np.inf, np.nan, -1e30, 0.0], np.float64)
    out = expcast_bytes(S, 8.0, np.full(5, 120.0), 120.0)
    assert list(out) == [120, 0, 0, 0, 120]
