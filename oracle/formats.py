"""Number formats and IEEE fp32 rounding helpers for the CPU oracle.

TEST INFRASTRUCTURE ONLY.  The oracle is a plain, slow restatement of the
VC-Attention forward pass used to check the HIP library; nothing in the
product path may import it.

Sources (web pages on VC-Attention; cited by title and section):
  [brief]   chooseai.io news brief on VC-Attention (Chinese), sections
            "V-Smooth" and "ExpCast-FP8".
  [clarity] "Quantizing value residuals and casting softmax to FP8 speeds
            Nunchux's attention kernel 1.46x on an H200" (theclarity.today).
  [zh]      "Nunchux AI Introduces VC-Attention: A Training-Free Low-Bit
            Attention Kernel ..." (zerohour.day summary), key-facts list.
  [rw]      "Nunchux speeds video diffusion with value smoothing and FP8
            softmax casting" (runtimewire via wpnews).

E4M3 is the 8-bit float of the pages: [brief, ExpCast-FP8] relates one E4M3
byte to 8*log2(p)+56, which only holds for the OCP E4M3 encoding (exponent
bias 7, so 1.0 is byte 56 = 0x38; max finite 448; no infinities; S.1111.111
is NaN).  E2M1 (OCP FP4) with E8M0 block scales is the 4-bit residual format
([zh] names NVFP4 residuals; OCP MXFP4 is this implementation's 4-bit format).

All encoders take exact real values (fp64 arrays holding fp32 or bf16 numbers)
and round to nearest, ties to even, saturating at the largest finite value;
the sign bit is always copied from the input (so -0 encodes with sign set).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def f32(x) -> np.ndarray:
    """Round to IEEE binary32 (nearest-even) and return as float64 values."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ---------------------------------------------------------------- E4M3 (OCP)
def e4m3_decode(codes) -> np.ndarray:
    """Byte -> value (float64).  Codes 0x01..0x07 are subnormal c*2^-9;
    exponent field e>0 gives 2^(e-7)*(1+m/8); 0x7F/0xFF are NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    out = s * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(x) -> np.ndarray:
    """Value -> byte, round-to-nearest-even, saturating to +-448 (never NaN
    for finite input; NaN input gives 0x7F)."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.abs(x)
    out = np.zeros(x.shape, dtype=np.int64)
    # subnormal range (below the smallest normal 2^-6): multiples of 2^-9;
    # rounding up to 8 lands exactly on code 0x08 = 2^-6.
    sub = a < 2.0 ** -6
    out[sub] = np.rint(a[sub] * 512.0).astype(np.int64)
    nrm = ~sub & np.isfinite(a)
    if nrm.any():
        an = a[nrm]
        _, ex = np.frexp(an)          # an = f * 2^ex, f in [0.5, 1)
        e = ex - 1                    # an in [2^e, 2^(e+1))
        m = np.rint((np.ldexp(an, -e) - 1.0) * 8.0).astype(np.int64)
        carry = m == 8
        e = e + carry
        m = np.where(carry, 0, m)
        code = ((e + 7) << 3) | m
        code = np.where((e + 7) > 15, 0x7E, code)
        code = np.where(code > 0x7E, 0x7E, code)   # 464 and above -> 448
        out[nrm] = code
    out[np.isinf(a)] = 0x7E
    # the sign bit is copied for every input, so -0 and negative values that
    # round to zero encode as 0x80
    out = np.where(sign, out | 0x80, out)
    out[np.isnan(x)] = 0x7F
    return out.astype(np.uint8)


# ---------------------------------------------------------------- E2M1 (OCP)
_E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    """4-bit code S.EE.M -> value: e=0 gives m*0.5, else 2^(e-1)*(1+m/2)."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    mag = _E2M1_VALUES[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode(x) -> np.ndarray:
    """Value -> 4-bit code, nearest-even on the E2M1 grid, saturating at 6."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    # representable magnitudes are k*0.5 (k<=4 -> steps 0.5 up to 2),
    # then 2,3,4,6.  Scale each binade so the step is 1, round-to-even there.
    mag = np.where(a < 2.0, np.rint(a * 2.0) / 2.0,
                   np.where(a < 4.0, np.rint(a), np.rint(a / 2.0) * 2.0))
    mag = np.minimum(mag, E2M1_MAX)
    idx = np.searchsorted(_E2M1_VALUES, mag)
    code = idx.astype(np.int64)
    code = np.where(np.signbit(x), code | 8, code)   # sign copied, also for zero
    return code.astype(np.uint8)


# ---------------------------------------------------------------- E8M0 scale
def e8m0_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, (c - 127).astype(np.int64)))


def mx_shared_exponent(amax, emax: int = 2) -> np.ndarray:
    """OCP MX v1.0 scale rule: X = 2^(floor(log2 amax) - emax), emax being the
    element format's largest exponent (E2M1: 2, E4M3: 8).  The exponent is
    clamped to E8M0's range; an all-zero block uses X = 1."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.where(a > 0, (ex - 1) - emax, 0)
    return np.clip(e, -127, 127).astype(np.int64)


def e4m3_group_exponent(amax) -> np.ndarray:
    """Power-of-two scale for a group of E4M3 elements: the smallest e with
    amax <= 448 * 2^e, so no element saturates (OCP MX's floor(log2 amax) - 8
    lets the group maximum clamp by up to 12.5%).  Clamped to E8M0's range; an
    all-zero group uses 2^0."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e0 = (ex - 1) - 8                                # floor(log2 amax) - 8
    e = np.where(a > 448.0 * np.ldexp(1.0, e0), e0 + 1, e0)
    e = np.where(a > 0, e, 0)
    return np.clip(e, -127, 127).astype(np.int64)


NV_TENSOR_MAX = E2M1_MAX * E4M3_MAX     # 2688: largest element times block scale


def nv_tensor_exponent(amax) -> np.ndarray:
    """Second-level (per tensor) scale of the NVFP4-style residual, taken as a
    power of two: the smallest t with amax <= 6 * 448 * 2^t, so that every
    16-element block scale amax16 / (6 * 2^t) fits E4M3 without saturating;
    t >= -126, so 2^t is a normal fp32.  An all-zero tensor uses 2^0."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))         # a = f * 2^ex, f in [0.5, 1)
    t0 = (ex - 1) - 11                                # 2688 * 2^t0 = 1.3125 * 2^(ex-1)
    t = np.where(a > NV_TENSOR_MAX * np.ldexp(1.0, t0), t0 + 1, t0)
    t = np.maximum(t, -126)                           # 2^t stays a normal fp32
    return np.where(a > 0, t, 0).astype(np.int64)


# ------------------------------------------------------- fp32 fused multiply-add
def fma_f32(a, b, c) -> np.ndarray:
    """Correctly rounded binary32 fma(a, b, c) for binary32 inputs.

    a*b is exact in binary64 (two 24-bit significands).  The sum with c is
    formed in binary64 together with its exact rounding error (TwoSum), and a
    tie at a binary32 midpoint is broken by the sign of that error, so the
    result is the single rounding of the exact a*b+c."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    c = np.asarray(c, np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        p = a * b
        s = p + c
        bp = s - p
        err = (p - (s - bp)) + (c - bp)
        r32 = s.astype(np.float32)
        r = r32.astype(np.float64)
        up = np.nextafter(r32, np.float32(np.inf)).astype(np.float64)
        dn = np.nextafter(r32, np.float32(-np.inf)).astype(np.float64)
        # s lies on a binary32 midpoint: between r and the neighbour on s's side
        other = np.where(s > r, up, dn)
        mid = (s != r) & (2.0 * s == r + other)
        fix_up = mid & (err > 0) & (other > r)
        fix_dn = mid & (err < 0) & (other < r)
        # s rounded to even onto r, but the exact value lies beyond s, away from r
        out = np.where(fix_up | fix_dn, other, r)
        finite = np.isfinite(p) & np.isfinite(s) & np.isfinite(err)
        out = np.where(finite, out, r)
    return out


def exp2_f64(x) -> np.ndarray:
    return np.exp2(np.asarray(x, np.float64))
