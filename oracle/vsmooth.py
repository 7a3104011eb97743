"""V-Smooth blocking and residual quantisation, K smoothing (CPU oracle;
TEST INFRASTRUCTURE ONLY).

V-Smooth ([brief] section "V-Smooth"; [clarity]; [zh] key facts; [rw]):
  1. similar value tokens are clustered and grouped into one hardware block;
  2. the block mean is subtracted and kept in high precision;
  3. only the residual goes through the 8-bit quantiser, with per-channel
     scales ([zh]: "per-channel E4M3/NVFP4 residuals after block-mean
     subtraction").
K and V are permuted together, so attention (non-causal) is unchanged.

Readings (the pages leave these open):
  * grouping = stable sort of tokens by cluster label, then fixed blocks of
    ``kv_block`` consecutive sorted tokens; only the last block is partial.
  * mean_b = fp32(fp64 mean over the block's real tokens);
    r = fp32(v - mean_b).
  * E4M3 residual scale: one per (head, channel), s_v = fp32(max|r| / 448)
    over the head's real tokens (1 when the channel's residual is all zero;
    floored at 2^-126, so its reciprocal stays finite);
    code = E4M3(fp32(r / s_v)).  The per-channel scale factors out of P.V.
  * MXFP4 residuals: per 32 consecutive sorted tokens x channel, E8M0 scale
    2^(floor(log2 amax) - 2) and E2M1 elements (OCP MX rule).
  * MXFP8 residuals (a variant with per-(token group, channel) scales in place
    of one scale per channel): per 32 consecutive sorted tokens x channel an
    E8M0 scale 2^e, e the smallest integer with amax <= 448 * 2^e (so no
    element saturates), and E4M3 elements of r / 2^e, round to nearest even.
  * NVFP4-style residuals ([zh] names NVFP4 for the 4-bit residuals): per 16
    consecutive sorted tokens x channel an E4M3 block scale
    s16 = E4M3(fp32(amax16 / (6 * s_t))) and E2M1 elements
    E2M1(fp32(r / (s16 * s_t))) (nearest even, saturating at 6; a block whose
    scale rounds to 0 holds zeros).  The second-level scale s_t, one per head,
    is a power of two here (the smallest 2^t with amax <= 6 * 448 * 2^t), so
    that it folds into the matrix core's power-of-two scales; dequantised
    value = e2m1 * s16 * s_t.
  * K smoothing (prior art the pages contrast V-Smooth with: "earlier
    low-bit methods ... smoothed queries and keys"): mu_K = fp32(fp64 mean over
    all tokens, per channel); K' = fp32(K - mu_K); per block
    s_k = fp32(max|K'_blk| / 448) (floored at 2^-126); Kq = E4M3(fp32(K' / s_k)).
  * padded tail rows hold code 0.

``quantize=False`` keeps every value in fp64 with no rounding (for the
quantisation-disabled self-check).
"""
from __future__ import annotations

import numpy as np

from .attention import scale_of
from .formats import (f32, e4m3_encode, e4m3_decode, e2m1_encode, e2m1_decode, mx_shared_exponent,
                      e4m3_group_exponent, nv_tensor_exponent)


def stable_sort_perm(labels: np.ndarray, k: int) -> np.ndarray:
    """Counting sort: perm[j] = original token index at sorted position j;
    equal labels keep token order."""
    labels = np.asarray(labels, dtype=np.int64)
    counts = np.bincount(labels, minlength=k)
    start = np.concatenate([[0], np.cumsum(counts)[:-1]])
    perm = np.empty(labels.shape[0], dtype=np.int32)
    nxt = start.copy()
    for tok, lab in enumerate(labels):
        perm[nxt[lab]] = tok
        nxt[lab] += 1
    return perm


def n_blocks(N: int, kv_block: int) -> int:
    return (N + kv_block - 1) // kv_block


def block_means(Vp: np.ndarray, N: int, kv_block: int, quantize: bool = True) -> np.ndarray:
    """Vp: [nblk*kv_block, d] permuted values (pad rows ignored)."""
    nblk = n_blocks(N, kv_block)
    d = Vp.shape[1]
    means = np.zeros((nblk, d), np.float64)
    for b in range(nblk):
        lo, hi = b * kv_block, min((b + 1) * kv_block, N)
        m = np.sum(Vp[lo:hi], axis=0, dtype=np.float64) / (hi - lo)
        means[b] = f32(m) if quantize else m
    return means


def vsmooth_values(V: np.ndarray, perm: np.ndarray, kv_block: int, fmt: str = "e4m3",
                   vsmooth: bool = True, quantize: bool = True) -> dict:
    """V: [N, d] fp64 (bf16 values).  Returns natural-layout results:
       codes [nblk*kv_block, d] (E4M3 bytes or E2M1 nibbles, one per element),
       vres  decoded residual values (E4M3: in units of s_v; MX formats: real units),
       col_scale [d] (E4M3: s_v; MX formats: ones), e8m0 [nblk*kv_block/32, d] (MX),
       means [nblk, d]."""
    N, d = V.shape
    nblk = n_blocks(N, kv_block)
    Np = nblk * kv_block
    Vp = np.zeros((Np, d), np.float64)
    Vp[:N] = V[perm] if vsmooth else V
    means = block_means(Vp, N, kv_block, quantize) if vsmooth else np.zeros((nblk, d))
    r = np.zeros((Np, d), np.float64)
    mexp = np.repeat(means, kv_block, axis=0)[:N]
    r[:N] = f32(Vp[:N] - mexp) if quantize else Vp[:N] - mexp
    out = {"means": means}
    if not quantize:
        out.update(codes=None, vres=r, col_scale=np.ones(d), e8m0=None)
        return out
    if fmt == "e4m3":
        amax = np.max(np.abs(r[:N]), axis=0)
        s_v = np.array([scale_of(float(a), 448.0) for a in amax])
        codes = e4m3_encode(f32(r / s_v[None, :]))
        codes[N:] = 0
        out.update(codes=codes, vres=e4m3_decode(codes), col_scale=s_v, e8m0=None)
    elif fmt == "mxfp4":
        g = r.reshape(Np // 32, 32, d)
        amax = np.max(np.abs(g), axis=1)                       # [Np/32, d]
        e = mx_shared_exponent(amax)
        codes = e2m1_encode(g / np.ldexp(1.0, e)[:, None, :]).reshape(Np, d)
        codes[N:] = 0
        vals = (e2m1_decode(codes).reshape(Np // 32, 32, d) * np.ldexp(1.0, e)[:, None, :]).reshape(Np, d)
        out.update(codes=codes, vres=vals, col_scale=np.ones(d), e8m0=(e + 127).astype(np.uint8))
    elif fmt == "mxfp8":
        g = r.reshape(Np // 32, 32, d)
        amax = np.max(np.abs(g), axis=1)
        e = e4m3_group_exponent(amax)
        codes = e4m3_encode(g / np.ldexp(1.0, e)[:, None, :]).reshape(Np, d)
        codes[N:] = 0
        vals = (e4m3_decode(codes).reshape(Np // 32, 32, d) * np.ldexp(1.0, e)[:, None, :]).reshape(Np, d)
        out.update(codes=codes, vres=vals, col_scale=np.ones(d), e8m0=(e + 127).astype(np.uint8))
    elif fmt == "nvfp4":
        amax = float(np.max(np.abs(r[:N]))) if N else 0.0
        t = int(nv_tensor_exponent(amax))
        s_t = np.ldexp(1.0, t)
        g = r.reshape(Np // 16, 16, d)
        a16 = np.max(np.abs(g), axis=1)                          # [Np/16, d]
        s16c = e4m3_encode(f32(a16 / (6.0 * s_t)))
        den = e4m3_decode(s16c) * s_t                            # exact: power-of-two factor
        with np.errstate(divide="ignore", invalid="ignore"):
            x = np.where(den[:, None, :] > 0, f32(g / den[:, None, :]), 0.0)
        codes = e2m1_encode(x).reshape(Np, d)
        codes[N:] = 0
        vals = (e2m1_decode(codes).reshape(Np // 16, 16, d) * den[:, None, :]).reshape(Np, d)
        out.update(codes=codes, vres=vals, col_scale=np.ones(d), e8m0=None, nv_scale=s16c, nv_t=t)
    else:
        raise ValueError(fmt)
    return out


def ksmooth(K: np.ndarray, perm: np.ndarray, kv_block: int, vsmooth: bool = True,
            quantize: bool = True) -> dict:
    N, d = K.shape
    nblk = n_blocks(N, kv_block)
    Np = nblk * kv_block
    mu = np.sum(K, axis=0, dtype=np.float64) / N
    if quantize:
        mu = f32(mu)
    Ks = f32(K - mu[None, :]) if quantize else K - mu[None, :]
    Kp = np.zeros((Np, d), np.float64)
    Kp[:N] = Ks[perm] if vsmooth else Ks
    if not quantize:
        return {"mu": mu, "codes": None, "kdec": Kp, "k_scale": np.ones(nblk)}
    k_scale = np.ones(nblk)
    codes = np.zeros((Np, d), np.uint8)
    for b in range(nblk):
        lo, hi = b * kv_block, min((b + 1) * kv_block, N)
        amax = np.max(np.abs(Kp[lo:hi]))
        s = scale_of(float(amax), 448.0)
        k_scale[b] = s
        codes[lo:hi] = e4m3_encode(f32(Kp[lo:hi] / s))
    return {"mu": mu, "codes": codes, "kdec": e4m3_decode(codes), "k_scale": k_scale}
