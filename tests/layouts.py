"""Test helpers: undo the library's blocked storage layouts (as documented in
include/vcattn.h) so GPU results can be compared with the oracle's
natural-order arrays, and move seeded inputs to the device."""
from __future__ import annotations

import numpy as np


def kstep_rows() -> np.ndarray:
    """row[kappa] = stored row of sorted position kappa inside a 64-key group:
    kappa = 32t + 16g + 4i + j is stored at 32t + 8i + 4g + j."""
    row = np.empty(64, np.int64)
    for t in range(2):
        for g in range(2):
            for i in range(4):
                for j in range(4):
                    row[32 * t + 16 * g + 4 * i + j] = 32 * t + 8 * i + 4 * g + j
    return row


def kq_natural(Kq: np.ndarray) -> np.ndarray:
    """[..., Np, d] stored rows -> sorted-position order."""
    Np = Kq.shape[-2]
    pos = np.arange(Np)
    src = (pos & ~63) | kstep_rows()[pos & 63]
    return Kq[..., src, :]


def vres_natural(Vres: np.ndarray, fmt: str) -> np.ndarray:
    """E4M3 [..., Np/64, d, 64] or MXFP4 [..., Np/64, d, 32] -> codes [..., Np, d]."""
    if fmt == "mxfp4":
        lo = Vres & 0x0F
        hi = Vres >> 4
        Vres = np.stack([lo, hi], axis=-1).reshape(*Vres.shape[:-1], 64)
    x = np.swapaxes(Vres, -1, -2)                     # [..., Np/64, 64, d]
    return x.reshape(*x.shape[:-3], x.shape[-3] * 64, x.shape[-1])


def to_device_bf16(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def mx_scales_natural(vs: np.ndarray) -> np.ndarray:
    """E8M0 scales [..., groups, d] stored in lane order (channel c = 32T + col
    at col * (d/32) + T) -> natural channel order."""
    d = vs.shape[-1]
    c = np.arange(d)
    return vs[..., (c & 31) * (d // 32) + (c >> 5)]


def nv_pair_natural(Vres: np.ndarray):
    """NVFP4-style residuals [..., nblk, 2, kv_block/64, d, 64] -> (high, low)
    E4M3 codes, each [..., Np, d] in sorted-position order."""
    def nat(x):
        x = x.reshape(*x.shape[:-4], x.shape[-4] * x.shape[-3], x.shape[-2], x.shape[-1])
        return vres_natural(x, "e4m3")
    return nat(Vres[..., 0, :, :, :]), nat(Vres[..., 1, :, :, :])


def nv_pair_expected(codes: np.ndarray, s16c: np.ndarray, t: int):
    """The library's documented storage of an NVFP4-style residual, computed
    from the oracle's E2M1 codes [Np, d], E4M3 block scales [Np/16, d] and
    second-level exponent t: v = e2m1 * s16; per 32 positions x channel e is
    the smallest integer with max|v| <= 448 * 2^e (0 for an all-zero group);
    high = E4M3(v / 2^e), low = E4M3(v / 2^e - high); E8M0 byte e + t + 127."""
    from oracle import formats as F
    Np, d = codes.shape
    v = F.e2m1_decode(codes) * np.repeat(F.e4m3_decode(s16c), 16, axis=0)
    e = F.e4m3_group_exponent(np.max(np.abs(v.reshape(Np // 32, 32, d)), axis=1))
    y = v / np.repeat(np.ldexp(1.0, e), 32, axis=0)
    hi = F.e4m3_encode(y)
    lo = F.e4m3_encode(y - F.e4m3_decode(hi))
    return hi, lo, np.clip(e + t + 127, 0, 254).astype(np.uint8)
