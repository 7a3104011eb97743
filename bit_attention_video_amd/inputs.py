"""Seeded synthetic inputs for the VC-Attention forward pass.

This module only draws random numbers; it holds none of the method's
arithmetic.  Both the HIP path (through the binding) and the CPU oracle are
fed from it, so the two always see the same bf16 tensors and the same
k-means initial token indices.

Workload recipe (stand-in for the four video DiTs x MovieGen prompts the
pages measure on, which are not available here):

* Q ~ N(0, 1).
* K ~ N(0, 1) + bias[h, c] with bias ~ N(0, 2^2): a per-channel offset that
  adds a per-query constant to every score (it exercises K mean-smoothing).
* V, per head: M centroids ~ N(0, 3^2 I); every token picks one uniformly and
  adds N(0, 0.5^2) noise.  A fraction f of tokens (chosen uniformly without
  replacement) gets 4 distinct random channels multiplied by 20: value
  outliers with no fixed channel and no spatio-temporal structure, as the
  chooseai.io brief describes them (section on V-Smooth).
* The k-means initial centroids are k distinct token indices drawn uniformly
  per head.  The method draws them at random; here they are an input.

Every head is drawn from its own generator, ``default_rng([seed, b, h])``, so
a single head can be regenerated on its own (the oracle samples heads).
Values are drawn in fp32 and rounded to bf16 (round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
from typing import Iterator

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    n_centroids_gen: int      # M: mixture components of the V generator
    outlier_frac: float       # f: fraction of outlier tokens
    k: int                    # k-means clusters
    iters: int                # k-means assignment passes
    kv_block: int
    q_tile: int = 128
    v_format: str = "e4m3"    # "e4m3" or "mxfp4"
    seed: int = 1000

    @property
    def flops(self) -> float:
        """Effective attention FLOPs 4*N^2*d*H*B (QK^T and PV, 2 flops per MAC)."""
        return 4.0 * self.N * self.N * self.d * self.H * self.B


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 1024, 64, 8, 0.01, 16, 3, 64, seed=1000),
    "mid": Workload("mid", 1, 24, 16384, 128, 32, 0.01, 256, 3, 64, seed=1001),
    "video": Workload("video", 1, 40, 75600, 128, 64, 0.005, 1024, 3, 128, seed=1002),
    "long": Workload("long", 1, 48, 245952, 128, 64, 0.005, 2048, 2, 128, seed=1003),
    "mxfp4": Workload("mxfp4", 1, 40, 75600, 128, 64, 0.005, 1024, 3, 128,
                      v_format="mxfp4", seed=1004),
}


def _bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u                      # no wrap: only NaN patterns exceed 0xFFFF7FFF
    r >>= 16
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def gen_head(w: Workload, b: int, h: int, N: int | None = None, d: int | None = None):
    """Draw one head.  Returns bf16 bit arrays q, k, v of shape [N, d] (uint16)
    and the k-means initial indices (int32 [k])."""
    N = w.N if N is None else N
    d = w.d if d is None else d
    rng = np.random.default_rng([w.seed, b, h])
    q = rng.standard_normal((N, d), dtype=np.float32)
    bias = (rng.standard_normal(d, dtype=np.float32) * 2.0).astype(np.float32)
    k = rng.standard_normal((N, d), dtype=np.float32) + bias[None, :]
    M = w.n_centroids_gen
    cent = (rng.standard_normal((M, d), dtype=np.float32) * 3.0).astype(np.float32)
    comp = rng.integers(0, M, size=N)
    v = cent[comp] + (rng.standard_normal((N, d), dtype=np.float32) * 0.5)
    n_out = int(round(w.outlier_frac * N))
    if n_out > 0:
        toks = rng.choice(N, size=n_out, replace=False)
        for t in toks:
            ch = rng.choice(d, size=min(4, d), replace=False)
            v[t, ch] *= 20.0
    kk = min(w.k, N)
    init = rng.choice(N, size=kk, replace=False).astype(np.int32)
    return _bf16_round(q), _bf16_round(k), _bf16_round(v.astype(np.float32)), init


def iter_heads(w: Workload, N: int | None = None, d: int | None = None) -> Iterator:
    for b in range(w.B):
        for h in range(w.H):
            yield b, h, gen_head(w, b, h, N, d)


def gen_all(w: Workload, N: int | None = None, d: int | None = None, H: int | None = None):
    """All heads as numpy arrays: q, k, v uint16 bf16 bits [B,H,N,d]; init int32 [B,H,k].
    Heads are drawn in parallel threads; each has its own generator, so the
    result does not depend on the thread count."""
    import concurrent.futures
    import os
    N = w.N if N is None else N
    d = w.d if d is None else d
    H = w.H if H is None else H
    kk = min(w.k, N)
    q = np.empty((w.B, H, N, d), np.uint16)
    k = np.empty_like(q)
    v = np.empty_like(q)
    init = np.empty((w.B, H, kk), np.int32)

    def one(bh):
        b, h = divmod(bh, H)
        q[b, h], k[b, h], v[b, h], init[b, h] = gen_head(w, b, h, N, d)

    workers = max(1, min(16, os.cpu_count() or 1, w.B * H))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, range(w.B * H)))
    return q, k, v, init


def small(w: Workload, N: int, H: int = 1, k: int | None = None, d: int | None = None,
          kv_block: int | None = None, seed: int | None = None, iters: int | None = None,
          v_format: str | None = None) -> Workload:
    """A reduced copy of a workload (same generator parameters)."""
    return dataclasses.replace(
        w, N=N, H=H, k=min(k if k is not None else w.k, N),
        d=d if d is not None else w.d,
        kv_block=kv_block if kv_block is not None else w.kv_block,
        seed=seed if seed is not None else w.seed,
        iters=iters if iters is not None else w.iters,
        v_format=v_format if v_format is not None else w.v_format)


def next_step(w: Workload, bits: np.ndarray, step: int, sigma: float, tag: int) -> np.ndarray:
    """A following denoising step's tensor: bf16 values plus N(0, sigma^2)
    noise, drawn per head from default_rng([seed, 7919, step, tag, b, h]) and
    rounded back to bf16.  bits: uint16 [B,H,N,d] (Q, K or V; tag tells them
    apart).  Stands in for the slowly changing activations of consecutive
    diffusion steps."""
    out = np.empty_like(bits)
    for b in range(bits.shape[0]):
        for h in range(bits.shape[1]):
            rng = np.random.default_rng([w.seed, 7919, step, tag, b, h])
            x = bf16_bits_to_f32(bits[b, h]) + rng.standard_normal(bits.shape[2:], dtype=np.float32) * np.float32(sigma)
            out[b, h] = _bf16_round(x.astype(np.float32))
    return out
