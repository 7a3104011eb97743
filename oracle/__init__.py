"""CPU oracle for the VC-Attention forward pass.

TEST INFRASTRUCTURE ONLY: a plain, slow restatement of the method from the
pages (see the module docstrings for the sources and every reading taken
where the pages are silent).  Only tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path never does.

Entry points:
  prepare_head(K, V, init_idx, ...)   V-Smooth + K smoothing for one head
  attend_rows(Q, prep, tiles, ...)    ExpCast online-softmax attention for
                                      selected 128-row query tiles
  exact_attention, psnr               fp64 reference and fidelity metric
"""
from __future__ import annotations

import numpy as np

from . import formats, kmeans, vsmooth, attention
from .attention import DEFAULT_BETA, exact_attention, psnr, softmax_scale

Q_TILE = 128


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def prepare_head(K: np.ndarray, V: np.ndarray, init_idx: np.ndarray | None, k: int, iters: int,
                 kv_block: int, fmt: str = "e4m3", vsmooth_on: bool = True,
                 quantize: bool = True, init_centroids: np.ndarray | None = None,
                 perm: np.ndarray | None = None, cluster_order: bool = False, balanced: bool = False) -> dict:
    """K, V: [N, d] fp64 bf16 values of one head.  With V-Smooth on, the
    clustering starts from V[init_idx] or, warm-started, from init_centroids
    (fp32 [k, d]); a given perm is reused as is (no clustering, no sort).
    cluster_order renumbers the clusters along their principal axis before
    the final pass (kmeans.order_clusters), so the blocks follow that order.
    balanced: k = ceil(N / kv_block) clusters with capacities kv_block (the
    last the tail), so every block is one cluster (kmeans.capped_assign).
    "final_centroids" are the member means of the final clusters."""
    N = V.shape[0]
    final = None
    if perm is not None:
        labels, cents = None, []
        perm = np.asarray(perm, np.int32)
    elif vsmooth_on:
        cap = kmeans.block_capacities(N, kv_block) if balanced else None
        if balanced:
            assert k == cap.size, "balanced clusters: k must be ceil(N / kv_block)"
        labels, cents, final = kmeans.kmeans(V, init_idx, iters, init_centroids, cluster_order, cap)
        perm = vsmooth.stable_sort_perm(labels, k)
    else:
        labels, cents = None, []
        perm = np.arange(N, dtype=np.int32)
    vs = vsmooth.vsmooth_values(V, perm, kv_block, fmt, vsmooth_on, quantize)
    ks = vsmooth.ksmooth(K, perm, kv_block, vsmooth_on, quantize)
    return {"labels": labels, "centroids": cents, "final_centroids": final, "perm": perm, "v": vs, "k": ks,
            "N": N, "kv_block": kv_block, "fmt": fmt, "quantize": quantize}


def attend_rows(Q: np.ndarray, prep: dict, tiles, scale: float = 0.0, beta: float = DEFAULT_BETA,
                trace: dict | None = None, mode: str = "expcast") -> dict:
    """Returns {tile index: O rows (fp64)} for the requested 128-row tiles.
    mode: "expcast" or "exp2" (ExpCast off), see attention.attend_tile."""
    N, d = Q.shape
    sc = softmax_scale(d, scale)
    out = {}
    for t in tiles:
        lo, hi = t * Q_TILE, min((t + 1) * Q_TILE, N)
        out[t] = attention.attend_tile(
            Q[lo:hi], prep["k"]["kdec"], prep["k"]["k_scale"], prep["v"]["vres"],
            prep["v"]["col_scale"], prep["v"]["means"], prep["N"], prep["kv_block"], sc,
            beta, prep["quantize"], trace, mode)
    return out


def n_q_tiles(N: int) -> int:
    return (N + Q_TILE - 1) // Q_TILE
