"""Per-head k-means over value tokens (CPU oracle; TEST INFRASTRUCTURE ONLY).

What the pages give: V-Smooth first runs one lightweight k-means that puts
similar value tokens together ([brief] section "V-Smooth", first of its three
steps; [rw] "lightweight online clustering"; [clarity] "clusters similar
value tokens online").  They give no distance arithmetic, initialisation or
iteration count.  The readings used here (all stated as readings):

* Distances are computed on int8 codes with one scale per head,
  sV = fp32(max|V| / 127), code = clamp(rne(fp32(x / sV)), -127, 127), for both
  tokens and centroids, as D = |c|^2 - 2 v.c in exact integers.  "Lightweight"
  is read as: cheap enough to run inside the attention call.
* Initial centroids are the value rows at k distinct token indices, either
  supplied by the caller or drawn from a seed (``seeded_init``: a partial
  Fisher-Yates shuffle of the token indices driven by splitmix64, one stream
  per head), or, warm-started
  across denoising steps (the pages run the clustering step by step and call
  its cost a scheduling trade), the centroids the previous call ended with.
* The centroids a call ends with are the member means of its final clusters
  (one more update after the last assignment pass).
* ``iters`` assignment passes, with a centroid update between consecutive
  passes; the final labels are those of the last pass.
* Ties go to the lowest cluster index.
* Update: the fp32 rounding of the fp64 mean of the members' original values;
  a cluster with no members keeps its centroid.

Optional balanced clusters (a blocking variant; [brief] "V-Smooth" asks that
similar tokens share one hardware block): k = ceil(N / kv_block) clusters
with capacities kv_block (the last one the tail, N - (k-1) * kv_block), so
that after the stable sort every block holds exactly one cluster.  Each
assignment pass is capped (``capped_assign``): in rounds, every unassigned
token proposes to its nearest cluster that still has room (ties to the
lowest cluster index), and a cluster with r places left takes the r nearest
of its proposers (ties to the lowest token index); tokens still unassigned
after BALANCED_ROUNDS rounds fill the remaining places in token order,
clusters in index order.  Distances are the same exact int8 scores.

Optional cluster ordering (a blocking variant; [brief] "V-Smooth" asks that
similar tokens share a hardware block but says nothing of the order of the
clusters): before the final assignment pass the centroids are renumbered by
their position along the principal axis of their int8 codes, so that blocks
which straddle two clusters join similar ones.  Everything is exact integer
arithmetic, so the order is reproducible bit for bit:

* s = column sums of the codes q [k, d]; S = k * q^T q - s s^T (k^2 times the
  covariance of the codes);
* A = S shifted right (floor) by max(0, bitlen(max|S|) - 24);
* start vector: the column of A with the largest diagonal entry (lowest
  index on ties); 16 power steps u = A v, each followed by v = u shifted right
  by max(0, bitlen(max|u|) - 24);
* projection p_c = q_c . v; rank = position in ascending (p_c, c) order.
"""
from __future__ import annotations

import numpy as np

from .formats import f32


GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_MASK64 = (1 << 64) - 1


def splitmix64(state: int):
    """The splitmix64 generator (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014): the state advances by the
    golden-ratio gamma, and each output is the state passed through the
    variant-13 finaliser.  Yields 64-bit integers."""
    state &= _MASK64
    while True:
        state = (state + GOLDEN_GAMMA) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        yield z ^ (z >> 31)


def partial_fisher_yates(N: int, k: int, draws) -> np.ndarray:
    """The first k entries of a Fisher-Yates shuffle of 0..N-1: for
    i = 0..k-1, j = i + (next draw mod (N - i)), swap entries i and j."""
    a = list(range(N))
    for i in range(k):
        j = i + next(draws) % (N - i)
        a[i], a[j] = a[j], a[i]
    return np.array(a[:k], dtype=np.int32)


def seeded_init(seed: int, bh: int, N: int, k: int) -> np.ndarray:
    """k distinct initial token indices of head bh = b*H + h: a partial
    Fisher-Yates shuffle driven by splitmix64 seeded with
    seed + 0x9E3779B97F4A7C15 * bh (mod 2^64)."""
    return partial_fisher_yates(N, k, splitmix64(seed + GOLDEN_GAMMA * bh))


def int8_scale(V: np.ndarray) -> float:
    """sV = fp32(max|V| / 127), floored at 2^-126 (1 if V == 0)."""
    amax = float(np.max(np.abs(V))) if V.size else 0.0
    return max(float(f32(amax / 127.0)), 2.0 ** -126) if amax > 0 else 1.0


def quant_i8(X: np.ndarray, sV: float) -> np.ndarray:
    return np.clip(np.rint(f32(X / sV)), -127, 127)


def assign(Vq: np.ndarray, Cq: np.ndarray) -> np.ndarray:
    """argmin_c (|c|^2 - 2 v.c); np.argmin returns the first (lowest) index on
    ties.  Integer products and sums stay below 2^53, so fp64 BLAS is exact."""
    cn = np.sum(Cq * Cq, axis=1)
    D = cn[None, :] - 2.0 * (Vq @ Cq.T)
    return np.argmin(D, axis=1).astype(np.int32)


BALANCED_ROUNDS = 12


def block_capacities(N: int, kv_block: int) -> np.ndarray:
    """Capacities of the balanced clusters: kv_block each, the last one the
    tail of the sequence."""
    k = (N + kv_block - 1) // kv_block
    cap = np.full(k, kv_block, dtype=np.int64)
    cap[-1] = N - (k - 1) * kv_block
    return cap


def capped_assign(Vq: np.ndarray, Cq: np.ndarray, cap: np.ndarray, rounds: int = BALANCED_ROUNDS) -> np.ndarray:
    """Assignment with cluster capacities cap (sum(cap) == N), see the module
    notes.  Squared distances |v|^2 + |c|^2 - 2 v.c of the int8 codes are
    exact integers."""
    N, k = Vq.shape[0], Cq.shape[0]
    assert int(np.sum(cap)) == N
    dist = np.sum(Vq * Vq, axis=1)[:, None] + np.sum(Cq * Cq, axis=1)[None, :] - 2.0 * (Vq @ Cq.T)
    labels = np.full(N, -1, dtype=np.int64)
    rem = np.asarray(cap, dtype=np.int64).copy()
    for _ in range(rounds):
        un = np.nonzero(labels < 0)[0]
        if un.size == 0:
            break
        dc = np.where(rem[None, :] > 0, dist[un], np.inf)
        prop = np.argmin(dc, axis=1)                 # first minimum: lowest cluster index
        for c in np.unique(prop):
            ts = un[prop == c]                       # proposers in token order
            order = np.lexsort((ts, dist[ts, c]))    # nearest first, then lowest token index
            take = ts[order][:rem[c]]
            labels[take] = c
            rem[c] -= take.size
    un = np.nonzero(labels < 0)[0]
    slots = np.repeat(np.arange(k), rem)             # the places left, clusters in index order
    labels[un] = slots[:un.size]
    return labels.astype(np.int32)


def update(V: np.ndarray, labels: np.ndarray, C_old: np.ndarray) -> np.ndarray:
    k = C_old.shape[0]
    sums = np.zeros_like(C_old, dtype=np.float64)
    np.add.at(sums, labels, V)                       # fp64, token order
    counts = np.bincount(labels, minlength=k).astype(np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        mean = f32(sums / counts[:, None])
    return np.where(counts[:, None] > 0, mean, C_old)


POWER_STEPS = 16
AXIS_BITS = 24


def _bitlen(x: int) -> int:
    return int(x).bit_length()


def principal_axis_int(q: np.ndarray) -> np.ndarray:
    """Integer power iteration on k^2 times the covariance of the codes q
    ([k, d] integers); returns the integer axis v [d] (see the module notes)."""
    q = np.asarray(q, dtype=np.int64)
    k, d = q.shape
    s = q.sum(axis=0)
    S = k * (q.T @ q) - np.outer(s, s)              # exact: |entries| < 2^40
    sh = max(0, _bitlen(int(np.max(np.abs(S)))) - AXIS_BITS)
    A = S >> sh
    v = A[:, int(np.argmax(np.diag(A)))].copy()
    for _ in range(POWER_STEPS):
        u = A @ v                                   # |u| < 2^24 * 2^24 * d
        m = int(np.max(np.abs(u)))
        if m == 0:
            break
        v = u >> max(0, _bitlen(m) - AXIS_BITS)
    return v


def order_clusters(q: np.ndarray) -> np.ndarray:
    """rank [k]: position of cluster c in ascending (q_c . axis, c) order."""
    q = np.asarray(q, dtype=np.int64)
    p = q @ principal_axis_int(q)
    order = np.lexsort((np.arange(q.shape[0]), p))  # by p, then by index
    rank = np.empty(q.shape[0], dtype=np.int32)
    rank[order] = np.arange(q.shape[0], dtype=np.int32)
    return rank


def kmeans(V: np.ndarray, init_idx: np.ndarray | None, iters: int, init_centroids: np.ndarray | None = None,
           order: bool = False, capacities: np.ndarray | None = None):
    """V: [N, d] float64 holding the bf16 values of one head.  Starts from the
    rows V[init_idx], or from init_centroids (fp32 [k, d]) when given.
    order: renumber the centroids along their principal axis before the final
    pass.  capacities: capped assignment passes (balanced clusters).
    Returns (labels int32 [N], centroids_per_pass: the centroids each
    assignment pass used, final: the member means of the final clusters)."""
    sV = int8_scale(V)
    Vq = quant_i8(V, sV)
    if init_centroids is not None:
        C = f32(np.asarray(init_centroids, np.float64)).astype(np.float64)
    else:
        C = V[np.asarray(init_idx, dtype=np.int64)].astype(np.float64)
    used = []
    labels = None
    for it in range(iters):
        if order and it + 1 == iters:
            rank = order_clusters(quant_i8(C, sV))
            Cn = np.empty_like(C)
            Cn[rank] = C
            C = Cn
        used.append(C.copy())
        if capacities is None:
            labels = assign(Vq, quant_i8(C, sV))
        else:
            labels = capped_assign(Vq, quant_i8(C, sV), capacities)
        if it + 1 < iters:
            C = update(V, labels, C)
    return labels, used, update(V, labels, C)
