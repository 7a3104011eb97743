"""Pins for the oracle's k-means, stable sort / blocking, V-Smooth residual
quantisation and K smoothing: brute force on tiny inputs, exact rational
arithmetic, a library sort, and the quantisers' error bounds."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import kmeans as KM
from oracle import vsmooth as VS
from oracle import formats as F
import oracle
from bit_attention_video_amd import inputs


def brute_assign(Vq, Cq):
    out = []
    for v in Vq.astype(int).tolist():
        best, bi = None, None
        for ci, c in enumerate(Cq.astype(int).tolist()):
            dist = sum(x * x for x in c) - 2 * sum(a * b for a, b in zip(v, c))
            if best is None or dist < best:        # strict: lowest index wins ties
                best, bi = dist, ci
        out.append(bi)
    return np.array(out)


def test_assign_matches_brute_force_with_ties():
    rng = np.random.default_rng(10)
    for trial in range(30):
        N, k, d = rng.integers(1, 12), rng.integers(1, 6), rng.integers(1, 5)
        Vq = rng.integers(-127, 128, size=(N, d)).astype(np.float64)
        Cq = rng.integers(-127, 128, size=(k, d)).astype(np.float64)
        if k > 1 and trial % 3 == 0:
            Cq[k - 1] = Cq[0]                      # exact duplicate: index 0 must win
        assert np.array_equal(KM.assign(Vq, Cq), brute_assign(Vq, Cq))
    # equidistant centroids: v=0, c=+-1 have the same distance; lower index wins
    assert list(KM.assign(np.zeros((1, 1)), np.array([[1.0], [-1.0]]))) == [0]
    assert list(KM.assign(np.zeros((1, 1)), np.array([[-1.0], [1.0]]))) == [0]


def test_int8_quantiser():
    V = np.array([[1.0, -2.0], [127.0, -127.5]])
    s = KM.int8_scale(V)
    assert s == float(F.f32(127.5 / 127.0))
    q = KM.quant_i8(V, s)
    assert q.min() >= -127 and q.max() <= 127
    assert np.array_equal(q, np.clip(np.rint(F.f32(V / s)), -127, 127))


def test_update_exact_mean_and_empty_cluster():
    rng = np.random.default_rng(11)
    V = F.f32(rng.standard_normal((20, 3)) * 3)
    labels = rng.integers(0, 3, 20)
    labels[labels == 2] = 1                       # cluster 2 empty
    C_old = np.arange(9.0).reshape(3, 3)
    C = KM.update(V, labels, C_old)
    assert np.array_equal(C[2], C_old[2])
    for c in (0, 1):
        mem = V[labels == c]
        for j in range(3):
            exact = sum(Fraction(float(x)) for x in mem[:, j]) / len(mem)
            assert C[c, j] == float(np.float32(float(exact)))


def sse(V, labels, k):
    tot = 0.0
    for c in range(k):
        m = V[labels == c]
        if len(m):
            tot += float(np.sum((m - m.mean(0)) ** 2))
    return tot


def test_kmeans_recovers_sse_optimum_on_separated_tiny_instances():
    rng = np.random.default_rng(12)
    for trial in range(10):
        k = int(rng.integers(2, 4))
        d = int(rng.integers(1, 4))
        N = int(rng.integers(k + 1, 9))
        while True:                                # well separated: centres >= 40 apart
            centers = rng.standard_normal((k, d)) * 100
            gaps = [np.linalg.norm(centers[i] - centers[j]) for i in range(k) for j in range(i)]
            if min(gaps) >= 40:
                break
        own = np.concatenate([np.arange(k), rng.integers(0, k, N - k)])
        V = F.f32(centers[own] + rng.standard_normal((N, d)) * 0.5)
        init = np.array([np.flatnonzero(own == c)[0] for c in range(k)], np.int32)
        labels, _, _ = KM.kmeans(V, init, iters=4)
        best = min(sse(V, np.array(lab), k) for lab in itertools.product(range(k), repeat=N))
        assert abs(sse(V, labels, k) - best) <= 1e-9 * max(1.0, best)


def test_kmeans_pass_count_and_used_centroids():
    rng = np.random.default_rng(13)
    V = F.f32(rng.standard_normal((50, 4)))
    init = rng.choice(50, 5, replace=False).astype(np.int32)
    labels, used, _ = KM.kmeans(V, init, iters=3)
    assert len(used) == 3
    assert np.array_equal(used[0], V[init])
    # the labels are the assignment made with the last centroids
    sV = KM.int8_scale(V)
    assert np.array_equal(labels, KM.assign(KM.quant_i8(V, sV), KM.quant_i8(used[2], sV)))
    assert np.array_equal(used[1], KM.update(V, KM.assign(KM.quant_i8(V, sV), KM.quant_i8(used[0], sV)), used[0]))


def test_stable_sort_matches_library_and_is_bijection():
    rng = np.random.default_rng(14)
    for N, k in [(1, 1), (100, 7), (5000, 300)]:
        lab = rng.integers(0, k, N)
        perm = VS.stable_sort_perm(lab, k)
        assert np.array_equal(perm, np.argsort(lab, kind="stable"))
        assert np.array_equal(np.sort(perm), np.arange(N))
        assert np.all(np.diff(lab[perm]) >= 0)


def test_block_means_exact():
    rng = np.random.default_rng(15)
    N, kvb, d = 150, 64, 3
    Vp = np.zeros((3 * kvb, d))
    Vp[:N] = F.f32(rng.standard_normal((N, d)))
    means = VS.block_means(Vp, N, kvb)
    for b in range(3):
        lo, hi = b * kvb, min((b + 1) * kvb, N)
        for j in range(d):
            exact = sum(Fraction(float(x)) for x in Vp[lo:hi, j]) / (hi - lo)
            assert means[b, j] == float(np.float32(float(exact)))


def test_e4m3_residuals_within_quantiser_bound():
    rng = np.random.default_rng(16)
    N, d, kvb = 300, 8, 64
    V = F.f32(rng.standard_normal((N, d)) * 3)
    V[5, 2] *= 20
    perm = rng.permutation(N).astype(np.int32)
    out = VS.vsmooth_values(V, perm, kvb, "e4m3")
    means, s_v = out["means"], out["col_scale"]
    r = np.zeros((5 * kvb, d))
    r[:N] = F.f32(V[perm] - np.repeat(means, kvb, 0)[:N])
    deq = out["vres"] * s_v[None, :]
    # E4M3 RNE: relative error <= 2^-4 in the normal range, absolute <= 2^-10*s below it
    assert np.all(np.abs(deq - r) <= np.maximum(np.abs(r) * 2 ** -4, s_v[None, :] * 2 ** -10) * (1 + 1e-12))
    assert np.all(out["codes"][N:] == 0)
    # per-channel scale is the residual's max magnitude over 448: that element maps to 448
    amax = np.max(np.abs(r[:N]), axis=0)
    assert np.array_equal(s_v, F.f32(amax / 448.0))


def test_mxfp4_residuals_within_block_bound():
    rng = np.random.default_rng(17)
    N, d, kvb = 200, 4, 64
    V = F.f32(rng.standard_normal((N, d)) * 3)
    perm = np.arange(N, dtype=np.int32)
    out = VS.vsmooth_values(V, perm, kvb, "mxfp4")
    r = np.zeros((256, d))
    r[:N] = F.f32(V - np.repeat(out["means"], kvb, 0)[:N])
    X = F.e8m0_decode(out["e8m0"].astype(np.int64))            # [8, d]
    Xe = np.repeat(X, 32, axis=0)
    # the block maximum sits in [4X, 8X); E2M1 error <= half a grid step (0.25X .. 1X),
    # plus clipping of values above 6X
    err = np.abs(out["vres"] - r)
    step = np.where(np.abs(r) < 2 * Xe, 0.5, np.where(np.abs(r) < 4 * Xe, 1.0, 2.0)) * Xe
    clip = np.maximum(np.abs(r) - 6 * Xe, 0)
    assert np.all(err <= step / 2 + clip + 1e-12)


def test_mxfp8_residuals_scale_rule_and_bound():
    # the group scale is the smallest power of two with amax <= 448 X, so the
    # group maximum lands in (224 X, 448 X] and nothing saturates; every
    # element rounds to nearest even on the E4M3 grid (relative step 2^-3 for
    # normals, absolute 2^-9 X below 2^-6 X)
    rng = np.random.default_rng(18)
    N, d, kvb = 300, 6, 64
    V = F.f32(rng.standard_normal((N, d)) * np.array([0.01, 0.3, 1, 3, 30, 200]))
    V[5, 2] = 0.0
    perm = rng.permutation(N).astype(np.int32)
    out = VS.vsmooth_values(V, perm, kvb, "mxfp8")
    Np = 320
    r = np.zeros((Np, d))
    r[:N] = F.f32(V[perm] - np.repeat(out["means"], kvb, 0)[:N])
    X = F.e8m0_decode(out["e8m0"].astype(np.int64))              # [Np/32, d]
    amax = np.max(np.abs(r.reshape(Np // 32, 32, d)), axis=1)
    live = amax > 0
    assert np.all((amax[live] / X[live] > 224) & (amax[live] / X[live] <= 448))
    Xe = np.repeat(X, 32, axis=0)
    a = np.abs(r) / Xe
    ulp = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    err = np.abs(out["vres"] - r) / Xe
    assert np.all(err <= ulp / 2 + 1e-12)
    # decoded = code value times the group scale, exactly
    assert np.array_equal(out["vres"], F.e4m3_decode(out["codes"]) * Xe)
    assert np.all(out["codes"][N:] == 0) and np.all(out["col_scale"] == 1)


def test_mx_exponent_rule_examples():
    # OCP MX X = 2^(floor(log2 amax) - emax) (E2M1: emax 2); E4M3 groups: the
    # smallest power of two with amax <= 448 X
    amax = np.array([1.0, 448.0, 449.0, 500.0, 0.75, 2.0 ** -130, 0.0, 224.0])
    assert list(F.mx_shared_exponent(amax, 2)) == [-2, 6, 6, 6, -3, -127, 0, 5]
    assert list(F.e4m3_group_exponent(amax)) == [-8, 0, 1, 1, -9, -127, 0, -1]


def test_nv_tensor_exponent_is_smallest_fitting_power():
    # brute force: the smallest t with amax <= 6 * 448 * 2^t
    rng = np.random.default_rng(21)
    amax = np.concatenate([[2688.0, 2688.0 * (1 + 2.0 ** -40), 1344.0, 1.0, 0.0, 3.5e-6],
                           np.exp(rng.uniform(-30, 30, 200))])
    t = F.nv_tensor_exponent(amax)
    for a, ti in zip(amax, t):
        if a == 0:
            assert ti == 0
            continue
        want = next(k for k in range(-80, 80) if a <= 2688.0 * 2.0 ** k)
        assert ti == want, (a, ti, want)
    assert list(t[:5]) == [0, 1, -1, -11, 0]


def _nvfp4_case(seed=22):
    rng = np.random.default_rng(seed)
    N, d, kvb = 300, 6, 64
    V = F.f32(rng.standard_normal((N, d)) * np.array([0.01, 0.3, 1, 3, 30, 200]))
    V[rng.integers(0, N, 5), 1] *= 50.0                  # a few outliers in one channel
    perm = rng.permutation(N).astype(np.int32)
    out = VS.vsmooth_values(V, perm, kvb, "nvfp4")
    Np = 320
    r = np.zeros((Np, d))
    r[:N] = F.f32(V[perm] - np.repeat(out["means"], kvb, 0)[:N])
    return N, d, Np, r, out


def test_nvfp4_residuals_nearest_on_the_block_grid():
    """Every dequantised residual is the nearest point of its block's grid
    {+-0, 0.5, 1, 1.5, 2, 3, 4, 6} * s16 * s_t (brute force over the grid;
    values beyond 6 clip), and the block scale is the E4M3 value nearest to
    amax16 / (6 s_t)."""
    N, d, Np, r, out = _nvfp4_case()
    t = out["nv_t"]
    amax = np.max(np.abs(r[:N]))
    assert amax <= 2688.0 * 2.0 ** t and amax > 1344.0 * 2.0 ** t
    s16 = F.e4m3_decode(out["nv_scale"])                             # [Np/16, d]
    a16 = np.max(np.abs(r.reshape(Np // 16, 16, d)), axis=1)
    want = a16 / (6.0 * 2.0 ** t)
    grid8 = F.e4m3_decode(np.arange(127, dtype=np.uint8))
    nearest = grid8[np.argmin(np.abs(grid8[None, :] - want.reshape(-1, 1)), axis=1)].reshape(want.shape)
    assert np.all(np.abs(s16 - want) <= np.abs(nearest - want) + 1e-300)
    den = np.repeat(s16 * 2.0 ** t, 16, axis=0)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    cand = np.sign(r)[..., None] * grid * den[..., None]
    best = np.min(np.abs(cand - r[..., None]), axis=-1)
    err = np.abs(out["vres"] - r)
    rel_ulp = 2.0 ** -20 * np.abs(r)                                 # the fp32 quotient's rounding
    assert np.all(err <= best + rel_ulp + 1e-300)
    assert np.array_equal(out["vres"], F.e2m1_decode(out["codes"]) * den)
    assert np.all(out["codes"][N:] == 0) and np.all(out["col_scale"] == 1)


def test_nvfp4_scales_with_powers_of_two():
    # scaling V by 2^k scales the residuals, the second-level scale and the
    # dequantised values by 2^k and leaves codes and block scales unchanged
    N, d, Np, r, out = _nvfp4_case(23)
    rng = np.random.default_rng(23)
    V = F.f32(rng.standard_normal((N, d)) * np.array([0.01, 0.3, 1, 3, 30, 200]))
    V[rng.integers(0, N, 5), 1] *= 50.0
    perm = rng.permutation(N).astype(np.int32)
    for k in (-7, 5):
        o2 = VS.vsmooth_values(V * 2.0 ** k, perm, 64, "nvfp4")
        assert o2["nv_t"] == out["nv_t"] + k
        assert np.array_equal(o2["codes"], out["codes"]) and np.array_equal(o2["nv_scale"], out["nv_scale"])
        assert np.array_equal(o2["vres"], out["vres"] * 2.0 ** k)


def test_vsmooth_off_is_plain_per_channel_quantisation():
    rng = np.random.default_rng(18)
    V = F.f32(rng.standard_normal((100, 4)))
    out = VS.vsmooth_values(V, np.arange(100, dtype=np.int32), 64, "e4m3", vsmooth=False)
    assert np.all(out["means"] == 0)
    s = F.f32(np.max(np.abs(V), 0) / 448)
    assert np.array_equal(out["codes"][:100], F.e4m3_encode(F.f32(V / s)))


def test_ksmooth_per_block_scale_and_shift():
    rng = np.random.default_rng(19)
    N, d, kvb = 130, 4, 64
    K = F.f32(rng.standard_normal((N, d)) + 5.0)
    perm = rng.permutation(N).astype(np.int32)
    ks = VS.ksmooth(K, perm, kvb)
    mu = ks["mu"]
    for j in range(d):
        exact = sum(Fraction(float(x)) for x in K[:, j]) / N
        assert mu[j] == float(np.float32(float(exact)))
    Kp = F.f32(K - mu)[perm]
    for b in range(3):
        lo, hi = b * kvb, min((b + 1) * kvb, N)
        s = ks["k_scale"][b]
        assert s == float(F.f32(np.max(np.abs(Kp[lo:hi])) / 448))
        assert np.max(np.abs(ks["kdec"][lo:hi])) == 448.0


# ---- carrying the clustering across denoising steps ----

def test_final_centroids_are_exact_member_means():
    # final = member means of the last pass's clusters, each the fp32
    # rounding of the exact rational mean; empty clusters keep the centroid
    rng = np.random.default_rng(21)
    V = F.f32(rng.standard_normal((60, 3)) * 4)
    init = np.array([0, 1, 2, 3, 4, 4 + 50], np.int32)
    labels, used, final = KM.kmeans(V, init, iters=2)
    for c in range(init.size):
        mem = V[labels == c]
        for j in range(3):
            if len(mem) == 0:
                assert final[c, j] == used[-1][c, j]
            else:
                exact = sum(Fraction(float(x)) for x in mem[:, j]) / len(mem)
                assert final[c, j] == float(np.float32(float(exact)))


def test_warm_start_from_converged_centroids_is_a_fixed_point():
    # Lloyd's fixed point: once the labels stop changing, one warm-started
    # pass from the final centroids reproduces the labels and the centroids
    rng = np.random.default_rng(22)
    centers = rng.standard_normal((6, 8)) * 10
    V = F.f32(centers[rng.integers(0, 6, 400)] + rng.standard_normal((400, 8)) * 0.3)
    init = rng.choice(400, 6, replace=False).astype(np.int32)
    labels, _, final = KM.kmeans(V, init, iters=12)
    l2, used2, f2 = KM.kmeans(V, None, 1, init_centroids=final)
    assert np.array_equal(used2[0], final)
    assert np.array_equal(l2, labels)
    assert np.array_equal(f2, final)


def test_warm_start_equals_continuing_the_passes():
    # I passes from V[init] then J passes from its final centroids equal
    # I + J passes: the carried state is exactly the centroids of pass I + 1
    rng = np.random.default_rng(23)
    V = F.f32(rng.standard_normal((300, 6)) * 3)
    init = rng.choice(300, 9, replace=False).astype(np.int32)
    l5, u5, f5 = KM.kmeans(V, init, iters=5)
    l2, u2, f2 = KM.kmeans(V, init, iters=2)
    l3, u3, f3 = KM.kmeans(V, None, 3, init_centroids=f2)
    assert np.array_equal(l3, l5) and np.array_equal(f3, f5)
    for a, b in zip(u2 + u3, u5):
        assert np.array_equal(a, b)


def test_prepare_with_given_perm_reproduces_the_clustered_prepare():
    # the residuals, means, scales and K codes depend on the clustering only
    # through the permutation
    w = inputs.small(inputs.WORKLOADS["tiny"], N=700, seed=31)
    q, k, v, init = inputs.gen_head(w, 0, 0)
    K, V = oracle.bf16_to_f64(k), oracle.bf16_to_f64(v)
    full = oracle.prepare_head(K, V, init, w.k, w.iters, w.kv_block)
    again = oracle.prepare_head(K, V, None, w.k, w.iters, w.kv_block, perm=full["perm"])
    assert np.array_equal(again["perm"], full["perm"])
    for part in ("v", "k"):
        for key, val in full[part].items():
            assert np.array_equal(np.asarray(again[part][key]), np.asarray(val)), (part, key)


# ---------------------------------------------------------------- cluster ordering
def test_order_of_collinear_centroids_is_monotone():
    # q_c = a_c * u: the principal axis is +-u, so the order follows a_c
    rng = np.random.default_rng(31)
    for _ in range(20):
        u = rng.integers(-4, 5, 16)
        u[0] = 3
        a = rng.permutation(np.arange(-25, 26))[:40]
        q = a[:, None] * u[None, :]
        rank = KM.order_clusters(q)
        seq = a[np.argsort(rank)]
        assert np.all(np.diff(seq) > 0) or np.all(np.diff(seq) < 0)


def test_integer_axis_matches_the_top_eigenvector():
    # a dominant direction plus noise: the integer power iteration lands on
    # the top eigenvector of the fp64 covariance (numpy.linalg.eigh)
    rng = np.random.default_rng(32)
    for d, k in ((16, 64), (64, 256), (128, 1024)):
        w = rng.standard_normal(d)
        w /= np.linalg.norm(w)
        t = rng.standard_normal(k) * 30.0
        q = np.clip(np.rint(t[:, None] * w[None, :] + rng.standard_normal((k, d)) * 3.0), -127, 127).astype(np.int64)
        v = KM.principal_axis_int(q).astype(np.float64)
        ev = np.linalg.eigh(np.cov(q.T.astype(np.float64)))[1][:, -1]
        cos = abs(v @ ev) / np.linalg.norm(v)
        assert cos > 0.9999, (d, k, cos)


def test_order_is_equivariant_under_relabelling():
    rng = np.random.default_rng(33)
    q = rng.integers(-127, 128, (200, 32))
    rank = KM.order_clusters(q)
    p = q @ KM.principal_axis_int(q)
    assert len(np.unique(p)) == len(p)          # no ties: the order is the projection order
    pi = rng.permutation(200)
    rank2 = KM.order_clusters(q[pi])
    assert np.array_equal(rank2, rank[pi])


def test_order_ties_and_degenerate_sets():
    rng = np.random.default_rng(34)
    q = rng.integers(-50, 51, (30, 8))
    q[17] = q[4]                                # duplicate: adjacent, lower index first
    rank = KM.order_clusters(q)
    assert rank[17] == rank[4] + 1
    same = np.tile(rng.integers(-9, 10, 8), (12, 1))
    assert np.array_equal(KM.order_clusters(same), np.arange(12))
    assert sorted(KM.order_clusters(q)) == list(range(30))


def test_ordered_kmeans_renumbers_the_unordered_result():
    # the final pass with renumbered centroids assigns every token without a
    # distance tie to the renumbered cluster; the final member means follow
    w = inputs.WORKLOADS["tiny"]
    q, k, v, init = inputs.gen_all(w, H=1)
    V = oracle.bf16_to_f64(v[0, 0])
    lab0, used0, fin0 = KM.kmeans(V, init[0, 0], w.iters)
    lab1, used1, fin1 = KM.kmeans(V, init[0, 0], w.iters, order=True)
    sV = KM.int8_scale(V)
    Cq = KM.quant_i8(used0[-1], sV)
    rank = KM.order_clusters(Cq)
    assert np.array_equal(used1[-1][rank], used0[-1])
    Vq = KM.quant_i8(V, sV)
    D = np.sum(Cq * Cq, axis=1)[None, :] - 2.0 * (Vq @ Cq.T)
    tie = np.sum(D == D.min(axis=1, keepdims=True), axis=1) > 1
    assert np.array_equal(lab1[~tie], rank[lab0[~tie]])
    if not tie.any():
        assert np.array_equal(fin1[rank], fin0)
    perm1 = oracle.prepare_head(oracle.bf16_to_f64(k[0, 0]), V, init[0, 0], w.k, w.iters, w.kv_block,
                                cluster_order=True)["perm"]
    assert np.all(np.diff(lab1[perm1]) >= 0)


# ---- seeded initialisation: splitmix64 + partial Fisher-Yates ----

def test_splitmix64_published_outputs():
    # reference outputs of splitmix64 (Steele, Lea and Flood 2014; the
    # generator's published test values from state 0 and state 1234567)
    from oracle.kmeans import splitmix64
    g = splitmix64(0)
    assert [next(g) for _ in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert next(splitmix64(1234567)) == 0x599ED017FB08FC85


def test_partial_fisher_yates_worked_example():
    # N = 5, k = 3 with draws 7, 2, 9 (worked by hand):
    #   i = 0: j = 0 + 7 mod 5 = 2 -> [2, 1, 0, 3, 4]
    #   i = 1: j = 1 + 2 mod 4 = 3 -> [2, 3, 0, 1, 4]
    #   i = 2: j = 2 + 9 mod 3 = 2 -> unchanged; result [2, 3, 0]
    from oracle.kmeans import partial_fisher_yates
    assert partial_fisher_yates(5, 3, iter([7, 2, 9])).tolist() == [2, 3, 0]
    # k = N is a whole permutation; a zero draw never moves anything
    assert partial_fisher_yates(4, 4, iter([0, 0, 0, 0])).tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("N,k", [(1024, 16), (4096, 4096), (75600, 1024), (7, 7), (1, 1)])
def test_seeded_init_draws_distinct_tokens(N, k):
    from oracle.kmeans import seeded_init
    a = seeded_init(1002, 0, N, k)
    b = seeded_init(1002, 1, N, k)
    assert a.dtype == np.int32 and a.shape == (k,)
    assert np.unique(a).size == k and a.min() >= 0 and a.max() < N
    if k == N:
        assert np.array_equal(np.sort(a), np.arange(N))
    if k > 4:
        assert not np.array_equal(a, b)          # every head has its own stream
    assert np.array_equal(a, seeded_init(1002, 0, N, k))


def test_seeded_init_is_uniform_over_tokens():
    # every token is equally likely to be drawn: over 2000 heads with N = 20,
    # k = 5, each token is drawn ~500 times (binomial sd ~19)
    from oracle.kmeans import seeded_init
    cnt = np.zeros(20)
    for bh in range(2000):
        cnt[seeded_init(7, bh, 20, 5)] += 1
    assert np.all(np.abs(cnt - 500) < 100)


# ---- balanced clusters: capped assignment ----

def test_capped_assign_worked_examples():
    # worked by hand on one channel (codes as given, scale irrelevant):
    # tokens 0 1 2 3 10 11, centroids 1 and 11, three places each.  Round 1:
    # tokens 0..3 propose to centroid 1 (distances 1 0 1 4), which takes
    # token 1, then 0 and 2 (a distance tie, lower token first); 10 and 11
    # go to centroid 11.  Round 2: token 3 proposes to the only cluster with
    # room left.
    Vq = np.array([[0.0], [1.0], [2.0], [3.0], [10.0], [11.0]])
    Cq = np.array([[1.0], [11.0]])
    assert KM.capped_assign(Vq, Cq, np.array([3, 3])).tolist() == [0, 0, 0, 1, 1, 1]
    # a distance tie between two tokens for one place goes to the lower token
    assert KM.capped_assign(np.array([[0.0], [2.0], [48.0]]), np.array([[1.0], [49.0]]),
                            np.array([1, 2])).tolist() == [0, 1, 1]
    # a token equidistant from two clusters proposes to the lower index
    assert KM.capped_assign(np.array([[5.0], [9.0]]), np.array([[3.0], [7.0]]),
                            np.array([1, 1])).tolist() == [0, 1]
    # with no rounds the places are filled in token order, clusters in index order
    assert KM.capped_assign(np.zeros((5, 1)), np.zeros((2, 1)), np.array([2, 3]), rounds=0).tolist() == \
        [0, 0, 1, 1, 1]


def test_capped_assign_is_plain_assignment_when_nothing_overflows():
    # capacities equal to the sizes of the unconstrained assignment: every
    # proposal is accepted in the first round, so the result is the plain
    # argmin with lowest-index ties
    rng = np.random.default_rng(31)
    Vq = rng.integers(-20, 21, (300, 6)).astype(np.float64)
    Cq = rng.integers(-20, 21, (9, 6)).astype(np.float64)
    plain = KM.assign(Vq, Cq)
    cap = np.bincount(plain, minlength=9)
    assert np.array_equal(KM.capped_assign(Vq, Cq, cap), plain)


@pytest.mark.parametrize("N,kvb", [(1000, 64), (300, 128), (64, 64), (77, 64)])
def test_capped_assign_fills_every_cluster_exactly(N, kvb):
    rng = np.random.default_rng(N)
    cap = KM.block_capacities(N, kvb)
    assert cap.sum() == N and np.all(cap[:-1] == kvb) and 1 <= cap[-1] <= kvb
    Vq = rng.integers(-127, 128, (N, 8)).astype(np.float64)
    Cq = Vq[rng.choice(N, cap.size, replace=False)]
    lab = KM.capped_assign(Vq, Cq, cap)
    assert np.array_equal(np.bincount(lab, minlength=cap.size), cap)


def test_balanced_kmeans_recovers_groups_of_block_size():
    # four well separated groups of exactly 64 tokens (one block each): the
    # balanced clustering puts every group in one cluster, whatever the start
    rng = np.random.default_rng(4)
    centers = np.array([[60.0, 0], [-60, 0], [0, 60], [0, -60]])
    grp = rng.permutation(np.repeat(np.arange(4), 64))
    V = F.f32(centers[grp] + rng.standard_normal((256, 2)))
    init = np.array([0, 1, 2, 3], dtype=np.int32)          # possibly two starts in one group
    lab, _, _ = KM.kmeans(V, init, 4, capacities=KM.block_capacities(256, 64))
    for g in range(4):
        assert np.unique(lab[grp == g]).size == 1
    assert np.unique(lab).size == 4


@pytest.mark.parametrize("N,kvb", [(1024, 64), (1000, 128), (333, 64)])
def test_balanced_prepare_gives_one_cluster_per_block(N, kvb):
    w = inputs.small(inputs.WORKLOADS["tiny"], N=N, kv_block=kvb)
    q, k, v, _ = inputs.gen_head(w, 0, 0)
    nblk = (N + kvb - 1) // kvb
    init = KM.seeded_init(5, 0, N, nblk)
    prep = oracle.prepare_head(oracle.bf16_to_f64(k), oracle.bf16_to_f64(v), init, nblk, 3, kvb, balanced=True)
    sorted_labels = prep["labels"][prep["perm"]]
    for b in range(nblk):
        assert np.all(sorted_labels[b * kvb:(b + 1) * kvb] == b)
