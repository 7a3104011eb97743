"""Pins for the oracle's attention: quantisation-disabled equals fp64 softmax
attention, the mean-restoration identity in exact rationals, and special
cases whose result is known in closed form."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import formats as F
from oracle.attention import attend_tile, exact_attention, softmax_scale
from bit_attention_video_amd import inputs
from closed_forms import unit_log2_scale


def _head(N, d=64, kvb=64, k=16, seed=7):
    w = inputs.small(inputs.WORKLOADS["tiny"], N=N, d=d, kv_block=kvb, k=k, seed=seed)
    q, kk, v, init = inputs.gen_head(w, 0, 0)
    return w, oracle.bf16_to_f64(q), oracle.bf16_to_f64(kk), oracle.bf16_to_f64(v), init


def _all_rows(Q, prep, scale=0.0):
    o = oracle.attend_rows(Q, prep, range(oracle.n_q_tiles(Q.shape[0])), scale)
    return np.concatenate([o[t] for t in sorted(o)])


@pytest.mark.parametrize("N,d,kvb,vs", [(1000, 64, 64, True), (1000, 64, 64, False),
                                        (700, 128, 128, True), (129, 64, 64, True), (64, 64, 64, True)])
def test_quantisation_disabled_equals_exact_attention(N, d, kvb, vs):
    w, Q, K, V, init = _head(N, d, kvb)
    prep = oracle.prepare_head(K, V, init, w.k, w.iters, kvb, vsmooth_on=vs, quantize=False)
    O = _all_rows(Q, prep)
    ref = exact_attention(Q, K, V, softmax_scale(d))
    assert np.max(np.abs(O - ref)) <= 1e-6 * np.max(np.abs(V))
    assert np.max(np.abs(O - ref)) <= 1e-12 * np.max(np.abs(V))


def test_mean_restoration_identity_exact():
    # P.(mean 1^T + R) = rowsum * mean^T + P.R, in exact rationals, with
    # P holding decoded E4M3 bytes and mean / R holding fp32 values
    rng = np.random.default_rng(20)
    n, kb, d = 3, 5, 4
    P = F.e4m3_decode(rng.integers(0, 57, (n, kb)))
    mean = F.f32(rng.standard_normal(d) * 3)
    R = F.e4m3_decode(rng.integers(0, 0x7E, (kb, d)))
    Pf = [[Fraction(float(x)) for x in row] for row in P]
    Mf = [Fraction(float(x)) for x in mean]
    Rf = [[Fraction(float(x)) for x in row] for row in R]
    for i in range(n):
        rs = sum(Pf[i])
        for c in range(d):
            lhs = sum(Pf[i][j] * (Mf[c] + Rf[j][c]) for j in range(kb))
            rhs = rs * Mf[c] + sum(Pf[i][j] * Rf[j][c] for j in range(kb))
            assert lhs == rhs
    # and at a moderate size in fp64
    P = F.e4m3_decode(rng.integers(0, 57, (128, 128)))
    mean = F.f32(rng.standard_normal(128) * 3)
    R = F.e4m3_decode(rng.integers(0, 0x7E, (128, 128)))
    lhs = P @ (mean[None, :] + R)
    rhs = P.sum(1)[:, None] * mean[None, :] + P @ R
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(lhs))


def _dequantised_values(prep, N):
    v = prep["v"]
    kvb = prep["kv_block"]
    return (v["vres"] * v["col_scale"][None, :] + np.repeat(v["means"], kvb, 0))[:N]


def test_equal_scores_give_mean_of_dequantised_values():
    # Q = 0: every score is 0, every byte is 56 (p = 1), so O is the plain mean
    # of the dequantised (permuted) values over the real keys
    w, Q, K, V, init = _head(200, 64, 64)
    prep = oracle.prepare_head(K, V, init, w.k, w.iters, 64)
    trace = {}
    O = oracle.attend_rows(np.zeros_like(Q[:128]), prep, [0], trace=trace)[0]
    assert all(np.all(c[:, :min(64, 200 - 64 * b)] == 56) for b, c in enumerate(trace["codes"]))
    want = _dequantised_values(prep, 200).mean(0)
    assert np.max(np.abs(O - want[None, :])) <= 1e-12 * np.max(np.abs(want))


def test_dominant_key_gives_its_value_row():
    # one key scores ~36 log2-units above every other key and sits in the
    # first block (identity order, V-Smooth off): every later byte is
    # round(8z+56+beta) with z <= -36, i.e. 0, so O is exactly that key's
    # dequantised value row.  (Keys in blocks before it would keep a
    # 2^-36-rescaled share, so the closed form needs it first.)
    w, Q, K, V, init = _head(300, 64, 64)
    Q = np.zeros_like(Q)
    Q[:, 0] = 1.0
    K = K.copy()
    K[:, 0] = 0.0
    K[0, 0] = 200.0
    prep = oracle.prepare_head(K, V, init, w.k, w.iters, 64, vsmooth_on=False)
    O = oracle.attend_rows(Q, prep, [0, 1, 2])
    want = _dequantised_values(prep, 300)[0]
    for t in O.values():
        assert np.max(np.abs(t - want[None, :])) <= 1e-12 * np.max(np.abs(want))


def test_single_block_and_rowsum_exact_in_fp32():
    w, Q, K, V, init = _head(64, 64, 64)
    prep = oracle.prepare_head(K, V, init, w.k, w.iters, 64)
    trace = {}
    oracle.attend_rows(Q, prep, [0], trace=trace)
    assert len(trace["codes"]) == 1
    p = F.e4m3_decode(trace["codes"][0])
    # decoded bytes are multiples of 2^-9 and <= 1: a 64- or 128-term sum is
    # exact in fp32 whatever the order
    s64 = p.sum(1)
    s32 = p.astype(np.float32)[:, ::-1].sum(1, dtype=np.float32)
    assert np.array_equal(s64, s32.astype(np.float64))
    assert np.all(np.max(p, axis=1) == 1.0)     # the row max always gets byte 56


def test_expcast_never_binds_upper_clamp_on_workload():
    # x = fma(S, 8c, 56+beta-8m) stays below 56.5 for every key, so the upper
    # clamp of [0, 56] is never what decides a byte on this data
    w, Q, K, V, init = _head(1024, 64, 64)
    prep = oracle.prepare_head(K, V, init, w.k, w.iters, 64)
    trace = {}
    oracle.attend_rows(Q, prep, range(8), trace=trace)
    for S32, A, B in zip(trace["S32"], trace["A"], trace["B"]):
        x = F.fma_f32(S32, A, B[:, None])
        assert np.nanmax(np.where(np.isfinite(x), x, -1)) < 56.5


def test_vsmooth_and_expcast_fidelity_direction():
    # directional claims of the pages on a synthetic head: with the 4-bit
    # residual format, V-Smooth raises PSNR against exact attention
    w, Q, K, V, init = _head(1024, 64, 64, k=16)
    ref = exact_attention(Q, K, V, softmax_scale(64))
    on = _all_rows(Q, oracle.prepare_head(K, V, init, 16, 3, 64, fmt="mxfp4", vsmooth_on=True))
    off = _all_rows(Q, oracle.prepare_head(K, V, init, 16, 3, 64, fmt="mxfp4", vsmooth_on=False))
    assert oracle.psnr(on, ref) > oracle.psnr(off, ref)


def test_vsmooth_direction_with_e4m3_residuals_per_probability_mode():
    # the headline configuration (E4M3 residuals, d=128, kv_block 128) on a
    # 2048-token head. With probabilities whose cut-off lies far below the
    # weights that matter (range-shifted ExpCast, exp2 + E4M3 cast) V-Smooth
    # raises PSNR, as the pages report. With the literal ExpCast bytes (cut-off
    # near p = 2^-7 of the running max, p-linear below 2^-6) the per-block
    # weight error turns coherent once a block is one cluster, and V-Smooth
    # lowers PSNR on these diffuse synthetic scores.
    w, Q, K, V, init = _head(2048, 128, 128, k=16)
    ref = exact_attention(Q, K, V, softmax_scale(128))
    p = {}
    for vs in (True, False):
        prep = oracle.prepare_head(K, V, init, 16, 3, 128, vsmooth_on=vs)
        for mode in ("expcast", "expcast_shifted", "exp2"):
            o = oracle.attend_rows(Q, prep, range(oracle.n_q_tiles(2048)), mode=mode)
            p[vs, mode] = oracle.psnr(np.concatenate([o[t] for t in sorted(o)]), ref)
    for mode in ("expcast_shifted", "exp2"):
        assert p[True, mode] > p[False, mode] + 0.5
    assert p[True, "expcast"] < p[False, "expcast"] - 3.0
    # shifted bytes cost well under a dB against exp2 + cast; literal ones cost far more
    assert p[True, "exp2"] - 1.0 < p[True, "expcast_shifted"] <= p[True, "exp2"]
    assert p[True, "expcast_shifted"] > p[True, "expcast"] + 5.0


# ---- ExpCast off: p = E4M3(2^x), x = fma(S, c, -m) ----

def test_exp2cast_bytes_at_integer_exponents():
    # 2^-k for integer k is an E4M3 value down to 2^-9 (normals to 2^-6, then
    # subnormal multiples of 2^-9); 2^-10 is the tie between 0 and 2^-9 and
    # goes to the even code 0; -inf (a padded key) gives 0
    from oracle.attention import exp2cast_bytes
    z = np.array([0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11, -40, -np.inf], np.float32)
    got = exp2cast_bytes(z, 1.0, np.zeros(1, np.float32))
    want = [0x38, 0x30, 0x28, 0x20, 0x18, 0x10, 0x08, 0x04, 0x02, 0x01, 0x00, 0x00, 0x00, 0x00]
    assert got.tolist() == want


def test_exp2cast_is_nearest_e4m3_of_the_power():
    # brute force over every non-negative E4M3 code: the byte is the code
    # nearest to 2^x (ties to even), checked against a scan of all 127 values
    from oracle.attention import exp2cast_bytes
    rng = np.random.default_rng(3)
    x = rng.uniform(-12.0, 0.0, 4000).astype(np.float32)
    got = exp2cast_bytes(x, 1.0, np.zeros(1, np.float32)).astype(np.int64)
    codes = np.arange(0, 127)
    vals = F.e4m3_decode(codes.astype(np.uint8))
    p = np.exp2(x.astype(np.float64))
    dist = np.abs(p[:, None] - vals[None, :])
    best = np.min(dist, axis=1)
    for i in range(x.size):
        cand = codes[dist[i] == best[i]]
        want = cand[0] if cand.size == 1 else cand[cand % 2 == 0][0]
        assert got[i] == want


def test_exp2cast_uses_the_same_argument_as_expcast():
    # both modes see the same scores, maxima and block order: on one block the
    # ExpCast bytes equal round(8x + 56 + beta) of the exp2 argument x up to
    # the two single roundings, so their decoded values agree within one
    # ExpCast step (a factor 2^(1/8) per code, plus the offset beta/8)
    w, Q, K, V, init = _head(64, 64, 64)
    prep = oracle.prepare_head(K, V, init, w.k, w.iters, 64)
    te, tx = {}, {}
    oracle.attend_rows(Q, prep, [0], trace=te, mode="expcast")
    oracle.attend_rows(Q, prep, [0], trace=tx, mode="exp2")
    assert np.array_equal(te["S32"][0], tx["S32"][0])
    pe = F.e4m3_decode(te["codes"][0])
    px = F.e4m3_decode(tx["codes"][0])
    big = px >= 2.0 ** -6            # normal range of both encodings
    ratio = pe[big] / px[big]
    assert np.all(ratio <= 2.0 ** (1.0 / 8 + 1.0 / 16 + 0.06)) and np.all(ratio >= 2.0 ** -(1.0 / 8 + 1.0 / 16 + 0.06))


def test_exp2cast_is_closer_to_exact_than_expcast():
    # the fidelity direction the pages report for ExpCast (it costs PSNR)
    w, Q, K, V, init = _head(1024, 64, 64, k=16)
    ref = exact_attention(Q, K, V, softmax_scale(64))
    prep = oracle.prepare_head(K, V, init, 16, 3, 64)
    on = np.concatenate([o for _, o in sorted(oracle.attend_rows(Q, prep, range(8), mode="expcast").items())])
    off = np.concatenate([o for _, o in sorted(oracle.attend_rows(Q, prep, range(8), mode="exp2").items())])
    assert oracle.psnr(off, ref) > oracle.psnr(on, ref)


@pytest.mark.parametrize("mode,window", [("expcast", 6), ("exp2", 9), ("expcast_shifted", 14)])
def test_integer_log2_scores_give_exact_base2_softmax(mode, window):
    """Closed form for the whole quantised composition (bytes from the FMA,
    decode, online rescaling across blocks, row sums, mean restoration, column
    scale, padded tail).  When every log2-domain score is an integer within
    `window` of the running maximum, the probability bytes are exactly
    2^(t - m): ExpCast's 8z + 56 + beta rounds to 8z + 56 for |beta| < 0.5 and
    z in [-6, 0], which is the E4M3 code of 2^z; the exp2 path is exact down to
    the smallest subnormal 2^-9; the range-shifted ExpCast's 8z + 120 + beta
    is the code of 2^(z+8) for z in [-14, 0], and the common 2^8 cancels.
    The output must then equal the base-2 softmax
    of the scores applied to col_scale * vres + mean, computed here in exact
    rationals from that definition alone."""
    rng = np.random.default_rng(7)
    d, kvb, N = 4, 4, 10                       # three blocks, the last with 2 real keys
    nblk = (N + kvb - 1) // kvb
    n = 5
    # channel 0 carries 448 in one query row (so s_q = 1) and is zero in every key
    Q = rng.integers(-2, 3, size=(n, d)).astype(np.float64)
    if window > 9:
        Q = rng.integers(-4, 5, size=(n, d)).astype(np.float64)
    Q[:, 0] = 0.0
    Q[0, 0] = 448.0
    kdec = np.zeros((nblk * kvb, d))
    kdec[:N, 1:] = rng.integers(-1, 2, size=(N, d - 1))
    kdec[N:, 1:] = 1.0                           # padded rows score like real keys unless masked
    S = Q @ kdec[:N].T
    # every score within `window` of the row maximum (so also of the running
    # maximum at its block); the running maximum moves after the first block in
    # some row (rescaling is exercised); unmasked, a padded key would carry
    # weight in some row
    assert np.all(S.max(axis=1, keepdims=True) - S <= window)
    assert np.any(S[:, :kvb].max(axis=1) < S.max(axis=1))
    assert np.any((Q @ kdec[N:].T).max(axis=1) >= S.max(axis=1) - 6)
    if window > 9:                               # the shifted mode reaches further down
        assert np.any(S.max(axis=1, keepdims=True) - S > 9)
    vres = np.zeros((nblk * kvb, d))
    vres[:N] = rng.integers(-16, 17, size=(N, d)) / 8.0
    vres[N:] = 123.0                             # padded rows must not contribute
    col_scale = np.array([0.5, 1.0, 2.0, 0.25])
    means = rng.integers(-8, 9, size=(nblk, d)) / 4.0
    scale = unit_log2_scale()
    O = attend_tile(Q, kdec, np.ones(nblk), vres, col_scale, means, N, kvb, scale, beta=-0.25, mode=mode)
    for i in range(n):
        w = [Fraction(2) ** int(S[i, j]) for j in range(N)]
        tot = sum(w)
        for c in range(d):
            want = sum(w[j] * (Fraction(col_scale[c]) * Fraction(vres[j, c]) + Fraction(means[j // kvb, c]))
                       for j in range(N)) / tot
            assert abs(O[i, c] - float(want)) <= 1e-13 * (1 + abs(float(want))), (mode, i, c, O[i, c], want)


@pytest.mark.parametrize("mode", ["expcast", "exp2"])
def test_integer_score_inputs_through_the_whole_oracle(mode):
    """The inputs of closed_forms.integer_score_qkv through the oracle's own
    preparation (V-Smooth off: identity order, K smoothing, per-block s_k,
    per-channel s_v) and attention reproduce the base-2 softmax of the integer
    scores; the same inputs pin the GPU path."""
    from closed_forms import integer_score_qkv, base2_softmax
    N, d, kvb = 300, 64, 64
    Q, K, V = integer_score_qkv(N, d, kvb)
    prep = oracle.prepare_head(K, V, None, 1, 1, kvb, "e4m3", False)
    assert np.all(prep["k"]["k_scale"] == 1.0) and np.all(prep["v"]["col_scale"] == 1.0)
    S = Q @ K.T
    assert np.all(np.abs(S) <= 3) and np.all(S == np.rint(S))
    tiles = list(range(oracle.n_q_tiles(N)))
    rows = oracle.attend_rows(Q, prep, tiles, unit_log2_scale(), -0.25, mode=mode)
    O = np.concatenate([rows[t] for t in tiles])
    want = base2_softmax(S, V)
    assert np.max(np.abs(O - want)) <= 1e-12 * np.max(np.abs(want))


# ---- small pins of the helpers every check uses ----

def test_softmax_scale_default_and_explicit():
    # 1/sqrt(64) = 0.125 exactly; 1/sqrt(128) = 2^-3 / sqrt(2), whose binary32
    # pattern is 0x3DB504F3 (the binary32 1/sqrt(2), 0x3F3504F3, three binades
    # down); an explicit scale is used as its binary32 value
    assert softmax_scale(64) == 0.125
    assert np.float32(softmax_scale(128)).view(np.uint32) == 0x3DB504F3
    assert softmax_scale(64, 0.07) == float(np.float32(0.07))


def test_psnr_worked_example():
    # peak |O_ref| = 4, squared 16; two of four entries off by 0.1, so
    # MSE = 0.02 / 4 = 0.005 and PSNR = 10 log10(3200) = 35.0515 dB
    ref = np.array([[1.0, -2.0], [0.0, 4.0]])
    out = ref + np.array([[0.1, 0.0], [0.0, -0.1]])
    assert abs(oracle.psnr(out, ref) - 35.05149978) < 1e-6
    assert oracle.psnr(ref.copy(), ref) == float("inf")
    # the peak is taken from the reference, not from the output
    assert abs(oracle.psnr(ref + 10.0, ref) - 10 * np.log10(16 / 100.0)) < 1e-9


# ---- the parity bound is tight enough to see a wrong ExpCast offset ----

TIGHT_REL_L2 = 1e-3       # the tighter O bound of the GPU parity tests (fp32 output)


def test_beta_and_mode_changes_exceed_the_tight_bound():
    """A mid-shaped head (N = 4096, d = 128, 64-key blocks): the oracle's O
    with a different ExpCast offset, or with ExpCast off, moves by more than
    twice the tight rel-L2 bound the GPU parity tests apply, so a kernel with
    a wrong beta, a wrong FMA addend or the wrong probability mode fails
    them."""
    w = inputs.small(inputs.WORKLOADS["mid"], N=4096, k=64)
    q, kk, v, init = inputs.gen_head(w, 0, 0)
    Q, K, V = (oracle.bf16_to_f64(a) for a in (q, kk, v))
    prep = oracle.prepare_head(K, V, init, 64, 3, 64)
    tiles = list(range(0, oracle.n_q_tiles(4096), 4))

    def run(beta=oracle.DEFAULT_BETA, mode="expcast"):
        o = oracle.attend_rows(Q, prep, tiles, 0.0, beta, mode=mode)
        return np.concatenate([o[t] for t in tiles])

    base = run()
    for other in (run(beta=0.0), run(beta=0.3), run(mode="exp2"), run(mode="expcast_shifted")):
        rel = np.linalg.norm(other - base) / np.linalg.norm(base)
        assert rel > 2 * TIGHT_REL_L2, rel


# ---- tiny nonzero inputs: every quantiser scale is floored at 2^-126 ----

def test_scale_floor():
    from oracle.attention import scale_of
    assert scale_of(0.0, 448.0) == 1.0
    assert scale_of(448.0, 448.0) == 1.0
    assert scale_of(1e-40, 448.0) == 2.0 ** -126          # would be subnormal
    assert scale_of(448.0 * 2.0 ** -126, 448.0) == 2.0 ** -126
    assert scale_of(448.0 * 2.0 ** -125, 448.0) == 2.0 ** -125


def test_tiny_value_channel_keeps_a_finite_scale():
    # one channel of V holds values near 1e-37 (normal fp32, but max/448 is
    # subnormal): its residual scale is floored at 2^-126, its codes stay
    # finite, and O for that channel matches exact attention to the
    # quantisation error of the other channels, relative to the channel
    w, Q, K, V, init = _head(512, 64, 64)
    rng = np.random.default_rng(9)
    V = V.copy()
    V[:, 5] = F.f32(rng.standard_normal(512) * 1e-37)
    V[:, 5] = np.asarray(V[:, 5], np.float32).astype(np.float64)
    prep = oracle.prepare_head(K, V, init, w.k, w.iters, 64)
    assert prep["v"]["col_scale"][5] == 2.0 ** -126
    O = _all_rows(Q, prep)
    assert np.all(np.isfinite(O))
    ref = exact_attention(Q, K, V, softmax_scale(64))
    rel5 = np.linalg.norm(O[:, 5] - ref[:, 5]) / np.linalg.norm(ref[:, 5])
    rel_all = np.linalg.norm(O - ref) / np.linalg.norm(ref)
    assert rel5 < 0.2 and rel_all < 0.2
