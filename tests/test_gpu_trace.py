"""GPU parity of the fused kernel's own in-loop arithmetic, read through its
trace instantiation (vc_dbg_attn_trace: the same kernel source with stores of
the per-block scores, scale, running maximum, probability bytes and row sums
of one 256-row workgroup).

Given the kernel's own fp32 scores S of each block, checked bit for bit
against the oracle's definitions (oracle.attention):
  * the block scale c = fp32(cq * s_k[b]), cq = fp32(fp32(s_q * scale) * log2 e)
    with s_q from the oracle's query-tile quantiser;
  * the running maximum m_b = max(m_{b-1}, fp32(c * max_j S_j));
  * the probability bytes = clamp(rne(fma(S, 8c, fp32(kc - 8 m_b))), 0, top)
    (ExpCast, kc = 56 + beta, top 56; range-shifted, kc = 120 + beta, top 120),
    or E4M3(2^fma(S, c, -m_b)) for ExpCast off (one code of slack where 2^x
    lies within 2^-21 of an E4M3 rounding midpoint: v_exp_f32 is not
    correctly rounded);
  * the row sums = the exact sum of the decoded bytes.
The scores themselves are checked against the exact dot products of the
query and key codes within the FP8 matrix instruction's accumulation window
(groups of 8 products aligned to the largest; bits about 13 places below it
dropped), and the trace instantiation's O equals the production kernel's.
A closed form with V-Smooth on pins the mean restoration.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from oracle.attention import LOG2E, expcast_bytes, exp2cast_bytes, quantize_q_tile, softmax_scale
from bit_attention_video_amd import binding as vb
from bit_attention_video_amd import inputs
from layouts import to_device_bf16

pytestmark = pytest.mark.gpu

MODES = {"expcast": vb.EXPCAST, "exp2": vb.EXP2_CAST, "shifted": vb.EXPCAST_SHIFTED}
ORACLE_MODE = {"expcast": "expcast", "exp2": "exp2", "shifted": "expcast_shifted"}
TOP = {"expcast": 56.0, "shifted": 120.0}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vb.lib()


def exp2_bytes_within_midpoint_slack(got, S, A, B):
    """ExpCast-off bytes: equal to the oracle's, except one code where 2^x is
    within 2^-21 (relative) of an E4M3 rounding midpoint.  Returns the number
    of such one-code differences; asserts there is no other difference."""
    want = exp2cast_bytes(S, A, B).astype(np.int64)
    got = got.astype(np.int64)
    x = F.fma_f32(S, A, B)
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.where(np.isnan(x) | np.isneginf(x), 0.0, np.exp2(x))
    lo = F.e4m3_decode(np.clip(want - 1, 0, 126).astype(np.uint8))
    here = F.e4m3_decode(want.astype(np.uint8))
    hi = F.e4m3_decode(np.clip(want + 1, 0, 126).astype(np.uint8))
    near = (np.abs(p - (lo + here) / 2) <= 2.0 ** -21 * p) | (np.abs(p - (here + hi) / 2) <= 2.0 ** -21 * p)
    bad = (got != want) & ~(near & (np.abs(got - want) == 1))
    assert not bad.any(), f"{np.count_nonzero(bad)} bytes differ away from a rounding midpoint"
    return int(np.count_nonzero(got != want))


def check_trace(w, host, prep_o, tr, h, group, mode, scale, beta):
    """Compare one traced workgroup (query rows 256*group ..) with the oracle's
    definitions, given the kernel's own scores."""
    N, d, kvb = w.N, w.d, w.kv_block
    S = tr["S"].cpu().numpy().astype(np.float64)      # [nblk, 256, kvb]
    P = tr["P"].cpu().numpy()
    m = tr["m"].cpu().numpy().astype(np.float64)
    c = tr["c"].cpu().numpy().astype(np.float64)
    rs = tr["rowsum"].cpu().numpy().astype(np.float64)
    nblk = S.shape[0]
    r0 = 256 * group
    rows = np.arange(r0, min(r0 + 256, N)) - r0          # real query rows of the group
    Q = oracle.bf16_to_f64(host[0][0, h])
    kdec = prep_o["k"]["kdec"]
    k_scale = prep_o["k"]["k_scale"]
    # block scale: one query scale per 128-row tile
    cq = np.empty(256)
    qdec = np.zeros((256, d))
    for t in range(2):
        lo, hi = r0 + 128 * t, min(r0 + 128 * (t + 1), N)
        if lo >= N:
            cq[128 * t:128 * (t + 1)] = np.nan
            continue
        codes, s_q = quantize_q_tile(Q[lo:hi])
        cq[128 * t:128 * (t + 1)] = float(F.f32(F.f32(s_q * scale) * F.f32(LOG2E)))
        qdec[lo - r0:hi - r0] = F.e4m3_decode(codes)
    want_c = F.f32(cq[:, None] * k_scale[None, :]).T        # [nblk, 256]
    assert np.array_equal(c[:, rows], want_c[:, rows]), "block scale c differs"
    # masking, running maximum and bytes, block by block
    kc = float(F.f32((56.0 if mode == "expcast" else 120.0 if mode == "shifted" else 0.0) + float(F.f32(beta))))
    m_prev = np.full(rows.size, -np.inf)
    n_exact = n_total = 0
    worst = 0.0
    rs_err = 0.0
    mid_diffs = 0
    for b in range(nblk):
        nvalid = min(kvb, N - b * kvb)
        Sb = S[b][rows]
        assert np.all(np.isneginf(Sb[:, nvalid:])), "padded keys not masked"
        assert np.all(np.isfinite(Sb[:, :nvalid]))
        m_new = np.maximum(m_prev, F.f32(c[b, rows] * np.max(Sb, axis=1)))
        assert np.array_equal(m[b, rows], m_new), f"running maximum differs in block {b}"
        m_prev = m_new
        if mode == "exp2":
            mid_diffs += exp2_bytes_within_midpoint_slack(P[b][rows], Sb, c[b, rows][:, None], -m_new[:, None])
        else:
            want = expcast_bytes(Sb, 8.0 * c[b, rows][:, None], F.f32(kc - 8.0 * m_new)[:, None], TOP[mode])
            nd = np.count_nonzero(P[b][rows] != want)
            assert nd == 0, f"{nd} probability bytes differ in block {b}"
        exact_rs = F.e4m3_decode(P[b][rows]).sum(axis=1)
        if mode == "shifted":
            # the products span 2^17 (bytes 2^-9 .. 2^8): the row-sum MFMA may
            # drop the low bits of small products next to a large one
            rs_err = max(rs_err, float(np.max(np.abs(rs[b, rows] - exact_rs) / exact_rs)))
            assert np.all(np.abs(rs[b, rows] - exact_rs) <= 2.0 ** -6 * exact_rs), f"row sums differ in block {b}"
        else:
            assert np.array_equal(rs[b, rows], exact_rs), f"row sums differ in block {b}"
        # scores against the exact dot products of the codes, within the
        # FP8 matrix instruction's accumulation window
        kb = kdec[b * kvb:b * kvb + nvalid]
        qr = qdec[rows]
        Sx = qr @ kb.T                                  # exact (multiples of 2^-18, below 2^25)
        bound = 2.0 ** -10 * (np.abs(qr) @ np.abs(kb).T) + 2.0 ** -22 * np.abs(Sx)
        err = np.abs(Sb[:, :nvalid] - Sx)
        assert np.all(err <= bound), f"scores outside the accumulation window in block {b}"
        n_exact += int(np.count_nonzero(Sb[:, :nvalid] == F.f32(Sx)))
        n_total += Sx.size
        worst = max(worst, float(np.max(err / np.maximum(bound, 1e-300))))
    log(f"  {w.name} N={N} h{h} group {group} {mode}: {nblk} blocks; scores equal to fp32(exact) "
        f"{n_exact}/{n_total}, worst error {worst:.3f} of the window bound"
        + (f"; {mid_diffs} exp2 bytes one code off at a midpoint" if mode == "exp2" else "")
        + (f"; row sums within {rs_err:.2e} relative" if mode == "shifted" else ""))


CASES = [
    ("tiny", 2, None, "expcast", (0, 1, 3)),
    ("tiny", 2, None, "exp2", (0, 3)),
    ("tiny", 2, None, "shifted", (0, 3)),
    ("tiny", 1, 1000, "expcast", (3,)),           # ragged: 1000 rows, 16 blocks with a partial tail
    ("mid", 1, None, "expcast", (0, 31, 63)),
    ("mid", 1, None, "exp2", (17,)),
    ("mid", 1, None, "shifted", (40,)),
    ("mid", 1, 5000, "expcast", (19,)),           # ragged tail block and last query group
    ("video", None, None, "expcast", (0, 295)),   # all 40 heads launched; the last head traced
    ("video", None, None, "exp2", (150,)),
    ("video", None, None, "shifted", (295,)),
]


@pytest.mark.parametrize("name,H,N,mode,groups", CASES)
def test_fused_kernel_trace_bit_exact(name, H, N, mode, groups):
    w = inputs.WORKLOADS[name]
    H = H or w.H
    N = N or w.N
    import dataclasses
    w = dataclasses.replace(w, H=H, N=N, k=min(w.k, N))
    host = inputs.gen_all(w)
    q, k, v, init = host
    dev = dict(Q=to_device_bf16(q), K=to_device_bf16(k), V=to_device_bf16(v), init=torch.from_numpy(init).cuda())
    beta = oracle.DEFAULT_BETA
    cfg = vb.make_config(w.B, H, N, w.d, w.kv_block, w.k, w.iters, True, vb.E4M3, True, 0.0, beta, MODES[mode])
    prep = vb.vsmooth_prepare(cfg, dev["K"], dev["V"], dev["init"])
    O_prod = vb.vc_attn_fwd(cfg, dev["Q"], prep)
    h = H - 1
    prep_o = oracle.prepare_head(oracle.bf16_to_f64(k[0, h]), oracle.bf16_to_f64(v[0, h]), init[0, h], w.k,
                                 w.iters, w.kv_block)
    for g in groups:
        O_tr, tr = vb.dbg_attn_trace(cfg, dev["Q"], prep, h, g)
        assert torch.equal(O_tr, O_prod), "the trace instantiation's O differs from the production kernel's"
        check_trace(w, host, prep_o, tr, h, g, mode, softmax_scale(w.d), beta)
        del tr
    torch.cuda.synchronize()


def test_trace_with_mxfp4_residuals_and_explicit_parameters():
    # the bytes do not depend on the residual format; an explicit softmax scale
    # and beta reach the FMA as given
    import dataclasses
    w = dataclasses.replace(inputs.WORKLOADS["tiny"], N=900, H=1)
    host = inputs.gen_all(w)
    q, k, v, init = host
    scale, beta = 0.07, 0.3
    cfg = vb.make_config(1, 1, 900, w.d, w.kv_block, w.k, w.iters, True, vb.MXFP4, True, scale, beta, vb.EXPCAST)
    prep = vb.vsmooth_prepare(cfg, to_device_bf16(k), to_device_bf16(v), torch.from_numpy(init).cuda())
    prep_o = oracle.prepare_head(oracle.bf16_to_f64(k[0, 0]), oracle.bf16_to_f64(v[0, 0]), init[0, 0], w.k,
                                 w.iters, w.kv_block, "mxfp4")
    O_tr, tr = vb.dbg_attn_trace(cfg, to_device_bf16(q), prep, 0, 2)
    check_trace(w, host, prep_o, tr, 0, 2, "expcast", float(F.f32(scale)), beta)


@pytest.mark.parametrize("fmt,name,N,mode,group", [("nvfp4", "tiny", 900, "expcast", 2),
                                                   ("nvfp4", "mid", 5000, "exp2", 19),
                                                   ("nvfp4", "mid", None, "shifted", 40),
                                                   ("mxfp8", "tiny", 900, "expcast", 2),
                                                   ("mxfp8", "mid", 5000, "shifted", 19)])
def test_trace_with_block_scaled_residuals(fmt, name, N, mode, group):
    # the two-phase block step of the NVFP4-style residuals, and the MXFP8
    # step with its two-deep operand ring, form the same scores, maxima,
    # bytes and row sums
    import dataclasses
    w = inputs.WORKLOADS[name]
    N = N or w.N
    w = dataclasses.replace(w, N=N, H=1, k=min(w.k, N))
    host = inputs.gen_all(w)
    q, k, v, init = host
    beta = oracle.DEFAULT_BETA
    vf = {"nvfp4": vb.NVFP4, "mxfp8": vb.MXFP8}[fmt]
    cfg = vb.make_config(1, 1, N, w.d, w.kv_block, w.k, w.iters, True, vf, True, 0.0, beta, MODES[mode])
    prep = vb.vsmooth_prepare(cfg, to_device_bf16(k), to_device_bf16(v), torch.from_numpy(init).cuda())
    O_prod = vb.vc_attn_fwd(cfg, to_device_bf16(q), prep)
    prep_o = oracle.prepare_head(oracle.bf16_to_f64(k[0, 0]), oracle.bf16_to_f64(v[0, 0]), init[0, 0], w.k,
                                 w.iters, w.kv_block, fmt)
    O_tr, tr = vb.dbg_attn_trace(cfg, to_device_bf16(q), prep, 0, group)
    assert torch.equal(O_tr, O_prod), "the trace instantiation's O differs from the production kernel's"
    check_trace(w, host, prep_o, tr, 0, group, mode, softmax_scale(w.d), beta)


# ------------------------------------------------------------------ mean restoration, closed form
def vsmooth_closed_form_inputs(N, d, kvb, seed=5):
    """Q, K with integer log2 scores in [-3, 3] (closed_forms.integer_score_qkv)
    and V = block mean + residual with every part exact: means are multiples
    of 32 up to 768 (natural-order blocks, so the identity permutation makes
    them the block means), residuals come in +-pairs (each block's residuals
    sum to zero) of multiples of 32 up to 448, with 448 reached in every
    channel (s_v = 1)."""
    from closed_forms import integer_score_qkv
    Q, K, _ = integer_score_qkv(N, d, kvb)
    rng = np.random.default_rng(seed)
    nblk = (N + kvb - 1) // kvb
    means = 32.0 * rng.integers(-24, 25, size=(nblk, d))
    r = np.zeros((N, d))
    half = 32.0 * rng.integers(-13, 14, size=(N // 2, d))
    r[0::2] = half
    r[1::2] = -half
    for c in range(d):
        r[2 * c, c], r[2 * c + 1, c] = 448.0, -448.0
    V = np.repeat(means, kvb, axis=0)[:N] + r
    return Q, K, V, means


@pytest.mark.parametrize("mode,d,kvb,fmt", [("expcast", 64, 64, "e4m3"), ("exp2", 128, 128, "e4m3"),
                                             ("shifted", 128, 64, "e4m3"), ("expcast", 128, 128, "e4m3"),
                                             ("expcast", 128, 128, "mxfp8"), ("shifted", 64, 64, "mxfp8")])
def test_mean_restoration_closed_form(mode, d, kvb, fmt):
    """V-Smooth on (identity permutation, so the blocks are natural order and
    their means are the constructed ones): every probability byte is exactly
    2^(t - m) (times 2^8 when range-shifted), every mean and row sum is exact
    in the bf16 hi + lo split the kernel restores the mean with, and every
    partial sum is exact in fp32.  O must then equal the base-2 softmax of the
    integer scores applied to V itself up to the final normalisation's
    roundings (4 * 2^-24 relative), which pins the mean restoration: the
    right block's mean, the rescaling of the mean term, and its scale.  The
    residuals (multiples of 32 up to 448) are exact in E4M3 under a unit
    scale and in MXFP8 under any power-of-two group scale."""
    from closed_forms import base2_softmax, unit_log2_scale
    N = 300
    Q, K, V, means = vsmooth_closed_form_inputs(N, d, kvb)
    assert np.all(np.abs(V) <= 1216) and np.all(V % 32 == 0)          # exact in bf16
    dv = {n: torch.from_numpy(x).to(torch.bfloat16).reshape(1, 1, N, d).cuda() for n, x in
          (("Q", Q), ("K", K), ("V", V))}
    vf = {"e4m3": vb.E4M3, "mxfp8": vb.MXFP8}[fmt]
    cfg = vb.make_config(1, 1, N, d, kvb, 1, 1, True, vf, True, unit_log2_scale(), -0.25, MODES[mode])
    ident = torch.arange(N, dtype=torch.int32, device="cuda").reshape(1, 1, N)
    prep = vb.vsmooth_prepare_warm(cfg, dv["K"], dv["V"], perm_in=ident)
    assert np.array_equal(prep.v_mean[0, 0].cpu().numpy(), means.astype(np.float32))
    assert torch.all(prep.k_scale == 1.0)
    if fmt == "e4m3":
        assert torch.all(prep.v_scale == 1.0)
    O = vb.vc_attn_fwd(cfg, dv["Q"], prep)[0, 0].cpu().numpy().astype(np.float64)
    S = Q @ K.T
    want = base2_softmax(S, V)
    err = np.abs(O - want)
    log(f"  {fmt} {mode} d {d} kv_block {kvb}: max rel err {np.max(err / np.maximum(np.abs(want), 1e-30)):.2e}, "
        f"mean term share {np.max(np.abs(base2_softmax(S, np.repeat(means, kvb, 0)[:N]))) / np.max(np.abs(want)):.2f}")
    assert np.all(err <= 4.0 * 2.0 ** -24 * np.abs(want) + 1e-30)
    # with the means dropped (a kernel that forgot to restore them) the output
    # would be far off: the closed form is sensitive to the mean term
    assert np.max(np.abs(base2_softmax(S, V - np.repeat(means, kvb, 0)[:N]) - want)) > 1.0
