"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/vcattn.h, and rejects invalid arguments with the right
status before anything is launched (all calls below fail validation, so no
device work is ever enqueued)."""
import ctypes
import os
import re

import pytest

from bit_attention_video_amd import binding as vb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vcattn.h")

VC_OK, VC_ERR_INVALID_ARG, VC_ERR_UNSUPPORTED, VC_ERR_WORKSPACE = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("vc", "vsmooth"))))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vb.LIB_PATH):
        pytest.skip("libvcattn.so not built")
    return vb.lib()


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for want in ("vsmooth_prepare", "vc_attn_fwd", "vc_attention", "vc_prepare_workspace_bytes",
                 "vc_attention_workspace_bytes", "vc_status_str", "vc_last_error", "vc_dbg_expcast",
                 "vc_dbg_kmeans_assign", "vc_dbg_sort", "vc_mfma_loop", "vc_dbg_exp2cast",
                 "vsmooth_prepare_warm", "vc_dbg_attn_trace", "vc_dbg_init_tokens", "vc_workspace_bytes",
                 "vc_last_hip_error"):
        assert want in names, want


def test_workspace_bytes_covers_every_call_and_error_aliases(lib):
    c = cfg()
    L = vb.lib()
    L.vc_workspace_bytes.restype = ctypes.c_size_t
    L.vc_attention_workspace_bytes.restype = ctypes.c_size_t
    L.vc_prepare_workspace_bytes.restype = ctypes.c_size_t
    w = L.vc_workspace_bytes(ctypes.byref(c))
    assert w == L.vc_attention_workspace_bytes(ctypes.byref(c)) >= L.vc_prepare_workspace_bytes(ctypes.byref(c)) > 0
    assert L.vc_workspace_bytes(ctypes.byref(cfg(d=96))) == 0
    L.vc_last_error.restype = ctypes.c_char_p
    L.vc_last_hip_error.restype = ctypes.c_char_p
    assert L.vc_last_hip_error() == L.vc_last_error()


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(vb.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} not exported"


def cfg(**kw):
    raw = {f: kw.pop(f) for f in ("cluster_order", "balanced") if f in kw and kw[f] not in (True, False)}
    base = dict(B=1, H=2, N=1000, d=64, kv_block=64, n_clusters=16, iters=3)
    base.update(kw)
    c = vb.make_config(**base)
    for f, x in raw.items():
        setattr(c, f, x)
    return c


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), VC_ERR_UNSUPPORTED),
    (dict(kv_block=32), VC_ERR_UNSUPPORTED),
    (dict(N=0), VC_ERR_INVALID_ARG),
    (dict(n_clusters=0), VC_ERR_INVALID_ARG),
    (dict(n_clusters=1001), VC_ERR_INVALID_ARG),      # k > N
    (dict(n_clusters=5000, N=10000), VC_ERR_INVALID_ARG),
    (dict(iters=0), VC_ERR_INVALID_ARG),
    (dict(beta=0.5), VC_ERR_INVALID_ARG),
    (dict(beta=-0.6), VC_ERR_INVALID_ARG),
    (dict(v_format=4), VC_ERR_UNSUPPORTED),
    (dict(p_mode=3), VC_ERR_UNSUPPORTED),
    (dict(p_mode=-1), VC_ERR_UNSUPPORTED),
    (dict(cluster_order=2), VC_ERR_UNSUPPORTED),
    (dict(N=(1 << 24), d=128, n_clusters=16), VC_ERR_UNSUPPORTED),     # 2^31 bytes of blocked keys per head
    (dict(balanced=True, n_clusters=15), VC_ERR_INVALID_ARG),           # n_clusters != ceil(N / kv_block) = 16
    (dict(balanced=2), VC_ERR_INVALID_ARG),
    (dict(balanced=True, n_clusters=16, vsmooth=False), VC_ERR_INVALID_ARG),
])
def test_invalid_config_rejected_before_launch(lib, kw, status):
    c = cfg(**kw)
    P = ctypes.c_void_p(16)      # never dereferenced: validation fails first
    r = lib.vsmooth_prepare(ctypes.byref(c), P, P, P, P, P, P, P, P, P, None, P, 1 << 40, None)
    assert r == status, (r, lib.vc_last_error())
    assert lib.vc_last_error().decode()
    assert lib.vc_prepare_workspace_bytes(ctypes.byref(c)) == 0


def test_null_and_misaligned_pointers_rejected(lib):
    c = cfg()
    P = ctypes.c_void_p(256)
    assert lib.vsmooth_prepare(ctypes.byref(c), None, P, P, P, P, P, P, P, P, None, P, 1 << 40, None) == VC_ERR_INVALID_ARG
    bad = ctypes.c_void_p(258)
    assert lib.vc_attn_fwd(ctypes.byref(c), bad, P, P, P, P, P, P, None) == VC_ERR_INVALID_ARG
    assert "aligned" in lib.vc_last_error().decode()
    assert lib.vc_attention(ctypes.byref(c), P, P, P, None, None, P, 1 << 40, None) == VC_ERR_INVALID_ARG  # no O
    assert lib.vc_dbg_expcast(None, None, None, -1, None, None) == VC_ERR_INVALID_ARG
    assert lib.vc_mfma_loop(0, 10, P, None) == VC_ERR_INVALID_ARG
    assert lib.vc_mfma_loop(4, 10, None, None) == VC_ERR_INVALID_ARG


def test_workspace_too_small_rejected(lib):
    c = cfg()
    need = lib.vc_prepare_workspace_bytes(ctypes.byref(c))
    assert need > 0 and lib.vc_attention_workspace_bytes(ctypes.byref(c)) > need
    P = ctypes.c_void_p(256)
    r = lib.vsmooth_prepare(ctypes.byref(c), P, P, P, P, P, P, P, P, P, None, P, need - 1, None)
    assert r == VC_ERR_WORKSPACE
    assert lib.vc_status_str(r).decode() == "workspace too small"


def test_workspace_sizes_grow_with_problem(lib):
    small = lib.vc_attention_workspace_bytes(ctypes.byref(cfg()))
    big = lib.vc_attention_workspace_bytes(ctypes.byref(cfg(N=4000)))
    assert big > 3 * small


def test_warm_prepare_takes_at_most_one_start(lib):
    # (no start at all is a seeded cold start; it passes validation and is
    # therefore not called here with placeholder pointers)
    c = cfg()
    P = ctypes.c_void_p(256)
    args = lambda init, cent, perm_in: (ctypes.byref(c), P, P, init, cent, perm_in, None, P, P, P, P, P, P, None, P,
                                         1 << 40, None)
    assert lib.vsmooth_prepare_warm(*args(P, P, None)) == VC_ERR_INVALID_ARG
    assert "at most one" in lib.vc_last_error().decode()
    assert lib.vsmooth_prepare_warm(*args(None, P, P)) == VC_ERR_INVALID_ARG
    assert lib.vsmooth_prepare_warm(*args(P, P, P)) == VC_ERR_INVALID_ARG
    c.vsmooth = 0
    assert lib.vsmooth_prepare_warm(*args(P, None, None)) == VC_ERR_INVALID_ARG


def test_trace_and_init_entry_points_validate(lib):
    c = cfg()
    P = ctypes.c_void_p(256)
    tr = lambda cc, bh, g: lib.vc_dbg_attn_trace(ctypes.byref(cc), P, P, P, P, P, P, P, bh, g, P, P, P, P, P, None)
    assert tr(c, 0, 0) == VC_ERR_UNSUPPORTED            # bf16 output: the trace needs fp32 output
    c.out_fp32 = 1
    assert tr(c, 2, 0) == VC_ERR_INVALID_ARG            # bh = B*H is out of range
    assert tr(c, 0, 4) == VC_ERR_INVALID_ARG            # N = 1000 has 4 groups of 256 rows
    assert tr(c, -1, 0) == VC_ERR_INVALID_ARG
    assert lib.vc_dbg_init_tokens(ctypes.byref(cfg()), None, None) == VC_ERR_INVALID_ARG
    assert lib.vc_dbg_init_tokens(ctypes.byref(cfg(n_clusters=0)), P, None) == VC_ERR_INVALID_ARG


def test_seed_and_balanced_fields():
    # the seed follows the 32-bit fields (8-byte aligned), then the balanced switch
    assert vb.VcConfig.seed.offset == 56 and vb.VcConfig.balanced.offset == 64
    assert ctypes.sizeof(vb.VcConfig) == 72
    c = vb.make_config(1, 1, 10, 64, 64, seed=-1)
    assert c.seed == 2 ** 64 - 1
