"""Thin Python binding over libvcattn.so (ctypes).

Argument marshalling only: torch provides device memory and the current HIP
stream; every step of the forward pass runs in the library's HIP kernels.
There is no fallback: a missing or unloadable library raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# VCATTN_LIBRARY selects another build of the library (same ABI)
LIB_PATH = os.environ.get("VCATTN_LIBRARY") or os.path.join(_HERE, "libvcattn.so")

# ExpCast offset default: fp32(8/ln2 - 12), the value that centres
# 8z + 56 + beta on the exact E4M3 code of 2^z over fractional z.
DEFAULT_BETA = 8.0 / math.log(2.0) - 12.0

E4M3, MXFP4, MXFP8, NVFP4 = 0, 1, 2, 3    # residual formats (NVFP4: 16-token E4M3 scales, emulated)
# p_mode: ExpCast-FP8 bytes; exp2 then E4M3 cast (ExpCast off); ExpCast moved up by 64 codes
EXPCAST, EXP2_CAST, EXPCAST_SHIFTED = 0, 1, 2


class VcConfig(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("kv_block", ctypes.c_int32), ("n_clusters", ctypes.c_int32), ("iters", ctypes.c_int32),
                ("vsmooth", ctypes.c_int32), ("v_format", ctypes.c_int32), ("out_fp32", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("beta", ctypes.c_float), ("p_mode", ctypes.c_int32),
                ("cluster_order", ctypes.c_int32), ("seed", ctypes.c_uint64), ("balanced", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libvcattn.so not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        cfgp = ctypes.POINTER(VcConfig)
        L.vc_prepare_workspace_bytes.argtypes = [cfgp]
        L.vc_prepare_workspace_bytes.restype = ctypes.c_size_t
        L.vc_attention_workspace_bytes.argtypes = [cfgp]
        L.vc_attention_workspace_bytes.restype = ctypes.c_size_t
        L.vsmooth_prepare.argtypes = [cfgp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.vsmooth_prepare.restype = ctypes.c_int
        L.vsmooth_prepare_warm.argtypes = [cfgp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           ctypes.c_size_t, _P]
        L.vsmooth_prepare_warm.restype = ctypes.c_int
        L.vc_attn_fwd.argtypes = [cfgp, _P, _P, _P, _P, _P, _P, _P, _P]
        L.vc_attn_fwd.restype = ctypes.c_int
        L.vc_attention.argtypes = [cfgp, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.vc_attention.restype = ctypes.c_int
        L.vc_attention_noalloc.argtypes = [cfgp, _P, _P, _P, _P, _P, _P]
        L.vc_attention_noalloc.restype = ctypes.c_int
        L.vc_noalloc_scratch_bytes.argtypes = []
        L.vc_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.vc_status_str.argtypes = [ctypes.c_int]
        L.vc_status_str.restype = ctypes.c_char_p
        L.vc_last_error.argtypes = []
        L.vc_last_error.restype = ctypes.c_char_p
        L.vc_dbg_expcast.argtypes = [_P, _P, _P, ctypes.c_int64, _P, _P]
        L.vc_dbg_expcast.restype = ctypes.c_int
        L.vc_dbg_exp2cast.argtypes = [_P, _P, _P, ctypes.c_int64, _P, _P]
        L.vc_dbg_exp2cast.restype = ctypes.c_int
        L.vc_dbg_kmeans_assign.argtypes = [cfgp, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.vc_dbg_kmeans_assign.restype = ctypes.c_int
        L.vc_dbg_sort.argtypes = [cfgp, _P, _P, _P, ctypes.c_size_t, _P]
        L.vc_dbg_sort.restype = ctypes.c_int
        L.vc_dbg_attn_trace.argtypes = [cfgp, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                        _P, _P, _P, _P]
        L.vc_dbg_attn_trace.restype = ctypes.c_int
        L.vc_dbg_init_tokens.argtypes = [cfgp, _P, _P]
        L.vc_dbg_init_tokens.restype = ctypes.c_int
        L.vc_mfma_loop.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P]
        L.vc_mfma_loop.restype = ctypes.c_int
        _lib = L
    return _lib


class VcError(RuntimeError):
    def __init__(self, status: int, what: str):
        L = lib()
        super().__init__(f"{what}: {L.vc_status_str(status).decode()} ({status}): {L.vc_last_error().decode()}")
        self.status = status


def _check(status: int, what: str):
    if status != 0:
        raise VcError(status, what)


def make_config(B: int, H: int, N: int, d: int, kv_block: int, n_clusters: int = 1, iters: int = 1,
                vsmooth: bool = True, v_format: int = E4M3, out_fp32: bool = False,
                softmax_scale: float = 0.0, beta: float = DEFAULT_BETA, p_mode: int = EXPCAST,
                cluster_order: bool = False, seed: int = 0, balanced: bool = False) -> VcConfig:
    """balanced: clusters sized to the blocks (n_clusters must then be
    ceil(N / kv_block); balanced_clusters() gives it)."""
    return VcConfig(B, H, N, d, kv_block, n_clusters, iters, int(bool(vsmooth)), int(v_format),
                    int(bool(out_fp32)), softmax_scale, beta, int(p_mode), int(bool(cluster_order)),
                    int(seed) & (2 ** 64 - 1), int(bool(balanced)))


def balanced_clusters(N: int, kv_block: int) -> int:
    """The cluster count of the balanced blocking variant: one cluster per block."""
    return (N + kv_block - 1) // kv_block


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t: torch.Tensor, dtype, shape, name: str):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_bytes(cfg: VcConfig, attention: bool = False) -> int:
    f = lib().vc_attention_workspace_bytes if attention else lib().vc_prepare_workspace_bytes
    n = f(ctypes.byref(cfg))
    if n == 0:
        raise VcError(-1, "workspace_bytes")
    return n


def _nblk(cfg):
    return (cfg.N + cfg.kv_block - 1) // cfg.kv_block


@dataclasses.dataclass
class Prepared:
    """Blocked K/V as written by vsmooth_prepare (layouts in include/vcattn.h)."""
    Kq: torch.Tensor
    k_scale: torch.Tensor
    Vres: torch.Tensor
    v_scale: torch.Tensor
    v_mean: torch.Tensor
    perm: torch.Tensor
    labels: torch.Tensor | None


def _prepared_layout(cfg: VcConfig) -> dict:
    """(dtype, shape) of every Prepared field for this configuration."""
    B, H, N, d, kvb = cfg.B, cfg.H, cfg.N, cfg.d, cfg.kv_block
    nblk = _nblk(cfg)
    Np = nblk * kvb
    return dict(
        Kq=(torch.uint8, (B, H, Np, d)),
        k_scale=(torch.float32, (B, H, nblk)),
        Vres=(torch.uint8, (B, H, nblk, 2, kvb // 64, d, 64) if cfg.v_format == NVFP4 else
              (B, H, Np // 64, d, 32 if cfg.v_format == MXFP4 else 64)),
        v_scale=(torch.float32, (B, H, d)) if cfg.v_format == E4M3 else (torch.uint8, (B, H, Np // 32, d)),
        v_mean=(torch.float32, (B, H, nblk, d)),
        perm=(torch.int32, (B, H, N)),
        labels=(torch.int32, (B, H, N)))


def alloc_prepared(cfg: VcConfig, device="cuda", with_labels: bool = True) -> Prepared:
    lay = _prepared_layout(cfg)
    t = {k: torch.empty(shape, dtype=dt, device=device) for k, (dt, shape) in lay.items()
         if k != "labels" or with_labels}
    return Prepared(labels=t.pop("labels", None), **t)


def _check_prepared(cfg: VcConfig, prep: Prepared):
    """The library cannot see buffer sizes: every field must match cfg."""
    for k, (dt, shape) in _prepared_layout(cfg).items():
        t = getattr(prep, k)
        if t is not None or k != "labels":
            _need(t, dt, shape, f"prep.{k}")


def _workspace(ws: torch.Tensor | None, nbytes: int, device) -> torch.Tensor:
    """The caller's workspace, checked; a new one only when none is given."""
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    _need(ws, torch.uint8, (ws.numel(),), "ws")
    if ws.numel() < nbytes:
        raise ValueError(f"ws holds {ws.numel()} bytes; this configuration needs {nbytes}")
    return ws


def vsmooth_prepare(cfg: VcConfig, K: torch.Tensor, V: torch.Tensor, init_idx: torch.Tensor | None,
                    out: Prepared | None = None, ws: torch.Tensor | None = None,
                    with_labels: bool = True) -> Prepared:
    shp = (cfg.B, cfg.H, cfg.N, cfg.d)
    _need(K, torch.bfloat16, shp, "K")
    _need(V, torch.bfloat16, shp, "V")
    if cfg.vsmooth and init_idx is not None:
        _need(init_idx, torch.int32, (cfg.B, cfg.H, cfg.n_clusters), "init_idx")
    if out is None:
        out = alloc_prepared(cfg, K.device, with_labels)
    else:
        _check_prepared(cfg, out)
    ws = _workspace(ws, workspace_bytes(cfg), K.device)
    _check(lib().vsmooth_prepare(ctypes.byref(cfg), _ptr(K), _ptr(V), _ptr(init_idx) if cfg.vsmooth else None,
                                 _ptr(out.Kq), _ptr(out.k_scale), _ptr(out.Vres), _ptr(out.v_scale),
                                 _ptr(out.v_mean), _ptr(out.perm), _ptr(out.labels), _ptr(ws), ws.numel(),
                                 _stream()), "vsmooth_prepare")
    return out


def vsmooth_prepare_warm(cfg: VcConfig, K: torch.Tensor, V: torch.Tensor, *,
                         init_idx: torch.Tensor | None = None, init_centroids: torch.Tensor | None = None,
                         perm_in: torch.Tensor | None = None, centroids_out: torch.Tensor | None = None,
                         out: Prepared | None = None, ws: torch.Tensor | None = None,
                         with_labels: bool = True) -> Prepared:
    """vsmooth_prepare carried across calls (include/vcattn.h): at most one of
    init_idx (cold start), init_centroids (warm start) or perm_in (reuse);
    none is a cold start from cfg.seed."""
    shp = (cfg.B, cfg.H, cfg.N, cfg.d)
    _need(K, torch.bfloat16, shp, "K")
    _need(V, torch.bfloat16, shp, "V")
    cshape = (cfg.B, cfg.H, cfg.n_clusters, cfg.d)
    if init_idx is not None:
        _need(init_idx, torch.int32, (cfg.B, cfg.H, cfg.n_clusters), "init_idx")
    if init_centroids is not None:
        _need(init_centroids, torch.float32, cshape, "init_centroids")
    if perm_in is not None:
        _need(perm_in, torch.int32, (cfg.B, cfg.H, cfg.N), "perm_in")
    if centroids_out is not None:
        _need(centroids_out, torch.float32, cshape, "centroids_out")
    if out is None:
        out = alloc_prepared(cfg, K.device, with_labels)
    else:
        _check_prepared(cfg, out)
    ws = _workspace(ws, workspace_bytes(cfg), K.device)
    _check(lib().vsmooth_prepare_warm(ctypes.byref(cfg), _ptr(K), _ptr(V), _ptr(init_idx), _ptr(init_centroids),
                                      _ptr(perm_in), _ptr(centroids_out), _ptr(out.Kq), _ptr(out.k_scale),
                                      _ptr(out.Vres), _ptr(out.v_scale), _ptr(out.v_mean), _ptr(out.perm),
                                      _ptr(out.labels), _ptr(ws), ws.numel(), _stream()), "vsmooth_prepare_warm")
    return out


def _out_dtype(cfg: VcConfig):
    return torch.float32 if cfg.out_fp32 else torch.bfloat16


def alloc_out(cfg: VcConfig, device="cuda") -> torch.Tensor:
    return torch.empty((cfg.B, cfg.H, cfg.N, cfg.d), device=device, dtype=_out_dtype(cfg))


def _output(cfg: VcConfig, out: torch.Tensor | None, device) -> torch.Tensor:
    if out is None:
        return alloc_out(cfg, device)
    _need(out, _out_dtype(cfg), (cfg.B, cfg.H, cfg.N, cfg.d), "out")
    return out


def vc_attn_fwd(cfg: VcConfig, Q: torch.Tensor, prep: Prepared, out: torch.Tensor | None = None) -> torch.Tensor:
    _need(Q, torch.bfloat16, (cfg.B, cfg.H, cfg.N, cfg.d), "Q")
    _check_prepared(cfg, prep)
    out = _output(cfg, out, Q.device)
    _check(lib().vc_attn_fwd(ctypes.byref(cfg), _ptr(Q), _ptr(prep.Kq), _ptr(prep.k_scale), _ptr(prep.Vres),
                             _ptr(prep.v_scale), _ptr(prep.v_mean), _ptr(out), _stream()), "vc_attn_fwd")
    return out


def vc_attention(cfg: VcConfig, Q, K, V, init_idx=None, out=None, ws=None) -> torch.Tensor:
    """(Q, K, V) -> O with the clustering inside the call; init_idx None draws
    the k-means start from cfg.seed."""
    shp = (cfg.B, cfg.H, cfg.N, cfg.d)
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, torch.bfloat16, shp, n)
    if cfg.vsmooth and init_idx is not None:
        _need(init_idx, torch.int32, (cfg.B, cfg.H, cfg.n_clusters), "init_idx")
    out = _output(cfg, out, Q.device)
    ws = _workspace(ws, workspace_bytes(cfg, attention=True), Q.device)
    _check(lib().vc_attention(ctypes.byref(cfg), _ptr(Q), _ptr(K), _ptr(V),
                              _ptr(init_idx) if cfg.vsmooth else None, _ptr(out), _ptr(ws), ws.numel(),
                              _stream()), "vc_attention")
    return out


def vc_attention_noalloc(cfg: VcConfig, Q, K, V, init_idx=None, out=None) -> torch.Tensor:
    """vc_attention with the library's static scratch in place of a workspace
    (include/vcattn.h): the library allocates nothing; pass `out` to keep the
    call free of allocations on this side too."""
    shp = (cfg.B, cfg.H, cfg.N, cfg.d)
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, torch.bfloat16, shp, n)
    if cfg.vsmooth and init_idx is not None:
        _need(init_idx, torch.int32, (cfg.B, cfg.H, cfg.n_clusters), "init_idx")
    out = _output(cfg, out, Q.device)
    _check(lib().vc_attention_noalloc(ctypes.byref(cfg), _ptr(Q), _ptr(K), _ptr(V),
                                      _ptr(init_idx) if cfg.vsmooth else None, _ptr(out), _stream()),
           "vc_attention_noalloc")
    return out


def noalloc_scratch_bytes() -> int:
    return int(lib().vc_noalloc_scratch_bytes())


TRACE_ROWS = 256     # query rows of one attention workgroup (one traced group)


def dbg_attn_trace(cfg: VcConfig, Q: torch.Tensor, prep: Prepared, bh: int, q_group: int,
                   out: torch.Tensor | None = None) -> tuple[torch.Tensor, dict]:
    """vc_attn_fwd through the trace instantiation (include/vcattn.h): returns
    O and the traced workgroup's per-block records S, P, m, c, rowsum."""
    _need(Q, torch.bfloat16, (cfg.B, cfg.H, cfg.N, cfg.d), "Q")
    _check_prepared(cfg, prep)
    out = _output(cfg, out, Q.device)
    nblk, R, kvb = _nblk(cfg), TRACE_ROWS, cfg.kv_block
    tr = dict(S=torch.empty((nblk, R, kvb), dtype=torch.float32, device=Q.device),
              P=torch.empty((nblk, R, kvb), dtype=torch.uint8, device=Q.device),
              m=torch.empty((nblk, R), dtype=torch.float32, device=Q.device),
              c=torch.empty((nblk, R), dtype=torch.float32, device=Q.device),
              rowsum=torch.empty((nblk, R), dtype=torch.float32, device=Q.device))
    _check(lib().vc_dbg_attn_trace(ctypes.byref(cfg), _ptr(Q), _ptr(prep.Kq), _ptr(prep.k_scale), _ptr(prep.Vres),
                                   _ptr(prep.v_scale), _ptr(prep.v_mean), _ptr(out), int(bh), int(q_group),
                                   _ptr(tr["S"]), _ptr(tr["P"]), _ptr(tr["m"]), _ptr(tr["c"]), _ptr(tr["rowsum"]),
                                   _stream()), "vc_dbg_attn_trace")
    return out, tr


def dbg_expcast(S: torch.Tensor, A: torch.Tensor, B: torch.Tensor) -> torch.Tensor:
    for t, n in ((S, "S"), (A, "A"), (B, "B")):
        _need(t, torch.float32, S.shape, n)
    out = torch.empty(S.shape, dtype=torch.uint8, device=S.device)
    _check(lib().vc_dbg_expcast(_ptr(S), _ptr(A), _ptr(B), S.numel(), _ptr(out), _stream()), "vc_dbg_expcast")
    return out


def dbg_exp2cast(S: torch.Tensor, A: torch.Tensor, B: torch.Tensor) -> torch.Tensor:
    for t, n in ((S, "S"), (A, "A"), (B, "B")):
        _need(t, torch.float32, S.shape, n)
    out = torch.empty(S.shape, dtype=torch.uint8, device=S.device)
    _check(lib().vc_dbg_exp2cast(_ptr(S), _ptr(A), _ptr(B), S.numel(), _ptr(out), _stream()), "vc_dbg_exp2cast")
    return out


def dbg_kmeans_assign(cfg: VcConfig, V: torch.Tensor, C: torch.Tensor) -> torch.Tensor:
    _need(V, torch.bfloat16, (cfg.B, cfg.H, cfg.N, cfg.d), "V")
    _need(C, torch.float32, (cfg.B, cfg.H, cfg.n_clusters, cfg.d), "C")
    labels = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.int32, device=V.device)
    c2 = VcConfig.from_buffer_copy(cfg)
    c2.vsmooth = 1
    ws = torch.empty(workspace_bytes(c2), dtype=torch.uint8, device=V.device)
    _check(lib().vc_dbg_kmeans_assign(ctypes.byref(cfg), _ptr(V), _ptr(C), _ptr(labels), _ptr(ws), ws.numel(),
                                      _stream()), "vc_dbg_kmeans_assign")
    return labels


def dbg_init_tokens(cfg: VcConfig, device="cuda") -> torch.Tensor:
    """The k-means initial token indices drawn from cfg.seed, int32 [B,H,k]."""
    out = torch.empty((cfg.B, cfg.H, cfg.n_clusters), dtype=torch.int32, device=device)
    _check(lib().vc_dbg_init_tokens(ctypes.byref(cfg), _ptr(out), _stream()), "vc_dbg_init_tokens")
    return out


def dbg_sort(cfg: VcConfig, labels: torch.Tensor) -> torch.Tensor:
    _need(labels, torch.int32, (cfg.B, cfg.H, cfg.N), "labels")
    perm = torch.empty_like(labels)
    c2 = VcConfig.from_buffer_copy(cfg)
    c2.vsmooth = 1
    ws = torch.empty(workspace_bytes(c2), dtype=torch.uint8, device=labels.device)
    _check(lib().vc_dbg_sort(ctypes.byref(cfg), _ptr(labels), _ptr(perm), _ptr(ws), ws.numel(), _stream()),
           "vc_dbg_sort")
    return perm


MFMA_LOOP_THREADS = 512
MFMA_LOOP_FLOPS_PER_ITER_WAVE = 8 * 2 * 32 * 32 * 64


def mfma_loop(blocks: int, iters: int, out: torch.Tensor | None = None) -> tuple[torch.Tensor, float]:
    """Runs the FP8 MFMA loop kernel; returns (checksum buffer, flops launched)."""
    n = blocks * MFMA_LOOP_THREADS
    out = torch.empty(n, dtype=torch.float32, device="cuda") if out is None else out
    _need(out, torch.float32, (n,), "out")
    _check(lib().vc_mfma_loop(blocks, iters, _ptr(out), _stream()), "vc_mfma_loop")
    return out, float(blocks) * (MFMA_LOOP_THREADS // 64) * iters * MFMA_LOOP_FLOPS_PER_ITER_WAVE
