// Host side of libvcattn: argument validation, workspace layout and the launch
// sequence of the VC-Attention forward pass.  Every check runs before the
// first launch; the library allocates nothing and never synchronises.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/vcattn.h"
#include "vc_internal.hpp"

namespace {

thread_local std::string g_err;

vc_status fail(vc_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

vc_status hip_fail(hipError_t e, const char* where) {
  g_err = std::string(where) + ": " + hipGetErrorString(e);
  return VC_ERR_HIP;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

constexpr int kTraceRows = 256;   // query rows per attention workgroup (one traced group)

struct Dims {
  int B, H, N, d, kvb, k, kpad, iters, nblk, nstat, nsort, balanced;
  size_t BH;
};

vc_status validate(const vc_config* c, bool need_kmeans, Dims* out) {
  if (!c) return fail(VC_ERR_INVALID_ARG, "cfg is NULL");
  if (c->B < 1 || c->H < 1 || c->N < 1) return fail(VC_ERR_INVALID_ARG, "B, H and N must be >= 1");
  if (static_cast<int64_t>(c->B) * c->H > 65535) return fail(VC_ERR_UNSUPPORTED, "B*H must be <= 65535");
  if (c->N > (1 << 26)) return fail(VC_ERR_UNSUPPORTED, "N must be <= 2^26");
  if (c->d != 64 && c->d != 128) return fail(VC_ERR_UNSUPPORTED, "d must be 64 or 128");
  if (c->kv_block != 64 && c->kv_block != 128) return fail(VC_ERR_UNSUPPORTED, "kv_block must be 64 or 128");
  // the attention kernel addresses one head's blocked keys and residuals
  // through buffer descriptors: 32-bit sizes and offsets
  if ((static_cast<int64_t>(c->N) + c->kv_block - 1) / c->kv_block * c->kv_block * c->d > INT32_MAX)
    return fail(VC_ERR_UNSUPPORTED, "N * d must stay below 2^31 (one head's blocked keys)");
  if (c->vsmooth != 0 && c->vsmooth != 1) return fail(VC_ERR_INVALID_ARG, "vsmooth must be 0 or 1");
  if (c->v_format < 0 || c->v_format > 3)
    return fail(VC_ERR_UNSUPPORTED, "v_format must be 0 (E4M3), 1 (MXFP4), 2 (MXFP8) or 3 (NVFP4 style)");
  if (c->out_fp32 != 0 && c->out_fp32 != 1) return fail(VC_ERR_INVALID_ARG, "out_fp32 must be 0 or 1");
  if (!(std::isfinite(c->softmax_scale) && c->softmax_scale >= 0.0f))
    return fail(VC_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (!(c->beta >= -0.5f && c->beta <= 0.45f)) return fail(VC_ERR_INVALID_ARG, "beta must lie in [-0.5, 0.45]");
  if (c->p_mode < 0 || c->p_mode > 2)
    return fail(VC_ERR_UNSUPPORTED, "p_mode must be 0 (ExpCast), 1 (exp2 + cast) or 2 (range-shifted ExpCast)");
  if (c->cluster_order != 0 && c->cluster_order != 1)
    return fail(VC_ERR_UNSUPPORTED, "cluster_order must be 0 (label order) or 1 (principal-axis order)");
  if (c->balanced != 0 && c->balanced != 1) return fail(VC_ERR_INVALID_ARG, "balanced must be 0 or 1");
  if (need_kmeans) {
    if (c->n_clusters < 1 || c->n_clusters > c->N || c->n_clusters > vc::kMaxClusters)
      return fail(VC_ERR_INVALID_ARG, "n_clusters must lie in [1, min(N, 4096)]");
    if (c->iters < 1 || c->iters > 16) return fail(VC_ERR_INVALID_ARG, "iters must lie in [1, 16]");
    if (c->balanced && c->n_clusters != (c->N + c->kv_block - 1) / c->kv_block)
      return fail(VC_ERR_INVALID_ARG, "balanced clusters need n_clusters = ceil(N / kv_block)");
  }
  if (c->balanced && !c->vsmooth) return fail(VC_ERR_INVALID_ARG, "balanced clusters need vsmooth on");
  Dims& D = *out;
  D.B = c->B; D.H = c->H; D.N = c->N; D.d = c->d; D.kvb = c->kv_block;
  D.k = need_kmeans ? c->n_clusters : 1;
  D.kpad = (D.k + 31) / 32 * 32;
  D.iters = c->iters;
  D.nblk = (c->N + c->kv_block - 1) / c->kv_block;
  D.nstat = (c->N + 1023) / 1024;
  D.nsort = (c->N + vc::kSortChunk - 1) / vc::kSortChunk;
  D.BH = static_cast<size_t>(c->B) * c->H;
  D.balanced = c->balanced;
  return VC_OK;
}

// Carves 256-byte aligned sub-buffers out of a workspace (base == nullptr
// only measures).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + 255) & ~static_cast<size_t>(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

void carve_prep(Carver& cv, const Dims& D, vc::PrepArgs& a) {
  const size_t BH = D.BH;
  a.vamax = cv.take<uint32_t>(BH);
  a.sV = cv.take<float>(BH);
  a.kpart = cv.take<double>(BH * D.nstat * D.d);
  a.mu = cv.take<float>(BH * D.d);
  a.vramax = cv.take<uint32_t>(BH * D.d);
  a.Vq = cv.take<int8_t>(BH * D.N * D.d);
  a.C = cv.take<float>(BH * D.k * D.d);
  a.Cq = cv.take<int8_t>(BH * D.kpad * D.d);
  a.cn32 = cv.take<int32_t>(BH * D.kpad);
  a.labels = cv.take<int32_t>(BH * D.N);
  a.perm_tmp = cv.take<int32_t>(BH * D.N);
  a.hist = cv.take<int32_t>(BH * D.nsort * D.k);
  a.counts = cv.take<int32_t>(BH * D.k);
  a.starts = cv.take<int32_t>(BH * D.k);
  a.rank = cv.take<int32_t>(BH * D.k);
  a.Ctmp = cv.take<float>(BH * D.k * D.d);
  a.init = cv.take<int32_t>(BH * D.k);
  if (D.balanced) {
    a.prop = cv.take<int32_t>(BH * D.N);
    a.pdist = cv.take<int32_t>(BH * D.N);
    a.rem = cv.take<int32_t>(BH * D.k);
    for (int i = 0; i < 2; ++i) {
      a.alist[i] = cv.take<int32_t>(BH * D.N);
      a.acnt[i] = cv.take<int32_t>(BH);
    }
    a.ccnt = cv.take<int32_t>(BH * D.nsort);
  }
}

struct OutSizes {
  size_t kq, ks, vres, vsc_bytes, vmean, perm;
};

OutSizes out_sizes(const Dims& D, int v_format) {
  const size_t Np = static_cast<size_t>(D.nblk) * D.kvb;
  OutSizes s;
  s.kq = D.BH * Np * D.d;
  s.ks = D.BH * D.nblk;
  s.vres = D.BH * Np * D.d * (v_format == 3 ? 2 : 1) / (v_format == 1 ? 2 : 1);
  s.vsc_bytes = v_format == 0 ? D.BH * D.d * sizeof(float) : D.BH * (Np / 32) * D.d;
  s.vmean = D.BH * D.nblk * D.d;
  s.perm = D.BH * D.N;
  return s;
}

void fill_prep_args(const vc_config* c, const Dims& D, const void* K, const void* V, vc::PrepArgs& a) {
  a.B = D.B; a.H = D.H; a.N = D.N; a.d = D.d; a.kvb = D.kvb; a.k = D.k; a.kpad = D.kpad;
  a.iters = D.iters; a.vsmooth = c->vsmooth; a.v_format = c->v_format;
  a.nblk = D.nblk; a.nstat = D.nstat; a.nsort = D.nsort;
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
}

#define VC_TRY(expr, where)                    \
  do {                                         \
    hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

// Clustering starts from V[init] or from init_centroids; perm_in skips it.
// centroids_out receives the member means of the final clusters.
vc_status run_prepare(const vc_config* c, const Dims& D, vc::PrepArgs& a, const int32_t* init,
                      const vc::PrepOut& o, int32_t* user_labels, hipStream_t st,
                      const float* init_centroids = nullptr, const int32_t* perm_in = nullptr,
                      float* centroids_out = nullptr) {
  VC_TRY(vc::launch_fill(a.vamax, 0u, D.BH, st), "fill");
  VC_TRY(vc::launch_fill(a.vramax, 0u, D.BH * D.d, st), "fill");
  VC_TRY(vc::launch_stats(a, st), "stats");
  if (perm_in) {
    if (perm_in != o.perm)
      VC_TRY(hipMemcpyAsync(o.perm, perm_in, D.BH * D.N * sizeof(int32_t), hipMemcpyDeviceToDevice, st),
             "copy perm");
  } else if (c->vsmooth) {
    VC_TRY(vc::launch_quant_v_i8(a, st), "quant_v_i8");
    if (init_centroids)
      VC_TRY(hipMemcpyAsync(a.C, init_centroids, D.BH * D.k * D.d * sizeof(float), hipMemcpyDeviceToDevice, st),
             "copy centroids");
    else {
      if (!init) {
        VC_TRY(vc::launch_init_seeded(a, c->seed, a.init, st), "init_seeded");
        init = a.init;
      }
      VC_TRY(vc::launch_init_centroids(a, init, st), "init_centroids");
    }
    for (int it = 0; it < D.iters; ++it) {
      const bool last = it + 1 == D.iters;
      int32_t* lab = (last && user_labels) ? user_labels : a.labels;
      if (last && c->cluster_order) VC_TRY(vc::launch_cluster_order(a, st), "cluster_order");
      if (c->balanced) VC_TRY(vc::launch_bal_assign(a, lab, st), "kmeans_assign (balanced)");
      else VC_TRY(vc::launch_assign(a, lab, st), "kmeans_assign");
      if (!last) {
        VC_TRY(vc::launch_sort(a, lab, a.perm_tmp, st), "sort");
        VC_TRY(vc::launch_update(a, a.perm_tmp, st), "kmeans_update");
      } else {
        VC_TRY(vc::launch_sort(a, lab, o.perm, st), "sort");
      }
    }
    if (centroids_out) {
      VC_TRY(vc::launch_update(a, o.perm, st), "kmeans_update");
      VC_TRY(hipMemcpyAsync(centroids_out, a.C, D.BH * D.k * D.d * sizeof(float), hipMemcpyDeviceToDevice, st),
             "copy centroids");
    }
  } else {
    VC_TRY(vc::launch_iota(o.perm, D.N, D.BH * D.N, st), "iota");
  }
  VC_TRY(vc::launch_vres_ksmooth(a, o.perm, o, st), "vres_ksmooth");
  return VC_OK;
}

void fill_attn_args(const vc_config* c, const Dims& D, vc::AttnArgs& a) {
  a.B = D.B; a.H = D.H; a.N = D.N; a.d = D.d; a.kvb = D.kvb; a.nblk = D.nblk;
  a.v_format = c->v_format; a.out_fp32 = c->out_fp32;
  a.scale = c->softmax_scale == 0.0f ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(D.d)))
                                     : c->softmax_scale;
  // ExpCast's addend: 56 + beta puts p = 1 at E4M3 byte 56 (1.0); the
  // range-shifted mode adds 64 codes (p = 1 at byte 120 = 2^8), so the bytes
  // stay normal E4M3 down to p = 2^-14 (the common factor 2^8 cancels in O)
  a.kc = (c->p_mode == 2 ? 120.0f : 56.0f) + c->beta;
  a.pm = c->p_mode == 1 ? 1 : 0;
}

}  // namespace

extern "C" {

const char* vc_status_str(vc_status s) {
  switch (s) {
    case VC_OK: return "ok";
    case VC_ERR_INVALID_ARG: return "invalid argument";
    case VC_ERR_UNSUPPORTED: return "unsupported configuration";
    case VC_ERR_WORKSPACE: return "workspace too small";
    case VC_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* vc_last_error(void) { return g_err.c_str(); }
const char* vc_last_hip_error(void) { return g_err.c_str(); }

size_t vc_prepare_workspace_bytes(const vc_config* cfg) {
  Dims D;
  if (validate(cfg, cfg && cfg->vsmooth, &D) != VC_OK) return 0;
  Carver cv(nullptr);
  vc::PrepArgs a{};
  carve_prep(cv, D, a);
  return cv.off + 256;
}

size_t vc_attention_workspace_bytes(const vc_config* cfg) {
  Dims D;
  if (validate(cfg, cfg && cfg->vsmooth, &D) != VC_OK) return 0;
  Carver cv(nullptr);
  vc::PrepArgs a{};
  carve_prep(cv, D, a);
  const OutSizes s = out_sizes(D, cfg->v_format);
  cv.take<uint8_t>(s.kq);
  cv.take<float>(s.ks);
  cv.take<uint8_t>(s.vres);
  cv.take<uint8_t>(s.vsc_bytes);
  cv.take<float>(s.vmean);
  cv.take<int32_t>(s.perm);
  return cv.off + 256;
}

size_t vc_workspace_bytes(const vc_config* cfg) { return vc_attention_workspace_bytes(cfg); }

vc_status vsmooth_prepare(const vc_config* cfg, const void* K, const void* V, const int32_t* init_idx,
                          uint8_t* Kq, float* k_scale, uint8_t* Vres, void* v_scale, float* v_mean,
                          int32_t* perm, int32_t* labels, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  Dims D;
  if (vc_status s = validate(cfg, cfg && cfg->vsmooth, &D)) return s;
  if (!K || !V || !Kq || !k_scale || !Vres || !v_scale || !v_mean || !perm || !ws)
    return fail(VC_ERR_INVALID_ARG, "required pointer is NULL");
  if (misaligned(K) || misaligned(V) || misaligned(Kq) || misaligned(Vres) || misaligned(v_scale) ||
      misaligned(v_mean) || misaligned(ws))
    return fail(VC_ERR_INVALID_ARG, "tensors and workspace must be 16-byte aligned");
  if (ws_bytes < vc_prepare_workspace_bytes(cfg)) return fail(VC_ERR_WORKSPACE, "workspace too small");
  vc::PrepArgs a{};
  fill_prep_args(cfg, D, K, V, a);
  Carver cv(reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~static_cast<uintptr_t>(255)));
  carve_prep(cv, D, a);
  vc::PrepOut o{Kq, k_scale, Vres, v_scale, v_mean, perm};
  return run_prepare(cfg, D, a, init_idx, o, labels, stream);
}

vc_status vsmooth_prepare_warm(const vc_config* cfg, const void* K, const void* V, const int32_t* init_idx,
                               const float* init_centroids, const int32_t* perm_in, float* centroids_out,
                               uint8_t* Kq, float* k_scale, uint8_t* Vres, void* v_scale, float* v_mean,
                               int32_t* perm, int32_t* labels, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  Dims D;
  if (vc_status s = validate(cfg, true, &D)) return s;
  if (!cfg->vsmooth) return fail(VC_ERR_INVALID_ARG, "vsmooth_prepare_warm needs vsmooth on");
  if (!K || !V || !Kq || !k_scale || !Vres || !v_scale || !v_mean || !perm || !ws)
    return fail(VC_ERR_INVALID_ARG, "required pointer is NULL");
  if ((init_idx != nullptr) + (init_centroids != nullptr) + (perm_in != nullptr) > 1)
    return fail(VC_ERR_INVALID_ARG, "at most one of init_idx, init_centroids, perm_in may be given");
  if (misaligned(K) || misaligned(V) || misaligned(Kq) || misaligned(Vres) || misaligned(v_scale) ||
      misaligned(v_mean) || misaligned(ws))
    return fail(VC_ERR_INVALID_ARG, "tensors and workspace must be 16-byte aligned");
  if (ws_bytes < vc_prepare_workspace_bytes(cfg)) return fail(VC_ERR_WORKSPACE, "workspace too small");
  vc::PrepArgs a{};
  fill_prep_args(cfg, D, K, V, a);
  Carver cv(reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~static_cast<uintptr_t>(255)));
  carve_prep(cv, D, a);
  vc::PrepOut o{Kq, k_scale, Vres, v_scale, v_mean, perm};
  return run_prepare(cfg, D, a, init_idx, o, perm_in ? nullptr : labels, stream, init_centroids, perm_in,
                     perm_in ? nullptr : centroids_out);
}

vc_status vc_attn_fwd(const vc_config* cfg, const void* Q, const uint8_t* Kq, const float* k_scale,
                      const uint8_t* Vres, const void* v_scale, const float* v_mean, void* O,
                      hipStream_t stream) {
  g_err.clear();
  Dims D;
  if (vc_status s = validate(cfg, false, &D)) return s;
  if (!Q || !Kq || !k_scale || !Vres || !v_scale || !v_mean || !O)
    return fail(VC_ERR_INVALID_ARG, "required pointer is NULL");
  if (misaligned(Q) || misaligned(Kq) || misaligned(Vres) || misaligned(v_scale) || misaligned(v_mean) ||
      misaligned(O))
    return fail(VC_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  vc::AttnArgs a{};
  fill_attn_args(cfg, D, a);
  a.Q = static_cast<const uint16_t*>(Q);
  a.Kq = Kq; a.k_scale = k_scale; a.Vres = Vres; a.v_scale = v_scale; a.v_mean = v_mean; a.O = O;
  VC_TRY(vc::launch_attn(a, stream), "attn_fwd");
  return VC_OK;
}

vc_status vc_dbg_attn_trace(const vc_config* cfg, const void* Q, const uint8_t* Kq, const float* k_scale,
                            const uint8_t* Vres, const void* v_scale, const float* v_mean, void* O, int32_t bh,
                            int32_t q_group, float* S, uint8_t* P, float* m, float* c, float* rowsum,
                            hipStream_t stream) {
  g_err.clear();
  Dims D;
  if (vc_status s = validate(cfg, false, &D)) return s;
  if (!cfg->out_fp32) return fail(VC_ERR_UNSUPPORTED, "the trace runs with fp32 output only (out_fp32 = 1)");
  if (!Q || !Kq || !k_scale || !Vres || !v_scale || !v_mean || !O || !S || !P || !m || !c || !rowsum)
    return fail(VC_ERR_INVALID_ARG, "required pointer is NULL");
  if (misaligned(Q) || misaligned(Kq) || misaligned(Vres) || misaligned(v_scale) || misaligned(v_mean) ||
      misaligned(O) || misaligned(S) || misaligned(P))
    return fail(VC_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  const int groups = (D.N + kTraceRows - 1) / kTraceRows;
  if (bh < 0 || static_cast<size_t>(bh) >= D.BH || q_group < 0 || q_group >= groups)
    return fail(VC_ERR_INVALID_ARG, "bh or q_group out of range");
  vc::AttnArgs a{};
  fill_attn_args(cfg, D, a);
  a.Q = static_cast<const uint16_t*>(Q);
  a.Kq = Kq; a.k_scale = k_scale; a.Vres = Vres; a.v_scale = v_scale; a.v_mean = v_mean; a.O = O;
  a.tr_wg = bh * groups + q_group;
  a.tr_S = S; a.tr_P = P; a.tr_m = m; a.tr_c = c; a.tr_l = rowsum;
  VC_TRY(vc::launch_attn(a, stream), "attn_fwd trace");
  return VC_OK;
}

}  // extern "C"

namespace {

vc_status attention_impl(const vc_config* cfg, const void* Q, const void* K, const void* V,
                         const int32_t* init_idx, void* O, void* ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  if (vc_status s = validate(cfg, cfg && cfg->vsmooth, &D)) return s;
  if (!Q || !K || !V || !O || !ws) return fail(VC_ERR_INVALID_ARG, "required pointer is NULL");
  if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(O) || misaligned(ws))
    return fail(VC_ERR_INVALID_ARG, "tensors and workspace must be 16-byte aligned");
  if (ws_bytes < vc_attention_workspace_bytes(cfg)) return fail(VC_ERR_WORKSPACE, "workspace too small");
  vc::PrepArgs a{};
  fill_prep_args(cfg, D, K, V, a);
  Carver cv(reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~static_cast<uintptr_t>(255)));
  carve_prep(cv, D, a);
  const OutSizes s = out_sizes(D, cfg->v_format);
  vc::PrepOut o;
  o.Kq = cv.take<uint8_t>(s.kq);
  o.k_scale = cv.take<float>(s.ks);
  o.Vres = cv.take<uint8_t>(s.vres);
  o.v_scale = cv.take<uint8_t>(s.vsc_bytes);
  o.v_mean = cv.take<float>(s.vmean);
  o.perm = cv.take<int32_t>(s.perm);
  if (vc_status st = run_prepare(cfg, D, a, init_idx, o, nullptr, stream)) return st;
  vc::AttnArgs at{};
  fill_attn_args(cfg, D, at);
  at.Q = static_cast<const uint16_t*>(Q);
  at.Kq = o.Kq; at.k_scale = o.k_scale; at.Vres = o.Vres; at.v_scale = o.v_scale; at.v_mean = o.v_mean; at.O = O;
  VC_TRY(vc::launch_attn(at, stream), "attn_fwd");
  return VC_OK;
}

// ---- vc_attention_noalloc: the library's own scratch in place of a workspace ----
// One file-scope device array per GPU (each GPU the library runs on holds its
// own copy until the process ends).  In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, once per device
// with that device current, and only that address is ever handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

vc_status scratch_of_current_device(void** out) {
  int dev = 0;
  VC_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(VC_ERR_UNSUPPORTED, "device index must be below 64");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    VC_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) return fail(VC_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return VC_OK;
}

}  // namespace

extern "C" {

vc_status vc_attention(const vc_config* cfg, const void* Q, const void* K, const void* V,
                       const int32_t* init_idx, void* O, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  return attention_impl(cfg, Q, K, V, init_idx, O, ws, ws_bytes, stream);
}

size_t vc_noalloc_scratch_bytes(void) { return kScratchBytes; }

vc_status vc_attention_noalloc(const vc_config* cfg, const void* Q, const void* K, const void* V,
                               const int32_t* init_idx, void* O, hipStream_t stream) {
  g_err.clear();
  Dims D;
  if (vc_status s = validate(cfg, cfg && cfg->vsmooth, &D)) return s;
  const size_t need = vc_attention_workspace_bytes(cfg);
  if (need > kScratchBytes)
    return fail(VC_ERR_WORKSPACE, "this configuration needs " + std::to_string(need) +
                                      " bytes of scratch; vc_attention_noalloc holds " +
                                      std::to_string(kScratchBytes) + " (use vc_attention with a workspace)");
  void* ws = nullptr;
  if (vc_status s = scratch_of_current_device(&ws)) return s;
  return attention_impl(cfg, Q, K, V, init_idx, O, ws, kScratchBytes, stream);
}

vc_status vc_dbg_expcast(const float* S, const float* A, const float* B, int64_t n, uint8_t* out,
                         hipStream_t stream) {
  g_err.clear();
  if (n < 0) return fail(VC_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && (!S || !A || !B || !out)) return fail(VC_ERR_INVALID_ARG, "required pointer is NULL");
  VC_TRY(vc::launch_dbg_expcast(S, A, B, n, out, stream), "dbg_expcast");
  return VC_OK;
}

vc_status vc_dbg_exp2cast(const float* S, const float* A, const float* B, int64_t n, uint8_t* out,
                          hipStream_t stream) {
  g_err.clear();
  if (n < 0) return fail(VC_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && (!S || !A || !B || !out)) return fail(VC_ERR_INVALID_ARG, "required pointer is NULL");
  VC_TRY(vc::launch_dbg_exp2cast(S, A, B, n, out, stream), "dbg_exp2cast");
  return VC_OK;
}

vc_status vc_mfma_loop(int32_t blocks, int32_t iters, float* out, hipStream_t stream) {
  g_err.clear();
  if (blocks < 1 || iters < 1) return fail(VC_ERR_INVALID_ARG, "blocks and iters must be >= 1");
  if (!out) return fail(VC_ERR_INVALID_ARG, "out is NULL");
  VC_TRY(vc::launch_mfma_loop(blocks, iters, out, stream), "mfma_loop");
  return VC_OK;
}

vc_status vc_dbg_kmeans_assign(const vc_config* cfg, const void* V, const float* C, int32_t* labels, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  Dims D;
  if (vc_status s = validate(cfg, true, &D)) return s;
  if (!V || !C || !labels || !ws) return fail(VC_ERR_INVALID_ARG, "required pointer is NULL");
  if (misaligned(V) || misaligned(ws)) return fail(VC_ERR_INVALID_ARG, "V and workspace must be 16-byte aligned");
  vc_config c2 = *cfg;
  c2.vsmooth = 1;
  if (ws_bytes < vc_prepare_workspace_bytes(&c2)) return fail(VC_ERR_WORKSPACE, "workspace too small");
  vc::PrepArgs a{};
  fill_prep_args(&c2, D, V, V, a);
  Carver cv(reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~static_cast<uintptr_t>(255)));
  carve_prep(cv, D, a);
  a.C = const_cast<float*>(C);
  VC_TRY(vc::launch_fill(a.vamax, 0u, D.BH, stream), "fill");
  VC_TRY(vc::launch_stats(a, stream), "stats");
  VC_TRY(vc::launch_quant_v_i8(a, stream), "quant_v_i8");
  VC_TRY(vc::launch_assign(a, labels, stream), "kmeans_assign");
  return VC_OK;
}

vc_status vc_dbg_init_tokens(const vc_config* cfg, int32_t* init, hipStream_t stream) {
  g_err.clear();
  Dims D;
  if (vc_status s = validate(cfg, true, &D)) return s;
  if (!init) return fail(VC_ERR_INVALID_ARG, "init is NULL");
  vc::PrepArgs a{};
  fill_prep_args(cfg, D, nullptr, nullptr, a);
  VC_TRY(vc::launch_init_seeded(a, cfg->seed, init, stream), "init_seeded");
  return VC_OK;
}

vc_status vc_dbg_sort(const vc_config* cfg, const int32_t* labels, int32_t* perm, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  g_err.clear();
  Dims D;
  if (vc_status s = validate(cfg, true, &D)) return s;
  if (!labels || !perm || !ws) return fail(VC_ERR_INVALID_ARG, "required pointer is NULL");
  vc_config c2 = *cfg;
  c2.vsmooth = 1;
  if (ws_bytes < vc_prepare_workspace_bytes(&c2)) return fail(VC_ERR_WORKSPACE, "workspace too small");
  vc::PrepArgs a{};
  fill_prep_args(&c2, D, nullptr, nullptr, a);
  Carver cv(reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~static_cast<uintptr_t>(255)));
  carve_prep(cv, D, a);
  VC_TRY(vc::launch_sort(a, labels, perm, stream), "sort");
  return VC_OK;
}

}  // extern "C"
