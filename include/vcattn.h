/*
 * vcattn.h - C ABI of the VC-Attention forward pass for AMD MI355X (gfx950).
 *
 * The method (web pages on VC-Attention):
 *   - V-Smooth: a lightweight k-means groups similar value tokens into the same
 *     fixed-size hardware block; each block's mean is subtracted and kept in
 *     high precision, only the residual is quantised (per-channel E4M3, or a
 *     4-bit format), and the mean is restored from the row sums the online
 *     softmax keeps.  (chooseai.io brief, section "V-Smooth"; zerohour.day
 *     summary, key facts: per-channel E4M3/NVFP4 residuals after block-mean
 *     subtraction; theclarity.today story: one pass over the values.)
 *   - ExpCast-FP8: the softmax probability byte is computed from the log2
 *     score z by one fused multiply-add, round(8z + 56 + beta), clamped to
 *     [0, 56], instead of an fp32 exp2 followed by a cast.  (chooseai.io brief,
 *     section "ExpCast-FP8".)
 *   - QK^T and PV both run on FP8 E4M3 matrix instructions.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers of the current HIP device.  The
 *     caller owns every buffer, including the workspace; the library never
 *     allocates or frees device memory and keeps no state between calls
 *     (except the per-thread error string).
 *   - Work is enqueued on `stream`; nothing synchronises.  Calls on different
 *     streams need different workspaces and outputs.
 *   - Arguments are validated before anything is launched.  On an invalid
 *     argument nothing runs and VC_ERR_INVALID_ARG / VC_ERR_UNSUPPORTED /
 *     VC_ERR_WORKSPACE is returned; a failed launch returns VC_ERR_HIP and
 *     vc_last_error() holds the HIP message.  No exception crosses the ABI.
 *   - bf16 tensors are raw 16-bit bfloat16 patterns.
 *   - Shapes: Q, K, V, O are [B, H, N, d] row-major.  d in {64, 128},
 *     kv_block in {64, 128}, query tiles are 128 rows (natural token order).
 *     nblk = ceil(N / kv_block); Np = nblk * kv_block (padded length).
 *
 * Blocked layouts written by vsmooth_prepare (all per (b, h), in that order):
 *   perm     int32 [B,H,N]   perm[j] = original index of the token at sorted
 *                            position j (stable sort by cluster label).
 *   Kq       uint8 [B,H,Np,d] E4M3 codes of the smoothed, permuted keys.  Rows
 *                            are stored in "k-step order": sorted positions
 *                            come in groups of 64; inside a group the sorted
 *                            position kappa = 32t + 16g + 4i + j (t,g in {0,1},
 *                            i,j in 0..3) is stored at row 32t + 8i + 4g + j.
 *                            Padded rows (position >= N) are 0.
 *   k_scale  fp32 [B,H,nblk] per-block key scale.
 *   Vres     E4M3:  uint8 [B,H,Np/64,d,64]  per group of 64 sorted positions,
 *                   one 64-byte row per channel (position order).
 *            MXFP4: uint8 [B,H,Np/64,d,32]  same, two E2M1 codes per byte, the
 *                   even position in the low nibble.
 *            MXFP8: as E4M3 (codes relative to the E8M0 scales below).
 *            NVFP4 style (zerohour.day summary, key facts: NVFP4 residuals):
 *                   uint8 [B,H,nblk,2,kv_block/64,d,64]  per block the
 *                   E4M3 "high" codes of all its 64-position groups (E4M3
 *                   layout), then the "low" codes.  The quantised residual
 *                   (per 16 sorted positions x channel an E4M3 block scale s16
 *                   = E4M3(amax16 / (6 * 2^t)), E2M1 elements, a power-of-two
 *                   second-level scale 2^t per head) is v = e2m1 * s16 * 2^t;
 *                   with e per 32 positions x channel the smallest integer with
 *                   max|e2m1 * s16| <= 448 * 2^e, high = E4M3(e2m1 * s16 / 2^e)
 *                   and low = E4M3(e2m1 * s16 / 2^e - high), so
 *                   v = (high + low) * 2^(e + t) (exactly, unless the low part
 *                   falls below E4M3's smallest subnormal).
 *   v_scale  E4M3:  fp32 [B,H,d]  per-channel residual scale.
 *            MXFP4, MXFP8, NVFP4 style: uint8 E8M0 [B,H,Np/32,d]  one scale
 *                   per 32 sorted positions and channel (NVFP4 style: e + t);
 *                   inside a group, channel c = 32T + u (u < 32) is stored at
 *                   byte u * (d/32) + T.
 *   v_mean   fp32 [B,H,nblk,d]  block means (zero when V-Smooth is off).
 */
#ifndef VCATTN_H
#define VCATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VC_OK = 0,
  VC_ERR_INVALID_ARG = -1,
  VC_ERR_UNSUPPORTED = -2,
  VC_ERR_WORKSPACE = -3,
  VC_ERR_HIP = -4
} vc_status;

typedef struct {
  int32_t B, H, N, d;       /* N >= 1 with N * d < 2^31; d in {64, 128}            */
  int32_t kv_block;         /* 64 or 128 tokens per hardware block                 */
  int32_t n_clusters;       /* k-means clusters k, 1 <= k <= min(N, 4096)          */
  int32_t iters;            /* k-means assignment passes I, 1..16                  */
  int32_t vsmooth;          /* 1: V-Smooth on; 0: identity order, zero means       */
  int32_t v_format;         /* 0: E4M3 residuals, per-channel scale; 1: MXFP4;     */
                            /*    2: MXFP8 (E4M3 codes, E8M0 scale per 32 sorted   */
                            /*    positions and channel); 3: NVFP4 style (E2M1,    */
                            /*    E4M3 scale per 16 sorted positions and channel), */
                            /*    stored and multiplied as two E4M3 parts          */
  int32_t out_fp32;         /* 0: O is bf16; 1: O is fp32                          */
  float softmax_scale;      /* 0 selects fp32(1/sqrt(d))                           */
  float beta;               /* ExpCast offset, -0.5 <= beta <= 0.45                */
  int32_t p_mode;           /* 0: ExpCast-FP8 probability bytes; 1: ExpCast off,   */
                            /*    p = E4M3(exp2(x)) (see below); 2: ExpCast moved  */
                            /*    up by 64 codes, round(8z + 120 + beta), so that  */
                            /*    p = 2^8 * 2^z stays a normal E4M3 value down to  */
                            /*    z = -14 (the factor 2^8 cancels in O)            */
  int32_t cluster_order;    /* 0: clusters in k-means label order; 1: renumbered   */
                            /*    along the principal axis of their int8 codes     */
                            /*    before the final pass (see vsmooth_prepare)      */
  uint64_t seed;            /* k-means initialisation when no init_idx is given:   */
                            /*    per head (b, h) the k initial tokens are a       */
                            /*    partial Fisher-Yates shuffle of 0..N-1 driven by */
                            /*    splitmix64 seeded with                           */
                            /*    seed + 0x9E3779B97F4A7C15 * (b*H + h): draw r_i, */
                            /*    j = i + r_i mod (N - i), swap positions i and j, */
                            /*    for i = 0..k-1; the first k positions are used   */
  int32_t balanced;         /* 1: balanced clusters sized to the hardware blocks   */
                            /*    (a blocking variant): n_clusters must be         */
                            /*    ceil(N / kv_block), cluster c holds kv_block     */
                            /*    tokens (the last one the tail), so every block   */
                            /*    is one cluster; see vsmooth_prepare              */
} vc_config;

/* Bytes of workspace vsmooth_prepare needs (k-means and sort scratch). */
size_t vc_prepare_workspace_bytes(const vc_config* cfg);
/* Bytes of workspace vc_attention needs (prepare scratch + blocked K/V). */
size_t vc_attention_workspace_bytes(const vc_config* cfg);
/* Bytes of workspace enough for every call that takes one (vsmooth_prepare,
 * vsmooth_prepare_warm, vc_attention): equals vc_attention_workspace_bytes;
 * 0 for an invalid configuration. */
size_t vc_workspace_bytes(const vc_config* cfg);

/*
 * vsmooth_prepare: V-Smooth and K smoothing (chooseai.io brief, "V-Smooth").
 *   K, V      bf16 [B,H,N,d]
 *   init_idx  int32 [B,H,k]  initial centroid token indices, distinct, in
 *             [0, N), or NULL: the library draws them from cfg->seed (see
 *             vc_config; the method clusters inside the attention call,
 *             theclarity.today story).  Ignored when vsmooth == 0.
 *   outputs   Kq, k_scale, Vres, v_scale, v_mean, perm in the layouts above;
 *             labels int32 [B,H,N] final cluster labels (nullable)
 *   ws        device workspace of at least vc_prepare_workspace_bytes(cfg)
 * Readings where the pages are silent: k-means distances on int8 codes with
 * one per-head scale, ties to the lowest cluster index, fp32 centroid means;
 * stable sort by label and fixed blocks; K smoothed by its per-channel mean
 * and quantised per block.
 * cfg->cluster_order == 1 (a blocking variant): before the final assignment
 * pass the centroids are renumbered by their position along the principal
 * axis of their int8 codes (exact integer covariance and power iteration;
 * ties to the lower index), so the blocks follow that order; labels and
 * centroids_out use the new numbering.
 * cfg->balanced == 1 (a blocking variant; the chooseai.io brief, "V-Smooth",
 * puts similar tokens into the same hardware block): every assignment pass is
 * capped.  In up to 12 rounds each unassigned token proposes to its nearest
 * cluster that still has room (ties to the lowest cluster index) and a
 * cluster with r places left takes the r nearest proposers (exact int8
 * squared distances, ties to the lowest token index); tokens left after the
 * rounds fill the remaining places in token order, clusters in index order.
 */
vc_status vsmooth_prepare(const vc_config* cfg, const void* K, const void* V,
                          const int32_t* init_idx, uint8_t* Kq, float* k_scale,
                          uint8_t* Vres, void* v_scale, float* v_mean, int32_t* perm,
                          int32_t* labels, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * vsmooth_prepare_warm: vsmooth_prepare that carries the clustering across
 * calls (denoising steps: the runtimewire article and the chooseai.io brief
 * describe running V-Smooth step by step and treating its cost as a
 * scheduling trade).  cfg->vsmooth must be 1.  At most one of
 *   init_idx        int32 [B,H,k]   cold start, as in vsmooth_prepare;
 *   init_centroids  fp32 [B,H,k,d]  warm start, e.g. the centroids_out of the
 *                   previous step; cfg->iters passes (1 is the usual choice);
 *   perm_in         int32 [B,H,N]   reuse a permutation: no clustering and no
 *                   sort.  It must be a permutation of 0..N-1 per head;
 *                   entries outside [0, N) are clamped, so a bad perm_in
 *                   gives meaningless output but reads nothing outside K, V.
 *                   perm may equal perm_in.
 * is non-NULL; with none, the cold start draws its tokens from cfg->seed.
 * centroids_out (nullable, fp32 [B,H,k,d]) receives the member
 * means of the final clusters (a cluster with no members keeps its
 * centroid); it is left untouched when perm_in is given, and labels too.
 * Other arguments as vsmooth_prepare.
 */
vc_status vsmooth_prepare_warm(const vc_config* cfg, const void* K, const void* V,
                               const int32_t* init_idx, const float* init_centroids,
                               const int32_t* perm_in, float* centroids_out, uint8_t* Kq,
                               float* k_scale, uint8_t* Vres, void* v_scale, float* v_mean,
                               int32_t* perm, int32_t* labels, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/*
 * vc_attn_fwd: fused forward (chooseai.io brief, "ExpCast-FP8" and the last
 * sentences of "V-Smooth").  Q bf16 [B,H,N,d] in natural order; Kq..v_mean as
 * written by vsmooth_prepare; O [B,H,N,d] bf16 or fp32 (cfg->out_fp32), rows in
 * natural token order.  Per 128-row query tile: E4M3 query codes with one
 * scale; per KV block in ascending order: S = Qq.Kq^T on FP8 MFMA, running
 * log2 maximum m, bytes = cvt_u8(fma(S, 8c, 56 + beta - 8m)), row sums of the
 * decoded bytes, acc = alpha*acc + P.Vres + rowsum * mean; O = scale*acc / l.
 */
vc_status vc_attn_fwd(const vc_config* cfg, const void* Q, const uint8_t* Kq,
                      const float* k_scale, const uint8_t* Vres, const void* v_scale,
                      const float* v_mean, void* O, hipStream_t stream);

/*
 * vc_dbg_attn_trace: test entry point.  Runs vc_attn_fwd (same arguments, O
 * written in full) with a trace instantiation of the same kernel, in which
 * the workgroup of query rows [256*q_group, 256*q_group + 256) of head
 * bh = b*H + h also records, for every KV block b in the order it is visited
 * (chooseai.io brief, "ExpCast-FP8": the byte comes from one FMA on the
 * log2-domain score relative to the running maximum):
 *   S       fp32  [nblk][256][kv_block]  the fp32 scores Qq.Kq^T of the block
 *                 after masking (padded keys -inf), key index = sorted
 *                 position inside the block;
 *   P       uint8 [nblk][256][kv_block]  the probability bytes, same order;
 *   m       fp32  [nblk][256]  running log2-domain maximum after the block;
 *   c       fp32  [nblk][256]  the block's log2-domain score scale
 *                 c = fp32(cq * k_scale[b]), cq = fp32(fp32(s_q*scale)*log2 e);
 *   rowsum  fp32  [nblk][256]  the block's row sum of the decoded bytes.
 * Rows at or beyond N hold the values for zero query codes.  Any residual
 * format; requires out_fp32 = 1 (VC_ERR_UNSUPPORTED otherwise); bh and
 * q_group out of range give VC_ERR_INVALID_ARG.  The caller owns all
 * buffers.
 */
vc_status vc_dbg_attn_trace(const vc_config* cfg, const void* Q, const uint8_t* Kq,
                            const float* k_scale, const uint8_t* Vres, const void* v_scale,
                            const float* v_mean, void* O, int32_t bh, int32_t q_group, float* S,
                            uint8_t* P, float* m, float* c, float* rowsum, hipStream_t stream);

/* vc_attention: vsmooth_prepare + vc_attn_fwd with the blocked K/V kept in the
 * workspace (the clustering happens inside the attention call, as the
 * theclarity.today story describes).  ws >= vc_attention_workspace_bytes.
 * init_idx may be NULL (initial tokens drawn from cfg->seed). */
vc_status vc_attention(const vc_config* cfg, const void* Q, const void* K, const void* V,
                       const int32_t* init_idx, void* O, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * vc_attention_noalloc: vc_attention for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and kernels, with the workspace
 * taken from a static device array inside the library, vc_noalloc_scratch_bytes()
 * = 64 MiB per GPU, held by every GPU the library runs on until the process
 * ends.  The caller still passes Q, K, V (and init_idx, nullable) and O.
 * Nothing is allocated or freed.  A configuration whose
 * vc_attention_workspace_bytes exceeds the scratch returns VC_ERR_WORKSPACE
 * before anything runs.  Every call on one GPU uses that GPU's one array and
 * leaves its contents behind: calls that overlap on one GPU (other streams or
 * threads) race and must be serialised by the caller.
 */
vc_status vc_attention_noalloc(const vc_config* cfg, const void* Q, const void* K, const void* V,
                               const int32_t* init_idx, void* O, hipStream_t stream);
size_t vc_noalloc_scratch_bytes(void);

const char* vc_status_str(vc_status s);
/* Message of the last failure on the calling thread ("" if none). */
const char* vc_last_error(void);
/* The same message as vc_last_error (HIP failures carry the HIP error string). */
const char* vc_last_hip_error(void);

/* ---- test entry points (same kernels as the path above) --------------------
 * vc_dbg_expcast: out[i] = the ExpCast byte the attention kernel computes from
 *   fp32 score S[i] with per-element A[i] = 8c and B[i] = 56 + beta - 8m.
 * vc_dbg_kmeans_assign: one assignment pass given centroids C fp32 [B,H,k,d]
 *   (int8 codes with the per-head scale of V), labels int32 [B,H,N].
 * vc_dbg_sort: perm int32 [B,H,N] = stable sort of labels int32 [B,H,N] with
 *   k = cfg->n_clusters. */
vc_status vc_dbg_expcast(const float* S, const float* A, const float* B, int64_t n,
                         uint8_t* out, hipStream_t stream);
/* vc_dbg_exp2cast: out[i] = the p_mode 1 byte: E4M3 (round to nearest even)
 *   of the fp32 exp2 of x = fma(S[i], A[i], B[i]) (A = c, B = -m). */
vc_status vc_dbg_exp2cast(const float* S, const float* A, const float* B, int64_t n,
                          uint8_t* out, hipStream_t stream);
vc_status vc_dbg_kmeans_assign(const vc_config* cfg, const void* V, const float* C,
                               int32_t* labels, void* ws, size_t ws_bytes, hipStream_t stream);
vc_status vc_dbg_sort(const vc_config* cfg, const int32_t* labels, int32_t* perm,
                      void* ws, size_t ws_bytes, hipStream_t stream);
/* vc_dbg_init_tokens: init int32 [B,H,k] = the k initial token indices that
 *   vsmooth_prepare draws from cfg->seed when it is given no init_idx (the
 *   seeded partial Fisher-Yates of vc_config.seed). */
vc_status vc_dbg_init_tokens(const vc_config* cfg, int32_t* init, hipStream_t stream);

/* ---- measurement entry point ------------------------------------------------
 * vc_mfma_loop: the attainable FP8 MFMA rate on this GPU at its sustained
 *   clock.  Launches `blocks` workgroups of 512 threads; every wave issues
 *   `iters` rounds of 8 independent v_mfma 32x32x64 FP8 instructions (131072
 *   flops each, so the launch does blocks*8*iters*8*131072 flops).  out:
 *   float[blocks*512] device buffer that receives a checksum per thread (keeps
 *   the results live).  Errors: INVALID_ARG for blocks < 1, iters < 1 or NULL
 *   out. */
vc_status vc_mfma_loop(int32_t blocks, int32_t iters, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* VCATTN_H */
