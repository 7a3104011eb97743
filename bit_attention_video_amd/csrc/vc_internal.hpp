// Internal declarations shared by the host library and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <algorithm>
#include "vc_device.hpp"

namespace vc {

constexpr int kMaxClusters = 4096;   // k-means clusters per head (LDS histogram size)
constexpr int kSortChunk = 4096;     // tokens per counting-sort chunk

struct PrepArgs {
  int B, H, N, d, kvb, k, kpad, iters, vsmooth, v_format;
  int nblk, nstat, nsort;
  const uint16_t* K;
  const uint16_t* V;
  // workspace
  uint32_t* vamax;     // [BH]       max |V| bits
  float* sV;           // [BH]       int8 scale of V
  double* kpart;       // [BH,nstat,d]
  float* mu;           // [BH,d]     K channel means
  int8_t* Vq;          // [BH,N,d]
  float* C;            // [BH,k,d]   centroids
  int8_t* Cq;          // [BH,kpad,d]
  int32_t* cn32;       // [BH,kpad]
  int32_t* labels;     // [BH,N]
  int32_t* perm_tmp;   // [BH,N]
  int32_t* hist;       // [BH,nsort,k]
  int32_t* counts;     // [BH,k]
  int32_t* starts;     // [BH,k]
  uint32_t* vramax;    // [BH,d]     residual channel max bits
  int32_t* rank;       // [BH,k]     cluster order (renumbering before the final pass)
  float* Ctmp;         // [BH,k,d]   renumbered centroids
  int32_t* init;       // [BH,k]     seeded initial token indices
  // balanced clusters (capped assignment)
  int32_t* prop;       // [BH,N]     proposed cluster of the round's i-th unplaced token
  int32_t* pdist;      // [BH,N]     squared int8 distance of each token to its proposal
  int32_t* rem;        // [BH,k]     places left per cluster
  int32_t* alist[2];   // [BH,N]     unplaced tokens in token order (a round reads one, fills the other)
  int32_t* acnt[2];    // [BH]       their numbers
  int32_t* ccnt;       // [BH,nsort] their numbers per chunk of kSortChunk list entries
};

struct PrepOut {
  uint8_t* Kq;
  float* k_scale;
  uint8_t* Vres;
  void* v_scale;
  float* v_mean;
  int32_t* perm;
};

struct AttnArgs {
  int B, H, N, d, kvb, nblk, v_format, out_fp32;
  int pm;              // kernel probability mode: 0 ExpCast (byte from one FMA), 1 exp2 + E4M3 cast
  float scale, kc;     // softmax scale; ExpCast addend fp32(56 + beta), or fp32(120 + beta) range-shifted
  const uint16_t* Q;
  const uint8_t* Kq;
  const float* k_scale;
  const uint8_t* Vres;
  const void* v_scale;
  const float* v_mean;
  void* O;
  // test-only trace of one workgroup (tr_S null: the production kernels)
  int tr_wg;
  float* tr_S;
  uint8_t* tr_P;
  float* tr_m;
  float* tr_c;
  float* tr_l;
};

hipError_t launch_fill(uint32_t* p, uint32_t v, size_t n, hipStream_t st);
hipError_t launch_stats(const PrepArgs& a, hipStream_t st);
hipError_t launch_quant_v_i8(const PrepArgs& a, hipStream_t st);
hipError_t launch_init_seeded(const PrepArgs& a, uint64_t seed, int32_t* init, hipStream_t st);
hipError_t launch_init_centroids(const PrepArgs& a, const int32_t* init, hipStream_t st);
hipError_t launch_assign(const PrepArgs& a, int32_t* labels, hipStream_t st);
hipError_t launch_bal_assign(const PrepArgs& a, int32_t* labels, hipStream_t st);
hipError_t launch_sort(const PrepArgs& a, const int32_t* labels, int32_t* perm, hipStream_t st);
hipError_t launch_sort_list(const PrepArgs& a, const int32_t* keys, const int32_t* ids, const int32_t* n,
                            int32_t* perm, hipStream_t st);
hipError_t launch_cluster_order(const PrepArgs& a, hipStream_t st);
hipError_t launch_update(const PrepArgs& a, const int32_t* perm, hipStream_t st);
hipError_t launch_iota(int32_t* perm, int N, size_t total, hipStream_t st);
hipError_t launch_vres_ksmooth(const PrepArgs& a, const int32_t* perm, const PrepOut& o, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);
template <int D, int KVB, int VF>
hipError_t launch_attn_cfg(const AttnArgs& a, hipStream_t st);
hipError_t launch_dbg_expcast(const float* S, const float* A, const float* B, int64_t n, uint8_t* out,
                              hipStream_t st);
hipError_t launch_dbg_exp2cast(const float* S, const float* A, const float* B, int64_t n, uint8_t* out,
                               hipStream_t st);
hipError_t launch_mfma_loop(int blocks, int iters, float* out, hipStream_t st);

}  // namespace vc
