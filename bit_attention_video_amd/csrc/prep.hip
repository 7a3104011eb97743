// V-Smooth preparation kernels for gfx950: statistics, int8 k-means on the
// matrix cores (optionally with the clusters renumbered along their principal
// axis), stable counting sort into fixed blocks, block means with per-channel
// E4M3 residuals (or MXFP4 / MXFP8 with E8M0 scales per 32 sorted tokens and
// channel), and K smoothing with per-block E4M3.
//
// Method: chooseai.io brief on VC-Attention, section "V-Smooth" (cluster
// similar value tokens into one hardware block, subtract the block mean kept
// in high precision, quantise only the residual); zerohour.day summary, key
// facts (per-channel E4M3/NVFP4 residuals after block-mean subtraction).
// Every sum that feeds a stored value is formed in fp64 in a fixed order, so
// runs are deterministic.
#include <climits>

#include "vc_internal.hpp"

namespace vc {

constexpr int kStatChunk = 1024;   // tokens per partial-sum chunk

__global__ void k_fill_u32(uint32_t* __restrict__ p, uint32_t v, size_t n) {
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i < n; i += static_cast<size_t>(gridDim.x) * blockDim.x) p[i] = v;
}

// Per chunk of tokens: fp64 per-channel sums of K (for its mean) and the
// max |V| of the head (for the int8 k-means scale).  Each thread reads
// 16-byte pieces (8 channels) of every RG-th row; partial sums are combined
// in a fixed order.
template <int D>
__global__ __launch_bounds__(256) void k_stats_partial(const uint16_t* __restrict__ K,
                                                       const uint16_t* __restrict__ V, int N,
                                                       int nch, double* __restrict__ kpart,
                                                       uint32_t* __restrict__ vamax) {
  constexpr int CG = D / 8;          // 16-byte channel groups per row
  constexpr int RG = 256 / CG;       // rows read in parallel
  __shared__ double sK[RG][D];
  __shared__ float sMax[4];
  const int bh = blockIdx.y, ch = blockIdx.x;
  const int cg = threadIdx.x % CG, r0 = threadIdx.x / CG;
  const size_t base = static_cast<size_t>(bh) * N * D + cg * 8;
  const int t0 = ch * kStatChunk, t1 = min(N, t0 + kStatChunk);
  double ks[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float vm = 0.0f;
  for (int t = t0 + r0; t < t1; t += RG) {
    const uint4 kr = *reinterpret_cast<const uint4*>(K + base + static_cast<size_t>(t) * D);
    const uint4 vr = *reinterpret_cast<const uint4*>(V + base + static_cast<size_t>(t) * D);
    const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w}, vw[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ks[e] += static_cast<double>(bf16_to_f32(static_cast<uint16_t>(kw[e >> 1] >> ((e & 1) * 16))));
      vm = fmaxf(vm, fabsf(bf16_to_f32(static_cast<uint16_t>(vw[e >> 1] >> ((e & 1) * 16)))));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sK[r0][cg * 8 + e] = ks[e];
  vm = wave_max(vm);
  if ((threadIdx.x & 63) == 0) sMax[threadIdx.x >> 6] = vm;
  __syncthreads();
  if (threadIdx.x < D) {
    double s = 0.0;
    for (int j = 0; j < RG; ++j) s += sK[j][threadIdx.x];
    kpart[(static_cast<size_t>(bh) * nch + ch) * D + threadIdx.x] = s;
  }
  if (threadIdx.x == 0) {
    const float m = fmaxf(fmaxf(sMax[0], sMax[1]), fmaxf(sMax[2], sMax[3]));
    atomicMax(vamax + bh, __float_as_uint(m));
  }
}

// mu_K = fp32(sum / N) per channel; sV = fp32(max|V| / 127) floored at 2^-126
// (1 if V == 0).
template <int D>
__global__ void k_stats_final(const double* __restrict__ kpart, const uint32_t* __restrict__ vamax,
                              int N, int nch, float* __restrict__ mu, float* __restrict__ sV) {
  const int bh = blockIdx.x, c = threadIdx.x;
  double s = 0.0;
  constexpr int U = 8;                          // partials loaded per batch, added in chunk order
  for (int c0 = 0; c0 < nch; c0 += U) {
    double v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = c0 + u < nch ? kpart[(static_cast<size_t>(bh) * nch + c0 + u) * D + c] : 0.0;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u < nch) s += v[u];
  }
  mu[static_cast<size_t>(bh) * D + c] = static_cast<float>(s / static_cast<double>(N));
  if (c == 0) {
    const float a = __uint_as_float(vamax[bh]);
    sV[bh] = a > 0.0f ? fmaxf(a / 127.0f, kScaleFloor) : 1.0f;
  }
}

// int8 codes of V for the k-means distances, 8 elements per thread.
__global__ void k_quant_v_i8(const uint16_t* __restrict__ V, const float* __restrict__ sV,
                             size_t per_head, size_t total, int8_t* __restrict__ Vq) {
  const size_t i8 = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
  if (i8 >= total) return;
  const float s = sV[i8 / per_head];
  const float y = 1.0f / s;
  const uint4 raw = *reinterpret_cast<const uint4*>(V + i8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t b = static_cast<uint16_t>(w[e >> 1] >> ((e & 1) * 16));
    const uint32_t q = static_cast<uint32_t>(i8_code(bf16_to_f32(b), s, y)) & 0xffu;
    out[e >> 2] |= q << ((e & 3) * 8);
  }
  *reinterpret_cast<uint2*>(Vq + i8) = make_uint2(out[0], out[1]);
}

// ---- seeded initial centroids --------------------------------------------------
// The k initial tokens of head bh are a partial Fisher-Yates shuffle of 0..N-1
// driven by splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014) seeded with seed + 0x9E3779B97F4A7C15 * bh: draw
// r_i (i = 0..k-1), j_i = i + r_i mod (N - i), swap positions i and j_i; the
// first k positions are the result.  The swaps are resolved in parallel: the
// value at position i just before step i is v(i) = v(i'') for the last earlier
// step i'' with j_i'' = i (i itself if none), and the value step i takes is
// v(i') for the last earlier step i' with j_i' = j_i (j_i itself if none;
// j_i = i gives v(i)).  One workgroup per head; k <= kMaxClusters.
constexpr int kInitThreads = 1024;

__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  // output i (from 0) of the generator started at state `seed`
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ __launch_bounds__(kInitThreads) void k_init_seeded(uint64_t seed, int N, int k,
                                                              int32_t* __restrict__ init) {
  __shared__ int32_t sJ[kMaxClusters];
  __shared__ int32_t sPrev[kMaxClusters];    // last earlier step whose j is this step's position i
  __shared__ int32_t sSame[kMaxClusters];    // last earlier step with the same j
  __shared__ int32_t sV[kMaxClusters];       // value at position i just before step i
  const int bh = blockIdx.x;
  const uint64_t hs = seed + 0x9E3779B97F4A7C15ull * static_cast<uint64_t>(bh);
  for (int i = threadIdx.x; i < k; i += kInitThreads)
    sJ[i] = i + static_cast<int>(splitmix64_at(hs, static_cast<uint64_t>(i)) % static_cast<uint64_t>(N - i));
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += kInitThreads) {
    const int ji = sJ[i];
    int prev = -1, same = -1;
    for (int t = 0; t < i; ++t) {
      const int jt = sJ[t];
      prev = jt == i ? t : prev;
      same = jt == ji ? t : same;
    }
    sPrev[i] = prev;
    sSame[i] = same;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += kInitThreads) {
    int t = i;
    while (sPrev[t] >= 0) t = sPrev[t];     // strictly decreasing chain
    sV[i] = t;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += kInitThreads) {
    const int ji = sJ[i];
    const int val = ji == i ? sV[i] : (sSame[i] >= 0 ? sV[sSame[i]] : ji);
    init[static_cast<size_t>(bh) * k + i] = val;
  }
}

template <int D>
__global__ void k_init_centroids(const uint16_t* __restrict__ V, const int32_t* __restrict__ init,
                                 int N, int k, float* __restrict__ C) {
  const int bh = blockIdx.y, i = blockIdx.x, c = threadIdx.x;
  const int tok = init[static_cast<size_t>(bh) * k + i];
  C[(static_cast<size_t>(bh) * k + i) * D + c] =
      bf16_to_f32(V[(static_cast<size_t>(bh) * N + tok) * D + c]);
}

// rows of one centroid chunk of the assignment; the packed keys order the rows
// of a chunk in their low log2(kKeyRows) bits
constexpr int kKeyRows = 128;

// column tiles of 32 tokens per wave of the assignment (workgroup: 128 x this):
// four share each centroid tile read from LDS and each chunk's overhead;
// the balanced proposal rounds keep two, as their late rounds have few
// tokens per workgroup and need the registers (and occupancy) less tight
constexpr int kAssignTiles = 4;
constexpr int kBalAssignTiles = 2;

// int8 centroid codes and the packed score offsets cn32 = (127 - row % 128) - 128*|c|^2;
// rows k..kpad-1 are padding (codes 0, offset INT_MIN: their key is never the maximum).
template <int D>
__global__ __launch_bounds__(256) void k_quant_centroids(const float* __restrict__ C,
                                                         const float* __restrict__ sV, int k,
                                                         int kpad, int8_t* __restrict__ Cq,
                                                         int32_t* __restrict__ cn32) {
  constexpr int PER = D / 64;
  const int bh = blockIdx.y;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= kpad) return;
  const float s = sV[bh];
  int32_t sq = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = lane * PER + e;
    int32_t q = 0;
    if (i < k) q = i8_code(C[(static_cast<size_t>(bh) * k + i) * D + c], s);
    Cq[(static_cast<size_t>(bh) * kpad + i) * D + c] = static_cast<int8_t>(q);
    sq += q * q;
  }
  for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
  if (lane == 0)
    cn32[static_cast<size_t>(bh) * kpad + i] = i < k ? (kKeyRows - 1 - (i & (kKeyRows - 1))) - sq * kKeyRows : INT_MIN;
}

// LDS operands of one 32-centroid tile: the centroid codes (the A operand)
// and the key offsets of the 16 rows this lane's accumulators hold
template <int NDC, int CSTR>
__device__ __forceinline__ void assign_load_a(const int8_t* sC, int tile, int g, int col, v4i (&a)[NDC]) {
#pragma unroll
  for (int c = 0; c < NDC; ++c)
    a[c] = *reinterpret_cast<const v4i*>(sC + (tile * 32 + col) * CSTR + 32 * c + 16 * g);
}

__device__ __forceinline__ void assign_load_off(const int32_t* sCn, int tile, int g, int32_t (&off)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int4 o4 = *reinterpret_cast<const int4*>(sCn + tile * 32 + 8 * i + 4 * g);
    off[4 * i + 0] = o4.x; off[4 * i + 1] = o4.y; off[4 * i + 2] = o4.z; off[4 * i + 3] = o4.w;
  }
}

// 32 x 32 tile of C^T = centroid codes a . token codes b (exact int32)
template <int NDC>
__device__ __forceinline__ v16i assign_chain(const v4i (&a)[NDC], const v4i (&b)[NDC]) {
  v16i acc = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int c = 0; c < NDC; ++c) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[c], b[c], acc, 0, 0, 0);
  return acc;
}

// the maximum of m and the tile's keys (acc << 8) + off
__device__ __forceinline__ int assign_fold(const v16i& acc, const int32_t (&off)[16], int m) {
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const int k0 = static_cast<int>((static_cast<uint32_t>(acc[r]) << 8) + off[r]);
    const int k1 = static_cast<int>((static_cast<uint32_t>(acc[r + 1]) << 8) + off[r + 1]);
    m = max(max(m, k0), k1);
  }
  return m;
}

// Scores one centroid chunk (ntile tiles of 32 rows, in LDS) against the
// wave's first NJ column tiles: per tile, each column tile's MFMA chain and
// then the folding of its keys.  (Issuing the next chain before the fold, or
// interleaving the two, measured slower: a wave then holds the matrix core
// for longer bursts and the other waves of its SIMD wait.)
template <int NJ, int NDC, int CSTR, int NJW>
__device__ __forceinline__ void assign_chunk(const int8_t* sC, const int32_t* sCn, int ntile,
                                             const v4i (&bop)[NJW][NDC], int (&cmax)[NJW], int g, int col) {
  for (int tile = 0; tile < ntile; ++tile) {
    v4i a[NDC];
    int32_t off[16];
    assign_load_a<NDC, CSTR>(sC, tile, g, col, a);
    assign_load_off(sCn, tile, g, off);
#pragma unroll
    for (int j = 0; j < NJ; ++j) cmax[j] = assign_fold(assign_chain<NDC>(a, bop[j]), off, cmax[j]);
  }
}

// One assignment pass: label = argmin_c (|c_q|^2 - 2 v_q.c_q), lowest index on
// ties.  C^T = Cq . Vq^T runs on v_mfma_i32_32x32x32_i8 (exact int32); each
// lane folds its 16 accumulator rows of a 32-centroid tile into keys
// 128*(2 v.c - |c|^2) + (127 - row-in-chunk) = (acc << 8) + cn32 (one
// shift-add; max = lowest distance, then lowest row of the 128-centroid
// chunk; key >> 7 is the score exactly: |2 v.c - |c|^2| < 3 * 128 * 127^2 <
// 2^23, so the key fits in 31 bits), keeps a chunk's maximum only if its
// score is strictly higher than the best so far, and the two lane halves that
// share a token column are merged on (score, index).
// A workgroup covers 128 * NJW tokens (4 waves x NJW column tiles of 32);
// centroids stream through LDS in chunks of 128.
// BAL (balanced clusters, one proposal round): the acnt[bh] unplaced tokens
// listed in alist take part; full clusters carry zero codes and the offset
// INT_MIN, so they are never chosen; the kernel writes the proposal (nearest
// cluster with room, lowest index on ties) of the i-th listed token to
// prop[i] and its exact squared distance |v|^2 - score to pdist[token].
template <int D, bool BAL, int NJW>
__global__ __launch_bounds__(256, BAL ? 4 : 2) void k_kmeans_assign(const int8_t* __restrict__ Vq,
                                                       const int8_t* __restrict__ Cq,
                                                       const int32_t* __restrict__ cn32, int N,
                                                       int kpad, int32_t* __restrict__ labels,
                                                       int32_t* __restrict__ prop = nullptr,
                                                       int32_t* __restrict__ pdist = nullptr,
                                                       const int32_t* __restrict__ alist = nullptr,
                                                       const int32_t* __restrict__ acnt = nullptr) {
  constexpr int NDC = D / 32;
  constexpr int CSTR = D + 16;
  constexpr int CCH = 128;
  constexpr int WT = 128 * NJW;                 // tokens per workgroup
  __shared__ __attribute__((aligned(16))) int8_t sC[CCH * CSTR];
  __shared__ __attribute__((aligned(16))) int32_t sCn[CCH];
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5, col = lane & 31;
  const int8_t* vq = Vq + static_cast<size_t>(bh) * N * D;
  const int8_t* cq = Cq + static_cast<size_t>(bh) * kpad * D;
  const int32_t* cn = cn32 + static_cast<size_t>(bh) * kpad;
  // token of column tile j of this wave (-1: none); the wave scores its
  // first nj column tiles (wave-uniform)
  int tokj[NJW];
  int nj = NJW;
  if constexpr (BAL) {
    // the round's unplaced tokens (alist, in token order) go to the
    // workgroups WT at a time; tile c of a workgroup is wave c % 4's tile
    // c / 4, so a part-filled workgroup fills the first tiles of every wave
    const int n = acnt[bh], j0 = blockIdx.x * WT;
    if (j0 >= n) return;                                    // past the round's tokens
    const int na = min(WT, n - j0);
    nj = 0;
#pragma unroll
    for (int j = 0; j < NJW; ++j) {
      const int c = wave + 4 * j, pos = c * 32 + col;
      tokj[j] = pos < na ? alist[static_cast<size_t>(bh) * N + j0 + pos] : -1;
      nj += c * 32 < na ? 1 : 0;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NJW; ++j) {
      const int tok = blockIdx.x * WT + wave * 32 * NJW + j * 32 + col;
      tokj[j] = tok < N ? tok : -1;
    }
  }

  v4i bop[NJW][NDC];
#pragma unroll
  for (int j = 0; j < NJW; ++j) {
    const int tok = tokj[j];
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      if (tok >= 0)
        bop[j][c] = *reinterpret_cast<const v4i*>(vq + static_cast<size_t>(tok) * D + 32 * c + 16 * g);
      else
        bop[j][c] = v4i{0, 0, 0, 0};
    }
  }
  int best[NJW], bchunk[NJW];
#pragma unroll
  for (int j = 0; j < NJW; ++j) { best[j] = INT_MIN; bchunk[j] = 0; }
  static_assert(CCH == kKeyRows, "a key orders the rows of one centroid chunk");
  // Centroid chunks are prefetched into registers one chunk ahead: the
  // global loads of chunk c+1 are issued before chunk c's tiles are scored
  // and written to LDS after them.
  constexpr int PF = CCH * (D / 16) / 256;     // 16-byte pieces per thread and chunk
  static_assert(CCH * (D / 16) % 256 == 0 && CCH <= 256, "chunk pieces spread evenly over the threads");
  uint4 pf[PF];
  int32_t pfn = INT_MIN;
#pragma unroll
  for (int i = 0; i < PF; ++i) {   // chunk 0
    const int p = static_cast<int>(threadIdx.x) + 256 * i;
    const int r = p / (D / 16), q16 = p % (D / 16);
    pf[i] = r < kpad ? *reinterpret_cast<const uint4*>(cq + static_cast<size_t>(r) * D + q16 * 16) : uint4{};
  }
  if (static_cast<int>(threadIdx.x) < min(CCH, kpad)) pfn = cn[threadIdx.x];
  // nothing loaded so far may still be in flight when the chunk loop starts:
  // the compiler then sees only the prefetch of the next chunk pending inside
  // the loop and does not make every chunk's first MFMA wait for it
  __builtin_amdgcn_s_waitcnt(0);
  for (int c0 = 0; c0 < kpad; c0 += CCH) {
    const int rows = min(CCH, kpad - c0);
    __syncthreads();                 // the previous chunk's tiles are scored
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int p = static_cast<int>(threadIdx.x) + 256 * i;
      const int r = p / (D / 16), q16 = p % (D / 16);
      if (r < rows) *reinterpret_cast<uint4*>(sC + r * CSTR + q16 * 16) = pf[i];
    }
    if (static_cast<int>(threadIdx.x) < rows) sCn[threadIdx.x] = pfn;
    const int n0 = c0 + CCH, nrows = min(CCH, kpad - n0);   // next chunk (nrows <= 0: none)
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int p = static_cast<int>(threadIdx.x) + 256 * i;
      const int r = p / (D / 16), q16 = p % (D / 16);
      if (r < nrows) pf[i] = *reinterpret_cast<const uint4*>(cq + static_cast<size_t>(n0 + r) * D + q16 * 16);
    }
    if (static_cast<int>(threadIdx.x) < nrows) pfn = cn[n0 + threadIdx.x];
    __syncthreads();
    int cmax[NJW];
#pragma unroll
    for (int j = 0; j < NJW; ++j) cmax[j] = INT_MIN;
    if (nj == NJW) {
      assign_chunk<NJW, NDC, CSTR, NJW>(sC, sCn, rows / 32, bop, cmax, g, col);
    } else if constexpr (BAL) {                             // wave-uniform
      if constexpr (NJW > 3) if (nj == 3) assign_chunk<3, NDC, CSTR, NJW>(sC, sCn, rows / 32, bop, cmax, g, col);
      if constexpr (NJW > 2) if (nj == 2) assign_chunk<2, NDC, CSTR, NJW>(sC, sCn, rows / 32, bop, cmax, g, col);
      if (nj == 1) assign_chunk<1, NDC, CSTR, NJW>(sC, sCn, rows / 32, bop, cmax, g, col);
    }
    // chunks arrive in increasing index order: a later chunk must win on
    // score alone (the packed row only orders rows inside one chunk)
#pragma unroll
    for (int j = 0; j < NJW; ++j)
      if ((cmax[j] >> 7) > (best[j] >> 7)) { best[j] = cmax[j]; bchunk[j] = c0 / CCH; }
  }
#pragma unroll
  for (int j = 0; j < NJW; ++j) {
    if (j >= nj) continue;                                  // wave-uniform
    const int score = best[j] >> 7;
    const int idx = bchunk[j] * CCH + (CCH - 1 - (best[j] & (CCH - 1)));
    const int ps = __shfl_xor(score, 32, 64);
    const int pi = __shfl_xor(idx, 32, 64);
    const bool other = ps > score || (ps == score && pi < idx);
    const int lab = other ? pi : idx;
    const int tok = tokj[j];
    if constexpr (BAL) {
      // |v|^2 of the token: this lane holds half of its codes, the lane 32
      // apart the other half
      int vn = 0;
#pragma unroll
      for (int c = 0; c < NDC; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) vn = __builtin_amdgcn_sdot4(bop[j][c][q], bop[j][c][q], vn, false);
      vn += __shfl_xor(vn, 32, 64);
      if (g == 0 && tok >= 0) {
        prop[static_cast<size_t>(bh) * N + blockIdx.x * WT + (wave + 4 * j) * 32 + col] = lab;   // list position
        pdist[static_cast<size_t>(bh) * N + tok] = vn - (other ? ps : score);
      }
    } else {
      if (g == 0 && tok >= 0) labels[static_cast<size_t>(bh) * N + tok] = lab;
    }
  }
}

// ---- balanced clusters (capped assignment) ------------------------------------
// Capacities: kv_block places per cluster, the last cluster the tail of the
// sequence, so that after the stable sort every block holds one cluster.
// Per pass: rem = capacities and labels = -1; then kBalRounds rounds of
// (proposals of the unplaced tokens by k_kmeans_assign<D, true>; proposals
// grouped by cluster with the stable counting sort; k_bal_accept; the tokens
// still unplaced listed for the next round by k_bal_count and k_bal_place);
// then k_bal_fill places whatever is left in token order, clusters in index
// order.
constexpr int kBalRounds = 12;
constexpr int kBalThreads = 256;
constexpr int kAcceptPer = 8;      // proposers per thread held in registers by k_bal_accept

__global__ void k_bal_init(int N, int k, int kvb, int32_t* __restrict__ rem, int32_t* __restrict__ labels,
                           int32_t* __restrict__ alist, int32_t* __restrict__ acnt) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) {
    labels[static_cast<size_t>(bh) * N + i] = -1;
    alist[static_cast<size_t>(bh) * N + i] = i;            // every token is unplaced
  }
  if (i < k) rem[static_cast<size_t>(bh) * k + i] = i + 1 < k ? kvb : N - (k - 1) * kvb;
  if (i == 0) acnt[bh] = N;
}

// The tokens of list `in` (cin[bh] of them, token order) that are still
// unplaced after a round go, in the same order, to list `out`, and their
// number to cout[bh]: k_bal_count counts them per chunk of kSortChunk list
// entries, k_bal_place writes each chunk's behind those of the chunks before
// it.  Each thread takes kCompactPer consecutive entries of its chunk.
constexpr int kCompactThreads = 256;
constexpr int kCompactPer = kSortChunk / kCompactThreads;

// the unplaced tokens among a thread's entries of chunk ch (-1: none or placed)
__device__ __forceinline__ int bal_survivors(const int32_t* li, const int32_t* lab, int n, int ch,
                                             int (&tok)[kCompactPer]) {
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < kCompactPer; ++e) {
    const int j = ch * kSortChunk + static_cast<int>(threadIdx.x) * kCompactPer + e;
    tok[e] = j < n ? li[j] : -1;
  }
#pragma unroll
  for (int e = 0; e < kCompactPer; ++e) {
    if (tok[e] >= 0 && lab[tok[e]] >= 0) tok[e] = -1;         // placed
    cnt += tok[e] >= 0 ? 1 : 0;
  }
  return cnt;
}

__global__ __launch_bounds__(kCompactThreads) void k_bal_count(const int32_t* __restrict__ in,
                                                               const int32_t* __restrict__ cin,
                                                               const int32_t* __restrict__ labels, int N,
                                                               int nch, int32_t* __restrict__ ccnt) {
  __shared__ int red[kCompactThreads / 64];
  const int bh = blockIdx.y, ch = blockIdx.x;
  const int n = cin[bh];
  int tok[kCompactPer];
  int cnt = ch * kSortChunk < n ? bal_survivors(in + static_cast<size_t>(bh) * N,
                                                 labels + static_cast<size_t>(bh) * N, n, ch, tok) : 0;
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < kCompactThreads / 64; ++w) t += red[w];
    ccnt[static_cast<size_t>(bh) * nch + ch] = t;
  }
}

__global__ __launch_bounds__(kCompactThreads) void k_bal_place(const int32_t* __restrict__ in,
                                                               const int32_t* __restrict__ cin,
                                                               const int32_t* __restrict__ labels, int N,
                                                               int nch, const int32_t* __restrict__ ccnt,
                                                               int32_t* __restrict__ out,
                                                               int32_t* __restrict__ cout) {
  __shared__ int part[kCompactThreads / 64];
  const int bh = blockIdx.y, ch = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n = cin[bh];
  const int32_t* cc = ccnt + static_cast<size_t>(bh) * nch;
  if (ch == 0 && t == 0) {
    int tot = 0;
    for (int c = 0; c < nch; ++c) tot += cc[c];
    cout[bh] = tot;
  }
  if (ch * kSortChunk >= n) return;
  int base = 0;                                   // survivors of the chunks before this one
  for (int c = lane; c < ch; c += 64) base += cc[c];
  for (int o = 32; o > 0; o >>= 1) base += __shfl_xor(base, o, 64);
  int tok[kCompactPer];
  const int cnt = bal_survivors(in + static_cast<size_t>(bh) * N, labels + static_cast<size_t>(bh) * N, n, ch, tok);
  int incl = cnt;                                 // inclusive scan in the wave
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  int pos = base + incl - cnt;
  for (int w = 0; w < wave; ++w) pos += part[w];
  int32_t* lo = out + static_cast<size_t>(bh) * N;
#pragma unroll
  for (int e = 0; e < kCompactPer; ++e)
    if (tok[e] >= 0) lo[pos++] = tok[e];
}

// sum of v over the workgroup (every thread gets it)
__device__ __forceinline__ int bal_block_sum(int v, int* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < kBalThreads / 64; ++w) t += red[w];
  return t;
}

// maximum of v over the workgroup (every thread gets it)
__device__ __forceinline__ int bal_block_max(int v, int* red) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int m = red[0];
  for (int w = 1; w < kBalThreads / 64; ++w) m = max(m, red[w]);
  return m;
}

// Cluster c (one workgroup) takes the rem_c nearest of its proposers (by
// exact squared distance, ties to the lowest token index; the proposers
// arrive in token order); a cluster that fills up gets zero codes and the
// offset INT_MIN, so the next rounds never propose to it.
template <int D>
__global__ __launch_bounds__(kBalThreads) void k_bal_accept(const int32_t* __restrict__ list_all,
                                                            const int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ starts,
                                                            const int32_t* __restrict__ pdist, int N, int k,
                                                            int kpad, int32_t* __restrict__ rem,
                                                            int32_t* __restrict__ labels, int8_t* __restrict__ Cq,
                                                            int32_t* __restrict__ cn32) {
  __shared__ int red[kBalThreads / 64];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int cnt = counts[static_cast<size_t>(bh) * k + c];
  int r = rem[static_cast<size_t>(bh) * k + c];
  if (cnt == 0 || r == 0) return;
  const int32_t* list = list_all + static_cast<size_t>(bh) * N + starts[static_cast<size_t>(bh) * k + c];
  const int32_t* dist = pdist + static_cast<size_t>(bh) * N;
  int32_t* lab = labels + static_cast<size_t>(bh) * N;
  if (cnt <= r) {
    for (int i = t; i < cnt; i += kBalThreads) lab[list[i]] = c;
    r -= cnt;
  } else if (cnt <= kAcceptPer * kBalThreads) {
    // the same selection with the proposers' tokens and distances held in
    // registers (proposer i: thread i % kBalThreads, slot i / kBalThreads),
    // so the binary search does not gather them again at every step
    int tk[kAcceptPer], dv[kAcceptPer];
#pragma unroll
    for (int e = 0; e < kAcceptPer; ++e) {
      const int i = e * kBalThreads + t;
      tk[e] = i < cnt ? list[i] : -1;
    }
#pragma unroll
    for (int e = 0; e < kAcceptPer; ++e) dv[e] = tk[e] >= 0 ? dist[tk[e]] : INT_MAX;
    int lo = INT_MAX, hi = INT_MIN;
#pragma unroll
    for (int e = 0; e < kAcceptPer; ++e)
      if (tk[e] >= 0) {
        lo = min(lo, dv[e]);
        hi = max(hi, dv[e]);
      }
    lo = -bal_block_max(-lo, red);
    hi = bal_block_max(hi, red);
    while (lo < hi) {                                   // uniform across the workgroup
      const int mid = lo + (hi - lo) / 2;
      int n = 0;
#pragma unroll
      for (int e = 0; e < kAcceptPer; ++e) n += tk[e] >= 0 && dv[e] <= mid ? 1 : 0;
      if (bal_block_sum(n, red) >= r) hi = mid;
      else lo = mid + 1;
    }
    const int theta = lo;
    int nl = 0;
#pragma unroll
    for (int e = 0; e < kAcceptPer; ++e) nl += tk[e] >= 0 && dv[e] < theta ? 1 : 0;
    const int need = r - bal_block_sum(nl, red);       // >= 1 proposers at distance theta, in token order
    const int lane = t & 63, wave = t >> 6;
    int run = 0;
#pragma unroll
    for (int e = 0; e < kAcceptPer; ++e) {
      if (e * kBalThreads >= cnt) break;                // uniform
      const bool eq = tk[e] >= 0 && dv[e] == theta;
      const uint64_t bal = __ballot(eq);
      __syncthreads();
      if (lane == 0) red[wave] = __popcll(bal);
      __syncthreads();
      int before = run + __popcll(bal & ((1ull << lane) - 1ull));
      for (int w = 0; w < wave; ++w) before += red[w];
      if (tk[e] >= 0 && (dv[e] < theta || (eq && before < need))) lab[tk[e]] = c;
      for (int w = 0; w < kBalThreads / 64; ++w) run += red[w];
    }
    r = 0;
  } else {
    // theta = the r-th smallest distance: the smallest value with
    // #(dist <= theta) >= r (binary search over the exact integers)
    int lo = INT_MAX, hi = INT_MIN;
    for (int i = t; i < cnt; i += kBalThreads) {
      const int dv = dist[list[i]];
      lo = min(lo, dv);
      hi = max(hi, dv);
    }
    lo = -bal_block_max(-lo, red);
    hi = bal_block_max(hi, red);
    while (lo < hi) {                                   // uniform across the workgroup
      const int mid = lo + (hi - lo) / 2;
      int n = 0;
      for (int i = t; i < cnt; i += kBalThreads) n += dist[list[i]] <= mid;
      if (bal_block_sum(n, red) >= r) hi = mid;
      else lo = mid + 1;
    }
    const int theta = lo;
    int nl = 0;
    for (int i = t; i < cnt; i += kBalThreads) nl += dist[list[i]] < theta;
    const int need = r - bal_block_sum(nl, red);       // >= 1 proposers at distance theta, in token order
    const int lane = t & 63, wave = t >> 6;
    int run = 0;
    for (int base = 0; base < cnt; base += kBalThreads) {
      const int i = base + t;
      const int dv = i < cnt ? dist[list[i]] : INT_MAX;
      const bool eq = dv == theta;
      const uint64_t bal = __ballot(eq);
      __syncthreads();
      if (lane == 0) red[wave] = __popcll(bal);
      __syncthreads();
      int before = run + __popcll(bal & ((1ull << lane) - 1ull));
      for (int w = 0; w < wave; ++w) before += red[w];
      if (i < cnt && (dv < theta || (eq && before < need))) lab[list[i]] = c;
      for (int w = 0; w < kBalThreads / 64; ++w) run += red[w];
    }
    r = 0;
  }
  __syncthreads();
  if (t == 0) rem[static_cast<size_t>(bh) * k + c] = r;
  if (r == 0) {
    int8_t* row = Cq + (static_cast<size_t>(bh) * kpad + c) * D;
    for (int i = t; i < D / 4; i += kBalThreads) reinterpret_cast<int32_t*>(row)[i] = 0;
    if (t == 0) cn32[static_cast<size_t>(bh) * kpad + c] = INT_MIN;
  }
}

// Tokens left after the rounds (the ucnt[bh] of list ul, token order) take
// the remaining places: the u-th goes to the cluster holding place u when the
// clusters' remaining places are laid out in index order.
constexpr int kFillThreads = 1024;
__global__ __launch_bounds__(kFillThreads) void k_bal_fill(const int32_t* __restrict__ rem, int N, int k,
                                                           const int32_t* __restrict__ ul,
                                                           const int32_t* __restrict__ ucnt,
                                                           int32_t* __restrict__ labels) {
  constexpr int PER = kMaxClusters / kFillThreads;
  __shared__ int cum[kMaxClusters];
  __shared__ int part[kFillThreads];
  const int bh = blockIdx.x, t = threadIdx.x;
  const int n = ucnt[bh];
  if (n == 0) return;
  int32_t* lab = labels + static_cast<size_t>(bh) * N;
  const int32_t* list = ul + static_cast<size_t>(bh) * N;
  // cum = exclusive prefix sum of rem over the clusters (PER per thread, then
  // an inclusive Hillis-Steele scan of the per-thread totals)
  int mine[PER];
  int tot = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = t * PER + e;
    mine[e] = c < k ? rem[static_cast<size_t>(bh) * k + c] : 0;
    tot += mine[e];
  }
  part[t] = tot;
  __syncthreads();
  for (int o = 1; o < kFillThreads; o <<= 1) {
    const int v = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int acc = part[t] - tot;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    cum[t * PER + e] = acc;
    acc += mine[e];
  }
  __syncthreads();
  for (int u = t; u < n; u += kFillThreads) {
    int a = 0, b = k - 1;                     // the last cluster with cum <= u
    while (a < b) {
      const int m = (a + b + 1) / 2;
      if (cum[m] <= u) a = m;
      else b = m - 1;
    }
    lab[list[u]] = a;
  }
}

// ---- stable counting sort by label ------------------------------------------------
// Keys outside [0, k) are left out.  With ncnt, only the first ncnt[bh] keys of
// a head take part (the chunks past them are skipped; chunk 0 always counts,
// so a head without keys gets zero counts); with ids, key i belongs to token
// ids[i] (the keys come in token order), which is what perm receives.
__global__ __launch_bounds__(256) void k_sort_hist(const int32_t* __restrict__ labels, int N, int k,
                                                   int nch, int32_t* __restrict__ hist,
                                                   const int32_t* __restrict__ ncnt) {
  __shared__ int32_t cnt[kMaxClusters];
  const int bh = blockIdx.y, ch = blockIdx.x;
  const int n = ncnt ? min(N, ncnt[bh]) : N;       // keys in use
  if (n > 0 && ch * kSortChunk >= n) return;       // a chunk past them (chunk 0 always counts)
  for (int i = threadIdx.x; i < k; i += 256) cnt[i] = 0;
  __syncthreads();
  const int t0 = ch * kSortChunk, t1 = min(n, t0 + kSortChunk);
  for (int t = t0 + threadIdx.x; t < t1; t += 256) {
    const int L = labels[static_cast<size_t>(bh) * N + t];
    if (static_cast<unsigned>(L) < static_cast<unsigned>(k)) atomicAdd(&cnt[L], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += 256)
    hist[(static_cast<size_t>(bh) * nch + ch) * k + i] = cnt[i];
}

// hist[ch][L] <- first sorted position of chunk ch's tokens with label L;
// counts[L] = cluster size, starts[L] = first sorted position of cluster L.
// Thread t owns labels t, t + 1024, ... (consecutive threads read consecutive
// words of a chunk's row); each label's chunk counts are read in batches of
// eight before they are added, so the loads overlap.  The label prefix is
// one workgroup scan per group of 1024 labels, in label order.
__global__ __launch_bounds__(1024) void k_sort_scan(int32_t* __restrict__ hist, int k, int nch_all,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ starts,
                                                    const int32_t* __restrict__ ncnt) {
  constexpr int PER = kMaxClusters / 1024;
  constexpr int CB = 8;                        // chunk counts read per batch
  __shared__ int32_t part[1024];
  const int bh = blockIdx.x;
  const int nch = ncnt ? max(1, min(nch_all, (ncnt[bh] + kSortChunk - 1) / kSortChunk)) : nch_all;   // chunks in use
  int32_t* h = hist + static_cast<size_t>(bh) * nch_all * k;
  int tot[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int L = e * 1024 + static_cast<int>(threadIdx.x);
    int run = 0;
    if (L < k) {
      for (int c0 = 0; c0 < nch; c0 += CB) {
        int v[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u) v[u] = c0 + u < nch ? h[static_cast<size_t>(c0 + u) * k + L] : 0;
#pragma unroll
        for (int u = 0; u < CB; ++u) {
          if (c0 + u < nch) h[static_cast<size_t>(c0 + u) * k + L] = run;
          run += v[u];
        }
      }
    }
    tot[e] = run;
  }
  int base = 0;                                // labels of the earlier groups
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (e * 1024 >= k) break;                  // uniform: k is a kernel argument
    part[threadIdx.x] = tot[e];
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {       // inclusive Hillis-Steele scan
      const int v = static_cast<int>(threadIdx.x) >= o ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    const int run = base + part[threadIdx.x] - tot[e];   // exclusive prefix of label L
    const int L = e * 1024 + static_cast<int>(threadIdx.x);
    if (L < k) {
      counts[static_cast<size_t>(bh) * k + L] = tot[e];
      starts[static_cast<size_t>(bh) * k + L] = run;
      for (int c0 = 0; c0 < nch; c0 += CB) {
        int v[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u) v[u] = c0 + u < nch ? h[static_cast<size_t>(c0 + u) * k + L] : 0;
#pragma unroll
        for (int u = 0; u < CB; ++u)
          if (c0 + u < nch) h[static_cast<size_t>(c0 + u) * k + L] = v[u] + run;
      }
    }
    base += part[1023];
    __syncthreads();                           // part is rewritten by the next group
  }
}

// Tokens of a chunk are placed in token order.  Each of the 4 waves owns a
// contiguous quarter of the chunk, whose labels (and token ids) it loads into
// registers at once: per-wave label counts (LDS) prefixed across the waves
// give each wave its own base per label, and the wave then walks its quarter
// 64 tokens at a time, ranking a token among the round's equal labels by
// matching label bits with ballots (the lanes whose label equals this
// lane's, below it) and advancing its bases.
__global__ __launch_bounds__(256) void k_sort_scatter(const int32_t* __restrict__ labels,
                                                      const int32_t* __restrict__ hist, int N,
                                                      int k, int nch, int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ ncnt) {
  constexpr int QW = kSortChunk / 4;            // tokens per wave
  constexpr int NR = QW / 64;                   // rounds of 64 per wave
  __shared__ int32_t base[4][kMaxClusters];
  const int bh = blockIdx.y, ch = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = ncnt ? min(N, ncnt[bh]) : N;
  if (ch * kSortChunk >= n) return;              // no key in this chunk
  const int t0 = ch * kSortChunk, t1 = min(n, t0 + kSortChunk);
  const int w0 = t0 + wave * QW, w1 = min(t1, w0 + QW);
  const int32_t* lab = labels + static_cast<size_t>(bh) * N;
  int key[NR], tok[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int t = w0 + 64 * i + lane;
    int L = t < w1 ? lab[t] : -1;
    if (static_cast<unsigned>(L) >= static_cast<unsigned>(k)) L = -1;   // out-of-range labels are dropped
    key[i] = L;
    tok[i] = ids && L >= 0 ? ids[static_cast<size_t>(bh) * N + t] : t;
  }
  for (int i = threadIdx.x; i < 4 * k; i += 256) base[i / k][i % k] = 0;   // the k labels in use
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NR; ++i)
    if (key[i] >= 0) atomicAdd(&base[wave][key[i]], 1);
  __syncthreads();
  for (int L = threadIdx.x; L < k; L += 256) {
    int run = hist[(static_cast<size_t>(bh) * nch + ch) * k + L];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = base[w][L];
      base[w][L] = run;
      run += c;
    }
  }
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) < k) ++nbits;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int L = key[i];
    uint64_t same = __ballot(L >= 0);
    if (same == 0) continue;                     // no label to place in these 64 tokens (wave-uniform)
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (L >> bit) & 1;
      const uint64_t m = __ballot(on);
      same &= on ? m : ~m;
    }
    const int before = __popcll(same & below);
    const int total = __popcll(same);
    int pos = 0;
    if (L >= 0) pos = base[wave][L];
    if (L >= 0) perm[static_cast<size_t>(bh) * N + pos + before] = tok[i];
    if (L >= 0 && before == total - 1) base[wave][L] = pos + total;
  }
}

// New centroid = fp32(fp64 mean of the members' values), summed in sorted
// (= token) order; an empty cluster keeps its centroid.  One wave per cluster:
// lane t owns channels CPL*t .. CPL*t + CPL - 1 (CPL = D / 64) and reads them
// with one 2- or 4-byte load per member row, so a wave instruction covers a
// whole 2D-byte row.  Members come in chunks of U: the chunk's U row loads are
// all issued before its additions, which stay in member order.
template <int D>
__global__ __launch_bounds__(64) void k_kmeans_update(const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ starts, int N, int k,
                                                      float* __restrict__ C) {
  constexpr int CPL = D / 64;
  constexpr int U = 32;
  static_assert(CPL == 1 || CPL == 2, "64 or 128 channels");
  const int bh = blockIdx.y, i = blockIdx.x, t = threadIdx.x;
  const int cnt = counts[static_cast<size_t>(bh) * k + i];
  if (cnt == 0) return;
  const int s = starts[static_cast<size_t>(bh) * k + i];
  const int32_t* pp = perm + static_cast<size_t>(bh) * N + s;
  const uint16_t* vv = V + static_cast<size_t>(bh) * N * D + CPL * t;
  double sum[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) sum[c] = 0.0;
  auto row = [&](int j) -> uint32_t {
    const uint16_t* r = vv + static_cast<size_t>(pp[j]) * D;
    if constexpr (CPL == 2) return *reinterpret_cast<const uint32_t*>(r);
    else return *r;
  };
  auto add = [&](uint32_t x) {
    sum[0] += static_cast<double>(bf16_to_f32(static_cast<uint16_t>(x & 0xffffu)));
    if constexpr (CPL == 2) sum[1] += static_cast<double>(bf16_to_f32(static_cast<uint16_t>(x >> 16)));
  };
  int j = 0;
  for (; j + U <= cnt; j += U) {
    uint32_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = row(j + u);
#pragma unroll
    for (int u = 0; u < U; ++u) add(x[u]);
  }
  for (; j + 8 <= cnt; j += 8) {
    uint32_t x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = row(j + u);
#pragma unroll
    for (int u = 0; u < 8; ++u) add(x[u]);
  }
  for (; j < cnt; ++j) add(row(j));
  float* out = C + (static_cast<size_t>(bh) * k + i) * D + CPL * t;
#pragma unroll
  for (int c = 0; c < CPL; ++c) out[c] = static_cast<float>(sum[c] / static_cast<double>(cnt));
}

__global__ void k_iota(int32_t* __restrict__ perm, int N, size_t total) {
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < total) perm[i] = static_cast<int32_t>(i % N);
}

// A permutation entry as a row index: a caller-supplied permutation with an
// entry outside [0, N) reads row 0 instead of memory outside the head.
__device__ __forceinline__ int clamp_tok(int t, int N) { return static_cast<unsigned>(t) < static_cast<unsigned>(N) ? t : 0; }

// ---- V-Smooth residuals -----------------------------------------------------------
// A workgroup owns one block.  Thread (cg, q) holds channels 8cg..8cg+7 of
// the sorted positions 4q..4q+3 (+ 4*RQ per pass), read as whole 16-byte
// pieces of the gathered rows and kept in registers.
template <int D, int KVB>
struct BlockRows {
  static constexpr int CG = D / 8;            // channel groups of 8
  static constexpr int RQ = 256 / CG;         // 4-row quads covered per pass
  static constexpr int PASS = (KVB / 4 + RQ - 1) / RQ;
  float v[PASS][4][8];
  // the 16-byte piece of pass ps, row rr of the quad (zeros past the block)
  static __device__ __forceinline__ uint4 piece(const uint16_t* vv, const int32_t* pp, int p0, int N, int ps,
                                                int rr) {
    const int cg = threadIdx.x % CG, q = threadIdx.x / CG;
    const int r = (ps * RQ + q) * 4 + rr;
    const int pos = p0 + r;
    uint4 raw = make_uint4(0u, 0u, 0u, 0u);
    if (r < KVB && pos < N) raw = *reinterpret_cast<const uint4*>(vv + static_cast<size_t>(clamp_tok(pp[pos], N)) * D + cg * 8);
    return raw;
  }
  __device__ __forceinline__ void load(const uint16_t* vv, const int32_t* pp, int p0, int N) {
#pragma unroll
    for (int ps = 0; ps < PASS; ++ps)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint4 raw = piece(vv, pp, p0, N, ps, rr);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[ps][rr][e] = bf16_to_f32(static_cast<uint16_t>(w[e >> 1] >> ((e & 1) * 16)));
      }
  }
};

// The same rows kept as packed bf16 (half the registers of BlockRows) and
// widened on each use, for kernels that read every value twice.
template <int D, int KVB>
struct BlockRowsPacked {
  using BR = BlockRows<D, KVB>;
  static constexpr int CG = BR::CG, RQ = BR::RQ, PASS = BR::PASS;
  uint32_t w[PASS][4][4];
  __device__ __forceinline__ void load(const uint16_t* vv, const int32_t* pp, int p0, int N) {
#pragma unroll
    for (int ps = 0; ps < PASS; ++ps)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint4 raw = BR::piece(vv, pp, p0, N, ps, rr);
        w[ps][rr][0] = raw.x; w[ps][rr][1] = raw.y; w[ps][rr][2] = raw.z; w[ps][rr][3] = raw.w;
      }
  }
  __device__ __forceinline__ float at(int ps, int rr, int e) const {
    return bf16_to_f32(static_cast<uint16_t>(w[ps][rr][e >> 1] >> ((e & 1) * 16)));
  }
};

// Block mean over the block's real tokens (fp64) and, for E4M3, the
// per-channel max |v - mean| of the head.
template <int D, int KVB>
__global__ __launch_bounds__(256) void k_vblock_stats(const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                      int N, int nblk, int vsmooth, int want_amax,
                                                      float* __restrict__ v_mean, uint32_t* __restrict__ vramax) {
  using BR = BlockRowsPacked<D, KVB>;
  // per-quad partial sums (fp64), then, once the mean is published, the
  // per-quad maxima |v - mean| in the same memory
  __shared__ double sPart[BR::RQ][D];
  __shared__ float sMean[D];
  float (*sAm)[D] = reinterpret_cast<float (*)[D]>(&sPart[0][0]);
  const int bh = blockIdx.y, b = blockIdx.x;
  const int p0 = b * KVB, nv = min(KVB, N - p0);
  const int cg = threadIdx.x % BR::CG, q = threadIdx.x / BR::CG;
  BR rows;
  rows.load(V + static_cast<size_t>(bh) * N * D, perm + static_cast<size_t>(bh) * N, p0, N);
  if (vsmooth) {
    double ps[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int pass = 0; pass < BR::PASS; ++pass)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int e = 0; e < 8; ++e) ps[e] += static_cast<double>(rows.at(pass, rr, e));   // padded rows hold 0
#pragma unroll
    for (int e = 0; e < 8; ++e) sPart[q][cg * 8 + e] = ps[e];
    __syncthreads();
    if (threadIdx.x < D) {
      double sm = 0.0;
      for (int j = 0; j < BR::RQ; ++j) sm += sPart[j][threadIdx.x];
      sMean[threadIdx.x] = static_cast<float>(sm / static_cast<double>(nv));
    }
  } else if (threadIdx.x < D) {
    sMean[threadIdx.x] = 0.0f;
  }
  __syncthreads();
  if (threadIdx.x < D) v_mean[(static_cast<size_t>(bh) * nblk + b) * D + threadIdx.x] = sMean[threadIdx.x];
  if (!want_amax) return;
  float am[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int pass = 0; pass < BR::PASS; ++pass)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = (pass * BR::RQ + q) * 4 + rr;
      if (r < nv) {
#pragma unroll
        for (int e = 0; e < 8; ++e) am[e] = fmaxf(am[e], fabsf(rows.at(pass, rr, e) - sMean[cg * 8 + e]));
      }
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) sAm[q][cg * 8 + e] = am[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float m = 0.0f;
    for (int j = 0; j < BR::RQ; ++j) m = fmaxf(m, sAm[j][threadIdx.x]);
    atomicMax(vramax + static_cast<size_t>(bh) * D + threadIdx.x, __float_as_uint(m));
  }
}

// E4M3 residual codes with the per-channel scale s_v = fp32(max|r| / 448),
// transposed through LDS into the [Np/64][d][64] layout.
template <int D, int KVB>
__global__ __launch_bounds__(256) void k_vres_e4m3(const uint16_t* __restrict__ V,
                                                   const int32_t* __restrict__ perm,
                                                   const float* __restrict__ v_mean,
                                                   const uint32_t* __restrict__ vramax, int N, int nblk,
                                                   uint8_t* __restrict__ Vres, float* __restrict__ v_scale) {
  using BR = BlockRows<D, KVB>;
  __shared__ float sMean[D];
  __shared__ float sS[D];
  __shared__ float sY[D];           // fp32(1 / scale)
  __shared__ __attribute__((aligned(16))) uint32_t sT[D][KVB / 4 + 1];   // codes [channel][position/4]
  const int bh = blockIdx.y, b = blockIdx.x;
  const int p0 = b * KVB;
  const int cg = threadIdx.x % BR::CG, q = threadIdx.x / BR::CG;
  if (threadIdx.x < D) {
    const float am = __uint_as_float(vramax[static_cast<size_t>(bh) * D + threadIdx.x]);
    const float sc = am > 0.0f ? fmaxf(am / 448.0f, kScaleFloor) : 1.0f;
    sS[threadIdx.x] = sc;
    sY[threadIdx.x] = 1.0f / sc;
    sMean[threadIdx.x] = v_mean[(static_cast<size_t>(bh) * nblk + b) * D + threadIdx.x];
    if (b == 0) v_scale[static_cast<size_t>(bh) * D + threadIdx.x] = sc;
  }
  BR rows;
  rows.load(V + static_cast<size_t>(bh) * N * D, perm + static_cast<size_t>(bh) * N, p0, N);
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < BR::PASS; ++pass) {
    const int r4 = pass * BR::RQ + q;            // quad index (positions 4r4..4r4+3)
    if (r4 * 4 < KVB) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = cg * 8 + e;
        const float mc = sMean[c], sc = sS[c], yc = sY[c];
        float qv[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int pos = p0 + r4 * 4 + rr;
          qv[rr] = pos < N ? div_rn(rows.v[pass][rr][e] - mc, sc, yc) : 0.0f;
        }
        sT[c][r4] = e4m3x4(qv[0], qv[1], qv[2], qv[3]);
      }
    }
  }
  __syncthreads();
  // output: per 64-position step, D rows of 64 bytes = 16 words per channel
  uint32_t* out = reinterpret_cast<uint32_t*>(Vres + (static_cast<size_t>(bh) * nblk * KVB + p0) * D);
  for (int i = threadIdx.x; i < (KVB / 64) * D * 4; i += 256) {   // 16-byte pieces
    const int step = i / (D * 4), rem = i % (D * 4), c = rem / 4, part = rem % 4;
    const uint32_t* src = &sT[c][step * 16 + part * 4];
    *reinterpret_cast<uint4*>(out + (static_cast<size_t>(step) * D + c) * 16 + part * 4) =
        make_uint4(src[0], src[1], src[2], src[3]);
  }
}

// MX residuals of one block, per 32 sorted positions x channel:
//   FMT 1, MXFP4: E8M0 exponent floor(log2 amax) - 2 (OCP MX rule), E2M1 codes
//     of r / 2^e; layout [Np/64][d][32 bytes], even position in the low nibble;
//   FMT 2, MXFP8: E8M0 exponent e, the smallest integer with amax <= 448 * 2^e
//     (no element saturates), E4M3 codes of r / 2^e (round to nearest even);
//     layout as the E4M3 residuals, [Np/64][d][64 bytes];
//   FMT 3, NVFP4-style residuals (the zerohour.day summary's key facts name
//     NVFP4 for the 4-bit residuals), in the exact form the FP8 matrix core takes:
//     the head's second-level scale 2^t (smallest t with max|r| <= 6*448*2^t),
//     per 16 positions x channel the E4M3 block scale
//     s16 = E4M3(fp32(amax16 / (6 * 2^t))) and E2M1 elements
//     q = E2M1(fp32(r / (s16 * 2^t))) (zeros where s16 rounds to 0).  The
//     value v = q * s16 has at most six significant bits; per 32 positions
//     e is the smallest integer with max|v| <= 448 * 2^e, and v / 2^e is
//     stored as two E4M3 codes, high = E4M3(v / 2^e) and
//     low = E4M3(v / 2^e - high), with the E8M0 byte e + t + 127.  Per block
//     all high codes ([KVB/64][d][64 bytes]), then all low codes.
// Exponents are clamped to E8M0's range (0 for an all-zero group); scales are
// stored in lane order (mx_scale_slot).  Rows are gathered whole by
// BlockRows; the group maxima meet in LDS (max of the fp32 bit patterns of
// |r|), then every thread encodes its values into a code tile in LDS, which
// is written out in 16-byte pieces.
template <int D, int KVB, int FMT>
__global__ __launch_bounds__(256) void k_vres_mx(const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                 const float* __restrict__ v_mean,
                                                 const uint32_t* __restrict__ vramax, int N, int nblk,
                                                 uint8_t* __restrict__ Vres, uint8_t* __restrict__ e8m0) {
  using BR = BlockRows<D, KVB>;
  constexpr bool NV = FMT == 3;
  constexpr int NG = KVB / 32;                       // scale groups per block
  constexpr int NA = NV ? KVB / 16 : NG;             // amax groups (16 positions for FMT 3)
  __shared__ float sMean[D];
  __shared__ uint32_t sAm[NA][D];
  __shared__ int sE[NG][D];
  __shared__ float sDen[NV ? NA : 1][D];             // FMT 3: s16 * 2^t per 16-position block
  __shared__ int sTx;                                 // FMT 3: t
  __shared__ __attribute__((aligned(16))) uint32_t sT[D][KVB / 4 + 1];   // codes [channel][position/4]
  __shared__ __attribute__((aligned(16))) uint32_t sT2[NV ? D : 1][KVB / 4 + 1];   // FMT 3: low codes
  const int bh = blockIdx.y, b = blockIdx.x;
  const int p0 = b * KVB;
  const int cg = threadIdx.x % BR::CG, q = threadIdx.x / BR::CG;
  for (int i = threadIdx.x; i < NA * D; i += 256) (&sAm[0][0])[i] = 0u;
  if (threadIdx.x < D) sMean[threadIdx.x] = v_mean[(static_cast<size_t>(bh) * nblk + b) * D + threadIdx.x];
  if constexpr (NV) {
    if (threadIdx.x < 64) {
      float m = 0.0f;
      for (int c = threadIdx.x; c < D; c += 64) m = fmaxf(m, __uint_as_float(vramax[static_cast<size_t>(bh) * D + c]));
      m = wave_max(m);
      if (threadIdx.x == 0) {
        int t = 0;
        if (m > 0.0f) {
          int fe;
          frexpf(m, &fe);                  // m = f * 2^fe, f in [0.5, 1); 2688 * 2^(fe-12) = 1.3125 * 2^(fe-1)
          t = fe - 12;
          if (m > ldexpf(2688.0f, t)) ++t;
          t = max(t, -126);   // 2^t stays a normal fp32
        }
        sTx = t;
      }
    }
  }
  BR rows;
  rows.load(V + static_cast<size_t>(bh) * N * D, perm + static_cast<size_t>(bh) * N, p0, N);
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < BR::PASS; ++pass) {
    const int r4 = pass * BR::RQ + q;
    if (r4 * 4 < KVB) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = cg * 8 + e;
        float am = 0.0f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float x = p0 + r4 * 4 + rr < N ? rows.v[pass][rr][e] - sMean[c] : 0.0f;
          rows.v[pass][rr][e] = x;
          am = fmaxf(am, fabsf(x));
        }
        atomicMax(&sAm[NV ? r4 / 4 : r4 / 8][c], __float_as_uint(am));
      }
    }
  }
  __syncthreads();
  if constexpr (NV) {
    // block scales, and each 16-position block's largest |q * s16| (the
    // quotient and E2M1 rounding are monotone, so it is the maximum's)
    const float st = ldexpf(1.0f, sTx);
    for (int i = threadIdx.x; i < NA * D; i += 256) {
      const int sub = i / D, c = i % D;
      const float am = __uint_as_float(sAm[sub][c]);
      const float s16 = e4m3_value(e4m3_encode(am / (6.0f * st)));
      const float den = s16 * st;
      sDen[sub][c] = den;
      const float vm = den > 0.0f ? fabsf(e2m1_value(e2m1_encode(am / den))) * s16 : 0.0f;
      sAm[sub][c] = __float_as_uint(vm);
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < NG * D; i += 256) {
    const int grp = i / D, c = i % D;
    const float am = NV ? fmaxf(__uint_as_float(sAm[2 * grp][c]), __uint_as_float(sAm[2 * grp + 1][c]))
                        : __uint_as_float(sAm[grp][c]);
    int ex = 0;
    if (am > 0.0f) {
      int fe;
      frexpf(am, &fe);                   // am = f * 2^fe, f in [0.5, 1)
      if constexpr (FMT == 1) {
        ex = fe - 1 - 2;
      } else {
        ex = fe - 1 - 8;
        if (am > ldexpf(448.0f, ex)) ++ex;
      }
      ex = min(max(ex, -127), 127);
    }
    sE[grp][c] = ex;
    const int byte = NV ? min(max(ex + sTx + 127, 0), 254) : ex + 127;
    e8m0[(static_cast<size_t>(bh) * (nblk * KVB / 32) + p0 / 32 + grp) * D + mx_scale_slot<D>(c)] =
        static_cast<uint8_t>(byte);
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < BR::PASS; ++pass) {
    const int r4 = pass * BR::RQ + q;
    if (r4 * 4 < KVB) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = cg * 8 + e;
        const int ex = sE[r4 / 8][c];
        if constexpr (NV) {
          const float den = sDen[r4 / 4][c];
          const float s16 = ldexpf(den, -sTx);
          float y[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float xq = den > 0.0f ? rows.v[pass][rr][e] / den : 0.0f;
            y[rr] = ldexpf(e2m1_value(e2m1_encode(xq)) * s16, -ex);    // exact; |y| <= 448
          }
          const uint32_t hi = e4m3x4(y[0], y[1], y[2], y[3]);
          float l[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) l[rr] = y[rr] - e4m3_value((hi >> (8 * rr)) & 0xffu);
          sT[c][r4] = hi;
          sT2[c][r4] = e4m3x4(l[0], l[1], l[2], l[3]);
        } else {
          float x[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) x[rr] = ldexpf(rows.v[pass][rr][e], -ex);
          if constexpr (FMT == 1) {
            sT[c][r4] = e2m1_encode(x[0]) | (e2m1_encode(x[1]) << 4) | (e2m1_encode(x[2]) << 8) |
                        (e2m1_encode(x[3]) << 12);
          } else {
            // |x| <= 448 unless the exponent clamp binds; the clamp keeps the
            // hardware convert (which does not saturate) finite then
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) x[rr] = fminf(fmaxf(x[rr], -448.0f), 448.0f);
            sT[c][r4] = e4m3x4(x[0], x[1], x[2], x[3]);
          }
        }
      }
    }
  }
  __syncthreads();
  if constexpr (FMT == 1) {
    // [Np/64][D][32 bytes]: 16 quads of 2 bytes per channel row
    uint8_t* out = Vres + (static_cast<size_t>(bh) * nblk * KVB + p0) * D / 2;
    for (int i = threadIdx.x; i < (KVB / 64) * D * 2; i += 256) {   // 16-byte pieces
      const int step = i / (D * 2), rem = i % (D * 2), c = rem / 2, part = rem % 2;
      const uint32_t* src = &sT[c][step * 16 + part * 8];
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = (src[2 * k] & 0xffffu) | (src[2 * k + 1] << 16);
      *reinterpret_cast<uint4*>(out + (static_cast<size_t>(step) * D + c) * 32 + part * 16) =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    // as the E4M3 residuals: per 64-position step, D rows of 64 bytes (FMT 3:
    // the high codes, then the low codes)
    constexpr int NSET = NV ? 2 : 1;
    uint32_t* out = reinterpret_cast<uint32_t*>(Vres + (static_cast<size_t>(bh) * nblk * KVB + p0) * D * NSET);
    for (int i = threadIdx.x; i < NSET * (KVB / 64) * D * 4; i += 256) {
      const int set = i / ((KVB / 64) * D * 4), j = i % ((KVB / 64) * D * 4);
      const int step = j / (D * 4), rem = j % (D * 4), c = rem / 4, part = rem % 4;
      const uint32_t* src = set == 0 ? &sT[c][step * 16 + part * 4] : &sT2[NV ? c : 0][step * 16 + part * 4];
      *reinterpret_cast<uint4*>(out + static_cast<size_t>(set) * KVB * D / 4 +
                                (static_cast<size_t>(step) * D + c) * 16 + part * 4) =
          make_uint4(src[0], src[1], src[2], src[3]);
    }
  }
}

// K smoothing and per-block E4M3: K' = K - mean_K (per channel over the
// head's tokens), gathered in sorted order; s_k = max|K'_block| / 448;
// Kq = E4M3(K' / s_k) in k-step row order.  Rows are read as whole 16-byte
// pieces (BlockRows), four rows per wave instruction.
template <int D, int KVB>
__global__ __launch_bounds__(256) void k_ksmooth(const uint16_t* __restrict__ K,
                                                 const int32_t* __restrict__ perm,
                                                 const float* __restrict__ mu, int N, int nblk,
                                                 uint8_t* __restrict__ Kq, float* __restrict__ k_scale) {
  using BR = BlockRowsPacked<D, KVB>;
  __shared__ float sMax[4];
  const int bh = blockIdx.y, b = blockIdx.x;
  const int p0 = b * KVB;
  const int cg = threadIdx.x % BR::CG, q = threadIdx.x / BR::CG;
  BR rows;
  rows.load(K + static_cast<size_t>(bh) * N * D, perm + static_cast<size_t>(bh) * N, p0, N);
  float m[8];
  {
    const float4 m0 = *reinterpret_cast<const float4*>(mu + static_cast<size_t>(bh) * D + cg * 8);
    const float4 m1 = *reinterpret_cast<const float4*>(mu + static_cast<size_t>(bh) * D + cg * 8 + 4);
    m[0] = m0.x; m[1] = m0.y; m[2] = m0.z; m[3] = m0.w; m[4] = m1.x; m[5] = m1.y; m[6] = m1.z; m[7] = m1.w;
  }
  float am = 0.0f;
#pragma unroll
  for (int ps = 0; ps < BR::PASS; ++ps)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = (ps * BR::RQ + q) * 4 + rr;
      const bool live = r < KVB && p0 + r < N;
#pragma unroll
      for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(live ? rows.at(ps, rr, e) - m[e] : 0.0f));
    }
  am = wave_max(am);
  if ((threadIdx.x & 63) == 0) sMax[threadIdx.x >> 6] = am;
  __syncthreads();
  const float bm = fmaxf(fmaxf(sMax[0], sMax[1]), fmaxf(sMax[2], sMax[3]));
  const float s = bm > 0.0f ? fmaxf(bm / 448.0f, kScaleFloor) : 1.0f;
  const float y = 1.0f / s;
  if (threadIdx.x == 0) k_scale[static_cast<size_t>(bh) * nblk + b] = s;
  uint8_t* dst = Kq + (static_cast<size_t>(bh) * nblk * KVB + p0) * D + cg * 8;
#pragma unroll
  for (int ps = 0; ps < BR::PASS; ++ps)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = (ps * BR::RQ + q) * 4 + rr;
      if (r < KVB) {
        const bool live = p0 + r < N;      // padded positions hold code 0
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = live ? rows.at(ps, rr, e) - m[e] : 0.0f;
        const uint32_t lo = e4m3x4(div_rn(x[0], s, y), div_rn(x[1], s, y), div_rn(x[2], s, y), div_rn(x[3], s, y));
        const uint32_t hi = e4m3x4(div_rn(x[4], s, y), div_rn(x[5], s, y), div_rn(x[6], s, y), div_rn(x[7], s, y));
        const int prow = (r & ~63) | kstep_row_of_pos(r & 63);
        *reinterpret_cast<uint2*>(dst + static_cast<size_t>(prow) * D) = make_uint2(lo, hi);
      }
    }
}

// ---- cluster order (a blocking variant) --------------------------------------------
// The clusters can be renumbered along the principal axis of their int8 codes
// before the final assignment pass, so that a block straddling two clusters
// joins similar ones (the chooseai.io brief, "V-Smooth", asks only that
// similar tokens share a hardware block).  All of it is exact integer
// arithmetic, so the order is reproducible bit for bit.  One workgroup per head:
//   M = q^T q and the column sums s of the codes q [k, D] in int32 (packed
//   int8 dot products; |M| <= 4096 * 127^2 < 2^31);
//   S = k M - s s^T in int64; A = S >> max(0, bitlen(max|S|) - 24), in LDS;
//   v = the column of A with the largest diagonal entry (lowest index on
//   ties), then 16 steps u = A v, v = u >> max(0, bitlen(max|u|) - 24);
//   p_c = q_c . v, rank[c] = #{c' : (p_c', c') < (p_c, c)}.
constexpr int kOrderThreads = 1024;
constexpr int kOrderChunk = 128;      // centroid rows per LDS chunk
constexpr int kOrderSteps = 16;
constexpr int kOrderBits = 24;

__device__ __forceinline__ int bitlen64(unsigned long long x) { return x ? 64 - __clzll(x) : 0; }

// maximum of x over the workgroup (every thread gets it)
__device__ __forceinline__ unsigned long long block_max_u64(unsigned long long x, unsigned long long* red) {
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long y = __shfl_xor(x, o, 64);
    x = y > x ? y : x;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = 0;
  for (int w = 0; w < kOrderThreads / 64; ++w) x = red[w] > x ? red[w] : x;
  return x;
}

template <int D>
__global__ __launch_bounds__(kOrderThreads) void k_cluster_order(const int8_t* __restrict__ Cq, int k, int kpad,
                                                                 int32_t* __restrict__ rank) {
  constexpr int EPT = D * D / kOrderThreads;        // entries of M per thread
  constexpr int JG = D / EPT;                       // threads per row of M
  constexpr int CW = kOrderChunk / 4;               // 4-code words per column of a chunk
  __shared__ __attribute__((aligned(16))) int8_t sT[D][kOrderChunk];   // chunk, transposed
  __shared__ int32_t sA[D][D];
  __shared__ long long sP[kMaxClusters];
  __shared__ long long sV[D];
  __shared__ int32_t sS[D];
  __shared__ unsigned long long sRed[kOrderThreads / 64];
  __shared__ int sArg;
  const int bh = blockIdx.x, t = threadIdx.x;
  const int8_t* q = Cq + static_cast<size_t>(bh) * kpad * D;
  const int i = t / JG, jb = (t % JG) * EPT;

  int32_t acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0;
  int32_t colsum = 0;
  for (int c0 = 0; c0 < k; c0 += kOrderChunk) {
    // 16 codes of one row per thread, scattered into the transposed chunk
    for (int x = t; x < kOrderChunk * D / 16; x += kOrderThreads) {
      const int r = x / (D / 16), j0 = (x % (D / 16)) * 16;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (c0 + r < k) w = *reinterpret_cast<const uint4*>(q + static_cast<size_t>(c0 + r) * D + j0);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int b = 0; b < 16; ++b) sT[j0 + b][r] = static_cast<int8_t>(ws[b >> 2] >> (8 * (b & 3)));
    }
    __syncthreads();
    const int32_t* Ti = reinterpret_cast<const int32_t*>(sT[i]);
#pragma unroll 4
    for (int w = 0; w < CW; ++w) {
      const int32_t a = Ti[w];
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        acc[e] = __builtin_amdgcn_sdot4(a, reinterpret_cast<const int32_t*>(sT[jb + e])[w], acc[e], false);
    }
    if (t < D) {
      const int32_t* Tt = reinterpret_cast<const int32_t*>(sT[t]);
      for (int w = 0; w < CW; ++w) colsum = __builtin_amdgcn_sdot4(Tt[w], 0x01010101, colsum, false);
    }
    __syncthreads();
  }
  if (t < D) sS[t] = colsum;
  __syncthreads();

  // S = k M - s s^T, its shift, and A in LDS
  long long Sv[EPT];
  unsigned long long smax = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    Sv[e] = static_cast<long long>(k) * acc[e] - static_cast<long long>(sS[i]) * sS[jb + e];
    const unsigned long long m = static_cast<unsigned long long>(Sv[e] < 0 ? -Sv[e] : Sv[e]);
    smax = m > smax ? m : smax;
  }
  smax = block_max_u64(smax, sRed);
  const int sh = max(0, bitlen64(smax) - kOrderBits);
#pragma unroll
  for (int e = 0; e < EPT; ++e) sA[i][jb + e] = static_cast<int32_t>(Sv[e] >> sh);
  __syncthreads();

  // start: the column with the largest diagonal entry, lowest index on ties
  if (t < 64) {
    int best = t, bval = sA[t][t];
    for (int j = t + 64; j < D; j += 64)
      if (sA[j][j] > bval) { bval = sA[j][j]; best = j; }
    for (int o = 32; o > 0; o >>= 1) {
      const int ov = __shfl_xor(bval, o, 64), oi = __shfl_xor(best, o, 64);
      if (ov > bval || (ov == bval && oi < best)) { bval = ov; best = oi; }
    }
    if (t == 0) sArg = best;
  }
  __syncthreads();
  if (t < D) sV[t] = sA[t][sArg];
  __syncthreads();

  // power steps: row i of A . v by 8 threads (D = 128) or 16 (D = 64)
  constexpr int TPR = kOrderThreads / D, SEG = D / TPR;
  for (int it = 0; it < kOrderSteps; ++it) {
    const int row = t / TPR, part = t % TPR;
    long long u = 0;
#pragma unroll
    for (int j = part * SEG; j < part * SEG + SEG; ++j) u += static_cast<long long>(sA[row][j]) * sV[j];
    for (int o = TPR / 2; o > 0; o >>= 1) u += __shfl_xor(u, o, 64);
    const unsigned long long um = block_max_u64(static_cast<unsigned long long>(u < 0 ? -u : u), sRed);
    if (um == 0) break;                                   // uniform
    const int s2 = max(0, bitlen64(um) - kOrderBits);
    __syncthreads();
    if (part == 0) sV[row] = u >> s2;
    __syncthreads();
  }

  // projections and ranks
  for (int c = t; c < k; c += kOrderThreads) {
    const int8_t* qc = q + static_cast<size_t>(c) * D;
    long long pc = 0;
    for (int j = 0; j < D; ++j) pc += static_cast<long long>(qc[j]) * sV[j];
    sP[c] = pc;
  }
  __syncthreads();
  for (int c = t; c < k; c += kOrderThreads) {
    const long long pc = sP[c];
    int r = 0;
    for (int c2 = 0; c2 < k; ++c2) {
      const long long p2 = sP[c2];
      r += (p2 < pc) | ((p2 == pc) & (c2 < c));
    }
    rank[static_cast<size_t>(bh) * k + c] = r;
  }
}

// Cn[rank[c]] = C[c] (fp32 centroid rows of one head)
template <int D>
__global__ __launch_bounds__(D) void k_permute_centroids(const float* __restrict__ C, const int32_t* __restrict__ rank,
                                                         int k, float* __restrict__ Cn) {
  const int c = blockIdx.x, bh = blockIdx.y;
  const int r = rank[static_cast<size_t>(bh) * k + c];
  Cn[(static_cast<size_t>(bh) * k + r) * D + threadIdx.x] = C[(static_cast<size_t>(bh) * k + c) * D + threadIdx.x];
}

// ---- host launchers ---------------------------------------------------------------
static inline unsigned blocks_for(size_t n, int per) { return static_cast<unsigned>((n + per - 1) / per); }

hipError_t launch_fill(uint32_t* p, uint32_t v, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned nb = static_cast<unsigned>(std::min<size_t>(blocks_for(n, 256), 4096));
  hipLaunchKernelGGL(k_fill_u32, dim3(nb), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

template <int D>
static hipError_t prep_stats_t(const PrepArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  hipLaunchKernelGGL(k_stats_partial<D>, dim3(a.nstat, BH), dim3(256), 0, st, a.K, a.V, a.N, a.nstat,
                     a.kpart, a.vamax);
  hipLaunchKernelGGL(k_stats_final<D>, dim3(BH), dim3(D), 0, st, a.kpart, a.vamax, a.N, a.nstat, a.mu, a.sV);
  return hipGetLastError();
}

hipError_t launch_stats(const PrepArgs& a, hipStream_t st) {
  return a.d == 64 ? prep_stats_t<64>(a, st) : prep_stats_t<128>(a, st);
}

hipError_t launch_quant_v_i8(const PrepArgs& a, hipStream_t st) {
  const size_t per_head = static_cast<size_t>(a.N) * a.d;
  const size_t total = per_head * a.B * a.H;
  hipLaunchKernelGGL(k_quant_v_i8, dim3(blocks_for(total / 8, 256)), dim3(256), 0, st, a.V, a.sV, per_head,
                     total, a.Vq);
  return hipGetLastError();
}

template <int D>
static hipError_t init_t(const PrepArgs& a, const int32_t* init, hipStream_t st) {
  hipLaunchKernelGGL(k_init_centroids<D>, dim3(a.k, a.B * a.H), dim3(D), 0, st, a.V, init, a.N, a.k, a.C);
  return hipGetLastError();
}
hipError_t launch_init_seeded(const PrepArgs& a, uint64_t seed, int32_t* init, hipStream_t st) {
  hipLaunchKernelGGL(k_init_seeded, dim3(a.B * a.H), dim3(kInitThreads), 0, st, seed, a.N, a.k, init);
  return hipGetLastError();
}

hipError_t launch_init_centroids(const PrepArgs& a, const int32_t* init, hipStream_t st) {
  return a.d == 64 ? init_t<64>(a, init, st) : init_t<128>(a, init, st);
}

template <int D>
static hipError_t assign_t(const PrepArgs& a, int32_t* labels, hipStream_t st) {
  const int BH = a.B * a.H;
  hipLaunchKernelGGL(k_quant_centroids<D>, dim3((a.kpad + 3) / 4, BH), dim3(256), 0, st, a.C, a.sV, a.k, a.kpad,
                     a.Cq, a.cn32);
  hipLaunchKernelGGL((k_kmeans_assign<D, false, kAssignTiles>), dim3((a.N + 128 * kAssignTiles - 1) / (128 * kAssignTiles), BH), dim3(256), 0, st, a.Vq, a.Cq, a.cn32, a.N,
                     a.kpad, labels);
  return hipGetLastError();
}
hipError_t launch_assign(const PrepArgs& a, int32_t* labels, hipStream_t st) {
  return a.d == 64 ? assign_t<64>(a, labels, st) : assign_t<128>(a, labels, st);
}

template <int D>
static hipError_t bal_assign_t(const PrepArgs& a, int32_t* labels, hipStream_t st) {
  const int BH = a.B * a.H;
  hipLaunchKernelGGL(k_quant_centroids<D>, dim3((a.kpad + 3) / 4, BH), dim3(256), 0, st, a.C, a.sV, a.k, a.kpad,
                     a.Cq, a.cn32);
  hipLaunchKernelGGL(k_bal_init, dim3((std::max(a.N, a.k) + 255) / 256, BH), dim3(256), 0, st, a.N, a.k, a.kvb,
                     a.rem, labels, a.alist[0], a.acnt[0]);
  // round r reads the unplaced tokens from list r % 2 and leaves the ones
  // still unplaced in the other list, so later rounds score (and sort) only
  // those: past the first rounds nearly every workgroup would hold a few
  constexpr int WT = 128 * kBalAssignTiles;
  for (int r = 0; r < kBalRounds; ++r) {
    const int32_t* lin = a.alist[r & 1];
    const int32_t* cin = a.acnt[r & 1];
    hipLaunchKernelGGL((k_kmeans_assign<D, true, kBalAssignTiles>), dim3((a.N + WT - 1) / WT, BH), dim3(256), 0, st,
                       a.Vq, a.Cq, a.cn32, a.N, a.kpad, labels, a.prop, a.pdist, lin, cin);
    if (hipError_t e = launch_sort_list(a, a.prop, lin, cin, a.perm_tmp, st)) return e;
    hipLaunchKernelGGL(k_bal_accept<D>, dim3(a.k, BH), dim3(kBalThreads), 0, st, a.perm_tmp, a.counts, a.starts,
                       a.pdist, a.N, a.k, a.kpad, a.rem, labels, a.Cq, a.cn32);
    hipLaunchKernelGGL(k_bal_count, dim3(a.nsort, BH), dim3(kCompactThreads), 0, st, lin, cin, labels, a.N,
                       a.nsort, a.ccnt);
    hipLaunchKernelGGL(k_bal_place, dim3(a.nsort, BH), dim3(kCompactThreads), 0, st, lin, cin, labels, a.N,
                       a.nsort, a.ccnt, a.alist[(r + 1) & 1], a.acnt[(r + 1) & 1]);
  }
  hipLaunchKernelGGL(k_bal_fill, dim3(BH), dim3(kFillThreads), 0, st, a.rem, a.N, a.k, a.alist[kBalRounds & 1],
                     a.acnt[kBalRounds & 1], labels);
  return hipGetLastError();
}
hipError_t launch_bal_assign(const PrepArgs& a, int32_t* labels, hipStream_t st) {
  return a.d == 64 ? bal_assign_t<64>(a, labels, st) : bal_assign_t<128>(a, labels, st);
}

template <int D>
static hipError_t order_t(const PrepArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  hipLaunchKernelGGL(k_quant_centroids<D>, dim3((a.kpad + 3) / 4, BH), dim3(256), 0, st, a.C, a.sV, a.k, a.kpad,
                     a.Cq, a.cn32);
  hipLaunchKernelGGL(k_cluster_order<D>, dim3(BH), dim3(kOrderThreads), 0, st, a.Cq, a.k, a.kpad, a.rank);
  hipLaunchKernelGGL(k_permute_centroids<D>, dim3(a.k, BH), dim3(D), 0, st, a.C, a.rank, a.k, a.Ctmp);
  return hipMemcpyAsync(a.C, a.Ctmp, static_cast<size_t>(BH) * a.k * D * sizeof(float), hipMemcpyDeviceToDevice, st);
}
hipError_t launch_cluster_order(const PrepArgs& a, hipStream_t st) {
  return a.d == 64 ? order_t<64>(a, st) : order_t<128>(a, st);
}

hipError_t launch_sort_list(const PrepArgs& a, const int32_t* keys, const int32_t* ids, const int32_t* n,
                            int32_t* perm, hipStream_t st) {
  const int BH = a.B * a.H;
  hipLaunchKernelGGL(k_sort_hist, dim3(a.nsort, BH), dim3(256), 0, st, keys, a.N, a.k, a.nsort, a.hist, n);
  hipLaunchKernelGGL(k_sort_scan, dim3(BH), dim3(1024), 0, st, a.hist, a.k, a.nsort, a.counts, a.starts, n);
  hipLaunchKernelGGL(k_sort_scatter, dim3(a.nsort, BH), dim3(256), 0, st, keys, a.hist, a.N, a.k, a.nsort, perm,
                     ids, n);
  return hipGetLastError();
}
hipError_t launch_sort(const PrepArgs& a, const int32_t* labels, int32_t* perm, hipStream_t st) {
  return launch_sort_list(a, labels, nullptr, nullptr, perm, st);
}

template <int D>
static hipError_t update_t(const PrepArgs& a, const int32_t* perm, hipStream_t st) {
  hipLaunchKernelGGL((k_kmeans_update<D>), dim3(a.k, a.B * a.H), dim3(64), 0, st, a.V, perm, a.counts, a.starts,
                     a.N, a.k, a.C);
  return hipGetLastError();
}
hipError_t launch_update(const PrepArgs& a, const int32_t* perm, hipStream_t st) {
  return a.d == 64 ? update_t<64>(a, perm, st) : update_t<128>(a, perm, st);
}

hipError_t launch_iota(int32_t* perm, int N, size_t total, hipStream_t st) {
  hipLaunchKernelGGL(k_iota, dim3(blocks_for(total, 256)), dim3(256), 0, st, perm, N, total);
  return hipGetLastError();
}

template <int D, int KVB>
static hipError_t vres_t(const PrepArgs& a, const int32_t* perm, const PrepOut& o, hipStream_t st) {
  const int BH = a.B * a.H;
  const int e4 = a.v_format == 0;
  // the per-channel max |r| of the head: the E4M3 scales, the NVFP4-style second-level scale
  const int want_amax = a.v_format == 0 || a.v_format == 3;
  hipLaunchKernelGGL((k_vblock_stats<D, KVB>), dim3(a.nblk, BH), dim3(256), 0, st, a.V, perm, a.N, a.nblk,
                     a.vsmooth, want_amax, o.v_mean, a.vramax);
  uint8_t* e8 = reinterpret_cast<uint8_t*>(o.v_scale);
  if (e4)
    hipLaunchKernelGGL((k_vres_e4m3<D, KVB>), dim3(a.nblk, BH), dim3(256), 0, st, a.V, perm, o.v_mean, a.vramax,
                       a.N, a.nblk, o.Vres, reinterpret_cast<float*>(o.v_scale));
  else if (a.v_format == 1)
    hipLaunchKernelGGL((k_vres_mx<D, KVB, 1>), dim3(a.nblk, BH), dim3(256), 0, st, a.V, perm, o.v_mean, a.vramax,
                       a.N, a.nblk, o.Vres, e8);
  else if (a.v_format == 2)
    hipLaunchKernelGGL((k_vres_mx<D, KVB, 2>), dim3(a.nblk, BH), dim3(256), 0, st, a.V, perm, o.v_mean, a.vramax,
                       a.N, a.nblk, o.Vres, e8);
  else
    hipLaunchKernelGGL((k_vres_mx<D, KVB, 3>), dim3(a.nblk, BH), dim3(256), 0, st, a.V, perm, o.v_mean, a.vramax,
                       a.N, a.nblk, o.Vres, e8);
  hipLaunchKernelGGL((k_ksmooth<D, KVB>), dim3(a.nblk, BH), dim3(256), 0, st, a.K, perm, a.mu, a.N, a.nblk, o.Kq,
                     o.k_scale);
  return hipGetLastError();
}
hipError_t launch_vres_ksmooth(const PrepArgs& a, const int32_t* perm, const PrepOut& o, hipStream_t st) {
  if (a.d == 64) return a.kvb == 64 ? vres_t<64, 64>(a, perm, o, st) : vres_t<64, 128>(a, perm, o, st);
  return a.kvb == 64 ? vres_t<128, 64>(a, perm, o, st) : vres_t<128, 128>(a, perm, o, st);
}

}  // namespace vc
