// Fused VC-Attention forward for gfx950.
//
// Per 128-row query tile (one workgroup, 4 waves x 32 queries):
//   * Q tile -> E4M3 codes with one scale s_q = max|Q|/448, kept in registers;
//   * for every KV block in ascending order (chooseai.io brief, "V-Smooth":
//     the mean comes back through the online-softmax row sums; theclarity.today
//     story: one pass over the values):
//       S^T = Kq . Qq^T                    v_mfma_f32_32x32x64_f8f6f4 (E4M3)
//       m_new = max(m, fp32(c_b * rowmax S)),  c_b = fp32(cq * s_k[b])
//       byte  = cvt_u8(fma(S, 8 c_b, fp32(56 + beta - 8 m_new)))
//               (ExpCast-FP8, chooseai.io brief section "ExpCast-FP8": one
//               fused multiply-add writes the E4M3 probability byte; the
//               byte convert rounds to nearest even and clamps at 0)
//       rowsum = sum of the decoded bytes (exact in fp32)
//       acc = alpha*acc + Vres^T . P^T (FP8 MFMA; MXFP4 residuals use the
//             scaled f8f6f4 MFMA with E8M0 block scales) + rowsum * mean_b/s_v
//       l   = alpha*l + rowsum
//   * O = s_v * acc / l.
// Operand layouts (measured on gfx950 with a one-wave probe):
//   * 32x32 accumulator: register r of lane l holds row 8(r/4) + 4(l/32) + r%4,
//     column l%32;
//   * fp8 A and B operands: byte s of lane group g (g = l/32) holds contraction
//     index 16g + s for s < 16 and 32 + 16g + (s-16) for s >= 16 (A and B agree);
//   * FP4 A operand: nibble s of lane group g holds contraction index 32g + s.
// A 64-key step therefore uses sorted position kappa as the contraction index:
// Kq rows are stored so that S^T tile t, register r, lane group g holds
// kappa = 32t + 16g + r, which is exactly where the P^T B operand wants the byte
// (bytes 0..15 from tile 0, 16..31 from tile 1); residual rows are stored in
// kappa order, so fp8 A reads bytes [16g, 16g+16) and [32+16g, 48+16g) and FP4 A
// reads nibbles [32g, 32g+32) = one E8M0 scale group.
#include "vc_internal.hpp"

namespace vc {

__device__ __forceinline__ uint32_t expcast4(float s0, float s1, float s2, float s3, float A, float B) {
  uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s0, A, B), 0, 0u);
  w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s1, A, B), 1, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s2, A, B), 2, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s3, A, B), 3, w);
  return w;
}

__device__ __forceinline__ float fp8x4_sum(uint32_t w) {
  const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  return (lo.x + lo.y) + (hi.x + hi.y);
}

__global__ void k_dbg_expcast(const float* __restrict__ S, const float* __restrict__ A,
                              const float* __restrict__ B, int64_t n, uint8_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = static_cast<uint8_t>(expcast4(S[i], 0.f, 0.f, 0.f, A[i], B[i]) & 0xffu);
}

template <int D, int KVB, int VF, int O32>
__global__ __launch_bounds__(256, 2) void k_attn_fwd(AttnArgs p) {
  constexpr int NDC = D / 64;     // 64-deep chunks of the QK^T contraction
  constexpr int NKT = KVB / 32;   // 32-key tiles of S^T per block
  constexpr int NKS = KVB / 64;   // 64-key steps of the PV contraction
  constexpr int NDT = D / 32;     // 32-channel tiles of O^T
  constexpr int KSTR = D + 16;    // padded LDS row strides (conflict-free 16-byte reads)
  constexpr int VROW = VF == 0 ? 64 : 32;
  constexpr int VSTR = VROW + 16;
  __shared__ __attribute__((aligned(16))) uint8_t sK[KVB * KSTR];
  __shared__ __attribute__((aligned(16))) uint8_t sV[NKS * D * VSTR];
  __shared__ __attribute__((aligned(16))) uint8_t sVs[VF == 1 ? (KVB / 32) * D : 16];
  __shared__ __attribute__((aligned(16))) float sMean[D];
  __shared__ __attribute__((aligned(16))) float sCol[D];
  __shared__ float sRed[4];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5, col = lane & 31;
  const int N = p.N, nblk = p.nblk;
  const int nqt = (N + kQTile - 1) / kQTile;
  const int bh = blockIdx.x / nqt, qt = blockIdx.x % nqt;
  const int qrow = qt * kQTile + wave * 32 + col;

  if (threadIdx.x < D)
    sCol[threadIdx.x] = VF == 0 ? reinterpret_cast<const float*>(p.v_scale)[static_cast<size_t>(bh) * D + threadIdx.x]
                                : 1.0f;

  // ---- query tile: E4M3 codes with one scale per 128 rows ----
  v8i qb[NDC];
  float cq;
  {
    float qv[NDC][32];
    float am = 0.0f;
    const uint16_t* qp = p.Q + (static_cast<size_t>(bh) * N + qrow) * D;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        if (qrow < N) raw = *reinterpret_cast<const uint4*>(qp + 64 * c + 32 * g + 8 * u);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = bf16_to_f32(static_cast<uint16_t>(w[e >> 1] >> ((e & 1) * 16)));
          qv[c][8 * u + e] = f;
          am = fmaxf(am, fabsf(f));
        }
      }
    }
    am = wave_max(am);
    if (lane == 0) sRed[wave] = am;
    __syncthreads();
    const float amax = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));
    const float sq = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        uint32_t word = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) word |= e4m3_encode(qv[c][4 * w + e] / sq) << (8 * e);
        qb[c][w] = static_cast<int>(word);
      }
    }
    const float t = sq * p.scale;
    cq = t * kLog2e;
  }

  float m_run = -__builtin_inff(), l_run = 0.0f;
  v16f acc[NDT];
#pragma unroll
  for (int T = 0; T < NDT; ++T)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[T][r] = 0.0f;

  const uint8_t* kq = p.Kq + static_cast<size_t>(bh) * nblk * KVB * D;
  const uint8_t* vr = p.Vres + static_cast<size_t>(bh) * nblk * NKS * D * VROW;
  const float* ks = p.k_scale + static_cast<size_t>(bh) * nblk;
  const float* vm = p.v_mean + static_cast<size_t>(bh) * nblk * D;

  for (int b = 0; b < nblk; ++b) {
    __syncthreads();
    for (int i = threadIdx.x; i < KVB * D / 16; i += 256) {
      const int r = i / (D / 16), q16 = i % (D / 16);
      *reinterpret_cast<uint4*>(sK + r * KSTR + q16 * 16) =
          *reinterpret_cast<const uint4*>(kq + static_cast<size_t>(b) * KVB * D + r * D + q16 * 16);
    }
    for (int i = threadIdx.x; i < NKS * D * VROW / 16; i += 256) {
      const int row = i / (VROW / 16), q16 = i % (VROW / 16);
      *reinterpret_cast<uint4*>(sV + row * VSTR + q16 * 16) =
          *reinterpret_cast<const uint4*>(vr + (static_cast<size_t>(b) * NKS * D + row) * VROW + q16 * 16);
    }
    if constexpr (VF == 1) {
      const uint8_t* sc = reinterpret_cast<const uint8_t*>(p.v_scale) +
                          (static_cast<size_t>(bh) * nblk * (KVB / 32) + static_cast<size_t>(b) * (KVB / 32)) * D;
      for (int i = threadIdx.x; i < (KVB / 32) * D / 16; i += 256)
        *reinterpret_cast<uint4*>(sVs + i * 16) = *reinterpret_cast<const uint4*>(sc + i * 16);
    }
    if (threadIdx.x < D) {
      const float mv = vm[static_cast<size_t>(b) * D + threadIdx.x];
      sMean[threadIdx.x] = VF == 0 ? mv / sCol[threadIdx.x] : mv;
    }
    __syncthreads();

    // ---- S^T = Kq . Qq^T ----
    v16f S[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[kt][r] = 0.0f;
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        const v8i a = *reinterpret_cast<const v8i*>(sK + (kt * 32 + col) * KSTR + 64 * c + 32 * g);
        S[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qb[c], S[kt], 0, 0, 0, 0, 0, 0);
      }
    }
    const int nvalid = min(KVB, N - b * KVB);
    if (nvalid < KVB) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kappa = (kt >> 1) * 64 + (kt & 1) * 32 + 16 * g + r;
          if (kappa >= nvalid) S[kt][r] = -__builtin_inff();
        }
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));

    const float cb = cq * ks[b];
    const float tmax = cb * mx;
    const float m_new = fmaxf(m_run, tmax);
    const float Bq = __builtin_fmaf(-8.0f, m_new, p.kc);
    const float A8 = 8.0f * cb;
    const float alpha = exp2f(m_run - m_new);

    // ---- ExpCast bytes, packed straight into the PV B operand ----
    v8i P[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const v16f& st = S[2 * s + t];
          P[s][4 * t + q4] = static_cast<int>(
              expcast4(st[4 * q4], st[4 * q4 + 1], st[4 * q4 + 2], st[4 * q4 + 3], A8, Bq));
        }
    float rs = 0.0f;
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int w = 0; w < 8; ++w) rs += fp8x4_sum(static_cast<uint32_t>(P[s][w]));
    rs += __shfl_xor(rs, 32, 64);
    l_run = alpha * l_run + rs;

#pragma unroll
    for (int T = 0; T < NDT; ++T)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[T][r] *= alpha;

    // ---- acc += Vres^T . P^T ----
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int T = 0; T < NDT; ++T) {
        const uint8_t* vrow = sV + (s * D + 32 * T + col) * VSTR;
        if constexpr (VF == 0) {
          const uint4 lo = *reinterpret_cast<const uint4*>(vrow + 16 * g);
          const uint4 hi = *reinterpret_cast<const uint4*>(vrow + 32 + 16 * g);
          const v8i a = {static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                         static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
          acc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, P[s], acc[T], 0, 0, 0, 0, 0, 0);
        } else {
          const uint4 q = *reinterpret_cast<const uint4*>(vrow + 16 * g);
          const v8i a = {static_cast<int>(q.x), static_cast<int>(q.y), static_cast<int>(q.z), static_cast<int>(q.w),
                         0, 0, 0, 0};
          const int sc = sVs[(2 * s + g) * D + 32 * T + col];
          acc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, P[s], acc[T], 4, 0, 0, sc, 0, 127);
        }
      }
    // ---- mean restoration from the block row sum ----
#pragma unroll
    for (int T = 0; T < NDT; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 mv = *reinterpret_cast<const float4*>(sMean + 32 * T + 8 * i + 4 * g);
        acc[T][4 * i + 0] = __builtin_fmaf(rs, mv.x, acc[T][4 * i + 0]);
        acc[T][4 * i + 1] = __builtin_fmaf(rs, mv.y, acc[T][4 * i + 1]);
        acc[T][4 * i + 2] = __builtin_fmaf(rs, mv.z, acc[T][4 * i + 2]);
        acc[T][4 * i + 3] = __builtin_fmaf(rs, mv.w, acc[T][4 * i + 3]);
      }
    m_run = m_new;
  }

  // ---- O = s_v * acc / l ----
  if (qrow < N) {
    const float inv_l = 1.0f / l_run;
#pragma unroll
    for (int T = 0; T < NDT; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c0 = 32 * T + 8 * i + 4 * g;
        const float4 cs = *reinterpret_cast<const float4*>(sCol + c0);
        const float o0 = acc[T][4 * i + 0] * cs.x * inv_l;
        const float o1 = acc[T][4 * i + 1] * cs.y * inv_l;
        const float o2 = acc[T][4 * i + 2] * cs.z * inv_l;
        const float o3 = acc[T][4 * i + 3] * cs.w * inv_l;
        const size_t off = (static_cast<size_t>(bh) * N + qrow) * D + c0;
        if constexpr (O32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.O) + off) = make_float4(o0, o1, o2, o3);
        } else {
          const uint32_t w0 = f32_to_bf16_rne(o0) | (static_cast<uint32_t>(f32_to_bf16_rne(o1)) << 16);
          const uint32_t w1 = f32_to_bf16_rne(o2) | (static_cast<uint32_t>(f32_to_bf16_rne(o3)) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.O) + off) = make_uint2(w0, w1);
        }
      }
  }
}

template <int D, int KVB, int VF>
static void launch_attn_t(const AttnArgs& a, hipStream_t st) {
  const int nqt = (a.N + kQTile - 1) / kQTile;
  const dim3 grid(static_cast<unsigned>(a.B * a.H * nqt));
  if (a.out_fp32)
    hipLaunchKernelGGL((k_attn_fwd<D, KVB, VF, 1>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn_fwd<D, KVB, VF, 0>), grid, dim3(256), 0, st, a);
}

template <int D, int KVB>
static void launch_attn_f(const AttnArgs& a, hipStream_t st) {
  if (a.v_format == 0) launch_attn_t<D, KVB, 0>(a, st);
  else launch_attn_t<D, KVB, 1>(a, st);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  if (a.d == 64) {
    if (a.kvb == 64) launch_attn_f<64, 64>(a, st);
    else launch_attn_f<64, 128>(a, st);
  } else {
    if (a.kvb == 64) launch_attn_f<128, 64>(a, st);
    else launch_attn_f<128, 128>(a, st);
  }
  return hipGetLastError();
}

hipError_t launch_dbg_expcast(const float* S, const float* A, const float* B, int64_t n, uint8_t* out,
                              hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_dbg_expcast, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, S, A, B, n,
                     out);
  return hipGetLastError();
}

}  // namespace vc
