// Host-side dispatch of the fused VC-Attention forward, the test-only byte
// probes of the probability codes, and the FP8 MFMA-loop measurement kernel.
// The forward's kernel templates are in attn_kernel.hpp; attn_inst.hip
// instantiates them once per (head dim, KV block, residual format), each in
// an object file of its own.
#include "attn_kernel.hpp"

namespace vc {

// the instantiations (attn_inst.hip)
#define VC_ATTN_EXTERN(D, KVB, VF) extern template hipError_t launch_attn_cfg<D, KVB, VF>(const AttnArgs&, hipStream_t);
#define VC_ATTN_EXTERN_F(D, KVB) VC_ATTN_EXTERN(D, KVB, 0) VC_ATTN_EXTERN(D, KVB, 1) VC_ATTN_EXTERN(D, KVB, 2) \
  VC_ATTN_EXTERN(D, KVB, 3)
VC_ATTN_EXTERN_F(64, 64)
VC_ATTN_EXTERN_F(64, 128)
VC_ATTN_EXTERN_F(128, 64)
VC_ATTN_EXTERN_F(128, 128)
#undef VC_ATTN_EXTERN_F
#undef VC_ATTN_EXTERN

template <int D, int KVB>
static hipError_t launch_attn_f(const AttnArgs& a, hipStream_t st) {
  switch (a.v_format) {
    case 0: return launch_attn_cfg<D, KVB, 0>(a, st);
    case 1: return launch_attn_cfg<D, KVB, 1>(a, st);
    case 2: return launch_attn_cfg<D, KVB, 2>(a, st);
    default: return launch_attn_cfg<D, KVB, 3>(a, st);
  }
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  if (a.d == 64) return a.kvb == 64 ? launch_attn_f<64, 64>(a, st) : launch_attn_f<64, 128>(a, st);
  return a.kvb == 64 ? launch_attn_f<128, 64>(a, st) : launch_attn_f<128, 128>(a, st);
}

__global__ void k_dbg_expcast(const float* __restrict__ S, const float* __restrict__ A,
                              const float* __restrict__ B, int64_t n, uint8_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = static_cast<uint8_t>(expcast4(S[i], 0.f, 0.f, 0.f, A[i], B[i]) & 0xffu);
}

__global__ void k_dbg_exp2cast(const float* __restrict__ S, const float* __restrict__ A,
                               const float* __restrict__ B, int64_t n, uint8_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = static_cast<uint8_t>(exp2cast4(S[i], 0.f, 0.f, 0.f, A[i], B[i]) & 0xffu);
}

// Eight independent FP8 32x32x64 MFMA chains per wave: the matrix core's
// sustained rate at the clock the part holds under full MFMA load.
__global__ __launch_bounds__(512) void k_mfma_loop(int iters, float* __restrict__ out) {
  v16f acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = v16f{};
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<int>(0x30303030u + threadIdx.x);
    b[i] = static_cast<int>(0x28282828u + i);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[m], 0, 0, 0, 0, 0, 0);
  }
  float r = 0.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[m][i];
  out[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = r;
}

hipError_t launch_mfma_loop(int blocks, int iters, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_mfma_loop, dim3(static_cast<unsigned>(blocks)), dim3(512), 0, st, iters, out);
  return hipGetLastError();
}

hipError_t launch_dbg_exp2cast(const float* S, const float* A, const float* B, int64_t n, uint8_t* out,
                               hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_dbg_exp2cast, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, S, A, B, n,
                     out);
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
