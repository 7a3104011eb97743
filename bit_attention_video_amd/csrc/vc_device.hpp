// Device helpers shared by the VC-Attention kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vc {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kQTile = 128;          // query rows per tile (one scale per tile)
// Smallest quantiser scale (the smallest normal fp32, 2^-126): amax / 448 or
// amax / 127 is floored here so that the reciprocal every quantiser uses
// stays finite for tiny nonzero inputs.
constexpr float kScaleFloor = 0x1p-126f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;   // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// OCP E4M3 (bias 7, max 448, no inf), round-to-nearest-even, saturating at
// +-448; the sign bit is copied from the input (also for zero); NaN -> 0x7f.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  const float af = __uint_as_float(a);
  uint32_t code;
  if (af >= 464.0f) {
    code = 0x7eu;                                   // [464, inf] rounds past 448
  } else if (af < 0.015625f) {                      // below 2^-6: grid of 2^-9
    code = static_cast<uint32_t>(rintf(af * 512.0f));   // exact scale, RNE; 8 = 2^-6
  } else {
    const int e = static_cast<int>(a >> 23) - 127;  // af in [2^e, 2^(e+1)), -6 <= e <= 8
    const uint32_t m23 = a & 0x7fffffu;
    uint32_t m = m23 >> 20;
    const uint32_t rem = m23 & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) m += 1u;
    const uint32_t c = (static_cast<uint32_t>(e + 7) << 3) + m;   // m == 8 carries
    code = c > 0x7eu ? 0x7eu : c;
  }
  return code | sign;
}

// OCP E2M1 nibble, nearest-even on {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
  const float a = fminf(fabsf(x), 6.0f);
  uint32_t code;
  if (a < 2.0f) {
    code = static_cast<uint32_t>(rintf(a * 2.0f));      // 0..4 (4 == value 2)
  } else if (a < 4.0f) {
    const float r = rintf(a);                           // 2, 3 or 4
    code = r == 2.0f ? 4u : (r == 3.0f ? 5u : 6u);
  } else {
    const float r = rintf(a * 0.5f);                    // 2 or 3 -> value 4 or 6
    code = r == 2.0f ? 6u : 7u;
  }
  return code | sign;
}

// value of an OCP E2M1 nibble (sign in bit 3)
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  const float v = m < 5u ? 0.5f * static_cast<float>(m) : (m == 5u ? 3.0f : (m == 6u ? 4.0f : 6.0f));
  return (c & 8u) ? -v : v;
}

// value of a finite OCP E4M3 code (sign in bit 7)
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const int e = static_cast<int>((c >> 3) & 15u);
  const float m = static_cast<float>(c & 7u);
  const float v = e == 0 ? ldexpf(m, -9) : ldexpf(1.0f + 0.125f * m, e - 7);
  return (c & 0x80u) ? -v : v;
}

// x / s rounded once to binary32, given y = fp32(1 / s) rounded once:
// q = x*y, then one correction from the exact residual x - q*s (Markstein's
// division with a correctly rounded reciprocal; s > 0 normal, x finite).
// The sign copy keeps -0 / s = -0.
__device__ __forceinline__ float div_rn(float x, float s, float y) {
  const float q = x * y;
  const float r = __builtin_fmaf(-q, s, x);
  return __builtin_copysignf(__builtin_fmaf(r, y, q), x);
}

// E4M3 codes (round to nearest even, sign kept) of four values with
// |x| < 464, packed little-endian; v_cvt_pk_fp8_f32 converts two per
// instruction.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// MX scale storage order inside one 32-position group: channel c = 32T + col
// sits at col * (D/32) + T, so the scales of one attention lane (one col, all
// 32-channel tiles T) are adjacent bytes.
template <int D>
__host__ __device__ __forceinline__ int mx_scale_slot(int c) {
  return (c & 31) * (D / 32) + (c >> 5);
}

// int8 code of x / s for the k-means distances: clamp(rne(fp32(x / s)), -127, 127)
__device__ __forceinline__ int32_t i8_code(float x, float s) {
  float r = rintf(x / s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return static_cast<int32_t>(r);
}
// the same with y = fp32(1 / s) given (see div_rn)
__device__ __forceinline__ int32_t i8_code(float x, float s, float y) {
  float r = rintf(div_rn(x, s, y));
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return static_cast<int32_t>(r);
}

// sorted position kappa (0..63) inside a 64-key group -> stored row.
// kappa = 32t + 16g + 4i + j is stored at row 32t + 8i + 4g + j, so that the
// 32x32 MFMA accumulator of QK^T lands each lane's keys exactly where the
// PV MFMA's B operand expects them.
__host__ __device__ __forceinline__ int kstep_row_of_pos(int kappa) {
  const int t = kappa >> 5, g = (kappa >> 4) & 1, i = (kappa >> 2) & 3, j = kappa & 3;
  return (t << 5) | (i << 3) | (g << 2) | j;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t as_u32_bits(float f) { return __float_as_uint(f); }

}  // namespace vc
