// Fused VC-Attention forward for gfx950 (kernel templates; instantiated per
// (head dim, KV block, residual format) by attn_inst.hip).
//
// Per 256 query rows (one workgroup, 8 waves x 32 queries):
//   * each 128-row Q tile -> E4M3 codes with one scale s_q = max|Q|/448, kept
//     in registers;
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
//       acc = alpha*acc + Vres^T . P^T (FP8 MFMA; MXFP4 and MXFP8 residuals
//             use the scaled f8f6f4 MFMA with E8M0 scales per 32 keys and
//             channel; NVFP4-style residuals, whose E4M3 scales per 16 keys
//             vary along the contraction, arrive as two E4M3 parts under one
//             E8M0 scale and take two MFMAs) + rowsum * mean_b/s_v
//       l   = alpha*l + rowsum
//   * O = s_v * acc / l.
// Operand layouts (measured on gfx950 with a one-wave probe):
//   * 32x32 accumulator: register r of lane l holds row 8(r/4) + 4(l/32) + r%4,
//     column l%32;
//   * fp8 A and B operands: byte s of lane group g (g = l/32) holds contraction
//     index 16g + s for s < 16 and 32 + 16g + (s-16) for s >= 16 (A and B agree);
//   * FP4 A operand: nibble s of lane group g holds contraction index 32g + s;
//   * E8M0 scales of the scaled MFMA: lane group b's scale covers contraction
//     block [32b, 32b+32), for FP8 and FP4 A operands alike.
// A 64-key step therefore uses sorted position kappa as the contraction index:
// Kq rows are stored so that S^T tile t, register r, lane group g holds
// kappa = 32t + 16g + r, which is exactly where the P^T B operand wants the byte
// (bytes 0..15 from tile 0, 16..31 from tile 1); residual rows are stored in
// kappa order, so fp8 A reads bytes [16g, 16g+16) and [32+16g, 48+16g) and FP4 A
// reads nibbles [32g, 32g+32) = one E8M0 scale group.
#pragma once
#include <type_traits>

#include "vc_internal.hpp"

namespace vc {

__device__ __forceinline__ uint32_t expcast4(float s0, float s1, float s2, float s3, float A, float B) {
  uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s0, A, B), 0, 0u);
  w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s1, A, B), 1, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s2, A, B), 2, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s3, A, B), 3, w);
  return w;
}

// ExpCast off: four E4M3 bytes of exp2(fma(s, A, B)) (fp32 exponential, then
// the packed FP8 conversion, round to nearest even; -inf scores give 0)
__device__ __forceinline__ uint32_t exp2cast4(float s0, float s1, float s2, float s3, float A, float B) {
  const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0, A, B));
  const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, A, B));
  const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2, A, B));
  const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s3, A, B));
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, lo, true));
}

// the probability word of one of the two modes (0: ExpCast, 1: exp2 + cast)
template <int PM>
__device__ __forceinline__ uint32_t pword4(float s0, float s1, float s2, float s3, float A, float B) {
  if constexpr (PM == 0) return expcast4(s0, s1, s2, s3, A, B);
  else return exp2cast4(s0, s1, s2, s3, A, B);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Swizzled 16-byte chunk inside an LDS row of RB bytes.  A 16-byte operand
// read is served 8 lanes per cycle from 32 banks or 16 lanes per cycle from
// 64 banks; the XOR below gives the consecutive rows read together distinct
// bank groups in both cases (rows sharing a 128-byte line differ in the bits
// above the line index, rows sharing a 256-byte line in the next bit up).
template <int RB>
__device__ __forceinline__ int swz(int row, int chunk) {
  // the XOR uses only row bits 0..3, so tiles and load rounds that start at
  // multiples of 32 rows share one per-lane pattern
  if constexpr (RB == 128) return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
  else if constexpr (RB == 64) return chunk ^ (((row >> 1) ^ (row >> 2)) & 3);
  else return chunk ^ (((row >> 2) ^ (row >> 3)) & 1);
}

// max of v over lanes l and l^32 (v_permlane32_swap returns both halves)
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(fmaxf(v, __uint_as_float(r[0])), __uint_as_float(r[1]));
}

constexpr int kAttnThreads = 512;   // threads per attention workgroup

template <int D, int KVB, int VF>
struct AttnTile {
  static constexpr int NDC = D / 64;      // 64-deep chunks of the QK^T contraction
  static constexpr int NKT = KVB / 32;    // 32-key tiles of S^T per block
  static constexpr int NKS = KVB / 64;    // 64-key steps of the PV contraction
  static constexpr int NDT = D / 32;      // 32-channel tiles of O^T
  static constexpr int VROW = VF == 1 ? 32 : 64;   // residual bytes per channel row of a 64-key step
  static constexpr int KBYTES = KVB * D;
  static constexpr int VHALF = NKS * D * VROW;                 // one code set of a block
  static constexpr int VBYTES = VF == 3 ? 2 * VHALF : VHALF;   // NVFP4 emulation: high, then low parts
  static constexpr int SBYTES = VF != 0 ? (KVB / 32) * D : 0;    // E8M0 scales (MX formats)
  static constexpr int STAGE = KBYTES + VBYTES + (SBYTES + 1023) / 1024 * 1024;
  static constexpr int MSLOT = 8;         // blocks per mean-restoration flush
  // NVFP4-style residuals take two P.V MFMAs per tile; interleaving the next
  // block's scores with them would keep both score and byte registers live
  // past the register file, so those blocks run in two phases (scores and
  // ExpCast, then row sums and P.V) with K and V staged one block ahead
  static constexpr bool SPLIT = VF == 3;
  static constexpr int NTH = kAttnThreads;
  static constexpr int NWV = NTH / 64;    // waves, 32 query rows each
  static constexpr int ROWS = NWV * 32;   // query rows per workgroup (NWV / 4 scale tiles)
};

// Per-lane offsets that stay fixed for the whole kernel.  With the swizzle
// above, the chunk a lane reads depends only on its lane position (tile rows
// start at multiples of 32), so every LDS operand address is lane offset +
// compile-time tile offset, and every direct-load source is block base + lane
// offset.
template <int D, int KVB, int VF>
struct LaneOffsets {
  using T = AttnTile<D, KVB, VF>;
  static constexpr int RB = T::NTH * 16;                  // bytes per direct-load round
  static constexpr int KR = (T::KBYTES + RB - 1) / RB;    // direct-load rounds for K
  static constexpr int VR = (T::VBYTES + RB - 1) / RB;    // ... and for the residuals
  int k_rd[T::NDC][2];   // K operand: 16-byte halves of the 32-byte chunk (c, h)
  int v_rd[2];           // residual operand chunks (E4M3, MXFP8: g and 2+g; MXFP4: g)
  int k_src, v_src;      // source offsets of this lane's direct loads (round 0)
  __device__ __forceinline__ LaneOffsets(int lane) {
    const int g = lane >> 5, col = lane & 31;
#pragma unroll
    for (int c = 0; c < T::NDC; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) k_rd[c][h] = col * D + swz<D>(col, 4 * c + 2 * g + h) * 16;
    v_rd[0] = col * T::VROW + swz<T::VROW>(col, g) * 16;
    v_rd[1] = col * T::VROW + swz<T::VROW>(col, VF != 1 ? 2 + g : g) * 16;
    // round r fetches chunk NTH*r + tid: its row is NTH*r/(D/16) rows further
    // down, a multiple of 32, so the swizzled chunk is the same as in round 0
    const int t = threadIdx.x;
    const int krow = t / (D / 16), vrow = t / (T::VROW / 16);
    k_src = krow * D + swz<D>(krow, t % (D / 16)) * 16;
    v_src = vrow * T::VROW + swz<T::VROW>(vrow, t % (T::VROW / 16)) * 16;
  }
};

// Stage one block (K rows, residual rows, E8M0 scales) into LDS with direct
// buffer->LDS loads (buffer_load_dwordx4 ... lds: lane i of a wave writes
// bytes [16i, 16i+16) after the wave-uniform LDS base in M0); the swizzle is
// applied on the global side by choosing which chunk each lane fetches.  The
// buffer form takes the block offset in an SGPR and the lane offset in a
// loop-invariant VGPR, so issuing a load costs no vector instructions.  (The
// FLAT form, global_load_lds, also works, but while one is in flight the
// compiler's wait-count pass can only drain LDS reads completely, which
// undoes the operand prefetch below.)
// raw buffer descriptor over [base, base + bytes) (stride 0, no swizzle)
#define VC_BUFFER_RSRC(base, bytes) \
  __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(static_cast<const void*>(base)), 0, static_cast<int>(bytes), 0x00020000)

// (R0, R1): the direct-load rounds to issue, [R0, R1)
template <int D, int KVB, int VF, int R0 = 0, int R1 = 64>
__device__ __forceinline__ void stage_block_k(uint8_t* st, const uint8_t* kq, uint32_t kq_bytes, uint32_t blk_off,
                                              const LaneOffsets<D, KVB, VF>& lo, int wave) {
  using T = AttnTile<D, KVB, VF>;
  using L = LaneOffsets<D, KVB, VF>;
  const auto rs = VC_BUFFER_RSRC(kq, kq_bytes);
#pragma unroll
  for (int r = R0; r < (R1 < L::KR ? R1 : L::KR); ++r)
    if ((r * T::NTH + wave * 64) * 16 < T::KBYTES)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(st + (r * T::NTH + wave * 64) * 16), 16,
                                               static_cast<uint32_t>(lo.k_src), blk_off + static_cast<uint32_t>(r * L::RB), 0, 0);
}

template <int D, int KVB, int VF, int R0 = 0, int R1 = 64>
__device__ __forceinline__ void stage_block_v(uint8_t* sv, const uint8_t* vr, uint32_t vr_bytes, uint32_t blk_off,
                                              const uint8_t* sc, uint32_t sc_bytes, uint32_t sc_off,
                                              const LaneOffsets<D, KVB, VF>& lo, int wave, int lane) {
  using T = AttnTile<D, KVB, VF>;
  using L = LaneOffsets<D, KVB, VF>;
  const auto rs = VC_BUFFER_RSRC(vr, vr_bytes);
#pragma unroll
  for (int r = R0; r < (R1 < L::VR ? R1 : L::VR); ++r)
    if ((r * T::NTH + wave * 64) * 16 < T::VBYTES)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(sv + (r * T::NTH + wave * 64) * 16), 16,
                                               static_cast<uint32_t>(lo.v_src), blk_off + static_cast<uint32_t>(r * L::RB), 0, 0);
  if constexpr (VF != 0 && R0 == 0) {
    const auto rsc = VC_BUFFER_RSRC(sc, sc_bytes);
    if (wave == 0 && lane < T::SBYTES / 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (lds_ptr_t)(sv + T::VBYTES), 16, static_cast<uint32_t>(lane * 16),
                                               sc_off, 0, 0);
  }
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// bf16 hi + lo split of two finite values (row sums, block means): hi rounds
// each to nearest even on the packed convert, lo rounds what hi leaves over;
// two packed words, element a in the low half
__device__ __forceinline__ void bf16_split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const v2bf h = v2bf{static_cast<__bf16>(a), static_cast<__bf16>(b)};
  const v2bf l = v2bf{static_cast<__bf16>(a - static_cast<float>(h[0])), static_cast<__bf16>(b - static_cast<float>(h[1]))};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

__device__ __forceinline__ v8i join8(uint4 lo, uint4 hi) {
  return v8i{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
             static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

// Bijection from the hardware workgroup index (dispatched round-robin over
// the 8 XCDs) to a logical index in which XCD x owns one contiguous range.
__device__ __forceinline__ int xcd_major_index(int i, int n) {
  constexpr int kXcds = 8;
  const int x = i % kXcds, local = i / kXcds;
  const int per = n / kXcds, rem = n % kXcds;
  return x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
}

// Per-wave running state of the online softmax.
template <int NDT, int MS>
struct SoftmaxState {
  v16f acc[NDT];
  float RS[MS];        // row sums of the blocks since the last mean flush
  float m_run, l_run;
};

// S^T = Kq . Qq^T for one block (8 MFMAs at d=128).
template <int D, int KVB, int VF>
__device__ __forceinline__ void qk_block(v16f* S, const uint8_t* sK,
                                         const LaneOffsets<D, KVB, VF>& lo, const v8i* qb) {
  using TT = AttnTile<D, KVB, VF>;
#pragma unroll
  for (int kt = 0; kt < TT::NKT; ++kt)
#pragma unroll
    for (int c = 0; c < TT::NDC; ++c) {
      const v8i a = join8(*reinterpret_cast<const uint4*>(sK + kt * 32 * D + lo.k_rd[c][0]),
                          *reinterpret_cast<const uint4*>(sK + kt * 32 * D + lo.k_rd[c][1]));
      S[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qb[c], c == 0 ? v16f{} : S[kt], 0, 0, 0, 0, 0, 0);
    }
}

// compile-time loop: f(integral_constant<int, I>) for I = 0..N-1
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(static_cast<F&&>(f));
  }
}

// IEEE maximum (NaN-propagating, so no operand canonicalisation; gfx950 has a
// three-input form).  Scores are never NaN; masked keys are -inf.
__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// maximum over the 16 scores of one S^T tile register set (and m), as a
// depth-3 tree of three-input maxima
__device__ __forceinline__ float tile_max(const v16f& t, float m) {
  const float a0 = fmax_ieee(fmax_ieee(t[0], t[1]), t[2]);
  const float a1 = fmax_ieee(fmax_ieee(t[3], t[4]), t[5]);
  const float a2 = fmax_ieee(fmax_ieee(t[6], t[7]), t[8]);
  const float a3 = fmax_ieee(fmax_ieee(t[9], t[10]), t[11]);
  const float a4 = fmax_ieee(fmax_ieee(t[12], t[13]), t[14]);
  const float b0 = fmax_ieee(fmax_ieee(a0, a1), a2);
  const float b1 = fmax_ieee(fmax_ieee(a3, a4), t[15]);
  return fmax_ieee(fmax_ieee(b0, b1), m);
}
__device__ __forceinline__ float tile_max(const v16f& t) { return tile_max(t, -__builtin_inff()); }

// Keeps a value computed here: the empty statement consumes it, so the
// compiler cannot sink the computation past this point (into a later, exposed
// part of the loop).  Emits no instruction.
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

// Issue order of one block step's matrix instructions.  Per 64-key step s:
// the S^T MFMAs of the NEXT block for key tiles 2s and 2s+1 (NDC each), the
// row-sum MFMA of this block's bytes P_s, then its NDT P.V MFMAs.  A score
// tile is overwritten only after ExpCast has consumed it, so the bytes of
// tile 0 are made first and the bytes of tiles 1.. are spread over the slots
// behind the MFMAs (RATE words of four bytes per slot after the first NDC
// slots, which carry tile 1); the next block's per-tile row maxima follow two
// slots after the MFMAs that produce the tile.  The wave issues in order, so
// vector work placed between two 64-cycle MFMAs runs in the matrix core's
// shadow.
template <int D, int KVB, int VF>
struct StepPlan {
  using TT = AttnTile<D, KVB, VF>;
  static_assert(!TT::SPLIT, "the two-part residuals take the two-phase step");
  static constexpr int NDC = TT::NDC, NKT = TT::NKT, NKS = TT::NKS, NDT = TT::NDT;
  static constexpr int NPV = NDT;                 // P.V MFMAs per 64 keys
  static constexpr int PER_S = 2 * NDC + 1 + NPV;
  static constexpr int M = NKS * PER_S;          // MFMAs per step
  static constexpr int NW = (NKT - 1) * 4;       // ExpCast words behind the MFMAs
  static constexpr int RATE = NDC == 1 ? 2 : 1;
  static constexpr int kind(int i) {             // 0: S^T, 1: row sum, 2: P.V
    return i % PER_S < 2 * NDC ? 0 : i % PER_S == 2 * NDC ? 1 : 2;
  }
  static constexpr int step_of(int i) { return i / PER_S; }
  static constexpr int qk_kt(int i) { return 2 * step_of(i) + (i % PER_S) / NDC; }
  static constexpr int qk_c(int i) { return (i % PER_S) % NDC; }
  static constexpr int pv_u(int i) { return i % PER_S - 2 * NDC - 1; }
  static constexpr int pv_T(int i) { return pv_u(i); }   // channel tile
  static constexpr int qk_slot(int kt) { return (kt / 2) * PER_S + (kt % 2) * NDC; }
  static constexpr int wbeg(int i) {
    const int w = i < NDC ? i * (4 / NDC) : 4 + (i - NDC) * RATE;
    return w < NW ? w : NW;
  }
  static constexpr int pm_slot(int kt) { return qk_slot(kt) + NDC + 1; }
  static constexpr bool valid() {
    for (int kt = 1; kt < NKT; ++kt)
      if (wbeg(qk_slot(kt)) < 4 * kt) return false;   // tile kt's bytes made before it is overwritten
    return wbeg(M) == NW;
  }
};

// acc += (mean/s_v)^T . rowsums of the last MS blocks on v_mfma_f32_32x32x16_bf16
// with both factors split into bf16 hi + lo (lane group 0 feeds the hi means,
// group 1 the lo means); runs after a chunk of MS row sums is complete.
template <int D, int KVB, int VF>
__device__ __forceinline__ void mean_flush(SoftmaxState<D / 32, AttnTile<D, KVB, VF>::MSLOT>& st,
                                           const uint16_t* sMhalf, int g, int col) {
  using TT = AttnTile<D, KVB, VF>;
  constexpr int NDT = TT::NDT, MS = TT::MSLOT;
  v4i bhi, blo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h, l;
    bf16_split2(st.RS[2 * i], st.RS[2 * i + 1], h, l);
    bhi[i] = static_cast<int>(h);
    blo[i] = static_cast<int>(l);
  }
  typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int T = 0; T < NDT; ++T) {
    const v4i a = *reinterpret_cast<const v4i*>(sMhalf + (g * D + 32 * T + col) * MS);
    st.acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, bhi),
                                                        st.acc[T], 0, 0, 0);
    st.acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, blo),
                                                        st.acc[T], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < MS; ++i) st.RS[i] = 0.0f;
}

// Where one lane's trace entries go in the test-only trace instantiation
// (all pointers null except in the one traced workgroup): per KV block b and
// query row, the scores after masking, the running maximum after the block,
// the block's log2-domain scale, the probability bytes and their row sum.
struct TraceRow {
  float* S = nullptr;     // [nblk][ROWS][KVB]
  uint8_t* P = nullptr;   // [nblk][ROWS][KVB]
  float* m = nullptr;     // [nblk][ROWS]
  float* c = nullptr;     // [nblk][ROWS]
  float* l = nullptr;     // [nblk][ROWS]
  int row = 0;            // query row of this lane inside the workgroup
};

// Trace stores of block b (test-only instantiation; lane (g, col) holds key
// 32*kt + 16*g + r of the block in S[kt][r], sorted order): the masked scores,
// the running maximum after the block and the block's log2-domain scale ...
template <int KVB, int NKT>
__device__ __forceinline__ void trace_scores(const TraceRow& tr, size_t trow, const v16f* S, float m_new, float cb,
                                             int g) {
  if (!tr.S) return;
  float* sp = tr.S + trow * KVB;
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<float4*>(sp + 32 * kt + 16 * g + 4 * r4) =
          make_float4(S[kt][4 * r4], S[kt][4 * r4 + 1], S[kt][4 * r4 + 2], S[kt][4 * r4 + 3]);
  if (g == 0) {
    tr.m[trow] = m_new;
    tr.c[trow] = cb;
  }
}
// ... and the probability bytes (word 4h + q of P[s] holds keys 64s + 32h +
// 16g + 4q .. +3) with their row sum
template <int KVB, int NKS>
__device__ __forceinline__ void trace_bytes(const TraceRow& tr, size_t trow, const v8i* P, float rs, int g) {
  if (!tr.S) return;
  uint8_t* pp = tr.P + trow * KVB;
#pragma unroll
  for (int s2 = 0; s2 < NKS; ++s2)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<uint4*>(pp + 64 * s2 + 32 * h + 16 * g) =
          make_uint4(static_cast<uint32_t>(P[s2][4 * h]), static_cast<uint32_t>(P[s2][4 * h + 1]),
                     static_cast<uint32_t>(P[s2][4 * h + 2]), static_cast<uint32_t>(P[s2][4 * h + 3]));
  if (g == 0) tr.l[trow] = rs;
}

// Masks the padded keys of the tail block, takes the row maximum across the
// two lane groups, moves the running maximum m (and with it the accumulator,
// the pending row sums and l) to max(m, c_b * rowmax S), and returns the word
// arguments of the probability bytes: ExpCast x = fma(S, 8c, 56 + beta - 8m),
// ExpCast off x = fma(S, c, -m), then exp2.  pmax: the per-lane maximum of S
// (recomputed here for the tail block).
template <int D, int KVB, int VF, int PM, bool MASK>
__device__ __forceinline__ void softmax_update(SoftmaxState<D / 32, AttnTile<D, KVB, VF>::MSLOT>& st, v16f* S,
                                               float& pmax, float cb, float kc, int nvalid, int g, float& A8,
                                               float& Bq) {
  using TT = AttnTile<D, KVB, VF>;
  constexpr int NKT = TT::NKT, NDT = TT::NDT, MS = TT::MSLOT;
  if constexpr (MASK) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const int lim = nvalid - ((kt >> 1) * 64 + (kt & 1) * 32 + 16 * g);   // keep r < lim
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r >= lim) S[kt][r] = -__builtin_inff();
    }
    pmax = tile_max(S[0]);
#pragma unroll
    for (int kt = 1; kt < NKT; ++kt) pmax = tile_max(S[kt], pmax);
  }
  const float mx = max_xor32(pmax);
  const float m_new = fmax_ieee(st.m_run, cb * mx);   // neither is NaN
  Bq = PM == 0 ? __builtin_fmaf(-8.0f, m_new, kc) : -m_new;
  A8 = PM == 0 ? 8.0f * cb : cb;

  // the accumulator moves to the new maximum before this block's P.V lands
  if (__builtin_amdgcn_ballot_w64(m_new > st.m_run)) {
    // the hardware exponential (one instruction; for a step below 2^-126
    // it may return 0 where a correctly rounded exp2 gives a subnormal)
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
#pragma unroll
    for (int T = 0; T < NDT; ++T)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[T][r] *= alpha;
#pragma unroll
    for (int i = 0; i < MS; ++i) st.RS[i] *= alpha;
    st.l_run *= alpha;
  }
  st.m_run = m_new;
}

// Row maximum, ExpCast, row sums and P.V of block b from its scores S, with
// the next block's S^T (into the same registers, tile by tile) interleaved
// as planned above.  pmax: per-lane maximum of S (before the cross-lane
// step); on return it holds the next block's.  hook(i) runs right after
// matrix instruction i is issued (the caller puts its direct loads there).
template <int D, int KVB, int VF, int PM, bool MASK, bool TR, typename Hook>
__device__ __forceinline__ void block_step(
    Hook&& hook, SoftmaxState<D / 32, AttnTile<D, KVB, VF>::MSLOT>& st, v16f* S, float& pmax,
    const uint8_t* sV, const uint8_t* sKn, const LaneOffsets<D, KVB, VF>& lo, const v8i* qb,
    float cb, float kc, int b, int slot, int nvalid, int g, int col, const TraceRow& tr) {
  using TT = AttnTile<D, KVB, VF>;
  using PL = StepPlan<D, KVB, VF>;
  static_assert(PL::valid(), "step plan overwrites a score tile before its bytes are made");
  constexpr int NKT = TT::NKT, NKS = TT::NKS, NDT = TT::NDT, VROW = TT::VROW, MS = TT::MSLOT;
  const uint8_t* sS = sV + TT::VBYTES;
  // Row sums on a 16x16x128 MFMA with P (E4M3) as its B operand.  Output
  // column n collects lanes n, n+16, n+32, n+48 of B, whose lane groups G
  // (of sixteen) hold query n for even G and n+16 for odd G; the FP8 B
  // operand of lane group G carries contraction indices 16G+s and
  // 64+16G+s, while the FP4 A operand carries 32G+s in nibble s, so A's
  // nibbles 0..15 meet even B groups and 16..31 odd ones (measured with a
  // one-wave probe).  A is 1.0 (E2M1) in the half whose parity matches the
  // row block of four that lane group receives in the 16x16 result (rows
  // 4(L/16)+i of lane L), so each lane gets the exact sum of its own query.
  const int rb = (col >> 2) & 1;     // (lane % 16) / 4, parity
  const int lo_one = rb ? 0 : 0x22222222, hi_one = rb ? 0x22222222 : 0;
  const v8i ones = {lo_one, lo_one, hi_one, hi_one, 0, 0, 0, 0};

  float A8, Bq;
  softmax_update<D, KVB, VF, PM, MASK>(st, S, pmax, cb, kc, nvalid, g, A8, Bq);
  [[maybe_unused]] const float m_new = st.m_run;
  // lane (g, col) holds key 32*kt + 16*g + r of block b in S[kt][r] (sorted order)
  [[maybe_unused]] const size_t trow = static_cast<size_t>(b) * TT::ROWS + tr.row;
  if constexpr (TR) trace_scores<KVB, NKT>(tr, trow, S, m_new, cb, g);

  v8i P[NKS];
  v4f rsum;
  // operand ring: loads run RD-1 matrix instructions ahead (two for E4M3 and
  // MXFP4; one for MXFP8, whose per-lane scales would otherwise push the
  // step past the register file)
  constexpr int RD = VF == 2 ? 2 : 3;
  v8i opnd[RD];
  // MX formats: the E8M0 scales of this lane for the NDT channel tiles of a
  // 64-key step, one byte each (stored adjacent), op_sel picks the tile's
  int osc[NKS];
  (void)osc;
  // operand of MFMA j into ring slot j % RD
  auto load_opnd = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if constexpr (j < PL::M) {
      if constexpr (PL::kind(j) == 0) {
        constexpr int kt = PL::qk_kt(j), c = PL::qk_c(j);
        opnd[j % RD] = join8(*reinterpret_cast<const uint4*>(sKn + kt * 32 * D + lo.k_rd[c][0]),
                            *reinterpret_cast<const uint4*>(sKn + kt * 32 * D + lo.k_rd[c][1]));
      } else if constexpr (PL::kind(j) == 2) {
        constexpr int sj = PL::step_of(j), T = PL::pv_T(j);
        const uint8_t* vb = sV + (sj * D + 32 * T) * VROW;
        if constexpr (VF != 1) {
          opnd[j % RD] = join8(*reinterpret_cast<const uint4*>(vb + lo.v_rd[0]),
                              *reinterpret_cast<const uint4*>(vb + lo.v_rd[1]));
        } else {
          const uint4 q = *reinterpret_cast<const uint4*>(vb + lo.v_rd[0]);
          opnd[j % RD] = v8i{static_cast<int>(q.x), static_cast<int>(q.y), static_cast<int>(q.z),
                            static_cast<int>(q.w), 0, 0, 0, 0};
        }
        // lane group g's scale covers contraction block g, i.e. sorted
        // positions [32g, 32g+32) of the step (measured for both MX formats)
        if constexpr (VF != 0 && PL::pv_u(j) == 0) {
          const uint8_t* sc = sS + (2 * sj + g) * D + col * NDT;
          if constexpr (NDT == 4) osc[sj] = *reinterpret_cast<const int*>(sc);
          else osc[sj] = *reinterpret_cast<const uint16_t*>(sc);
        }
      }
    }
  };
  // ExpCast word w of the tiles behind tile 0 (tile 1 + w/4, word w%4)
  auto ecast = [&](auto wc) {
    constexpr int w = decltype(wc)::value;
    constexpr int kt = 1 + w / 4, q = w % 4;
    const v16f& sv = S[kt];
    P[kt / 2][4 * (kt % 2) + q] =
        static_cast<int>(pword4<PM>(sv[4 * q], sv[4 * q + 1], sv[4 * q + 2], sv[4 * q + 3], A8, Bq));
  };

  static_for<RD - 1>([&](auto jc) { load_opnd(jc); });
#pragma unroll
  for (int q = 0; q < 4; ++q)
    P[0][q] = static_cast<int>(pword4<PM>(S[0][4 * q], S[0][4 * q + 1], S[0][4 * q + 2], S[0][4 * q + 3], A8, Bq));
  __builtin_amdgcn_sched_barrier(0);

  static_for<PL::M>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    load_opnd(std::integral_constant<int, i + RD - 1>{});
    if constexpr (PL::kind(i) == 0) {
      constexpr int kt = PL::qk_kt(i), c = PL::qk_c(i);
      S[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(opnd[i % RD], qb[c], c == 0 ? v16f{} : S[kt], 0, 0,
                                                             0, 0, 0, 0);
    } else if constexpr (PL::kind(i) == 1) {
      constexpr int sj = PL::step_of(i);
      // row sums of the decoded bytes on the matrix core (exact: multiples of
      // 2^-9 below 2^8)
      rsum = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, P[sj], sj == 0 ? v4f{} : rsum, 4, 0, 0, 127, 0,
                                                              127);
    } else {
      constexpr int sj = PL::step_of(i), T = PL::pv_T(i);
      if constexpr (VF == 0)
        st.acc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(opnd[i % RD], P[sj], st.acc[T], 0, 0, 0, 0, 0,
                                                                   0);
      else if constexpr (VF == 2)
        st.acc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(opnd[i % RD], P[sj], st.acc[T], 0, 0, T,
                                                                   osc[sj], 0, 127);
      else
        st.acc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(opnd[i % RD], P[sj], st.acc[T], 4, 0, T,
                                                                   osc[sj], 0, 127);
    }
    static_for<PL::wbeg(i + 1) - PL::wbeg(i)>([&](auto kc2) {
      ecast(std::integral_constant<int, PL::wbeg(i) + decltype(kc2)::value>{});
    });
    static_for<NKT>([&](auto ktc) {
      constexpr int kt = decltype(ktc)::value;
      if constexpr (PL::pm_slot(kt) == i) {
        pmax = kt == 0 ? tile_max(S[0]) : tile_max(S[kt], pmax);
        pin(pmax);
      }
    });
    hook(ic);
    __builtin_amdgcn_sched_barrier(0);
  });
  static_for<NKT>([&](auto ktc) {
    constexpr int kt = decltype(ktc)::value;
    if constexpr (PL::pm_slot(kt) >= PL::M) pmax = kt == 0 ? tile_max(S[0]) : tile_max(S[kt], pmax);
  });

  const float rs = rsum[0];
  if constexpr (TR) trace_bytes<KVB, NKS>(tr, trow, P, rs, g);
  st.l_run += rs;
#pragma unroll
  for (int i = 0; i < MS; ++i) st.RS[i] = i == slot ? rs : st.RS[i];
}

// Block b in two phases (the NVFP4-style residuals): S^T of block b from its
// staged K, the softmax update and ExpCast of all its scores, then the row
// sums and P.V (two scaled MFMAs per channel tile and 64 keys: the high and
// the low E4M3 parts under one E8M0 byte).  Only the accumulator, the bytes
// and one operand pair stay live in the second phase.  hook(i) runs right
// after matrix instruction i is issued (QK^T: 0 .. NKT*NDC-1, then per 64
// keys the row sum and the P.V MFMAs).
template <int D, int KVB, int VF, int PM, bool MASK, bool TR, typename Hook>
__device__ __forceinline__ void block_step_split(
    Hook&& hook, SoftmaxState<D / 32, AttnTile<D, KVB, VF>::MSLOT>& st, v16f* S, const uint8_t* sV,
    const uint8_t* sK, const LaneOffsets<D, KVB, VF>& lo, const v8i* qb, float cb, float kc, int b, int slot,
    int nvalid, int g, int col, const TraceRow& tr) {
  using TT = AttnTile<D, KVB, VF>;
  constexpr int NKT = TT::NKT, NKS = TT::NKS, NDT = TT::NDT, NDC = TT::NDC, VROW = TT::VROW, MS = TT::MSLOT;
  constexpr int NQK = NKT * NDC, NPV = 2 * NDT;
  static_assert(VF == 3, "the two-phase step serves the two-part residuals");
  const uint8_t* sS = sV + TT::VBYTES;
  // row-sum operand: see block_step
  const int rb = (col >> 2) & 1;
  const int lo_one = rb ? 0 : 0x22222222, hi_one = rb ? 0x22222222 : 0;
  const v8i ones = {lo_one, lo_one, hi_one, hi_one, 0, 0, 0, 0};

  // phase 1: scores, softmax update, bytes
  static_for<NQK>([&](auto ic) {
    constexpr int i = decltype(ic)::value, kt = i / NDC, c = i % NDC;
    const v8i a = join8(*reinterpret_cast<const uint4*>(sK + kt * 32 * D + lo.k_rd[c][0]),
                        *reinterpret_cast<const uint4*>(sK + kt * 32 * D + lo.k_rd[c][1]));
    S[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qb[c], c == 0 ? v16f{} : S[kt], 0, 0, 0, 0, 0, 0);
    hook(ic);
    __builtin_amdgcn_sched_barrier(0);
  });
  float pmax = tile_max(S[0]);
#pragma unroll
  for (int kt = 1; kt < NKT; ++kt) pmax = tile_max(S[kt], pmax);
  float A8, Bq;
  softmax_update<D, KVB, VF, PM, MASK>(st, S, pmax, cb, kc, nvalid, g, A8, Bq);
  [[maybe_unused]] const size_t trow = static_cast<size_t>(b) * TT::ROWS + tr.row;
  if constexpr (TR) trace_scores<KVB, NKT>(tr, trow, S, st.m_run, cb, g);
  v8i P[NKS];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      P[kt / 2][4 * (kt % 2) + q] = static_cast<int>(
          pword4<PM>(S[kt][4 * q], S[kt][4 * q + 1], S[kt][4 * q + 2], S[kt][4 * q + 3], A8, Bq));

  // phase 2: row sums and P.V; operand u of a 64-key step is channel tile
  // u/2, part u%2 (0 high, 1 low), loaded one MFMA ahead
  v4f rsum;
  auto vopnd = [&](int sj, int u) __attribute__((always_inline)) -> v8i {
    const uint8_t* vb = sV + (u % 2) * TT::VHALF + (sj * D + 32 * (u / 2)) * VROW;
    return join8(*reinterpret_cast<const uint4*>(vb + lo.v_rd[0]), *reinterpret_cast<const uint4*>(vb + lo.v_rd[1]));
  };
  static_for<NKS>([&](auto sc) {
    constexpr int sj = decltype(sc)::value;
    // lane group g's E8M0 bytes cover sorted positions [32g, 32g+32) of the
    // step, one byte per channel tile (op_sel picks it)
    const uint8_t* scp = sS + (2 * sj + g) * D + col * NDT;
    int osc;
    if constexpr (NDT == 4) osc = *reinterpret_cast<const int*>(scp);
    else osc = *reinterpret_cast<const uint16_t*>(scp);
    v8i cur = vopnd(sj, 0);
    constexpr int base = NQK + sj * (1 + NPV);
    rsum = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, P[sj], sj == 0 ? v4f{} : rsum, 4, 0, 0, 127, 0,
                                                            127);
    hook(std::integral_constant<int, base>{});
    static_for<NPV>([&](auto uc) {
      constexpr int u = decltype(uc)::value, T = u / 2;
      const v8i nxt = u + 1 < NPV ? vopnd(sj, u + 1) : cur;
      st.acc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur, P[sj], st.acc[T], 0, 0, T, osc, 0, 127);
      hook(std::integral_constant<int, base + 1 + u>{});
      __builtin_amdgcn_sched_barrier(0);
      cur = nxt;
    });
  });
  const float rs = rsum[0];
  if constexpr (TR) trace_bytes<KVB, NKS>(tr, trow, P, rs, g);
  st.l_run += rs;
#pragma unroll
  for (int i = 0; i < MS; ++i) st.RS[i] = i == slot ? rs : st.RS[i];
}

// The fused forward.  Per workgroup 256 query rows (8 waves x 32 rows, two
// 128-row tiles with a query scale each), so every staged K/V block serves
// 256 queries.  Block b+1's S^T MFMAs run inside block b's step, so each block
// starts with its scores ready: K is staged two blocks ahead and V one block
// ahead, each in a two-slot LDS ring filled by direct buffer->LDS loads.  The
// NVFP4-style residuals (two P.V MFMAs per tile) take the two-phase step
// instead, with K and V both staged one block ahead.
// TR = 1: the test-only trace instantiation (same arithmetic; the workgroup
// with logical index p.tr_wg also writes its TraceRow entries).
template <int D, int KVB, int VF, int O32, int PM, int TR>
__global__ __launch_bounds__(kAttnThreads, 1) void k_attn_fwd(AttnArgs p) {
  using TT = AttnTile<D, KVB, VF>;
  static_assert(kQTile == 4 * 32 && TT::ROWS % kQTile == 0, "a query scale tile is four waves");
  constexpr int NDC = TT::NDC, NKT = TT::NKT, NDT = TT::NDT;
  constexpr int MS = TT::MSLOT;
  constexpr int VSTAGE = TT::VBYTES + (TT::SBYTES + 1023) / 1024 * 1024;
  // Every ring slot is an LDS object of its own and every block step below
  // names its slots at compile time: the compiler then knows that a step's
  // operand reads do not touch the slots its direct loads are filling, and
  // does not make those reads wait for the loads.
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[TT::KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[TT::KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[VSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[VSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t sM[2 * 2 * D * MS];   // [2 halves][2 hi/lo][D][MS]
  __shared__ __attribute__((aligned(16))) float sCol[D];
  __shared__ float sRcol[D];      // 1 / column scale: block means enter the accumulator in residual units
  __shared__ float sRed[TT::NWV];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5, col = lane & 31;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // the wave index in a scalar register
  const int N = p.N, nblk = p.nblk;
  const int nqt = (N + TT::ROWS - 1) / TT::ROWS;
  // Workgroups reach the 8 XCDs round-robin by index; renumber them so that
  // each XCD takes a contiguous range of (head, query tile) pairs, and the
  // workgroups sharing an XCD's L2 stream the same heads' blocks.
  const int wg = xcd_major_index(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int bh = wg / nqt, qt = wg % nqt;
  const int qrow = qt * TT::ROWS + wave * 32 + col;
  TraceRow tr;
  tr.row = wave * 32 + col;
  if constexpr (TR != 0) {
    if (wg == p.tr_wg) {
      tr.S = p.tr_S;
      tr.P = p.tr_P;
      tr.m = p.tr_m;
      tr.c = p.tr_c;
      tr.l = p.tr_l;
    }
  }

  const uint8_t* kq = p.Kq + static_cast<size_t>(bh) * nblk * KVB * D;
  const uint8_t* vr = p.Vres + static_cast<size_t>(bh) * nblk * TT::VBYTES;
  const uint8_t* scb = VF != 0 ? reinterpret_cast<const uint8_t*>(p.v_scale) +
                                     static_cast<size_t>(bh) * nblk * (KVB / 32) * D
                               : nullptr;
  const float* ks = p.k_scale + static_cast<size_t>(bh) * nblk;
  const float* vm = p.v_mean + static_cast<size_t>(bh) * nblk * D;
  const LaneOffsets<D, KVB, VF> lo(lane);

  // slot j & 1 of each ring, chosen at compile time
  auto kslot = [&](auto par) -> uint8_t* {
    if constexpr (decltype(par)::value) return sK1; else return sK0;
  };
  auto vslot = [&](auto par) -> uint8_t* {
    if constexpr (decltype(par)::value) return sV1; else return sV0;
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // direct loads address this head's Kq, residual rows and E8M0 scales
  // through buffer descriptors: block offset in a scalar, lane offset fixed
  const uint32_t kq_bytes = static_cast<uint32_t>(nblk) * TT::KBYTES;
  const uint32_t vr_bytes = static_cast<uint32_t>(nblk) * TT::VBYTES;
  const uint32_t sc_bytes = VF != 0 ? static_cast<uint32_t>(nblk) * TT::SBYTES : 0u;
  // K_j into slot par = j & 1 (direct-load rounds [R0, R1))
  auto stage_k = [&](int j, auto par, auto r0, auto r1) {
    stage_block_k<D, KVB, VF, decltype(r0)::value, decltype(r1)::value>(
        kslot(par), kq, kq_bytes, static_cast<uint32_t>(j) * TT::KBYTES, lo, wave_s);
  };
  // V_j (and its E8M0 scales) into slot par = j & 1 (rounds [R0, R1))
  auto stage_v = [&](int j, auto par, auto r0, auto r1) {
    stage_block_v<D, KVB, VF, decltype(r0)::value, decltype(r1)::value>(
        vslot(par), vr, vr_bytes, static_cast<uint32_t>(j) * TT::VBYTES, scb, sc_bytes,
        static_cast<uint32_t>(j) * TT::SBYTES, lo, wave_s, lane);
  };
  using RA = std::integral_constant<int, 0>;    // all rounds: [0, 64)
  using RB = std::integral_constant<int, 64>;
  stage_k(0, P0{}, RA{}, RB{});
  stage_v(0, P0{}, RA{}, RB{});
  if constexpr (!TT::SPLIT) {
    if (nblk > 1) stage_k(1, P1{}, RA{}, RB{});
  }

  for (int i = threadIdx.x; i < 2 * 2 * D * MS; i += TT::NTH) sM[i] = 0;
  float colv = 1.0f;
  if (threadIdx.x < D) {
    if (VF == 0) colv = reinterpret_cast<const float*>(p.v_scale)[static_cast<size_t>(bh) * D + threadIdx.x];
    sCol[threadIdx.x] = colv;
    sRcol[threadIdx.x] = 1.0f / colv;
  }
  const float rcol = 1.0f / colv;

  // ---- query tile: E4M3 codes with one scale per 128 rows ----
  v8i qb[NDC];
  float cq;
  {
    float qv[NDC][32];
    float am = 0.0f;
    const uint16_t* qp = p.Q + (static_cast<size_t>(bh) * N + qrow) * D;
#pragma unroll
    for (int c = 0; c < NDC; ++c)
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
    am = wave_max(am);
    if (lane == 0) sRed[wave] = am;
    __syncthreads();
    const float* tr = sRed + (wave & ~3);      // the four waves of this wave's 128-row scale tile
    const float amax = fmaxf(fmaxf(tr[0], tr[1]), fmaxf(tr[2], tr[3]));
    const float sq = amax > 0.0f ? fmaxf(amax / 448.0f, kScaleFloor) : 1.0f;
    const float yq = 1.0f / sq;
    // codes of fp32(q / s_q) (correctly rounded quotient, see div_rn), round to
    // nearest even by the packed convert; |q / s_q| <= 448 (up to one rounding
    // of s_q, well below 464 where the non-saturating convert would overflow)
#pragma unroll
    for (int c = 0; c < NDC; ++c)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float* x = &qv[c][4 * w];
        const uint32_t word = e4m3x4(div_rn(x[0], sq, yq), div_rn(x[1], sq, yq), div_rn(x[2], sq, yq),
                                     div_rn(x[3], sq, yq));
        qb[c][w] = static_cast<int>(word);
      }
    const float t = sq * p.scale;
    cq = t * kLog2e;
  }

  // mean of block 0 into the restoration ring (slot 0 of half 0)
  if (threadIdx.x < D) {
    uint32_t hi, lo;
    bf16_split2(vm[threadIdx.x] * rcol, 0.0f, hi, lo);
    sM[(0 * D + threadIdx.x) * MS + 0] = static_cast<uint16_t>(hi);
    sM[(1 * D + threadIdx.x) * MS + 0] = static_cast<uint16_t>(lo);
  }

  SoftmaxState<NDT, MS> st;
  st.m_run = -__builtin_inff();
  st.l_run = 0.0f;
#pragma unroll
  for (int T = 0; T < NDT; ++T) st.acc[T] = v16f{};
#pragma unroll
  for (int i = 0; i < MS; ++i) st.RS[i] = 0.0f;

  // block scales travel one step ahead in a register: a load issued inside a
  // step would make its first use wait on the block loads issued before it
  float k_cur = ks[0];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  v16f S[NKT];
  float pmax = 0.0f;
  if constexpr (!TT::SPLIT) {
    qk_block<D, KVB, VF>(S, sK0, lo, qb);
    pmax = tile_max(S[0]);
#pragma unroll
    for (int kt = 1; kt < NKT; ++kt) pmax = tile_max(S[kt], pmax);
    // every wave has read K_0 before the first step refills its slot
    __syncthreads();
  }

  const int ntail = N - (nblk - 1) * KVB;            // real keys of the last block
  const int nfull = ntail < KVB ? nblk - 1 : nblk;   // blocks without padded keys

  // one block step: softmax and P.V of block b from S, then (into the same
  // registers, whose scores ExpCast has consumed) S^T of block b+1, whose K
  // was staged two blocks ahead; the mean flush follows (par = b & 1 names
  // the slots: V_b and K_{b+2} in slot par, K_{b+1} and V_{b+1} in the
  // other).  The direct loads of K_{b+2} and V_{b+1} are spread over the
  // step, one round (one instruction per wave) behind every second matrix
  // instruction: issued together at the step's start, the eight waves' loads
  // queue up and hold the waves back.
  auto step = [&](const int b, auto par, auto masked, const int slot) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(masked)::value;
    constexpr int PAR = decltype(par)::value;
    using Q = std::integral_constant<int, 1 - PAR>;
    using PL = StepPlan<D, KVB, VF>;
    using LO = LaneOffsets<D, KVB, VF>;
    float mnext = 0.0f, k_next = 0.0f;
    if (b + 1 < nblk) {
      k_next = ks[b + 1];
      if (threadIdx.x < D) mnext = vm[static_cast<size_t>(b + 1) * D + threadIdx.x];
    }
    if constexpr (TT::SPLIT) {
      // two-phase step: K_{b+1} and V_{b+1} into the other slots, K round r
      // behind matrix instruction 4r, V round r behind 4r+2
      constexpr int M = NKT * NDC + TT::NKS * (1 + 2 * NDT);
      auto hook = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        static_for<LO::KR>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          constexpr int at = 4 * r;
          if constexpr (i == (at < M ? at : M - 1)) {
            if (b + 1 < nblk) stage_k(b + 1, Q{}, rc, std::integral_constant<int, r + 1>{});
          }
        });
        static_for<LO::VR>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          constexpr int at = 4 * r + 2;
          if constexpr (i == (at < M ? at : M - 1)) {
            if (b + 1 < nblk) stage_v(b + 1, Q{}, rc, std::integral_constant<int, r + 1>{});
          }
        });
      };
      block_step_split<D, KVB, VF, PM, MASK, TR != 0>(hook, st, S, vslot(par), kslot(par), lo, qb, cq * k_cur,
                                                       p.kc, b, slot, MASK ? ntail : KVB, g, col, tr);
    } else {
      // K round r behind matrix instruction 4r, V round r behind 4r+2
      auto hook = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        static_for<LO::KR>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          constexpr int at = 4 * r;
          if constexpr (i == (at < PL::M ? at : PL::M - 1)) {
            if (b + 2 < nblk) stage_k(b + 2, par, rc, std::integral_constant<int, r + 1>{});
          }
        });
        static_for<LO::VR>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          constexpr int at = 4 * r + 2;
          if constexpr (i == (at < PL::M ? at : PL::M - 1)) {
            if (b + 1 < nblk) stage_v(b + 1, Q{}, rc, std::integral_constant<int, r + 1>{});
          }
        });
      };
      // softmax and P.V of block b, with block b+1's scores made in between
      // (for the last block they come from a stale slot and are discarded)
      block_step<D, KVB, VF, PM, MASK, TR != 0>(hook, st, S, pmax, vslot(par), kslot(Q{}), lo, qb, cq * k_cur,
                                                p.kc, b, slot, MASK ? ntail : KVB, g, col, tr);
    }
    if (slot == MS - 1 || b == nblk - 1)
      mean_flush<D, KVB, VF>(st, sM + ((b >> 3) & 1) * 2 * D * MS, g, col);
    if (b + 1 < nblk && threadIdx.x < D) {
      const int nb = b + 1;
      uint32_t hi, lo;
      bf16_split2(mnext * sRcol[threadIdx.x], 0.0f, hi, lo);
      uint16_t* mh = sM + ((nb >> 3) & 1) * 2 * D * MS;
      mh[(0 * D + threadIdx.x) * MS + ((slot + 1) & (MS - 1))] = static_cast<uint16_t>(hi);
      mh[(1 * D + threadIdx.x) * MS + ((slot + 1) & (MS - 1))] = static_cast<uint16_t>(lo);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    k_cur = k_next;
  };

  int b = 0;
  for (; b + 2 <= nfull; b += 2) {
    step(b, P0{}, std::false_type{}, b & (MS - 1));
    step(b + 1, P1{}, std::false_type{}, (b + 1) & (MS - 1));
  }
  if (b < nfull) {
    step(b, P0{}, std::false_type{}, b & (MS - 1));
    ++b;
  }
  if (nfull < nblk) {      // b == nblk - 1
    if (b & 1) step(b, P1{}, std::true_type{}, b & (MS - 1));
    else step(b, P0{}, std::true_type{}, b & (MS - 1));
  }

  // ---- O = s_v * acc / l ----
  if (qrow < N) {
    const float inv_l = 1.0f / st.l_run;
#pragma unroll
    for (int T = 0; T < NDT; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c0 = 32 * T + 8 * i + 4 * g;
        const float4 cs = *reinterpret_cast<const float4*>(sCol + c0);
        // 1/l first: acc / l is of the order of the residual codes, so the
        // column scale (as small as 2^-126) does not push it into subnormals
        const float o0 = st.acc[T][4 * i + 0] * inv_l * cs.x;
        const float o1 = st.acc[T][4 * i + 1] * inv_l * cs.y;
        const float o2 = st.acc[T][4 * i + 2] * inv_l * cs.z;
        const float o3 = st.acc[T][4 * i + 3] * inv_l * cs.w;
        const size_t off = (static_cast<size_t>(bh) * N + qrow) * D + c0;
        if constexpr (O32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.O) + off) = make_float4(o0, o1, o2, o3);
        } else {
          // bf16 round to nearest even (v_cvt_pk_bf16_f32)
          const uint32_t w0 = __builtin_bit_cast(uint32_t, v2bf{static_cast<__bf16>(o0), static_cast<__bf16>(o1)});
          const uint32_t w1 = __builtin_bit_cast(uint32_t, v2bf{static_cast<__bf16>(o2), static_cast<__bf16>(o3)});
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.O) + off) = make_uint2(w0, w1);
        }
      }
  }
}

// Launches the forward for one (head dim, KV block, residual format); the
// instantiations live in attn_inst.hip, one object file per combination.
template <int D, int KVB, int VF>
hipError_t launch_attn_cfg(const AttnArgs& a, hipStream_t st) {
  using TT = AttnTile<D, KVB, VF>;
  const int nqt = (a.N + TT::ROWS - 1) / TT::ROWS;
  const dim3 grid(static_cast<unsigned>(a.B * a.H * nqt));
  const dim3 blk(TT::NTH);
  if (a.tr_S) {
    if (a.pm == 0) hipLaunchKernelGGL((k_attn_fwd<D, KVB, VF, 1, 0, 1>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_attn_fwd<D, KVB, VF, 1, 1, 1>), grid, blk, 0, st, a);
  } else if (a.out_fp32) {
    if (a.pm == 0) hipLaunchKernelGGL((k_attn_fwd<D, KVB, VF, 1, 0, 0>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_attn_fwd<D, KVB, VF, 1, 1, 0>), grid, blk, 0, st, a);
  } else {
    if (a.pm == 0) hipLaunchKernelGGL((k_attn_fwd<D, KVB, VF, 0, 0, 0>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_attn_fwd<D, KVB, VF, 0, 1, 0>), grid, blk, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace vc
