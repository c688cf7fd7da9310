// Device helpers and the fp32 chunk record shared by the backward kernels
// (kda_bwd.hip, kda_bwd_grad.hip).  Internal header: not part of the C ABI.
#pragma once

#include "kda_bwd.h"

namespace kda {

constexpr int QP = KD + 4;  // pitch (floats) of [64][128] LDS tiles
constexpr int MP = CH + 4;  // pitch of [64][64] LDS tiles
constexpr int VH = VD / 2;  // state columns per recurrence workgroup

// Chunk record of the backward (offsets in floats).  T and KK are fp32,
// row-major.  The four operands of the reverse recurrence are bf16 hi/lo
// pairs in the forward record's MFMA fragment order (frag_tc / frag_tt /
// frag_ct): the hi array of a region, then its lo array.  The output scale is
// folded into A_qk^T and QG^T, and W^T is stored negated.
constexpr int BR_T = 0;                   // T = (I + diag(beta) KK)^-1, unit lower, [64][64] row-major
constexpr int BR_KK = BR_T + CH * CH;     // KK = K^ K^T . decay, strictly lower,     [64][64] row-major
constexpr int BR_AQKT = BR_KK + CH * CH;  // scale A_qk^T (rows i, contraction j),  frag_tt, hi + lo
constexpr int BR_WT = BR_AQKT + CH * CH;  // -W^T (rows k, contraction i),          frag_ct, hi + lo
constexpr int BR_KT = BR_WT + CH * KD;    // Kt = K^ exp(G_L - G) (rows i, contraction k), frag_tc, hi + lo
constexpr int BR_QGT = BR_KT + CH * KD;   // scale QG^T (rows k, contraction i),     frag_ct, hi + lo
constexpr int BR_GL = BR_QGT + CH * KD;   // exp(G_L)                                 [128]
constexpr int BR_BETA = BR_GL + KD;       // beta                                     [64]
static_assert(BR_BETA + CH == BWD_REC_FLOATS, "record size");

// Store x0..x3 (4 consecutive fragment elements starting at idx) of an n-element
// bf16 hi/lo region: hi at idx, lo = x - hi at n + idx.
__device__ __forceinline__ void store_hl4(float* region, int n, int idx, float x0, float x1, float x2, float x3) {
  __bf16* hi = reinterpret_cast<__bf16*>(region);
  const float x[4] = {x0, x1, x2, x3};
  bf16x4 h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = (__bf16)x[e];
    l[e] = (__bf16)(x[e] - (float)h[e]);
  }
  *reinterpret_cast<bf16x4*>(hi + idx) = h;
  *reinterpret_cast<bf16x4*>(hi + n + idx) = l;
}

__device__ __forceinline__ void split_hl8(const float (&x)[8], bf16x8& h, bf16x8& l) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (__bf16)x[e];
    l[e] = (__bf16)(x[e] - (float)h[e]);
  }
}
// 8 consecutive floats from global memory as a bf16 hi/lo pair
__device__ __forceinline__ void ld_hl8(const float* p, bf16x8& h, bf16x8& l) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  split_hl8(x, h, l);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float el(const float4& v, int s) {
  return s == 0 ? v.x : (s == 1 ? v.y : (s == 2 ? v.z : v.w));
}
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even (finite inputs)
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + expf(-x)); }
// sigmoid from the hardware exp2 and reciprocal (about 2 ulp; 0 and 1 at the ends)
__device__ __forceinline__ float fsigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + fexp2(-x * LOG2E)); }

// (sequence, first token, length) of global chunk gch
__device__ __forceinline__ void chunk_of(const ChunkMap& m, int64_t gch, int64_t& c0, int& L) {
  const int seq = chunk_owner(m, gch);
  int64_t bos, eos;
  seq_bounds(m, seq, bos, eos);
  c0 = bos + (gch - first_chunk(m, seq)) * CH;
  L = (int)((eos - c0) < CH ? (eos - c0) : CH);
}

__device__ __forceinline__ void split_hl4(const f32x4& x, bf16x4& h, bf16x4& l) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = (__bf16)x[e];
    l[e] = (__bf16)(x[e] - (float)h[e]);
  }
}

// 16x16x16 bf16 MFMA: lane (gq, tl) supplies A[tl][4gq + 0..3] and
// B[4gq + 0..3][tl], the layout of four steps of the fp32 16x16x4 MFMA.
// Operands are fp32 values split into bf16 hi/lo pairs (three passes).
typedef short s16x4 __attribute__((ext_vector_type(4)));
struct HL4 {
  bf16x4 h, l;
};
__device__ __forceinline__ HL4 hl4(float x0, float x1, float x2, float x3) {
  HL4 r;
  split_hl4(f32x4{x0, x1, x2, x3}, r.h, r.l);
  return r;
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_hl(const HL4& a, const HL4& b, f32x4 c) {
  c = mfma16(a.h, b.h, c);
  c = mfma16(a.h, b.l, c);
  c = mfma16(a.l, b.h, c);
  return c;
}

// Sums over the lanes of a 16-lane DPP row without the LDS crossbar: xor 1
// and xor 2 by quad permutes, then the half-row and row mirrors (after each
// step the lanes being paired hold equal partial sums, so a mirror is an
// exchange).  sum8 stops after 8 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp<0x141>(x);  // row_half_mirror
  return x;
}
__device__ __forceinline__ float sum16(float x) { return sum8(x) + dpp<0x140>(sum8(x)); }  // + row_mirror

}  // namespace kda
