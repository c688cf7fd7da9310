// KDA chunked forward for MI355X (gfx950): one fused kernel + a tiny varlen
// scheduling kernel, and the C ABI declared in include/kda.h.
//
// Method (per sequence n, head h; 64-token chunks, partial tail allowed).
// The pages fix the op and its arguments (vLLM PR report "[Kimi-K3] Bump
// FlashKDA to fix unstable inverse", section "关键源码片段"; instagit FlashKDA
// page, "Usage Examples": chunk_kda with in-kernel L2 norm, beta sigmoid and
// gate) but print neither the recurrence nor the chunk algebra.  The chunk
// algebra below is derived from the per-token gated delta rule
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = scale S_t^T q_t.
// For one chunk of L <= 64 tokens, start state S0 and per-channel cumulative
// log-decay G_i (reset at the chunk start):
//     A_kk[i,j] = b_i <k_i * exp(G_i - G_j), k_j>   (j < i)      T = (I + A_kk)^-1
//     W = T diag(b) (K * exp(G))      U = T diag(b) V      D = U - W S0
//     A_qk[i,j] = <q_i * exp(G_i - G_j), k_j>       (j <= i)
//     O  = scale [ (Q * exp(G)) S0 + A_qk D ]
//     S_L = Diag(exp(G_L)) S0 + (K * exp(G_L - G))^T D
// (q, k here are L2-normalised.)  The decay ratios exp(G_i - G_j) are never
// formed as exp(G_i) * exp(-G_j), which would span exp(+-320) at
// lower_bound = -5.  Instead the chunk is cut into four 16-token sub-chunks
// and every ratio is split through a per-channel reference point between j
// and i (for the diagonal 16x16 blocks the reference is the sub-chunk start,
// so one factor is >= 1 but <= exp(16*5) < FLT_MAX, still inside bf16 range).
//
// Work decomposition: one workgroup (4 waves, 256 threads) per
// (sequence, head, V-half); it walks the sequence's chunks in order and keeps
// its 128 x 64 fp32 slice of the state in MFMA accumulator registers the whole
// time.  Per chunk:
//   1 prep      wave w handles tokens 16w..16w+15: bf16 loads, L2 norms, gate,
//               16-lane DPP scan of the log-decay; every operand of the chunk is
//               formed once and staged in LDS.
//   2 A blocks  wave w computes row-block w of A_kk (bf16 hi/lo, 3 MFMA passes)
//               and A_qk (1 pass).
//   3 inverse   T = (I + A_kk)^-1 in fp32: 16x16 diagonal blocks by forward
//               substitution, off-diagonal blocks by fp32 MFMA.
//   4 W, U      W = T diag(b) K^G (fp16 hi/lo, 3 passes), U = T diag(b) V
//               (bf16 hi/lo x exact bf16 V, 2 passes).
//   5 state     D = U - W S; O = QG S + A_qk D; S = G_L S + Kt^T D
//               (Kt and D as fp16 hi/lo, 3 passes), fp32 accumulation.
// Precision of each product was chosen so that the final state stays within
// 1e-3 relative L2 of an fp64 reference even for identical (collinear) keys,
// where the chunk sums telescope and 16-bit rounding of T, W, Kt or D alone
// would exceed it.
//
// fp16 operands assume |v|, |state|, |D| stay below 6.5e4.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/kda.h"

namespace {

constexpr int KD = 128;          // head dim K
constexpr int VD = 128;          // head dim V
constexpr int CH = 64;           // chunk length
constexpr int NV = 2;            // V slices per (sequence, head)
constexpr int VT = VD / NV;      // 64 state columns per workgroup
constexpr int NTHREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float L2_EPS = 1e-6f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- LDS carve-up (bytes) -------------------------------------------------
// token-row arrays: [token][channel], row pitch KP halves; channel-row arrays:
// [channel][token], row pitch TP halves; fp32 square arrays pitch AP floats.
constexpr int KP = KD + 8;   // 136 halves = 272 B
constexpr int TP = CH + 8;   // 72 halves = 144 B (16-byte aligned rows)
constexpr int AP = CH + 4;   // 68 floats
constexpr int TBP = CH + 8;  // 72 halves

// region R1: sKRF (prep -> A blocks) aliased with the four T*diag(b) copies
constexpr int OFF_KRF_HI = 0;                               // bf16 [48][KP]
constexpr int OFF_KRF_LO = OFF_KRF_HI + 48 * KP * 2;
constexpr int OFF_TB16_HI = 0;                              // f16 [64][TBP]
constexpr int OFF_TB16_LO = OFF_TB16_HI + CH * TBP * 2;
constexpr int OFF_TBB_HI = OFF_TB16_LO + CH * TBP * 2;      // bf16 [64][TBP]
constexpr int OFF_TBB_LO = OFF_TBB_HI + CH * TBP * 2;
constexpr int R1_END = OFF_TBB_LO + CH * TBP * 2;           // 36864
static_assert(OFF_KRF_LO + 48 * KP * 2 <= R1_END, "R1");
// region R2: A_kk / T (fp32) aliased with -W (f16 token-row)
constexpr int OFF_A = R1_END;                               // f32 [64][AP]
constexpr int OFF_W = R1_END;                               // f16 [64][KP]
constexpr int R2_END = OFF_A + CH * AP * 4;
static_assert(CH * KP * 2 <= CH * AP * 4, "R2");
constexpr int OFF_KG = R2_END;                              // f16 [128][TP]
constexpr int OFF_KT_HI = OFF_KG + KD * TP * 2;             // f16 [128][TP]
constexpr int OFF_KT_LO = OFF_KT_HI + KD * TP * 2;
constexpr int OFF_QG = OFF_KT_LO + KD * TP * 2;             // f16 [64][KP]
constexpr int OFF_AQK = OFF_QG + CH * KP * 2;               // f16 [64][TBP]
constexpr int OFF_P = OFF_AQK + CH * TBP * 2;               // f32 [5][128] sub-chunk prefixes
constexpr int OFF_TOT = OFF_P + 5 * KD * 4;                 // f32 [4][128] sub-chunk totals
constexpr int NFAC = 15;
constexpr int OFF_FAC = OFF_TOT + 4 * KD * 4;               // f32 [NFAC][128] decay factors
constexpr int OFF_NB = OFF_FAC + NFAC * KD * 4;             // f32 [128] gate offsets
constexpr int OFF_ROW = OFF_NB + KD * 4;                    // f32 [64] beta
constexpr int OFF_GL = OFF_ROW + CH * 4;                    // f32 [128] exp(G_L)
constexpr int LDS_BYTES = OFF_GL + KD * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

// decay-factor table rows (per channel c, log2 units, P_w = prefix before sub-chunk w):
//   FAC_ET + w : exp2(P_{w+1} - P_w)   (whole sub-chunk w)
//   FAC_EP + w : exp2(P_w)             (chunk start -> sub-chunk w start)
//   FAC_EL + w : exp2(P_4 - P_w)       (sub-chunk w start -> chunk end)
//   FAC_F20, FAC_F30, FAC_F31 : exp2(P_w - P_{b+1}) for the off-diagonal A
//   blocks (w, b) with b < w - 1
constexpr int FAC_ET = 0, FAC_EP = 4, FAC_EL = 8, FAC_F20 = 12, FAC_F30 = 13, FAC_F31 = 14;

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  uint16_t* out;
  const float* A_log;
  const float* dt_bias;
  const float* init;
  float* fin;
  const int32_t* cu;     // nullptr: N sequences of length T
  const int32_t* order;  // nullptr: identity processing order
  int64_t T;
  int H;
  int N;
  int n_items;           // N * H
  float scale;
  float lb2;             // lower_bound * log2(e)
#ifdef KDA_PHASE_TIMERS
  unsigned long long* timers;  // [grid][16] per-phase cycle totals seen by wave 0
#endif
};

// Optional per-phase cycle counters (compiled out unless KDA_PHASE_TIMERS is
// defined): thread 0 accumulates cycle-counter deltas between phase marks.
#ifdef KDA_PHASE_TIMERS
#define KDA_TIMER_DECL unsigned long long tacc_[12] = {0}; unsigned long long tlast_ = 0;
#define KDA_TIMER_MARK(i) do { if (tid == 0) { const unsigned long long t_ = __builtin_readcyclecounter(); \
    if ((i) > 0) tacc_[(i) - 1] += t_ - tlast_; tlast_ = t_; } } while (0)
#define KDA_TIMER_STORE() do { if (tid == 0 && p.timers) for (int i_ = 0; i_ < 12; ++i_) \
    p.timers[blockIdx.x * 16 + i_] = tacc_[i_]; } while (0)
#else
#define KDA_TIMER_DECL
#define KDA_TIMER_MARK(i) do { } while (0)
#define KDA_TIMER_STORE() do { } while (0)
#endif

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// inclusive prefix sum over the 16 lanes of a DPP row
__device__ __forceinline__ float row_scan16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, true));
  return x;
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// two 8-byte LDS reads forming one 16x16x32 operand in the "C-layout" k order:
// k slots 0..3 <- elements [o, o+4), slots 4..7 <- [o+16, o+20)
__device__ __forceinline__ f16x8 lds_f16x8_split(const _Float16* row, int o) {
  f16x4 a = *reinterpret_cast<const f16x4*>(row + o);
  f16x4 b = *reinterpret_cast<const f16x4*>(row + o + 16);
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ void lds_f32x8(const float* src, float (&d)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(src);
  const float4 b = *reinterpret_cast<const float4*>(src + 4);
  d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
  d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4 v, float (&d)[8]) {
  const uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    d[2 * u] = __uint_as_float(a[u] << 16);
    d[2 * u + 1] = __uint_as_float(a[u] & 0xffff0000u);
  }
}

__global__ void __launch_bounds__(NTHREADS, 1) kda_fwd_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  __bf16* sKRFh = reinterpret_cast<__bf16*>(smem + OFF_KRF_HI);
  __bf16* sKRFl = reinterpret_cast<__bf16*>(smem + OFF_KRF_LO);
  _Float16* sTb16h = reinterpret_cast<_Float16*>(smem + OFF_TB16_HI);
  _Float16* sTb16l = reinterpret_cast<_Float16*>(smem + OFF_TB16_LO);
  __bf16* sTbbh = reinterpret_cast<__bf16*>(smem + OFF_TBB_HI);
  __bf16* sTbbl = reinterpret_cast<__bf16*>(smem + OFF_TBB_LO);
  float* sA = reinterpret_cast<float*>(smem + OFF_A);
  _Float16* sW = reinterpret_cast<_Float16*>(smem + OFF_W);
  _Float16* sKG = reinterpret_cast<_Float16*>(smem + OFF_KG);
  _Float16* sKth = reinterpret_cast<_Float16*>(smem + OFF_KT_HI);
  _Float16* sKtl = reinterpret_cast<_Float16*>(smem + OFF_KT_LO);
  _Float16* sQG = reinterpret_cast<_Float16*>(smem + OFF_QG);
  _Float16* sAqk = reinterpret_cast<_Float16*>(smem + OFF_AQK);
  float* sP = reinterpret_cast<float*>(smem + OFF_P);
  float* sTot = reinterpret_cast<float*>(smem + OFF_TOT);
  float* sFac = reinterpret_cast<float*>(smem + OFF_FAC);
  float* sNB = reinterpret_cast<float*>(smem + OFF_NB);
  float* sB = reinterpret_cast<float*>(smem + OFF_ROW);
  float* sGL = reinterpret_cast<float*>(smem + OFF_GL);

  // ---- work item: XCD-aware mapping.  Workgroup ids are dispatched
  // round-robin over the 8 XCDs, so the NV slices of one (sequence, head) get
  // ids with the same residue mod 8 and share that XCD's L2 for q/k/g.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int r = bid >> 3;
  const int item = 8 * (r / NV) + xcd;
  const int slice = r % NV;
  if (item >= p.n_items) return;
  const int pos = item / p.H;
  const int h = item - pos * p.H;
  const int seq = p.order ? p.order[pos] : pos;
  int64_t bos, eos;
  if (p.cu) {
    bos = p.cu[seq];
    eos = p.cu[seq + 1];
  } else {
    bos = (int64_t)seq * p.T;
    eos = bos + p.T;
  }
  const int vs = slice * VT;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int tl = lane & 15;
  const int gq = lane >> 4;
  const int H = p.H;

  // gate: sigmoid(x) = 1 / (1 + 2^(raw * na + nb_c)) with na = -exp(A_log) log2(e)
  const float na = -__expf(p.A_log[h]) * LOG2E;
  if (tid < KD) sNB[tid] = na * p.dt_bias[h * KD + tid];

  // ---- state slice S[c][vs + 16w + tl], c = 16mt + 4gq + ii
  f32x4 S[8];
  const int vcol = 16 * w + tl;
  {
    const float* src = p.init ? p.init + ((int64_t)seq * H + h) * KD * VD : nullptr;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int c = 16 * mt + 4 * gq + ii;
        S[mt][ii] = src ? src[c * VD + vs + vcol] : 0.0f;
      }
  }

  // prefetched bf16 inputs of the next chunk: lane (token 16w + tl, channels
  // 32kb + 8gq + e)
  uint4 pq[4], pk[4], pg[4];
  uint16_t pb = 0;
  auto load_chunk = [&](int64_t cstart) {
    const int ti = 16 * w + tl;
    const bool valid = cstart + ti < eos;
    const int64_t trow = (cstart + ti) * H + h;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      pq[kb] = make_uint4(0, 0, 0, 0);
      pk[kb] = pq[kb];
      pg[kb] = pq[kb];
      if (valid) {
        const int64_t off = trow * KD + 32 * kb + 8 * gq;
        pq[kb] = *reinterpret_cast<const uint4*>(p.q + off);
        pk[kb] = *reinterpret_cast<const uint4*>(p.k + off);
        pg[kb] = *reinterpret_cast<const uint4*>(p.g + off);
      }
    }
    pb = valid ? p.beta[trow] : (uint16_t)0;
  };
  if (bos < eos) load_chunk(bos);
  __syncthreads();  // sNB

  KDA_TIMER_DECL
  for (int64_t c0 = bos; c0 < eos; c0 += CH) {
    const int L = (int)((eos - c0) < CH ? (eos - c0) : CH);
    KDA_TIMER_MARK(0);

    // V operand for phase 4, issued now so its latency hides behind prep:
    // lane (col vcol, k-group gq) holds tokens 32ks + 8gq + e of column vs + vcol
    bf16x8 vop[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tj = 32 * ks + 8 * gq + e;
        uint16_t bits = 0;
        if (tj < L) bits = p.v[((c0 + tj) * H + h) * VD + vs + vcol];
        vop[ks][e] = __builtin_bit_cast(__bf16, bits);
      }

    // =========================== 1. prep ===================================
    const int ti = 16 * w + tl;  // chunk-local token of this lane
    const bool valid = ti < L;
    // q and k stay packed (bf16) in pq/pk and are unpacked where used
    float gl[4][8];
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float qf[8], kf[8];
      unpack_bf16x8(pq[kb], qf);
      unpack_bf16x8(pk[kb], kf);
      unpack_bf16x8(pg[kb], gl[kb]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ssq += qf[e] * qf[e];
        ssk += kf[e] * kf[e];
      }
    }
    const float braw = bf16_bits_to_f32(pb);
    ssq += __shfl_xor(ssq, 16);
    ssq += __shfl_xor(ssq, 32);
    ssk += __shfl_xor(ssk, 16);
    ssk += __shfl_xor(ssk, 32);
    const float rq = __builtin_amdgcn_rsqf(ssq + L2_EPS);
    const float rk = __builtin_amdgcn_rsqf(ssk + L2_EPS);
    const float beta = valid ? __builtin_amdgcn_rcpf(1.0f + fexp2(-braw * LOG2E)) : 0.0f;

    // gate in log2 units, then the inclusive scan over the sub-chunk's 16 tokens
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float nb[8];
      lds_f32x8(sNB + 32 * kb + 8 * gq, nb);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float g2 = p.lb2 * __builtin_amdgcn_rcpf(1.0f + fexp2(gl[kb][e] * na + nb[e]));
        g2 = valid ? g2 : 0.0f;
        gl[kb][e] = row_scan16(g2);
      }
    }
    if (tl == 15) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float4* dst = reinterpret_cast<float4*>(sTot + w * KD + 32 * kb + 8 * gq);
        dst[0] = make_float4(gl[kb][0], gl[kb][1], gl[kb][2], gl[kb][3]);
        dst[1] = make_float4(gl[kb][4], gl[kb][5], gl[kb][6], gl[kb][7]);
      }
    }
    if (gq == 0) sB[ti] = beta;
    __syncthreads();
    KDA_TIMER_MARK(1);
    if (tid < KD) {
      float P[5];
      P[0] = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) P[b + 1] = P[b] + sTot[b * KD + tid];
#pragma unroll
      for (int b = 0; b < 5; ++b) sP[b * KD + tid] = P[b];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        sFac[(FAC_ET + b) * KD + tid] = fexp2(P[b + 1] - P[b]);
        sFac[(FAC_EP + b) * KD + tid] = fexp2(P[b]);
        sFac[(FAC_EL + b) * KD + tid] = fexp2(P[4] - P[b]);
      }
      sFac[FAC_F20 * KD + tid] = fexp2(P[2] - P[1]);
      sFac[FAC_F30 * KD + tid] = fexp2(P[3] - P[1]);
      sFac[FAC_F31 * KD + tid] = fexp2(P[3] - P[2]);
      sGL[tid] = fexp2(P[4]);
    }
    __syncthreads();
    KDA_TIMER_MARK(2);

    // operands of this lane's token (32 channels)
    bf16x8 kLFh[4], kLFl[4], kEh[4], kEl[4], qLF[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float ET[8], EP[8], EL[8];
      lds_f32x8(sFac + (FAC_ET + w) * KD + 32 * kb + 8 * gq, ET);
      lds_f32x8(sFac + (FAC_EP + w) * KD + 32 * kb + 8 * gq, EP);
      lds_f32x8(sFac + (FAC_EL + w) * KD + 32 * kb + 8 * gq, EL);
      bf16x8 krh, krl;
      f16x8 qg;
      float qf[8], kf[8];
      unpack_bf16x8(pq[kb], qf);
      unpack_bf16x8(pk[kb], kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 32 * kb + 8 * gq + e;
        const float Gl = gl[kb][e];
        const float LF = fexp2(Gl);   // exp(G_t - P_w) <= 1
        const float E = fexp2(-Gl);   // exp(P_w - G_t) in [1, 2^116]
        const float kn = kf[e] * rk;
        const float qn = qf[e] * rq;
        const float a = kn * LF;
        const __bf16 ah = (__bf16)a;
        kLFh[kb][e] = ah;
        kLFl[kb][e] = (__bf16)(a - (float)ah);
        const float b = kn * E;
        const __bf16 bh = (__bf16)b;
        kEh[kb][e] = bh;
        kEl[kb][e] = (__bf16)(b - (float)bh);
        const float ql = qn * LF;
        qLF[kb][e] = (__bf16)ql;
        const float rf = b * ET[e];  // k^ exp(P_{w+1} - G_t) <= |k^|
        const __bf16 rh = (__bf16)rf;
        krh[e] = rh;
        krl[e] = (__bf16)(rf - (float)rh);
        sKG[c * TP + ti] = (_Float16)(a * EP[e]);       // k^ exp(G_t)
        const float kt = b * EL[e];                      // k^ exp(G_L - G_t)
        const _Float16 kth = (_Float16)kt;
        sKth[c * TP + ti] = kth;
        sKtl[c * TP + ti] = (_Float16)(kt - (float)kth);
        qg[e] = (_Float16)(ql * EP[e]);                 // q^ exp(G_t)
      }
      *reinterpret_cast<f16x8*>(sQG + ti * KP + 32 * kb + 8 * gq) = qg;
      if (w < 3) {
        *reinterpret_cast<bf16x8*>(sKRFh + ti * KP + 32 * kb + 8 * gq) = krh;
        *reinterpret_cast<bf16x8*>(sKRFl + ti * KP + 32 * kb + 8 * gq) = krl;
      }
    }
    __syncthreads();
    KDA_TIMER_MARK(3);

    // ======================= 2. A_kk and A_qk ==============================
    // wave w owns row-block w; lane holds C[16w + 4gq + ii][16b + tl]
    {
      const int i0 = 16 * w + 4 * gq;
      for (int b = 0; b <= w; ++b) {
        f32x4 akk = {0.f, 0.f, 0.f, 0.f};
        f32x4 aqk = {0.f, 0.f, 0.f, 0.f};
        if (b == w) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            akk = mfma_bf16(kLFh[kb], kEh[kb], akk);
            akk = mfma_bf16(kLFh[kb], kEl[kb], akk);
            akk = mfma_bf16(kLFl[kb], kEh[kb], akk);
            aqk = mfma_bf16(qLF[kb], kEh[kb], aqk);
          }
        } else {
          const int jrow = 16 * b + tl;
          const int frow = (b == w - 1) ? -1 : (w == 2 ? FAC_F20 : (b == 0 ? FAC_F30 : FAC_F31));
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 rh = *reinterpret_cast<const bf16x8*>(sKRFh + jrow * KP + 32 * kb + 8 * gq);
            const bf16x8 rl = *reinterpret_cast<const bf16x8*>(sKRFl + jrow * KP + 32 * kb + 8 * gq);
            bf16x8 lh = kLFh[kb], ll = kLFl[kb], lq = qLF[kb];
            if (frow >= 0) {
              // left factor exp(G_i - P_{b+1}) = LF * exp(P_w - P_{b+1})
              float f[8];
              lds_f32x8(sFac + frow * KD + 32 * kb + 8 * gq, f);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float a = ((float)kLFh[kb][e] + (float)kLFl[kb][e]) * f[e];
                const __bf16 ah = (__bf16)a;
                lh[e] = ah;
                ll[e] = (__bf16)(a - (float)ah);
                lq[e] = (__bf16)((float)qLF[kb][e] * f[e]);
              }
            }
            akk = mfma_bf16(lh, rh, akk);
            akk = mfma_bf16(lh, rl, akk);
            akk = mfma_bf16(ll, rh, akk);
            aqk = mfma_bf16(lq, rh, aqk);
          }
        }
        // operands are already L2-normalised: only beta_i scales A_kk rows
        const int j = 16 * b + tl;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int i = i0 + ii;
          const float vkk = (j < i) ? akk[ii] * sB[i] : 0.0f;
          const float vqk = (j <= i) ? aqk[ii] : 0.0f;
          sA[i * AP + j] = vkk;
          sAqk[i * TBP + j] = (_Float16)vqk;
        }
      }
      // zero the upper blocks of this row-block of A_qk (read by 32-wide k-steps)
      for (int b = w + 1; b < 4; ++b) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sAqk[(i0 + ii) * TBP + 16 * b + tl] = (_Float16)0.0f;
      }
      // diagonal block inverse T_ww = (I + A_ww)^-1 by forward substitution,
      // lane cc < 16 owns column cc.  This wave wrote A_ww itself just above
      // (LDS operations of one wave complete in order), so no barrier is needed.
      if (lane < 16) {
        const int cc = lane;
        const float* Ab = sA + (16 * w) * AP + 16 * w;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = (i == cc) ? 1.0f : 0.0f;
#pragma unroll
          for (int m = 0; m < i; ++m) s -= Ab[i * AP + m] * x[m];
          x[i] = (i < cc) ? 0.0f : s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sA[(16 * w + i) * AP + 16 * w + cc] = x[i];
      }
    }
    __syncthreads();
    KDA_TIMER_MARK(4);
    KDA_TIMER_MARK(5);

    // ======================= 3. T = (I + A_kk)^-1 ==========================
    // off-diagonal blocks, row-block by row-block:
    //     T_{b,b'} = -T_bb * sum_{m=b'}^{b-1} A_{b,m} T_{m,b'}
    for (int b = 1; b < 4; ++b) {
      f32x4 res = {0.f, 0.f, 0.f, 0.f};
      const int bp = w;  // wave w computes T_{b, w}
      if (bp < b) {
        f32x4 X = {0.f, 0.f, 0.f, 0.f};
        for (int m = bp; m < b; ++m) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float a = sA[(16 * b + tl) * AP + 16 * m + 4 * s + gq];
            const float t = sA[(16 * m + 4 * s + gq) * AP + 16 * bp + tl];
            X = mfma_f32(a, t, X);
          }
        }
        // res = -T_bb X; X sits in C-layout, so k-step s uses rows {4g + s}
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float a = sA[(16 * b + tl) * AP + 16 * b + 4 * gq + s];
          res = mfma_f32(-a, X[s], res);
        }
      }
      __syncthreads();
      if (bp < b) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sA[(16 * b + 4 * gq + ii) * AP + 16 * bp + tl] = res[ii];
      }
      __syncthreads();
    }
    KDA_TIMER_MARK(6);
    // Tb = T diag(b) (lower triangle, zeros above) in fp16 and bf16 hi/lo;
    // thread handles 8 consecutive columns of one row
    for (int it = tid; it < CH * 8; it += NTHREADS) {
      const int i = it >> 3;
      const int j0 = (it & 7) * 8;
      float t8[8], b8[8];
      lds_f32x8(sA + i * AP + j0, t8);
      lds_f32x8(sB + j0, b8);
      f16x8 h16, l16;
      bf16x8 hb, lb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + e;
        const float t = (j < i) ? t8[e] * b8[e] : ((j == i) ? b8[e] : 0.0f);
        const _Float16 th = (_Float16)t;
        h16[e] = th;
        l16[e] = (_Float16)(t - (float)th);
        const __bf16 tb = (__bf16)t;
        hb[e] = tb;
        lb[e] = (__bf16)(t - (float)tb);
      }
      *reinterpret_cast<f16x8*>(sTb16h + i * TBP + j0) = h16;
      *reinterpret_cast<f16x8*>(sTb16l + i * TBP + j0) = l16;
      *reinterpret_cast<bf16x8*>(sTbbh + i * TBP + j0) = hb;
      *reinterpret_cast<bf16x8*>(sTbbl + i * TBP + j0) = lb;
    }
    __syncthreads();
    KDA_TIMER_MARK(7);

    // ======================= 4. W and U ====================================
    f32x4 U[4];
    {
      f32x4 Wacc[4][2];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        U[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        Wacc[m][0] = U[m];
        Wacc[m][1] = U[m];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks == 1 && m < 2) continue;  // T is lower triangular
          const int arow = (16 * m + tl) * TBP + 32 * ks + 8 * gq;
          const f16x8 th = *reinterpret_cast<const f16x8*>(sTb16h + arow);
          const f16x8 tlo = *reinterpret_cast<const f16x8*>(sTb16l + arow);
          const bf16x8 tbh = *reinterpret_cast<const bf16x8*>(sTbbh + arow);
          const bf16x8 tbl = *reinterpret_cast<const bf16x8*>(sTbbl + arow);
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            const int ch = 32 * w + 16 * n + tl;
            const f16x8 kg = *reinterpret_cast<const f16x8*>(sKG + ch * TP + 32 * ks + 8 * gq);
            Wacc[m][n] = mfma_f16(th, kg, Wacc[m][n]);
            Wacc[m][n] = mfma_f16(tlo, kg, Wacc[m][n]);
          }
          U[m] = mfma_bf16(tbh, vop[ks], U[m]);
          U[m] = mfma_bf16(tbl, vop[ks], U[m]);
        }
      }
      // -W overwrites the fp32 T array; the barrier above ordered the reads
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            sW[(16 * m + 4 * gq + ii) * KP + 32 * w + 16 * n + tl] = (_Float16)(-Wacc[m][n][ii]);
    }
    __syncthreads();
    KDA_TIMER_MARK(8);

    // ======================= 5. state recurrence ===========================
    // prefetch the next chunk's q/k/gate/beta; consumed at the top of the loop
    if (c0 + CH < eos) load_chunk(c0 + CH);
    {
      f16x8 Sb[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          Sb[kb][ii] = (_Float16)S[2 * kb][ii];
          Sb[kb][4 + ii] = (_Float16)S[2 * kb + 1][ii];
        }
      f32x4 D[4], O[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        D[m] = U[m];
        O[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        const _Float16* wrow = sW + (16 * m + tl) * KP;
        const _Float16* qrow = sQG + (16 * m + tl) * KP;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          D[m] = mfma_f16(lds_f16x8_split(wrow, 32 * kb + 4 * gq), Sb[kb], D[m]);
          O[m] = mfma_f16(lds_f16x8_split(qrow, 32 * kb + 4 * gq), Sb[kb], O[m]);
        }
      }
      // D as B operand (k = tokens, C-layout order) in fp16 hi/lo
      f16x8 Dh[2], Dl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float d0 = D[2 * ks][ii];
          const float d1 = D[2 * ks + 1][ii];
          const _Float16 h0 = (_Float16)d0, h1 = (_Float16)d1;
          Dh[ks][ii] = h0;
          Dh[ks][4 + ii] = h1;
          Dl[ks][ii] = (_Float16)(d0 - (float)h0);
          Dl[ks][4 + ii] = (_Float16)(d1 - (float)h1);
        }
      // O += A_qk D (lower triangular)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const _Float16* arow = sAqk + (16 * m + tl) * TBP;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks == 1 && m < 2) continue;
          O[m] = mfma_f16(lds_f16x8_split(arow, 32 * ks + 4 * gq), Dh[ks], O[m]);
        }
      }
      // write the output slice (valid tokens only)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int tt = 16 * m + 4 * gq + ii;
          if (tt < L) {
            const __bf16 o = (__bf16)(O[m][ii] * p.scale);
            p.out[((c0 + tt) * H + h) * VD + vs + vcol] = __builtin_bit_cast(uint16_t, o);
          }
        }
      // S = Diag(G_L) S + Kt^T D
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const float4 gl4 = *reinterpret_cast<const float4*>(sGL + 16 * mt + 4 * gq);
        S[mt][0] *= gl4.x;
        S[mt][1] *= gl4.y;
        S[mt][2] *= gl4.z;
        S[mt][3] *= gl4.w;
        const _Float16* khrow = sKth + (16 * mt + tl) * TP;
        const _Float16* klrow = sKtl + (16 * mt + tl) * TP;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const f16x8 kh = lds_f16x8_split(khrow, 32 * ks + 4 * gq);
          const f16x8 kl = lds_f16x8_split(klrow, 32 * ks + 4 * gq);
          S[mt] = mfma_f16(kh, Dh[ks], S[mt]);
          S[mt] = mfma_f16(kh, Dl[ks], S[mt]);
          S[mt] = mfma_f16(kl, Dh[ks], S[mt]);
        }
      }
    }
    __syncthreads();
    KDA_TIMER_MARK(9);
  }
  KDA_TIMER_STORE();

  if (p.fin) {
    float* dst = p.fin + ((int64_t)seq * H + h) * KD * VD;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) dst[(16 * mt + 4 * gq + ii) * VD + vs + vcol] = S[mt][ii];
  }
}

// Longest-first processing order of the sequences of a packed batch: the rank
// of sequence i is the number of sequences that are longer, or equally long
// with a smaller index.  O(N^2) comparisons; used for N <= kMaxSortN.
__global__ void kda_order_kernel(const int32_t* __restrict__ cu, int N, int32_t* __restrict__ order) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const int li = cu[i + 1] - cu[i];
  int rank = 0;
  for (int j = 0; j < N; ++j) {
    const int lj = cu[j + 1] - cu[j];
    rank += (lj > li) || (lj == li && j < i);
  }
  order[rank] = i;
}

constexpr int kMaxSortN = 16384;

// The launch's own return code (not hipGetLastError, which also reports
// errors left behind by earlier, unrelated runtime calls).  KDA_DEBUG=1 in the
// environment prints the HIP error behind KDA_ERR_LAUNCH.
kda_status_t launch_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return KDA_SUCCESS;
  if (getenv("KDA_DEBUG")) fprintf(stderr, "kda: %s launch failed: %s\n", what, hipGetErrorString(err));
  return KDA_ERR_LAUNCH;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

extern "C" {

size_t kda_workspace_size(int64_t T_total, int64_t H, int64_t N) {
  if (T_total < 0 || H < 1 || N < 1) return 0;
  return 256 + align_up((size_t)N * sizeof(int32_t), 256);
}

int kda_is_supported(int64_t K, int64_t V, float lower_bound) {
  return K == KD && V == VD && lower_bound >= -5.0f && lower_bound <= 0.0f;
}

const char* kda_status_string(kda_status_t s) {
  switch (s) {
    case KDA_SUCCESS: return "KDA_SUCCESS";
    case KDA_ERR_INVALID: return "KDA_ERR_INVALID";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH";
  }
  return "KDA_ERR_UNKNOWN";
}

kda_status_t kda_fwd(const void* q, const void* k, const void* v, const void* raw_gate,
                     const void* raw_beta, float scale, void* out, void* workspace,
                     size_t workspace_bytes, const float* A_log, const float* dt_bias,
                     float lower_bound, const float* initial_state, float* final_state,
                     const int32_t* cu_seqlens, int64_t B, int64_t T, int64_t H, int64_t K,
                     int64_t V, int64_t N, void* stream) {
  if (!q || !k || !v || !raw_gate || !raw_beta || !out || !A_log || !dt_bias) return KDA_ERR_INVALID;
  if (B < 1 || T < 0 || H < 1 || N < 1) return KDA_ERR_INVALID;
  if (cu_seqlens ? (B != 1) : (N != B)) return KDA_ERR_INVALID;
  if (!(scale == scale)) return KDA_ERR_INVALID;
  if (!kda_is_supported(K, V, lower_bound)) return KDA_ERR_UNSUPPORTED;
  if (B * T * H > ((int64_t)1 << 40) || N * H > ((int64_t)1 << 28)) return KDA_ERR_INVALID;
  const size_t need = kda_workspace_size(B * T, H, N);
  if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int32_t* order = nullptr;
  if (cu_seqlens && N > 1 && N <= kMaxSortN) {
    order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + 256);
    int n32 = (int)N;
    void* oargs[] = {(void*)&cu_seqlens, (void*)&n32, (void*)&order};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&kda_order_kernel),
                                         dim3((unsigned)((N + 255) / 256)), dim3(256), oargs, 0, st);
    if (launch_status(e, "order") != KDA_SUCCESS) return KDA_ERR_LAUNCH;
  }
  Params prm;
  prm.q = static_cast<const uint16_t*>(q);
  prm.k = static_cast<const uint16_t*>(k);
  prm.v = static_cast<const uint16_t*>(v);
  prm.g = static_cast<const uint16_t*>(raw_gate);
  prm.beta = static_cast<const uint16_t*>(raw_beta);
  prm.out = static_cast<uint16_t*>(out);
  prm.A_log = A_log;
  prm.dt_bias = dt_bias;
  prm.init = initial_state;
  prm.fin = final_state;
  prm.cu = cu_seqlens;
  prm.order = order;
  prm.T = T;
  prm.H = (int)H;
  prm.N = (int)N;
  prm.n_items = (int)(N * H);
  prm.scale = scale;
  prm.lb2 = lower_bound * LOG2E;
#ifdef KDA_PHASE_TIMERS
  // timer build only: the caller's workspace is extended past the order array
  prm.timers = reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + need);
#endif
  // 8 XCDs x NV slices per group of 8 items
  const int64_t groups = (prm.n_items + 7) / 8;
  const unsigned grid = (unsigned)(groups * 8 * NV);
  void* args[] = {(void*)&prm};
  return launch_status(hipLaunchKernel(reinterpret_cast<const void*>(&kda_fwd_kernel), dim3(grid),
                                       dim3(NTHREADS), args, 0, st),
                       "forward");
}

}  // extern "C"
