// Backward pass of the gfx950 KDA chunked forward.
//
// Reverse-mode differentiation of the chunk algebra.  For one chunk with
// entering state S0, leaving-state gradient dS' and output gradient dO
// (Tb = T diag(beta), KG = K^ exp(G), QG = Q^ exp(G), Kt = K^ exp(G_L - G)):
//   dD   = scale A_qk^T dO + Kt dS'                       (errors' gradient)
//   dS0  = Diag(exp(G_L)) dS' + scale QG^T dO - W^T dD      (reverse recurrence)
// and, per chunk and in parallel once dS' and dD are known,
//   Z = V - KG S0,  dTb = dD Z^T,  dv = Tb^T dD,
//   dQG = scale dO S0^T,  dKG = -dv S0^T,  dKt = D dS'^T,  dA_qk = scale dO D^T,
//   dA_kk = -(T^T (dTb diag(beta)) T^T) (strictly lower),
// then the pairwise products A[i,j] = sum_c x_ic k^_jc exp(G_ic - G_jc) pass
// their gradients to q^, k^ and G, and everything goes back through the
// per-token preparation (L2 norm, sigmoid gate, sigmoid beta).
//
// Kernels, after the forward's intra-chunk kernel and the checkpointing
// inter-chunk kernel (entering states S0 and D of every chunk):
//   kda_bwd_prep_kernel    per (chunk, head): fp32 T, A_kk / beta, A_qk, W, Kt, QG, exp(G_L)
//   kda_bwd_dhu_kernel     per (sequence, head, V half): the reverse recurrence -> dS', dD
//   kda_bwd_grad_kernel    per (chunk, head): dq, dk, dv, d raw_gate, d raw_beta, partials
//   kda_bwd_reduce_kernel  per head: dA_log and d dt_bias from the per-chunk partials
// All arithmetic is fp32 (fp32 MFMA 16x16x4).  Exponents are kept in log2
// units and every exp(G_i - G_j) factor is split at a reference token between
// i and j (16-token sub-chunks), so no factor leaves fp32 range.
//
// fp32 MFMA convention used throughout: in k-step s of a 16-wide contraction
// block starting at `base`, lane (gq = lane / 16, tl = lane % 16) supplies
// A[row tl][base + 4 gq + s] and B[base + 4 gq + s][col tl]; the result lane
// holds C[4 gq + ii][tl].  A C-layout tile therefore serves directly as the B
// operand of a product that contracts over its rows.

#include "kda_common.h"

namespace kda {
namespace {

constexpr int NT = 256;
constexpr int QP = KD + 4;  // pitch (floats) of [64][128] LDS tiles
constexpr int MP = CH + 4;  // pitch of [64][64] LDS tiles
constexpr int VH = VD / 2;  // state columns per recurrence workgroup
constexpr int DP = VH + 4;  // pitch of the recurrence kernel's LDS tiles

// fp32 chunk record of the backward (offsets in floats)
constexpr int BR_T = 0;                   // T = (I + diag(beta) KK)^-1, unit lower [64][64]
constexpr int BR_KK = BR_T + CH * CH;     // KK = K^ K^T . decay, strictly lower     [64][64]
constexpr int BR_AQK = BR_KK + CH * CH;   // A_qk, lower incl. diagonal              [64][64]
constexpr int BR_W = BR_AQK + CH * CH;    // W = Tb KG                               [64][128]
constexpr int BR_KT = BR_W + CH * KD;     // Kt = K^ exp(G_L - G)                    [64][128]
constexpr int BR_QG = BR_KT + CH * KD;    // QG = Q^ exp(G)                          [64][128]
constexpr int BR_GL = BR_QG + CH * KD;    // exp(G_L)                                [128]
constexpr int BR_BETA = BR_GL + KD;       // beta                                    [64]
static_assert(BR_BETA + CH == BWD_REC_FLOATS, "record size");

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

// (sequence, first token, length) of global chunk gch
__device__ __forceinline__ void chunk_of(const ChunkMap& m, int64_t gch, int64_t& c0, int& L) {
  const int seq = chunk_owner(m, gch);
  int64_t bos, eos;
  seq_bounds(m, seq, bos, eos);
  c0 = bos + (gch - first_chunk(m, seq)) * CH;
  L = (int)((eos - c0) < CH ? (eos - c0) : CH);
}

// Per-token preparation of one chunk into LDS: q^, k^ (rows past the end are
// zero), G = cumulative log2-decay (constant past the end), beta, the row
// norms of q and k.  Thread t handles token t / 4 and channels 32 (t % 4)...
__device__ void prep_chunk(const BwdArgs& a, int64_t c0, int L, int h, float* sQn, float* sKn, float* sG,
                           float* sBeta, float* sRq, float* sRk, float* sTmp) {
  const int t = threadIdx.x;
  const int i = t >> 2;
  const int cq = t & 3;
  const bool ok = i < L;
  const int64_t row = c0 + (ok ? i : L - 1);  // L >= 1: the clamped row is in range
  const size_t base = ((size_t)row * a.H + h) * KD + 32 * cq;
  float qv[32], kv[32], gv[32];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float tq[8], tk[8], tg[8];
    unpack_bf16x8(reinterpret_cast<const uint4*>(a.q + base)[u], tq);
    unpack_bf16x8(reinterpret_cast<const uint4*>(a.k + base)[u], tk);
    unpack_bf16x8(reinterpret_cast<const uint4*>(a.g + base)[u], tg);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[8 * u + e] = tq[e];
      kv[8 * u + e] = tk[e];
      gv[8 * u + e] = tg[e];
    }
  }
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    sq += qv[c] * qv[c];
    sk += kv[c] * kv[c];
  }
  sq += __shfl_xor(sq, 1);
  sq += __shfl_xor(sq, 2);
  sk += __shfl_xor(sk, 1);
  sk += __shfl_xor(sk, 2);
  const float rq = sqrtf(sq + L2_EPS), rk = sqrtf(sk + L2_EPS);
  const float iq = ok ? 1.0f / rq : 0.f, ik = ok ? 1.0f / rk : 0.f;
  const float al = expf(a.A_log[h]);
  const float* dtb = a.dt_bias + (size_t)h * KD + 32 * cq;
#pragma unroll
  for (int c = 0; c < 32; c += 4) {
    float4 qo, ko, go;
    float gg[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) gg[e] = ok ? a.lb * sigmoidf(al * (gv[c + e] + dtb[c + e])) * LOG2E : 0.f;
    qo = make_float4(qv[c] * iq, qv[c + 1] * iq, qv[c + 2] * iq, qv[c + 3] * iq);
    ko = make_float4(kv[c] * ik, kv[c + 1] * ik, kv[c + 2] * ik, kv[c + 3] * ik);
    go = make_float4(gg[0], gg[1], gg[2], gg[3]);
    *reinterpret_cast<float4*>(sQn + i * QP + 32 * cq + c) = qo;
    *reinterpret_cast<float4*>(sKn + i * QP + 32 * cq + c) = ko;
    *reinterpret_cast<float4*>(sG + i * QP + 32 * cq + c) = go;
  }
  if (cq == 0) {
    sBeta[i] = ok ? sigmoidf(bf2f(a.beta[(size_t)row * a.H + h])) : 0.f;
    sRq[i] = rq;
    sRk[i] = rk;
  }
  __syncthreads();
  // inclusive cumulative sum over the 64 tokens: thread -> channel t % 128, half t / 128
  {
    const int c = t & 127;
    const int hf = t >> 7;
    float run = 0.f;
    for (int r = 32 * hf; r < 32 * hf + 32; ++r) {
      run += sG[r * QP + c];
      sG[r * QP + c] = run;
    }
    if (hf == 0) sTmp[c] = run;
    __syncthreads();
    if (hf == 1) {
      const float off = sTmp[c];
      for (int r = 32; r < 64; ++r) sG[r * QP + c] += off;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// kda_bwd_prep_kernel: per (chunk, head), the chunk factors in fp32.
// ---------------------------------------------------------------------------
constexpr int PREP_FLOATS = 3 * CH * QP + 3 * CH * MP + 3 * CH + NT;

__global__ void __launch_bounds__(NT, 1) kda_bwd_prep_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float smem[PREP_FLOATS];
  float* sQn = smem;
  float* sKn = sQn + CH * QP;
  float* sG = sKn + CH * QP;
  float* sKK = sG + CH * QP;
  float* sAQ = sKK + CH * MP;
  float* sT = sAQ + CH * MP;
  float* sBeta = sT + CH * MP;
  float* sRq = sBeta + CH;
  float* sRk = sRq + CH;
  float* sTmp = sRk + CH;

  const int H = a.H;
  const int64_t gch = blockIdx.x / H;
  const int h = blockIdx.x - (int)gch * H;
  if (gch >= total_chunks(a.map)) return;
  int64_t c0;
  int L;
  chunk_of(a.map, gch, c0, L);
  float* br = a.br + (size_t)blockIdx.x * BWD_REC_FLOATS;

  prep_chunk(a, c0, L, h, sQn, sKn, sG, sBeta, sRq, sRk, sTmp);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int tl = lane & 15;
  const int gq = lane >> 4;

  // ---- KK and A_qk, row block w, column blocks b <= w.  Reference token r
  // between i and j: the last token of block b (b < w), else the first of w.
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b > w) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * w + 4 * gq + ii, j = 16 * b + tl;
        sKK[i * MP + j] = 0.f;
        sAQ[i * MP + j] = 0.f;
        br[BR_KK + i * CH + j] = 0.f;
        br[BR_AQK + i * CH + j] = 0.f;
      }
      continue;
    }
    const int r = (b < w) ? 16 * b + 15 : 16 * w;
    f32x4 ak = zero4(), aq = zero4();
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int c = 16 * t + 4 * gq;
      const float4 kx = ld4(sKn + (16 * w + tl) * QP + c), qx = ld4(sQn + (16 * w + tl) * QP + c);
      const float4 gx = ld4(sG + (16 * w + tl) * QP + c);
      const float4 ky = ld4(sKn + (16 * b + tl) * QP + c), gy = ld4(sG + (16 * b + tl) * QP + c);
      const float4 gr = ld4(sG + r * QP + c);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float fx = fexp2(el(gx, s) - el(gr, s));
        const float yb = el(ky, s) * fexp2(el(gr, s) - el(gy, s));
        ak = mfma_f32(el(kx, s) * fx, yb, ak);
        aq = mfma_f32(el(qx, s) * fx, yb, aq);
      }
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 16 * w + 4 * gq + ii, j = 16 * b + tl;
      const float kk = (b < w || j < i) ? ak[ii] : 0.f;
      const float qk = (b < w || j <= i) ? aq[ii] : 0.f;
      sKK[i * MP + j] = kk;
      sAQ[i * MP + j] = qk;
      br[BR_KK + i * CH + j] = kk;
      br[BR_AQK + i * CH + j] = qk;
    }
  }
  __syncthreads();

  // ---- T = (I + diag(beta) KK)^-1.  Diagonal 16x16 blocks by forward
  // substitution (lane tl owns column tl), zero upper blocks.
  {
    const int j = tl;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = (i == j) ? 1.f : 0.f;
      const float bi = sBeta[16 * w + i];
#pragma unroll
      for (int m = 0; m < i; ++m) acc -= bi * sKK[(16 * w + i) * MP + 16 * w + m] * x[m];
      x[i] = acc;
    }
    if (gq == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sT[(16 * w + i) * MP + 16 * w + j] = x[i];
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (b > w) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sT[(16 * w + 4 * gq + ii) * MP + 16 * b + tl] = 0.f;
      }
  }
  __syncthreads();
  // off-diagonal blocks by diagonals: T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (w >= d) {
      const int aa = w, bb = w - d;
      f32x4 X = zero4();
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c < bb || c >= aa) continue;
        const float ba = sBeta[16 * aa + tl];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int kap = 16 * c + 4 * gq + s;
          X = mfma_f32(ba * sKK[(16 * aa + tl) * MP + kap], sT[kap * MP + 16 * bb + tl], X);
        }
      }
      f32x4 res = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) res = mfma_f32(-sT[(16 * aa + tl) * MP + 16 * aa + 4 * gq + s], X[s], res);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sT[(16 * aa + 4 * gq + ii) * MP + 16 * bb + tl] = res[ii];
    }
    __syncthreads();
  }
  for (int e = tid; e < CH * CH; e += NT) br[BR_T + e] = sT[(e >> 6) * MP + (e & 63)];

  // ---- W = Tb KG, row block w, contraction over tokens j < 16w + 16
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    f32x4 acc = zero4();
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      if (jb > w) continue;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kap = 16 * jb + 4 * gq + s;
        const int c = 16 * n + tl;
        const float av = sT[(16 * w + tl) * MP + kap] * sBeta[kap];
        const float bv = sKn[kap * QP + c] * fexp2(sG[kap * QP + c]);
        acc = mfma_f32(av, bv, acc);
      }
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) br[BR_W + (16 * w + 4 * gq + ii) * KD + 16 * n + tl] = acc[ii];
  }

  // ---- Kt, QG, exp(G_L), beta
  {
    const int i = tid >> 2;
    const int cq = tid & 3;
#pragma unroll
    for (int c = 32 * cq; c < 32 * cq + 32; c += 4) {
      const float4 kn = ld4(sKn + i * QP + c), qn = ld4(sQn + i * QP + c), gg = ld4(sG + i * QP + c);
      const float4 gl = ld4(sG + (CH - 1) * QP + c);
      float4 kt, qg;
      kt.x = kn.x * fexp2(gl.x - gg.x); kt.y = kn.y * fexp2(gl.y - gg.y);
      kt.z = kn.z * fexp2(gl.z - gg.z); kt.w = kn.w * fexp2(gl.w - gg.w);
      qg.x = qn.x * fexp2(gg.x); qg.y = qn.y * fexp2(gg.y);
      qg.z = qn.z * fexp2(gg.z); qg.w = qn.w * fexp2(gg.w);
      *reinterpret_cast<float4*>(br + BR_KT + i * KD + c) = kt;
      *reinterpret_cast<float4*>(br + BR_QG + i * KD + c) = qg;
    }
    if (tid < KD) br[BR_GL + tid] = fexp2(sG[(CH - 1) * QP + tid]);
    if (tid < CH) br[BR_BETA + tid] = sBeta[tid];
  }
}

// ---------------------------------------------------------------------------
// kda_bwd_dhu_kernel: per (sequence, head, V half), chunks in reverse order.
// The state gradient dS (rows = channels 32w + 16mt + 4gq + ii, columns
// vs + 16nn + tl) stays in registers.
// ---------------------------------------------------------------------------
constexpr int DHU_FLOATS = KD * DP + 2 * CH * DP;

__global__ void __launch_bounds__(NT, 1) kda_bwd_dhu_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float smem[DHU_FLOATS];
  float* sdS = smem;             // [128 k][DP]  dS' columns of this half
  float* sdO = sdS + KD * DP;    // [64 i][DP]   scale * dO
  float* sdD = sdO + CH * DP;    // [64 i][DP]   dD

  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int rr = bid >> 3;
  const int item = 8 * (rr >> 1) + xcd;
  const int slice = rr & 1;
  const int H = a.H;
  if (item >= a.map.N * H) return;
  const int pos = item / H;
  const int h = item - pos * H;
  const int seq = a.order ? a.order[pos] : pos;
  int64_t bos, eos;
  seq_bounds(a.map, seq, bos, eos);
  const int64_t gfirst = first_chunk(a.map, seq);
  const int vs = slice * VH;
  const int nch = (int)((eos - bos + CH - 1) / CH);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int tl = lane & 15;
  const int gq = lane >> 4;

  f32x4 dS[2][4];
  {
    const float* src = a.dfin ? a.dfin + ((size_t)seq * H + h) * KD * VD : nullptr;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          dS[mt][nn][ii] = src ? src[(32 * w + 16 * mt + 4 * gq + ii) * VD + vs + 16 * nn + tl] : 0.f;
  }

  for (int ci = nch - 1; ci >= 0; --ci) {
    const int64_t gch = gfirst + ci;
    const int64_t c0 = bos + (int64_t)ci * CH;
    const int L = (int)((eos - c0) < CH ? (eos - c0) : CH);
    const size_t it = (size_t)gch * H + h;
    const float* br = a.br + it * BWD_REC_FLOATS;

    // dS' of this chunk: to the checkpoint buffer and to LDS
    float* dsg = a.dstates + it * KD * VD;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int kr = 32 * w + 16 * mt + 4 * gq + ii;
          const int vc = 16 * nn + tl;
          dsg[kr * VD + vs + vc] = dS[mt][nn][ii];
          sdS[kr * DP + vc] = dS[mt][nn][ii];
        }
    // scale * dO tile (zero past the chunk end)
    {
      const int r = tid >> 2;
      const int cg = 16 * (tid & 3);
      float d[16];
      if (r < L) {
        const uint4* src = reinterpret_cast<const uint4*>(a.dout + ((size_t)(c0 + r) * H + h) * VD + vs + cg);
        float t0[8], t1[8];
        unpack_bf16x8(src[0], t0);
        unpack_bf16x8(src[1], t1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          d[e] = t0[e] * a.scale;
          d[8 + e] = t1[e] * a.scale;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) d[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 16; e += 4)
        *reinterpret_cast<float4*>(sdO + r * DP + cg + e) = make_float4(d[e], d[e + 1], d[e + 2], d[e + 3]);
    }
    __syncthreads();

    // dD rows 16w.. = Kt dS' + A_qk^T (scale dO)
    f32x4 dD[4];
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) dD[nn] = zero4();
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float4 kt = ld4(br + BR_KT + (16 * w + tl) * KD + 16 * t + 4 * gq);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kap = 16 * t + 4 * gq + s;
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) dD[nn] = mfma_f32(el(kt, s), sdS[kap * DP + 16 * nn + tl], dD[nn]);
      }
    }
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      if (jb < w) continue;  // A_qk[j][i] = 0 for j < i
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kap = 16 * jb + 4 * gq + s;
        const float av = br[BR_AQK + kap * CH + 16 * w + tl];
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) dD[nn] = mfma_f32(av, sdO[kap * DP + 16 * nn + tl], dD[nn]);
      }
    }
    float* ddg = a.ddtile + it * CH * VD;
#pragma unroll
    for (int nn = 0; nn < 4; ++nn)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * w + 4 * gq + ii;
        ddg[i * VD + vs + 16 * nn + tl] = dD[nn][ii];
        sdD[i * DP + 16 * nn + tl] = dD[nn][ii];
      }
    __syncthreads();

    // dS = Diag(exp(G_L)) dS' + QG^T (scale dO) - W^T dD
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const float4 gl = ld4(br + BR_GL + 32 * w + 16 * mt + 4 * gq);
#pragma unroll
      for (int nn = 0; nn < 4; ++nn) {
        dS[mt][nn][0] *= gl.x;
        dS[mt][nn][1] *= gl.y;
        dS[mt][nn][2] *= gl.z;
        dS[mt][nn][3] *= gl.w;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int kap = 16 * t + 4 * gq + s;
          const float aqg = br[BR_QG + kap * KD + 32 * w + 16 * mt + tl];
          const float aw = -br[BR_W + kap * KD + 32 * w + 16 * mt + tl];
#pragma unroll
          for (int nn = 0; nn < 4; ++nn) {
            dS[mt][nn] = mfma_f32(aqg, sdO[kap * DP + 16 * nn + tl], dS[mt][nn]);
            dS[mt][nn] = mfma_f32(aw, sdD[kap * DP + 16 * nn + tl], dS[mt][nn]);
          }
        }
    }
    __syncthreads();
  }

  if (a.dinit) {
    float* dst = a.dinit + ((size_t)seq * H + h) * KD * VD;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          dst[(32 * w + 16 * mt + 4 * gq + ii) * VD + vs + 16 * nn + tl] = dS[mt][nn][ii];
  }
}

// ---------------------------------------------------------------------------
// kda_bwd_grad_kernel: per (chunk, head).  Wave w owns token block
// 16w..16w+15 in the roles listed at each step.
// ---------------------------------------------------------------------------
constexpr int GRAD_FLOATS = 3 * CH * QP + 3 * CH * MP + 4 * CH + NT + 4 * KD + KD + 4 * KD;

__global__ void __launch_bounds__(NT, 1) kda_bwd_grad_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float smem[GRAD_FLOATS];
  float* sQn = smem;
  float* sKn = sQn + CH * QP;
  float* sG = sKn + CH * QP;
  float* sT = sG + CH * QP;
  float* sM1 = sT + CH * MP;   // dA_qk
  float* sM2 = sM1 + CH * MP;  // dT, then X = dT T^T, then dKK
  float* sBeta = sM2 + CH * MP;
  float* sRq = sBeta + CH;
  float* sRk = sRq + CH;
  float* sdB = sRk + CH;       // gradient of beta
  float* sTmp = sdB + CH;      // [256]
  float* sGLw = sTmp + NT;     // [4][128] per-wave sums of dKt . Kt
  float* sGL2 = sGLw + 4 * KD; // [128] exp(G_L) sum_v dS' . S0
  float* sCS = sGL2 + KD;      // [4][128] per-wave column totals

  const int H = a.H;
  const int64_t gch = blockIdx.x / H;
  const int h = blockIdx.x - (int)gch * H;
  if (gch >= total_chunks(a.map)) return;
  int64_t c0;
  int L;
  chunk_of(a.map, gch, c0, L);
  const size_t it = blockIdx.x;
  const float* br = a.br + it * BWD_REC_FLOATS;
  const float* S0 = a.states + it * KD * VD;
  const float* dSn = a.dstates + it * KD * VD;
  const float* Dt = a.dtile + it * CH * VD;
  const float* dDt = a.ddtile + it * CH * VD;

  prep_chunk(a, c0, L, h, sQn, sKn, sG, sBeta, sRq, sRk, sTmp);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int tl = lane & 15;
  const int gq = lane >> 4;
  const int jw = 16 * w + tl;  // this lane's token as an A row / B column

  for (int e = tid; e < CH * CH; e += NT) sT[(e >> 6) * MP + (e & 63)] = br[BR_T + e];
  // exp(G_L) sum_v dS'[c][v] S0[c][v]: thread -> channel tid / 2, half of v
  {
    const int c = tid >> 1;
    const int v0 = 64 * (tid & 1);
    float acc = 0.f;
#pragma unroll 4
    for (int v = v0; v < v0 + 64; v += 4) {
      const float4 x = ld4(dSn + c * VD + v), y = ld4(S0 + c * VD + v);
      acc += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
    }
    acc += __shfl_xor(acc, 1);
    if ((tid & 1) == 0) sGL2[c] = acc * fexp2(sG[(CH - 1) * QP + c]);
  }
  __syncthreads();

  // ---- Z^T[:, block w] = V^T - S0^T KG^T   (rows v = 16m + 4gq + ii, column jw)
  float kgb[8][4];  // KG[jw][16t + 4gq + s]
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float4 kn = ld4(sKn + jw * QP + 16 * t + 4 * gq), gg = ld4(sG + jw * QP + 16 * t + 4 * gq);
#pragma unroll
    for (int s = 0; s < 4; ++s) kgb[t][s] = el(kn, s) * fexp2(el(gg, s));
  }
  const bool jok = jw < L;
  const size_t jrow = ((size_t)(c0 + (jok ? jw : 0)) * H + h);
  f32x4 Zt[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    f32x4 acc = zero4();
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma_f32(S0[(16 * t + 4 * gq + s) * VD + 16 * m + tl], kgb[t][s], acc);
    // V[jw][16m + 4gq + ii]
    float vv[4] = {0.f, 0.f, 0.f, 0.f};
    if (jok) {
      const uint2 raw = *reinterpret_cast<const uint2*>(a.v + jrow * VD + 16 * m + 4 * gq);
      vv[0] = __uint_as_float(raw.x << 16);
      vv[1] = __uint_as_float(raw.x & 0xffff0000u);
      vv[2] = __uint_as_float(raw.y << 16);
      vv[3] = __uint_as_float(raw.y & 0xffff0000u);
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) Zt[m][ii] = vv[ii] - acc[ii];
  }

  // ---- dv^T[:, block w] = dD^T Tb[:, block w]   (contraction over i >= 16w)
  float tbb[4][4];
  const float bj = sBeta[jw];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int s = 0; s < 4; ++s) tbb[ib][s] = sT[(16 * ib + 4 * gq + s) * MP + jw] * bj;
  f32x4 dvT[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    f32x4 acc = zero4();
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      if (ib < w) continue;
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma_f32(dDt[(16 * ib + 4 * gq + s) * VD + 16 * m + tl], tbb[ib][s], acc);
    }
    dvT[m] = acc;
    if (jok) {
      const uint32_t lo = (uint32_t)f2bf(acc[0]) | ((uint32_t)f2bf(acc[1]) << 16);
      const uint32_t hi = (uint32_t)f2bf(acc[2]) | ((uint32_t)f2bf(acc[3]) << 16);
      *reinterpret_cast<uint2*>(a.dv + jrow * VD + 16 * m + 4 * gq) = make_uint2(lo, hi);
    }
  }

  // ---- scale * dO rows jw as A operands (contraction over v = 16m + 4gq + s)
  float doa[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (jok) {
      const uint2 raw = *reinterpret_cast<const uint2*>(a.dout + jrow * VD + 16 * m + 4 * gq);
      doa[m][0] = __uint_as_float(raw.x << 16) * a.scale;
      doa[m][1] = __uint_as_float(raw.x & 0xffff0000u) * a.scale;
      doa[m][2] = __uint_as_float(raw.y << 16) * a.scale;
      doa[m][3] = __uint_as_float(raw.y & 0xffff0000u) * a.scale;
    } else {
      doa[m][0] = doa[m][1] = doa[m][2] = doa[m][3] = 0.f;
    }
  }

  // ---- dQG, dKG, dKt (rows 16w + 4gq + ii, channels 16n + tl) and their
  // elementwise contributions to dq^, dk^, dG
  f32x4 dqh[8], dkh[8], dGa[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    f32x4 aQ = zero4(), aK = zero4(), aT = zero4();
    const int kc = 16 * n + tl;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float4 s0 = ld4(S0 + kc * VD + 16 * m + 4 * gq);
      const float4 dsn = ld4(dSn + kc * VD + 16 * m + 4 * gq);
      const float4 dd = ld4(Dt + jw * VD + 16 * m + 4 * gq);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        aQ = mfma_f32(doa[m][s], el(s0, s), aQ);
        aK = mfma_f32(-dvT[m][s], el(s0, s), aK);
        aT = mfma_f32(el(dd, s), el(dsn, s), aT);
      }
    }
    float glsum = 0.f;
    const float gl2 = sG[(CH - 1) * QP + kc];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int j = 16 * w + 4 * gq + ii;
      const float qn = sQn[j * QP + kc], kn = sKn[j * QP + kc], g2 = sG[j * QP + kc];
      const float gam = fexp2(g2), el2 = fexp2(gl2 - g2);
      const float kt = kn * el2;
      dqh[n][ii] = aQ[ii] * gam;
      dkh[n][ii] = aK[ii] * gam + aT[ii] * el2;
      dGa[n][ii] = aQ[ii] * qn * gam + aK[ii] * kn * gam - aT[ii] * kt;
      glsum += aT[ii] * kt;
    }
    glsum += __shfl_xor(glsum, 16);
    glsum += __shfl_xor(glsum, 32);
    if (gq == 0) sGLw[w * KD + kc] = glsum;
  }

  // ---- dTb[i][block w] for i >= 16w = dD Z^T; dT = dTb diag(beta) -> sM2;
  // column sums of dTb . T -> dbeta
  {
    float colsum = 0.f;
#pragma unroll
    for (int ab = 0; ab < 4; ++ab) {
      if (ab < w) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sM2[(16 * ab + 4 * gq + ii) * MP + jw] = 0.f;
        continue;
      }
      f32x4 acc = zero4();
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float4 dd = ld4(dDt + (16 * ab + tl) * VD + 16 * m + 4 * gq);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma_f32(el(dd, s), Zt[m][s], acc);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * ab + 4 * gq + ii;
        colsum += acc[ii] * sT[i * MP + jw];
        sM2[i * MP + jw] = acc[ii] * bj;
      }
    }
    colsum += __shfl_xor(colsum, 16);
    colsum += __shfl_xor(colsum, 32);
    if (gq == 0) sdB[jw] = colsum;
  }

  // ---- dA_qk[block w][j <= i] = scale dO D^T -> sM1
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f32x4 acc = zero4();
    if (b <= w) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float4 dd = ld4(Dt + (16 * b + tl) * VD + 16 * m + 4 * gq);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma_f32(doa[m][s], el(dd, s), acc);
      }
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 16 * w + 4 * gq + ii, j = 16 * b + tl;
      sM1[i * MP + j] = (j <= i) ? acc[ii] : 0.f;
    }
  }
  __syncthreads();

  // ---- X = dT T^T, row block w, column blocks q <= w (in place in sM2)
  {
    f32x4 X[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      X[q] = zero4();
      if (q > w) continue;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b > q) continue;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int kap = 16 * b + 4 * gq + s;
          X[q] = mfma_f32(sM2[jw * MP + kap], sT[(16 * q + tl) * MP + kap], X[q]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q <= w) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sM2[(16 * w + 4 * gq + ii) * MP + 16 * q + tl] = X[q][ii];
      }
  }
  __syncthreads();
  // ---- dA_kk[block w][m < a] = -T^T X; row sums of dA_kk . KK -> dbeta; dKK = dA_kk beta_a
  f32x4 dkk[4];
  {
    float rows[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 acc = zero4();
      if (q <= w) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if (p < w) continue;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int kap = 16 * p + 4 * gq + s;
            acc = mfma_f32(-sT[kap * MP + jw], sM2[kap * MP + 16 * q + tl], acc);
          }
        }
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int ar = 16 * w + 4 * gq + ii, mc = 16 * q + tl;
        const float v = (mc < ar) ? acc[ii] : 0.f;
        rows[ii] += v * br[BR_KK + ar * CH + mc];
        acc[ii] = v * sBeta[ar];
      }
      dkk[q] = acc;
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float r = rows[ii];
      r += __shfl_xor(r, 1);
      r += __shfl_xor(r, 2);
      r += __shfl_xor(r, 4);
      r += __shfl_xor(r, 8);
      if (tl == 0) sdB[16 * w + 4 * gq + ii] += r;
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) sM2[(16 * w + 4 * gq + ii) * MP + 16 * q + tl] = dkk[q][ii];
  __syncthreads();

  // ---- pairwise products, row role: i in block w, j in blocks b <= w
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b > w) continue;
    const int r = (b < w) ? 16 * b + 15 : 16 * w;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int c = 16 * n + tl;
      const float gr = sG[r * QP + c];
      f32x4 a1 = zero4(), a2 = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kap = 16 * b + 4 * gq + s;
        const float y = sKn[kap * QP + c] * fexp2(gr - sG[kap * QP + c]);
        a1 = mfma_f32(sM1[jw * MP + kap], y, a1);
        a2 = mfma_f32(sM2[jw * MP + kap], y, a2);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * w + 4 * gq + ii;
        const float f = fexp2(sG[i * QP + c] - gr);
        const float v1 = a1[ii] * f, v2 = a2[ii] * f;
        dqh[n][ii] += v1;
        dkh[n][ii] += v2;
        dGa[n][ii] += sQn[i * QP + c] * v1 + sKn[i * QP + c] * v2;
      }
    }
  }
  // ---- pairwise products, column role: j in block w, i in blocks a >= w
#pragma unroll
  for (int ab = 0; ab < 4; ++ab) {
    if (ab < w) continue;
    const int r = (ab > w) ? 16 * w + 15 : 16 * w;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int c = 16 * n + tl;
      const float gr = sG[r * QP + c];
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kap = 16 * ab + 4 * gq + s;
        const float f = fexp2(sG[kap * QP + c] - gr);
        acc = mfma_f32(sM1[kap * MP + jw], sQn[kap * QP + c] * f, acc);
        acc = mfma_f32(sM2[kap * MP + jw], sKn[kap * QP + c] * f, acc);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = 16 * w + 4 * gq + ii;
        const float v = acc[ii] * fexp2(gr - sG[j * QP + c]);
        dkh[n][ii] += v;
        dGa[n][ii] -= sKn[j * QP + c] * v;
      }
    }
  }

  // ---- dG_L on the last token, then the reverse cumulative sum -> dg (log-decay gradient)
  const int lastw = (L - 1) >> 4;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int c = 16 * n + tl;
    if (w == lastw) {
      const float dgl = sGL2[c] + sGLw[c] + sGLw[KD + c] + sGLw[2 * KD + c] + sGLw[3 * KD + c];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        if (16 * w + 4 * gq + ii == L - 1) dGa[n][ii] += dgl;
    }
    // suffix sums within the lane's 4 rows, then over the later lane groups
    f32x4 x = dGa[n];
    x[2] += x[3];
    x[1] += x[2];
    x[0] += x[1];
    const float tot = x[0];
    const float t1 = __shfl(tot, tl + 16), t2 = __shfl(tot, tl + 32), t3 = __shfl(tot, tl + 48);
    const float off = (gq < 1 ? t1 : 0.f) + (gq < 2 ? t2 : 0.f) + (gq < 3 ? t3 : 0.f);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) x[ii] += off;
    dGa[n] = x;
    if (gq == 0) sCS[w * KD + c] = x[0];  // the whole block's column total
  }
  __syncthreads();

  // ---- outputs: d raw_gate, dq, dk, d raw_beta; partial sums of d dt_bias, dA_log
  const float al = expf(a.A_log[h]);
  float pA = 0.f;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int c = 16 * n + tl;
    float later = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u > w) later += sCS[u * KD + c];
    const float dtb = a.dt_bias[(size_t)h * KD + c];
    float pdt = 0.f;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int j = 16 * w + 4 * gq + ii;
      const float dgv = dGa[n][ii] + later;  // natural-log gradient of g_j
      if (j < L) {
        const size_t o = ((size_t)(c0 + j) * H + h) * KD + c;
        const float x = al * (bf2f(a.g[o]) + dtb);
        const float sg = sigmoidf(x);
        const float dx = dgv * a.lb * sg * (1.f - sg);
        a.dg[o] = f2bf(dx * al);
        pdt += dx * al;
        pA += dx * x;
      }
    }
    pdt += __shfl_xor(pdt, 16);
    pdt += __shfl_xor(pdt, 32);
    if (gq == 0) sGLw[w * KD + c] = pdt;  // sGLw is free again: dG_L was added before the barrier
  }
  // dq = (dq^ - q^ (q^ . dq^)) / |q|, same for k
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int j = 16 * w + 4 * gq + ii;
    float dq_dot = 0.f, dk_dot = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      dq_dot += sQn[j * QP + 16 * n + tl] * dqh[n][ii];
      dk_dot += sKn[j * QP + 16 * n + tl] * dkh[n][ii];
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      dq_dot += __shfl_xor(dq_dot, d);
      dk_dot += __shfl_xor(dk_dot, d);
    }
    if (j < L) {
      const float irq = 1.f / sRq[j], irk = 1.f / sRk[j];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int c = 16 * n + tl;
        const size_t o = ((size_t)(c0 + j) * H + h) * KD + c;
        a.dq[o] = f2bf((dqh[n][ii] - sQn[j * QP + c] * dq_dot) * irq);
        a.dk[o] = f2bf((dkh[n][ii] - sKn[j * QP + c] * dk_dot) * irk);
      }
    }
  }
  // block reduction of pA
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) pA += __shfl_xor(pA, d);
  if (lane == 0) sTmp[w] = pA;
  if (lane < 16 && jw < L) {
    const float b = sBeta[jw];
    a.dbeta[(size_t)(c0 + jw) * H + h] = f2bf(sdB[jw] * b * (1.f - b));
  }
  __syncthreads();
  float* part = a.part + it * (KD + 1);
  if (tid < KD) part[tid] = sGLw[tid] + sGLw[KD + tid] + sGLw[2 * KD + tid] + sGLw[3 * KD + tid];
  if (tid == KD) part[KD] = sTmp[0] + sTmp[1] + sTmp[2] + sTmp[3];
}

// ---------------------------------------------------------------------------
// kda_bwd_reduce_kernel: per head, sum the per-chunk partials.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(NT) kda_bwd_reduce_kernel(BwdArgs a) {
  const int h = blockIdx.x;
  const int H = a.H;
  const int64_t nch = total_chunks(a.map);
  const int t = threadIdx.x;
  if (t > KD) return;
  float acc = 0.f;
  for (int64_t g = 0; g < nch; ++g) acc += a.part[((size_t)g * H + h) * (KD + 1) + t];
  if (t < KD)
    a.ddt[(size_t)h * KD + t] = acc;
  else
    a.dA_log[h] = acc;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& args, int64_t max_chunks, hipStream_t st) {
  BwdArgs a = args;
  void* kargs[] = {(void*)&a};
  const int64_t items = max_chunks * a.H;
  hipError_t e;
  if (items > 0) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&kda_bwd_prep_kernel), dim3((unsigned)items), dim3(NT),
                        kargs, 0, st);
    if (e != hipSuccess) return e;
  }
  const int64_t seqs = (int64_t)a.map.N * a.H;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&kda_bwd_dhu_kernel), dim3((unsigned)((seqs + 7) / 8 * 8 * 2)),
                      dim3(NT), kargs, 0, st);
  if (e != hipSuccess) return e;
  if (items > 0) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&kda_bwd_grad_kernel), dim3((unsigned)items), dim3(NT),
                        kargs, 0, st);
    if (e != hipSuccess) return e;
  }
  return hipLaunchKernel(reinterpret_cast<const void*>(&kda_bwd_reduce_kernel), dim3((unsigned)a.H), dim3(NT),
                         kargs, 0, st);
}

}  // namespace kda
