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
// Arithmetic is fp32 throughout: fp32 MFMA 16x16x4, or bf16 MFMA 16x16x32 with
// every fp32 operand split into a bf16 hi/lo pair (3 passes; 2 where the other
// side is an exact bf16 input), which keeps about 16 significant bits per
// operand.  Exponents are kept in log2 units and every exp(G_i - G_j) factor
// is split at a reference token between i and j (16-token sub-chunks), so no
// factor leaves fp32 range.
//
// fp32 MFMA convention used throughout: in k-step s of a 16-wide contraction
// block starting at `base`, lane (gq = lane / 16, tl = lane % 16) supplies
// A[row tl][base + 4 gq + s] and B[base + 4 gq + s][col tl]; the result lane
// holds C[4 gq + ii][tl].  A C-layout tile therefore serves directly as the B
// operand of a product that contracts over its rows.

#include "kda_bwd.h"
#include "kda_host.h"

namespace kda {
namespace {

constexpr int NT = 256;  // recurrence kernel: 4 waves
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
// norms of q and k.  NTH threads: NTH / 64 per token, KD / (NTH / 64) channels
// each.  sTmp needs NTH floats.
template <int NTH>
__device__ void prep_chunk(const BwdArgs& a, int64_t c0, int L, int h, float* sQn, float* sKn, float* sG,
                           float* sBeta, float* sRq, float* sRk, float* sTmp) {
  constexpr int TPR = NTH / CH;  // threads per token
  constexpr int CPT = KD / TPR;  // channels per thread
  const int t = threadIdx.x;
  const int i = t / TPR;
  const int part = t % TPR;
  const bool ok = i < L;
  const int64_t row = c0 + (ok ? i : L - 1);  // L >= 1: the clamped row is in range
  const size_t base = ((size_t)row * a.H + h) * KD + CPT * part;
  float qv[CPT], kv[CPT], gv[CPT];
#pragma unroll
  for (int u = 0; u < CPT / 8; ++u) {
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
  for (int c = 0; c < CPT; ++c) {
    sq += qv[c] * qv[c];
    sk += kv[c] * kv[c];
  }
#pragma unroll
  for (int d = 1; d < TPR; d <<= 1) {
    sq += __shfl_xor(sq, d);
    sk += __shfl_xor(sk, d);
  }
  const bool norm = !(a.flags & FLAG_NO_QK_NORM);
  const bool gate_given = a.flags & FLAG_GATE_GIVEN;
  const float rq = norm ? sqrtf(sq + L2_EPS) : 1.0f, rk = norm ? sqrtf(sk + L2_EPS) : 1.0f;
  const float iq = ok ? 1.0f / rq : 0.f, ik = ok ? 1.0f / rk : 0.f;
  // with the gate given, A_log and dt_bias may be absent and are not read
  const float al = gate_given ? 0.f : expf(a.A_log[h]);
#pragma unroll
  for (int c = 0; c < CPT; c += 4) {
    float gg[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float gn;
      if (gate_given)
        gn = fminf(fmaxf(gv[c + e], a.lb), 0.f);
      else
        gn = a.lb * sigmoidf(al * (gv[c + e] + a.dt_bias[(size_t)h * KD + CPT * part + c + e]));
      gg[e] = ok ? gn * LOG2E : 0.f;
    }
    *reinterpret_cast<float4*>(sQn + i * QP + CPT * part + c) =
        make_float4(qv[c] * iq, qv[c + 1] * iq, qv[c + 2] * iq, qv[c + 3] * iq);
    *reinterpret_cast<float4*>(sKn + i * QP + CPT * part + c) =
        make_float4(kv[c] * ik, kv[c + 1] * ik, kv[c + 2] * ik, kv[c + 3] * ik);
    *reinterpret_cast<float4*>(sG + i * QP + CPT * part + c) = make_float4(gg[0], gg[1], gg[2], gg[3]);
  }
  if (part == 0) {
    const float rb = bf2f(a.beta[(size_t)row * a.H + h]);
    sBeta[i] = ok ? ((a.flags & FLAG_BETA_GIVEN) ? rb : sigmoidf(rb)) : 0.f;
    sRq[i] = rq;
    sRk[i] = rk;
  }
  __syncthreads();
  // inclusive cumulative sum over the 64 tokens: thread -> channel t % 128,
  // segment t / 128 of 64 / (NTH / 128) tokens
  {
    constexpr int NSEG = NTH / KD;
    constexpr int RS = CH / NSEG;
    const int c = t % KD;
    const int sg = t / KD;
    float run = 0.f;
#pragma unroll 4
    for (int r = RS * sg; r < RS * sg + RS; ++r) {
      run += sG[r * QP + c];
      sG[r * QP + c] = run;
    }
    sTmp[sg * KD + c] = run;
    __syncthreads();
    float off = 0.f;
#pragma unroll
    for (int u = 0; u < NSEG; ++u)
      if (u < sg) off += sTmp[u * KD + c];
    if (sg > 0) {
#pragma unroll 4
      for (int r = RS * sg; r < RS * sg + RS; ++r) sG[r * QP + c] += off;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// kda_bwd_prep_kernel: per (chunk, head), the chunk factors in fp32.  8 waves:
// wave (w, p) = (wave % 4, wave / 4) owns row block w and the column blocks
// (or channel tiles) of parity p.
// ---------------------------------------------------------------------------
constexpr int NTP = 512;
constexpr int PREP_FLOATS = 3 * CH * QP + 2 * CH * MP + 3 * CH + NTP;

__global__ void __launch_bounds__(NTP, 1) kda_bwd_prep_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float smem[PREP_FLOATS];
  float* sQn = smem;
  float* sKn = sQn + CH * QP;
  float* sG = sKn + CH * QP;
  float* sKK = sG + CH * QP;
  float* sT = sKK + CH * MP;
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

  prep_chunk<NTP>(a, c0, L, h, sQn, sKn, sG, sBeta, sRq, sRk, sTmp);

  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int w = wv & 3;
  const int p = wv >> 2;
  const int lane = tid & 63;
  const int tl = lane & 15;
  const int gq = lane >> 4;

  // ---- KK and A_qk, row block w, column blocks b of parity p.  Reference
  // token r between i and j: the last token of block b (b < w), else the
  // first of w.  Blocks above the diagonal are zero.
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int b = 2 * bb + p;
    if (b > w) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * w + 4 * gq + ii, j = 16 * b + tl;
        sKK[i * MP + j] = 0.f;
        br[BR_KK + i * CH + j] = 0.f;
      }
      // A_qk^T tile (rows block b, contraction block w) is above the diagonal: zero
      store_hl4(br + BR_AQKT, CH * CH, frag_tt(16 * b + tl, 16 * w + 4 * gq), 0.f, 0.f, 0.f, 0.f);
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
    float qk4[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 16 * w + 4 * gq + ii, j = 16 * b + tl;
      const float kk = (b < w || j < i) ? ak[ii] : 0.f;
      qk4[ii] = (b < w || j <= i) ? aq[ii] : 0.f;
      sKK[i * MP + j] = kk;
      br[BR_KK + i * CH + j] = kk;
    }
    // scale A_qk^T[j][i]: rows j = 16b + tl, contraction i = 16w + 4gq + ii
    store_hl4(br + BR_AQKT, CH * CH, frag_tt(16 * b + tl, 16 * w + 4 * gq), a.scale * qk4[0], a.scale * qk4[1],
              a.scale * qk4[2], a.scale * qk4[3]);
  }
  __syncthreads();

  // ---- T = (I + diag(beta) KK)^-1.  Diagonal 16x16 blocks by forward
  // substitution (waves with p = 0; lane tl owns column tl); waves with p = 1
  // zero the upper blocks.
  if (p == 0) {
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
  } else {
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (b > w) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sT[(16 * w + 4 * gq + ii) * MP + 16 * b + tl] = 0.f;
      }
  }
  __syncthreads();
  // off-diagonal blocks by diagonals: T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb,
  // one 16 x 16 block per block row and level (waves with p = 0)
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (p == 0 && w >= d) {
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
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = 4 * (tid + NTP * u);
    *reinterpret_cast<float4*>(br + BR_T + e) = ld4(sT + (e >> 6) * MP + (e & 63));
  }

  // ---- W = Tb KG, row block w, channel tiles n of parity p; contraction over tokens j < 16w + 16
  {
    float tb[4][4];  // Tb[16w + tl][16 jb + 4 gq + s]
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kap = 16 * jb + 4 * gq + s;
        tb[jb][s] = sT[(16 * w + tl) * MP + kap] * sBeta[kap];
      }
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4) {
      const int n = 2 * n4 + p;
      f32x4 acc = zero4();
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        if (jb > w) continue;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int kap = 16 * jb + 4 * gq + s;
          const int c = 16 * n + tl;
          acc = mfma_f32(tb[jb][s], sKn[kap * QP + c] * fexp2(sG[kap * QP + c]), acc);
        }
      }
      // -W^T[k][i]: rows k = 16n + tl, contraction i = 16w + 4gq + ii
      store_hl4(br + BR_WT, CH * KD, frag_ct(16 * n + tl, 16 * w + 4 * gq), -acc[0], -acc[1], -acc[2], -acc[3]);
    }
  }

  // ---- Kt (thread: token tid / 8, 16 channels), QG^T (thread: channel tid / 4,
  // 16 tokens), exp(G_L), beta
  {
    const int i = tid >> 3;
    const int c8 = 16 * (tid & 7);
#pragma unroll
    for (int c = c8; c < c8 + 16; c += 4) {
      const float4 kn = ld4(sKn + i * QP + c), gg = ld4(sG + i * QP + c);
      const float4 gl = ld4(sG + (CH - 1) * QP + c);
      float4 kt;
      kt.x = kn.x * fexp2(gl.x - gg.x); kt.y = kn.y * fexp2(gl.y - gg.y);
      kt.z = kn.z * fexp2(gl.z - gg.z); kt.w = kn.w * fexp2(gl.w - gg.w);
      store_hl4(br + BR_KT, CH * KD, frag_tc(i, c), kt.x, kt.y, kt.z, kt.w);
    }
    const int k = tid >> 2;
    const int i0 = 16 * (tid & 3);
#pragma unroll
    for (int ib = i0; ib < i0 + 16; ib += 4) {
      float q4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q4[u] = a.scale * sQn[(ib + u) * QP + k] * fexp2(sG[(ib + u) * QP + k]);
      store_hl4(br + BR_QGT, CH * KD, frag_ct(k, ib), q4[0], q4[1], q4[2], q4[3]);
    }
    if (tid < KD) br[BR_GL + tid] = fexp2(sG[(CH - 1) * QP + tid]);
    if (tid < CH) br[BR_BETA + tid] = sBeta[tid];
  }
}

// ---------------------------------------------------------------------------
// kda_bwd_dhu_kernel: per (sequence, head, V half), chunks in reverse order.
// bf16 MFMA 16x16x32 with hi/lo splits on both sides of every product that
// has an fp32 operand (3 passes), 2 passes where one side is the exact bf16
// dO.  The state gradient dS stays in fp32 MFMA accumulators: wave w holds
// channels 32w + 16mt + 4gq + ii, columns vs + 16nn + tl.  Its bf16 hi/lo
// copy, the dO tile and dD hi/lo live in LDS column-major, so every B operand
// is one 16-byte LDS read.  The next chunk's record operands and dO rows are
// loaded one chunk ahead.
// ---------------------------------------------------------------------------
constexpr int TPB = CH + 8;  // token pitch of the [v][i] bf16 dO tile
// dS' hi/lo: 16 split-plane fragments each (column tile nn, k-block kb);
// dD hi/lo: 8 each (nn, token block ks); then the dO tile
constexpr int DHU_SH = 0, DHU_SL = 16 * FRAG, DHU_DH = 32 * FRAG, DHU_DL = 40 * FRAG, DHU_O = 48 * FRAG;
constexpr int DHU_BYTES = DHU_O + VH * TPB * 2;

struct DhuOps {
  bf16x8 kth[4], ktl[4];          // Kt rows 16w + tl, channels 32kb + 8gq ..
  bf16x8 aqh[2], aql[2];          // scale A_qk^T rows 16w + tl, tokens 32ks + 8gq ..
  bf16x8 qgh[2][2], qgl[2][2];    // scale QG^T rows 32w + 16mt + tl, tokens 32ks + 8gq ..
  bf16x8 wth[2][2], wtl[2][2];    // -W^T
  float4 gl[2];                   // exp(G_L) of channels 32w + 16mt + 4gq + 0..3
  uint4 dob[2];                   // dO row tid / 4, columns vs + 16 (tid % 4) .. + 15 (zero past the end)
};

__device__ __forceinline__ void dhu_load(DhuOps& o, const float* br, const uint16_t* dorow, bool rowok, int w,
                                         int lane, int gq) {
  const bf16x8* kt = reinterpret_cast<const bf16x8*>(br + BR_KT) + lane;
  const bf16x8* aq = reinterpret_cast<const bf16x8*>(br + BR_AQKT) + lane;
  const bf16x8* qg = reinterpret_cast<const bf16x8*>(br + BR_QGT) + lane;
  const bf16x8* wt = reinterpret_cast<const bf16x8*>(br + BR_WT) + lane;
  constexpr int LO_TC = CH * KD / 8, LO_TT = CH * CH / 8;  // lo arrays, in 16-byte units
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    o.kth[kb] = kt[(w * 4 + kb) * 64];
    o.ktl[kb] = kt[LO_TC + (w * 4 + kb) * 64];
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    o.aqh[ks] = aq[(w * 2 + ks) * 64];
    o.aql[ks] = aq[LO_TT + (w * 2 + ks) * 64];
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int f = ((2 * w + mt) * 2 + ks) * 64;
      o.qgh[mt][ks] = qg[f];
      o.qgl[mt][ks] = qg[LO_TC + f];
      o.wth[mt][ks] = wt[f];
      o.wtl[mt][ks] = wt[LO_TC + f];
    }
    o.gl[mt] = ld4(br + BR_GL + 32 * w + 16 * mt + 4 * gq);
  }
  if (rowok) {
    o.dob[0] = reinterpret_cast<const uint4*>(dorow)[0];
    o.dob[1] = reinterpret_cast<const uint4*>(dorow)[1];
  } else {
    o.dob[0] = o.dob[1] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// dO tile, transposed into sO[v][i] (2 tokens per dword).  Thread -> (token
// tid / 4, columns 16 (tid % 4) .. + 15); lanes of tokens t, t ^ 1 (4 lanes
// apart) trade half their columns, so each lane writes 8 packed dwords.
__device__ __forceinline__ void store_dot(__bf16* sO, const uint4 (&vv)[2], int tid) {
  const int t = tid >> 2;
  const int cg = tid & 3;
  const bool odd = t & 1;
  const uint32_t wds[8] = {vv[0].x, vv[0].y, vv[0].z, vv[0].w, vv[1].x, vv[1].y, vv[1].z, vv[1].w};
  uint32_t mine[4], recv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mine[j] = odd ? wds[4 + j] : wds[j];
    recv[j] = (uint32_t)__shfl_xor((int)(odd ? wds[j] : wds[4 + j]), 4);
  }
  const int tp = t & ~1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 16 * cg + (odd ? 8 : 0) + 2 * j;
    const uint32_t lo = odd ? recv[j] : mine[j];  // token tp
    const uint32_t hi = odd ? mine[j] : recv[j];  // token tp + 1
    *reinterpret_cast<uint32_t*>(sO + c * TPB + tp) = (lo & 0xffffu) | (hi << 16);
    *reinterpret_cast<uint32_t*>(sO + (c + 1) * TPB + tp) = (lo >> 16) | (hi & 0xffff0000u);
  }
}

__device__ __forceinline__ void split_hl4(const f32x4& x, bf16x4& h, bf16x4& l) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = (__bf16)x[e];
    l[e] = (__bf16)(x[e] - (float)h[e]);
  }
}

__global__ void __launch_bounds__(NT, 1) kda_bwd_dhu_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[DHU_BYTES];
  char* sSh = smem + DHU_SH;                        // dS' hi, fragments (nn, kb)
  char* sSl = smem + DHU_SL;                        // dS' lo
  char* sDh = smem + DHU_DH;                        // dD hi, fragments (nn, ks)
  char* sDl = smem + DHU_DL;                        // dD lo
  __bf16* sO = reinterpret_cast<__bf16*>(smem + DHU_O);  // [64 v][TPB]  dO (unscaled, exact)

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
  const int orow = tid >> 2;  // dO staging: row and 16 columns
  const int ocol = 16 * (tid & 3);

  f32x4 dS[2][4];
  const bool svk = a.flags & FLAG_STATE_VK;  // d_final / d_initial_state stored [V][K]
  {
    const float* src = a.dfin ? a.dfin + ((size_t)seq * H + h) * KD * VD : nullptr;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          dS[mt][nn][ii] = src ? src[svk ? (vs + 16 * nn + tl) * KD + 32 * w + 16 * mt + 4 * gq + ii
                                         : (32 * w + 16 * mt + 4 * gq + ii) * VD + vs + 16 * nn + tl]
                               : 0.f;
  }
  auto dorow_of = [&](int ci, bool& ok) {
    const int64_t c0 = bos + (int64_t)ci * CH;
    ok = c0 + orow < eos;
    return a.dout + ((size_t)(c0 + (ok ? orow : 0)) * H + h) * VD + vs + ocol;
  };

  DhuOps cur, nxt;
  if (nch > 0) {
    bool ok;
    const uint16_t* dr = dorow_of(nch - 1, ok);
    dhu_load(cur, a.br + ((size_t)(gfirst + nch - 1) * H + h) * BWD_REC_FLOATS, dr, ok, w, lane, gq);
  }

  for (int ci = nch - 1; ci >= 0; --ci) {
    const int64_t gch = gfirst + ci;
    const size_t it = (size_t)gch * H + h;
    {  // next (earlier) chunk's operands; the first chunk re-reads itself
      const int cn = ci > 0 ? ci - 1 : ci;
      bool ok;
      const uint16_t* dr = dorow_of(cn, ok);
      dhu_load(nxt, a.br + ((size_t)(gfirst + cn) * H + h) * BWD_REC_FLOATS, dr, ok, w, lane, gq);
    }

    // dS' of this chunk: fp32 to the checkpoint buffer (unless only the
    // entering gradient is wanted), bf16 hi/lo to LDS
    float* dsg = a.dstates ? a.dstates + it * KD * VD : nullptr;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < 4; ++nn) {
        const int k0 = 32 * w + 16 * mt + 4 * gq;
        const int col = 16 * nn + tl;
        if (dsg) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) dsg[(k0 + ii) * VD + vs + col] = dS[mt][nn][ii];
        }
        bf16x4 hv, lv;
        split_hl4(dS[mt][nn], hv, lv);
        frag_write4(sSh, 4 * nn + w, 4 * mt + gq, tl, hv);
        frag_write4(sSl, 4 * nn + w, 4 * mt + gq, tl, lv);
      }
    store_dot(sO, cur.dob, tid);
    __syncthreads();

    // dD rows 16w.. = Kt dS' + (scale A_qk^T) dO.  The B operands come in six
    // groups of four (one per column tile): four k-blocks of dS' hi/lo, then
    // two token blocks of dO.  Each group feeds four or eight independent MFMA
    // chains and is read one group ahead behind a scheduling barrier, so one
    // LDS latency is exposed per group instead of one per read.
    float* ddg = a.ddtile ? a.ddtile + it * CH * VD : nullptr;
    {
      f32x4 acc[4];
#pragma unroll
      for (int nn = 0; nn < 4; ++nn) acc[nn] = zero4();
      uint4 bq[2][4][2];
      auto read_group = [&](int g, uint4(&dst)[4][2]) {
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
          if (g < 4) {
            dst[nn][0] = frag_read(sSh, 4 * nn + g, lane);
            dst[nn][1] = frag_read(sSl, 4 * nn + g, lane);
          } else {
            dst[nn][0] = *reinterpret_cast<const uint4*>(sO + (16 * nn + tl) * TPB + 32 * (g - 4) + 8 * gq);
          }
        }
      };
      read_group(0, bq[0]);
#pragma unroll
      for (int g = 0; g < 6; ++g) {
        if (g + 1 < 6) read_group(g + 1, bq[(g + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
          if (g < 4) {
            const bf16x8 bh = __builtin_bit_cast(bf16x8, bq[g & 1][nn][0]);
            const bf16x8 bl = __builtin_bit_cast(bf16x8, bq[g & 1][nn][1]);
            acc[nn] = mfma_bf16(cur.kth[g], bh, acc[nn]);
            acc[nn] = mfma_bf16(cur.kth[g], bl, acc[nn]);
            acc[nn] = mfma_bf16(cur.ktl[g], bh, acc[nn]);
          } else {
            const bf16x8 ob = __builtin_bit_cast(bf16x8, bq[g & 1][nn][0]);
            acc[nn] = mfma_bf16(cur.aqh[g - 4], ob, acc[nn]);
            acc[nn] = mfma_bf16(cur.aql[g - 4], ob, acc[nn]);
          }
        }
      }
#pragma unroll
      for (int nn = 0; nn < 4; ++nn) {
        const int col = 16 * nn + tl;
        if (ddg) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) ddg[(16 * w + 4 * gq + ii) * VD + vs + col] = acc[nn][ii];
        }
        bf16x4 hv, lv;
        split_hl4(acc[nn], hv, lv);
        frag_write4(sDh, 2 * nn + (w >> 1), 4 * (w & 1) + gq, tl, hv);
        frag_write4(sDl, 2 * nn + (w >> 1), 4 * (w & 1) + gq, tl, lv);
      }
    }
    __syncthreads();

    // dS = Diag(exp(G_L)) dS' + (scale QG^T) dO + (-W^T) dD; a column tile's six
    // B operands are read one tile ahead
    {
      uint4 dq[2][6];
      auto read_tile = [&](int nn, uint4(&dst)[6]) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          dst[ks] = *reinterpret_cast<const uint4*>(sO + (16 * nn + tl) * TPB + 32 * ks + 8 * gq);
          dst[2 + ks] = frag_read(sDh, 2 * nn + ks, lane);
          dst[4 + ks] = frag_read(sDl, 2 * nn + ks, lane);
        }
      };
      read_tile(0, dq[0]);
#pragma unroll
      for (int nn = 0; nn < 4; ++nn) {
        if (nn + 1 < 4) read_tile(nn + 1, dq[(nn + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 ob[2], dh[2], dl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          ob[ks] = __builtin_bit_cast(bf16x8, dq[nn & 1][ks]);
          dh[ks] = __builtin_bit_cast(bf16x8, dq[nn & 1][2 + ks]);
          dl[ks] = __builtin_bit_cast(bf16x8, dq[nn & 1][4 + ks]);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          f32x4 st = dS[mt][nn];
          st[0] *= cur.gl[mt].x;
          st[1] *= cur.gl[mt].y;
          st[2] *= cur.gl[mt].z;
          st[3] *= cur.gl[mt].w;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            st = mfma_bf16(cur.qgh[mt][ks], ob[ks], st);
            st = mfma_bf16(cur.qgl[mt][ks], ob[ks], st);
            st = mfma_bf16(cur.wth[mt][ks], dh[ks], st);
            st = mfma_bf16(cur.wth[mt][ks], dl[ks], st);
            st = mfma_bf16(cur.wtl[mt][ks], dh[ks], st);
          }
          dS[mt][nn] = st;
        }
      }
    }
    __syncthreads();
    cur = nxt;
  }

  if (a.dinit) {
    float* dst = a.dinit + ((size_t)seq * H + h) * KD * VD;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          dst[svk ? (vs + 16 * nn + tl) * KD + 32 * w + 16 * mt + 4 * gq + ii
                  : (32 * w + 16 * mt + 4 * gq + ii) * VD + vs + 16 * nn + tl] = dS[mt][nn][ii];
  }
}

// ---------------------------------------------------------------------------
// kda_bwd_grad_kernel: per (chunk, head), 8 waves.  Wave (w, p) = (wave % 4,
// wave / 4) owns token block 16w..16w+15 and half p of the work: channels
// 64p..64p+63 of every token-by-channel product, V half p of Z, alternate
// column blocks of the 64 x 64 products.  Two waves per SIMD hide each
// other's memory latency.
//
// V index permutation: a float4 load gives a lane 4 consecutive v, so in a
// 64-wide V half hv the A-operand row tl of "virtual tile" e is
// v = 64 hv + 4 tl + e, and C row 4 gq + ii of that tile is
// v = 64 hv + 16 gq + 4 ii + e.  Contractions over v use the same order, so
// every v-operand is a float4 (or 16-bf16) load.
// ---------------------------------------------------------------------------
constexpr int NT8 = 512;
constexpr int GRAD_FLOATS = 3 * CH * QP + 3 * CH * MP + 4 * CH + NT8 + 4 * KD + KD + 4 * KD + 4 * CH;
static_assert(GRAD_FLOATS * 4 <= 163840, "LDS");

__global__ void __launch_bounds__(NT8, 1) kda_bwd_grad_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float smem[GRAD_FLOATS];
  float* sQn = smem;
  float* sKn = sQn + CH * QP;
  float* sG = sKn + CH * QP;
  float* sT = sG + CH * QP;
  float* sM1 = sT + CH * MP;   // dA_qk
  float* sM2 = sM1 + CH * MP;  // dTb -> dT, then X = dT T^T, then dKK
  float* sBeta = sM2 + CH * MP;
  float* sRq = sBeta + CH;
  float* sRk = sRq + CH;
  float* sdB = sRk + CH;       // gradient of beta (atomically accumulated)
  float* sTmp = sdB + CH;      // [512]
  float* sGLw = sTmp + NT8;    // [4][128] per-block sums of dKt . Kt, later of d dt_bias
  float* sGL2 = sGLw + 4 * KD; // [128] exp(G_L) sum_v dS' . S0
  float* sCS = sGL2 + KD;      // [4][128] per-block column totals of dG
  float* sDot = sCS + 4 * KD;  // [2][64][2] half-row dots q^.dq^, k^.dk^
  // bf16 output staging, over sT / sM1 / sM2 once the pairwise products are done
  uint16_t* sOut = reinterpret_cast<uint16_t*>(sT);  // [3][64][128]: dq, dk, d raw_gate

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

  KDA_TIMER_DECL
  KDA_TIMER_MARK(0);
  const int tid = threadIdx.x;
  // loads that do not depend on the preparation, issued first
  float4 tcp[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) tcp[u] = ld4(br + BR_T + 4 * (tid + NT8 * u));
  float gl2 = 0.f;
  {
    const int c = tid >> 2;
    const int v0 = 32 * (tid & 3);
    float4 x[8], y[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      x[u] = ld4(dSn + c * VD + v0 + 4 * u);
      y[u] = ld4(S0 + c * VD + v0 + 4 * u);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) gl2 += x[u].x * y[u].x + x[u].y * y[u].y + x[u].z * y[u].z + x[u].w * y[u].w;
    gl2 += __shfl_xor(gl2, 1);
    gl2 += __shfl_xor(gl2, 2);
  }
  prep_chunk<NT8>(a, c0, L, h, sQn, sKn, sG, sBeta, sRq, sRk, sTmp);
  KDA_TIMER_MARK(1);

  const int wv = tid >> 6;
  const int w = wv & 3;
  const int p = wv >> 2;
  const int lane = tid & 63;
  const int tl = lane & 15;
  const int gq = lane >> 4;
  const int jw = 16 * w + tl;  // this lane's token as an A row / B column

#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = 4 * (tid + NT8 * u);
    *reinterpret_cast<float4*>(sT + (e >> 6) * MP + (e & 63)) = tcp[u];
  }
  if ((tid & 3) == 0) sGL2[tid >> 2] = gl2 * fexp2(sG[(CH - 1) * QP + (tid >> 2)]);
  for (int e = tid; e < CH * MP; e += NT8) {
    sM1[e] = 0.f;
    sM2[e] = 0.f;
  }
  if (tid < CH) sdB[tid] = 0.f;
  __syncthreads();
  KDA_TIMER_MARK(2);

  const bool jok = jw < L;
  const size_t jrow = ((size_t)(c0 + (jok ? jw : 0)) * H + h);
  const float bj = sBeta[jw];

  // ---- Z^T, V half p: Z^T[v][jw] = V[jw][v] - sum_k S0[k][v] KG[jw][k]
  f32x4 Zt[4];
  {
#pragma unroll
    for (int e = 0; e < 4; ++e) Zt[e] = zero4();
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float4 kn = ld4(sKn + jw * QP + 16 * t + 4 * gq), gg = ld4(sG + jw * QP + 16 * t + 4 * gq);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float kg = el(kn, s) * fexp2(el(gg, s));
        const float4 a4 = ld4(S0 + (16 * t + 4 * gq + s) * VD + 64 * p + 4 * tl);
#pragma unroll
        for (int e = 0; e < 4; ++e) Zt[e] = mfma_f32(el(a4, e), kg, Zt[e]);
      }
    }
    float vv[16];
    if (jok) {
      const uint4* src = reinterpret_cast<const uint4*>(a.v + jrow * VD + 64 * p + 16 * gq);
      unpack_bf16x8(src[0], *reinterpret_cast<float(*)[8]>(vv));
      unpack_bf16x8(src[1], *reinterpret_cast<float(*)[8]>(vv + 8));
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) vv[r] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) Zt[e][ii] = vv[4 * ii + e] - Zt[e][ii];
  }
  // ---- dTb[i][jw] for i >= 16w, V half p (atomically summed over p): dD Z^T on
  // bf16 MFMA, hi/lo on both sides.  k-step `half` takes v = 64p + 16gq + 8half + 0..7,
  // which Zt holds as Zt[e8 % 4][2 half + e8 / 4].
  {
    bf16x8 zh[2], zl[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float zx[8];
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) zx[e8] = Zt[e8 & 3][2 * half + (e8 >> 2)];
      split_hl8(zx, zh[half], zl[half]);
    }
#pragma unroll
    for (int ab = 0; ab < 4; ++ab) {
      if (ab < w) continue;
      f32x4 acc = zero4();
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 ah, al;
        ld_hl8(dDt + (16 * ab + tl) * VD + 64 * p + 16 * gq + 8 * half, ah, al);
        acc = mfma_bf16(ah, zh[half], acc);
        acc = mfma_bf16(ah, zl[half], acc);
        acc = mfma_bf16(al, zh[half], acc);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) atomicAdd(sM2 + (16 * ab + 4 * gq + ii) * MP + jw, acc[ii]);
    }
  }
  KDA_TIMER_MARK(3);

  // ---- dv^T, both V halves: dv[jw][v] = sum_{i >= jw} Tb[i][jw] dD[i][v]
  f32x4 dvT[2][4];
  {
#pragma unroll
    for (int hv = 0; hv < 2; ++hv)
#pragma unroll
      for (int e = 0; e < 4; ++e) dvT[hv][e] = zero4();
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      if (ib < w) continue;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kap = 16 * ib + 4 * gq + s;
        const float tb = sT[kap * MP + jw] * bj;
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
          const float4 a4 = ld4(dDt + kap * VD + 64 * hv + 4 * tl);
#pragma unroll
          for (int e = 0; e < 4; ++e) dvT[hv][e] = mfma_f32(el(a4, e), tb, dvT[hv][e]);
        }
      }
    }
    if (jok) {  // wave p writes V half p: 16 consecutive v per lane
      uint32_t pk[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int r0 = 2 * r, r1 = 2 * r + 1;  // r = 4 ii + e
        const float x0 = p ? dvT[1][r0 & 3][r0 >> 2] : dvT[0][r0 & 3][r0 >> 2];
        const float x1 = p ? dvT[1][r1 & 3][r1 >> 2] : dvT[0][r1 & 3][r1 >> 2];
        pk[r] = (uint32_t)f2bf(x0) | ((uint32_t)f2bf(x1) << 16);
      }
      uint4* dst = reinterpret_cast<uint4*>(a.dv + jrow * VD + 64 * p + 16 * gq);
      dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    }
  }
  KDA_TIMER_MARK(4);

  // ---- bf16 MFMA operands over v for the products below.  k-step (hv, half)
  // takes v = 64hv + 16gq + 8half + 0..7 in lane group gq:
  //   dO[jw][v] (exact bf16, the scale is applied to the results),
  //   -dv[jw][v] hi/lo (dvT holds it as dvT[hv][e8 % 4][2 half + e8 / 4]),
  //   D[jw][v] hi/lo (loaded where it is used).
  bf16x8 doA[2][2], dvh[2][2], dvl[2][2];
#pragma unroll
  for (int hv = 0; hv < 2; ++hv)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (jok)
        doA[hv][half] = *reinterpret_cast<const bf16x8*>(a.dout + jrow * VD + 64 * hv + 16 * gq + 8 * half);
      else
        doA[hv][half] = bf16x8{};
      float x[8];
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) x[e8] = -dvT[hv][e8 & 3][2 * half + (e8 >> 2)];
      split_hl8(x, dvh[hv][half], dvl[hv][half]);
    }
  // ---- dA_qk[block w][block b] = scale dO D^T (j <= i), column blocks b <= w of parity p
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b > w || (b & 1) != p) continue;
    f32x4 acc = zero4();
#pragma unroll
    for (int hv = 0; hv < 2; ++hv)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 bh, bl;
        ld_hl8(Dt + (16 * b + tl) * VD + 64 * hv + 16 * gq + 8 * half, bh, bl);
        acc = mfma_bf16(doA[hv][half], bh, acc);
        acc = mfma_bf16(doA[hv][half], bl, acc);
      }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 16 * w + 4 * gq + ii, j = 16 * b + tl;
      sM1[i * MP + j] = (j <= i) ? acc[ii] * a.scale : 0.f;
    }
  }

  // ---- dQG = scale dO S0^T, dKG = -dv S0^T, dKt = D dS'^T for channels 64p..64p+63,
  // and their elementwise contributions to dq^, dk^, dG
  f32x4 dqh[4], dkh[4], dGa[4];
#pragma unroll
  for (int nn = 0; nn < 4; ++nn) {
    const int kc = 64 * p + 16 * nn + tl;
    f32x4 aQ = zero4(), aK = zero4(), aT = zero4();
#pragma unroll
    for (int hv = 0; hv < 2; ++hv)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 sh, sl, th, tl8, dah, dal;
        ld_hl8(S0 + kc * VD + 64 * hv + 16 * gq + 8 * half, sh, sl);
        ld_hl8(dSn + kc * VD + 64 * hv + 16 * gq + 8 * half, th, tl8);
        ld_hl8(Dt + jw * VD + 64 * hv + 16 * gq + 8 * half, dah, dal);
        aQ = mfma_bf16(doA[hv][half], sh, aQ);
        aQ = mfma_bf16(doA[hv][half], sl, aQ);
        aK = mfma_bf16(dvh[hv][half], sh, aK);
        aK = mfma_bf16(dvh[hv][half], sl, aK);
        aK = mfma_bf16(dvl[hv][half], sh, aK);
        aT = mfma_bf16(dah, th, aT);
        aT = mfma_bf16(dah, tl8, aT);
        aT = mfma_bf16(dal, th, aT);
      }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) aQ[ii] *= a.scale;
    const int c = 64 * p + 16 * nn + tl;
    float glsum = 0.f;
    const float gl2c = sG[(CH - 1) * QP + c];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int j = 16 * w + 4 * gq + ii;
      const float qn = sQn[j * QP + c], kn = sKn[j * QP + c], g2 = sG[j * QP + c];
      const float gam = fexp2(g2), el2 = fexp2(gl2c - g2);
      const float kt = kn * el2;
      dqh[nn][ii] = aQ[ii] * gam;
      dkh[nn][ii] = aK[ii] * gam + aT[ii] * el2;
      dGa[nn][ii] = aQ[ii] * qn * gam + aK[ii] * kn * gam - aT[ii] * kt;
      glsum += aT[ii] * kt;
    }
    glsum += __shfl_xor(glsum, 16);
    glsum += __shfl_xor(glsum, 32);
    if (gq == 0) sGLw[w * KD + c] = glsum;
  }
  KDA_TIMER_MARK(5);

  __syncthreads();
  KDA_TIMER_MARK(6);

  // ---- dT = dTb diag(beta) in place; column sums of dTb . T -> dbeta (rows split by p)
  {
    float colsum = 0.f;
#pragma unroll
    for (int ab = 0; ab < 4; ++ab) {
      if (ab < w || ((ab - w) & 1) != p) continue;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * ab + 4 * gq + ii;
        const float v = sM2[i * MP + jw];
        colsum += v * sT[i * MP + jw];
        sM2[i * MP + jw] = v * bj;
      }
    }
    colsum += __shfl_xor(colsum, 16);
    colsum += __shfl_xor(colsum, 32);
    if (gq == 0) atomicAdd(sdB + jw, colsum);
  }
  __syncthreads();
  // ---- X = dT T^T, row block w, column blocks q <= w of parity p
  {
    f32x4 X[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int q = 2 * qq + p;
      X[qq] = zero4();
      if (q > w) continue;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b > q) continue;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int kap = 16 * b + 4 * gq + s;
          X[qq] = mfma_f32(sM2[jw * MP + kap], sT[(16 * q + tl) * MP + kap], X[qq]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int q = 2 * qq + p;
      if (q > w) continue;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sM2[(16 * w + 4 * gq + ii) * MP + 16 * q + tl] = X[qq][ii];
    }
  }
  __syncthreads();
  // ---- dA_kk[block w][m < a] = -T^T X; row sums of dA_kk . KK -> dbeta; dKK = dA_kk beta_a
  {
    f32x4 dkk[2];
    float rows[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int q = 2 * qq + p;
      f32x4 acc = zero4();
      if (q <= w) {
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
          if (pb < w) continue;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int kap = 16 * pb + 4 * gq + s;
            acc = mfma_f32(-sT[kap * MP + jw], sM2[kap * MP + 16 * q + tl], acc);
          }
        }
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int ar = 16 * w + 4 * gq + ii, mc = 16 * q + tl;
        const float v = (q <= w && mc < ar) ? acc[ii] : 0.f;
        rows[ii] += v * br[BR_KK + ar * CH + (mc & 63)];
        acc[ii] = v * sBeta[ar];
      }
      dkk[qq] = acc;
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float r = rows[ii];
      r += __shfl_xor(r, 1);
      r += __shfl_xor(r, 2);
      r += __shfl_xor(r, 4);
      r += __shfl_xor(r, 8);
      if (tl == 0) atomicAdd(sdB + 16 * w + 4 * gq + ii, r);
    }
    __syncthreads();
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int q = 2 * qq + p;
      if (q > w) continue;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sM2[(16 * w + 4 * gq + ii) * MP + 16 * q + tl] = dkk[qq][ii];
    }
  }
  __syncthreads();
  KDA_TIMER_MARK(7);

  // ---- pairwise products, row role: i in block w, j in blocks b <= w
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b > w) continue;
    const int r = (b < w) ? 16 * b + 15 : 16 * w;
    float m1[4], m2[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      m1[s] = sM1[jw * MP + 16 * b + 4 * gq + s];
      m2[s] = sM2[jw * MP + 16 * b + 4 * gq + s];
    }
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int c = 64 * p + 16 * nn + tl;
      const float gr = sG[r * QP + c];
      f32x4 a1 = zero4(), a2 = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kap = 16 * b + 4 * gq + s;
        const float y = sKn[kap * QP + c] * fexp2(gr - sG[kap * QP + c]);
        a1 = mfma_f32(m1[s], y, a1);
        a2 = mfma_f32(m2[s], y, a2);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * w + 4 * gq + ii;
        const float f = fexp2(sG[i * QP + c] - gr);
        const float v1 = a1[ii] * f, v2 = a2[ii] * f;
        dqh[nn][ii] += v1;
        dkh[nn][ii] += v2;
        dGa[nn][ii] += sQn[i * QP + c] * v1 + sKn[i * QP + c] * v2;
      }
    }
  }
  KDA_TIMER_MARK(8);
  // ---- pairwise products, column role: j in block w, i in blocks a >= w
#pragma unroll
  for (int ab = 0; ab < 4; ++ab) {
    if (ab < w) continue;
    const int r = (ab > w) ? 16 * w + 15 : 16 * w;
    float m1[4], m2[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      m1[s] = sM1[(16 * ab + 4 * gq + s) * MP + jw];
      m2[s] = sM2[(16 * ab + 4 * gq + s) * MP + jw];
    }
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int c = 64 * p + 16 * nn + tl;
      const float gr = sG[r * QP + c];
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kap = 16 * ab + 4 * gq + s;
        const float f = fexp2(sG[kap * QP + c] - gr);
        acc = mfma_f32(m1[s], sQn[kap * QP + c] * f, acc);
        acc = mfma_f32(m2[s], sKn[kap * QP + c] * f, acc);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = 16 * w + 4 * gq + ii;
        const float v = acc[ii] * fexp2(gr - sG[j * QP + c]);
        dkh[nn][ii] += v;
        dGa[nn][ii] -= sKn[j * QP + c] * v;
      }
    }
  }
  KDA_TIMER_MARK(9);

  // ---- dG_L on the last token, then the reverse cumulative sum -> dg
  const int lastw = (L - 1) >> 4;
#pragma unroll
  for (int nn = 0; nn < 4; ++nn) {
    const int c = 64 * p + 16 * nn + tl;
    if (w == lastw) {
      const float dgl = sGL2[c] + sGLw[c] + sGLw[KD + c] + sGLw[2 * KD + c] + sGLw[3 * KD + c];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        if (16 * w + 4 * gq + ii == L - 1) dGa[nn][ii] += dgl;
    }
    f32x4 x = dGa[nn];
    x[2] += x[3];
    x[1] += x[2];
    x[0] += x[1];
    const float tot = x[0];
    const float t1 = __shfl(tot, tl + 16), t2 = __shfl(tot, tl + 32), t3 = __shfl(tot, tl + 48);
    const float off = (gq < 1 ? t1 : 0.f) + (gq < 2 ? t2 : 0.f) + (gq < 3 ? t3 : 0.f);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) x[ii] += off;
    dGa[nn] = x;
    if (gq == 0) sCS[w * KD + c] = x[0];
  }
  // half-row dots q^.dq^ and k^.dk^ over this wave's 64 channels
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int j = 16 * w + 4 * gq + ii;
    float dq_dot = 0.f, dk_dot = 0.f;
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int c = 64 * p + 16 * nn + tl;
      dq_dot += sQn[j * QP + c] * dqh[nn][ii];
      dk_dot += sKn[j * QP + c] * dkh[nn][ii];
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      dq_dot += __shfl_xor(dq_dot, d);
      dk_dot += __shfl_xor(dk_dot, d);
    }
    if (tl == 0) {
      sDot[(p * CH + j) * 2] = dq_dot;
      sDot[(p * CH + j) * 2 + 1] = dk_dot;
    }
  }
  __syncthreads();
  KDA_TIMER_MARK(10);

  // ---- outputs, staged in LDS: d raw_gate, dq, dk; partial sums of d dt_bias, dA_log
  const bool gate_given = a.flags & FLAG_GATE_GIVEN;
  const float al = gate_given ? 0.f : expf(a.A_log[h]);
  float pA = 0.f;
  uint16_t* oq = sOut;
  uint16_t* ok_ = sOut + CH * KD;
  uint16_t* og = sOut + 2 * CH * KD;
#pragma unroll
  for (int nn = 0; nn < 4; ++nn) {
    const int c = 64 * p + 16 * nn + tl;
    float later = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u > w) later += sCS[u * KD + c];
    const float dtb = gate_given ? 0.f : a.dt_bias[(size_t)h * KD + c];
    float pdt = 0.f;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int j = 16 * w + 4 * gq + ii;
      const float dgv = dGa[nn][ii] + later;  // gradient of the natural-log decay g_j
      float dgo = 0.f;
      if (j < L) {
        const size_t o = ((size_t)(c0 + j) * H + h) * KD + c;
        const float rg = bf2f(a.g[o]);
        if (gate_given) {
          // g = clamp(raw_gate, lower_bound, 0): the gradient passes inside the closed interval
          dgo = (rg >= a.lb && rg <= 0.f) ? dgv : 0.f;
        } else {
          const float x = al * (rg + dtb);
          const float sg = sigmoidf(x);
          const float dx = dgv * a.lb * sg * (1.f - sg);
          dgo = dx * al;
          pdt += dgo;
          pA += dx * x;
        }
      }
      og[j * KD + c] = f2bf(dgo);
    }
    pdt += __shfl_xor(pdt, 16);
    pdt += __shfl_xor(pdt, 32);
    if (gq == 0) sGLw[w * KD + c] = pdt;  // sGLw is free again: dG_L was added before the barrier
  }
  // dq = (dq^ - q^ (q^ . dq^)) / |q|, same for k
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int j = 16 * w + 4 * gq + ii;
    // dq = dq^ when q is used without the L2 norm (the projection term and the row norm drop)
    const bool norm = !(a.flags & FLAG_NO_QK_NORM);
    const float dq_dot = norm ? sDot[j * 2] + sDot[(CH + j) * 2] : 0.f;
    const float dk_dot = norm ? sDot[j * 2 + 1] + sDot[(CH + j) * 2 + 1] : 0.f;
    const float irq = 1.f / sRq[j], irk = 1.f / sRk[j];
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int c = 64 * p + 16 * nn + tl;
      oq[j * KD + c] = f2bf((dqh[nn][ii] - sQn[j * QP + c] * dq_dot) * irq);
      ok_[j * KD + c] = f2bf((dkh[nn][ii] - sKn[j * QP + c] * dk_dot) * irk);
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) pA += __shfl_xor(pA, d);
  if (lane == 0) sTmp[wv] = pA;
  if (p == 0 && lane < 16 && jw < L) {
    const float b = sBeta[jw];
    a.dbeta[(size_t)(c0 + jw) * H + h] = f2bf((a.flags & FLAG_BETA_GIVEN) ? sdB[jw] : sdB[jw] * b * (1.f - b));
  }
  __syncthreads();
  // 16-byte stores of the staged rows: thread -> (row, 16-byte column block)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + NT8 * u;  // 0 .. 1023
    const int row = e >> 4;
    const int cb = 8 * (e & 15);
    if (row < L) {
      const size_t o = ((size_t)(c0 + row) * H + h) * KD + cb;
      *reinterpret_cast<uint4*>(a.dq + o) = *reinterpret_cast<const uint4*>(oq + row * KD + cb);
      *reinterpret_cast<uint4*>(a.dk + o) = *reinterpret_cast<const uint4*>(ok_ + row * KD + cb);
      *reinterpret_cast<uint4*>(a.dg + o) = *reinterpret_cast<const uint4*>(og + row * KD + cb);
    }
  }
  float* part = a.part + it * (KD + 1);
  if (tid < KD) part[tid] = sGLw[tid] + sGLw[KD + tid] + sGLw[2 * KD + tid] + sGLw[3 * KD + tid];
  if (tid == KD) {
    float sA = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) sA += sTmp[u];
    part[KD] = sA;
  }
  KDA_TIMER_MARK(11);
  KDA_TIMER_STORE(a.timers ? a.timers + (size_t)gridDim.x * 16 : nullptr);
}

// ---------------------------------------------------------------------------
// kda_bwd_reduce_kernel: per head, sum the per-chunk partials.  Thread t sums
// column t % 129 over the chunks of residue t / 129 mod 4, then the four
// partial sums meet in LDS.
// ---------------------------------------------------------------------------
constexpr int NTR = 4 * (KD + 1);

__global__ void __launch_bounds__(NTR) kda_bwd_reduce_kernel(BwdArgs a) {
  __shared__ float red[NTR];
  const int h = blockIdx.x;
  const int H = a.H;
  const int64_t nch = total_chunks(a.map);
  const int t = threadIdx.x;
  const int col = t % (KD + 1);
  const int rr = t / (KD + 1);
  float acc = 0.f;
  for (int64_t g = rr; g < nch; g += 4) acc += a.part[((size_t)g * H + h) * (KD + 1) + col];
  red[t] = acc;
  __syncthreads();
  if (rr == 0) {
    const float v = red[col] + red[(KD + 1) + col] + red[2 * (KD + 1) + col] + red[3 * (KD + 1) + col];
    if (col < KD) {
      if (a.ddt) a.ddt[(size_t)h * KD + col] = v;
    } else if (a.dA_log) {
      a.dA_log[h] = v;
    }
  }
}

}  // namespace

hipError_t launch_dhu(const BwdArgs& args, hipStream_t st) {
  BwdArgs a = args;
  void* kargs[] = {(void*)&a};
  const int64_t seqs = (int64_t)a.map.N * a.H;
  return hipLaunchKernel(reinterpret_cast<const void*>(&kda_bwd_dhu_kernel),
                         dim3((unsigned)((seqs + 7) / 8 * 8 * 2)), dim3(NT), kargs, 0, st);
}

hipError_t launch_bwd(const BwdArgs& args, int64_t max_chunks, const BwdShards* sh, hipStream_t st) {
  BwdArgs a = args;
  void* kargs[] = {(void*)&a};
  const int64_t items = max_chunks * a.H;
  hipError_t e;
  if (items > 0) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&kda_bwd_prep_kernel), dim3((unsigned)items), dim3(NTP),
                        kargs, 0, st);
    if (e != hipSuccess) return e;
  }
  if (!sh) {
    e = launch_dhu(a, st);
  } else {
    BwdArgs a1 = a;  // each shard's own entering gradient, no per-chunk stores
    a1.map = sh->m2;
    a1.order = nullptr;
    a1.dfin = nullptr;
    a1.dinit = sh->b;
    a1.dstates = nullptr;
    a1.ddtile = nullptr;
    e = launch_dhu(a1, st);
    const size_t kv = (size_t)KD * VD;
    for (int64_t n = 0; n < sh->N && e == hipSuccess; ++n) {
      const size_t o = (size_t)(n * sh->S * a.H) * kv, oq = (size_t)(n * a.H) * kv;
      e = launch_shard_scan_rev(sh->P + o, sh->b + o, a.dfin ? a.dfin + oq : nullptr, sh->ends + o,
                                a.dinit ? a.dinit + oq : nullptr, (int)sh->S, a.H, st);
    }
    if (e != hipSuccess) return e;
    BwdArgs a2 = a;  // the per-chunk gradients from every shard's leaving gradient
    a2.map = sh->m2;
    a2.order = nullptr;
    a2.dfin = sh->ends;
    a2.dinit = nullptr;
    e = launch_dhu(a2, st);
  }
  if (e != hipSuccess) return e;
  if (items > 0) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&kda_bwd_grad_kernel), dim3((unsigned)items), dim3(NT8),
                        kargs, 0, st);
    if (e != hipSuccess) return e;
  }
  return hipLaunchKernel(reinterpret_cast<const void*>(&kda_bwd_reduce_kernel), dim3((unsigned)a.H), dim3(NTR),
                         kargs, 0, st);
}

}  // namespace kda

namespace kda {
namespace {

// The backward pass keeps, after the forward's areas: the state entering and
// the state gradient leaving every chunk, every chunk's D and dD, its fp32
// factor record and its partial parameter-gradient sums.
struct BwdLayout {
  Layout fwd;
  size_t states, dtile, dstates, ddtile, br, part, total;
};

BwdLayout bwd_layout(int64_t T_total, int64_t H, int64_t N) {
  BwdLayout l;
  l.fwd = workspace_layout(T_total, H, N);
  const size_t items = ((size_t)(T_total / CH) + (size_t)N) * (size_t)H;
  l.states = align256(l.fwd.total);
  l.dtile = l.states + align256(items * KD * VD * 4);
  l.dstates = l.dtile + align256(items * CH * VD * 4);
  l.ddtile = l.dstates + align256(items * KD * VD * 4);
  l.br = l.ddtile + align256(items * CH * VD * 4);
  l.part = l.br + align256(items * BWD_REC_FLOATS * 4);
  l.total = l.part + align256(items * (KD + 1) * 4);
  return l;
}

}  // namespace
}  // namespace kda

using namespace kda;

extern "C" {

size_t kda_bwd_workspace_size(int64_t T_total, int64_t H, int64_t N) {
  if (T_total < 0 || H < 1 || N < 1) return 0;
  return bwd_layout(T_total, H, N).total;
}

kda_status_t kda_bwd_ex(const void* q, const void* k, const void* v, const void* raw_gate,
                        const void* raw_beta, float scale, const void* d_out, const float* d_final,
                        void* dq, void* dk, void* dv, void* d_raw_gate, void* d_raw_beta, float* dA_log,
                        float* d_dt_bias, float* d_initial_state, void* workspace, size_t workspace_bytes,
                        const float* A_log, const float* dt_bias, float lower_bound,
                        const float* initial_state, const int32_t* cu_seqlens, int64_t B, int64_t T,
                        int64_t H, int64_t K, int64_t V, int64_t N, unsigned flags, void* stream) {
  if (flags & ~(unsigned)(FLAG_GATE_GIVEN | FLAG_BETA_GIVEN | FLAG_NO_QK_NORM | FLAG_STATE_VK |
                          FLAG_REUSE_RECORDS))
    return KDA_ERR_INVALID;
  if (B * T > 0 && (!v || !d_out || !dq || !dk || !dv || !d_raw_gate || !d_raw_beta)) return KDA_ERR_INVALID;
  if (!(flags & FLAG_GATE_GIVEN) && (!dA_log || !d_dt_bias || !A_log || !dt_bias)) return KDA_ERR_INVALID;
  if (!(scale == scale)) return KDA_ERR_INVALID;
  if (B < 1 || T < 0 || H < 1 || N < 1) return KDA_ERR_INVALID;
  if (B * T * H > ((int64_t)1 << 40) || N * H > ((int64_t)1 << 28) || N > ((int64_t)1 << 30))
    return KDA_ERR_INVALID;
  const BwdLayout bl = bwd_layout(B * T, H, N);
  if (!workspace || workspace_bytes < bl.total) return KDA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Prepared pr;
  const kda_status_t s = prepare(q, k, raw_gate, raw_beta, workspace, workspace_bytes, A_log, dt_bias,
                                 lower_bound, cu_seqlens, B, T, H, K, V, N, st, pr, flags);
  if (s != KDA_SUCCESS) return s;
  // forward recurrence, keeping the state entering each chunk and each chunk's D;
  // with few long chains it runs on shards from their folded entering states,
  // which writes the same per-chunk checkpoints
  InterArgs xa = inter_args(pr, H);
  xa.v = static_cast<const uint16_t*>(v);
  xa.init = initial_state;
  xa.state_vk = (flags & FLAG_STATE_VK) ? 1 : 0;
  const bool split = use_split(pr, flags, B, T);
  ChunkMap m2;
  if (split) {
    const kda_status_t ss = shard_states(pr, v, initial_state, nullptr, T, H, N, st, m2);
    if (ss != KDA_SUCCESS) return ss;
    xa = shard_inter_args(pr, H, m2);
    xa.v = static_cast<const uint16_t*>(v);
    xa.init = reinterpret_cast<const float*>(pr.ws + pr.lay.sstart);
  }
  xa.states = reinterpret_cast<float*>(pr.ws + bl.states);
  xa.dtile = reinterpret_cast<float*>(pr.ws + bl.dtile);
  xa.timers = nullptr;  // (timer builds: the forward's counter area overlaps these checkpoints)
  if (launch_status(launch_inter(xa, st), "inter (checkpoints)") != KDA_SUCCESS) return KDA_ERR_LAUNCH;

  BwdArgs ba;
  ba.q = static_cast<const uint16_t*>(q);
  ba.k = static_cast<const uint16_t*>(k);
  ba.v = static_cast<const uint16_t*>(v);
  ba.g = static_cast<const uint16_t*>(raw_gate);
  ba.beta = static_cast<const uint16_t*>(raw_beta);
  ba.A_log = A_log;
  ba.dt_bias = dt_bias;
  ba.dout = static_cast<const uint16_t*>(d_out);
  ba.dfin = d_final;
  ba.dq = static_cast<uint16_t*>(dq);
  ba.dk = static_cast<uint16_t*>(dk);
  ba.dv = static_cast<uint16_t*>(dv);
  ba.dg = static_cast<uint16_t*>(d_raw_gate);
  ba.dbeta = static_cast<uint16_t*>(d_raw_beta);
  ba.dinit = d_initial_state;
  ba.dA_log = dA_log;
  ba.ddt = d_dt_bias;
  ba.states = xa.states;
  ba.dtile = xa.dtile;
  ba.dstates = reinterpret_cast<float*>(pr.ws + bl.dstates);
  ba.ddtile = reinterpret_cast<float*>(pr.ws + bl.ddtile);
  ba.br = reinterpret_cast<float*>(pr.ws + bl.br);
  ba.part = reinterpret_cast<float*>(pr.ws + bl.part);
  ba.order = pr.order;
  ba.map = pr.map;
  ba.H = (int)H;
  ba.scale = scale;
  ba.lb = lower_bound;
  ba.flags = (int)flags;
  ba.timers = nullptr;
#ifdef KDA_PHASE_TIMERS
  // timer builds only: 16 counters per workgroup of each backward kernel after the workspace
  ba.timers = reinterpret_cast<unsigned long long*>(pr.ws + bl.total);
#endif
  // with shards, the reverse recurrence runs on them too: the shard maps P
  // are still in the workspace, R's area (consumed by the fold) takes each
  // shard's own entering gradient and the final-state area the leaving ones
  BwdShards sh;
  if (split) {
    sh.m2 = m2;
    sh.N = N;
    sh.S = pr.lay.S;
    sh.P = reinterpret_cast<const float*>(pr.ws + pr.lay.sP);
    sh.b = reinterpret_cast<float*>(pr.ws + pr.lay.sR);
    sh.ends = reinterpret_cast<float*>(pr.ws + pr.lay.sfin);
  }
  return launch_status(launch_bwd(ba, pr.max_chunks, split ? &sh : nullptr, st), "backward");
}

kda_status_t kda_bwd(const void* q, const void* k, const void* v, const void* raw_gate,
                     const void* raw_beta, float scale, const void* d_out, const float* d_final,
                     void* dq, void* dk, void* dv, void* d_raw_gate, void* d_raw_beta, float* dA_log,
                     float* d_dt_bias, float* d_initial_state, void* workspace, size_t workspace_bytes,
                     const float* A_log, const float* dt_bias, float lower_bound,
                     const float* initial_state, const int32_t* cu_seqlens, int64_t B, int64_t T,
                     int64_t H, int64_t K, int64_t V, int64_t N, void* stream) {
  return kda_bwd_ex(q, k, v, raw_gate, raw_beta, scale, d_out, d_final, dq, dk, dv, d_raw_gate, d_raw_beta,
                    dA_log, d_dt_bias, d_initial_state, workspace, workspace_bytes, A_log, dt_bias, lower_bound,
                    initial_state, cu_seqlens, B, T, H, K, V, N, 0u, stream);
}

}  // extern "C"
