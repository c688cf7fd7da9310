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
//   kda_bwd_prep_kernel    per (chunk, head), persistent: fp32 T, A_kk / beta, A_qk, W, Kt, QG, exp(G_L)
//   kda_bwd_dhu_kernel     per (sequence, head, V half): the reverse recurrence -> dS', dD
//   kda_bwd_grad_kernel    per (chunk, head): dq, dk, dv, d raw_gate, d raw_beta, partials
//   kda_bwd_reduce_kernel  per head: dA_log and d dt_bias from the per-chunk partials
// Arithmetic is fp32 throughout: fp32 MFMA 16x16x4, or bf16 MFMA (16x16x32 and
// 16x16x16) with every fp32 operand split into a bf16 hi/lo pair (3 passes; 2 where the other
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
#include "kda_bwd_dev.h"
#include "kda_host.h"

namespace kda {
namespace {

constexpr int NT = 256;  // recurrence kernel: 4 waves
// One chunk's raw per-token inputs for the NTH threads of prep_chunk (NTH / 64
// per token, KD / (NTH / 64) channels each), loaded into registers ahead of
// their use: a persistent workgroup loads the next item's while it works on
// the current one.
template <int NTH>
struct PrepIn {
  static constexpr int CPT = KD / (NTH / CH);  // channels per thread
  uint4 q[CPT / 8], k[CPT / 8], g[CPT / 8];
  float db[CPT];       // dt_bias of the thread's channels (zero with the gate given)
  float A_log;         // the head's A_log (zero with the gate given)
  uint16_t beta;       // raw beta of the thread's token, bf16 bits (converted at use,
                       // so that nothing waits for the load)
};

template <int NTH, bool FULL>
__device__ __forceinline__ void prep_load(const BwdArgs& a, int64_t c0, int L, int h, PrepIn<NTH>& in) {
  constexpr int TPR = NTH / CH;
  constexpr int CPT = PrepIn<NTH>::CPT;
  const int t = threadIdx.x;
  const int i = t / TPR;
  const int part = t % TPR;
  const int64_t row = c0 + (i < L ? i : L - 1);  // L >= 1: the clamped row is in range
  const int kd = FULL ? KD : a.kd;
  // channels past the head dim: the loads go to channel 0 (kept unconditional,
  // so they stay 16-byte loads) and prep_chunk drops them
  const int c0l = FULL || CPT * part < kd ? CPT * part : 0;
  const size_t base = ((size_t)row * a.H + h) * kd + c0l;
#pragma unroll
  for (int u = 0; u < CPT / 8; ++u) {
    in.q[u] = reinterpret_cast<const uint4*>(a.q + base)[u];
    in.k[u] = reinterpret_cast<const uint4*>(a.k + base)[u];
    in.g[u] = reinterpret_cast<const uint4*>(a.g + base)[u];
  }
  // with the gate given, A_log and dt_bias may be absent and are not read
  const bool gate_given = a.flags & FLAG_GATE_GIVEN;
#pragma unroll
  for (int c = 0; c < CPT; ++c) in.db[c] = gate_given ? 0.f : a.dt_bias[(size_t)h * kd + c0l + c];
  in.A_log = gate_given ? 0.f : a.A_log[h];
  in.beta = a.beta[(size_t)row * a.H + h];
}

// Per-token preparation of one chunk into LDS from its loaded inputs: q^, k^
// (rows past the end are zero), G = cumulative log2-decay (constant past the
// end), beta, the row norms of q and k.  sTmp needs NTH floats.  FULL: K ==
// 128, where no channel is masked.
template <int NTH, bool FULL>
__device__ void prep_chunk(const BwdArgs& a, const PrepIn<NTH>& in, int L, float* sQn, float* sKn, float* sG,
                           float* sBeta, float* sRq, float* sRk, float* sTmp) {
  constexpr int TPR = NTH / CH;  // threads per token
  constexpr int CPT = KD / TPR;  // channels per thread
  const int t = threadIdx.x;
  const int i = t / TPR;
  const int part = t % TPR;
  const bool ok = i < L;
  const int kd = FULL ? KD : a.kd;
  const bool cok = FULL || CPT * part < kd;  // channels past the head dim read as zero
  float qv[CPT], kv[CPT], gv[CPT];
#pragma unroll
  for (int u = 0; u < CPT / 8; ++u) {
    float tq[8], tk[8], tg[8];
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    unpack_bf16x8(cok ? in.q[u] : z, tq);
    unpack_bf16x8(cok ? in.k[u] : z, tk);
    unpack_bf16x8(cok ? in.g[u] : z, tg);
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
  static_assert(TPR == 8, "one token per 8 lanes");
  sq = sum8(sq);
  sk = sum8(sk);
  const bool norm = !(a.flags & FLAG_NO_QK_NORM);
  const bool gate_given = a.flags & FLAG_GATE_GIVEN;
  const float rq = norm ? sqrtf(sq + L2_EPS) : 1.0f, rk = norm ? sqrtf(sk + L2_EPS) : 1.0f;
  const float iq = ok ? 1.0f / rq : 0.f, ik = ok ? 1.0f / rk : 0.f;
  const float al = gate_given ? 0.f : expf(in.A_log);
#pragma unroll
  for (int c = 0; c < CPT; c += 4) {
    float gg[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float gn;
      if (gate_given)
        gn = fminf(fmaxf(gv[c + e], a.lb), 0.f);
      else
        gn = a.lb * fsigmoid(al * (gv[c + e] + (cok ? in.db[c + e] : 0.f)));
      gg[e] = ok ? gn * LOG2E : 0.f;
    }
    *reinterpret_cast<float4*>(sQn + i * QP + CPT * part + c) =
        make_float4(qv[c] * iq, qv[c + 1] * iq, qv[c + 2] * iq, qv[c + 3] * iq);
    *reinterpret_cast<float4*>(sKn + i * QP + CPT * part + c) =
        make_float4(kv[c] * ik, kv[c + 1] * ik, kv[c + 2] * ik, kv[c + 3] * ik);
    *reinterpret_cast<float4*>(sG + i * QP + CPT * part + c) = make_float4(gg[0], gg[1], gg[2], gg[3]);
  }
  if (part == 0) {
    const float rb = bf2f(in.beta);
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
// (or channel tiles) of parity p.  Persistent: workgroup b takes items b,
// b + grid, ... and loads each next item's inputs while it works on the
// current one (its LDS allows one workgroup per CU).
// ---------------------------------------------------------------------------
constexpr int NTP = 512;
constexpr int PREP_FLOATS = 3 * CH * QP + 2 * CH * MP + 3 * CH + NTP;
constexpr int PREP_WGS = 256;  // one per CU

template <bool FULL>
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
  const int64_t n_items = total_chunks(a.map) * H;
  auto geometry = [&](int64_t item, int64_t& c0, int& L, int& h) {
    const int64_t gch = item / H;
    h = (int)(item - gch * H);
    chunk_of(a.map, gch, c0, L);
  };
  KDA_TIMER_DECL
  KDA_TIMER_MARK(0);
  PrepIn<NTP> in;
  int64_t item = blockIdx.x;
  int L = 0;  // the current item's token count
  if (item < n_items) {
    int64_t c0;
    int h;
    geometry(item, c0, L, h);
    prep_load<NTP, FULL>(a, c0, L, h, in);
  }
  // Wait for the first item's loads here.  The loop's own wait for its
  // inputs then only has to cover the loads issued in the previous iteration,
  // not the record stores issued after them (a vmcnt wait is in order).
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  for (; item < n_items; item += gridDim.x) {
    float* br = a.br + (size_t)item * BWD_REC_FLOATS;

    prep_chunk<NTP, FULL>(a, in, L, sQn, sKn, sG, sBeta, sRq, sRk, sTmp);
    KDA_TIMER_MARK(1);
    // the next item's inputs, while this one is worked on
    int Ln = 0;
    if (item + gridDim.x < n_items) {
      int64_t c0n;
      int hn;
      geometry(item + gridDim.x, c0n, Ln, hn);
      prep_load<NTP, FULL>(a, c0n, Ln, hn, in);
    }
    KDA_TIMER_MARK(2);

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
        for (int ii = 0; ii < 4; ++ii) sKK[(16 * w + 4 * gq + ii) * MP + 16 * b + tl] = 0.f;
        // A_qk^T tile (rows block b, contraction block w) is above the diagonal: zero
        store_hl4(br + BR_AQKT, CH * CH, frag_tt(16 * b + tl, 16 * w + 4 * gq), 0.f, 0.f, 0.f, 0.f);
        continue;
      }
      const int r = (b < w) ? 16 * b + 15 : 16 * w;
      f32x4 ak = zero4(), aq = zero4();
      // 16x16x16 hi/lo MFMAs, contraction over channels 16t + 4gq + 0..3
  #pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int c = 16 * t + 4 * gq;
        const float4 kx = ld4(sKn + (16 * w + tl) * QP + c), qx = ld4(sQn + (16 * w + tl) * QP + c);
        const float4 gx = ld4(sG + (16 * w + tl) * QP + c);
        const float4 ky = ld4(sKn + (16 * b + tl) * QP + c), gy = ld4(sG + (16 * b + tl) * QP + c);
        const float4 gr = ld4(sG + r * QP + c);
        float fx[4], yb[4];
  #pragma unroll
        for (int s = 0; s < 4; ++s) {
          fx[s] = fexp2(el(gx, s) - el(gr, s));
          yb[s] = el(ky, s) * fexp2(el(gr, s) - el(gy, s));
        }
        const HL4 y = hl4(yb[0], yb[1], yb[2], yb[3]);
        ak = mfma_hl(hl4(kx.x * fx[0], kx.y * fx[1], kx.z * fx[2], kx.w * fx[3]), y, ak);
        aq = mfma_hl(hl4(qx.x * fx[0], qx.y * fx[1], qx.z * fx[2], qx.w * fx[3]), y, aq);
      }
      float qk4[4];
  #pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * w + 4 * gq + ii, j = 16 * b + tl;
        const float kk = (b < w || j < i) ? ak[ii] : 0.f;
        qk4[ii] = (b < w || j <= i) ? aq[ii] : 0.f;
        sKK[i * MP + j] = kk;
      }
      // scale A_qk^T[j][i]: rows j = 16b + tl, contraction i = 16w + 4gq + ii
      store_hl4(br + BR_AQKT, CH * CH, frag_tt(16 * b + tl, 16 * w + 4 * gq), a.scale * qk4[0], a.scale * qk4[1],
                a.scale * qk4[2], a.scale * qk4[3]);
    }
    __syncthreads();
    KDA_TIMER_MARK(3);

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
    for (int u = 0; u < 2; ++u) {  // T and KK (zero on and above the diagonal) to the record, 16 bytes a lane
      const int e = 4 * (tid + NTP * u);
      *reinterpret_cast<float4*>(br + BR_T + e) = ld4(sT + (e >> 6) * MP + (e & 63));
      *reinterpret_cast<float4*>(br + BR_KK + e) = ld4(sKK + (e >> 6) * MP + (e & 63));
    }
    KDA_TIMER_MARK(4);

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
          const int c = 16 * n + tl;
          const float* kp = sKn + (16 * jb + 4 * gq) * QP + c;
          const float* gp = sG + (16 * jb + 4 * gq) * QP + c;
          acc = mfma_hl(hl4(tb[jb][0], tb[jb][1], tb[jb][2], tb[jb][3]),
                        hl4(kp[0] * fexp2(gp[0]), kp[QP] * fexp2(gp[QP]), kp[2 * QP] * fexp2(gp[2 * QP]),
                            kp[3 * QP] * fexp2(gp[3 * QP])),
                        acc);
        }
        // -W^T[k][i]: rows k = 16n + tl, contraction i = 16w + 4gq + ii
        store_hl4(br + BR_WT, CH * KD, frag_ct(16 * n + tl, 16 * w + 4 * gq), -acc[0], -acc[1], -acc[2], -acc[3]);
      }
    }
    KDA_TIMER_MARK(5);

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
    KDA_TIMER_MARK(6);
    __syncthreads();  // the next item's preparation rewrites the LDS tiles
    L = Ln;
  }
  KDA_TIMER_STORE(a.timers);
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
    const int kd = a.kd, vd = a.vd;
    const float* src = a.dfin ? a.dfin + ((size_t)seq * H + h) * kd * vd : nullptr;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int k = 32 * w + 16 * mt + 4 * gq + ii, v = vs + 16 * nn + tl;
          dS[mt][nn][ii] = src && k < kd && v < vd ? src[svk ? v * kd + k : k * vd + v] : 0.f;
        }
  }
  auto dorow_of = [&](int ci, bool& ok) {
    const int64_t c0 = bos + (int64_t)ci * CH;
    ok = c0 + orow < eos && vs + ocol < a.vd;  // columns past the head dim read as zero
    return a.dout + ((size_t)(c0 + (ok ? orow : 0)) * H + h) * a.vd + (ok ? vs + ocol : 0);
  };

  KDA_TIMER_DECL
  KDA_TIMER_MARK(0);
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
    KDA_TIMER_MARK(1);

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
    KDA_TIMER_MARK(2);
    __syncthreads();
    KDA_TIMER_MARK(3);

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
    KDA_TIMER_MARK(4);
    __syncthreads();
    KDA_TIMER_MARK(5);

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
    KDA_TIMER_MARK(6);
    __syncthreads();
    KDA_TIMER_MARK(7);
    cur = nxt;
    KDA_TIMER_MARK(8);
  }
  KDA_TIMER_STORE(a.timers);

  if (a.dinit) {
    const int kd = a.kd, vd = a.vd;
    float* dst = a.dinit + ((size_t)seq * H + h) * kd * vd;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int k = 32 * w + 16 * mt + 4 * gq + ii, v = vs + 16 * nn + tl;
          if (k < kd && v < vd) dst[svk ? v * kd + k : k * vd + v] = dS[mt][nn][ii];
        }
  }
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
  const float* src = a.part + (size_t)h * (KD + 1) + col;
  const size_t stride = (size_t)4 * H * (KD + 1);  // four chunks on
  float acc = 0.f;
  int64_t g = rr;
  // eight loads in flight, then added in chunk order (the sum's order is fixed)
  constexpr int U = 8;
  for (; g + 4 * (U - 1) < nch; g += 4 * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[(size_t)g * H * (KD + 1) + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc += v[u];
  }
  for (; g < nch; g += 4) acc += src[(size_t)g * H * (KD + 1)];
  red[t] = acc;
  __syncthreads();
  if (rr == 0) {
    const float v = red[col] + red[(KD + 1) + col] + red[2 * (KD + 1) + col] + red[3 * (KD + 1) + col];
    if (col < KD) {
      if (a.ddt && col < a.kd) a.ddt[(size_t)h * a.kd + col] = v;
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
    e = hipLaunchKernel(a.kd == KD ? reinterpret_cast<const void*>(&kda_bwd_prep_kernel<true>)
                                    : reinterpret_cast<const void*>(&kda_bwd_prep_kernel<false>),
                        dim3((unsigned)(items < PREP_WGS ? items : PREP_WGS)), dim3(NTP), kargs, 0, st);
    if (e != hipSuccess) return e;
  }
  if (!sh) {
    BwdArgs ad = a;
    if (ad.timers) ad.timers += (size_t)2 * 16 * items;  // timer builds: after the prep and grad counters
    e = launch_dhu(ad, st);
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
    e = launch_grad(a, items, st);
    if (e != hipSuccess) return e;
  }
  return hipLaunchKernel(reinterpret_cast<const void*>(&kda_bwd_reduce_kernel), dim3((unsigned)a.H), dim3(NTR),
                         kargs, 0, st);
}

}  // namespace kda

namespace kda {
namespace {

// The backward pass keeps, besides the forward's areas: the state entering
// and the state gradient leaving every chunk, every chunk's D and dD, its fp32
// factor record and its partial parameter-gradient sums.  The factor record is
// written after the checkpointing pass has read the forward's chunk records
// for the last time, so it starts where they start, unless the call splits
// its sequences (the shard maps after the records are read after it).
struct BwdLayout {
  Layout fwd;
  size_t states, dtile, dstates, ddtile, br, part, total;
};

BwdLayout bwd_layout(int64_t T_total, int64_t H, int64_t N) {
  BwdLayout l;
  l.fwd = workspace_layout(T_total, H, N);
  const size_t items = ((size_t)(T_total / CH) + (size_t)N) * (size_t)H;
  const size_t brb = align256(items * BWD_REC_FLOATS * 4);
  l.br = l.fwd.S > 1 ? align256(l.fwd.total) : l.fwd.rec;
  const size_t after = l.br + brb > l.fwd.total ? l.br + brb : l.fwd.total;
  l.states = align256(after);
  l.dtile = l.states + align256(items * KD * VD * 4);
  l.dstates = l.dtile + align256(items * CH * VD * 4);
  l.ddtile = l.dstates + align256(items * KD * VD * 4);
  l.part = l.ddtile + align256(items * CH * VD * 4);
  l.total = l.part + align256(items * (KD + 1) * 4);
  return l;
}

}  // namespace
}  // namespace kda

using namespace kda;

extern "C" {

size_t kda_bwd_workspace_size(int64_t T_total, int64_t H, int64_t N) {
  if (T_total < 0 || H < 1 || N < 1) return 0;
  // the largest layout of any call with N' <= N sequences: only N' with
  // N' H <= kSplitChains / kMinShards can split (which moves the later areas
  // up by a shard area), and above those the layout grows with N'
  size_t best = bwd_layout(T_total, H, N).total;
  const int64_t top = N < kSplitChains / kMinShards ? N : kSplitChains / kMinShards;
  for (int64_t n = 1; n <= top; ++n) {
    const size_t t = bwd_layout(T_total, H, n).total;
    if (t > best) best = t;
  }
  return best;
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
  if ((K != 64 && K != KD) || (V != 64 && V != VD)) return KDA_ERR_UNSUPPORTED;  // head dims 64 or 128
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
  ba.kd = (int)K;
  ba.vd = (int)V;
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
