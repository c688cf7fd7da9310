// Token gradients of the gfx950 KDA backward (launched by kda_bwd.hip after
// the reverse recurrence): one workgroup per (chunk, head).

#include "kda_bwd_dev.h"

namespace kda {
namespace {

// ---------------------------------------------------------------------------
// kda_bwd_grad_kernel: per (chunk, head), 8 waves, two per SIMD.
// Token-by-channel quantities are split by channel: wave wv owns the tile of
// channels 16wv..16wv+15 for all 64 tokens and keeps k^, G and dG of its
// tile in registers in MFMA C layout (lane (gq, tl) holds tokens
// 16b + 4gq + ii, b = 0..3, of channel 16wv + tl); q^ is read from the raw
// rows in LDS where it is used, and dq^, dk^ wait in LDS during the 64 x 64
// work.
//  - Its 16 rows of S0 and dS' (all 128 columns) are read once, split into
//    bf16 hi/lo, and serve every product that contracts over v:
//    dQG = scale dO S0^T, dKG = -dv S0^T, dKt = D dS'^T and Y^T = S0 dD^T
//    (rows: its channels).  The S0 . dS' row dots come from the same loads.
//  - The token-side operands of those products (D and dD as bf16 hi/lo, dO,
//    dv) are staged in LDS as A-operand fragments, one 1 KB fragment per
//    (16-token block, 32-column step), half a chunk at a time.
//  - dTb = dD Z^T with Z = V - KG S0 is formed as dD V^T - Y KG^T; the second
//    term contracts over channels, so every wave adds its part, in a fixed
//    order (the sums do not depend on timing).
//  - dv = Tb^T dD is computed by column slices (wave wv: columns 16wv..) and
//    stored as fragments; their hi half is the bf16 output.
//  - The 64 x 64 work (dA_qk, dT, X, dA_kk and their beta terms) is shared
//    out by 16 x 16 blocks.  The pairwise products contract over tokens, so
//    each tile runs them alone, with its B operands from registers.
// Products whose operands are fp32 use bf16 hi/lo splits (three MFMA passes,
// about 16 significant bits per operand) except the T chain (X, dA_kk),
// which stays on fp32 MFMA.
// ---------------------------------------------------------------------------
constexpr int NTG = 512;
constexpr int SP = KD + 8;   // pitch (halves) of the bf16 [64][128] rows
constexpr int XP = 16 + 1;   // pitch (floats) of the per-wave KG rows [64][16]
constexpr int GR_T = 0;                     // f32 [64][MP] T
constexpr int GR_M1 = GR_T + CH * MP * 4;   // f32 [64][MP] dA_qk
constexpr int GR_M2 = GR_M1 + CH * MP * 4;  // f32 [64][MP] dTb -> dT -> X -> dA_kk beta
constexpr int GR_G = GR_M2 + CH * MP * 4;   // bf16 [64][SP] raw gate
constexpr int GR_Q = GR_G + CH * SP * 2;    // bf16 [64][SP] raw q
constexpr int GR_X = GR_Q + CH * SP * 2;    // region X, one use per phase:
//   raw k rows ([64][SP] bf16)
//   -> dv hi/lo fragments + half a chunk of D hi/lo, dD hi/lo and dO fragments
//   -> per-wave KG rows (8 x [64][XP] f32)
//   -> dq^ and dk^ of every lane (fp32, 16 bytes per lane and token block), the
//      row dots [8][64][2] and their totals [64][2]
constexpr int GX_DV = 0;                    // dv hi, lo: 16 fragments each
constexpr int GX_D = GX_DV + 2 * 16 * FRAG; // D hi, lo: 8 fragments each (2 token blocks x 4 column steps)
constexpr int GX_E = GX_D + 2 * 8 * FRAG;   // dD hi, lo
constexpr int GX_O = GX_E + 2 * 8 * FRAG;   // dO
constexpr int GR_X_BYTES = GX_O + 8 * FRAG;
constexpr int GX_DQ = 0;                    // dq^: [wave][block][lane] x 4 floats
constexpr int GX_DK = GX_DQ + CH * KD * 4;  // dk^, same layout
constexpr int GX_DOT = GX_DK + CH * KD * 4;
constexpr int GR_S = GR_X + GR_X_BYTES;     // beta, 1/|q|, 1/|k| [64] each, dbeta parts [4][64], [8] dA_log parts
constexpr int GR_S_FLOATS = 7 * CH + 8;
constexpr int GRAD_LDS = GR_S + GR_S_FLOATS * 4;
static_assert(FRAG == 1024, "1 KB fragments");
static_assert(CH * SP * 2 <= GR_X_BYTES && 8 * CH * XP * 4 <= GR_X_BYTES && 4 * 10 * FRAG <= GR_X_BYTES &&
              GX_DOT + (8 * CH * 2 + CH * 2) * 4 <= GR_X_BYTES, "region X");
static_assert(GRAD_LDS <= 163840, "LDS");

// A-operand fragment f (rows 16 blk + lane % 16, columns 32 ks + 8 (lane / 16) .. + 7)
// of an array whose lane-based address is xl (= array + 16 lane)
__device__ __forceinline__ bf16x8 lds_frag(const char* xl, int f) {
  return *reinterpret_cast<const bf16x8*>(xl + f * FRAG);
}

// Staging of half a chunk (token blocks 2 half, 2 half + 1) of D and dD (fp32,
// split into bf16 hi/lo) and dO (bf16) as A-operand fragments.  Thread tid
// takes fragment f = tid / 64 (token block f / 4, column step f % 4), lane
// l = tid % 64.
struct TokStage {
  float4 d[2], e[2];
  uint4 o;
};
__device__ __forceinline__ void tok_load(TokStage& s, const BwdArgs& a, const float* Dt, const float* dDt,
                                         int64_t c0, int L, int h, int half, int tid, int vd) {
  const int f = tid >> 6, l = tid & 63;
  const int r = 32 * half + 16 * (f >> 2) + (l & 15), col = 32 * (f & 3) + 8 * (l >> 4);
  const bool cok = col < vd;  // columns past the head dim: zero (the checkpoints leave them unwritten)
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  s.d[0] = cok ? ld4(Dt + r * VD + col) : z;
  s.d[1] = cok ? ld4(Dt + r * VD + col + 4) : z;
  s.e[0] = cok ? ld4(dDt + r * VD + col) : z;
  s.e[1] = cok ? ld4(dDt + r * VD + col + 4) : z;
  s.o = r < L && cok ? *reinterpret_cast<const uint4*>(a.dout + ((size_t)(c0 + r) * a.H + h) * vd + col)
                     : make_uint4(0u, 0u, 0u, 0u);
}
__device__ __forceinline__ void tok_store(const TokStage& s, char* sX, int tid) {
  const int f = tid >> 6, l = tid & 63;
  const float xd[8] = {s.d[0].x, s.d[0].y, s.d[0].z, s.d[0].w, s.d[1].x, s.d[1].y, s.d[1].z, s.d[1].w};
  const float xe[8] = {s.e[0].x, s.e[0].y, s.e[0].z, s.e[0].w, s.e[1].x, s.e[1].y, s.e[1].z, s.e[1].w};
  bf16x8 hh, ll;
  split_hl8(xd, hh, ll);
  *reinterpret_cast<bf16x8*>(sX + GX_D + f * FRAG + l * 16) = hh;
  *reinterpret_cast<bf16x8*>(sX + GX_D + (8 + f) * FRAG + l * 16) = ll;
  split_hl8(xe, hh, ll);
  *reinterpret_cast<bf16x8*>(sX + GX_E + f * FRAG + l * 16) = hh;
  *reinterpret_cast<bf16x8*>(sX + GX_E + (8 + f) * FRAG + l * 16) = ll;
  *reinterpret_cast<uint4*>(sX + GX_O + f * FRAG + l * 16) = s.o;
}

// FULL: K == V == 128, where none of the head-dim masks below can be false
template <bool FULL>
__global__ void __launch_bounds__(NTG, 1) kda_bwd_grad_kernel(BwdArgs a) {
  const int kd = FULL ? KD : a.kd, vd = FULL ? VD : a.vd;  // the caller's head dims
  __shared__ __attribute__((aligned(16))) char smem[GRAD_LDS];
  float* sT = reinterpret_cast<float*>(smem + GR_T);
  float* sM1 = reinterpret_cast<float*>(smem + GR_M1);  // dA_qk
  float* sM2 = reinterpret_cast<float*>(smem + GR_M2);
  uint16_t* sGr = reinterpret_cast<uint16_t*>(smem + GR_G);
  uint16_t* sQr = reinterpret_cast<uint16_t*>(smem + GR_Q);
  char* sX = smem + GR_X;
  float* sBeta = reinterpret_cast<float*>(smem + GR_S);
  float* sIq = sBeta + CH;            // 1 / |q|, 1 / |k| (1 without the L2 norm)
  float* sIk = sIq + CH;
  float* sdBp = sIk + CH;             // [4][64] parts of the gradient of beta, one writer each
  float* sRed = sdBp + 4 * CH;        // [8] per-wave dA_log parts
  float* sDot = reinterpret_cast<float*>(sX + GX_DOT);  // [8][64][2] per-wave row dots q^.dq^, k^.dk^
  float* sDotT = sDot + 8 * CH * 2;   // [64][2] their totals

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
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int tl = lane & 15;
  const int gq = lane >> 4;
  const int cw = 16 * wv;  // this wave's channel tile, and its column slice of dv
  const int c = cw + tl;   // this lane's channel in C-layout tiles
  const bool gate_given = a.flags & FLAG_GATE_GIVEN;
  const bool norm = !(a.flags & FLAG_NO_QK_NORM);
  // lane bases: every index below is one of these plus a compile-time constant
  // (or a wave-uniform term); "q" bases sit at row 4gq, column tl of a
  // [64][pitch] array, "r" bases at row tl, column 4gq
  const float* sTq = sT + 4 * gq * MP + tl;
  const float* sTr = sT + tl * MP + 4 * gq;
  float* sM1q = sM1 + 4 * gq * MP + tl;
  float* sM1r = sM1 + tl * MP + 4 * gq;
  float* sM2q = sM2 + 4 * gq * MP + tl;
  float* sM2r = sM2 + tl * MP + 4 * gq;
  const char* xl = sX + 16 * lane;

  // ---- loads issued first: this lane's pieces of row c of S0 and dS'
  // (columns 32ks + 8gq + 0..7), its dD column pieces for dv, T, and the raw
  // q, k, gate rows (thread -> token tid / 8, channels 16 (tid % 8) .. + 15)
  float4 s0r[4][2], dsr[4][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bool vok = 8 * gq + 32 * ks < vd;  // columns past the head dim: zero
      s0r[ks][hf] = vok ? ld4(S0 + c * VD + 8 * gq + 32 * ks + 4 * hf) : make_float4(0.f, 0.f, 0.f, 0.f);
      dsr[ks][hf] = vok ? ld4(dSn + c * VD + 8 * gq + 32 * ks + 4 * hf) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  float ddv[4][4];  // dD[16ib + 4gq + s][c]
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int s = 0; s < 4; ++s) ddv[ib][s] = c < vd ? (dDt + 4 * gq * VD + c)[(16 * ib + s) * VD] : 0.f;
  float4 tcp[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) tcp[u] = ld4(br + BR_T + 4 * (tid + NTG * u));
  const int sr = tid >> 3, sc = 16 * (tid & 7);
  const bool sok = sr < L;
  uint4 rq[2], rk[2], rg[2];
  if (sok && sc < kd) {  // channels past the head dim: zero
    const size_t o = ((size_t)(c0 + sr) * H + h) * kd + sc;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      rq[u] = reinterpret_cast<const uint4*>(a.q + o)[u];
      rk[u] = reinterpret_cast<const uint4*>(a.k + o)[u];
      rg[u] = reinterpret_cast<const uint4*>(a.g + o)[u];
    }
  } else {
#pragma unroll
    for (int u = 0; u < 2; ++u) rq[u] = rk[u] = rg[u] = make_uint4(0u, 0u, 0u, 0u);
  }
  {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float x[8], y[8];
      unpack_bf16x8(rq[u], x);
      unpack_bf16x8(rk[u], y);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq += x[e] * x[e];
        sk += y[e] * y[e];
      }
    }
    sq = sum8(sq);
    sk = sum8(sk);
    if ((tid & 7) == 0) {
      sIq[sr] = norm ? 1.0f / sqrtf(sq + L2_EPS) : 1.0f;
      sIk[sr] = norm ? 1.0f / sqrtf(sk + L2_EPS) : 1.0f;
      const float rb = sok ? bf2f(a.beta[(size_t)(c0 + sr) * H + h]) : 0.f;
      sBeta[sr] = sok ? ((a.flags & FLAG_BETA_GIVEN) ? rb : sigmoidf(rb)) : 0.f;
    }
    uint16_t* sKr = reinterpret_cast<uint16_t*>(sX);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<uint4*>(sQr + sr * SP + sc + 8 * u) = rq[u];
      *reinterpret_cast<uint4*>(sKr + sr * SP + sc + 8 * u) = rk[u];
      *reinterpret_cast<uint4*>(sGr + sr * SP + sc + 8 * u) = rg[u];
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = 4 * (tid + NTG * u);
    *reinterpret_cast<float4*>(sT + (e >> 6) * MP + (e & 63)) = tcp[u];
  }
  for (int e = tid; e < CH * MP; e += NTG) {
    sM1[e] = 0.f;
    sM2[e] = 0.f;
  }
  __syncthreads();
  KDA_TIMER_MARK(1);

  // ---- k^ and G = cumulative log2-decay (constant past the chunk's end) of
  // the tile, a scan over ii in the lane, over gq across lanes, over b; q^
  // is read from the raw rows where it is used
  const float al = gate_given ? 0.f : expf(a.A_log[h]);
  const float dtb = gate_given || c >= kd ? 0.f : a.dt_bias[(size_t)h * kd + c];
  f32x4 Kn[4], G[4];
  auto prep = [&](auto given) {
    // lane bases: token 4gq (+ 16b + ii as immediate offsets), channel c
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(sX) + 4 * gq * SP + c;
    const uint16_t* gb = sGr + 4 * gq * SP + c;
    const float* ikb = sIk + 4 * gq;
    float run = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float x[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int jj = 16 * b + ii;  // token 4gq + jj
        Kn[b][ii] = bf2f(kb[jj * SP]) * ikb[jj];
        const float gv = bf2f(gb[jj * SP]);
        const float gn = decltype(given)::value ? fminf(fmaxf(gv, a.lb), 0.f) : a.lb * fsigmoid(al * (gv + dtb));
        x[ii] = 4 * gq + jj < L ? gn * LOG2E : 0.f;
      }
      x[1] += x[0];
      x[2] += x[1];
      x[3] += x[2];
      const float s = x[3];
      const float s0 = __shfl(s, tl), s1 = __shfl(s, tl + 16), s2 = __shfl(s, tl + 32), s3 = __shfl(s, tl + 48);
      const float off = run + (gq > 0 ? s0 : 0.f) + (gq > 1 ? s1 : 0.f) + (gq > 2 ? s2 : 0.f);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) G[b][ii] = x[ii] + off;
      run += (s0 + s1) + (s2 + s3);
    }
  };
  if (gate_given)
    prep(std::true_type{});
  else
    prep(std::false_type{});
  // q^ of token 4gq + jj (jj = 16b + ii), channel c
  const uint16_t* qlb = sQr + 4 * gq * SP + c;
  const float* iqlb = sIq + 4 * gq;
  auto qn = [&](int jj) { return bf2f(qlb[jj * SP]) * iqlb[jj]; };
  // G of the chunk's last token; S0 . dS' over row c; both rows as bf16 hi/lo
  const float GL = __shfl(G[3][3], tl + 48);
  float gl2 = 0.f;
  bf16x8 s0h[4], s0l[4], dsh[4], dsl[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const float xs[8] = {s0r[ks][0].x, s0r[ks][0].y, s0r[ks][0].z, s0r[ks][0].w,
                         s0r[ks][1].x, s0r[ks][1].y, s0r[ks][1].z, s0r[ks][1].w};
    const float xd[8] = {dsr[ks][0].x, dsr[ks][0].y, dsr[ks][0].z, dsr[ks][0].w,
                         dsr[ks][1].x, dsr[ks][1].y, dsr[ks][1].z, dsr[ks][1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) gl2 += xs[e] * xd[e];
    split_hl8(xs, s0h[ks], s0l[ks]);
    split_hl8(xd, dsh[ks], dsl[ks]);
  }
  gl2 += __shfl_xor(gl2, 16);
  gl2 += __shfl_xor(gl2, 32);
  TokStage stg;
  tok_load(stg, a, Dt, dDt, c0, L, h, 0, tid, vd);
  __syncthreads();  // the raw k rows are read: region X takes dv and the staged halves
  KDA_TIMER_MARK(2);

  // ---- dv^T, columns c (this wave's slice cw..cw+15): dv^T[v][j] =
  // sum_{i >= j} dD[i][v] Tb[i][j] (16x16x16 hi/lo MFMA), stored as bf16 hi/lo
  // fragments: element (j, v) is in fragment 4 (j / 16) + v / 32, lane
  // 16 ((v % 32) / 8) + j % 16, element v % 8
  {
    __bf16* dvh = reinterpret_cast<__bf16*>(sX + GX_DV);
    __bf16* dvl = dvh + CH * VD;
    HL4 dda[4];  // A operands: dD[16ib + 4gq + 0..3][c]
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) dda[ib] = hl4(ddv[ib][0], ddv[ib][1], ddv[ib][2], ddv[ib][3]);
    const int lo = ((wv >> 1) * 64 + 16 * (2 * (wv & 1) + (gq >> 1)) + tl) * 8 + 4 * (gq & 1);  // lane part
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const float bj = (sBeta + tl)[16 * jb];
      f32x4 acc = zero4();
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        if (ib < jb) continue;
        const float* tq = sTq + 16 * ib * MP + 16 * jb;
        acc = mfma_hl(dda[ib], hl4(tq[0] * bj, tq[MP] * bj, tq[2 * MP] * bj, tq[3 * MP] * bj), acc);
      }
      // acc[ii] = dv[16jb + tl][cw + 4gq + ii]
      bf16x4 hv, lv;
      split_hl4(acc, hv, lv);
      *reinterpret_cast<bf16x4*>(dvh + lo + jb * 4 * 512) = hv;
      *reinterpret_cast<bf16x4*>(dvl + lo + jb * 4 * 512) = lv;
    }
  }
  tok_store(stg, sX, tid);
  __syncthreads();
  // the bf16 output dv is the hi half: 16-byte stores, thread -> (fragment, lane)
  {
    const char* dvh = sX + GX_DV;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + NTG * u;  // 0 .. 1023
      const int f = e >> 6, ln = e & 63;
      const int j = 16 * (f >> 2) + (ln & 15), col = 32 * (f & 3) + 8 * (ln >> 4);
      if (j < L && col < vd)
        *reinterpret_cast<uint4*>(a.dv + ((size_t)(c0 + j) * H + h) * vd + col) =
            *reinterpret_cast<const uint4*>(dvh + 16 * e);
    }
  }
  KDA_TIMER_MARK(3);

  // ---- per half chunk: for token blocks b, dKt = D dS'^T, dQG = scale dO S0^T,
  // dKG = -dv S0^T and Y^T = S0 dD^T, with their elementwise contributions to
  // dq^, dk^, dG; then the 64 x 64 blocks (ab, bb <= ab) whose row block ab is
  // staged: dA_qk = scale dO D^T (masked to j <= i) and the dD V^T part of dTb,
  // one block per wave
  f32x4 dqh[4], dkh[4], dGa[4], Yt[4];
  float glsum = 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (half == 1) {
      tok_load(stg, a, Dt, dDt, c0, L, h, 1, tid, vd);
      __syncthreads();  // the first half's fragments are read
      tok_store(stg, sX, tid);
      __syncthreads();
    }
#pragma unroll
    for (int bl = 0; bl < 2; ++bl) {
      const int b = 2 * half + bl;
      f32x4 aT = zero4(), aQ = zero4(), aK = zero4(), aY = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int f = 4 * bl + ks;
        const bf16x8 dh = lds_frag(xl + GX_D, f), dl = lds_frag(xl + GX_D, 8 + f);
        const bf16x8 eh = lds_frag(xl + GX_E, f), el8 = lds_frag(xl + GX_E, 8 + f);
        const bf16x8 doa = lds_frag(xl + GX_O, f);
        const bf16x8 vh = lds_frag(xl + GX_DV, 4 * b + ks), vl = lds_frag(xl + GX_DV, 16 + 4 * b + ks);
        aT = mfma_bf16(dh, dsh[ks], aT);
        aT = mfma_bf16(dh, dsl[ks], aT);
        aT = mfma_bf16(dl, dsh[ks], aT);
        aQ = mfma_bf16(doa, s0h[ks], aQ);
        aQ = mfma_bf16(doa, s0l[ks], aQ);
        aK = mfma_bf16(vh, s0h[ks], aK);
        aK = mfma_bf16(vh, s0l[ks], aK);
        aK = mfma_bf16(vl, s0h[ks], aK);
        aY = mfma_bf16(s0h[ks], eh, aY);
        aY = mfma_bf16(s0h[ks], el8, aY);
        aY = mfma_bf16(s0l[ks], eh, aY);
      }
      Yt[b] = aY;  // Y^T[cw + 4gq + ii][16b + tl]
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float g2 = G[b][ii];
        const float gam = fexp2(g2), el2 = fexp2(GL - g2);
        const float kt = Kn[b][ii] * el2;
        const float q = aQ[ii] * a.scale * gam, kk = -aK[ii] * gam;
        dqh[b][ii] = q;
        dkh[b][ii] = kk + aT[ii] * el2;
        dGa[b][ii] = q * qn(16 * b + ii) + kk * Kn[b][ii] - aT[ii] * kt;
        glsum += aT[ii] * kt;
      }
    }
    // 64 x 64 blocks with row block in this half: (0,0) (1,0) (1,1), then
    // (2,2) (3,2) (3,3) (2,0) (2,1) (3,0) (3,1); wave wv takes block wv
    const int pi = wv;
    if (pi < (half ? 7 : 3)) {  // wave-uniform
      int ab, bb;
      if (!half) {
        ab = pi ? 1 : 0;
        bb = pi == 2 ? 1 : 0;
      } else {
        ab = (pi == 0 || pi == 3 || pi == 4) ? 2 : 3;
        bb = pi < 3 ? (pi == 2 ? 3 : 2) : ((pi - 3) & 1);
      }
      const int jr = 16 * bb + tl;
      const bool jok = jr < L;
      const size_t jo = ((size_t)(c0 + (jok ? jr : 0)) * H + h) * vd;
      const bool bstaged = (bb >> 1) == half;
      f32x4 accQ = zero4(), accV = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int fa = 4 * (ab & 1) + ks;
        const bf16x8 doa = lds_frag(xl + GX_O, fa);
        const bf16x8 eh = lds_frag(xl + GX_E, fa), el8 = lds_frag(xl + GX_E, 8 + fa);
        const bool vok = 32 * ks + 8 * gq < vd;
        const bf16x8 vb = jok && vok ? *reinterpret_cast<const bf16x8*>(a.v + jo + 32 * ks + 8 * gq) : bf16x8{};
        bf16x8 dh, dl;
        if (bstaged) {
          dh = lds_frag(xl + GX_D, 4 * (bb & 1) + ks);
          dl = lds_frag(xl + GX_D, 8 + 4 * (bb & 1) + ks);
        } else if (vok) {
          ld_hl8(Dt + jr * VD + 32 * ks + 8 * gq, dh, dl);
        } else {
          dh = dl = bf16x8{};
        }
        accQ = mfma_bf16(doa, dh, accQ);
        accQ = mfma_bf16(doa, dl, accQ);
        accV = mfma_bf16(eh, vb, accV);
        accV = mfma_bf16(el8, vb, accV);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const bool low = (ab > bb) || (tl <= 4 * gq + ii);  // j <= i
        sM1q[(16 * ab + ii) * MP + 16 * bb] = low ? accQ[ii] * a.scale : 0.f;
        sM2q[(16 * ab + ii) * MP + 16 * bb] = accV[ii];
      }
    }
  }
  __syncthreads();  // the staged fragments are read: region X takes the KG rows
  KDA_TIMER_MARK(4);

  // ---- -Y KG^T over this wave's 16 channels, into every block (ab, bb <= ab)
  // of dTb: A = Y (the Y^T tiles' C layout), B = KG turned through this
  // wave's rows in LDS; the waves subtract their parts in turn
  {
    float* xr = reinterpret_cast<float*>(sX) + wv * CH * XP;  // KG [64 tokens][16 channels]
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) (xr + 4 * gq * XP + tl)[(16 * b + ii) * XP] = Kn[b][ii] * fexp2(G[b][ii]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    HL4 kg[4], yh[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float* k4 = xr + tl * XP + 4 * gq + 16 * b * XP;  // KG[16b + tl][cw + 4gq + 0..3]
      kg[b] = hl4(k4[0], k4[1], k4[2], k4[3]);
      yh[b] = hl4(Yt[b][0], Yt[b][1], Yt[b][2], Yt[b][3]);
    }
    f32x4 P[10];
#pragma unroll
    for (int ab = 0; ab < 4; ++ab)
#pragma unroll
      for (int bb = 0; bb <= ab; ++bb) P[ab * (ab + 1) / 2 + bb] = mfma_hl(yh[ab], kg[bb], zero4());
    // a fixed-order tree over the waves (4..7 into 0..3, 2..3 into 0..1, 1
    // into 0) through LDS slots of 10 x 1 KB per sending wave, over the KG
    // rows (every wave has read its own before the first barrier below)
    f32x4* slot = reinterpret_cast<f32x4*>(sX) + lane;  // + ((sender - lv) * 10 + k) * 64
#pragma unroll
    for (int lv = 4; lv >= 1; lv >>= 1) {
      __syncthreads();
      if (wv >= lv && wv < 2 * lv) {
#pragma unroll
        for (int k = 0; k < 10; ++k) slot[((wv - lv) * 10 + k) * 64] = P[k];
      }
      __syncthreads();
      if (wv < lv) {
#pragma unroll
        for (int k = 0; k < 10; ++k) P[k] += slot[(wv * 10 + k) * 64];
      }
    }
    if (wv == 0) {
#pragma unroll
      for (int ab = 0; ab < 4; ++ab)
#pragma unroll
        for (int bb = 0; bb <= ab; ++bb)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) sM2q[(16 * ab + ii) * MP + 16 * bb] -= P[ab * (ab + 1) / 2 + bb][ii];
    }
  }
  __syncthreads();
  KDA_TIMER_MARK(5);
  // dq^ and dk^ wait in region X (each lane its own 16-byte slots) until the
  // pairwise products add to them
  f32x4* pdq = reinterpret_cast<f32x4*>(sX + GX_DQ) + wv * 4 * 64 + lane;  // + b * 64
  f32x4* pdk = reinterpret_cast<f32x4*>(sX + GX_DK) + wv * 4 * 64 + lane;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    pdq[b * 64] = dqh[b];
    pdk[b * 64] = dkh[b];
  }

  // ---- the 64 x 64 chain of dTb: row block w and parity p of the blocks.
  // Every sum that two waves add to goes to a slot of its own and the slots
  // are added in a fixed order.
  const int w = wv & 3;
  const int p = wv >> 2;
  const float bj = sBeta[16 * w + tl];
  // dT = dTb diag(beta) in place; column sums of dTb . T -> dbeta (rows split by p)
  {
    float colsum = 0.f;
#pragma unroll
    for (int ab = 0; ab < 4; ++ab) {
      if (ab < w || ((ab - w) & 1) != p) continue;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int o = (16 * ab + ii) * MP + 16 * w;
        const float v = sM2q[o];
        colsum += v * sTq[o];
        sM2q[o] = v * bj;
      }
    }
    colsum += __shfl_xor(colsum, 16);
    colsum += __shfl_xor(colsum, 32);
    if (gq == 0) sdBp[p * CH + 16 * w + tl] = colsum;
  }
  __syncthreads();
  // X = dT T^T, row block w, column blocks q <= w of parity p
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
        for (int s = 0; s < 4; ++s) X[qq] = mfma_f32(sM2r[16 * w * MP + 16 * b + s], sTr[16 * q * MP + 16 * b + s], X[qq]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int q = 2 * qq + p;
      if (q > w) continue;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sM2q[(16 * w + ii) * MP + 16 * q] = X[qq][ii];
    }
  }
  __syncthreads();
  // dA_kk[block w][m < a] = -T^T X; row sums of dA_kk . KK -> dbeta; dKK = dA_kk beta_a
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
          for (int s = 0; s < 4; ++s)
            acc = mfma_f32(-sTq[(16 * pb + s) * MP + 16 * w], sM2q[(16 * pb + s) * MP + 16 * q], acc);
        }
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const bool low = q < w || (q == w && tl < 4 * gq + ii);  // column 16q + tl < row 16w + 4gq + ii
        const float v = low ? acc[ii] : 0.f;
        rows[ii] += v * (br + BR_KK + 4 * gq * CH + tl)[(16 * w + ii) * CH + 16 * q];
        acc[ii] = v * (sBeta + 4 * gq)[16 * w + ii];
      }
      dkk[qq] = acc;
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float r = rows[ii];
      r = sum16(r);
      if (tl == 0) (sdBp + (2 + p) * CH + 4 * gq)[16 * w + ii] = r;
    }
    __syncthreads();
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int q = 2 * qq + p;
      if (q > w) continue;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sM2q[(16 * w + ii) * MP + 16 * q] = dkk[qq][ii];
    }
  }
  __syncthreads();
  KDA_TIMER_MARK(7);

  // ---- pairwise products of the tile, by blocks (ab, bb <= ab) of the
  // 64 x 64 matrices.  Each factor exp(G_i - G_j) is split at a reference
  // token r between i and j (the last token of block bb when bb < ab, else
  // the first of ab), so E1[s] = exp(G_r - G_j) of the tokens j of block bb
  // and E2[s] = exp(G_i - G_r) of the tokens i of block ab serve both roles:
  //   rows i:    dq^_i += sum_j dA_qk[i][j] k^_j E1 E2_i, dk^_i likewise with dKK
  //   columns j: dk^_j += sum_i (dA_qk[i][j] q^_i + dKK[i][j] k^_i) E2_i E1_j
  // on 16x16x16 hi/lo MFMAs, contraction over the 16 tokens of a block
  {
    float Gf[4], Gl[4];  // G of each block's first and last token
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      Gf[b] = __shfl(G[b][0], tl);
      Gl[b] = __shfl(G[b][3], tl + 48);
    }
#pragma unroll
    for (int ab = 0; ab < 4; ++ab)
#pragma unroll
      for (int bb = 0; bb <= ab; ++bb) {
        const float gr = bb < ab ? Gl[bb] : Gf[ab];
        float E1[4], E2[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          E1[s] = fexp2(gr - G[bb][s]);
          E2[s] = fexp2(G[ab][s] - gr);
        }
        const HL4 y = hl4(Kn[bb][0] * E1[0], Kn[bb][1] * E1[1], Kn[bb][2] * E1[2], Kn[bb][3] * E1[3]);
        const float4 m1 = *reinterpret_cast<const float4*>(sM1r + 16 * ab * MP + 16 * bb);
        const float4 m2 = *reinterpret_cast<const float4*>(sM2r + 16 * ab * MP + 16 * bb);
        const f32x4 a1 = mfma_hl(hl4(m1.x, m1.y, m1.z, m1.w), y, zero4());
        const f32x4 a2 = mfma_hl(hl4(m2.x, m2.y, m2.z, m2.w), y, zero4());
        const float* c1 = sM1q + 16 * ab * MP + 16 * bb;
        const float* c2 = sM2q + 16 * ab * MP + 16 * bb;
        f32x4 ac = mfma_hl(hl4(c1[0], c1[MP], c1[2 * MP], c1[3 * MP]),
                           hl4(qn(16 * ab) * E2[0], qn(16 * ab + 1) * E2[1], qn(16 * ab + 2) * E2[2],
                               qn(16 * ab + 3) * E2[3]),
                           zero4());
        ac = mfma_hl(hl4(c2[0], c2[MP], c2[2 * MP], c2[3 * MP]),
                     hl4(Kn[ab][0] * E2[0], Kn[ab][1] * E2[1], Kn[ab][2] * E2[2], Kn[ab][3] * E2[3]), ac);
        f32x4 xq = pdq[ab * 64], xk = pdk[ab * 64];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float v1 = a1[ii] * E2[ii], v2 = a2[ii] * E2[ii];
          xq[ii] += v1;
          xk[ii] += v2;
          dGa[ab][ii] += qn(16 * ab + ii) * v1 + Kn[ab][ii] * v2;
        }
        pdq[ab * 64] = xq;
        pdk[ab * 64] = xk;
        f32x4 xb = pdk[bb * 64];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float v = ac[ii] * E1[ii];
          xb[ii] += v;
          dGa[bb][ii] -= Kn[bb][ii] * v;
        }
        pdk[bb * 64] = xb;
      }
  }
  KDA_TIMER_MARK(9);

  // ---- dG_L (the S0 . dS' row dot and the dKt . Kt terms over the chunk) on
  // the last token, then the reverse cumulative sum over tokens -> dg
  {
    float gs = glsum;
    gs += __shfl_xor(gs, 16);
    gs += __shfl_xor(gs, 32);
    const float dgl = gl2 * fexp2(GL) + gs;
    float run = 0.f;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      f32x4 x = dGa[b];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        if (4 * gq == L - 1 - 16 * b - ii) x[ii] += dgl;
      x[2] += x[3];
      x[1] += x[2];
      x[0] += x[1];
      const float s = x[0];
      const float s0 = __shfl(s, tl), s1 = __shfl(s, tl + 16), s2 = __shfl(s, tl + 32), s3 = __shfl(s, tl + 48);
      const float off = run + (gq < 1 ? s1 : 0.f) + (gq < 2 ? s2 : 0.f) + (gq < 3 ? s3 : 0.f);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) x[ii] += off;
      dGa[b] = x;
      run += (s0 + s1) + (s2 + s3);
    }
  }
  // row dots q^.dq^ and k^.dk^ over the tile's 16 channels, then over the tiles
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x4 xq = pdq[b * 64], xk = pdk[b * 64];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float dq_dot = qn(16 * b + ii) * xq[ii], dk_dot = Kn[b][ii] * xk[ii];
      dq_dot = sum16(dq_dot);
      dk_dot = sum16(dk_dot);
      if (tl == 0) {
        float* d = sDot + (wv * CH + 4 * gq) * 2;
        d[(16 * b + ii) * 2] = dq_dot;
        d[(16 * b + ii) * 2 + 1] = dk_dot;
      }
    }
  }
  __syncthreads();
  if (tid < 2 * CH) {
    float x = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) x += sDot[u * 2 * CH + tid];
    sDotT[tid] = x;
  }
  __syncthreads();
  KDA_TIMER_MARK(10);

  // ---- outputs, staged as bf16 rows over T, dA_qk and dKK (no longer read):
  // d raw_gate, dq, dk; partial sums of d dt_bias (per channel) and dA_log
  float pA = 0.f, pdt = 0.f;
  float* part = a.part + it * (KD + 1);
  uint16_t* og = reinterpret_cast<uint16_t*>(sT);  // [64][128] each (16 KB of the 17 KB)
  uint16_t* oq = reinterpret_cast<uint16_t*>(sM1);
  uint16_t* ok_ = reinterpret_cast<uint16_t*>(sM2);
  {
    const uint16_t* gb = sGr + 4 * gq * SP + c;
    const float* dtq = sDotT + 8 * gq;
    const float* ikb = sIk + 4 * gq;
    uint16_t* ogb = og + 4 * gq * KD + c;
    uint16_t* oqb = oq + 4 * gq * KD + c;
    uint16_t* okb = ok_ + 4 * gq * KD + c;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f32x4 xq = pdq[b * 64], xk = pdk[b * 64];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int jj = 16 * b + ii;  // token 4gq + jj
        const float dgv = dGa[b][ii];  // gradient of the natural-log decay g_j
        float dgo = 0.f;
        if (4 * gq + jj < L) {
          const float rg = bf2f(gb[jj * SP]);
          if (gate_given) {
            // g = clamp(raw_gate, lower_bound, 0): the gradient passes inside the closed interval
            dgo = (rg >= a.lb && rg <= 0.f) ? dgv : 0.f;
          } else {
            const float x = al * (rg + dtb);
            const float sg = fsigmoid(x);
            const float dx = dgv * a.lb * sg * (1.f - sg);
            dgo = dx * al;
            pdt += dgo;
            pA += dx * x;
          }
        }
        // dq = (dq^ - q^ (q^ . dq^)) / |q|, same for k; without the L2 norm dq = dq^
        const float dqd = norm ? dtq[2 * jj] : 0.f, dkd = norm ? dtq[2 * jj + 1] : 0.f;
        ogb[jj * KD] = f2bf(dgo);
        oqb[jj * KD] = f2bf((xq[ii] - qn(jj) * dqd) * iqlb[jj]);
        okb[jj * KD] = f2bf((xk[ii] - Kn[b][ii] * dkd) * ikb[jj]);
      }
    }
  }
  pdt += __shfl_xor(pdt, 16);
  pdt += __shfl_xor(pdt, 32);
  if (gq == 0) part[c] = pdt;
  pA = sum16(pA);
  pA += __shfl_xor(pA, 16);
  pA += __shfl_xor(pA, 32);
  if (lane == 0) sRed[wv] = pA;
  if (tid < CH && tid < L) {
    const float bt = sBeta[tid];
    const float db = (sdBp[tid] + sdBp[CH + tid]) + (sdBp[2 * CH + tid] + sdBp[3 * CH + tid]);
    a.dbeta[(size_t)(c0 + tid) * H + h] = f2bf((a.flags & FLAG_BETA_GIVEN) ? db : db * bt * (1.f - bt));
  }
  __syncthreads();
  // 16-byte stores of the staged rows: thread -> (row, 16-byte column block)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + NTG * u;  // 0 .. 1023
    const int row = e >> 4;
    const int cb = 8 * (e & 15);
    if (row < L && cb < kd) {
      const size_t o = ((size_t)(c0 + row) * H + h) * kd + cb;
      *reinterpret_cast<uint4*>(a.dq + o) = *reinterpret_cast<const uint4*>(oq + row * KD + cb);
      *reinterpret_cast<uint4*>(a.dk + o) = *reinterpret_cast<const uint4*>(ok_ + row * KD + cb);
      *reinterpret_cast<uint4*>(a.dg + o) = *reinterpret_cast<const uint4*>(og + row * KD + cb);
    }
  }
  if (tid == 0) {
    float sA = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) sA += sRed[u];
    part[KD] = sA;
  }
  KDA_TIMER_MARK(11);
  KDA_TIMER_STORE(a.timers ? a.timers + (size_t)gridDim.x * 16 : nullptr);
}

}  // namespace

hipError_t launch_grad(const BwdArgs& args, int64_t items, hipStream_t st) {
  if (items <= 0) return hipSuccess;
  BwdArgs a = args;
  void* kargs[] = {(void*)&a};
  const void* fn = a.kd == KD && a.vd == VD ? reinterpret_cast<const void*>(&kda_bwd_grad_kernel<true>)
                                             : reinterpret_cast<const void*>(&kda_bwd_grad_kernel<false>);
  return hipLaunchKernel(fn, dim3((unsigned)items), dim3(NTG), kargs, 0, st);
}

}  // namespace kda
