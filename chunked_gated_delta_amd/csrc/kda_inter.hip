// Inter-chunk kernel of the gfx950 KDA forward: the sequential recurrence over
// chunks.  For every chunk, with the per-chunk record of the intra-chunk
// kernel (W, Q exp(G), (K exp(G_L - G))^T, A_qk, T diag(b), exp(G_L)):
//     U = T diag(b) V                       (bf16 hi/lo x exact bf16 V, 2 passes)
//     D = U - W S                           (fp16 W, fp16 copy of S)
//     O = scale [ (Q exp(G)) S + A_qk D ]   -> bf16 output
//     S = Diag(exp(G_L)) S + (K exp(G_L - G))^T D   (fp16 hi/lo x fp16 hi/lo, 3 passes;
//                                                   the Kt lo pass accumulates on its own)
// The state S is fp32 and stays in MFMA accumulator registers for the whole
// sequence; its fp16 copy, the chunk's V tile and D live in LDS in
// column-major form so that every B operand is one 16-byte LDS read.
//
// One workgroup (4 waves) per (sequence, head, V slice of 16 NN columns;
// NN = 4 gives the two V halves).  Wave w computes the token rows
// 16w..16w+15 of U, D and O (its A operands are 16-byte global loads from the
// record) and the state rows (channels) 32w..32w+31 of the slice.

#include "kda_common.h"

namespace kda {
namespace {

constexpr int NTHREADS = 256;
constexpr int TP = CH + 8;       // token pitch of [v][token] arrays (halves)

// A workgroup owns NN 16-column tiles of the state (VT = 16 NN columns; NN = 4
// normally, 2 or 1 when there are too few (sequence, head) chains to fill the
// GPU).  LDS carve-up: the V tile, then the state copy and D hi/lo as
// split-plane B-operand fragments (frag_read / frag_write4), then the output
// staging tile.
template <int NN>
struct Cfg {
  static constexpr int VT = 16 * NN;                     // state columns per workgroup
  static constexpr int NV = VD / VT;                     // V slices per (sequence, head) at V = 128
  static constexpr int OFF_VT = 0;                       // bf16 [VT][TP]   V^T
  static constexpr int OFF_ST = OFF_VT + VT * TP * 2;    // f16  4 NN fragments (nn, kb)   state copy
  static constexpr int OFF_DTH = OFF_ST + 4 * NN * FRAG; // f16  2 NN fragments (nn, ks)   D hi
  static constexpr int OFF_DTL = OFF_DTH + 2 * NN * FRAG;// f16  2 NN fragments (nn, ks)   D lo
  static constexpr int OP = VT + 8;                      // token-row pitch of the output tile
  static constexpr int OFF_O = OFF_DTL + 2 * NN * FRAG;  // bf16 [CH][OP]   output staging
  static constexpr int LDS_BYTES = OFF_O + CH * OP * 2;
};

// the record operands one wave needs per chunk
struct Ops {
  f16x8 nw[4];        // -W rows 16w+tl, channels 32kb + 8gq..
  f16x8 qg[4];        // Q exp(G) rows
  f16x8 aqk[2];       // A_qk rows, tokens 32ks + 8gq..
  bf16x8 tbh[2], tbl[2];
  f16x8 kth[2][2], ktl[2][2];  // [mt][ks]: channel 32w + 16mt + tl, tokens 32ks + 8gq..
  float4 gl[2];       // exp(G_L) of channels 32w + 16mt + 4gq + 0..3
};

// One group of a chunk's record operands (P = 0..4).  The groups are issued
// at different points of the previous step so that the vector-memory path
// drains them while that step's MFMAs run, instead of stalling one block of
// issue.  Every load is one contiguous 1 KB fragment (64 lanes x 16 bytes).
template <int P, bool HAS_V = true, bool WRITE_OUT = true>
__device__ __forceinline__ void load_ops(Ops& o, const char* rec, int w, int lane, int gq, int ksmax) {
  if constexpr (P == 0) {
    const f16x8* nw = reinterpret_cast<const f16x8*>(rec + REC_NW) + lane;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) o.nw[kb] = nw[(4 * w + kb) * 64];
  } else if constexpr (P == 1) {
    if constexpr (WRITE_OUT) {
      const f16x8* qg = reinterpret_cast<const f16x8*>(rec + REC_QG) + lane;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) o.qg[kb] = qg[(4 * w + kb) * 64];
    }
  } else if constexpr (P == 2) {
    const f16x8* aq = reinterpret_cast<const f16x8*>(rec + REC_AQK) + lane;
    const bf16x8* th = reinterpret_cast<const bf16x8*>(rec + REC_TBH) + lane;
    const bf16x8* tlw = reinterpret_cast<const bf16x8*>(rec + REC_TBL) + lane;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // rows 16w.. of the lower-triangular A_qk and T only see tokens < 16w + 16:
      // waves 0 and 1 re-read their first k-step instead of the zero upper half
      const int kk = ks < ksmax ? ks : 0;
      if constexpr (WRITE_OUT) o.aqk[ks] = aq[(2 * w + kk) * 64];
      if constexpr (HAS_V) {
        o.tbh[ks] = th[(2 * w + kk) * 64];
        o.tbl[ks] = tlw[(2 * w + kk) * 64];
      }
    }
  } else if constexpr (P == 3) {
    const f16x8* kh = reinterpret_cast<const f16x8*>(rec + REC_KTH) + lane;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) o.kth[mt][ks] = kh[(4 * w + 2 * mt + ks) * 64];
  } else {
    const f16x8* kl = reinterpret_cast<const f16x8*>(rec + REC_KTL) + lane;
    const float* gl = reinterpret_cast<const float*>(rec + REC_GL);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) o.ktl[mt][ks] = kl[(4 * w + 2 * mt + ks) * 64];
      o.gl[mt] = *reinterpret_cast<const float4*>(gl + 32 * w + 16 * mt + 4 * gq);
    }
  }
}

template <bool HAS_V, bool WRITE_OUT>
__device__ __forceinline__ void load_ops_all(Ops& o, const char* rec, int w, int lane, int gq, int ksmax) {
  load_ops<0, HAS_V, WRITE_OUT>(o, rec, w, lane, gq, ksmax);
  load_ops<1, HAS_V, WRITE_OUT>(o, rec, w, lane, gq, ksmax);
  load_ops<2, HAS_V, WRITE_OUT>(o, rec, w, lane, gq, ksmax);
  load_ops<3, HAS_V, WRITE_OUT>(o, rec, w, lane, gq, ksmax);
  load_ops<4, HAS_V, WRITE_OUT>(o, rec, w, lane, gq, ksmax);
}

// V tile of a chunk: thread -> (token tid/4, columns 4NN*(tid%4) .. +4NN-1),
// held as 2NN packed dwords.  Rows past the chunk end are loaded from the
// clamped last row and zeroed only when written to LDS, so issuing the
// prefetch never waits for its data.
template <int NN>
struct VRow {
  uint32_t d[2 * NN];
};
template <int NN>
__device__ __forceinline__ void load_v(VRow<NN>& vv, const uint16_t* v, int64_t c0, int L, int H, int h,
                                       int vs, int tid, int vd) {
  const int t = tid >> 2;
  const int cg = tid & 3;
  const int tc = t < L ? t : L - 1;  // L >= 1: the clamped row is inside the sequence
  const uint16_t* row = v + ((c0 + tc) * H + h) * vd + vs + 4 * NN * cg;
  if constexpr (NN == 1) {
    const uint2 x = *reinterpret_cast<const uint2*>(row);
    vv.d[0] = x.x; vv.d[1] = x.y;
  } else {
#pragma unroll
    for (int u = 0; u < NN / 2; ++u) {
      const uint4 x = reinterpret_cast<const uint4*>(row)[u];
      vv.d[4 * u] = x.x; vv.d[4 * u + 1] = x.y; vv.d[4 * u + 2] = x.z; vv.d[4 * u + 3] = x.w;
    }
  }
}

// Token slot of V^T: token t of column c sits at t ^ vt_swz(c).  The XOR
// moves whole 8-token (16-byte) groups, so a B-operand read of 8 consecutive
// tokens stays one 16-byte read, while the packed 2-token writes below spread
// over all banks instead of hitting 8 column groups in the same ones.
__device__ __forceinline__ int vt_swz(int c) { return 8 * ((c >> 3) & 7); }

// Write the V tile transposed (column-major, 2 tokens per dword).  Lanes of
// neighbouring tokens t, t^1 (lanes 4 apart) trade half their columns, so
// each lane writes 2NN packed dwords: the even token's lane columns
// 4NN cg + 0..2NN-1, the odd token's lane columns 4NN cg + 2NN..4NN-1.
template <int NN>
__device__ __forceinline__ void store_vt(__bf16* sVt, const VRow<NN>& vv, int tid, int L) {
  const int t = tid >> 2;
  const int cg = tid & 3;
  const bool keep = t < L;
  const bool odd = t & 1;
  uint32_t mine[NN], recv[NN];
#pragma unroll
  for (int j = 0; j < NN; ++j) {
    mine[j] = keep ? (odd ? vv.d[NN + j] : vv.d[j]) : 0u;
    const uint32_t send = keep ? (odd ? vv.d[j] : vv.d[NN + j]) : 0u;
    recv[j] = (uint32_t)__shfl_xor((int)send, 4);
  }
  const int tp = t & ~1;
#pragma unroll
  for (int j = 0; j < NN; ++j) {
    const int c = 4 * NN * cg + (odd ? 2 * NN : 0) + 2 * j;
    const uint32_t lo = odd ? recv[j] : mine[j];  // token tp
    const uint32_t hi = odd ? mine[j] : recv[j];  // token tp + 1
    const uint32_t d0 = (lo & 0xffffu) | (hi << 16);           // column c
    const uint32_t d1 = (lo >> 16) | (hi & 0xffff0000u);       // column c + 1
    *reinterpret_cast<uint32_t*>(sVt + c * TP + (tp ^ vt_swz(c))) = d0;
    *reinterpret_cast<uint32_t*>(sVt + (c + 1) * TP + (tp ^ vt_swz(c + 1))) = d1;
  }
}

// HAS_V = false runs the recurrence with V = 0 (the homogeneous part of the
// chunk map, used for the per-shard affine map); WRITE_OUT = false computes
// only the final state; CKPT also stores every chunk's entering state and its
// D tile for the backward pass.
template <bool HAS_V, bool WRITE_OUT, bool CKPT = false, int NN = 4>
__global__ void __launch_bounds__(NTHREADS, 1) kda_inter_kernel(InterArgs a) {
  using C = Cfg<NN>;
  constexpr int VT = C::VT, OP = C::OP;
  // V slices per (sequence, head): V / VT.  Head dims 64 (K or V) use the
  // 128-channel, 128-column layout in registers and LDS: state rows c >= K
  // start at zero and stay there (their Kt rows are zero), and V = 64 has
  // half the slices.
  const int kd = a.kd, vd = a.vd;
  const int NV = vd / VT;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  __bf16* sVt = reinterpret_cast<__bf16*>(smem + C::OFF_VT);
  char* sSt = smem + C::OFF_ST;
  char* sDth = smem + C::OFF_DTH;
  char* sDtl = smem + C::OFF_DTL;

  // XCD-aware mapping: ids are dispatched round-robin over the 8 XCDs, so the
  // V slices of one (sequence, head) get ids with equal residue mod 8 and
  // read the chunk records through the same L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int r = bid >> 3;
  const int item = 8 * (r / NV) + xcd;
  const int slice = r % NV;
  const int H = a.H;
  if (item >= a.map.N * H) return;
  const int pos = item / H;
  const int h = item - pos * H;
  const int seq = a.order ? a.order[pos] : pos;
  int64_t bos, eos;
  seq_bounds(a.map, seq, bos, eos);
  const int64_t gfirst = first_chunk(a.map, seq);
  const int vs = slice * VT;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int tl = lane & 15;
  const int gq = lane >> 4;
  const int ksmax = (w >= 2) ? 2 : 1;  // token rows 16w.. only see tokens <= 16w + 15

  // state rows (channels) 32w + 16mt + 4gq + ii, columns vs + 16n + tl
  f32x4 S[2][NN];
  {
    const float* src = a.init ? a.init + ((int64_t)seq * H + h) * kd * vd : nullptr;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < NN; ++nn)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int c = 32 * w + 16 * mt + 4 * gq + ii;
          const int col = vs + 16 * nn + tl;
          S[mt][nn][ii] = src ? (c < kd ? src[a.state_vk ? col * kd + c : c * vd + col] : 0.0f)
                              : ((a.init_identity && c == col) ? 1.0f : 0.0f);
        }
  }
  // fp16 copy of the state's column tile nn (both row tiles of this wave)
  auto store_st_tile = [&](int nn) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const f16x4 hv = {(_Float16)S[mt][nn][0], (_Float16)S[mt][nn][1], (_Float16)S[mt][nn][2],
                        (_Float16)S[mt][nn][3]};
      frag_write4(sSt, 4 * nn + w, 4 * mt + gq, tl, hv);
    }
  };
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) store_st_tile(nn);
  __bf16* sO = reinterpret_cast<__bf16*>(smem + C::OFF_O);
  // Record operands are prefetched one chunk ahead into two register sets
  // that alternate through the 2x unrolled loop below; the loads of chunk c+1
  // are spread over chunk c's step.
  // With an odd number of chunks the first step is peeled off, so that the
  // loop always runs whole pairs: a conditional exit between the two steps
  // would merge a path with set B's loads still in flight into the loop head
  // and force shallow waits there.
  Ops opsA, opsB;
  auto chunk_len = [&](int64_t c) { return (int)((eos - c) < CH ? (eos - c) : CH); };
  const bool odd = ((eos - bos + CH - 1) / CH) & 1;
  if (bos < eos) {
    VRow<NN> v0;
    if constexpr (HAS_V) load_v(v0, a.v, bos, chunk_len(bos), H, h, vs, tid, vd);
    const char* r0 = a.rec + ((size_t)gfirst * H + h) * REC_BYTES;
    if (odd)
      load_ops_all<HAS_V, WRITE_OUT>(opsA, r0, w, lane, gq, ksmax);
    else
      load_ops_all<HAS_V, WRITE_OUT>(opsB, r0, w, lane, gq, ksmax);
    if constexpr (HAS_V) store_vt<NN>(sVt, v0, tid, chunk_len(bos));
  }
  __syncthreads();

  KDA_TIMER_DECL
  // one chunk step: `cur` holds this chunk's record operands; chunk c+1's
  // operands are issued into `pre` and its V tile is written to LDS at the end
  auto step = [&](Ops& cur, Ops& pre, int64_t c0, int64_t gch) {
    KDA_TIMER_MARK(0);
    const int L = chunk_len(c0);
    const int64_t c1 = c0 + CH;
    // Chunk c+1's loads are issued unconditionally (past the end of the
    // sequence the current chunk is re-read and ignored) so that every path
    // has the same number of outstanding loads.
    const bool in1 = c1 < eos;
    const char* prec = a.rec + ((size_t)(in1 ? gch + 1 : gch) * H + h) * REC_BYTES;
    // issue point of a load group, pinned between compute blocks
#define KDA_ISSUE(stmt)                   \
  do {                                    \
    __builtin_amdgcn_sched_barrier(0);    \
    stmt;                                 \
    __builtin_amdgcn_sched_barrier(0);    \
  } while (0)
    VRow<NN> vn;
    if constexpr (CKPT) {
      float* dst = a.states + ((size_t)gch * H + h) * KD * VD;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nn = 0; nn < NN; ++nn)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            dst[(32 * w + 16 * mt + 4 * gq + ii) * VD + vs + 16 * nn + tl] = S[mt][nn][ii];
    }
    if constexpr (HAS_V) KDA_ISSUE(load_v(vn, a.v, in1 ? c1 : c0, in1 ? chunk_len(c1) : L, H, h, vs, tid, vd));
    KDA_ISSUE((load_ops<0, HAS_V, WRITE_OUT>(pre, prec, w, lane, gq, ksmax)));
    KDA_TIMER_MARK(1);

    // ---- U, D = U - W S, O = QG S (token rows 16w.., all VT columns).  The
    // B operands come in six groups of NN 16-byte LDS reads (one per column
    // tile): groups 0-1 the V tile (k-steps of U), groups 2-5 the state copy
    // (k-blocks of W S and QG S).  Each group feeds 2 NN independent MFMA
    // chains and is read one group ahead, pinned there by a scheduling
    // barrier (left alone, the scheduler sinks every read to its first use
    // and waits for it there).  The two products share each state-copy read.
    f32x4 O[NN], u[NN];
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      u[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
      O[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    uint4 bq[2][NN];
    auto read_group = [&](int g, uint4(&dst)[NN]) {
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) {
        const int col = 16 * nn + tl;
        dst[nn] = g < 2 ? *reinterpret_cast<const uint4*>(sVt + col * TP + ((32 * g + 8 * gq) ^ vt_swz(col)))
                        : frag_read(sSt, 4 * nn + (g - 2), lane);
      }
    };
    constexpr int G0 = HAS_V ? 0 : 2;
    read_group(G0, bq[G0 & 1]);
#pragma unroll
    for (int g = G0; g < 6; ++g) {
      if (g + 1 < 6) read_group(g + 1, bq[(g + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      if (g < 2) {
        // Uniform control flow: every loaded operand register is consumed on
        // every path, so no load is still outstanding when its register is
        // reloaded (waves 0 and 1 multiply by zero for their upper k-step).
        const bf16x8 th = g < ksmax ? cur.tbh[g] : bf16x8{};
        const bf16x8 tlo = g < ksmax ? cur.tbl[g] : bf16x8{};
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) {
          const bf16x8 vb = __builtin_bit_cast(bf16x8, bq[g & 1][nn]);
          u[nn] = mfma_bf16(th, vb, u[nn]);
          u[nn] = mfma_bf16(tlo, vb, u[nn]);
        }
      } else {
        const int kb = g - 2;
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) {
          const f16x8 sb = __builtin_bit_cast(f16x8, bq[g & 1][nn]);
          u[nn] = mfma_f16(cur.nw[kb], sb, u[nn]);
          // O^T = S^T (QG)^T: lane holds token 16w + tl, columns 16nn + 4gq + 0..3
          if constexpr (WRITE_OUT) O[nn] = mfma_f16(sb, cur.qg[kb], O[nn]);
        }
      }
      if (g == 2) KDA_ISSUE((load_ops<1, HAS_V, WRITE_OUT>(pre, prec, w, lane, gq, ksmax)));
      if (g == 3) KDA_ISSUE((load_ops<2, HAS_V, WRITE_OUT>(pre, prec, w, lane, gq, ksmax)));
    }
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const int col = 16 * nn + tl;
      if constexpr (CKPT) {
        float* dst = a.dtile + ((size_t)gch * H + h) * CH * VD;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int i = 16 * w + 4 * gq + ii;
          dst[i * VD + vs + col] = i < L ? u[nn][ii] : 0.0f;
        }
      }
      // D^T hi/lo: lane holds tokens 16w + 4gq + 0..3 of column col
      f16x4 dh, dl;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const _Float16 hv = (_Float16)u[nn][ii];
        dh[ii] = hv;
        dl[ii] = (_Float16)(u[nn][ii] - (float)hv);
      }
      frag_write4(sDth, 2 * nn + (w >> 1), 4 * (w & 1) + gq, tl, dh);
      frag_write4(sDtl, 2 * nn + (w >> 1), 4 * (w & 1) + gq, tl, dl);
    }
    KDA_TIMER_MARK(2);
    __syncthreads();
    KDA_TIMER_MARK(3);

    // ---- O += A_qk D; S = Diag(exp(G_L)) S + Kt^T D.  The D^T hi/lo reads
    // of a column tile are issued one tile ahead; unlike the groups above they
    // are not pinned by a scheduling barrier (measured: the scheduler's own
    // placement is faster here, C3 forward 2.628 -> 2.614 ms).
    // Every wave finished reading the state copy and the V tile before the
    // barrier above, so both are rewritten for the next chunk inside this
    // phase: the fp16 copy of column tile nn - 1 while tile nn's MFMAs run,
    // and the V tile at tile 2 (the last tile when NN < 3).
    uint4 dq[2][4];
    auto read_d = [&](int nn, uint4(&dst)[4]) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        dst[ks] = frag_read(sDth, 2 * nn + ks, lane);
        dst[2 + ks] = frag_read(sDtl, 2 * nn + ks, lane);
      }
    };
    read_d(0, dq[0]);
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      if (nn + 1 < NN) read_d(nn + 1, dq[(nn + 1) & 1]);
      if (nn > 0) store_st_tile(nn - 1);
      // past the end of the sequence this rewrites the current tile, which
      // nothing reads
      if constexpr (HAS_V)
        if (nn == (NN > 2 ? 2 : NN - 1)) store_vt<NN>(sVt, vn, tid, in1 ? chunk_len(c1) : L);
      f16x8 dh[2], dl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        dh[ks] = __builtin_bit_cast(f16x8, dq[nn & 1][ks]);
        dl[ks] = __builtin_bit_cast(f16x8, dq[nn & 1][2 + ks]);
      }
      if constexpr (WRITE_OUT) {
        // O^T += D^T (A_qk)^T; the lane's 4 consecutive bf16 columns of token
        // row 16w + tl are staged in LDS with one 8-byte write
        f32x4 o = O[nn];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) o = mfma_f16(dh[ks], ks < ksmax ? cur.aqk[ks] : f16x8{}, o);
        const bf16x4 ob = {(__bf16)(o[0] * a.scale), (__bf16)(o[1] * a.scale), (__bf16)(o[2] * a.scale),
                           (__bf16)(o[3] * a.scale)};
        *reinterpret_cast<bf16x4*>(sO + (16 * w + tl) * OP + 16 * nn + 4 * gq) = ob;
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x4 s = S[mt][nn];
        s[0] *= cur.gl[mt].x;
        s[1] *= cur.gl[mt].y;
        s[2] *= cur.gl[mt].z;
        s[3] *= cur.gl[mt].w;
        // the Kt lo pass in its own accumulator: the record holds lo * 2^11
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          s = mfma_f16(cur.kth[mt][ks], dh[ks], s);
          s = mfma_f16(cur.kth[mt][ks], dl[ks], s);
          c = mfma_f16(cur.ktl[mt][ks], dh[ks], c);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) s[ii] = __builtin_fmaf(c[ii], KT_LO_UNSCALE, s[ii]);
        S[mt][nn] = s;
      }
      if (nn == 0) KDA_ISSUE((load_ops<3, HAS_V, WRITE_OUT>(pre, prec, w, lane, gq, ksmax)));
      if (nn == (NN > 1 ? 1 : 0)) KDA_ISSUE((load_ops<4, HAS_V, WRITE_OUT>(pre, prec, w, lane, gq, ksmax)));
    }
#undef KDA_ISSUE
    // this wave's 16 output rows: NN lanes per row, 16 columns per lane
    if constexpr (WRITE_OUT) {
      const int orow = 16 * w + lane / NN;
      const int ocol = 16 * (lane % NN);
      if (lane < 16 * NN && orow < L) {
        const uint4* srcp = reinterpret_cast<const uint4*>(sO + orow * OP + ocol);
        uint4* dstp = reinterpret_cast<uint4*>(a.out + ((c0 + orow) * H + h) * vd + vs + ocol);
        dstp[0] = srcp[0];
        dstp[1] = srcp[1];
      }
    }
    KDA_TIMER_MARK(4);
    store_st_tile(NN - 1);
    KDA_TIMER_MARK(5);
    __syncthreads();
    KDA_TIMER_MARK(6);
  };

  int64_t c0 = bos, gch = gfirst;
  if (odd) {
    step(opsA, opsB, c0, gch);
    c0 += CH;
    ++gch;
  }
  for (; c0 < eos; c0 += 2 * CH, gch += 2) {
    step(opsB, opsA, c0, gch);
    step(opsA, opsB, c0 + CH, gch + 1);
  }
  KDA_TIMER_STORE(a.timers);

  if (a.fin) {
    float* dst = a.fin + ((int64_t)seq * H + h) * kd * vd;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < NN; ++nn)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int c = 32 * w + 16 * mt + 4 * gq + ii;
          const int col = vs + 16 * nn + tl;
          if (c < kd) dst[a.state_vk ? col * kd + c : c * vd + col] = S[mt][nn][ii];
        }
  }
}

}  // namespace

// Column tiles per workgroup of the output-producing forward.  Each
// (sequence, head) chain is a sequential walk over its chunks, so with few
// chains the 64-column slices leave most CUs idle; narrower slices give each
// chain more workgroups (every one re-reads the chunk's record, through the
// L2 of its XCD).  Wide slices stay in use once the chains alone fill half
// the CUs.
int inter_tiles(int64_t chains, int cus) {
  if (chains * 2 >= cus / 2) return 4;
  if (chains * 4 >= cus / 2) return 2;
  return 1;
}

hipError_t launch_inter(const InterArgs& args, hipStream_t st) {
  const int64_t items = (int64_t)args.map.N * args.H;
  InterArgs a = args;
  void* kargs[] = {(void*)&a};
  int nn = 4;
  if (a.v && a.out && !a.states) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    nn = inter_tiles(items, cus);
  }
  const void* fn;
  if (a.states)
    fn = reinterpret_cast<const void*>(&kda_inter_kernel<true, false, true>);
  else if (a.v)
    fn = !a.out    ? reinterpret_cast<const void*>(&kda_inter_kernel<true, false>)
         : nn == 1 ? reinterpret_cast<const void*>(&kda_inter_kernel<true, true, false, 1>)
         : nn == 2 ? reinterpret_cast<const void*>(&kda_inter_kernel<true, true, false, 2>)
                   : reinterpret_cast<const void*>(&kda_inter_kernel<true, true>);
  else
    fn = a.out ? reinterpret_cast<const void*>(&kda_inter_kernel<false, true>)
               : reinterpret_cast<const void*>(&kda_inter_kernel<false, false>);
  // ids 8m + x (x = XCD) cover the V / (16 nn) slices of items 8(m / slices) + x
  const int64_t grid = (items + 7) / 8 * 8 * (a.vd / (16 * nn));
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(NTHREADS), kargs, 0, st);
}

}  // namespace kda
