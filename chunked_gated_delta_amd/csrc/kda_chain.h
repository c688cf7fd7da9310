// Chain kernel of the gfx950 KDA forward: the sequential recurrence over the
// chunks of one (sequence, head), on NQ column quarters of 32 state columns
// (NQ = 4: all 128 columns in one workgroup; NQ = 2: one 64-column half, two
// workgroups per (sequence, head)).
//
// It computes what the inter-chunk kernel computes, from the same per-chunk
// records of the intra-chunk kernel (kda_common.h), for each chunk:
//     U = T diag(b) V                       (bf16 hi/lo x exact bf16 V)
//     D = U - W S                           (fp16 W, fp16 copy of S)
//     O = scale [ (Q exp(G)) S + A_qk D ]   -> bf16 output
//     S = Diag(exp(G_L)) S + (K exp(G_L - G))^T D   (fp16 hi/lo x fp16 hi/lo)
// with every product, operand split and accumulation order of that kernel,
// so the two give the same bits.  Where the inter kernel holds 337 registers
// per lane (its record operands prefetched a whole chunk ahead), this one
// holds at most 256, so that two of its workgroups, or one of them and one
// intra-chunk workgroup, fit on a CU.  The cost is that record operands are
// not prefetched a whole chunk ahead (no room for a second register set):
// each group is loaded when its previous use ends.
//
// Wave w owns the state rows (channels) 32w..32w+31 of the workgroup's
// columns (16 NQ registers of fp32 accumulators per row tile) and the token
// rows 16w..16w+15 of U, D and O.  A chunk step runs the column quarters q
// (32 columns, tiles 2q, 2q+1):
//     A_q: U and D of quarter q, and the state part of O      -> D hi/lo to LDS
//     barrier
//     B_q: O += A_qk D; the state update of quarter q; the new fp16 state
//          copy of quarter q; quarter q of the next chunk's V tile
// in the order A0 | B0 A1 | B1 ... | B(NQ-1).  D alternates between two LDS
// buffers, so B_q and A_{q+1} need no barrier between them; every LDS region
// a phase writes was last read before the barrier that precedes it.

#pragma once

#include "kda_common.h"

namespace kda {
namespace chain {

constexpr int NTHREADS = 256;
constexpr int VTP = CH + 8;      // token pitch of the V^T tile (halves)
constexpr int OQP = 32 + 8;      // column pitch of the output staging rows (halves)
template <int NQ>
struct Lay {
  static constexpr int NCOL = 32 * NQ;                      // state columns of the workgroup
  static constexpr int OFF_VT = 0;                          // bf16 [NCOL columns][VTP]   V^T
  static constexpr int OFF_ST = OFF_VT + NCOL * VTP * 2;    // f16 8 NQ fragments (4 nn + kb)  state copy
  static constexpr int OFF_D = OFF_ST + 8 * NQ * FRAG;      // 2 buffers x 8 fragments   D hi (0-3), lo (4-7)
  static constexpr int OFF_O = OFF_D + 2 * 8 * FRAG;        // bf16 [64 tokens][OQP]      output staging
  static constexpr int LDS_BYTES = OFF_O + CH * OQP * 2;    // NQ = 4: 72,704; NQ = 2: 47,104
  static_assert(LDS_BYTES <= 80 * 1024, "two workgroups per CU");
};

// Record operands of the A phases (U, D, the state part of O) and of the B
// phases (the A_qk D part of O, the state update), per wave.
struct AOps {
  f16x8 nw[4];       // -W rows 16w + tl, channels 32kb + 8gq..
  f16x8 qg[4];       // Q exp(G) rows
  bf16x8 tbh[2], tbl[2];  // T diag(b) rows, tokens 32ks + 8gq..
};
struct BOps {
  f16x8 kth[2][2], ktl[2][2];  // [mt][ks]: channel 32w + 16mt + tl, tokens 32ks + 8gq..
  f16x8 aqk[2];                // A_qk rows, tokens 32ks + 8gq..
  float4 gl[2];                // exp(G_L) of channels 32w + 16mt + 4gq + 0..3
};

// Record and V loads are buffer loads (kda_common.h): one descriptor per
// chunk and a single lane offset, every fragment's place a wave-uniform
// scalar offset.  Per-load 64-bit addresses would cost about 60 vector
// registers, which a 256-register chain cannot spare.

// Rows 16w.. of the lower-triangular A_qk and T only see tokens < 16w + 16:
// waves 0 and 1 re-read their first k-step in place of the zero upper half.
// `lo16` is lane * 16, `w` wave-uniform.
// POLICY SC1 reads records another CU wrote into this XCD's L2 (the fused
// pipeline), 0 those of a finished earlier kernel.
template <int P>
__device__ __forceinline__ void load_a(AOps& o, __amdgpu_buffer_rsrc_t r, int w, int lo16, int ksmax) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    o.nw[kb] = bload<f16x8, P>(r, lo16, (int)REC_NW + (4 * w + kb) * FRAG);
    o.qg[kb] = bload<f16x8, P>(r, lo16, (int)REC_QG + (4 * w + kb) * FRAG);
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int kk = ks < ksmax ? ks : 0;
    o.tbh[ks] = bload<bf16x8, P>(r, lo16, (int)REC_TBH + (2 * w + kk) * FRAG);
    o.tbl[ks] = bload<bf16x8, P>(r, lo16, (int)REC_TBL + (2 * w + kk) * FRAG);
  }
}

template <int P>
__device__ __forceinline__ void load_b(BOps& o, __amdgpu_buffer_rsrc_t r, int w, int lo16, int gq16, int ksmax) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      o.kth[mt][ks] = bload<f16x8, P>(r, lo16, (int)REC_KTH + (4 * w + 2 * mt + ks) * FRAG);
      o.ktl[mt][ks] = bload<f16x8, P>(r, lo16, (int)REC_KTL + (4 * w + 2 * mt + ks) * FRAG);
    }
    o.gl[mt] = bload<float4, P>(r, gq16, (int)REC_GL + (32 * w + 16 * mt) * 4);
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    o.aqk[ks] = bload<f16x8, P>(r, lo16, (int)REC_AQK + (2 * w + (ks < ksmax ? ks : 0)) * FRAG);
}

// The V tile of a chunk, per thread: token t = tid / 4 and, for each quarter
// q, the 8 columns 32q + 8p..+7 (p = tid % 4) of the workgroup's columns, as
// 4 packed dwords.  Rows past the chunk end are loaded from the clamped last
// row and zeroed when written.  `r` covers the chunk's rows from its first
// token and the workgroup's first column.
template <int NQ>
struct VTile {
  uint32_t d[NQ][4];
};
template <int NQ>
__device__ __forceinline__ void load_vtile(VTile<NQ>& vv, __amdgpu_buffer_rsrc_t r, int L, int H, int tid) {
  const int t = tid >> 2;
  const int p = tid & 3;
  const int tc = t < L ? t : L - 1;  // L >= 1: the clamped row is inside the sequence
  const int voff = (tc * H * VD + 8 * p) * 2;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const u32x4 x = bload<u32x4>(r, voff, 64 * q);
    vv.d[q][0] = x[0]; vv.d[q][1] = x[1]; vv.d[q][2] = x[2]; vv.d[q][3] = x[3];
  }
}

// V^T is stored plainly, column c at c * VTP: every read and write address is
// a per-lane base plus a compile-time offset.  (A bank-spreading XOR of the
// token slot would mix lane and tile bits and cost a register per address.)
// Write quarter q of the V tile transposed, 2 tokens per dword: the threads of
// tokens t and t ^ 1 (4 lanes apart) trade half of their 8 columns, so each
// writes 4 columns x 2 tokens.
template <int NQ>
__device__ __forceinline__ void store_vt_quarter(__bf16* sVt, const VTile<NQ>& vv, int q, int tid, int L) {
  const int t = tid >> 2;
  const int p = tid & 3;
  const bool keep = t < L;
  const bool odd = t & 1;
  uint32_t mine[2], recv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    mine[j] = keep ? (odd ? vv.d[q][2 + j] : vv.d[q][j]) : 0u;
    const uint32_t send = keep ? (odd ? vv.d[q][j] : vv.d[q][2 + j]) : 0u;
    recv[j] = (uint32_t)__shfl_xor((int)send, 4);
  }
  const int tp = t & ~1;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = 32 * q + 8 * p + (odd ? 4 : 0) + 2 * j;
    const uint32_t lo = odd ? recv[j] : mine[j];  // token tp
    const uint32_t hi = odd ? mine[j] : recv[j];  // token tp + 1
    *reinterpret_cast<uint32_t*>(sVt + c * VTP + tp) = (lo & 0xffffu) | (hi << 16);
    *reinterpret_cast<uint32_t*>(sVt + (c + 1) * VTP + tp) = (lo >> 16) | (hi & 0xffff0000u);
  }
}

// Load (STORE = false) or store the workgroup's columns vs.. of a (sequence,
// head)'s state held as S[mt][nn] (channels 32w + 16mt + 4gq + ii, columns
// vs + 16nn + tl) through buffer operations: one lane offset, every element's
// place a compile-time or wave-uniform offset.  The lane offsets are
// re-derived from an opaque thread id, so none of them stays live across the
// chunk loop.  A null pointer leaves zeros (load) or writes nothing (store).
template <bool STORE, int NQ>
__device__ __forceinline__ void state_io(f32x4 (&S)[2][2 * NQ], const float* p, int vk, int seq, int h, int H,
                                         int vs) {
  if (!STORE) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < 2 * NQ; ++nn) S[mt][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (!p) return;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tl = tid & 15;
  const int gq = (tid >> 4) & 3;
  const __amdgpu_buffer_rsrc_t r = buf(p + ((int64_t)seq * H + h) * KD * VD, (uint32_t)(KD * VD * 4));
  if (vk) {
    // S[c][col] at col * K + c: the lane's 4 channels are one 16-byte access
    const int voff = (tl * KD + 4 * gq) * 4;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < 2 * NQ; ++nn) {
        const int soff = ((vs + 16 * nn) * KD + 32 * w + 16 * mt) * 4;
        if (STORE)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, S[mt][nn]), r, voff, soff, 0);
        else
          S[mt][nn] = bload<f32x4>(r, voff, soff);
      }
  } else {
    // S[c][col] at c * V + col: 16 lanes of one channel cover 64 contiguous bytes
    const int voff = (4 * gq * VD + tl) * 4;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nn = 0; nn < 2 * NQ; ++nn) {
        // whole-vector bit casts: a cast of one element of S[mt][nn] straight
        // into the store builtin has stored element 0 for every element
        u32x4 bits = __builtin_bit_cast(u32x4, S[mt][nn]);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int soff = ((32 * w + 16 * mt + ii) * VD + vs + 16 * nn) * 4;
          if (STORE)
            __builtin_amdgcn_raw_buffer_store_b32(bits[ii], r, voff, soff, 0);
          else
            bits[ii] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
        }
        if (!STORE) S[mt][nn] = __builtin_bit_cast(f32x4, bits);
      }
  }
}

// One (sequence, head) chain on the state columns vs .. vs + 32 NQ - 1: all
// its chunks, from its initial state to its final state.  `smem` is this
// workgroup's Lay<NQ>::LDS_BYTES.  FUSED: the single sequence of a fused
// pipeline; each chunk's record is read once its ready flag says where it is
// (ring slot or record area), and after every chunk the chain publishes how
// many records it has finished reading (ChainFused::consumed, its own line).
template <bool FUSED, int NQ>
__device__ __forceinline__ void chain_run(const ChainArgs& a, const ChainFused& fz, int seq, int h, int vs,
                                          char* smem) {
  using LY = Lay<NQ>;
  __bf16* sVt = reinterpret_cast<__bf16*>(smem + LY::OFF_VT);
  char* sSt = smem + LY::OFF_ST;
  __bf16* sO = reinterpret_cast<__bf16*>(smem + LY::OFF_O);
  const int H = a.H;
  int64_t bos, eos;
  seq_bounds(a.map, seq, bos, eos);
  const int64_t gfirst = first_chunk(a.map, seq);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int tl = lane & 15;
  const int gq = lane >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // wave-uniform: scalar offsets
  const int ksmax = (wu >= 2) ? 2 : 1;

  // state rows (channels) 32w + 16mt + 4gq + ii, columns vs + 16nn + tl
  f32x4 S[2][2 * NQ];
  state_io<false, NQ>(S, a.init, a.state_vk, seq, h, H, vs);
  // fp16 copy of the state's column tile nn (both row tiles of this wave):
  // fragment (nn, kb = w) holds channels 32w.. of columns 16nn..
  auto store_st_tile = [&](int nn) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const f16x4 hv = {(_Float16)S[mt][nn][0], (_Float16)S[mt][nn][1], (_Float16)S[mt][nn][2],
                        (_Float16)S[mt][nn][3]};
      frag_write4(sSt, 4 * nn + w, 4 * mt + gq, tl, hv);
    }
  };
#pragma unroll
  for (int nn = 0; nn < 2 * NQ; ++nn) store_st_tile(nn);

  auto chunk_len = [&](int64_t c) { return (int)((eos - c) < CH ? (eos - c) : CH); };
  // buffer descriptors of a chunk's record and of its V rows (64 token rows
  // of H * VD halves from its first token)
  // A ready flag is polled with L1-bypassing loads and a short sleep, for a
  // bounded time: a wait that gives up records FAULT_WAIT_TIMEOUT, and the
  // chain then stops waiting at all (every later record reads the record
  // area), so the kernel still ends.
  bool poisoned = false;
  auto rec_buf = [&](int64_t g) {
    const char* base = a.rec + ((size_t)g * H + h) * REC_BYTES;
    if constexpr (FUSED) {
      int v = 2;
      if (!poisoned) {
        const __amdgpu_buffer_rsrc_t fr = buf(fz.flags, (uint32_t)fz.nchunk * H * 4);
        for (int spin = 0;; ++spin) {
          v = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(fr, 0, (int)(g * H + h) * 4, SC1));
          if (v != 0) break;
          if (spin == FUSED_SPIN_LIMIT) {
            if ((threadIdx.x & 63) == 0) atomicOr(fz.faults, FAULT_WAIT_TIMEOUT);
            poisoned = true;
            v = 2;
            break;
          }
          __builtin_amdgcn_s_sleep(4);
          asm volatile("" ::: "memory");
        }
      }
      if (v == 1) base = fz.ringbuf + ((size_t)h * fz.ring + (size_t)(g % fz.ring)) * REC_BYTES;
    }
    return buf(base, (uint32_t)REC_BYTES);
  };
  constexpr int LP = FUSED ? SC1 : 0;
  // (the last row's columns vs.. end inside the row, which ends the range)
  auto v_buf = [&](int64_t c) {
    return buf(a.v + (c * H + h) * VD + vs, (uint32_t)(((CH - 1) * H + 1) * VD * 2 - vs * 2));
  };
  const int lo16 = lane * 16;
  const int gq16 = gq * 16;
  AOps ao;
  BOps bo;
  VTile<NQ> vn;
  if (bos < eos) {
    VTile<NQ> v0;
    load_vtile(v0, v_buf(bos), chunk_len(bos), H, tid);
    const __amdgpu_buffer_rsrc_t r0 = rec_buf(gfirst);
    load_a<LP>(ao, r0, wu, lo16, ksmax);
    load_b<LP>(bo, r0, wu, lo16, gq16, ksmax);
#pragma unroll
    for (int q = 0; q < NQ; ++q) store_vt_quarter(sVt, v0, q, tid, chunk_len(bos));
  }
  __syncthreads();

  int64_t gch = gfirst;
  for (int64_t c0 = bos; c0 < eos; c0 += CH, ++gch) {
    const int L = chunk_len(c0);
    const int64_t c1 = c0 + CH;
    const bool in1 = c1 < eos;
    // the next chunk's V tile (past the end: this chunk's again, never read)
    load_vtile(vn, v_buf(in1 ? c1 : c0), in1 ? chunk_len(c1) : L, H, tid);
    // the next chunk's record (past the end: this one's again), found when its
    // A operands are first loaded, at the end of the last A phase
    __amdgpu_buffer_rsrc_t nrec;

#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      char* sDh = smem + LY::OFF_D + (q & 1) * 8 * FRAG;
      char* sDl = sDh + 4 * FRAG;
      // ---- A_q: U = T diag(b) V, D = U - W S, O = (Q exp(G)) S on the two
      // column tiles 2q, 2q + 1 of this wave's token rows.  The B operands
      // (V^T k-steps, then the state copy's k-blocks) are read one group ahead.
      f32x4 u[2], O[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        O[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      uint4 bq[2][2];
      auto read_group = [&](int g, uint4(&dst)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int nn = 2 * q + j;
          const int col = 16 * nn + tl;
          dst[j] = g < 2 ? *reinterpret_cast<const uint4*>(sVt + col * VTP + 32 * g + 8 * gq)
                         : frag_read(sSt, 4 * nn + (g - 2), lane);
        }
      };
      read_group(0, bq[0]);
#pragma unroll
      for (int g = 0; g < 6; ++g) {
        if (g + 1 < 6) read_group(g + 1, bq[(g + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        if (g < 2) {
          // uniform control flow: waves 0 and 1 multiply by zero for their upper k-step
          const bf16x8 th = g < ksmax ? ao.tbh[g] : bf16x8{};
          const bf16x8 tlo = g < ksmax ? ao.tbl[g] : bf16x8{};
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const bf16x8 vb = __builtin_bit_cast(bf16x8, bq[g & 1][j]);
            u[j] = mfma_bf16(th, vb, u[j]);
            u[j] = mfma_bf16(tlo, vb, u[j]);
          }
        } else {
          const int kb = g - 2;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const f16x8 sb = __builtin_bit_cast(f16x8, bq[g & 1][j]);
            u[j] = mfma_f16(ao.nw[kb], sb, u[j]);
            // O^T = S^T (QG)^T: lane holds token 16w + tl, columns 16nn + 4gq + 0..3
            O[j] = mfma_f16(sb, ao.qg[kb], O[j]);
          }
        }
      }
      // D^T hi/lo: lane holds tokens 16w + 4gq + 0..3 of column 16nn + tl;
      // fragment (j, ks) of this quarter's D
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f16x4 dh, dl;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const _Float16 hv = (_Float16)u[j][ii];
          dh[ii] = hv;
          dl[ii] = (_Float16)(u[j][ii] - (float)hv);
        }
        frag_write4(sDh, 2 * j + (w >> 1), 4 * (w & 1) + gq, tl, dh);
        frag_write4(sDl, 2 * j + (w >> 1), 4 * (w & 1) + gq, tl, dl);
      }
      if (q == NQ - 1) {
        // the A operands are dead: the next chunk's (past the end, this one's again)
        nrec = rec_buf(in1 ? gch + 1 : gch);
        __builtin_amdgcn_sched_barrier(0);
        load_a<LP>(ao, nrec, wu, lo16, ksmax);
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
      if constexpr (FUSED) {
        // every wave has used (so finished loading) all of this chunk's record
        if (q == NQ - 1 && threadIdx.x == 0)
          __builtin_amdgcn_raw_buffer_store_b32((int)(gch + 1), buf(fz.consumed, (uint32_t)FUSED_LINE), 0, 0,
                                                SC1);
      }

      // ---- B_q: O += A_qk D; S = Diag(exp(G_L)) S + Kt^T D on tiles 2q, 2q + 1
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nn = 2 * q + j;
        f16x8 dh[2], dl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          dh[ks] = __builtin_bit_cast(f16x8, frag_read(sDh, 2 * j + ks, lane));
          dl[ks] = __builtin_bit_cast(f16x8, frag_read(sDl, 2 * j + ks, lane));
        }
        // O^T += D^T (A_qk)^T; the lane's 4 consecutive bf16 columns of token
        // row 16w + tl are staged in LDS with one 8-byte write
        f32x4 o = O[j];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) o = mfma_f16(dh[ks], ks < ksmax ? bo.aqk[ks] : f16x8{}, o);
        const bf16x4 ob = {(__bf16)(o[0] * a.scale), (__bf16)(o[1] * a.scale), (__bf16)(o[2] * a.scale),
                           (__bf16)(o[3] * a.scale)};
        *reinterpret_cast<bf16x4*>(sO + (16 * w + tl) * OQP + 16 * j + 4 * gq) = ob;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          f32x4 s = S[mt][nn];
          s[0] *= bo.gl[mt].x;
          s[1] *= bo.gl[mt].y;
          s[2] *= bo.gl[mt].z;
          s[3] *= bo.gl[mt].w;
          // the Kt lo pass in its own accumulator: the record holds lo * 2^11
          f32x4 cl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            s = mfma_f16(bo.kth[mt][ks], dh[ks], s);
            s = mfma_f16(bo.kth[mt][ks], dl[ks], s);
            cl = mfma_f16(bo.ktl[mt][ks], dh[ks], cl);
          }
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) s[ii] = __builtin_fmaf(cl[ii], KT_LO_UNSCALE, s[ii]);
          S[mt][nn] = s;
        }
        store_st_tile(nn);
      }
      // this wave's 16 output rows of the quarter (64 bytes each): 4 lanes per row
      {
        const int orow = 16 * w + (lane >> 2);
        const int ocol = 8 * (lane & 3);
        if (orow < L) {
          const uint4 val = *reinterpret_cast<const uint4*>(sO + orow * OQP + ocol);
          *reinterpret_cast<uint4*>(a.out + ((c0 + orow) * H + h) * VD + vs + 32 * q + ocol) = val;
        }
      }
      // quarter q of the next chunk's V tile (every wave read this chunk's
      // quarter q before the barrier above)
      store_vt_quarter(sVt, vn, q, tid, in1 ? chunk_len(c1) : L);
      if (q == NQ - 1) {
        // the B operands are dead: the next chunk's
        __builtin_amdgcn_sched_barrier(0);
        load_b<LP>(bo, nrec, wu, lo16, gq16, ksmax);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  state_io<true, NQ>(S, a.fin, a.state_vk, seq, h, H, vs);
}

}  // namespace chain
}  // namespace kda
