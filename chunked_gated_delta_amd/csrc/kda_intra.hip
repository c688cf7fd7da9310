// Intra-chunk kernel of the gfx950 KDA forward: everything that does not
// depend on the running state, computed once per (64-token chunk, head) and
// fully parallel over chunks.
//
// The chunk algebra is derived from the per-token gated delta rule
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = scale S_t^T q_t
// with L2-normalised q, k, b = sigmoid(raw_beta) and the bounded gate
// log a = lower_bound * sigmoid(exp(A_log) (raw_gate + dt_bias)) — the op and
// its flags as named on the instagit FlashKDA page ("Usage Examples") and the
// argument roles of the 14-argument call in the vLLM PR report ("关键源码片段");
// the pages print neither the recurrence nor the chunk form.  For one chunk of
// L <= 64 tokens with per-channel cumulative log-decay G (reset at the chunk
// start):
//     A_kk[i,j] = b_i <k_i exp(G_i - G_j), k_j>  (j < i)     T = (I + A_kk)^-1
//     W = T diag(b) (K exp(G))      A_qk[i,j] = <q_i exp(G_i - G_j), k_j>  (j <= i)
// The inter-chunk kernel then applies D = T diag(b) V - W S, O = scale [(Q exp(G)) S
// + A_qk D], S <- exp(G_L) S + (K exp(G_L - G))^T D.
//
// Decay ratios exp(G_i - G_j) are never formed as exp(G_i) exp(-G_j) (that
// spans exp(+-320) at lower_bound = -5).  The chunk is cut into four 16-token
// sub-chunks w with start prefix P_w; a pair (i, j) is split through a
// per-channel point between them: for i in w and j in an earlier sub-chunk b
// through P_{b+1} (both factors <= 1), inside sub-chunk w through P_w (one
// factor in [1, exp(80)], inside fp32/bf16 range).
//
// Precision: A_kk is built from bf16 hi/lo operands in 3 MFMA passes; T is
// fp32 (16x16 diagonal blocks by forward substitution, off-diagonal blocks on
// fp32 MFMA); W = (T diag(b) as fp16 hi/lo) x (K exp(G) as fp16), 2 passes.
// These were chosen so that the final state stays within 1e-3 relative L2 of
// an fp64 reference for identical (collinear) keys, where the chunk sums
// telescope and 16-bit rounding of A, T or W alone would exceed it.
//
// Persistent workgroups (4 waves) loop over (chunk, head) items; in each item
// every wave owns one 16-token sub-chunk, in a role that rotates per item.

#include "kda_chain.h"
#include "kda_common.h"

namespace kda {
namespace {

constexpr int NTHREADS = 256;
constexpr int KP = KD + 8;   // token-row pitch (halves)
constexpr int TP = CH + 8;   // channel-row pitch (halves), 16-byte aligned rows
constexpr int AP = CH + 4;   // fp32 square pitch
constexpr int TBP = CH + 8;  // fp16 square pitch

// LDS carve-up (bytes).  R1: k^ exp(P_{w+1} - G) for the off-diagonal A blocks,
// later reused for T diag(b) in fp16 hi/lo.  R2: A_kk, inverted in place to T.
constexpr int OFF_KRF_HI = 0;                          // bf16 [48][KP]
constexpr int OFF_KRF_LO = OFF_KRF_HI + 48 * KP * 2;
constexpr int OFF_TB_HI = 0;                           // f16 [64][TBP]
constexpr int OFF_TB_LO = OFF_TB_HI + CH * TBP * 2;
constexpr int R1_END = OFF_KRF_LO + 48 * KP * 2;
static_assert(OFF_TB_LO + CH * TBP * 2 <= R1_END, "R1");
constexpr int OFF_A = R1_END;                          // f32 [64][AP]
constexpr int OFF_KG = OFF_A + CH * AP * 4;            // f16 [128][TP] (k^ exp(G))^T
constexpr int OFF_P = OFF_KG + KD * TP * 2;            // f32 [5][128] sub-chunk prefixes
constexpr int OFF_TOT = OFF_P + 5 * KD * 4;            // f32 [4][128] sub-chunk totals
constexpr int NFAC = 15;
constexpr int OFF_FAC = OFF_TOT + 4 * KD * 4;          // f32 [NFAC][128] decay factors
constexpr int OFF_NB = OFF_FAC + NFAC * KD * 4;        // f32 [128] gate offsets
constexpr int OFF_B = OFF_NB + KD * 4;                 // f32 [64] beta
constexpr int OFF_FLAG = OFF_B + CH * 4;               // int [8] ready tags, [1] claim, [1] record place
constexpr int LDS_BYTES = OFF_FLAG + 12 * 4;
static_assert(LDS_BYTES <= 80 * 1024, "two workgroups per CU");

// decay-factor rows (per channel, log2 units, P_w = prefix before sub-chunk w):
//   ET+w: exp2(P_{w+1} - P_w)   EP+w: exp2(P_w)   EL+w: exp2(P_4 - P_w)
//   F20, F30, F31: exp2(P_w - P_{b+1}) for off-diagonal blocks (w, b), b < w - 1
constexpr int FAC_ET = 0, FAC_EP = 4, FAC_EL = 8, FAC_F20 = 12, FAC_F30 = 13, FAC_F31 = 14;

// inclusive prefix sum over the 16 lanes of a DPP row
__device__ __forceinline__ float row_scan16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, true));
  return x;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 hi/lo split of 8 floats, two at a time: hi = RNE(x), lo = RNE(x - hi).
// Converting pairs (one packed conversion each) and reading hi back with a
// shift or a mask takes 3 instructions per element, against 4 when every
// element is converted on its own first.
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const f32x2 v = {x[2 * p], x[2 * p + 1]};
    h[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    const f32x2 r = {x[2 * p] - __uint_as_float(h[p] << 16), x[2 * p + 1] - __uint_as_float(h[p] & 0xffff0000u)};
    l[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float (&x)[8]) {
  uint32_t h[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const f32x2 v = {x[2 * p], x[2 * p + 1]};
    h[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  return __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A store to the chunk record.  Non-temporal (NT) when the call's record area
// is too large to stay in the Infinity Cache, so that the next kernel reads
// every record back from HBM anyway (B=1, T=32768, H=96 forward 2.652 ->
// 2.610 ms); plain when it fits (B=2, T=4096, H=12: 139 MB of records, 0.228
// -> 0.190 ms cold, the inter kernel then reading them from the cache) and in
// the single-launch schedule, whose chains read the records through the
// producer's L2.
template <bool NT, typename T>
__device__ __forceinline__ void rec_store(T* p, T v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

}  // namespace

// The chunk table, A_log and the record base are also passed as separate
// __restrict__ arguments: with no possible aliasing by the record stores, the
// wave-uniform loads from them can go through the scalar unit and never wait
// behind the vector memory queue.  GATE_GIVEN is a template switch: a runtime
// choice inside the per-element gate loop would split it into 32 branches and
// keep the scan from interleaving.
//
// One workgroup's share of the (chunk, head) items.  Standalone (FUSED =
// false): items are (last chunk - chunk) * H + head over every sequence, the
// workgroup's first two are `first` and first + stride, later ones are claimed
// from `claim`, and each record goes to recs[chunk][head].  FUSED: the items
// of one XCD's heads of a single sequence in chunk order (chunk * hx + l for
// head xcd + 8 l), each record goes to its head's ring slot or to
// recs[chunk][head] (IntraFused), and its ready flag then says which.
// KIN: the head dim K of q, k, raw_gate and dt_bias in memory (64 or 128).
// With K = 64 the item is computed in the 128-channel layout with channels
// 64..127 of q and k zero (so they add nothing to any norm, dot product or
// record entry) and their gate inputs zero (a finite decay that multiplies
// only those zero channels); the record layout is that of K = 128.
template <bool GATE_GIVEN, bool FUSED, int KIN = KD, bool NT = false>
__device__ __forceinline__ void intra_items(IntraArgs a, const int32_t* __restrict__ cu,
                                            const int32_t* __restrict__ choff, const float* __restrict__ A_log,
                                            char* __restrict__ recs, char* smem, int first, int stride, int* claim,
                                            const IntraFused& fz) {
  __bf16* sKRFh = reinterpret_cast<__bf16*>(smem + OFF_KRF_HI);
  __bf16* sKRFl = reinterpret_cast<__bf16*>(smem + OFF_KRF_LO);
  _Float16* sTbh = reinterpret_cast<_Float16*>(smem + OFF_TB_HI);
  _Float16* sTbl = reinterpret_cast<_Float16*>(smem + OFF_TB_LO);
  float* sA = reinterpret_cast<float*>(smem + OFF_A);
  _Float16* sKG = reinterpret_cast<_Float16*>(smem + OFF_KG);
  float* sP = reinterpret_cast<float*>(smem + OFF_P);
  float* sTot = reinterpret_cast<float*>(smem + OFF_TOT);
  float* sFac = reinterpret_cast<float*>(smem + OFF_FAC);
  float* sNB = reinterpret_cast<float*>(smem + OFF_NB);
  float* sB = reinterpret_cast<float*>(smem + OFF_B);
  int* sFlag = reinterpret_cast<int*>(smem + OFF_FLAG);
  int* sClaim = sFlag + 8;
  int* sDest = sFlag + 9;

  const int H = a.H;

  // Work items are (chunk, head) pairs, item = (last chunk - chunk) * H + head,
  // taken in grid-stride order.  The next item's inputs are loaded while the
  // current one is in its MFMA phases, so their latency is hidden.  (The host
  // checks that chunks x heads fits in an int.)
  ChunkMap map = a.map;
  map.cu = cu;
  map.choff = choff;
  const int64_t nchunk = FUSED ? (int64_t)fz.nchunk : total_chunks(map);
  const int items = FUSED ? (int)nchunk * fz.hx : (int)(nchunk * H);
  // The first two items of a workgroup are blockIdx.x and blockIdx.x + grid;
  // after that it claims items from a counter (one claim per processed item,
  // made an item ahead so that its latency stays hidden), so workgroups that
  // run faster take more items and all finish together.  Claims only grow:
  // once a workgroup's next item is past the end, so is every later claim.
  int item = first;
  if (item >= items) return;
  int next = item + stride;
  // ready tags hold the item whose data they publish; no item is -1.  Tags
  // 0-3: row-block b (its A blocks, and T_bb for b < 3); 5: A_33; 6: T_33.
  if (threadIdx.x < 8) sFlag[threadIdx.x] = -1;

  // inputs of one item for this lane's token: channels 32kb + 8gq + e.  All
  // loads are unconditional: rows past the chunk end read the last valid row
  // and are zeroed through their norms, gate and beta, so no load waits
  // behind a branch.
  uint4 pq[4], pk[4], pg[4];
  uint16_t braw16;
  float dtb, alog;
  auto locate = [&](int it, int& hh, int64_t& gg, int64_t& cc0, int& LL) {
    it = __builtin_amdgcn_readfirstlane(it);  // wave-uniform: scalar math and loads
    if constexpr (FUSED) {
      // one sequence: chunk it / hx of head xcd + 8 (it % hx), first to last
      const int ch = it / fz.hx;
      hh = fz.xcd + 8 * (it - ch * fz.hx);
      gg = ch;
      int64_t bos, eos;
      seq_bounds(map, 0, bos, eos);
      cc0 = bos + (int64_t)ch * CH;
      LL = (int)((eos - cc0) < CH ? (eos - cc0) : CH);
      return;
    }
    // chunks are produced last to first: the consumer starts at chunk 0, whose
    // records are then the most recently written (likeliest still in cache)
    hh = it % H;
    gg = nchunk - 1 - it / H;
    int nn;
    if (map.cu) {
      nn = chunk_owner(map, gg);
    } else {
      // 32-bit division by an opaque divisor: recomputed per item rather
      // than a reciprocal hoisted out of the item loop
      int nch = (int)((map.T + CH - 1) / CH);
      asm volatile("" : "+s"(nch));
      nn = (int)gg / nch;
    }
    int64_t bos, eos;
    seq_bounds(map, nn, bos, eos);
    cc0 = bos + (gg - first_chunk(map, nn)) * CH;
    LL = (int)((eos - cc0) < CH ? (eos - cc0) : CH);
  };
  // Loads of one item in two parts (P = 0: q and k; P = 1: raw gate, beta,
  // dt_bias, A_log), so that the next item's prefetch is spread over two
  // phases.  Lane offsets come from an opaque thread id: nothing lane-derived
  // stays live across the item loop.  A_log is read with an index the
  // compiler cannot prove uniform, so it is a vector load (a scalar load would
  // share its wait counter with every LDS access in between).
  auto issue = [&](int part, int it, int hh, int64_t cc0, int LL) {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const int tok = 16 * (((t >> 6) + it) & 3) + (t & 15);  // sub-chunk role of item `it`
    const int grp = (t >> 4) & 3;
    const int64_t trow = (cc0 + (tok < LL ? tok : LL - 1)) * H + hh;
    if (part == 0) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int64_t off = trow * KIN + 32 * kb + 8 * grp;
        if (32 * kb < KIN) {
          pq[kb] = *reinterpret_cast<const uint4*>(a.q + off);
          pk[kb] = *reinterpret_cast<const uint4*>(a.k + off);
        } else {
          pq[kb] = make_uint4(0u, 0u, 0u, 0u);
          pk[kb] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    } else {
      braw16 = a.beta[trow];
      alog = A_log[hh + (t >> 31)];
      const int ch = t & (KD - 1);
      dtb = a.dt_bias[hh * KIN + (ch & (KIN - 1))];
      if (KIN < KD && ch >= KIN) dtb = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int64_t off = trow * KIN + 32 * kb + 8 * grp;
        if (32 * kb < KIN)
          pg[kb] = *reinterpret_cast<const uint4*>(a.g + off);
        else
          pg[kb] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  int h, L;
  int64_t g, c0;
  locate(item, h, g, c0, L);
  issue(1, item, h, c0, L);
  issue(0, item, h, c0, L);
  // Wait for the first item's loads here, once.  On the loop's back edge the
  // prefetched loads are followed by the record stores; without this wait the
  // entry path (no stores after its loads) makes the compiler's merged wait at
  // the loop head a full vmcnt(0), which would also wait for every record
  // store of the previous item to complete.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) only
  KDA_TIMER_DECL

  for (;;) {
  // Lane-derived indices are re-derived from an opaque copy of the thread id
  // every item, so the compiler recomputes the (cheap) per-lane addresses in
  // the body instead of hoisting dozens of them out of the loop into spills.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  // Sub-chunk role of this wave for this item.  The roles rotate from item
  // to item: the A blocks of sub-chunk w cost w + 1 block products and the
  // off-diagonal T blocks 3 - w, so a fixed role would load the SIMDs
  // unevenly.
  const int w = ((tid >> 6) + item) & 3;
  const int lane = tid & 63;
  const int tl = lane & 15;
  const int gq = lane >> 4;
  const int ti = 16 * w + tl;  // this lane's token within the chunk
  KDA_TIMER_MARK(0);
  // Fused: a ring slot once every chain of the head has moved past the slot's
  // previous chunk (consumed >= g - R + 1), waited for at most slot_wait
  // polls; else the record's own place in recs.  One thread decides (before
  // the sNB barrier below, shared through LDS), so that every wave writes the
  // record to the same place.
  if constexpr (FUSED) {
    if (threadIdx.x == 0) {
      const __amdgpu_buffer_rsrc_t cr = buf(fz.consumed, (uint32_t)(fz.H * FUSED_CHAINS * FUSED_LINE));
      int dest = 2;
      for (int spin = 0;; ++spin) {
        int done = 0x7fffffff;
#pragma unroll
        for (int c = 0; c < FUSED_CHAINS; ++c) {
          const int d = __builtin_amdgcn_raw_buffer_load_b32(cr, 0, (h * FUSED_CHAINS + c) * FUSED_LINE, SC1);
          done = d < done ? d : done;
        }
        if (g < (int64_t)done + fz.ring) {
          dest = 1;
          break;
        }
        if (spin >= fz.slot_wait) break;
        __builtin_amdgcn_s_sleep(8);
        asm volatile("" ::: "memory");
      }
      sDest[0] = dest;
    }
  }
  char* rec = recs + ((size_t)g * H + h) * REC_BYTES;
  _Float16 *gNW, *gQG, *gKTH, *gKTL, *gAQK;
  __bf16 *gTBH, *gTBL;
  float* gGL;
  const bool valid = ti < L;
  // claim the item after next (the value is shared before the operands barrier)
  int claimed = 0;
  if (threadIdx.x == 0) claimed = atomicAdd(claim, 1);
  // the next item's place (scalar table lookups, overlapped with this item)
  const bool more = next < items;
  int h2, L2;
  int64_t g2, c02;
  if (more)
    locate(next, h2, g2, c02, L2);
  else {
    h2 = h; g2 = g; c02 = c0; L2 = L;
  }

  // gate: sigmoid(x) = 1 / (1 + 2^(raw * na + nb_c)), na = -exp(A_log) log2(e)
  const float na = -__expf(alog) * LOG2E;
  if (tid < KD) sNB[tid] = na * dtb;
  __syncthreads();  // sNB
  KDA_TIMER_MARK(1);
  int dest = 2;
  if constexpr (FUSED) {
    dest = __builtin_amdgcn_readfirstlane(sDest[0]);
    if (dest == 1) rec = fz.ringbuf + ((size_t)h * fz.ring + (size_t)(g % fz.ring)) * REC_BYTES;
  }
  gNW = reinterpret_cast<_Float16*>(rec + REC_NW);
  gQG = reinterpret_cast<_Float16*>(rec + REC_QG);
  gKTH = reinterpret_cast<_Float16*>(rec + REC_KTH);
  gKTL = reinterpret_cast<_Float16*>(rec + REC_KTL);
  gAQK = reinterpret_cast<_Float16*>(rec + REC_AQK);
  gTBH = reinterpret_cast<__bf16*>(rec + REC_TBH);
  gTBL = reinterpret_cast<__bf16*>(rec + REC_TBL);
  gGL = reinterpret_cast<float*>(rec + REC_GL);

  // ============================ prep ======================================
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
  // sums over the 4 lanes (gq) that share the token: lane ^ 16, lane ^ 32
  auto xor_lane = [&](float v, int m) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __float_as_int(v)));
  };
  ssq += xor_lane(ssq, 16);
  ssq += xor_lane(ssq, 32);
  ssk += xor_lane(ssk, 16);
  ssk += xor_lane(ssk, 32);
  const bool qk_norm = !(a.flags & FLAG_NO_QK_NORM);
  // without the in-kernel norm the caller keeps |q|, |k| <= 1 (the fp16
  // operands assume unit scale); a row beyond that is recorded, not rejected
  if (!qk_norm && __any(valid && (ssq > 1.0625f || ssk > 1.0625f)) && lane == 0)
    atomicOr(a.faults, FAULT_QK_NORM);
  const float rq = valid ? (qk_norm ? __builtin_amdgcn_rsqf(ssq + L2_EPS) : 1.0f) : 0.0f;
  const float rk = valid ? (qk_norm ? __builtin_amdgcn_rsqf(ssk + L2_EPS) : 1.0f) : 0.0f;
  const float braw = __uint_as_float((uint32_t)braw16 << 16);
  const float beta =
      valid ? ((a.flags & FLAG_BETA_GIVEN) ? braw : __builtin_amdgcn_rcpf(1.0f + fexp2(-braw * LOG2E))) : 0.0f;

  // a given decay outside [lower_bound, 0] is outside the call's contract: it
  // is recorded in the fault word (and saturated below, so every decay ratio
  // stays in range)
  if constexpr (GATE_GIVEN) {
    bool bad = false;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) bad |= !(gl[kb][e] >= a.lb && gl[kb][e] <= 0.0f);
    if (__any(valid && bad) && lane == 0) atomicOr(a.faults, FAULT_GATE_RANGE);
  }
  // log-decay in log2 units, inclusive scan over the sub-chunk's 16 tokens
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    float nb[8];
    lds_f32x8(sNB + 32 * kb + 8 * gq, nb);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // log2 decay: lb2 * sigmoid(exp(A_log)(raw + dt)), or the given natural-log
      // decay clamped to [lower_bound, 0]
      float g2 = GATE_GIVEN ? fminf(fmaxf(gl[kb][e] * LOG2E, a.lb2), 0.0f)
                            : a.lb2 * __builtin_amdgcn_rcpf(1.0f + fexp2(gl[kb][e] * na + nb[e]));
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
  KDA_TIMER_MARK(2);
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
    rec_store<NT>(&gGL[tid], fexp2(P[4]));
  }
  __syncthreads();
  KDA_TIMER_MARK(3);

  // ============================ operands ==================================
  bf16x8 kLFh[4], kLFl[4], kEh[4], kEl[4], qLF[4];
  // identity B operands: idt[s] selects channels 16s..16s+15 of a 32-channel
  // k-block, so that an A fragment [16 tokens][32 channels] comes out of the
  // MFMA transposed (lane: 4 consecutive tokens of one channel)
  f16x8 idt[2];
#pragma unroll
  for (int sv = 0; sv < 2; ++sv)
#pragma unroll
    for (int e = 0; e < 8; ++e) idt[sv][e] = (_Float16)((8 * gq + e == 16 * sv + tl) ? 1.0f : 0.0f);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    float ET[8], EP[8], EL[8], qf[8], kf[8];
    lds_f32x8(sFac + (FAC_ET + w) * KD + 32 * kb + 8 * gq, ET);
    lds_f32x8(sFac + (FAC_EP + w) * KD + 32 * kb + 8 * gq, EP);
    lds_f32x8(sFac + (FAC_EL + w) * KD + 32 * kb + 8 * gq, EL);
    unpack_bf16x8(pq[kb], qf);
    unpack_bf16x8(pk[kb], kf);
    bf16x8 krh, krl;
    f16x8 qg, kg8, kth8, ktl8;
    float xv[8], yv[8], qv[8], rv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float Gl = gl[kb][e];
      const float LF = fexp2(Gl);   // exp(G_t - P_w) <= 1
      const float E = fexp2(-Gl);   // exp(P_w - G_t) in [1, 2^116]
      const float kn = kf[e] * rk;
      const float qn = qf[e] * rq;
      xv[e] = kn * LF;
      yv[e] = kn * E;
      qv[e] = qn * LF;
      rv[e] = yv[e] * ET[e];                        // k^ exp(P_{w+1} - G_t), |.| <= |k^|
      kg8[e] = (_Float16)(xv[e] * EP[e]);           // k^ exp(G_t)
      const float kt = yv[e] * EL[e];               // k^ exp(G_L - G_t)
      const _Float16 kth = (_Float16)kt;
      kth8[e] = kth;
      ktl8[e] = (_Float16)((kt - (float)kth) * KT_LO_SCALE);
      qg[e] = (_Float16)(qv[e] * EP[e]);            // q^ exp(G_t)
    }
    split_bf16x8(xv, kLFh[kb], kLFl[kb]);
    split_bf16x8(yv, kEh[kb], kEl[kb]);
    qLF[kb] = to_bf16x8(qv);
    split_bf16x8(rv, krh, krl);
    rec_store<NT>(reinterpret_cast<f16x8*>(gQG + frag_tc(ti, 32 * kb + 8 * gq)), qg);
    // (K^ exp(G_L - G))^T hi/lo and (K^ exp(G))^T: f16 x 1 products summed in
    // fp32 are exact, so these transposes are exact
#pragma unroll
    for (int sv = 0; sv < 2; ++sv) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 th = mfma_f16(kth8, idt[sv], zero);
      const f32x4 tlo = mfma_f16(ktl8, idt[sv], zero);
      const f32x4 tg = mfma_f16(kg8, idt[sv], zero);
      const int cc = 32 * kb + 16 * sv + tl;  // lane: channel cc, tokens 16w + 4gq + 0..3
      const f16x4 h4 = {(_Float16)th[0], (_Float16)th[1], (_Float16)th[2], (_Float16)th[3]};
      const f16x4 l4 = {(_Float16)tlo[0], (_Float16)tlo[1], (_Float16)tlo[2], (_Float16)tlo[3]};
      const f16x4 g4 = {(_Float16)tg[0], (_Float16)tg[1], (_Float16)tg[2], (_Float16)tg[3]};
      rec_store<NT>(reinterpret_cast<f16x4*>(gKTH + frag_ct(cc, 16 * w + 4 * gq)), h4);
      rec_store<NT>(reinterpret_cast<f16x4*>(gKTL + frag_ct(cc, 16 * w + 4 * gq)), l4);
      *reinterpret_cast<f16x4*>(sKG + cc * TP + 16 * w + 4 * gq) = g4;
    }
    if (w < 3) {
      *reinterpret_cast<bf16x8*>(sKRFh + ti * KP + 32 * kb + 8 * gq) = krh;
      *reinterpret_cast<bf16x8*>(sKRFl + ti * KP + 32 * kb + 8 * gq) = krl;
    }
  }
  if (threadIdx.x == 0) *sClaim = claimed;
  __syncthreads();
  KDA_TIMER_MARK(4);
  const int next2 = __builtin_amdgcn_readfirstlane(*sClaim) + 2 * stride;

  // Wait until tag `t` holds this item (release/acquire on the LDS tag word).
  // Tags 0-3 and 5 are published with no wait before them, and tag 6 only
  // after tag 5, so every wait ends; the spin is bounded all the same, and a
  // wait that gives up marks the call's results invalid in the fault word.
  auto wait_tag = [&](int t) {
    for (int spin = 0;; ++spin) {
      if (__hip_atomic_load(&sFlag[t], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == item) break;
      if (spin == (1 << 22)) {
        if (lane == 0) atomicOr(a.faults, FAULT_WAIT_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  };
  auto publish = [&](int t) { __hip_atomic_store(&sFlag[t], item, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP); };
  // T_bb = (I + A_bb)^-1 of diagonal block blk, in place, by forward
  // substitution: lane cc < 16 owns column cc.  The block's lower triangle is
  // read into registers first (36 16-byte reads), so the substitution chain
  // never waits on LDS.
  auto diag_inverse = [&](int blk) {
    if (lane < 16) {
      const int cc = lane;
      const float* Ab = sA + (16 * blk) * AP + 16 * blk;
      float Ar[16][16];
#pragma unroll
      for (int i = 1; i < 16; ++i)
#pragma unroll
        for (int m4 = 0; m4 < i; m4 += 4) {
          const float4 v4 = *reinterpret_cast<const float4*>(Ab + i * AP + m4);
          Ar[i][m4] = v4.x; Ar[i][m4 + 1] = v4.y; Ar[i][m4 + 2] = v4.z; Ar[i][m4 + 3] = v4.w;
        }
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = (i == cc) ? 1.0f : 0.0f;
#pragma unroll
        for (int m = 0; m < i; ++m) s -= Ar[i][m] * x[m];
        x[i] = (i < cc) ? 0.0f : s;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sA[(16 * blk + i) * AP + 16 * blk + cc] = x[i];
    }
  };

  // ======================= A_kk and A_qk ==================================
  // wave w owns row-block w; lane holds C[16w + 4gq + ii][16b + tl].  The
  // diagonal block comes first: row-block 3 publishes it at once, and the
  // role-0 wave, whose own A work is one block, inverts it while row-block 3
  // computes its three off-diagonal blocks.
  {
    const int i0 = 16 * w + 4 * gq;
    // beta of this lane's four rows, read once (not inside the masked stores)
    const float4 bi4 = *reinterpret_cast<const float4*>(sB + i0);
    const float bi[4] = {bi4.x, bi4.y, bi4.z, bi4.w};
#pragma unroll 1
    for (int it = 0; it <= w; ++it) {
      const int b = it == 0 ? w : it - 1;
      f32x4 akk = {0.f, 0.f, 0.f, 0.f};
      f32x4 aqk = {0.f, 0.f, 0.f, 0.f};
      if (b == w) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          akk = mfma_bf16(kLFh[kb], kEh[kb], akk);
          akk = mfma_bf16(kLFh[kb], kEl[kb], akk);
          akk = mfma_bf16(kLFl[kb], kEh[kb], akk);
          aqk = mfma_bf16(kEh[kb], qLF[kb], aqk);  // transposed tile
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
              const float x = ((float)kLFh[kb][e] + (float)kLFl[kb][e]) * f[e];
              const __bf16 xh = (__bf16)x;
              lh[e] = xh;
              ll[e] = (__bf16)(x - (float)xh);
              lq[e] = (__bf16)((float)qLF[kb][e] * f[e]);
            }
          }
          akk = mfma_bf16(lh, rh, akk);
          akk = mfma_bf16(lh, rl, akk);
          akk = mfma_bf16(ll, rh, akk);
          aqk = mfma_bf16(rh, lq, aqk);  // transposed tile
        }
      }
      // operands are L2-normalised: only beta_i scales the rows of A_kk
      const int j = 16 * b + tl;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = i0 + ii;
        sA[i * AP + j] = (j < i) ? akk[ii] * bi[ii] : 0.0f;
      }
      // A_qk came out transposed: lane holds row 16w + tl, columns 16b + 4gq + 0..3
      f16x4 q4;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) q4[ii] = (_Float16)((16 * b + 4 * gq + ii <= ti) ? aqk[ii] : 0.0f);
      rec_store<NT>(reinterpret_cast<f16x4*>(gAQK + frag_tt(ti, 16 * b + 4 * gq)), q4);
      if (w == 3 && it == 0) publish(5);  // A_33
    }
    // zero blocks above the diagonal; rows 0..31 skip tokens 32..63, a whole
    // record fragment that the reader never loads
    for (int b = w + 1; b < (w < 2 ? 2 : 4); ++b) {
      const f16x4 z4 = {(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
      rec_store<NT>(reinterpret_cast<f16x4*>(gAQK + frag_tt(ti, 16 * b + 4 * gq)), z4);
    }
    // T_ww for w < 3 (T_33 is the role-0 wave's, below).  This wave wrote A_ww
    // above and LDS operations of one wave complete in order.
    if (w < 3) diag_inverse(w);
  }
  // Publish row-block w.  LDS operations of one wave complete in order and the
  // release orders the tag after them.
  publish(w);
  if (w == 0) {
    wait_tag(5);
    diag_inverse(3);
    publish(6);
  }
  // The A operands of this item are dead: start the next item's loads (the
  // last item re-reads its own, so every path has the same loads in flight).
  issue(0, more ? next : item, h2, c02, L2);
  KDA_TIMER_MARK(5);

  // ======= T column-block by column-block, and T diag(b) from registers =====
  //     T_{b,w} = -T_bb * sum_{m=w}^{b-1} A_{b,m} T_{m,w}   (fp32 MFMA)
  // Wave w walks down its own column-block.  The blocks T_{m,w} it needs are
  // its own earlier results, kept in registers in C layout (which is the
  // B-operand layout); the A blocks of row-block b are final once tag b is
  // published, and T_bb with it (T_33 with tag 6).  So no barrier separates
  // this phase from the A phase or its levels from each other: the A work
  // grows with the row index and this work with the column index, and the two
  // overlap.  Instruction s of a block product contracts over index 4gq + s:
  // a lane's four A-operand values of one row are a single 16-byte LDS read.
  //
  // Each block is also formed transposed, T_{b,w}^T = X^T (-T_bb^T), whose C
  // layout gives a lane four consecutive columns 16w + 4gq + 0..3 of row
  // 16b + tl.  T diag(b) is formed from that right away: bf16 hi/lo 8-byte
  // stores to the record, fp16 hi/lo kept in registers for the LDS copy that
  // W reads (written after the barrier below, because that region still holds
  // the A-phase right factors).  Odd waves also own the all-zero upper block
  // (w - 1, w) that the readers of rows 0..15 and 32..47 load.
  {
    const float4 bj4 = *reinterpret_cast<const float4*>(sB + 16 * w + 4 * gq);
    const float bj[4] = {bj4.x, bj4.y, bj4.z, bj4.w};
    f16x4 tbh16[5], tbl16[5];
    auto emit = [&](int b, const f32x4& tt, f16x4& h16, f16x4& l16) {
      const int i = 16 * b + tl;
      float t[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = 16 * w + 4 * gq + ii;
        t[ii] = (j < i) ? tt[ii] * bj[ii] : ((j == i) ? bj[ii] : 0.0f);
        const _Float16 hv = (_Float16)t[ii];
        h16[ii] = hv;
        l16[ii] = (_Float16)(t[ii] - (float)hv);
      }
      uint32_t hb[2], lb[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const f32x2 v = {t[2 * p], t[2 * p + 1]};
        hb[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
        const f32x2 r = {t[2 * p] - __uint_as_float(hb[p] << 16), t[2 * p + 1] - __uint_as_float(hb[p] & 0xffff0000u)};
        lb[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
      }
      rec_store<NT>(reinterpret_cast<u32x2*>(gTBH + frag_tt(i, 16 * w + 4 * gq)), u32x2{hb[0], hb[1]});
      rec_store<NT>(reinterpret_cast<u32x2*>(gTBL + frag_tt(i, 16 * w + 4 * gq)), u32x2{lb[0], lb[1]});
    };
    if (w == 3) wait_tag(6);
    f32x4 Tc[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) Tc[0][ii] = sA[(16 * w + 4 * gq + ii) * AP + 16 * w + tl];
    {
      const float4 d4 = *reinterpret_cast<const float4*>(sA + (16 * w + tl) * AP + 16 * w + 4 * gq);
      emit(w, f32x4{d4.x, d4.y, d4.z, d4.w}, tbh16[0], tbl16[0]);
    }
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      Tc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (w + d < 4) {
        const int b = w + d;
        wait_tag(b);
        if (b == 3) wait_tag(6);
        const float* arow = sA + (16 * b + tl) * AP + 4 * gq;
        f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mm = 0; mm < d; ++mm) {
          const float4 a4 = *reinterpret_cast<const float4*>(arow + 16 * (w + mm));
          X = mfma_f32(a4.x, Tc[mm][0], X);
          X = mfma_f32(a4.y, Tc[mm][1], X);
          X = mfma_f32(a4.z, Tc[mm][2], X);
          X = mfma_f32(a4.w, Tc[mm][3], X);
        }
        const float4 t4 = *reinterpret_cast<const float4*>(arow + 16 * b);
        f32x4 r = {0.f, 0.f, 0.f, 0.f};
        r = mfma_f32(-t4.x, X[0], r);
        r = mfma_f32(-t4.y, X[1], r);
        r = mfma_f32(-t4.z, X[2], r);
        r = mfma_f32(-t4.w, X[3], r);
        Tc[d] = r;
        f32x4 tt = {0.f, 0.f, 0.f, 0.f};
        tt = mfma_f32(X[0], -t4.x, tt);
        tt = mfma_f32(X[1], -t4.y, tt);
        tt = mfma_f32(X[2], -t4.z, tt);
        tt = mfma_f32(X[3], -t4.w, tt);
        emit(b, tt, tbh16[d], tbl16[d]);
      }
    }
    if (w & 1) emit(w - 1, f32x4{0.f, 0.f, 0.f, 0.f}, tbh16[4], tbl16[4]);
    KDA_TIMER_MARK(6);
    issue(1, more ? next : item, h2, c02, L2);
    __syncthreads();  // every wave is done with the A phase's right factors
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (w + d < 4) {
        const int i = 16 * (w + d) + tl;
        *reinterpret_cast<f16x4*>(sTbh + i * TBP + 16 * w + 4 * gq) = tbh16[d];
        *reinterpret_cast<f16x4*>(sTbl + i * TBP + 16 * w + 4 * gq) = tbl16[d];
      }
    }
    if (w & 1) {
      const int i = 16 * (w - 1) + tl;
      *reinterpret_cast<f16x4*>(sTbh + i * TBP + 16 * w + 4 * gq) = tbh16[4];
      *reinterpret_cast<f16x4*>(sTbl + i * TBP + 16 * w + 4 * gq) = tbl16[4];
    }
    __syncthreads();
  }
  KDA_TIMER_MARK(7);

  // ======================= -W = -(T diag(b)) (K^ exp(G)) ===================
  // wave w: channels 32w..32w+31 (2 column tiles), all 64 rows; the tiles are
  // computed transposed so that each lane stores 4 consecutive channels
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks == 1 && m < 2) continue;  // T is lower triangular
      const int arow = (16 * m + tl) * TBP + 32 * ks + 8 * gq;
      const f16x8 th = *reinterpret_cast<const f16x8*>(sTbh + arow);
      const f16x8 tlo = *reinterpret_cast<const f16x8*>(sTbl + arow);
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        const int ch = 32 * w + 16 * nn + tl;
        const f16x8 kg = *reinterpret_cast<const f16x8*>(sKG + ch * TP + 32 * ks + 8 * gq);
        acc[nn] = mfma_f16(kg, th, acc[nn]);   // transposed tile
        acc[nn] = mfma_f16(kg, tlo, acc[nn]);
      }
    }
    // lane: row 16m + tl, channels 32w + 16nn + 4gq + 0..3
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const f16x4 w4 = {(_Float16)(-acc[nn][0]), (_Float16)(-acc[nn][1]), (_Float16)(-acc[nn][2]),
                        (_Float16)(-acc[nn][3])};
      rec_store<NT>(reinterpret_cast<f16x4*>(gNW + frag_tc(16 * m + tl, 32 * w + 16 * nn + 4 * gq)), w4);
    }
  }
  KDA_TIMER_MARK(8);
  if constexpr (FUSED) {
    // publish: every wave's record stores have completed (reached L2) before
    // the ready flag is written (it holds where the record went)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0)
      __builtin_amdgcn_raw_buffer_store_b32(dest, buf(fz.flags, (uint32_t)fz.nchunk * fz.H * 4), 0,
                                            (int)(g * H + h) * 4, SC1);
    if (!more) break;
  } else {
    if (!more) break;
    __syncthreads();  // LDS of this item is read above until the W phase
  }
  item = next;
  next = next2;
  h = h2; g = g2; c0 = c02; L = L2;
  KDA_TIMER_MARK(9);
  }
  KDA_TIMER_STORE(a.timers);
}

namespace {

template <bool GATE_GIVEN, int KIN, bool NT>
__global__ void __launch_bounds__(NTHREADS, 2)
    kda_intra_kernel(IntraArgs a, const int32_t* __restrict__ cu, const int32_t* __restrict__ choff,
                     const float* __restrict__ A_log, char* __restrict__ recs) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  const IntraFused none{};
  intra_items<GATE_GIVEN, false, KIN, NT>(a, cu, choff, A_log, recs, smem, (int)blockIdx.x, (int)gridDim.x,
                                          a.claim, none);
}

}  // namespace

namespace {

constexpr int FUSED_NQ = 2;  // chain workgroups own 64-column halves
constexpr int FUSED_LDS =
    LDS_BYTES > chain::Lay<FUSED_NQ>::LDS_BYTES ? LDS_BYTES : chain::Lay<FUSED_NQ>::LDS_BYTES;
static_assert(FUSED_CHAINS * 32 * FUSED_NQ == VD, "chains cover the state columns");
constexpr int HW_REG_XCC_ID = (3 << 11) | 20;  // s_getreg operand: XCC_ID, bits 0-3

// Clears the fused pipeline's ready flags, consumed and claim counters, the
// XCD-of-residue words and the call's fault word (a kernel rather than a memset, so that a captured
// graph replays it as a kernel node).
__global__ void kda_fused_reset_kernel(int* __restrict__ flags, int nflags, int* __restrict__ consumed, int H,
                                       int* __restrict__ claims, unsigned* __restrict__ faults) {
  const int stride = (int)(gridDim.x * blockDim.x);
  const int i0 = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  for (int i = i0; i < nflags; i += stride) flags[i] = 0;
  for (int i = i0; i < H * FUSED_CHAINS; i += stride) consumed[i * (FUSED_LINE / 4)] = 0;
  if (i0 < 8) claims[i0 * (FUSED_LINE / 4)] = 0;                  // claim counters
  if (i0 < 8) claims[(8 + i0) * (FUSED_LINE / 4)] = -1;           // XCD of each id residue: none yet
  if (i0 == 0) *faults = 0u;
}

// The fused pipeline over one sequence.  The dispatcher hands workgroups to
// the 8 XCDs round robin, so the workgroups b = 8 j + x of one residue x all
// run on one XCD, though not necessarily XCD x (under graph replay the round
// robin starts elsewhere): residue x, local workgroup j of nw = grid / 8, owns
// heads x, x + 8, ... (hx of them).  Its last FUSED_CHAINS hx workgroups are
// their chains (highest ids, so dispatched last; the two column halves of a
// head are neighbours), the others intra-chunk producers of those heads'
// items in chunk order; all of them meet in the one XCD's L2.  Each workgroup
// records the XCD (XCC_ID register) of its residue; one that finds its residue
// on another XCD reports KDA_FAULT_PLACEMENT (records may then have crossed
// XCDs).
// A producer waits for a chain only a bounded time (a record whose ring slot
// is still in use after FusedArgs::slot_wait polls goes to the record area
// instead), so all items get produced whatever the residency, and every
// chain's waits end.
template <bool GATE_GIVEN>
__global__ void __launch_bounds__(NTHREADS, 2)
    kda_fused_kernel(IntraArgs ia, ChainArgs ca, FusedArgs fa, const float* __restrict__ A_log,
                     char* __restrict__ recs) {
  __shared__ __attribute__((aligned(16))) char smem[FUSED_LDS];
  const int x = (int)(blockIdx.x & 7);
  const int j = (int)(blockIdx.x >> 3);
  const int nw = (int)(gridDim.x >> 3);
  if (threadIdx.x == 0) {
    const int xr = (int)(__builtin_amdgcn_s_getreg(HW_REG_XCC_ID) & 7);
    const int seen = atomicCAS(fa.claims + (8 + x) * (FUSED_LINE / 4), -1, xr);
    if (seen != -1 && seen != xr) atomicOr(fa.faults, FAULT_PLACEMENT);
  }
  const int H = ia.H;
  const int hx = x < H ? (H - 1 - x) / 8 + 1 : 0;
  const int nchains = FUSED_CHAINS * hx;
  if (j >= nw - nchains) {
    const int c = nw - 1 - j;  // FUSED_CHAINS l + half
    const int l = c / FUSED_CHAINS;
    const int half = c - FUSED_CHAINS * l;
    const int h = x + 8 * l;
    ChainFused cf;
    cf.ringbuf = fa.ringbuf;
    cf.ring = fa.ring;
    cf.flags = fa.flags;
    cf.consumed = fa.consumed + (h * FUSED_CHAINS + half) * (FUSED_LINE / 4);
    cf.faults = fa.faults;
    cf.nchunk = fa.nchunk;
    chain::chain_run<true, FUSED_NQ>(ca, cf, 0, h, 32 * FUSED_NQ * half, smem);
  } else {
    IntraFused f;
    f.xcd = x;
    f.hx = hx;
    f.ring = fa.ring;
    f.slot_wait = fa.slot_wait;
    f.ringbuf = fa.ringbuf;
    f.consumed = fa.consumed;
    f.flags = fa.flags;
    f.H = H;
    f.nchunk = fa.nchunk;
    intra_items<GATE_GIVEN, true>(ia, nullptr, nullptr, A_log, recs, smem, j, nw - nchains,
                                  fa.claims + x * (FUSED_LINE / 4), f);
  }
}

}  // namespace

hipError_t launch_fused(const IntraArgs& iargs, const ChainArgs& cargs, const FusedArgs& fargs, hipStream_t st) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  IntraArgs ia = iargs;
  ChainArgs ca = cargs;
  FusedArgs fa = fargs;
  int nflags = fa.nchunk * ia.H, H = ia.H;
  void* rargs[] = {(void*)&fa.flags, (void*)&nflags, (void*)&fa.consumed, (void*)&H, (void*)&fa.claims,
                   (void*)&fa.faults};
  e = hipLaunchKernel(reinterpret_cast<const void*>(&kda_fused_reset_kernel), dim3(64), dim3(256), rargs, 0, st);
  if (e != hipSuccess) return e;
  const float* alog = ia.A_log;
  char* recs = ia.rec;
  void* kargs[] = {(void*)&ia, (void*)&ca, (void*)&fa, (void*)&alog, (void*)&recs};
  const void* fn = (ia.flags & FLAG_GATE_GIVEN) ? reinterpret_cast<const void*>(&kda_fused_kernel<true>)
                                                : reinterpret_cast<const void*>(&kda_fused_kernel<false>);
  // two workgroups per CU: all of them resident at once on an idle GPU
  return hipLaunchKernel(fn, dim3((unsigned)(2 * cus)), dim3(NTHREADS), kargs, 0, st);
}

// Record areas up to this size are written with plain stores and stay in the
// 256 MB Infinity Cache until the inter kernel reads them; larger ones would
// only evict each other and go out non-temporally.
constexpr size_t kRecordsCachedBytes = (size_t)160 << 20;

hipError_t launch_intra(const IntraArgs& args, int64_t max_chunks, hipStream_t st) {
  // persistent grid: two resident workgroups per CU (LDS and register budget)
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t items = max_chunks * args.H;
  const int64_t grid = items < 2 * (int64_t)cus ? items : 2 * (int64_t)cus;
  if (grid <= 0) return hipSuccess;
  IntraArgs a = args;
  const int32_t* cu = a.map.cu;
  const int32_t* choff = a.map.choff;
  const float* alog = a.A_log;
  char* recs = a.rec;
  void* kargs[] = {(void*)&a, (void*)&cu, (void*)&choff, (void*)&alog, (void*)&recs};
  const bool given = a.flags & FLAG_GATE_GIVEN;
  // records that fit the Infinity Cache are stored plainly, larger areas non-temporally
  const bool nt = (size_t)items * REC_BYTES > kRecordsCachedBytes;
  const void* fn;
  if (a.kd == KD)
    fn = given ? (nt ? reinterpret_cast<const void*>(&kda_intra_kernel<true, KD, true>)
                     : reinterpret_cast<const void*>(&kda_intra_kernel<true, KD, false>))
               : (nt ? reinterpret_cast<const void*>(&kda_intra_kernel<false, KD, true>)
                     : reinterpret_cast<const void*>(&kda_intra_kernel<false, KD, false>));
  else
    fn = given ? (nt ? reinterpret_cast<const void*>(&kda_intra_kernel<true, 64, true>)
                     : reinterpret_cast<const void*>(&kda_intra_kernel<true, 64, false>))
               : (nt ? reinterpret_cast<const void*>(&kda_intra_kernel<false, 64, true>)
                     : reinterpret_cast<const void*>(&kda_intra_kernel<false, 64, false>));
  return hipLaunchKernel(fn, dim3((unsigned)grid),
                         dim3(NTHREADS), kargs, 0, st);
}

}  // namespace kda
