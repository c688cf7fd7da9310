// Host-side pieces of the forward launch sequence (kda_api.hip) that the
// backward entry point (kda_bwd.hip) reuses.  Internal: not part of the C ABI.
#pragma once

#include "../../include/kda.h"
#include "kda_common.h"

namespace kda {

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// A forward with few (sequence, head) chains and long sequences runs its
// recurrence on shards: each of the N sequences is cut into S shards of cs
// whole chunks, the per-shard affine maps S -> P S + R are folded, and the
// forward runs over the shards from the folded entering states.  Three passes
// over chains S times shorter, on S times more workgroups.  Only without
// cu_seqlens, where the host knows every length (T per sequence).
constexpr int64_t kSplitChains = 128;   // aim: about this many (shard, head) chains
constexpr int64_t kMinShardChunks = 32;  // shards of at least 2048 tokens
constexpr int64_t kMinShards = 4;        // below 4 shards the three passes do not pay
struct SplitPlan {
  int64_t S;   // shards per sequence (1: no split)
  int64_t cs;  // chunks per shard (the last one of a sequence may be shorter)
};
inline SplitPlan split_plan(int64_t T, int64_t H, int64_t N) {
  const int64_t nc = (T + CH - 1) / CH;
  if (T <= 0 || H < 1 || N < 1) return {1, nc};
  const int64_t a = kSplitChains / (N * H), b = nc / kMinShardChunks;
  const int64_t S = a < b ? a : b;
  if (S < kMinShards) return {1, nc};
  const int64_t cs = (nc + S - 1) / S;
  return {(nc + cs - 1) / cs, cs};
}

// The fused pipeline (one launch of intra-chunk producers and per-head
// chains, records handed over through a ring in L2) serves calls with one
// sequence and at least this many heads (two per XCD).
constexpr int64_t kFusedMinHeads = 16;

struct Layout {
  size_t claim, faults, choff, order, rec, base, total;  // base: end of the records
  // shard areas (split forwards only): shard offsets in tokens and in chunks
  // [N S + 1], and the per-shard P, R, entering and final states
  int64_t S;
  size_t scu, schoff, sP, sR, sstart, sfin;
  // fused-pipeline areas (N == 1, H >= kFusedMinHeads): the ring of
  // FUSED_RING records per head, ready flags [chunks][H], consumed counters
  // [H][FUSED_CHAINS], per-XCD claim counters [8] and the XCD of each id residue [8]
  // (FUSED_LINE apart)
  bool fused;
  size_t fring, fflags, fcons, fclaims;
};

// T_total / N is the per-sequence length the split plan assumes (the mean
// length of a varlen call, whose shards follow each sequence's own length).
inline Layout workspace_layout(int64_t T_total, int64_t H, int64_t N) {
  Layout l;
  l.claim = 0;   // the intra kernel's work-item counter (one int)
  l.faults = 4;  // the call's fault word (FAULT_* bits)
  l.choff = 256;
  l.order = l.choff + align256((size_t)(N + 1) * sizeof(int32_t));
  l.rec = l.order + align256((size_t)N * sizeof(int32_t));
  const size_t max_chunks = (size_t)(T_total / CH) + (size_t)N;
  l.total = l.rec + max_chunks * (size_t)H * REC_BYTES;
  l.base = l.total;
  l.S = N > 0 ? split_plan(T_total / N, H, N).S : 1;
  l.scu = l.schoff = l.sP = l.sR = l.sstart = l.sfin = l.total;
  if (l.S > 1) {
    const size_t ns = (size_t)(N * l.S), st = ns * (size_t)H * KD * VD * sizeof(float);
    l.scu = align256(l.total);
    l.schoff = l.scu + align256((ns + 1) * sizeof(int32_t));
    l.sP = l.schoff + align256((ns + 1) * sizeof(int32_t));
    l.sR = l.sP + st;  // P is [ns, H, K, K] with K == V
    l.sstart = l.sR + st;
    l.sfin = l.sstart + st;
    l.total = l.sfin + st;
  }
  l.fused = N == 1 && H >= kFusedMinHeads;
  l.fring = l.fflags = l.fcons = l.fclaims = l.total;
  if (l.fused) {
    l.fring = align256(l.total);
    l.fflags = l.fring + (size_t)H * FUSED_RING * REC_BYTES;
    l.fcons = l.fflags + align256(max_chunks * (size_t)H * 4);
    l.fclaims = l.fcons + align256((size_t)H * FUSED_CHAINS * FUSED_LINE);
    l.total = l.fclaims + 16 * FUSED_LINE;
  }
  return l;
}

// The workspace size reported to callers: the largest layout of any call
// with N' <= N sequences over the same T_total tokens, so that one size bought
// for an upper bound on the batch serves every smaller one.  The base part
// (records and tables) grows with N; the shard area does not (it follows the
// mean length), but only N' H <= kSplitChains / kMinShards chains can split,
// so the maximum of the shard area runs over at most 32 values of N'.
inline size_t workspace_bound(int64_t T_total, int64_t H, int64_t N) {
  const Layout l = workspace_layout(T_total, H, N);
  size_t shards = 0;
  const int64_t top = N < kSplitChains / kMinShards ? N : kSplitChains / kMinShards;
  for (int64_t n = 1; n <= top; ++n) {
    const Layout m = workspace_layout(T_total, H, n);
    const size_t a = m.total - m.base;
    if (a > shards) shards = a;
  }
  const size_t bound = l.base + shards;
  return bound > l.total ? bound : l.total;
}

// What the intra-chunk pass of one call leaves for the inter-chunk passes.
struct Prepared {
  ChunkMap map;
  int32_t* order;
  char* rec;
  char* ws;
  Layout lay;
  int64_t max_chunks;
  int kd = KD, vd = VD;  // the call's head dims (64 or 128 each)
  IntraArgs ia;  // the intra-chunk pass's arguments
};

// Argument checks shared by every entry point that runs the chunked forward,
// then the varlen bookkeeping and (run_intra) the intra-chunk kernel on `st`.
kda_status_t prepare(const void* q, const void* k, const void* raw_gate, const void* raw_beta,
                     void* workspace, size_t workspace_bytes, const float* A_log,
                     const float* dt_bias, float lower_bound, const int32_t* cu_seqlens, int64_t B,
                     int64_t T, int64_t H, int64_t K, int64_t V, int64_t N, hipStream_t st,
                     Prepared& pr, unsigned flags = 0, bool run_intra = true);

// Inter-chunk arguments for the prepared call (no v, outputs or states set).
InterArgs inter_args(const Prepared& pr, int64_t H);

// Whether a prepared call runs its recurrence on shards (split_plan of the
// mean sequence length): only with the [K][V] state layout and a token count
// that fits the int32 shard offsets.
inline bool use_split(const Prepared& pr, unsigned flags, int64_t B, int64_t T) {
  // the shard maps P are K x K products started from the identity: K == V == 128
  return pr.lay.S > 1 && !(flags & FLAG_STATE_VK) && T > 0 && B * T < ((int64_t)1 << 31) && pr.kd == KD &&
         pr.vd == VD;
}

// Inter-chunk arguments over the shard map m2 (no v, outputs or states set).
InterArgs shard_inter_args(const Prepared& pr, int64_t H, const ChunkMap& m2);

// After prepare(): the shard map (into m2), the shards' R and P and their
// fold, leaving every shard's entering state at pr.ws + pr.lay.sstart and
// writing final_state (if not NULL; it must not overlap initial_state).
kda_status_t shard_states(const Prepared& pr, const void* v, const float* initial_state, float* final_state,
                          int64_t T, int64_t H, int64_t N, hipStream_t st, ChunkMap& m2);

// The forward's recurrence on shards (split_plan), after prepare().
kda_status_t split_forward(const Prepared& pr, const void* v, void* out, const float* initial_state,
                           float* final_state, float scale, int64_t T, int64_t H, int64_t N, hipStream_t st);

// KDA_SUCCESS, or KDA_ERR_LAUNCH for a failed launch (KDA_DEBUG=1 prints why).
kda_status_t launch_status(hipError_t err, const char* what);

}  // namespace kda
