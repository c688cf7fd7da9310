// Internal declarations of the backward pass (kda_bwd.hip).  Not part of the C ABI.
#pragma once

#include "kda_common.h"

namespace kda {

// Backward pass (kda_bwd.hip).  Per-(chunk, head) buffers are indexed by
// item = global chunk * H + head.
struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;      // raw gate
  const uint16_t* beta;   // raw beta
  const float* A_log;
  const float* dt_bias;
  const uint16_t* dout;   // bf16 [tokens][H][V]
  const float* dfin;      // [N][H][K][V] gradient of the final state, or nullptr
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dg;           // gradient of the raw gate
  uint16_t* dbeta;        // gradient of the raw beta
  float* dinit;           // [N][H][K][V] or nullptr
  float* dA_log;          // [H]
  float* ddt;             // [H][K]
  const float* states;    // [items][K][V] state entering each chunk
  const float* dtile;     // [items][64][V] D of each chunk
  float* dstates;         // [items][K][V] gradient of the state leaving each chunk
  float* ddtile;          // [items][64][V] dD of each chunk
  float* br;              // [items][BWD_REC_FLOATS] fp32 chunk factors
  float* part;            // [items][K + 1] per-chunk partial sums of d dt_bias and dA_log
  const int32_t* order;   // nullptr: identity order of sequences
  ChunkMap map;
  int H;
  int kd, vd;             // head dims of the caller's tensors (64 or 128); the internal layouts keep 128
  float scale;
  float lb;               // lower_bound
  int flags;              // FLAG_GATE_GIVEN | FLAG_BETA_GIVEN | FLAG_NO_QK_NORM | FLAG_STATE_VK
  unsigned long long* timers;  // phase timers (KDA_PHASE_TIMERS builds only), else nullptr
};
constexpr int BWD_REC_FLOATS = 3 * CH * CH + 3 * CH * KD + KD + CH;  // 37056

// The reverse recurrence on shards (sequences of the same length split into
// S shards each, map m2 over the same global chunks): a pass from a zero
// leaving gradient gives each shard's own entering-state gradient B_r (into
// `b`), the reverse fold with the shard maps P (`P`, [N S][H][K][K]) gives
// every shard's leaving gradient (into `ends`) and d_initial_state, and a
// second pass from those writes the per-chunk gradients.
struct BwdShards {
  ChunkMap m2;
  int64_t N, S;
  const float* P;
  float* b;     // [N S][H][K][V]
  float* ends;  // [N S][H][K][V]
};
// `sh` == nullptr: one reverse pass over whole sequences
hipError_t launch_bwd(const BwdArgs& a, int64_t max_chunks, const BwdShards* sh, hipStream_t st);
// the token-gradient kernel over `items` (chunk, head) workgroups (kda_bwd_grad.hip)
hipError_t launch_grad(const BwdArgs& a, int64_t items, hipStream_t st);

}  // namespace kda
