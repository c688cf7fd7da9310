// Host-side pieces of the forward launch sequence (kda_api.hip) that the
// backward entry point (kda_bwd.hip) reuses.  Internal: not part of the C ABI.
#pragma once

#include "../../include/kda.h"
#include "kda_common.h"

namespace kda {

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct Layout {
  size_t claim, choff, order, rec, total;
};

inline Layout workspace_layout(int64_t T_total, int64_t H, int64_t N) {
  Layout l;
  l.claim = 0;  // the intra kernel's work-item counter (one int)
  l.choff = 256;
  l.order = l.choff + align256((size_t)(N + 1) * sizeof(int32_t));
  l.rec = l.order + align256((size_t)N * sizeof(int32_t));
  const size_t max_chunks = (size_t)(T_total / CH) + (size_t)N;
  l.total = l.rec + max_chunks * (size_t)H * REC_BYTES;
  return l;
}

// What the intra-chunk pass of one call leaves for the inter-chunk passes.
struct Prepared {
  ChunkMap map;
  int32_t* order;
  char* rec;
  char* ws;
  Layout lay;
  int64_t max_chunks;
};

// Argument checks shared by every entry point that runs the chunked forward,
// then the varlen bookkeeping and the intra-chunk kernel on `st`.
kda_status_t prepare(const void* q, const void* k, const void* raw_gate, const void* raw_beta,
                     void* workspace, size_t workspace_bytes, const float* A_log,
                     const float* dt_bias, float lower_bound, const int32_t* cu_seqlens, int64_t B,
                     int64_t T, int64_t H, int64_t K, int64_t V, int64_t N, hipStream_t st,
                     Prepared& pr, unsigned flags = 0);

// Inter-chunk arguments for the prepared call (no v, outputs or states set).
InterArgs inter_args(const Prepared& pr, int64_t H);

// KDA_SUCCESS, or KDA_ERR_LAUNCH for a failed launch (KDA_DEBUG=1 prints why).
kda_status_t launch_status(hipError_t err, const char* what);

}  // namespace kda
