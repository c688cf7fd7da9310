// C ABI of the gfx950 KDA forward (include/kda.h): argument checks, workspace
// layout, varlen scheduling and the launch sequence
//     [varlen only] chunk offsets + longest-first order  ->  intra  ->  inter
// all asynchronous on the caller's stream.  The argument list follows the
// 14-argument torch.ops._flashkda_C.fwd call and get_workspace_size(T, H, N)
// of the vLLM PR report ("关键源码片段"), with sizes and the stream appended.

#include <stdio.h>
#include <stdlib.h>

#include "../../include/kda.h"
#include "kda_host.h"

namespace kda {
namespace {

constexpr int kMaxSortN = 16384;

// choff[n] = sum_{m<n} ceil(len_m / 64), choff[N] = total chunks (one block).
// Also zeroes the intra kernel's work-item counter and the call's fault word
// (claim[0], claim[1]).
__global__ void __launch_bounds__(1024) kda_chunk_offsets_kernel(const int32_t* __restrict__ cu, int N,
                                                                 int32_t* __restrict__ choff,
                                                                 int32_t* __restrict__ claim) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  if (tid == 0) {
    carry = 0;
    claim[0] = 0;
    claim[1] = 0;
  }
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int i = base + tid;
    const int c = (i < N) ? (cu[i + 1] - cu[i] + CH - 1) / CH : 0;
    int x = c;  // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int before = carry;
    for (int u = 0; u < wv; ++u) before += wsum[u];
    if (i < N) choff[i] = before + x - c;
    __syncthreads();
    if (tid == 1023) carry = before + x;
    __syncthreads();
  }
  if (tid == 0) choff[N] = carry;
}

// Shard offsets of a split forward, shard i = n S + s of sequence n.
// Without cu: N sequences of T tokens (nc chunks) cut into S shards of cs
// chunks; shard i starts at token n T + s cs 64 and at global chunk
// n nc + s cs (the intra kernel's numbering).  With cu (and the chunk
// offsets choff of the intra kernel's varlen numbering): sequence n of
// nc_n chunks is cut into S shards of ceil(nc_n / S) chunks, the last ones
// shorter or empty.
__global__ void kda_shard_map_kernel(int32_t* __restrict__ scu, int32_t* __restrict__ schoff,
                                     const int32_t* __restrict__ cu, const int32_t* __restrict__ choff, int N,
                                     int S, int T, int nc, int cs) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int ns = N * S;
  if (i > ns) return;
  const int n = i < ns ? i / S : N;
  const int sh = i < ns ? i - n * S : 0;
  if (cu) {
    const int bos = cu[n];
    const int len = i < ns ? cu[n + 1] - bos : 0;
    const int ncn = (len + CH - 1) / CH;
    const int csn = (ncn + S - 1) / S;
    const int c = sh * csn < ncn ? sh * csn : ncn;
    scu[i] = bos + (c < ncn ? c * CH : len);
    schoff[i] = choff[n] + c;
  } else {
    scu[i] = n * T + sh * cs * CH;
    schoff[i] = n * nc + sh * cs;
  }
}

// Zeroes the intra kernel's work-item counter and the call's fault word (a
// kernel rather than a memset, so that a captured graph replays it as a
// kernel node).
__global__ void kda_zero_claim_kernel(int32_t* __restrict__ claim) {
  claim[0] = 0;
  claim[1] = 0;
}

// Longest-first processing order of the sequences: rank of sequence i = number
// of sequences that are longer, or equally long with a smaller index.
__global__ void kda_order_kernel(const int32_t* __restrict__ cu, int N, int32_t* __restrict__ order) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const int li = cu[i + 1] - cu[i];
  int rank = 0;
  for (int j = 0; j < N; ++j) {
    const int lj = cu[j + 1] - cu[j];
    rank += (lj > li) || (lj == li && j < i);
  }
  order[rank] = i;
}

}  // namespace

// The launch's own return code (not hipGetLastError, which also reports
// errors left behind by earlier, unrelated runtime calls).  KDA_DEBUG=1 in the
// environment prints the HIP error behind KDA_ERR_LAUNCH.
kda_status_t launch_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return KDA_SUCCESS;
  if (getenv("KDA_DEBUG")) fprintf(stderr, "kda: %s launch failed: %s\n", what, hipGetErrorString(err));
  return KDA_ERR_LAUNCH;
}

}  // namespace kda

using namespace kda;

extern "C" {

size_t kda_workspace_size(int64_t T_total, int64_t H, int64_t N) {
  if (T_total < 0 || H < 1 || N < 1) return 0;
  return workspace_bound(T_total, H, N);
}

int kda_is_supported(int64_t K, int64_t V, float lower_bound) {
  return (K == 64 || K == KD) && (V == 64 || V == VD) && lower_bound >= -5.0f && lower_bound <= 0.0f;
}

kda_status_t kda_workspace_faults(const void* workspace, uint32_t* faults, void* stream) {
  if (!workspace || !faults) return KDA_ERR_INVALID;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, static_cast<const char*>(workspace) + workspace_layout(0, 1, 1).faults,
                                sizeof word, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return launch_status(e, "fault word copy");
  *faults = word;
  return KDA_SUCCESS;
}

const char* kda_status_string(kda_status_t s) {
  switch (s) {
    case KDA_SUCCESS: return "KDA_SUCCESS";
    case KDA_ERR_INVALID: return "KDA_ERR_INVALID";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH";
  }
  return "KDA_ERR_UNKNOWN";
}

}  // extern "C"

namespace kda {

// Argument checks shared by every entry point that runs the chunked forward,
// then the varlen bookkeeping and the intra-chunk kernel on `st`.
kda_status_t prepare(const void* q, const void* k, const void* raw_gate, const void* raw_beta,
                     void* workspace, size_t workspace_bytes, const float* A_log,
                     const float* dt_bias, float lower_bound, const int32_t* cu_seqlens, int64_t B,
                     int64_t T, int64_t H, int64_t K, int64_t V, int64_t N, hipStream_t st,
                     Prepared& pr, unsigned flags, bool run_intra) {
  if (B < 1 || T < 0 || H < 1 || N < 1) return KDA_ERR_INVALID;
  if (flags & ~(unsigned)(FLAG_GATE_GIVEN | FLAG_BETA_GIVEN | FLAG_NO_QK_NORM | FLAG_STATE_VK |
                          FLAG_REUSE_RECORDS | FLAG_KEEP_RECORDS | FLAG_SINGLE_LAUNCH))
    return KDA_ERR_INVALID;
  // token arrays may be NULL only when there are no tokens (empty tensors)
  if (B * T > 0 && (!q || !k || !raw_gate || !raw_beta)) return KDA_ERR_INVALID;
  const bool gate_given = flags & FLAG_GATE_GIVEN;
  if (!gate_given && (!A_log || !dt_bias)) return KDA_ERR_INVALID;
  if (cu_seqlens ? (B != 1) : (N != B)) return KDA_ERR_INVALID;
  if (!kda_is_supported(K, V, lower_bound)) return KDA_ERR_UNSUPPORTED;
  if (B * T * H > ((int64_t)1 << 40) || N * H > ((int64_t)1 << 28) || N > ((int64_t)1 << 30))
    return KDA_ERR_INVALID;
  const int64_t T_total = B * T;
  pr.lay = workspace_layout(T_total, H, N);
  if (!workspace || workspace_bytes < pr.lay.total) return KDA_ERR_WORKSPACE;
  pr.max_chunks = cu_seqlens ? T_total / CH + N : B * ((T + CH - 1) / CH);
  if (pr.max_chunks * H > ((int64_t)1 << 31) - 1) return KDA_ERR_INVALID;

  pr.ws = static_cast<char*>(workspace);
  int32_t* choff = reinterpret_cast<int32_t*>(pr.ws + pr.lay.choff);
  int32_t* claim = reinterpret_cast<int32_t*>(pr.ws + pr.lay.claim);
  pr.order = nullptr;
  int n32 = (int)N;
  if (!cu_seqlens) {
    void* zargs[] = {(void*)&claim};
    if (launch_status(hipLaunchKernel(reinterpret_cast<const void*>(&kda_zero_claim_kernel), dim3(1), dim3(1),
                                      zargs, 0, st),
                      "claim reset") != KDA_SUCCESS)
      return KDA_ERR_LAUNCH;
  } else {
    void* cargs[] = {(void*)&cu_seqlens, (void*)&n32, (void*)&choff, (void*)&claim};
    if (launch_status(hipLaunchKernel(reinterpret_cast<const void*>(&kda_chunk_offsets_kernel), dim3(1),
                                      dim3(1024), cargs, 0, st),
                      "chunk offsets") != KDA_SUCCESS)
      return KDA_ERR_LAUNCH;
    if (N > 1 && N <= kMaxSortN) {
      pr.order = reinterpret_cast<int32_t*>(pr.ws + pr.lay.order);
      void* oargs[] = {(void*)&cu_seqlens, (void*)&n32, (void*)&pr.order};
      if (launch_status(hipLaunchKernel(reinterpret_cast<const void*>(&kda_order_kernel),
                                        dim3((unsigned)((N + 255) / 256)), dim3(256), oargs, 0, st),
                        "order") != KDA_SUCCESS)
        return KDA_ERR_LAUNCH;
    }
  }
  pr.map.cu = cu_seqlens;
  pr.map.choff = cu_seqlens ? choff : nullptr;
  pr.map.T = T;
  pr.map.N = (int)N;
  pr.rec = pr.ws + pr.lay.rec;

  IntraArgs& ia = pr.ia;
  ia.q = static_cast<const uint16_t*>(q);
  ia.k = static_cast<const uint16_t*>(k);
  ia.g = static_cast<const uint16_t*>(raw_gate);
  ia.beta = static_cast<const uint16_t*>(raw_beta);
  // With the gate given, A_log and dt_bias are unused but the prefetch still
  // reads them unconditionally (fixed wait depths): point absent ones at the
  // record area, which is large enough and whose values are then ignored.
  ia.A_log = A_log ? A_log : reinterpret_cast<const float*>(pr.rec);
  ia.dt_bias = dt_bias ? dt_bias : reinterpret_cast<const float*>(pr.rec);
  ia.flags = (int)(flags & (FLAG_GATE_GIVEN | FLAG_BETA_GIVEN | FLAG_NO_QK_NORM));
  ia.kd = (int)K;
  pr.kd = (int)K;
  pr.vd = (int)V;
  ia.claim = claim;
  ia.faults = reinterpret_cast<unsigned*>(pr.ws + pr.lay.faults);
  ia.rec = pr.rec;
  ia.map = pr.map;
  ia.H = (int)H;
  ia.lb2 = lower_bound * LOG2E;
  ia.lb = lower_bound;
  ia.timers = nullptr;
#ifdef KDA_PHASE_TIMERS
  // timer builds only: the caller extends the workspace by 16 counters per
  // workgroup of each kernel, intra first
  ia.timers = reinterpret_cast<unsigned long long*>(pr.ws + pr.lay.total);
#endif
  // with REUSE the records are already in the workspace
  if (!run_intra || (flags & FLAG_REUSE_RECORDS)) return KDA_SUCCESS;
  return launch_status(launch_intra(ia, pr.max_chunks, st), "intra");
}

// Whether a prepared forward runs as the fused pipeline: one sequence of at
// least one token, enough heads, its records not wanted afterwards (KEEP) and
// not given (REUSE), not split into shards, on a GPU of 8 equal XCDs.
static bool use_fused(const Prepared& pr, unsigned flags, int64_t T_total, bool split) {
  if (!(flags & FLAG_SINGLE_LAUNCH) || !pr.lay.fused || split || T_total < 1 || pr.kd != KD || pr.vd != VD ||
      (flags & (FLAG_REUSE_RECORDS | FLAG_KEEP_RECORDS)))
    return false;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  // per XCD 2 cus / 8 workgroups, at most half of them chains
  const int64_t hx = (pr.ia.H + 7) / 8;
  return cus >= 192 && cus % 8 == 0 && FUSED_CHAINS * hx <= cus / 8;
}

InterArgs inter_args(const Prepared& pr, int64_t H) {
  InterArgs xa;
  xa.v = nullptr;
  xa.out = nullptr;
  xa.init = nullptr;
  xa.fin = nullptr;
  xa.init_identity = 0;
  xa.state_vk = 0;
  xa.rec = pr.rec;
  xa.order = pr.order;
  xa.map = pr.map;
  xa.H = (int)H;
  xa.kd = pr.kd;
  xa.vd = pr.vd;
  xa.scale = 1.0f;
  xa.states = nullptr;
  xa.dtile = nullptr;
  xa.timers = nullptr;
#ifdef KDA_PHASE_TIMERS
  xa.timers = reinterpret_cast<unsigned long long*>(pr.ws + pr.lay.total) + (size_t)pr.max_chunks * H * 16;
#endif
  return xa;
}

// The shard states of a prepared call (records built for the N sequences of
// T tokens, split_plan(T, H, N).S > 1): the shard map, R and P of every shard
// (the shard passes of kda_shard_affine), and their fold per sequence, which
// leaves the entering state of every shard in the workspace (lay.sstart) and
// writes final_state if given.  The records are indexed by global chunk, so
// the shard map reuses them as they are.  `m2` receives the shard map.
kda_status_t shard_states(const Prepared& pr, const void* v, const float* initial_state, float* final_state,
                          int64_t T, int64_t H, int64_t N, hipStream_t st, ChunkMap& m2) {
  // varlen calls take S from the mean length and cut each sequence by its own
  const SplitPlan sp = pr.map.cu ? SplitPlan{pr.lay.S, 0} : split_plan(T, H, N);
  const int64_t ns = N * sp.S;
  const int64_t nc = pr.map.cu ? 0 : (T + CH - 1) / CH;
  int32_t* scu = reinterpret_cast<int32_t*>(pr.ws + pr.lay.scu);
  int32_t* schoff = reinterpret_cast<int32_t*>(pr.ws + pr.lay.schoff);
  float* sP = reinterpret_cast<float*>(pr.ws + pr.lay.sP);
  float* sR = reinterpret_cast<float*>(pr.ws + pr.lay.sR);
  float* sstart = reinterpret_cast<float*>(pr.ws + pr.lay.sstart);
  const int32_t* cu = pr.map.cu;
  const int32_t* choff = pr.map.choff;
  int n32 = (int)N, s32 = (int)sp.S, t32 = (int)T, nc32 = (int)nc, cs32 = (int)sp.cs;
  void* margs[] = {(void*)&scu,  (void*)&schoff, (void*)&cu,   (void*)&choff, (void*)&n32,
                   (void*)&s32,  (void*)&t32,    (void*)&nc32, (void*)&cs32};
  if (launch_status(hipLaunchKernel(reinterpret_cast<const void*>(&kda_shard_map_kernel),
                                    dim3((unsigned)((ns + 1 + 255) / 256)), dim3(256), margs, 0, st),
                    "shard map") != KDA_SUCCESS)
    return KDA_ERR_LAUNCH;
  m2.cu = scu;
  m2.choff = schoff;
  m2.T = T;
  m2.N = (int)ns;
  InterArgs xr = shard_inter_args(pr, H, m2);  // R: from a zero state, with V
  xr.v = static_cast<const uint16_t*>(v);
  xr.fin = sR;
  if (launch_status(launch_inter(xr, st), "inter (shard R)") != KDA_SUCCESS) return KDA_ERR_LAUNCH;
  InterArgs xp = shard_inter_args(pr, H, m2);  // P: V = 0 from the identity
  xp.fin = sP;
  xp.init_identity = 1;
  if (launch_status(launch_inter(xp, st), "inter (shard P)") != KDA_SUCCESS) return KDA_ERR_LAUNCH;
  const size_t kv = (size_t)KD * VD;
  for (int64_t n = 0; n < N; ++n) {
    const size_t sh = (size_t)n * sp.S * H * kv, sq = (size_t)n * H * kv;
    if (launch_status(launch_shard_scan(sP + sh, sR + sh, initial_state ? initial_state + sq : nullptr,
                                        sstart + sh, final_state ? final_state + sq : nullptr, (int)sp.S,
                                        (int)H, st),
                      "shard fold") != KDA_SUCCESS)
      return KDA_ERR_LAUNCH;
  }
  return KDA_SUCCESS;
}

InterArgs shard_inter_args(const Prepared& pr, int64_t H, const ChunkMap& m2) {
  InterArgs x = inter_args(pr, H);
  x.map = m2;
  x.order = nullptr;
  x.timers = nullptr;
  return x;
}

// The forward's recurrence on shards: the shard states, then the forward over
// the shards from them.  Not for in-place states (the fold reads
// initial_state while it writes final_state).
kda_status_t split_forward(const Prepared& pr, const void* v, void* out, const float* initial_state,
                           float* final_state, float scale, int64_t T, int64_t H, int64_t N, hipStream_t st) {
  ChunkMap m2;
  const kda_status_t s = shard_states(pr, v, initial_state, final_state, T, H, N, st, m2);
  if (s != KDA_SUCCESS) return s;
  InterArgs xf = shard_inter_args(pr, H, m2);  // the outputs, from the folded entering states
  xf.v = static_cast<const uint16_t*>(v);
  xf.out = static_cast<uint16_t*>(out);
  xf.init = reinterpret_cast<const float*>(pr.ws + pr.lay.sstart);
  xf.fin = reinterpret_cast<float*>(pr.ws + pr.lay.sfin);
  xf.scale = scale;
  return launch_status(launch_inter(xf, st), "inter (shards)");
}

}  // namespace kda

extern "C" {

kda_status_t kda_fwd_ex(const void* q, const void* k, const void* v, const void* raw_gate,
                        const void* raw_beta, float scale, void* out, void* workspace,
                        size_t workspace_bytes, const float* A_log, const float* dt_bias,
                        float lower_bound, const float* initial_state, float* final_state,
                        const int32_t* cu_seqlens, int64_t B, int64_t T, int64_t H, int64_t K,
                        int64_t V, int64_t N, unsigned flags, void* stream) {
  if (B * T > 0 && (!v || !out)) return KDA_ERR_INVALID;
  if (!(scale == scale)) return KDA_ERR_INVALID;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Prepared pr;
  const kda_status_t s = prepare(q, k, raw_gate, raw_beta, workspace, workspace_bytes, A_log, dt_bias,
                                 lower_bound, cu_seqlens, B, T, H, K, V, N, st, pr, flags, false);
  if (s != KDA_SUCCESS) return s;
  const bool split = use_split(pr, flags, B, T) && !(initial_state && initial_state == final_state);
  if (use_fused(pr, flags, B * T, split)) {
    // one sequence: its bounds are [0, B T) with or without cu_seqlens
    ChunkMap m1;
    m1.cu = nullptr;
    m1.choff = nullptr;
    m1.T = B * T;
    m1.N = 1;
    IntraArgs ia = pr.ia;
    ia.map = m1;
    ChainArgs ca;
    ca.v = static_cast<const uint16_t*>(v);
    ca.out = static_cast<uint16_t*>(out);
    ca.init = initial_state;
    ca.fin = final_state;
    ca.state_vk = (flags & FLAG_STATE_VK) ? 1 : 0;
    ca.rec = pr.rec;
    ca.order = nullptr;
    ca.map = m1;
    ca.H = (int)H;
    ca.scale = scale;
    FusedArgs fa;
    fa.ringbuf = pr.ws + pr.lay.fring;
    fa.flags = reinterpret_cast<int*>(pr.ws + pr.lay.fflags);
    fa.consumed = reinterpret_cast<int*>(pr.ws + pr.lay.fcons);
    fa.claims = reinterpret_cast<int*>(pr.ws + pr.lay.fclaims);
    fa.faults = reinterpret_cast<unsigned*>(pr.ws + pr.lay.faults);
    fa.nchunk = (int)((B * T + CH - 1) / CH);
    fa.ring = FUSED_RING;
    fa.slot_wait = FUSED_SLOT_WAIT;
    return launch_status(launch_fused(ia, ca, fa, st), "fused");
  }
  if (!(flags & FLAG_REUSE_RECORDS) &&
      launch_status(launch_intra(pr.ia, pr.max_chunks, st), "intra") != KDA_SUCCESS)
    return KDA_ERR_LAUNCH;
  if (split) return split_forward(pr, v, out, initial_state, final_state, scale, T, H, N, st);
  InterArgs xa = inter_args(pr, H);
  xa.v = static_cast<const uint16_t*>(v);
  xa.out = static_cast<uint16_t*>(out);
  xa.init = initial_state;
  xa.fin = final_state;
  xa.scale = scale;
  xa.state_vk = (flags & FLAG_STATE_VK) ? 1 : 0;
  return launch_status(launch_inter(xa, st), "inter");
}

kda_status_t kda_fwd(const void* q, const void* k, const void* v, const void* raw_gate,
                     const void* raw_beta, float scale, void* out, void* workspace,
                     size_t workspace_bytes, const float* A_log, const float* dt_bias,
                     float lower_bound, const float* initial_state, float* final_state,
                     const int32_t* cu_seqlens, int64_t B, int64_t T, int64_t H, int64_t K,
                     int64_t V, int64_t N, void* stream) {
  return kda_fwd_ex(q, k, v, raw_gate, raw_beta, scale, out, workspace, workspace_bytes, A_log, dt_bias,
                    lower_bound, initial_state, final_state, cu_seqlens, B, T, H, K, V, N, 0u, stream);
}

kda_status_t kda_shard_affine(const void* q, const void* k, const void* v, const void* raw_gate,
                              const void* raw_beta, void* workspace, size_t workspace_bytes,
                              const float* A_log, const float* dt_bias, float lower_bound, float* P,
                              float* R, const int32_t* cu_seqlens, int64_t B, int64_t T, int64_t H,
                              int64_t K, int64_t V, int64_t N, void* stream) {
  if ((B * T > 0 && !v) || !P || !R) return KDA_ERR_INVALID;
  if (K != KD || V != VD) return KDA_ERR_UNSUPPORTED;  // P starts from the identity: K == V == 128
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Prepared pr;
  const kda_status_t s = prepare(q, k, raw_gate, raw_beta, workspace, workspace_bytes, A_log, dt_bias,
                                 lower_bound, cu_seqlens, B, T, H, K, V, N, st, pr);
  if (s != KDA_SUCCESS) return s;
  // R: the shard's own contribution, its final state from a zero start
  InterArgs xr = inter_args(pr, H);
  xr.v = static_cast<const uint16_t*>(v);
  xr.fin = R;
  if (launch_status(launch_inter(xr, st), "inter (R)") != KDA_SUCCESS) return KDA_ERR_LAUNCH;
  // P: the homogeneous map, the final state of V = 0 from S0 = I (K == V)
  InterArgs xp = inter_args(pr, H);
  xp.fin = P;
  xp.init_identity = 1;
  return launch_status(launch_inter(xp, st), "inter (P)");
}

kda_status_t kda_shard_scan(const float* P, const float* R, const float* initial_state, float* starts,
                            float* final_state, int64_t n_shards, int64_t H, int64_t K, int64_t V,
                            void* stream) {
  if (!P || !R || !starts) return KDA_ERR_INVALID;
  if (n_shards < 1 || H < 1 || n_shards * H > ((int64_t)1 << 28)) return KDA_ERR_INVALID;
  if (K != KD || V != VD) return KDA_ERR_UNSUPPORTED;
  return launch_status(launch_shard_scan(P, R, initial_state, starts, final_state, (int)n_shards, (int)H,
                                         reinterpret_cast<hipStream_t>(stream)),
                       "shard scan");
}

}  // extern "C"
