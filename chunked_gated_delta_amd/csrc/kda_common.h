// Shared definitions of the gfx950 KDA forward kernels (intra-chunk kernel,
// inter-chunk kernel, host API).  Internal header: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int KD = 128;   // head dim K
constexpr int VD = 128;   // head dim V
constexpr int CH = 64;    // chunk length
constexpr int SUB = 16;   // sub-chunk length (decay reference granularity)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float L2_EPS = 1e-6f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Per (chunk, head) record written by the intra-chunk kernel and read by the
// inter-chunk kernel.  Arrays are stored in the reader's MFMA fragment order:
// fragment f of an operand is 64 lanes x 16 bytes, contiguous, so every load
// instruction of the reader moves one aligned 1 KB block.
//   NW   : -W = -T diag(beta) (K^ * exp(G))      f16  [64 tok][128 ch]
//   QG   : Q^ * exp(G)                           f16  [64 tok][128 ch]
//   KTH/L: (K^ * exp(G_L - G))^T  hi / lo        f16  [128 ch][64 tok]
//          (the lo half is stored times KT_LO_SCALE, see below)
//   AQK  : A_qk (zero above the diagonal)        f16  [64 tok][64 tok]
//   TBH/L: T diag(beta) (zero above diagonal)    bf16 [64 tok][64 tok] hi / lo
//   GL   : exp(G_L) per channel                  f32  [128]
// ---------------------------------------------------------------------------
constexpr size_t REC_NW = 0;
constexpr size_t REC_QG = REC_NW + CH * KD * 2;
constexpr size_t REC_KTH = REC_QG + CH * KD * 2;
constexpr size_t REC_KTL = REC_KTH + KD * CH * 2;
constexpr size_t REC_AQK = REC_KTL + KD * CH * 2;
constexpr size_t REC_TBH = REC_AQK + CH * CH * 2;
constexpr size_t REC_TBL = REC_TBH + CH * CH * 2;
constexpr size_t REC_GL = REC_TBL + CH * CH * 2;
constexpr size_t REC_BYTES = REC_GL + KD * 4;  // 90624
static_assert(REC_BYTES % 256 == 0, "record alignment");

// The lo half of the fp16 hi/lo split of Kt is stored times 2^11.  A lo part
// is at most half an fp16 ulp of its hi part (2^-11 of it), which puts it in
// the fp16 subnormal range (below 2^-14) for every |Kt| < 1/8: there its
// error is an absolute 2^-25 instead of 11 bits relative.  With one key
// repeated at every position that error is the same in every chunk and adds
// up along the sequence.  Scaled by 2^11 the lo part keeps 11 bits wherever
// the hi part is normal; the reader multiplies its pass by KT_LO_UNSCALE.
constexpr float KT_LO_SCALE = 2048.0f;
constexpr float KT_LO_UNSCALE = 1.0f / 2048.0f;

// Element index (in 16-bit units) of the fragment-ordered record arrays.  The
// reader's lane l = 16 gq + tl of wave w loads 8 consecutive k elements:
//   [64 tok][128 ch] (NW, QG): row 16w + tl, channels 32kb + 8gq + 0..7, fragment 4w + kb
//   [64 tok][64 tok] (AQK, TB): row 16w + tl, tokens 32ks + 8gq + 0..7, fragment 2w + ks
//   [128 ch][64 tok] (KT):      channel 32w + 16mt + tl, tokens 32ks + 8gq + 0..7,
//                               fragment 4w + 2mt + ks
__host__ __device__ constexpr int frag_tc(int i, int c) {  // [64][128]
  return ((((i >> 4) * 4 + (c >> 5)) * 64 + ((c >> 3) & 3) * 16 + (i & 15)) << 3) + (c & 7);
}
__host__ __device__ constexpr int frag_tt(int i, int j) {  // [64][64]
  return ((((i >> 4) * 2 + (j >> 5)) * 64 + ((j >> 3) & 3) * 16 + (i & 15)) << 3) + (j & 7);
}
__host__ __device__ constexpr int frag_ct(int c, int t) {  // [128][64]
  return ((((c >> 4) * 2 + (t >> 5)) * 64 + ((t >> 3) & 3) * 16 + (c & 15)) << 3) + (t & 7);
}

// Chunk bookkeeping shared by both kernels.  Without cu_seqlens there are N
// sequences of length T and sequence n owns chunks [n*ceil(T/64), ...).  With
// cu_seqlens the chunk offsets come from a device prefix sum (choff[N+1]).
struct ChunkMap {
  const int32_t* cu;     // nullptr: N sequences of length T
  const int32_t* choff;  // [N+1] exclusive prefix of per-sequence chunk counts (varlen)
  int64_t T;
  int N;
};

__device__ __forceinline__ void seq_bounds(const ChunkMap& m, int n, int64_t& bos, int64_t& eos) {
  if (m.cu) {
    bos = m.cu[n];
    eos = m.cu[n + 1];
  } else {
    bos = (int64_t)n * m.T;
    eos = bos + m.T;
  }
}

__device__ __forceinline__ int64_t first_chunk(const ChunkMap& m, int n) {
  return m.cu ? (int64_t)m.choff[n] : (int64_t)n * ((m.T + CH - 1) / CH);
}

__device__ __forceinline__ int64_t total_chunks(const ChunkMap& m) {
  return m.cu ? (int64_t)m.choff[m.N] : (int64_t)m.N * ((m.T + CH - 1) / CH);
}

// sequence owning global chunk g (g < total_chunks)
__device__ __forceinline__ int chunk_owner(const ChunkMap& m, int64_t g) {
  if (!m.cu) return (int)(g / ((m.T + CH - 1) / CH));
  int lo = 0, hi = m.N - 1;  // largest n with choff[n] <= g and g < choff[n+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (m.choff[mid] <= g) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void unpack_bf16x8(const uint4 v, float (&d)[8]) {
  const uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    d[2 * u] = __uint_as_float(a[u] << 16);
    d[2 * u + 1] = __uint_as_float(a[u] & 0xffff0000u);
  }
}

__device__ __forceinline__ void lds_f32x8(const float* src, float (&d)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(src);
  const float4 b = *reinterpret_cast<const float4*>(src + 4);
  d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
  d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
}

// Buffer loads and stores: a 128-bit descriptor (scalar registers) per array
// and one lane offset, every element's place a compile-time or wave-uniform
// offset, instead of a 64-bit address per load.  The last argument of the
// load and store builtins is the cache policy: 0 for the default, SC1
// (device scope) for data that another CU writes while this kernel runs: such
// a load misses this CU's L1 and reads the L2 that CUs of one XCD share,
// where a store has landed once the writer's s_waitcnt vmcnt(0) returned.
// (Workgroup scope, SC0, may still hit a stale line of this CU's L1.)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int BUF_DESC3 = 0x00020000;  // raw 32-bit buffer, no format conversion
constexpr int SC1 = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, BUF_DESC3);
}
template <typename T, int POLICY = 0>
__device__ __forceinline__ T bload(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POLICY));
}

// Split-plane B-operand fragments in LDS.  Fragment f holds one 16-column
// tile x 32-k block of a 16-bit operand: the 16 bytes (8 k) of MFMA lane
// l = 16gq + tl, split into two planes, bytes 0-7 at l*8 and bytes 8-15 at
// 512 + l*8.  A lane's operand is two 8-byte reads, and both the reads (64
// contiguous lanes) and the writes from the accumulator layout (4 consecutive
// k of one column) are free of LDS bank conflicts on gfx950, where row-pitched
// layouts doubled the read and the write time.
constexpr int FRAG = 1024;  // bytes per fragment

__device__ __forceinline__ uint4 frag_read(const char* base, int frag, int lane) {
  const char* p = base + frag * FRAG + lane * 8;
  const uint2 lo = *reinterpret_cast<const uint2*>(p);
  const uint2 hi = *reinterpret_cast<const uint2*>(p + FRAG / 2);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Store 4 consecutive k (k0 = 4q within the fragment's 32-k block, q = 0..7)
// of column tl into fragment `frag`: MFMA lane 16 (q / 2) + tl, plane q % 2.
template <typename V4>
__device__ __forceinline__ void frag_write4(char* base, int frag, int q, int tl, V4 v) {
  static_assert(sizeof(V4) == 8, "4 x 16-bit");
  *reinterpret_cast<V4*>(base + frag * FRAG + (q & 1) * (FRAG / 2) + (16 * (q >> 1) + tl) * 8) = v;
}

// Optional per-phase cycle counters, compiled out unless KDA_PHASE_TIMERS is
// defined: every wave accumulates cycle-counter deltas between phase marks
// (wave-uniform values, so they stay in scalar registers) and thread 0 stores
// its wave's to timers[blockIdx.x * 16 + i].
#ifdef KDA_PHASE_TIMERS
#define KDA_TIMER_DECL unsigned long long tacc_[15] = {0}; unsigned long long tlast_ = 0;
#define KDA_TIMER_MARK(i) do { const unsigned long long t_ = __builtin_readcyclecounter(); \
    if ((i) > 0) tacc_[(i) - 1] += t_ - tlast_; tlast_ = t_; } while (0)
#define KDA_TIMER_STORE(ptr) do { if (threadIdx.x == 0 && (ptr)) for (int i_ = 0; i_ < 15; ++i_) \
    (ptr)[(size_t)blockIdx.x * 16 + i_] = tacc_[i_]; } while (0)
#else
#define KDA_TIMER_DECL
#define KDA_TIMER_MARK(i) do { } while (0)
#define KDA_TIMER_STORE(ptr) do { } while (0)
#endif

// Variant bits (same values as the KDA_FLAG_* constants of the C ABI).
constexpr int FLAG_GATE_GIVEN = 1;   // raw_gate holds the natural-log decay g
constexpr int FLAG_BETA_GIVEN = 2;   // raw_beta holds beta
constexpr int FLAG_NO_QK_NORM = 4;   // q, k used without L2 normalisation
constexpr int FLAG_STATE_VK = 8;     // states stored transposed, [N, H, V, K]
constexpr int FLAG_REUSE_RECORDS = 16;  // the workspace already holds this call's chunk records
constexpr int FLAG_KEEP_RECORDS = 32;   // leave every chunk record in the workspace (for REUSE)
constexpr int FLAG_SINGLE_LAUNCH = 64;  // one-sequence calls: the one-launch producer/chain pipeline

// Fault bits a call ORs into the workspace's fault word (same values as the
// KDA_FAULT_* constants of the C ABI): conditions the kernels detect on the
// device, where no status can be returned.
constexpr unsigned FAULT_WAIT_TIMEOUT = 1u;  // a bounded wait gave up; results are invalid
constexpr unsigned FAULT_GATE_RANGE = 2u;    // FLAG_GATE_GIVEN: a decay outside [lower_bound, 0]
constexpr unsigned FAULT_QK_NORM = 4u;       // FLAG_NO_QK_NORM: a q or k row with |x|^2 > 1 + 1/16
constexpr unsigned FAULT_PLACEMENT = 8u;     // single launch: the workgroups of one id residue ran on two XCDs

// The fused forward pipeline (one sequence): per XCD, intra-chunk producer
// workgroups hand the chunk records of that XCD's heads (h = xcd + 8 l) to the
// FUSED_CHAINS chain workgroups of each head (one per 64-column half of the
// state) through a ring of FUSED_RING records per head, in that XCD's L2.  The
// per-chain and per-XCD words sit FUSED_LINE bytes apart (one L2 line each).
constexpr int FUSED_LINE = 128;
constexpr int FUSED_RING = 8;     // ring slots per head (workspace capacity)
constexpr int FUSED_CHAINS = 2;
// Polls (each an L2 round trip plus a 512-cycle sleep) a producer spends
// waiting for its ring slot to be freed before it writes the record to the
// record area instead: producers pace themselves to the chains while every
// chain is running, and still finish on their own if a chain is not.
constexpr int FUSED_SLOT_WAIT = 4096;
struct IntraFused {
  int xcd = 0;               // the producer's XCD
  int hx = 0;                // heads of that XCD
  int ring = 1;              // ring slots per head in use
  int slot_wait = 0;         // polls for a free slot before the record area is used
  char* ringbuf = nullptr;   // [H][FUSED_RING] records
  const int* consumed = nullptr;  // [H][FUSED_CHAINS]: chunks each chain has finished reading
  int* flags = nullptr;      // [chunks][H]: 0 not ready, 1 in the ring, 2 in the record area
  int H = 0;
  int nchunk = 0;
};
struct ChainFused {
  const char* ringbuf = nullptr;  // [H][FUSED_RING] records
  int ring = 1;                   // ring slots per head in use
  const int* flags = nullptr;     // [chunks][H] ready flags
  int* consumed = nullptr;        // this chain's own consumed word
  unsigned* faults = nullptr;
  int nchunk = 0;
};
// Polls of one ready flag before a chain gives up on it (about a second: each
// poll is an L2 round trip plus a 256-cycle sleep).
constexpr int FUSED_SPIN_LIMIT = 1 << 21;

// Host-side launchers (defined next to their kernels).
struct IntraArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* g;
  const uint16_t* beta;
  const float* A_log;
  const float* dt_bias;
  char* rec;        // records [max_chunks][H]
  ChunkMap map;
  int H;
  float lb2;        // lower_bound * log2(e)
  float lb;         // lower_bound
  int flags;        // FLAG_GATE_GIVEN | FLAG_BETA_GIVEN | FLAG_NO_QK_NORM
  int kd;           // head dim K of the inputs: 64 or 128 (records always use the 128-channel layout)
  int* claim;       // work-item counter, zero when the kernel starts
  unsigned* faults; // the call's fault word (FAULT_* bits)
  unsigned long long* timers;  // phase timers (KDA_PHASE_TIMERS builds only), else nullptr
};
struct InterArgs {
  const uint16_t* v;     // nullptr: V = 0 (homogeneous recurrence)
  uint16_t* out;         // nullptr: no outputs, final state only
  const float* init;     // nullptr: zero state, or the identity if init_identity
  float* fin;
  int init_identity;     // with init == nullptr: start every (sequence, head) from I (needs K == V)
  int state_vk;          // states stored transposed: S[c][j] at j * K + c
  const char* rec;
  const int32_t* order;  // nullptr: identity order of sequences
  ChunkMap map;
  int H;
  int kd, vd;            // head dims of the states, v and out: 64 or 128 each (state rows c >= kd are zero)
  float scale;
  unsigned long long* timers;  // phase timers (KDA_PHASE_TIMERS builds only), else nullptr
  // checkpoints for the backward pass (both nullptr in the forward):
  float* states;         // [chunks][H][K][V] state entering every chunk (fp32)
  float* dtile;          // [chunks][H][64][V] the chunk's D = U - W S (rows past the chunk end zero)
};
// The chain kernel: the inter-chunk recurrence with two workgroups per
// (sequence, head), one per 64-column half (same results as the inter kernel).
struct ChainArgs {
  const uint16_t* v;
  uint16_t* out;
  const float* init;     // nullptr: zero state
  float* fin;            // nullptr: not written
  int state_vk;          // states stored transposed, S[c][j] at j * K + c
  const char* rec;       // records [chunks][H]
  const int32_t* order;  // nullptr: identity order of sequences
  ChunkMap map;
  int H;
  float scale;
};
hipError_t launch_intra(const IntraArgs& a, int64_t max_chunks, hipStream_t st);
hipError_t launch_chain(const ChainArgs& a, hipStream_t st);
// The fused pipeline over one sequence: intra-chunk producers and
// FUSED_CHAINS chain workgroups per head in a single persistent launch (`fa`
// carries the ring, flags, consumed counters, per-XCD claim counters and the
// fault word, all cleared by the launcher first).  Needs 8 XCDs of equal size
// and N == 1.
struct FusedArgs {
  char* ringbuf;
  int* flags;      // [chunks][H]
  int* consumed;   // [H][FUSED_CHAINS] FUSED_LINE apart
  int* claims;     // [8] claim counters, then [8] XCDs of the id residues, FUSED_LINE apart
  unsigned* faults;
  int nchunk;
  int ring;        // ring slots per head in use, 1..FUSED_RING
  int slot_wait;   // a producer's polls for a free ring slot
};
hipError_t launch_fused(const IntraArgs& ia, const ChainArgs& ca, const FusedArgs& fa, hipStream_t st);
hipError_t launch_inter(const InterArgs& a, hipStream_t st);
hipError_t launch_shard_scan(const float* P, const float* R, const float* init, float* starts, float* fin,
                             int n_shards, int H, hipStream_t st);
// the backward's reverse fold: ends[r] = gradient leaving shard r, dinit = P_0^T g_0 + B_0
hipError_t launch_shard_scan_rev(const float* P, const float* B, const float* dfin, float* ends, float* dinit,
                                 int n_shards, int H, hipStream_t st);

}  // namespace kda
