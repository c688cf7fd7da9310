// Shard scan for splitting one long sequence into shards (context
// parallelism, named KCP on the torchtitan PR page, section "Summary"; the
// page gives no algorithm).  The gated delta rule is affine in the state: a
// shard maps its entering state S to P S + R, with P (K x K) the product of
// the per-token maps (I - b k k^T) Diag(a) and R the shard's final state from
// a zero start (both computed by kda_shard_affine).  Shard r is entered with
//     S_0 = initial state (or 0),   S_{r+1} = P_r S_r + R_r,
// a sequential fold over shards that this kernel evaluates in fp32.
//
// One workgroup per (head, 16-column slab of the state); the slab stays in LDS
// across shards.  Thread t owns row t/2, columns 8 (t % 2) .. + 7 of the slab.

#include "kda_common.h"

namespace kda {
namespace {

constexpr int SLAB = 16;
constexpr int NSLAB = VD / SLAB;

constexpr int PP = KD + 1;  // LDS pitch of a staged P: rows and columns both read without bank conflicts

// One fold over the n_shards shards of one sequence, for the workgroup's head
// and slab.  REV = false: acc starts at `first`, each[r] = acc (the state
// entering shard r), acc = P_r acc + R_r.  REV = true: shards in reverse
// order, each[r] = acc (the gradient leaving shard r), acc = P_r^T acc + R_r.
// `last` (if not NULL) receives acc at the end.  P_r is staged in LDS; the
// next shard's P and R slab are loaded into registers while this one
// computes, so a step waits on one batch of loads rather than a chain of them.
template <bool REV>
__device__ __forceinline__ void fold(const float* __restrict__ P, const float* __restrict__ R,
                                     const float* first, float* __restrict__ each, float* last, int n_shards,
                                     int H) {
  __shared__ float sP[KD * PP];
  __shared__ __attribute__((aligned(16))) float sS[KD][SLAB];
  const int h = blockIdx.x / NSLAB;
  const int c0 = (blockIdx.x % NSLAB) * SLAB;
  const int t = threadIdx.x;
  const int row = t >> 1;
  const int cl = 8 * (t & 1);
  const size_t hs = (size_t)KD * VD;  // one (head) state
  const size_t ps = (size_t)KD * KD;  // one (head) P

  float acc[8];
  {
    const float* src = first ? first + h * hs + (size_t)row * VD + c0 + cl : nullptr;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = src ? src[j] : 0.0f;
  }
  float4 pn[KD * KD / 4 / 256];  // next P: float4 t + 256 j of the K x K matrix
  float rn[8];                   // next R, this thread's row and columns
  auto load = [&](int r) {
    const float4* p4 = reinterpret_cast<const float4*>(P + ((size_t)r * H + h) * ps);
#pragma unroll
    for (int j = 0; j < KD * KD / 4 / 256; ++j) pn[j] = p4[t + 256 * j];
    const float* rs = R + ((size_t)r * H + h) * hs + (size_t)row * VD + c0 + cl;
#pragma unroll
    for (int j = 0; j < 8; ++j) rn[j] = rs[j];
  };
  if (n_shards > 0) load(REV ? n_shards - 1 : 0);
  for (int s = 0; s < n_shards; ++s) {
    const int r = REV ? n_shards - 1 - s : s;
    float* dst = each + ((size_t)r * H + h) * hs + (size_t)row * VD + c0 + cl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dst[j] = acc[j];
      sS[row][cl + j] = acc[j];
      acc[j] = rn[j];
    }
#pragma unroll
    for (int j = 0; j < KD * KD / 4 / 256; ++j) {
      const int e = t + 256 * j;
      float* d = sP + (e >> 5) * PP + 4 * (e & 31);
      d[0] = pn[j].x;
      d[1] = pn[j].y;
      d[2] = pn[j].z;
      d[3] = pn[j].w;
    }
    __syncthreads();
    if (s + 1 < n_shards) load(REV ? r - 1 : r + 1);
#pragma unroll 4
    for (int k = 0; k < KD; ++k) {
      const float c = REV ? sP[k * PP + row] : sP[row * PP + k];
      const float4 s0 = *reinterpret_cast<const float4*>(&sS[k][cl]);
      const float4 s1 = *reinterpret_cast<const float4*>(&sS[k][cl + 4]);
      acc[0] += c * s0.x;
      acc[1] += c * s0.y;
      acc[2] += c * s0.z;
      acc[3] += c * s0.w;
      acc[4] += c * s1.x;
      acc[5] += c * s1.y;
      acc[6] += c * s1.z;
      acc[7] += c * s1.w;
    }
    __syncthreads();  // every thread has read sS and sP before the next shard overwrites them
  }
  if (last) {
    float* dst = last + h * hs + (size_t)row * VD + c0 + cl;
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = acc[j];
  }
}

__global__ void __launch_bounds__(256) kda_shard_scan_kernel(const float* __restrict__ P,
                                                             const float* __restrict__ R,
                                                             const float* __restrict__ init,
                                                             float* __restrict__ starts,
                                                             float* __restrict__ fin, int n_shards, int H) {
  fold<false>(P, R, init, starts, fin, n_shards, H);
}

// Reverse fold of the state gradient over the shards of one sequence, for the
// backward pass.  With g_r the gradient of the state leaving shard r and B_r
// the gradient of the state entering shard r from the shard's own outputs (a
// zero leaving gradient), the entering gradient is P_r^T g_r + B_r, so
//     g_{n-1} = d_final (or 0),   g_{r-1} = P_r^T g_r + B_r,
// and d_initial = P_0^T g_0 + B_0.  `ends` receives every g_r.  d_final and
// d_initial may be the same array: each thread reads its elements before the
// fold and writes them after it.
__global__ void __launch_bounds__(256) kda_shard_scan_rev_kernel(const float* __restrict__ P,
                                                                 const float* __restrict__ B,
                                                                 const float* dfin, float* __restrict__ ends,
                                                                 float* dinit, int n_shards, int H) {
  fold<true>(P, B, dfin, ends, dinit, n_shards, H);
}

}  // namespace

hipError_t launch_shard_scan(const float* P, const float* R, const float* init, float* starts, float* fin,
                             int n_shards, int H, hipStream_t st) {
  void* args[] = {(void*)&P, (void*)&R, (void*)&init, (void*)&starts, (void*)&fin, (void*)&n_shards, (void*)&H};
  return hipLaunchKernel(reinterpret_cast<const void*>(&kda_shard_scan_kernel), dim3((unsigned)(H * NSLAB)),
                         dim3(256), args, 0, st);
}

hipError_t launch_shard_scan_rev(const float* P, const float* B, const float* dfin, float* ends, float* dinit,
                                 int n_shards, int H, hipStream_t st) {
  void* args[] = {(void*)&P, (void*)&B, (void*)&dfin, (void*)&ends, (void*)&dinit, (void*)&n_shards, (void*)&H};
  return hipLaunchKernel(reinterpret_cast<const void*>(&kda_shard_scan_rev_kernel), dim3((unsigned)(H * NSLAB)),
                         dim3(256), args, 0, st);
}

}  // namespace kda
