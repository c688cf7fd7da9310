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

__global__ void __launch_bounds__(256) kda_shard_scan_kernel(const float* __restrict__ P,
                                                             const float* __restrict__ R,
                                                             const float* __restrict__ init,
                                                             float* __restrict__ starts,
                                                             float* __restrict__ fin, int n_shards, int H) {
  __shared__ __attribute__((aligned(16))) float sS[KD][SLAB];
  const int h = blockIdx.x / NSLAB;
  const int c0 = (blockIdx.x % NSLAB) * SLAB;
  const int t = threadIdx.x;
  const int row = t >> 1;
  const int cl = 8 * (t & 1);
  const size_t hs = (size_t)KD * VD;  // one (head) state

  float acc[8];
  {
    const float* src = init ? init + h * hs + (size_t)row * VD + c0 + cl : nullptr;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = src ? src[j] : 0.0f;
  }
  for (int r = 0; r < n_shards; ++r) {
    // state entering shard r
    float* dst = starts + ((size_t)r * H + h) * hs + (size_t)row * VD + c0 + cl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dst[j] = acc[j];
      sS[row][cl + j] = acc[j];
    }
    __syncthreads();
    const float* prow = P + ((size_t)r * H + h) * KD * KD + (size_t)row * KD;
    const float* rrow = R + ((size_t)r * H + h) * hs + (size_t)row * VD + c0 + cl;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = rrow[j];
    for (int k = 0; k < KD; k += 4) {
      const float4 p4 = *reinterpret_cast<const float4*>(prow + k);
      const float pk[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float4 s0 = *reinterpret_cast<const float4*>(&sS[k + kk][cl]);
        const float4 s1 = *reinterpret_cast<const float4*>(&sS[k + kk][cl + 4]);
        acc[0] += pk[kk] * s0.x;
        acc[1] += pk[kk] * s0.y;
        acc[2] += pk[kk] * s0.z;
        acc[3] += pk[kk] * s0.w;
        acc[4] += pk[kk] * s1.x;
        acc[5] += pk[kk] * s1.y;
        acc[6] += pk[kk] * s1.z;
        acc[7] += pk[kk] * s1.w;
      }
    }
    __syncthreads();  // every thread has read sS before the next shard overwrites it
  }
  if (fin) {
    float* dst = fin + h * hs + (size_t)row * VD + c0 + cl;
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = acc[j];
  }
}


// Reverse fold of the state gradient over the shards of one sequence, for the
// backward pass.  With g_r the gradient of the state leaving shard r and B_r
// the gradient of the state entering shard r from the shard's own outputs (a
// zero leaving gradient), the entering gradient is P_r^T g_r + B_r, so
//     g_{n-1} = d_final (or 0),   g_{r-1} = P_r^T g_r + B_r,
// and d_initial = P_0^T g_0 + B_0.  `ends` receives every g_r.  Same
// workgroups and thread layout as the forward fold; P_r^T is read as columns
// of P_r, which the lanes of a wave load as consecutive rows.
__global__ void __launch_bounds__(256) kda_shard_scan_rev_kernel(const float* __restrict__ P,
                                                                 const float* __restrict__ B,
                                                                 const float* __restrict__ dfin,
                                                                 float* __restrict__ ends,
                                                                 float* __restrict__ dinit, int n_shards, int H) {
  __shared__ __attribute__((aligned(16))) float sS[KD][SLAB];
  const int h = blockIdx.x / NSLAB;
  const int c0 = (blockIdx.x % NSLAB) * SLAB;
  const int t = threadIdx.x;
  const int row = t >> 1;
  const int cl = 8 * (t & 1);
  const size_t hs = (size_t)KD * VD;

  float acc[8];
  {
    const float* src = dfin ? dfin + h * hs + (size_t)row * VD + c0 + cl : nullptr;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = src ? src[j] : 0.0f;
  }
  for (int r = n_shards - 1; r >= 0; --r) {
    float* dst = ends + ((size_t)r * H + h) * hs + (size_t)row * VD + c0 + cl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dst[j] = acc[j];
      sS[row][cl + j] = acc[j];
    }
    __syncthreads();
    const float* pcol = P + ((size_t)r * H + h) * KD * KD + row;  // P_r[k][row] at pcol[k * KD]
    const float* brow = B + ((size_t)r * H + h) * hs + (size_t)row * VD + c0 + cl;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = brow[j];
    for (int k = 0; k < KD; k += 4) {
      float pk[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) pk[kk] = pcol[(size_t)(k + kk) * KD];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float4 s0 = *reinterpret_cast<const float4*>(&sS[k + kk][cl]);
        const float4 s1 = *reinterpret_cast<const float4*>(&sS[k + kk][cl + 4]);
        acc[0] += pk[kk] * s0.x;
        acc[1] += pk[kk] * s0.y;
        acc[2] += pk[kk] * s0.z;
        acc[3] += pk[kk] * s0.w;
        acc[4] += pk[kk] * s1.x;
        acc[5] += pk[kk] * s1.y;
        acc[6] += pk[kk] * s1.z;
        acc[7] += pk[kk] * s1.w;
      }
    }
    __syncthreads();
  }
  if (dinit) {
    float* dst = dinit + h * hs + (size_t)row * VD + c0 + cl;
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = acc[j];
  }
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
