// Standalone launch of the chain kernel (kda_chain.h): two workgroups per
// (sequence, head) chain, one per 64-column half of the state, on records
// that an earlier intra-chunk kernel has finished writing.

#include "kda_chain.h"

namespace kda {
namespace {

constexpr int NQ = 2;  // 32-column quarters per workgroup

__global__ void __launch_bounds__(chain::NTHREADS, 2) kda_chain_kernel(ChainArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[chain::Lay<NQ>::LDS_BYTES];
  // XCD-aware ids: ids are dispatched round-robin over the 8 XCDs, so the two
  // halves of a chain get ids with equal residue mod 8 and read its records
  // through the same L2
  const int bid = blockIdx.x;
  const int r = bid >> 3;
  const int item = 8 * (r >> 1) + (bid & 7);
  const int half = r & 1;
  if (item >= a.map.N * a.H) return;
  const int pos = item / a.H;
  const int h = item - pos * a.H;
  const int seq = a.order ? a.order[pos] : pos;
  const ChainFused none{};
  chain::chain_run<false, NQ>(a, none, seq, h, 32 * NQ * half, smem);
}

}  // namespace

hipError_t launch_chain(const ChainArgs& args, hipStream_t st) {
  const int64_t items = (int64_t)args.map.N * args.H;
  if (items <= 0) return hipSuccess;
  // ids 16 r' + 8 half + x cover items 8 r' + x: round the item count up to 8
  const int64_t grid = 2 * ((items + 7) / 8) * 8;
  ChainArgs a = args;
  void* kargs[] = {(void*)&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&kda_chain_kernel), dim3((unsigned)grid),
                         dim3(chain::NTHREADS), kargs, 0, st);
}

}  // namespace kda
