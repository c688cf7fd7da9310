// Standalone launch of the chain kernel (kda_chain.h): one workgroup per
// (sequence, head) chain, on records that an earlier intra-chunk kernel has
// finished writing.

#include "kda_chain.h"

namespace kda {
namespace {

__global__ void __launch_bounds__(chain::NTHREADS, 2) kda_chain_kernel(ChainArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[chain::LDS_BYTES];
  const int item = blockIdx.x;
  if (item >= a.map.N * a.H) return;
  const int pos = item / a.H;
  const int h = item - pos * a.H;
  const int seq = a.order ? a.order[pos] : pos;
  const ChainFused none{};
  chain::chain_run<false>(a, none, seq, h, smem);
}

}  // namespace

hipError_t launch_chain(const ChainArgs& args, hipStream_t st) {
  const int64_t items = (int64_t)args.map.N * args.H;
  if (items <= 0) return hipSuccess;
  ChainArgs a = args;
  void* kargs[] = {(void*)&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&kda_chain_kernel), dim3((unsigned)items),
                         dim3(chain::NTHREADS), kargs, 0, st);
}

}  // namespace kda
