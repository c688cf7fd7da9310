// kda_fwd_noalloc: the chunked forward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  The call's scratch (the intra kernel's work-item
// counter, the fault word, the varlen tables and the chunk records) lives in
// a file-scope device array of fixed size instead of a caller workspace.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.  The host never passes the array's name to
// a kernel (in host code it is only a stand-in for the symbol): on the first
// call on a device, with that device current, hipGetSymbolAddress resolves
// that device's copy, and every launch then receives that address.  The
// kernels themselves are the ones kda_fwd runs; they clear the counter and
// the fault word with a kernel at the start of every call, so nothing depends
// on what a previous call left in the array.

#include <mutex>

#include "../../include/kda.h"
#include "kda_host.h"

namespace kda {
namespace {

constexpr size_t kScratchBytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch alignment");

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

// This device's copy of `scratch`, resolved once per device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace kda

using namespace kda;

extern "C" {

kda_status_t kda_fwd_noalloc(const void* q, const void* k, const void* v, const void* raw_gate,
                             const void* raw_beta, float scale, void* out, const float* A_log,
                             const float* dt_bias, float lower_bound, const float* initial_state,
                             float* final_state, const int32_t* cu_seqlens, int64_t B, int64_t T, int64_t H,
                             int64_t K, int64_t V, int64_t N, void* stream) {
  if (B < 1 || T < 0 || H < 1 || N < 1) return KDA_ERR_INVALID;
  // the exact layout of this call (not the bound kda_workspace_size reports)
  if (workspace_layout(B * T, H, N).total > kScratchBytes) return KDA_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return launch_status(e, "scratch address");
  return kda_fwd(q, k, v, raw_gate, raw_beta, scale, out, ws, kScratchBytes, A_log, dt_bias, lower_bound,
                 initial_state, final_state, cu_seqlens, B, T, H, K, V, N, stream);
}

}  // extern "C"
