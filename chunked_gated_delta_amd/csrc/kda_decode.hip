// Token-by-token KDA step for decoding and short continuations: B sequences of
// T tokens each (T small, typically 1), the fp32 state updated in place.  It
// applies the per-token gated delta rule directly,
//     S = Diag(exp(g)) S;  d = b (v - S^T k^);  S = S + k^ d^T;  o = scale S^T q^,
// with q^, k^ = x / sqrt(|x|^2 + 1e-6), b = sigmoid(raw_beta) and
// g = lower_bound * sigmoid(exp(A_log) (raw_gate + dt_bias)), the same op and
// argument roles as the chunked forward (vLLM PR report, "关键源码片段";
// instagit FlashKDA page, "Usage Examples"), for the serving path that the
// vLLM report's risk section mentions.  All arithmetic is fp32.
//
// The work is bound by the state's HBM traffic (4 K V bytes read and written
// per sequence and head), so it runs on the vector ALUs: one workgroup of 256
// threads per (sequence, head, 32-column slice).  Thread t owns column
// j = t % 32 of the slice and rows (K / 8) (t / 32) .. + K / 8 - 1, so a state
// row of the slice is one contiguous 128-byte access per 32 lanes.  Per token,
// threads 0..K-1 compute the per-channel factors (normalised k and q, exp(g))
// into LDS; the two column reductions S^T k^ and S^T q^ go through LDS.  The
// head dims K, V (64 or 128 each) are template parameters.

#include "../../include/kda.h"
#include "kda_common.h"

namespace kda {
namespace {

constexpr int DT = 256;       // threads
constexpr int DSL = 32;       // state columns per workgroup
constexpr int NRG = DT / DSL; // row groups

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  uint16_t* out;
  const float* A_log;
  const float* dt_bias;
  const float* init;
  float* fin;
  float scale;
  float lb2;  // lower_bound * log2(e)
  int B, T, H;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

template <int KK, int VV>
__global__ void __launch_bounds__(DT) kda_decode_kernel(DecodeArgs a) {
  constexpr int NDSL = VV / DSL;  // slices per (sequence, head)
  constexpr int DRG = KK / NRG;   // rows per thread
  constexpr int NKW = KK / 64;    // waves holding the per-channel factors
  __shared__ float sK[KK], sQ[KK], sE[KK];  // k^, q^, exp(g) of the current token
  __shared__ float sRed[2][NRG][DSL];       // column partial sums (S^T k^, S^T q^)
  __shared__ float sNorm[NKW][2];           // per-wave partial |k|^2, |q|^2 (threads 0..K-1)
  __shared__ float sBeta;

  const int H = a.H;
  const int sl = blockIdx.x % NDSL;
  const int bh = blockIdx.x / NDSL;  // b * H + h
  const int h = bh % H;
  const int b = bh / H;
  const int t = threadIdx.x;
  const int j = t % DSL;
  const int rg = t / DSL;
  const int col = sl * DSL + j;
  const size_t st0 = (size_t)bh * KK * VV;

  float S[DRG];
#pragma unroll
  for (int r = 0; r < DRG; ++r) S[r] = a.init ? a.init[st0 + (size_t)(DRG * rg + r) * VV + col] : 0.0f;

  // per-channel constants of this head (threads 0..K-1 own channel t)
  const float na = -__expf(a.A_log[h]) * LOG2E;
  const float nb = t < KK ? na * a.dt_bias[h * KK + t] : 0.0f;

  for (int tok = 0; tok < a.T; ++tok) {
    const size_t row = ((size_t)b * a.T + tok) * H + h;  // token row of [B, T, H, *]
    // ---- per-channel factors of this token
    if (t < KK) {
      const float kv = bf16_to_f32(a.k[row * KK + t]);
      const float qv = bf16_to_f32(a.q[row * KK + t]);
      const float gv = bf16_to_f32(a.g[row * KK + t]);
      float ssk = kv * kv, ssq = qv * qv;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        ssk += __shfl_xor(ssk, m);
        ssq += __shfl_xor(ssq, m);
      }
      if ((t & 63) == 0) {
        sNorm[t >> 6][0] = ssk;
        sNorm[t >> 6][1] = ssq;
      }
      // exp(g) = 2^(lb2 * sigmoid(exp(A_log) (raw_gate + dt_bias)))
      sE[t] = __builtin_amdgcn_exp2f(a.lb2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gv * na + nb)));
      sK[t] = kv;
      sQ[t] = qv;
      if (t == 0) sBeta = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-bf16_to_f32(a.beta[row]) * LOG2E));
    }
    __syncthreads();
    float nk = 0.0f, nq = 0.0f;
#pragma unroll
    for (int u = 0; u < NKW; ++u) {
      nk += sNorm[u][0];
      nq += sNorm[u][1];
    }
    const float rk = __builtin_amdgcn_rsqf(nk + L2_EPS);
    const float rq = __builtin_amdgcn_rsqf(nq + L2_EPS);
    const float beta = sBeta;
    const float vj = bf16_to_f32(a.v[row * VV + col]);

    // ---- decay, then this thread's part of S^T k^
    float pk = 0.0f;
#pragma unroll
    for (int r = 0; r < DRG; ++r) {
      const int i = DRG * rg + r;
      S[r] *= sE[i];
      pk += S[r] * sK[i];
    }
    sRed[0][rg][j] = pk;
    __syncthreads();
    float dk = 0.0f;
#pragma unroll
    for (int u = 0; u < NRG; ++u) dk += sRed[0][u][j];
    const float delta = beta * (vj - dk * rk);

    // ---- write, then this thread's part of S^T q^
    float pq = 0.0f;
#pragma unroll
    for (int r = 0; r < DRG; ++r) {
      const int i = DRG * rg + r;
      S[r] += (sK[i] * rk) * delta;
      pq += S[r] * sQ[i];
    }
    sRed[1][rg][j] = pq;
    __syncthreads();
    if (rg == 0) {
      float o = 0.0f;
#pragma unroll
      for (int u = 0; u < NRG; ++u) o += sRed[1][u][j];
      a.out[row * VV + col] = __builtin_bit_cast(uint16_t, (__bf16)(o * rq * a.scale));
    }
    // the next token overwrites sK/sQ/sE/sNorm/sRed only after everyone has read them
    __syncthreads();
  }
  if (a.fin) {
#pragma unroll
    for (int r = 0; r < DRG; ++r) a.fin[st0 + (size_t)(DRG * rg + r) * VV + col] = S[r];
  }
}

}  // namespace
}  // namespace kda

using namespace kda;

extern "C" kda_status_t kda_decode(const void* q, const void* k, const void* v, const void* raw_gate,
                                   const void* raw_beta, float scale, void* out, const float* A_log,
                                   const float* dt_bias, float lower_bound, const float* initial_state,
                                   float* final_state, int64_t B, int64_t T, int64_t H, int64_t K,
                                   int64_t V, void* stream) {
  if (B < 1 || T < 0 || H < 1 || !(scale == scale)) return KDA_ERR_INVALID;
  // token arrays may be NULL only when there are no tokens (empty tensors)
  if (T > 0 && (!q || !k || !v || !raw_gate || !raw_beta || !out)) return KDA_ERR_INVALID;
  if (!A_log || !dt_bias) return KDA_ERR_INVALID;
  if (!kda_is_supported(K, V, lower_bound)) return KDA_ERR_UNSUPPORTED;  // K, V each 64 or 128
  const int64_t ndsl = V / DSL;
  if (B * H * ndsl > ((int64_t)1 << 31) - 1 || B * T * H > ((int64_t)1 << 40)) return KDA_ERR_INVALID;
  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.g = static_cast<const uint16_t*>(raw_gate);
  a.beta = static_cast<const uint16_t*>(raw_beta);
  a.out = static_cast<uint16_t*>(out);
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.init = initial_state;
  a.fin = final_state;
  a.scale = scale;
  a.lb2 = lower_bound * LOG2E;
  a.B = (int)B;
  a.T = (int)T;
  a.H = (int)H;
  void* args[] = {(void*)&a};
  const void* fn = K == KD ? (V == VD ? reinterpret_cast<const void*>(&kda_decode_kernel<KD, VD>)
                                      : reinterpret_cast<const void*>(&kda_decode_kernel<KD, 64>))
                           : (V == VD ? reinterpret_cast<const void*>(&kda_decode_kernel<64, VD>)
                                      : reinterpret_cast<const void*>(&kda_decode_kernel<64, 64>));
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)(B * H * ndsl)), dim3(DT), args, 0,
                                       reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_SUCCESS : KDA_ERR_LAUNCH;
}
