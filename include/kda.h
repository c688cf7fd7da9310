/*
 * kda.h — C ABI of the MI355X (gfx950) KDA chunked forward library (libkda.so).
 *
 * KDA (Kimi Delta Attention) is a gated delta-rule linear attention with a
 * per-channel decay gate.  Per sequence and head it carries a K x V fp32 state
 * S and, token by token, computes
 *     q^ = q / sqrt(|q|^2 + 1e-6),  k^ = k / sqrt(|k|^2 + 1e-6)
 *     beta  = sigmoid(raw_beta)
 *     g_c   = lower_bound * sigmoid(exp(A_log[h]) * (raw_gate_c + dt_bias[h, c]))
 *     S     = (I - beta k^ k^T) Diag(exp(g)) S + beta k^ v^T
 *     o     = scale * S^T q^
 * The library evaluates this with 64-token chunks (partial tail chunks
 * allowed) on one GPU.
 *
 * Sources.  The argument list and roles follow the 14-argument
 * torch.ops._flashkda_C.fwd call and get_workspace_size(T, H, N) in the vLLM
 * PR report "[Kimi-K3] Bump FlashKDA to fix unstable inverse" (section
 * "关键源码片段", the near-collinear-keys test).  The in-kernel L2 norm, beta
 * sigmoid and gate come from the chunk_kda flags on the instagit page "What
 * CUDA Version Is Required to Use FlashKDA?" (section "Usage Examples").  The
 * pages never print the gate formula; the one above is this library's stated
 * reading, as is eps = 1e-6 and reading the output from the updated state.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous,
 *     in the layouts given below.  Per-token arrays (q, k, v, raw_gate,
 *     raw_beta, out) may be NULL when the call has no tokens (B * T == 0).  The library never allocates, frees or
 *     synchronises; kda_fwd is asynchronous on `stream`.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Argument checks happen on the host before any device work; a rejected
 *     call returns its status and touches no memory.
 *   - There is no fallback path: unsupported shapes are rejected.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_SUCCESS = 0,
  KDA_ERR_INVALID = 1,     /* NULL required pointer, bad sizes, inconsistent B/N */
  KDA_ERR_UNSUPPORTED = 2, /* head dims or lower_bound outside what the entry point supports */
  KDA_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than kda_workspace_size() */
  KDA_ERR_LAUNCH = 4       /* a kernel launch failed (hipGetLastError after launch) */
} kda_status_t;

/*
 * Bytes of device workspace kda_fwd needs for T_total packed tokens, H heads
 * and N sequences (the page's get_workspace_size(T, H, 1) for one sequence).
 * The caller allocates it (any alignment >= 256 bytes) and passes it to
 * kda_fwd.  Its contents are scratch: undefined before a call, and afterwards
 * meaningful only as the chunk records that KDA_FLAG_REUSE_RECORDS lets a
 * following call with the same inputs reuse.
 * Returns 0 if any argument is < 1 (T_total may be 0).
 */
size_t kda_workspace_size(int64_t T_total, int64_t H, int64_t N);

/*
 * 1 if kda_fwd supports head dims K, V with this lower_bound, else 0 (the
 * page's is_flashkda_supported(128, bf16, lower_bound) probe, whose first
 * argument is the head size).  Supported: K and V each 64 or 128, and
 * -5 <= lower_bound <= 0.  The -5 limit keeps every 16-token decay ratio
 * inside fp32/bf16 range (exp(16 * 5) < FLT_MAX).  kda_fwd, kda_fwd_ex,
 * kda_decode, kda_bwd and kda_bwd_ex take every supported pair;
 * kda_shard_affine and kda_shard_scan take K == V == 128 only
 * (KDA_ERR_UNSUPPORTED otherwise).
 * Head dim 64 runs in the 128-channel layout of the kernels with the missing
 * channels held at zero, so it costs about what 128 costs.
 */
int kda_is_supported(int64_t K, int64_t V, float lower_bound);

/*
 * KDA chunked forward.
 *
 *   q, k        bf16 [B, T, H, K]   (q == k is allowed: the pages pass one
 *                                    tensor twice)
 *   v           bf16 [B, T, H, V]
 *   raw_gate    bf16 [B, T, H, K]   (pre-activation gate)
 *   raw_beta    bf16 [B, T, H]      (pre-sigmoid write strength)
 *   scale       output scale (e.g. K^-0.5)
 *   out         bf16 [B, T, H, V]   written; must not overlap any input
 *   workspace   device scratch of workspace_bytes >= kda_workspace_size(B*T, H, N)
 *   A_log       fp32 [H]
 *   dt_bias     fp32 [H, K]
 *   lower_bound log-decay floor, in [-5, 0]
 *   initial_state fp32 [N, H, K, V] (S[k][v] at offset k*V + v), or NULL for zeros
 *   final_state   fp32 [N, H, K, V] written, or NULL to skip; may equal
 *                 initial_state (in-place update)
 *   cu_seqlens  int32 [N + 1] device array of packed sequence offsets, or NULL.
 *               With cu_seqlens, B must be 1 and T is the packed token count;
 *               cu_seqlens[0] == 0, non-decreasing, cu_seqlens[N] == T is the
 *               caller's contract (not checked: that would need a device sync).
 *               Zero-length sequences are allowed (final = initial).
 *               Without cu_seqlens there are N == B sequences of length T.
 *   B, T, H, K, V, N sizes as above (T >= 0; B, H, N >= 1)
 *   stream      hipStream_t as void*
 *
 * The call builds the chunk records of all chunks first (one launch) and runs
 * the recurrence over them afterwards (a second launch); kda_fwd_ex with
 * KDA_FLAG_SINGLE_LAUNCH offers a one-launch pipeline for one sequence.
 *
 * With few (sequence, head) pairs and long sequences (states not in place, not
 * KDA_FLAG_STATE_VK), the call runs its recurrence on shards of each sequence
 * and folds their affine maps (the kda_shard_affine / kda_shard_scan algebra)
 * to shorten the sequential chain.  The shard count follows the mean length
 * T_total / N; with cu_seqlens each sequence is cut by its own length.
 * kda_workspace_size already covers it.
 *
 * Returns KDA_SUCCESS after enqueueing the work, or an error status.
 */
kda_status_t kda_fwd(const void* q, const void* k, const void* v, const void* raw_gate,
                     const void* raw_beta, float scale, void* out, void* workspace,
                     size_t workspace_bytes, const float* A_log, const float* dt_bias,
                     float lower_bound, const float* initial_state, float* final_state,
                     const int32_t* cu_seqlens, int64_t B, int64_t T, int64_t H, int64_t K,
                     int64_t V, int64_t N, void* stream);

/*
 * Per-shard affine map, for splitting one long sequence over several devices
 * (context parallelism: the torchtitan PR page names KDA context parallelism,
 * KCP, in its "Summary" section, without giving an algorithm).  The gated
 * delta rule is affine in the state, so each sequence of the call (a shard)
 * maps the state it is entered with, S, to
 *     S_end = P S + R,
 * where P (K x K) is the product of the per-token maps (I - b k k^T) Diag(a)
 * over the shard and R is the shard's final state from a zero start.
 *
 *   q, k, v, raw_gate, raw_beta, workspace, A_log, dt_bias, lower_bound,
 *   cu_seqlens, B, T, H, K, V, N   exactly as for kda_fwd (no scale or out:
 *                                  no outputs are produced)
 *   P   fp32 [N, H, K, K] written: P[n][h][i][j] multiplies S[j][:] into row i
 *   R   fp32 [N, H, K, V] written
 *
 * Needs K == V == 128 (P is computed as the final state of the V = 0
 * recurrence from S = I).  Shards then combine with kda_shard_scan, and kda_fwd with the
 * scanned entering states as initial_state produces the shards' outputs.
 * Same errors as kda_fwd; P and R must not overlap the inputs.
 */
kda_status_t kda_shard_affine(const void* q, const void* k, const void* v, const void* raw_gate,
                              const void* raw_beta, void* workspace, size_t workspace_bytes,
                              const float* A_log, const float* dt_bias, float lower_bound, float* P,
                              float* R, const int32_t* cu_seqlens, int64_t B, int64_t T, int64_t H,
                              int64_t K, int64_t V, int64_t N, void* stream);

/*
 * Fold the affine maps of n_shards consecutive shards of one sequence:
 *     starts[0] = initial_state (or zeros),
 *     starts[r + 1] = P[r] starts[r] + R[r],
 * in fp32, and final_state = P[n-1] starts[n-1] + R[n-1].
 *
 *   P       fp32 [n_shards, H, K, K]   from kda_shard_affine
 *   R       fp32 [n_shards, H, K, V]   from kda_shard_affine
 *   initial_state fp32 [H, K, V] or NULL for zeros
 *   starts  fp32 [n_shards, H, K, V] written (the entering state of every shard,
 *           ready to pass as kda_fwd's initial_state for the shard batch)
 *   final_state fp32 [H, K, V] written, or NULL to skip
 *
 * Supported: K == V == 128.  Returns KDA_ERR_INVALID for NULL P, R or starts
 * or n_shards, H < 1; outputs must not overlap the inputs.
 */
kda_status_t kda_shard_scan(const float* P, const float* R, const float* initial_state, float* starts,
                            float* final_state, int64_t n_shards, int64_t H, int64_t K, int64_t V,
                            void* stream);

/*
 * Token-by-token step for decoding and short continuations: B sequences of T
 * tokens each (T small, typically 1), applying the same per-token gated delta
 * rule as kda_fwd directly in fp32 (the serving decode path named in the vLLM
 * PR report's risk section).  The state is read once, kept on chip across the
 * T tokens and written once, so the cost is the state's 2 x 64 KiB of HBM
 * traffic per sequence and head; no workspace is needed.
 *
 *   q, k, raw_gate  bf16 [B, T, H, K];  v, out bf16 [B, T, H, V];  raw_beta bf16 [B, T, H]
 *   scale, A_log fp32 [H], dt_bias fp32 [H, K], lower_bound   as for kda_fwd
 *   initial_state fp32 [B, H, K, V] or NULL for zeros
 *   final_state   fp32 [B, H, K, V] written, or NULL; may equal initial_state
 *                 (the usual in-place decode update)
 *   B, H >= 1, T >= 0; K and V each 64 or 128, lower_bound in [-5, 0]
 *
 * Returns KDA_SUCCESS after enqueueing, KDA_ERR_INVALID / KDA_ERR_UNSUPPORTED
 * from the host checks, or KDA_ERR_LAUNCH.  For long prompts use kda_fwd,
 * whose chunked form is far faster per token; both give the same results up
 * to rounding.
 */
kda_status_t kda_decode(const void* q, const void* k, const void* v, const void* raw_gate,
                        const void* raw_beta, float scale, void* out, const float* A_log,
                        const float* dt_bias, float lower_bound, const float* initial_state,
                        float* final_state, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                        void* stream);

/*
 * Variants of kda_fwd (kda_fwd_ex `flags`), the in-kernel switches of the
 * chunk_kda call on the instagit FlashKDA page ("Usage Examples"):
 *   KDA_FLAG_GATE_GIVEN  (use_gate_in_kernel off) raw_gate already holds the
 *       natural-log decay g, bf16.  Every g must lie in [lower_bound, 0]: the
 *       range the in-kernel gate maps into, which the page's chunk_kda call
 *       bounds with safe_gate=True and lower_bound.  That is the caller's
 *       contract (checking it on the host would need the data): a value
 *       outside it sets KDA_FAULT_GATE_RANGE in the workspace's fault word
 *       (kda_workspace_faults), and the results are then unspecified.
 *       A_log and dt_bias are unused and may be NULL.
 *   KDA_FLAG_BETA_GIVEN  (use_beta_sigmoid_in_kernel off) raw_beta already
 *       holds beta; keep it in [0, 1] for the documented accuracy.
 *   KDA_FLAG_NO_QK_NORM  (use_qk_l2norm_in_kernel off) q and k are used as
 *       given; the caller keeps |k|, |q| <= 1 (the rule is only stable for
 *       beta |k|^2 <= 2, and the kernel's fp16 operands assume unit scale).
 *       A row with |q|^2 or |k|^2 above 1 + 1/16 sets KDA_FAULT_QK_NORM in
 *       the fault word; the call still runs, at unspecified accuracy.
 *   KDA_FLAG_STATE_VK    (transpose_state_layout) initial_state and
 *       final_state are stored transposed, [N, H, V, K]: S[k][v] at v*K + k.
 */
#define KDA_FLAG_GATE_GIVEN 1u
#define KDA_FLAG_BETA_GIVEN 2u
#define KDA_FLAG_NO_QK_NORM 4u
#define KDA_FLAG_STATE_VK 8u

/*
 * KDA_FLAG_REUSE_RECORDS (kda_fwd_ex, kda_bwd_ex): skip the intra-chunk pass and use
 * the per-(chunk, head) records that the previous call on this workspace left
 * there, for the second pass of the split-sequence flow (the KCP item of the
 * torchtitan PR page, "Summary"): kda_shard_affine, kda_shard_scan, then
 * kda_fwd_ex over the same shard batch from the scanned entering states; or for
 * a backward after its forward (kda_bwd_ex after kda_fwd_ex with
 * KDA_FLAG_KEEP_RECORDS on the backward-sized workspace).  Records are left in
 * the workspace by kda_shard_affine and by kda_fwd_ex with KDA_FLAG_KEEP_RECORDS;
 * a forward without it may keep only a bounded ring of them.  The records
 * depend on q, k, raw_gate, raw_beta, A_log, dt_bias, lower_bound, cu_seqlens,
 * B, T, H, N and the GATE_GIVEN, BETA_GIVEN and NO_QK_NORM bits, not on v or
 * the states.  The caller guarantees that all of these equal those of the call
 * that wrote the records and that the workspace is unchanged since; nothing
 * checks it, and other records give wrong results.  A backward uses up the
 * records: it writes its own factor record over them once its checkpointing
 * pass has read them (unless the call splits its sequences into shards), so a
 * second backward on the same records needs the forward again.
 */
#define KDA_FLAG_REUSE_RECORDS 16u

/*
 * KDA_FLAG_KEEP_RECORDS (kda_fwd_ex only): build every chunk record into the
 * workspace and leave it there for a later call with KDA_FLAG_REUSE_RECORDS
 * (this rules out KDA_FLAG_SINGLE_LAUNCH).
 */
#define KDA_FLAG_KEEP_RECORDS 32u

/*
 * KDA_FLAG_SINGLE_LAUNCH (kda_fwd_ex only): with one sequence (N == 1), at
 * least 16 heads, no shard split and a GPU of 8 equal XCDs (MI355X), run the
 * forward as one persistent launch: per XCD, workgroups that build the chunk
 * records of that XCD's heads hand them, through a small ring in the XCD's
 * L2, to one workgroup per head that runs the recurrence, so records need not
 * travel to HBM and back.  It gives the same bits as the two-launch schedule.
 * Where the call does not meet these conditions the bit is ignored; it is
 * also ignored with KDA_FLAG_KEEP_RECORDS or KDA_FLAG_REUSE_RECORDS.
 */
#define KDA_FLAG_SINGLE_LAUNCH 64u

/*
 * kda_fwd with variant flags (any OR of the KDA_FLAG_* bits above,
 * KDA_FLAG_KEEP_RECORDS and KDA_FLAG_SINGLE_LAUNCH; other bits give KDA_ERR_INVALID).  Every other argument is as for kda_fwd, and
 * kda_fwd(...) == kda_fwd_ex(..., 0, stream).
 */
kda_status_t kda_fwd_ex(const void* q, const void* k, const void* v, const void* raw_gate,
                        const void* raw_beta, float scale, void* out, void* workspace,
                        size_t workspace_bytes, const float* A_log, const float* dt_bias,
                        float lower_bound, const float* initial_state, float* final_state,
                        const int32_t* cu_seqlens, int64_t B, int64_t T, int64_t H, int64_t K,
                        int64_t V, int64_t N, unsigned flags, void* stream);

/*
 * Bytes of device workspace kda_bwd needs for T_total packed tokens, H heads
 * and N sequences (more than kda_workspace_size: the backward keeps fp32
 * per-chunk states, state gradients and chunk factors).  Returns 0 if any
 * argument is < 1 (T_total may be 0).
 */
size_t kda_bwd_workspace_size(int64_t T_total, int64_t H, int64_t N);

/*
 * Gradients of kda_fwd.  The torchtitan page "[Kimi K3] allow KDA using inline
 * Attention Gym reference eager implementation ..." (section "Results") runs
 * the KDA kernel's forward and gradient against packed-versus-separate
 * documents; the pages print no backward algorithm.  This computes the exact
 * gradient of
 *     loss = <d_out, out> + <d_final, final_state>
 * of the kda_fwd call with the same inputs (flags 0), with respect to every
 * input, by reverse-mode differentiation of the chunked algebra (fp32
 * arithmetic; the forward states it needs are recomputed inside the call).
 * Where kda_fwd splits sequences into shards inside the call, both the
 * recomputed forward recurrence and the reverse one run on those shards, the
 * reverse one from leaving gradients folded in reverse shard order; results
 * match the unsplit path up to rounding order.
 *
 *   q, k, v, raw_gate, raw_beta, scale, A_log, dt_bias, lower_bound,
 *   initial_state, cu_seqlens, B, T, H, K, V, N   exactly as for kda_fwd
 *                (A_log and dt_bias are required)
 *   d_out        bf16 [B, T, H, V]   gradient of out
 *   d_final      fp32 [N, H, K, V]   gradient of final_state, or NULL for zero
 *   dq, dk       bf16 [B, T, H, K]   written
 *   dv           bf16 [B, T, H, V]   written
 *   d_raw_gate   bf16 [B, T, H, K]   written
 *   d_raw_beta   bf16 [B, T, H]      written
 *   dA_log       fp32 [H]            written
 *   d_dt_bias    fp32 [H, K]         written
 *   d_initial_state fp32 [N, H, K, V] written, or NULL to skip; may equal d_final
 *   workspace    device scratch of >= kda_bwd_workspace_size(B*T, H, N) bytes
 *
 * Outputs must not overlap the inputs or each other (except as stated).
 * Same errors as kda_fwd; KDA_ERR_INVALID also for a NULL required output.
 */
kda_status_t kda_bwd(const void* q, const void* k, const void* v, const void* raw_gate,
                     const void* raw_beta, float scale, const void* d_out, const float* d_final,
                     void* dq, void* dk, void* dv, void* d_raw_gate, void* d_raw_beta, float* dA_log,
                     float* d_dt_bias, float* d_initial_state, void* workspace, size_t workspace_bytes,
                     const float* A_log, const float* dt_bias, float lower_bound,
                     const float* initial_state, const int32_t* cu_seqlens, int64_t B, int64_t T,
                     int64_t H, int64_t K, int64_t V, int64_t N, void* stream);

/*
 * kda_bwd for the variants of kda_fwd_ex (any OR of KDA_FLAG_GATE_GIVEN,
 * KDA_FLAG_BETA_GIVEN, KDA_FLAG_NO_QK_NORM, KDA_FLAG_STATE_VK and
 * KDA_FLAG_REUSE_RECORDS; other bits give KDA_ERR_INVALID): the gradients of the kda_fwd_ex call with the
 * same inputs and flags.  With KDA_FLAG_GATE_GIVEN, d_raw_gate is the gradient
 * with respect to the given decay (which must lie in [lower_bound, 0], as for
 * kda_fwd_ex); A_log and dt_bias are
 * unused and may be NULL, and dA_log, d_dt_bias may be NULL (else zero-filled).
 * With KDA_FLAG_BETA_GIVEN, d_raw_beta is the gradient with respect to beta;
 * with KDA_FLAG_NO_QK_NORM, dq and dk are those of the unnormalised q, k; with
 * KDA_FLAG_STATE_VK, initial_state, d_final and d_initial_state are [N, H, V, K].
 * With KDA_FLAG_REUSE_RECORDS the gradients use the chunk records that a
 * kda_fwd / kda_fwd_ex call with the same inputs and flags left at the start of
 * this workspace (the backward workspace begins with the forward's layout), and
 * the intra-chunk pass is skipped; the conditions are those of kda_fwd_ex.
 * kda_bwd(...) == kda_bwd_ex(..., 0, stream).
 */
kda_status_t kda_bwd_ex(const void* q, const void* k, const void* v, const void* raw_gate,
                        const void* raw_beta, float scale, const void* d_out, const float* d_final,
                        void* dq, void* dk, void* dv, void* d_raw_gate, void* d_raw_beta, float* dA_log,
                        float* d_dt_bias, float* d_initial_state, void* workspace, size_t workspace_bytes,
                        const float* A_log, const float* dt_bias, float lower_bound,
                        const float* initial_state, const int32_t* cu_seqlens, int64_t B, int64_t T,
                        int64_t H, int64_t K, int64_t V, int64_t N, unsigned flags, void* stream);

/*
 * Faults the kernels of a kda_fwd / kda_fwd_ex / kda_shard_affine / kda_bwd /
 * kda_bwd_ex call detect on the device, where no status can be returned.
 * Each such call clears the fault word of its workspace when it starts and
 * ORs these bits into it:
 *   KDA_FAULT_WAIT_TIMEOUT  a bounded wait between waves or workgroups gave
 *                           up: the call's results are invalid
 *   KDA_FAULT_GATE_RANGE    KDA_FLAG_GATE_GIVEN with a decay outside
 *                           [lower_bound, 0]
 *   KDA_FAULT_QK_NORM       KDA_FLAG_NO_QK_NORM with |q|^2 or |k|^2 > 1 + 1/16
 *   KDA_FAULT_PLACEMENT     KDA_FLAG_SINGLE_LAUNCH: workgroups whose ids agree
 *                           mod 8 (planned as one XCD's share, handing records
 *                           over through its L2) ran on two different XCDs:
 *                           the results are invalid
 */
#define KDA_FAULT_WAIT_TIMEOUT 1u
#define KDA_FAULT_GATE_RANGE 2u
#define KDA_FAULT_QK_NORM 4u
#define KDA_FAULT_PLACEMENT 8u

/*
 * Read the fault word of the last call on `workspace` (a device buffer passed
 * to one of the calls above) into *faults, after the work already enqueued on
 * `stream` (hipStream_t as void*) has finished: unlike every other entry
 * point, this one synchronises the stream.  Returns KDA_ERR_INVALID for NULL
 * arguments, KDA_ERR_LAUNCH if the copy fails, else KDA_SUCCESS.
 */
kda_status_t kda_workspace_faults(const void* workspace, uint32_t* faults, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  kda_fwd
 * with the same arguments minus the workspace, whose scratch (counter, fault
 * word, varlen tables, chunk records) is instead a static device array of
 * KDA_NOALLOC_SCRATCH_BYTES inside the library.  Every GPU the library runs on
 * holds its own copy of that array until the process ends.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 *
 * Limits and sharing:
 *   - the call's workspace layout must fit: kda_workspace_size-sized calls up
 *     to KDA_NOALLOC_SCRATCH_BYTES (e.g. B=2, T=4096, H=12 needs about 142 MB);
 *     larger calls return KDA_ERR_WORKSPACE before any device work;
 *   - every call on one GPU uses that GPU's one array: calls that overlap on a
 *     GPU (different streams, host threads or processes sharing a context)
 *     race and give wrong results; serialise them;
 *   - the array keeps the last call's contents, which no call depends on (the
 *     kernels clear the counter and fault word themselves);
 *   - kda_workspace_faults is not available for it (the array has no host
 *     handle); the kernels' bounded waits are the same as kda_fwd's.
 * Arguments, layouts, results and other errors are those of kda_fwd.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)
kda_status_t kda_fwd_noalloc(const void* q, const void* k, const void* v, const void* raw_gate,
                             const void* raw_beta, float scale, void* out, const float* A_log,
                             const float* dt_bias, float lower_bound, const float* initial_state,
                             float* final_state, const int32_t* cu_seqlens, int64_t B, int64_t T, int64_t H,
                             int64_t K, int64_t V, int64_t N, void* stream);

/* Static, human-readable name of a status code. */
const char* kda_status_string(kda_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
