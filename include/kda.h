/*
 * kda.h — C ABI of the MI355X (gfx950) KDA library, libkda.so.
 *
 * KDA (Kimi Delta Attention) is a gated delta-rule linear attention: each
 * head keeps a fixed-size state S (K x V, fp32) instead of a KV cache, and
 * every token applies, per batch row b and head h,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * with a per-key-channel forget gate alpha_t = exp(g_t), g clamped to
 * [-5, 0] (alpha in [e^-5, 1]) inside the library.
 *
 * Page: "Kimi K3 — открытая модель, которая обошла закрытых лидеров рынка"
 * (aiblin.ru).  Section "Как хранить миллион токенов в памяти": the state
 * matrix S of fixed size, the delta rule (partly erase, then write), beta as
 * write strength in [0, 1], alpha as forgetting coefficient and its clamp to
 * [e^-5, 1].  Section "Как распараллелили последовательное обновление":
 * chunk-parallel evaluation (all tokens of a chunk at once, then the state
 * passed on, in parallel over heads) and the one-card segment planner for
 * long prefill (per segment a local state and a transition matrix,
 * recombined exactly).  The update formula itself is lost on the page; the
 * equation above is the reading used throughout.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers (HIP), row-major, contiguous.
 *     Alignment: states and the workspace 16 bytes; for prefill q, k, v, g
 *     and o 16 bytes and beta its element size; for decode every token
 *     tensor its element size.  The caller owns every buffer, the workspace
 *     included; the library allocates no device memory.
 *   - Work is enqueued asynchronously on `stream` (NULL is the default
 *     stream) of the current HIP device.  Nothing is synchronised.
 *   - Arguments are validated on the host before anything is launched; on an
 *     error nothing is launched.  KDA_ERR_INVALID_ARG: a null pointer, a
 *     negative size, a misaligned pointer, a partially overlapping state
 *     pair.  KDA_ERR_UNSUPPORTED: sizes or a dtype the kernels do not
 *     implement.  KDA_ERR_WORKSPACE: workspace missing or too small.
 *     KDA_ERR_HIP: a HIP launch or query failed.
 *   - Token tensors (q, k, v, g, beta, o) share one dtype `dt`; states are
 *     always fp32.  o is rounded to `dt` (round to nearest even).
 *   - Results are deterministic: no floating-point atomics.
 *   - The library keeps no state between calls and every call is reentrant,
 *     with one opt-in exception: the launch timing of kda_profile_start /
 *     kda_profile_stop below keeps one process-wide record (guarded by a
 *     mutex) while it is on.
 *   - Non-finite inputs propagate; they are not detected.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>   /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,
    KDA_ERR_UNSUPPORTED = 2,
    KDA_ERR_WORKSPACE = 3,
    KDA_ERR_HIP = 4,
    /* never returned: they stretch the enum's value range over all of int,
     * so that any code a caller passes to kda_status_string is a valid
     * kda_status (in C++ a value outside the range is undefined) */
    KDA_STATUS_RANGE_MIN_ = -2147483647 - 1,
    KDA_STATUS_RANGE_MAX_ = 2147483647
} kda_status;

typedef enum kda_dtype {
    KDA_F32 = 0,
    KDA_BF16 = 1,
    /* never valid: the same value range as kda_status, so that an unknown
     * code reaches the argument checks (which reject it) with defined
     * behaviour */
    KDA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    KDA_DTYPE_RANGE_MAX_ = 2147483647
} kda_dtype;

/*
 * Execution plan of a prefill call.
 *   split:   1 = single pass: one kernel per (b, h, segment, column block)
 *            walks the chunks and does all chunk work in order;
 *            2 = two passes: an intra-chunk pass over every (b, h, chunk) at
 *            once writes per-chunk operands to the workspace, then a state
 *            pass walks the chunks (the workspace holds those records);
 *            3 = token-serial: one workgroup per (b, h, 64-column block)
 *            applies the recurrence token by token (the defining equation of
 *            the page's section "Как хранить миллион токенов в памяти"), the
 *            state in registers; no workspace, n_seg 1, v_block 64.  The
 *            library's choice only where no chunk kernel exists (fp32 with
 *            K = 128); a chain's time grows with its length;
 *            4 = fused: one workgroup per (b, h, segment) in which four waves
 *            prepare chunk c + 1 (gate cumsum, in-chunk products, the
 *            triangular solve) while four waves carry the state through
 *            chunk c, the operands passed through LDS: the inputs are read
 *            once and nothing per chunk touches HBM.  bf16 with K = V = 128
 *            only, v_block 128 (0 or V); the library's choice for those
 *            sizes.
 *   n_seg:   number of sequence segments evaluated side by side on one card
 *            (1 = none; > 1 adds the segment summary and segment scan passes).
 *   v_block: value columns per workgroup of the state-carrying pass (64 or
 *            128; at most V, and with n_seg > 1 it must divide K).
 * Any field 0 means "let the library choose".  Any valid plan gives the same
 * result up to fp32/bf16 rounding.
 */
typedef struct kda_plan {
    int n_seg;
    int v_block;
    int split;
} kda_plan;

/* Sizes supported by the kernels: K, V in {64, 128}; bf16 or fp32 inputs
 * (fp32 with K = 128 runs the token-serial form, split 3).  T >= 0 is
 * arbitrary (the tail chunk is masked); B, H >= 0. */

/*
 * The plan kda_chunk_fwd uses for these sizes on the current device.
 * Fills *plan.  Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED or
 * KDA_ERR_HIP (device query failed).
 */
kda_status kda_chunk_fwd_plan(int B, int T, int H, int K, int V, kda_dtype dt,
                              kda_plan* plan);

/*
 * Bytes of device workspace kda_chunk_fwd needs for these sizes in the plan
 * the library picks on the current device (kda_chunk_fwd_plan).  0 when none
 * is needed; (size_t)-1 for invalid or unsupported arguments or a failed
 * device query.
 */
size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int K, int V, kda_dtype dt);

/*
 * Chunked prefill (the page's chunk-parallel form, section "Как
 * распараллелили последовательное обновление"), optionally resuming from an
 * initial state and returning the final state (the prefix-cache mechanism),
 * in the plan the library picks for the current device.
 *
 *   q, k, g : [B, T, H, K]  dtype dt   (g = log alpha before the clamp)
 *   v       : [B, T, H, V]  dtype dt
 *   beta    : [B, T, H]     dtype dt   (write strength; not clamped)
 *   initial_state : [B, H, K, V] fp32, or NULL for zeros
 *   o       : [B, T, H, V]  dtype dt   (written; may be NULL only if T == 0)
 *   final_state   : [B, H, K, V] fp32, or NULL (not written).  It may alias
 *                   initial_state exactly (in-place resume); a partial
 *                   overlap is KDA_ERR_INVALID_ARG.
 *   workspace / workspace_bytes : device scratch of at least
 *             kda_chunk_fwd_workspace_size(...) bytes (may be NULL when that
 *             size is 0); its contents on entry do not matter.
 * T == 0 writes final_state = initial_state (or zeros) and nothing else.
 */
kda_status kda_chunk_fwd(int B, int T, int H, int K, int V, kda_dtype dt,
                         const void* q, const void* k, const void* v,
                         const void* g,
                         const void* beta,
                         const float* initial_state,
                         void* o,
                         float* final_state,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * kda_chunk_fwd in a caller-chosen execution plan, and its workspace size.
 *   plan : NULL or a kda_plan; fields 0 are the library's choice.  A plan the
 *          kernels cannot run is KDA_ERR_INVALID_ARG (a field out of range) or
 *          KDA_ERR_UNSUPPORTED (a valid field these sizes have no kernel for).
 * The workspace size in a plan: with split = 2 one record per (b, h, chunk)
 * (for K = V = 128 bf16, 72.5 KiB; splits 1, 3 and 4 keep none); with
 * n_seg > 1 the segment transitions
 * and local states ((n_seg - 1) * B * H * K * (K + V) fp32) plus
 * B * H * K * V fp32 (a redirected final state).  Every other argument, and
 * the result up to fp32/bf16 rounding, as kda_chunk_fwd.
 */
size_t kda_chunk_fwd_planned_workspace_size(int B, int T, int H, int K, int V, kda_dtype dt,
                                            const kda_plan* plan);
kda_status kda_chunk_fwd_planned(int B, int T, int H, int K, int V, kda_dtype dt,
                                 const void* q, const void* k, const void* v,
                                 const void* g, const void* beta,
                                 const float* initial_state,
                                 void* o, float* final_state,
                                 const kda_plan* plan,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * kda_chunk_fwd_planned for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  No workspace argument: the workspace comes from a device array
 * of KDA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library defines and that
 * each GPU it runs on holds until the process ends; the call allocates
 * nothing.
 *   plan : NULL = the plan kda_chunk_fwd picks when its workspace
 *          (kda_chunk_fwd_planned_workspace_size) fits the array, else the
 *          single-pass plan (split 1) with as many of the library's segments
 *          as fit (one segment needs none, so every size runs); an explicit
 *          plan whose workspace exceeds the array is KDA_ERR_WORKSPACE.
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (from several streams or host threads) race and give wrong
 * results; calls ordered on one stream are safe (nothing in the array needs
 * to start at zero).  Every other argument, and the result, as
 * kda_chunk_fwd_planned in the same plan.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_chunk_fwd_noalloc(int B, int T, int H, int K, int V, kda_dtype dt,
                                 const void* q, const void* k, const void* v,
                                 const void* g, const void* beta,
                                 const float* initial_state,
                                 void* o, float* final_state,
                                 const kda_plan* plan,
                                 hipStream_t stream);

/*
 * kda_chunk_fwd_planned with the output gate of the KDA block fused into the
 * store of o (aiblin.ru page, section "KV‑кэш все‑таки не исчез полностью":
 * after the attention a gate decides what share of its result passes on into
 * the model's main stream, and the KDA blocks use the same gate; its form is
 * not given there, the plainest reading is taken):
 *
 *   o[b,t,h,:] = RNE_dt( RNE_dt(S_t^T q_t) * sigmoid(gate[b,t,h,:]) )
 *
 *   gate : [B, T, H, V] dtype dt, the gate pre-activation, 16-byte aligned;
 *          NULL is KDA_ERR_INVALID_ARG when there is work.
 * The same result as kda_chunk_fwd followed by an elementwise o * sigmoid(gate)
 * in fp32 rounded to dt, up to the 1-ulp exp2 and reciprocal of the sigmoid;
 * it saves that pass over o.  Every other argument as kda_chunk_fwd_planned
 * (workspace size: kda_chunk_fwd_planned_workspace_size).
 */
kda_status kda_chunk_fwd_gated(int B, int T, int H, int K, int V, kda_dtype dt,
                               const void* q, const void* k, const void* v,
                               const void* g, const void* beta, const void* gate,
                               const float* initial_state,
                               void* o, float* final_state,
                               const kda_plan* plan,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * Prefill of a packed batch of N variable-length sequences (the
 * prefix-caching and multi-token-verification use: every sequence resumes
 * from its own state and returns its own final state).  The habr.com
 * article on the Kimi K3 technical report notes that KDA needs its own
 * prefix-caching support in serving engines; this is that call.
 *
 *   cu_seqlens : DEVICE int32 [N + 1]: sequence i is tokens
 *                [cu_seqlens[i], cu_seqlens[i+1]) of the packed axis;
 *                cu_seqlens[0] = 0, non-decreasing, cu_seqlens[N] = T_total.
 *                Read on the device (nothing is synchronised).  Offsets
 *                outside that contract are clamped to [0, T_total] (results
 *                for such sequences are then unspecified, but every access
 *                stays inside the buffers).
 *   q, k, g    : [T_total, H, K] dtype dt;  v, o : [T_total, H, V];
 *   beta       : [T_total, H]
 *   initial_state : [N, H, K, V] fp32 or NULL (zeros)
 *   final_state   : [N, H, K, V] fp32 or NULL; may alias initial_state exactly
 *   workspace  : device scratch of at least
 *                kda_chunk_fwd_varlen_workspace_size(...) bytes
 * Runs the two-pass plan (intra-chunk pass over every chunk of every
 * sequence, then one state-carrying workgroup column block per (sequence,
 * head)); sequences of length 0 copy their state.  Same conventions, dtypes
 * and error codes as kda_chunk_fwd; sizes: K, V in {64, 128}, bf16 or fp32.
 * fp32 other than K = V = 64 runs the token-serial form per (sequence, head)
 * and needs no workspace (the size function returns 0).
 */
size_t kda_chunk_fwd_varlen_workspace_size(int N, int T_total, int H, int K, int V, kda_dtype dt);
kda_status kda_chunk_fwd_varlen(int N, const int* cu_seqlens, int T_total, int H, int K, int V, kda_dtype dt,
                                const void* q, const void* k, const void* v,
                                const void* g, const void* beta,
                                const float* initial_state,
                                void* o, float* final_state,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * kda_chunk_fwd_varlen with the output gate fused as in kda_chunk_fwd_gated;
 * gate : [T_total, H, V] dtype dt.
 */
kda_status kda_chunk_fwd_varlen_gated(int N, const int* cu_seqlens, int T_total, int H, int K, int V,
                                      kda_dtype dt, const void* q, const void* k, const void* v,
                                      const void* g, const void* beta, const void* gate,
                                      const float* initial_state, void* o, float* final_state,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd_varlen that also returns state snapshots at fixed block
 * boundaries (prefix caching: a later request sharing the first m tokens of
 * a sequence resumes from the snapshot at the largest boundary <= m).
 *
 *   snapshot_interval : tokens between snapshots; a positive multiple of 64
 *                       (the chunk length), else KDA_ERR_INVALID_ARG.
 *   snapshots         : DEVICE fp32 [max_snapshots, H, K, V], 16-byte aligned
 *                       (may be NULL when max_snapshots == 0).
 *   max_snapshots     : capacity in snapshots (>= 0); slots past it are not
 *                       written.  With valid cu_seqlens the count needed is
 *                       sum_i floor(len_i / snapshot_interval) <=
 *                       floor(T_total / snapshot_interval).
 * Snapshot m (m = 0, 1, ...) of sequence i, the state after its first
 * (m + 1) * snapshot_interval tokens, is written to slot snap_off_i + m with
 * snap_off_i = sum_{j < i} floor(len_j / snapshot_interval); nothing else in
 * `snapshots` is touched.  o and final_state are exactly those of
 * kda_chunk_fwd_varlen with the same arguments; the workspace is the same.
 * Snapshots come from the chunk state pass: sizes that run the token-serial
 * form (fp32 other than K = V = 64) return KDA_ERR_UNSUPPORTED.
 */
kda_status kda_chunk_fwd_varlen_snapshots(int N, const int* cu_seqlens, int T_total, int H, int K, int V,
                                          kda_dtype dt, const void* q, const void* k, const void* v,
                                          const void* g, const void* beta, const float* initial_state,
                                          void* o, float* final_state, int snapshot_interval,
                                          float* snapshots, int max_snapshots,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step for N independent sequences (page section "Как хранить
 * миллион токенов в памяти": the fixed-size state replaces the KV cache).
 * Reads and writes the state once.
 *
 *   q, k, g : [N, H, K] dtype dt;  v : [N, H, V] dtype dt;  beta : [N, H] dtype dt
 *   state   : [N, H, K, V] fp32, updated IN PLACE to S_t
 *   o       : [N, H, V] dtype dt (written), o = S_t^T q
 */
kda_status kda_recurrent_step(int N, int H, int K, int V, kda_dtype dt,
                              const void* q, const void* k, const void* v,
                              const void* g, const void* beta,
                              float* state, void* o, hipStream_t stream);

/*
 * T consecutive tokens of each of N sequences in one call (multi-token
 * verification of a draft, as in speculative decoding): the same update as T
 * calls of kda_recurrent_step, with the state read once and written once.
 *
 *   q, k, g : [N, T, H, K] dtype dt;  v : [N, T, H, V];  beta : [N, T, H]
 *   state   : [N, H, K, V] fp32, updated IN PLACE to the state after token T
 *   o       : [N, T, H, V] dtype dt (written), o_t = S_t^T q_t
 *   step_states : [N, T, H, K, V] fp32, the state after each token (so that a
 *                 caller can resume after any accepted prefix), or NULL.  It
 *                 must not overlap state.
 * T == 0 or N * H == 0 does nothing.  Sizes and dtypes as kda_recurrent_step.
 */
kda_status kda_recurrent_steps(int N, int T, int H, int K, int V, kda_dtype dt,
                               const void* q, const void* k, const void* v,
                               const void* g, const void* beta,
                               float* state, void* o, float* step_states, hipStream_t stream);

/*
 * Backward of kda_chunk_fwd: the gradients of a loss L with respect to q, k,
 * v, g (log alpha before the clamp), beta and the initial state, given dL/do
 * and dL/dS_T.  The pages give no backward; this is the chain rule applied
 * to the recurrence (section "Как хранить миллион токенов в памяти") in its
 * chunk form (section "Как распараллелили последовательное обновление"): the
 * forward's state after every chunk, a reverse state pass for dL/dS at every
 * chunk boundary, then every chunk's gradients at once.  fp32 with K or V =
 * 128 (no two-pass forward) runs a token-level form instead.  The clamp
 * passes the gradient inside its closed range [-5, 0] and blocks it outside.
 *
 *   q, k, g, v, beta, initial_state : the forward's inputs (same layouts)
 *   d_o           : [B, T, H, V] dtype dt, dL/do, or NULL (zeros)
 *   d_final_state : [B, H, K, V] fp32, dL/dS_T, or NULL (zeros)
 *   dq, dk, dg    : [B, T, H, K] dtype dt (written)
 *   dv            : [B, T, H, V] dtype dt (written)
 *   dbeta         : [B, T, H] dtype dt (written)
 *   d_initial_state : [B, H, K, V] fp32 (written) or NULL.  It must not
 *                     overlap d_final_state (not even exactly: the reverse
 *                     pass reads dL/dS_T while it writes dL/dS_0), else
 *                     KDA_ERR_INVALID_ARG.
 *   workspace     : at least kda_chunk_bwd_workspace_size(...) bytes (the
 *                   size does not depend on the device).  Chunk form: the
 *                   forward plan's segment arrays (with n_seg > 1, the
 *                   transitions of all n_seg segments: one K x K fp32 slot
 *                   per (b, h) more than the forward's), its chunk records, the
 *                   state and dL/dS after every chunk (2 B*H*ceil(T/64)*K*V
 *                   values) and per-chunk fp32 intermediates.  bf16 at
 *                   K = V = 128: one workgroup computes every gradient of a
 *                   chunk from bf16 states and adjoints, and the workspace
 *                   holds those bf16, dL/dU (fp32, 64 x V per chunk) and bf16
 *                   copies of S0 and dL/dS_T.  Otherwise the states and
 *                   adjoints are fp32 and the products the three chunk stages
 *                   hand on are kept too.
 *                   Token-level
 *                   form: the state every 8 tokens (B*H*ceil(T/8)*K*V fp32)
 *                   and the per-16-column partial sums
 *                   (V/16 * B*T*H*(3K+1) fp32).
 * Sizes: K, V in {64, 128}; bf16 or fp32.  The forward states are recomputed
 * (no saved activations are needed).  Results are deterministic.
 */
size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int K, int V, kda_dtype dt);
kda_status kda_chunk_bwd(int B, int T, int H, int K, int V, kda_dtype dt,
                         const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* initial_state, const void* d_o, const float* d_final_state,
                         void* dq, void* dk, void* dv, void* dg, void* dbeta, float* d_initial_state,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Optional per-launch timing, for benchmarks and tracing.  After
 * kda_profile_start(max_launches), each kernel launched by the library
 * (up to max_launches of them) is bracketed by two HIP
 * events recorded on its own stream; launches beyond that are not timed.
 * kda_profile_stop waits for the recorded events, writes up to `cap` launch
 * names (static strings: "intra_chunk", "state_output", "state_summary",
 * "chunk_output", "chunk_summary", "segment_scan", "copy_state",
 * "varlen_prep", "decode_step", "decode_steps", "backward"; the chunk-form
 * backward's "bwd_intra_chunk", "bwd_state_summary", "bwd_segment_scan",
 * "bwd_states", "bwd_reverse_summary", "bwd_reverse_scan", "bwd_state_reverse",
 * "bwd_value_side", "bwd_solve", "bwd_gated") and durations in milliseconds, releases the
 * events, and returns the number of timed launches (-1: profiling was not
 * started or a HIP event query failed).  The record is process-wide (the one
 * piece of state the library keeps, opt-in): launches from several threads
 * while it is on are each recorded whole (a mutex guards it), in the order
 * they took their slots.  Profiling is off unless started.
 * kda_profile_start returns KDA_ERR_INVALID_ARG for max_launches outside
 * [1, 2^20] and KDA_ERR_HIP if an event cannot be created.
 */
kda_status kda_profile_start(int max_launches);
int kda_profile_stop(const char** names, float* ms, int cap);

/* Static description of a status code. */
const char* kda_status_string(kda_status s);

/* Library version string. */
const char* kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
