/*
 * kda.h -- C ABI of the MI355X (gfx950) chunked KDA forward library.
 *
 * The operation is the chunked forward of Kimi Delta Attention, the gated
 * delta rule of the page "feat(kda): integrate KDA attention with tokamax
 * backend and CP support" (Implementation Details, "Delta Rule
 * formulation"): per batch row b and head h, token by token,
 *     S <- diag(exp(g_t)) S                      (decay on the key axis)
 *     S <- S + beta_t k_t (v_t - k_t^T S)^T      (delta-rule write)
 *     o_t = scale * q_t^T S                      (read-out after the write)
 * evaluated in 64-token chunks.  The argument list mirrors the chunk_kda
 * entry point of that page's Public API section (q, k, v, g, beta, scale,
 * initial_state, output_final_state, chunk_size, use_qk_l2norm_in_kernel,
 * safe_gate, lower_bound, segment_ids, N_max).
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer, contiguous, 16-byte aligned.
 *    The caller owns all memory; the library allocates nothing and keeps no
 *    state between calls (the optional launch observer aside).
 *  - Layouts are batch-first: q, k, g [B,T,H,K]; v and o [B,T,H,V];
 *    beta [B,T,H]; segment_ids [B,T] int32; states fp32 [B,H,K,V], or
 *    [B,N_max,H,K,V] when segment_ids are given (one state per segment, in
 *    order of appearance within the row).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *    the default stream).  KDA_OK means the arguments were valid and the
 *    kernels were enqueued.  No exception crosses the ABI.
 *  - On any other status nothing was enqueued and kda_last_error() returns a
 *    message for the calling thread.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1,   /* a value or combination the method rejects */
  KDA_ERR_NOT_IMPLEMENTED = 2,    /* a valid request this library does not cover */
  KDA_ERR_WORKSPACE_TOO_SMALL = 3,
  KDA_ERR_HIP = 4                 /* a HIP runtime call failed */
} kda_status_t;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;

/* Flags reported by kda_chunk_fwd_flags(). */
#define KDA_FLAG_SEGMENT_OVERFLOW 0x1u  /* a row held more than max_segments segments */
#define KDA_FLAG_FUSED_TIMEOUT 0x2u     /* a bounded wait of the fused forward ran out (not
                                           expected: it only waits for records a running
                                           workgroup is producing); the outputs of that call
                                           are undefined */
#define KDA_FLAG_GATE_POSITIVE 0x4u     /* some g > 0 reached a forward that takes g as the log
                                           decay (g <= 0 is a precondition, page "feat(kda):
                                           integrate KDA attention with tokamax backend and CP
                                           support", Implementation Details: g is a log decay).
                                           Checked only by the debug build of the library,
                                           libkda_debug.so (KDA_DEBUG_CHECKS), whose results are
                                           otherwise those of libkda.so; the release build never
                                           sets it. */

typedef struct {
  int64_t B, T, H;        /* >= 0 each; a zero size makes the call a no-op */
  int64_t K, V;           /* key / value head dims: 64 or 128 each (else NOT_IMPLEMENTED) */
  kda_dtype_t dtype;      /* element type of q, k, v, g, beta */
  kda_dtype_t o_dtype;    /* element type of o (states are always fp32) */
  float scale;            /* read-out scale; NaN selects 1/sqrt(K); must be finite otherwise */
  int32_t chunk_size;     /* must be 64 (else NOT_IMPLEMENTED) */
  int32_t use_qk_l2norm;  /* 0/1: divide q, k by sqrt(sum x^2 + 1e-6) inside the kernel */
  int32_t safe_gate;      /* 0/1: caller promises lower_bound <= g <= 0 everywhere */
  float lower_bound;      /* with safe_gate: must lie in [-5, 0) (else INVALID_ARGUMENT);
                             ignored without safe_gate */
  int32_t max_segments;   /* N_max: upper bound on segments per row; required >= 1 when
                             segment_ids are given (else INVALID_ARGUMENT), ignored otherwise */
} kda_fwd_desc_t;

/*
 * Bytes of device workspace kda_chunk_fwd needs for `desc` and for whether
 * segment_ids will be passed: has_segment_ids must be non-zero exactly when
 * the forward call will get a non-NULL segment_ids (the segment and chunk
 * tables are only laid out then).  The size depends on nothing else (sizes,
 * dtype, max_segments).  Returns INVALID_ARGUMENT / NOT_IMPLEMENTED for
 * descriptors kda_chunk_fwd would reject (with has_segment_ids non-zero,
 * max_segments < 1 is INVALID_ARGUMENT).
 */
kda_status_t kda_chunk_fwd_workspace_size(const kda_fwd_desc_t* desc, int has_segment_ids,
                                          size_t* bytes);

/*
 * Chunked KDA forward.
 *   q, k, g       [B,T,H,K] of desc->dtype.  g is the per-key-channel log decay,
 *                 required to satisfy g <= 0 (and g >= lower_bound under
 *                 safe_gate); results for g > 0 are unspecified.
 *   v             [B,T,H,V] of desc->dtype.
 *   beta          [B,T,H] of desc->dtype.
 *   initial_state NULL (zero state) or fp32 [B,H,K,V] / [B,N_max,H,K,V].
 *   segment_ids   NULL (each row is one sequence) or int32 [B,T]: 1-based ids,
 *                 0 = padding.  A new segment starts at every token whose id
 *                 is non-zero and differs from the previous token's id.
 *                 Padding tokens get o = 0 and do not touch any state.
 *   o             [B,T,H,V] of desc->o_dtype; every element is written.
 *   final_state   NULL (not requested) or fp32, same shape as initial_state;
 *                 slots of segments that do not occur are set to zero.
 *   workspace     device scratch of at least kda_chunk_fwd_workspace_size()
 *                 bytes; its contents on entry do not matter.
 * If a row holds more than max_segments segments, the excess segments get
 * o = 0, their states are not read or written, and KDA_FLAG_SEGMENT_OVERFLOW
 * is raised in the workspace (read it with kda_chunk_fwd_flags).
 */
kda_status_t kda_chunk_fwd(const kda_fwd_desc_t* desc,
                           const void* q, const void* k, const void* v,
                           const void* g, const void* beta,
                           const float* initial_state, const int32_t* segment_ids,
                           void* o, float* final_state,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same forward, with its workspace taken from a fixed region of device
 * memory inside the library instead of a caller's buffer.  The region holds
 * KDA_STATIC_WORKSPACE_BYTES; each GPU the library runs on keeps its own copy
 * from the library's load until the process ends.  A request whose
 * kda_chunk_fwd_workspace_size exceeds it returns KDA_ERR_WORKSPACE_TOO_SMALL
 * and enqueues nothing.  The call itself allocates nothing.  The region of
 * the current device is used (the stream must belong to it); every call on
 * one GPU shares it, so calls that overlap in time on one GPU (other streams,
 * other threads) race and their results are undefined.  The segment-overflow
 * flag of such a call cannot be read back.  All other arguments, the results
 * and the errors are those of kda_chunk_fwd.
 */
#define KDA_STATIC_WORKSPACE_BYTES (64u << 20)
kda_status_t kda_chunk_fwd_noalloc(const kda_fwd_desc_t* desc,
                                   const void* q, const void* k, const void* v,
                                   const void* g, const void* beta,
                                   const float* initial_state, const int32_t* segment_ids,
                                   void* o, float* final_state, void* stream);

/*
 * The forward with the gate activated inside the kernel (chunk_kda options
 * use_gate_in_kernel, A_log and dt_bias of the page "feat(kda): integrate KDA
 * attention with tokamax backend and CP support", Public API; the layer's
 * "Gate generation" step there activates the gate with a sigmoid from A_log
 * and dt_bias; the safe gate has sigmoid lower-bound semantics).  g holds
 * raw gate values; for head h and key channel c the kernel uses
 *     z = exp(A_log[h]) * (g + dt_bias[h*K + c])
 *     safe_gate:  log decay = lower_bound * sigmoid(z)   (in (lower_bound, 0))
 *     otherwise:  log decay = log(sigmoid(z))            (decay = sigmoid(z))
 * evaluated in fp32.
 *   A_log    NULL (exp(A_log) = 1) or fp32 [H], device memory.
 *   dt_bias  NULL (zero) or fp32 [H,K], device memory.
 * Every other argument, the workspace size and the errors are those of
 * kda_chunk_fwd.  A_log and dt_bias need no alignment beyond that of float.
 */
kda_status_t kda_chunk_fwd_gated(const kda_fwd_desc_t* desc,
                                 const void* q, const void* k, const void* v,
                                 const void* g, const void* beta,
                                 const float* A_log, const float* dt_bias,
                                 const float* initial_state, const int32_t* segment_ids,
                                 void* o, float* final_state,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of kda_chunk_fwd (g taken as the log decay): the gradients of
 *     L = sum(o * d_o) + sum(final_state * d_final_state)
 * with respect to q, k, v, g, beta and initial_state, for the forward that
 * desc, q, k, v, g, beta, initial_state and segment_ids describe (page
 * "feat(kda): integrate KDA attention with tokamax backend and CP support":
 * the Delta Rule formulation is the function differentiated; its CP
 * gradient-equivalence test checks the backward against the unsplit one).
 * Evaluated in fp32 in 16-token chunks (recomputing the forward's chunk
 * quantities and states; nothing is kept from a forward call).
 *   d_o            [B,T,H,V] of desc->o_dtype; rows of padding tokens are ignored.
 *   d_final_state  NULL (zero) or fp32 in the initial state's shape.
 *   dq, dk, dg     fp32 [B,T,H,K];  dv fp32 [B,T,H,V];  dbeta fp32 [B,T,H];
 *                  every element is written (zero for padding tokens and for
 *                  segments past max_segments).
 *   d_initial_state NULL (not wanted) or fp32 in the initial state's shape
 *                  (written also when initial_state is NULL: the gradient
 *                  with respect to a zero start state); slots of absent
 *                  segments get zero.
 *   workspace      at least kda_chunk_bwd_workspace_size() bytes (about
 *                  (5 K V / 64 + 4 K + 3 V) * 4 bytes per token and head: the
 *                  state entering every 64-token chunk, its gradient at every
 *                  16-token chunk, and the chunk quantities).
 * desc->use_qk_l2norm differentiates through the in-kernel L2 norm;
 * safe_gate and lower_bound play no part.  Errors as for kda_chunk_fwd.
 */
kda_status_t kda_chunk_bwd_workspace_size(const kda_fwd_desc_t* desc, int has_segment_ids, size_t* bytes);
kda_status_t kda_chunk_bwd(const kda_fwd_desc_t* desc,
                           const void* q, const void* k, const void* v,
                           const void* g, const void* beta,
                           const float* initial_state, const int32_t* segment_ids,
                           const void* d_o, const float* d_final_state,
                           float* dq, float* dk, float* dv, float* dg, float* dbeta,
                           float* d_initial_state,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_bwd again on a workspace that a kda_chunk_bwd call with the same
 * desc, inputs and gradient buffers filled: the chunk quantities and the
 * forward states do not depend on the cotangents, so only the reverse state
 * recurrence and the per-chunk gradients run, for new d_o / d_final_state.
 * Positions the first call zeroed (padding tokens, absent slots) are not
 * written again.  The second backward pass of a context-parallel rank.
 */
kda_status_t kda_chunk_bwd_rerun(const kda_fwd_desc_t* desc,
                                 const void* q, const void* k, const void* v,
                                 const void* g, const void* beta,
                                 const float* initial_state, const int32_t* segment_ids,
                                 const void* d_o, const float* d_final_state,
                                 float* dq, float* dk, float* dv, float* dg, float* dbeta,
                                 float* d_initial_state,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward, plus each row's transition: the recurrence is affine in the
 * state the row's first segment starts from, so the state after the row's
 * last token is  M * S_start + (that state for S_start = 0),  with M the
 * K x K matrix this call writes (the product over the tokens t of the
 * segment, last on the left, of (I - beta_t k_t k_t^T) diag(exp(g_t))).
 * This is what a context-parallel rank hands on with its end state (page
 * "feat(kda): integrate KDA attention with tokamax backend and CP support",
 * Context Parallelism Support: the recurrent state is coordinated across
 * ranks).
 *   transition  fp32 [B,H,K,K], row-major (row = key channel of the end
 *               state, column = key channel of S_start), device memory,
 *               non-NULL.  M is zero for a row whose first and last tokens
 *               are not in one segment (a segment boundary or padding in
 *               between, or padding at either end) and for T = 0.
 * Every other argument, the workspace size and the errors are those of
 * kda_chunk_fwd.  The workspace keeps the chunk records for
 * kda_chunk_fwd_rerun.
 */
kda_status_t kda_chunk_fwd_transition(const kda_fwd_desc_t* desc,
                                      const void* q, const void* k, const void* v,
                                      const void* g, const void* beta,
                                      const float* initial_state, const int32_t* segment_ids,
                                      void* o, float* final_state, float* transition,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Runs again only the inter-chunk recurrence of the last forward call
 * (kda_chunk_fwd, kda_chunk_fwd_gated or kda_chunk_fwd_transition) made on
 * `workspace`, with new start states: the chunk-local work does not depend
 * on the state, and the workspace still holds its results.  desc and
 * segment_ids (only whether it is NULL matters) must be those of that call,
 * and the workspace must be untouched since.  Writes o for every token of a
 * segment and final_state for every segment that occurs; positions the
 * earlier call zeroed (padding tokens, slots of absent segments) are not
 * written again, so pass the same o and final_state buffers to keep them.
 * This is the second pass of a context-parallel rank, once the state its
 * slice continues from is known.
 */
kda_status_t kda_chunk_fwd_rerun(const kda_fwd_desc_t* desc, const float* initial_state,
                                 const int32_t* segment_ids, void* o, float* final_state,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Context-parallel state chaining (page "feat(kda): integrate KDA attention
 * with tokamax backend and CP support", Context Parallelism Support: the
 * kernel derives per-rank sequence metadata from segment_ids and carries the
 * recurrent state across ranks; its tests split T over 2 or 4 ranks,
 * including packed segments that cross a split or begin exactly at one).
 * Each of B rows of T tokens is cut into P slices of T/P tokens, slice r
 * being rank r's share; one call handles all B*P slices, which are the rows
 * of the per-slice forward calls ([B*P, T/P, ...] views of the inputs).
 *   1. kda_cp_plan                per slice: continues the previous slice's
 *                                 segment?, global index of its first local
 *                                 segment, local segment count.
 *   2. kda_cp_gather_states       per-slice start states, carry = NULL (the
 *                                 continued segment starts from zero).
 *   3. kda_chunk_fwd_transition   on the slices: end states and transitions.
 *   4. kda_cp_chain               C_{r+1} = E_r + [slice r continues] M_r C_r,
 *                                 the state each continuing slice starts from.
 *   5. kda_cp_gather_states       with carry = C.
 *   6. kda_chunk_fwd_rerun        on the same workspace: exact o and states.
 *   7. kda_cp_scatter_states      per-segment final states, global layout.
 * Across GPUs step 4 is P-1 point-to-point hops of one state per (row,
 * head); this library runs all hops on one GPU.
 *
 * n_states is the number of state slots per row: max_segments with segment
 * ids (states [B,n_states,H,K,V] globally, [B*P,n_states,H,K,V] per slice),
 * 1 without (the [B,H,K,V] / [B*P,H,K,V] layouts).  A row with more than
 * n_states segments sets the overflow field of the plan; results for such
 * rows are unspecified.  All pointers are device pointers, 16-byte aligned;
 * calls are asynchronous on `stream` and allocate nothing.
 */
typedef struct {
  int64_t B, T, H;   /* rows, tokens per row (a multiple of P), heads */
  int64_t K, V;      /* 64 or 128 each */
  int32_t P;         /* slices per row (ranks), >= 1 */
  int32_t n_states;  /* state slots per row, >= 1 */
} kda_cp_desc_t;

/*
 * plan: int32 [B,P,4] written per slice (b, r): {continues (0/1), global
 * index of the first local segment, local segments, overflow (0/1)}.
 * segment_ids: NULL (each row one sequence) or int32 [B,T] as for
 * kda_chunk_fwd.  T must be >= 1.
 */
kda_status_t kda_cp_plan(const kda_cp_desc_t* desc, const int32_t* segment_ids, int32_t* plan, void* stream);

/*
 * local_states [B*P,n_states,H,K,V]: slot l of slice (b, r) gets the start
 * state of its local segment l: carry[b*P + r] (zero if carry is NULL) for a
 * continued segment, else initial_state of its global segment (zero if
 * initial_state is NULL); unused slots get zero.
 * initial_state: NULL or [B,n_states,H,K,V];  carry: NULL or [B*P,H,K,V].
 */
kda_status_t kda_cp_gather_states(const kda_cp_desc_t* desc, const int32_t* plan, const float* initial_state,
                                  const float* carry, float* local_states, void* stream);

/*
 * carry [B*P,H,K,V]: the state slice (b, r) continues from (C_r above; zero
 * for r = 0 and for slices that start a new segment or padding).
 * local_final [B*P,n_states,H,K,V] and transition [B*P,H,K,K] are the outputs
 * of step 3.  Accumulates in fp32.
 */
kda_status_t kda_cp_chain(const kda_cp_desc_t* desc, const int32_t* plan, const float* local_final,
                          const float* transition, float* carry, void* stream);

/*
 * final_state [B,n_states,H,K,V]: each segment's state after its last token,
 * taken from the last slice that holds it; slots of segments that do not
 * occur get zero.  local_final is the final_state of step 6.
 */
kda_status_t kda_cp_scatter_states(const kda_cp_desc_t* desc, const int32_t* plan, const float* local_final,
                                   float* final_state, void* stream);

/*
 * The backward under the same slicing (the pages' CP gradient equivalence):
 * each slice's backward (kda_chunk_bwd on the slice rows, with the start
 * states of the forward's step 5) needs the gradient of the state it hands
 * on, which the next slice's backward produces.  In order:
 *   1. kda_cp_gather_final_grads   per-slice final-state gradients, carry_grad
 *                                  = NULL (a handed-on state gets zero).
 *   2. kda_chunk_bwd               on the slices: local initial-state gradients.
 *   3. kda_cp_chain_bwd            X_r = [slice r+1 continues]
 *                                  (dInit_{r+1} + M_{r+1}^T X_{r+1}), X_{P-1} = 0.
 *   4. kda_cp_gather_final_grads   with carry_grad = X.
 *   5. kda_chunk_bwd_rerun         on the same workspace: exact gradients.
 *   6. kda_cp_scatter_initial_grads  per-segment initial-state gradients,
 *                                  global layout (from the slice where each
 *                                  segment starts).
 * Across GPUs step 3 is P-1 point-to-point hops of one state gradient, from
 * the last rank back.
 *
 * local_d_final [B*P,n_states,H,K,V]: slot l of slice (b, r) gets, for the
 * slice's last local segment when slice r+1 continues it, carry_grad[b*P + r]
 * (zero if carry_grad is NULL), else d_final_state of its global segment
 * (zero if d_final_state is NULL); unused slots get zero.
 */
kda_status_t kda_cp_gather_final_grads(const kda_cp_desc_t* desc, const int32_t* plan, const float* d_final_state,
                                       const float* carry_grad, float* local_d_final, void* stream);
/*
 * carry_grad [B*P,H,K,V]: X_r above (zero for the last slice and for slices
 * whose last token does not continue into the next).  local_d_initial
 * [B*P,n_states,H,K,V] is the d_initial_state of step 2 and transition
 * [B*P,H,K,K] the forward's.  Accumulates in fp32.
 */
kda_status_t kda_cp_chain_bwd(const kda_cp_desc_t* desc, const int32_t* plan, const float* local_d_initial,
                              const float* transition, float* carry_grad, void* stream);
/*
 * d_initial_state [B,n_states,H,K,V]: each segment's initial-state gradient,
 * taken from the first slice that holds it; slots of segments that do not
 * occur get zero.  local_d_initial is the d_initial_state of step 5.
 */
kda_status_t kda_cp_scatter_initial_grads(const kda_cp_desc_t* desc, const int32_t* plan,
                                          const float* local_d_initial, float* d_initial_state, void* stream);

/*
 * Short convolution, the layer step that q, k and v each pass through before
 * the kernel (page "feat(kda): integrate KDA attention with tokamax backend
 * and CP support", Implementation Details, Layer architecture, step 1: a
 * causal depthwise 1D convolution with SiLU; kernel size
 * linear_conv_kernel_dim of its configuration table; its review notes make
 * the convolution segment-aware):
 *     y[b,t,d] = SiLU( sum_{j<W} weight[d*W + j] * x[b, t-(W-1)+j, d] )
 * where a tap before the start of t's segment (or before t = 0) reads zero and
 * padding tokens (segment id 0) get y = 0.  No bias.
 *   x, y         [B,T,D] of `dtype` (fp32 or bf16), device memory, 16-byte
 *                aligned; y may not overlap x.
 *   weight       fp32 [D,W] (PyTorch's depthwise Conv1d weight [D,1,W]),
 *                device memory; tap W-1 multiplies the current token.
 *   segment_ids  NULL (one segment per row) or int32 [B,T] as for
 *                kda_chunk_fwd.
 * W must be 1..8 and D a multiple of 8 (else NOT_IMPLEMENTED; W = 0, which
 * the configuration uses to disable the convolution, is INVALID_ARGUMENT:
 * the caller skips the call).  Asynchronous on `stream`; allocates nothing.
 */
kda_status_t kda_short_conv_fwd(int64_t B, int64_t T, int64_t D, int32_t W, kda_dtype_t dtype,
                                const void* x, const float* weight, const int32_t* segment_ids,
                                void* y, void* stream);

/*
 * Output stage after the kernel (same page, Layer architecture: a per-head
 * RMSNorm and a sigmoid output gate), over rows of V values (one row per
 * token and head):
 *     y = weight * o / sqrt(mean(o^2) + eps) * sigmoid(gate)
 *   o       [rows, V] of o_dtype; gate [rows, V] of gate_dtype; y [rows, V]
 *           of y_dtype (each fp32 or bf16), device memory, 4-byte aligned.
 *   weight  fp32 [V], shared by the heads.   eps >= 0, finite.
 * V must be 64, 128 or 256 (else NOT_IMPLEMENTED).  Asynchronous on
 * `stream`; allocates nothing.
 */
kda_status_t kda_gated_rmsnorm_fwd(int64_t rows, int64_t V, kda_dtype_t o_dtype, kda_dtype_t gate_dtype,
                                   kda_dtype_t y_dtype, const void* o, const void* gate,
                                   const float* weight, float eps, void* y, void* stream);

/*
 * Waits for `stream`, then reads the KDA_FLAG_* word the last kda_chunk_fwd
 * call on this workspace left behind (0 when nothing was flagged).
 */
kda_status_t kda_chunk_fwd_flags(const void* workspace, size_t workspace_bytes, void* stream,
                                 uint32_t* flags);

/*
 * Launch observer, for measurement tools: when set, kda_chunk_fwd calls
 * fn(kernel_name, stream, phase, user) on the calling thread right before
 * (phase 0) and right after (phase 1) it enqueues each kernel, so a caller
 * can record timing events on `stream` around every kernel.  NULL removes
 * it.  Process-wide; set it while no other thread is inside kda_chunk_fwd.
 */
typedef void (*kda_launch_observer_t)(const char* kernel_name, void* stream, int phase, void* user);
void kda_set_launch_observer(kda_launch_observer_t fn, void* user);

/*
 * Forward schedule.  By default the forward runs the intra-chunk step and
 * the recurrence as two kernels ("kda_intra", then "kda_recur") with the
 * per-chunk records in HBM.  After kda_set_fused_forward(1), calls with
 * bf16 inputs, no segment_ids, no transition output and K = V = 128 on a
 * gfx950 device of 8 XCDs run both as one persistent kernel ("kda_fused",
 * the fused forward of the page "Add packed KDA forward megakernel",
 * Summary), which hands each record from the workgroup that produces it to
 * the recurrence workgroups of the same XCD (the records still go through
 * HBM when producers run far ahead of the recurrence, as they do); other
 * calls keep the two kernels.  Both compute the same function of the inputs
 * (up to fp32 rounding: the kernels are compiled apart); the setting only
 * selects the schedule.  Default 0: on MI355X the two kernels are the faster
 * schedule at the sizes measured so far.  Process-wide; set it while no
 * other thread is inside a forward call.
 */
void kda_set_fused_forward(int enable);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* kda_last_error(void);

/* Library version string. */
const char* kda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
