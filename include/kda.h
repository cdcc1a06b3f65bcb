/*
 * kda.h -- C ABI of the KDA (Kimi Delta Attention) forward recurrence on
 * AMD MI355X (gfx950). Link with libkda.so.
 *
 * The operation. For every sequence, head and token t, with the head's state
 * S (d_k x d_v, one row per key channel, float32):
 *
 *   S~  = Diag(exp(g_t)) S          decay each key channel
 *   v^  = S~^T k_t                  predict the value stored at k_t
 *   e   = beta_t (v_t - v^)         beta-scaled error
 *   S   = S~ + k_t e^T              rank-one write
 *   o_t = S^T (scale * q_t)         read of the updated state
 *
 * These are the five steps of "Module 03 - KDA I: The Delta-Rule Recurrence"
 * (jared-hpc.com), section 2, with beta folded into the error as on "Kimi
 * Delta Attention (KDA)" (brain.bigb.es), where the log-decay g = log(alpha)
 * and the [.., d_k, d_v] state layout are also given (section "KDA: one gate
 * per key channel"). kda_fwd_chunked evaluates whole sequences with the
 * chunkwise schedule of that page's section "Two schedules for the same
 * recurrence" (chunks of 64 tokens); kda_decode_step applies one step.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous, owned
 *    by the caller. The library allocates no memory; its only global state is
 *    a per-device cache of the compute-unit count (filled on first use,
 *    thread-safe) and a per-device parity of decode calls, which makes
 *    successive decode steps visit the states in alternating order (each
 *    state is updated on its own, so results never depend on it). Calls on
 *    different streams are independent.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream). Arguments are validated on the host before anything is
 *    enqueued: on any error nothing runs and no output is touched. Faults that
 *    happen while kernels execute surface at the caller's next
 *    synchronisation, not in the returned status.
 *  - Supported head sizes: Dk, Dv in {16, 32, 64, 128}.
 *  - dtype selects the element type of q, k, v and beta, o_dtype that of o:
 *    KDA_DTYPE_F32 (float) or KDA_DTYPE_BF16 (bfloat16). g and all states are
 *    always float32. Pointers must be 16-byte aligned.
 *  - Precision. With float32 inputs every product runs on fp32 MFMA. With
 *    bfloat16 inputs every operand is carried as a pair of bfloat16 values
 *    (high part and rounding residue, about 16 significant bits) and each
 *    product takes three bf16 MFMAs with fp32 accumulation; states and
 *    accumulators are float32 throughout. A float32 o keeps the full result;
 *    a bfloat16 o is the float32 result rounded to nearest even.
 *  - Preconditions that are documented, not checked: g is finite; states and
 *    inputs are finite; o does not overlap any input; cu_seqlens is
 *    non-decreasing with cu[0] = 0 and cu[num_seqs] = T.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_SUCCESS = 0,
    KDA_ERROR_INVALID_VALUE = 1,  /* bad pointer, size, alignment or combination */
    KDA_ERROR_NOT_SUPPORTED = 2,  /* valid request the library does not implement */
    KDA_ERROR_WORKSPACE = 3,      /* workspace missing or smaller than required */
    KDA_ERROR_LAUNCH = 4,         /* the HIP runtime refused a kernel launch */
    KDA_STATUS_FORCE_INT32 = 0x7fffffff   /* not a status: gives the type the range of int32 */
} kda_status;

/* KDA_DTYPE_FORCE_INT32 is not a type: it makes every int32 value a valid kda_dtype, so
 * that an unknown value passed from C is rejected (KDA_ERROR_INVALID_VALUE) rather than
 * being undefined behaviour in the C++ implementation. */
typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1, KDA_DTYPE_FORCE_INT32 = 0x7fffffff } kda_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_status_string(kda_status s);

/* Bytes of device workspace kda_fwd_chunked needs for these sizes.
 * Host only: touches no device memory. cu_seqlens_given says whether the
 * call will pass cu_seqlens (then B must be 1 and num_seqs is the number of
 * packed sequences); the bound used is floor(T/64) + num_seqs chunks per head
 * for packed input and B * ceil(T/64) otherwise, so cu_seqlens is never read
 * on the host. The size depends on dtype: for bf16 input the per-chunk
 * operands take 2.5 bytes per element (W, Qd, Kd^T: 12 significant bits) or 3
 * (A_qk, U: 16 significant bits); for fp32 input every operand takes 4 bytes.
 * Errors: KDA_ERROR_INVALID_VALUE for a NULL `bytes`, a non-positive size,
 * or an unsupported head size. */
kda_status kda_fwd_chunked_workspace_size(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                          int cu_seqlens_given, kda_dtype dtype, size_t* bytes);

/* Chunked prefill over B x T tokens (or num_seqs packed sequences).
 *
 *  q, k   [B, T, H, Dk]  dtype         (q normally carries d_k^-1/2 already)
 *  v      [B, T, H, Dv]  dtype
 *  g      [B, T, H, Dk]  float32       log-decay per key channel, g <= 0
 *  beta   [B, T, H]      dtype         write strength
 *  scale                               multiplies q in the read
 *  h0     [N, H, Dk, Dv] float32 or NULL (zero initial state)
 *  ht     [N, H, Dk, Dv] float32 or NULL (final state not stored); may equal h0
 *  o      [B, T, H, Dv]  o_dtype       output, every element written
 *  cu_seqlens  device int32[num_seqs + 1] or NULL. When given, B must be 1
 *              and the sequences are the packed segments of T; otherwise the
 *              N = B rows are the sequences and num_seqs is ignored.
 *  workspace   device buffer of at least kda_fwd_chunked_workspace_size()
 *              bytes (256-byte aligned); its contents are scratch.
 *
 * Sequences never share a chunk; a zero-length sequence leaves ht = h0 (or
 * zeros). Any finite g is handled exactly up to float32 rounding: every
 * in-chunk decay factor the kernels form is bounded by 2^120 in magnitude,
 * and 16-token blocks whose decay is too steep for that bound take a slower
 * pairwise path.
 * Errors (nothing is enqueued): KDA_ERROR_INVALID_VALUE for NULL q, k, v, g,
 * beta or o, non-positive sizes, B != 1 with cu_seqlens, num_seqs < 1 with
 * cu_seqlens, misaligned pointers or an unsupported head size;
 * KDA_ERROR_WORKSPACE if workspace is NULL or too small; KDA_ERROR_LAUNCH if
 * a launch fails. */
kda_status kda_fwd_chunked(const void* q, const void* k, const void* v, const float* g,
                           const void* beta, float scale, const float* h0, float* ht, void* o,
                           const int32_t* cu_seqlens, int num_seqs, int B, int T, int H, int Dk,
                           int Dv, kda_dtype dtype, kda_dtype o_dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

/* One decode step for N independent requests against persistent states.
 *
 *  q, k   [N, H, Dk]  dtype
 *  v      [N, H, Dv]  dtype
 *  g      [N, H, Dk]  float32
 *  beta   [N, H]      dtype
 *  state  [N, H, Dk, Dv] float32, read and updated in place (each element is
 *         read once and written once)
 *  o      [N, H, Dv]  o_dtype
 *
 * Errors (nothing is enqueued): KDA_ERROR_INVALID_VALUE for NULL pointers,
 * non-positive sizes, misalignment or an unsupported head size;
 * KDA_ERROR_LAUNCH if the launch fails. */
kda_status kda_decode_step(const void* q, const void* k, const void* v, const float* g,
                           const void* beta, float scale, float* state, void* o, int N, int H,
                           int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype, void* stream);

/* Chunked prefill from the raw projections: the input preparation of kda_prepare_inputs
 * (q^ = scale q / |q|, k^ = k / |k| over the Dk channels of each row, g = log sigmoid(a),
 * beta = sigmoid(b)) applied inside the prefill as the inputs are read, instead of as a
 * separate pass that writes the prepared tensors to memory. The prepared values stay in
 * float32 (they are not rounded to the input type), so results agree with kda_prepare_inputs
 * followed by kda_fwd_chunked up to that rounding. Normalised queries and keys are those of
 * "Notes on Linear Attention" (zhilingong.com), sections 4 and 5.3; the recurrence and its
 * chunkwise evaluation are those of kda_fwd_chunked.
 *
 *  q, k   [B, T, H, Dk]  bfloat16      raw projections (a zero row stays zero)
 *  v      [B, T, H, Dv]  bfloat16
 *  a      [B, T, H, Dk]  bfloat16      gate logits: g = log sigmoid(a)
 *  b      [B, T, H]      bfloat16      write-strength logits: beta = sigmoid(b)
 *
 * Every other argument, the workspace (sized by kda_fwd_chunked_workspace_size with
 * KDA_DTYPE_BF16), the aliasing rules and the errors are those of kda_fwd_chunked, except
 * that b needs only 2-byte alignment; KDA_ERROR_NOT_SUPPORTED unless dtype is
 * KDA_DTYPE_BF16 and Dk = Dv = 128 (kda_prepare_inputs and kda_fwd_chunked cover the other
 * cases). */
kda_status kda_fwd_chunked_raw(const void* q, const void* k, const void* v, const void* a,
                               const void* b, float scale, const float* h0, float* ht, void* o,
                               const int32_t* cu_seqlens, int num_seqs, int B, int T, int H,
                               int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device scratch built into the library for kda_fwd_chunked_noalloc:
 * 64 MiB on each device the library runs on, held until the process ends. */
#define KDA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

/* kda_fwd_chunked without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). The workspace is a fixed array of KDA_NOALLOC_SCRATCH_BYTES in the
 * library's device memory, one per device; the call itself allocates nothing (no
 * hipMalloc, hipFree or allocating library routine). Its address is looked up once per
 * device on the first call made with that device current.
 *
 * Every other argument, the results and the errors are those of kda_fwd_chunked, plus:
 * KDA_ERROR_WORKSPACE when kda_fwd_chunked_workspace_size() for these sizes exceeds
 * KDA_NOALLOC_SCRATCH_BYTES (about 680 chunk-heads of 64 tokens at d = 128 with bf16
 * input, e.g. H = 16 and T = 2700); KDA_ERROR_LAUNCH if the scratch address cannot be
 * obtained. All calls on one device share its scratch, and each call's results depend
 * only on its own inputs (nothing in the scratch needs clearing between calls), but two
 * calls whose execution overlaps on one device race on it: serialise them (one stream,
 * or events between streams). */
kda_status kda_fwd_chunked_noalloc(const void* q, const void* k, const void* v, const float* g,
                                   const void* beta, float scale, const float* h0, float* ht,
                                   void* o, const int32_t* cu_seqlens, int num_seqs, int B, int T,
                                   int H, int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                                   void* stream);

/* Gated DeltaNet: the same recurrence with one scalar retention gate per
 * token and head instead of one per key channel. Step (1) becomes
 * S~ = exp(g_t) S, every row decaying alike; steps (2)-(5) are unchanged.
 * This is the gated delta rule of "Notes on Linear Attention"
 * (zhilingong.com), section 6 (decay first, then the delta rule on the
 * decayed state), and of "From Fast Weight Programmers to KDA"
 * (jonahsamost.bearblog.dev), section "Gated Delta Networks" (written there
 * for the transposed state). It equals kda_fwd_chunked with g repeated over
 * the Dk channels; the kernels read the one value per token instead.
 *
 *  g      [B, T, H]      float32       log-decay, one per token and head
 *
 * Every other argument, the workspace (sized by
 * kda_fwd_chunked_workspace_size), the aliasing rules and the errors are
 * those of kda_fwd_chunked. */
kda_status kda_gdn_fwd_chunked(const void* q, const void* k, const void* v, const float* g,
                               const void* beta, float scale, const float* h0, float* ht,
                               void* o, const int32_t* cu_seqlens, int num_seqs, int B, int T,
                               int H, int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/* One Gated DeltaNet decode step: as kda_decode_step with g [N, H] float32,
 * one log-decay per request and head applied to every row of its state.
 * Arguments and errors are those of kda_decode_step. */
kda_status kda_gdn_decode_step(const void* q, const void* k, const void* v, const float* g,
                               const void* beta, float scale, float* state, void* o, int N,
                               int H, int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                               void* stream);

/* Gated DeltaNet-2: KDA's per-channel decay with beta split into an erase
 * gate b (one value per key channel) and a write gate w (one per value
 * channel), as on "From Fast Weight Programmers to KDA"
 * (jonahsamost.bearblog.dev), section "Gated DeltaNet-2" (written there for
 * the transposed state). Steps (2) and (3) become
 *
 *   v^  = S~^T (b_t * k_t)          read the old value through the gated key
 *   e   = w_t * v_t - v^            gated target minus the old value
 *
 * and the write S = S~ + k_t e^T stays at the original key. b = beta and
 * w = beta on every channel give kda_fwd_chunked.
 *
 *  b      [B, T, H, Dk]  dtype         erase gate (replaces beta)
 *  w      [B, T, H, Dv]  dtype         write gate
 *
 * Every other argument (g per key channel as for KDA), the workspace (sized
 * by kda_fwd_chunked_workspace_size), the aliasing rules and the errors are
 * those of kda_fwd_chunked; a NULL b or w is KDA_ERROR_INVALID_VALUE. */
kda_status kda_gdn2_fwd_chunked(const void* q, const void* k, const void* v, const float* g,
                                const void* b, const void* w, float scale, const float* h0,
                                float* ht, void* o, const int32_t* cu_seqlens, int num_seqs,
                                int B, int T, int H, int Dk, int Dv, kda_dtype dtype,
                                kda_dtype o_dtype, void* workspace, size_t workspace_bytes,
                                void* stream);

/* One Gated DeltaNet-2 decode step: as kda_decode_step with b [N, H, Dk] and
 * w [N, H, Dv] (dtype) in place of beta. */
kda_status kda_gdn2_decode_step(const void* q, const void* k, const void* v, const float* g,
                                const void* b, const void* w, float scale, float* state, void* o,
                                int N, int H, int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                                void* stream);

/* Serving state. A request's state is request-scoped serving state, kept
 * like a KV-cache slot: carried across turns, and copied or restored when a
 * request forks or a speculative draft is rolled back ("Module 03 - KDA I:
 * The Delta-Rule Recurrence", jared-hpc.com, section 5). */

/* T consecutive decode steps per request against a pool of states.
 *
 *  q, k, g    [N, T, H, Dk]  (g float32)     tokens t = 0 .. T-1 of request n
 *  v          [N, T, H, Dv]
 *  beta       [N, T, H]
 *  pool       [num_slots, H, Dk, Dv] float32; request n uses state slot
 *             slots[n] (device int32[N]), or slot n when slots is NULL
 *             (then num_slots >= N). On return the slot holds the state after
 *             the request's T tokens.
 *  snapshots  [N, T, H, Dk, Dv] float32 or NULL: the state after each token,
 *             so that the state after any accepted prefix of the T tokens can
 *             be restored with kda_state_copy (speculative verification).
 *  o          [N, T, H, Dv]  o_dtype
 *
 * Each step is the recurrent step of kda_decode_step, in token order; the
 * state stays in registers between steps, so it is read and written once per
 * call (plus the snapshots). Requests must use distinct slots. A slot outside
 * [0, num_slots) is skipped on the device: its request's o, snapshots and
 * state are not touched.
 * Errors (nothing is enqueued): KDA_ERROR_INVALID_VALUE for NULL q, k, v, g,
 * beta, pool or o, non-positive sizes, slots NULL with num_slots < N,
 * misalignment or an unsupported head size; KDA_ERROR_LAUNCH if the launch
 * fails. */
kda_status kda_decode_multi(const void* q, const void* k, const void* v, const float* g,
                            const void* beta, float scale, float* pool, int num_slots,
                            const int32_t* slots, float* snapshots, void* o, int N, int T,
                            int H, int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                            void* stream);

/* Copy whole states: dst[dst_slots[i]] = src[src_slots[i]] for i < pairs,
 * where dst holds dst_count states and src holds src_count states, each
 * [H, Dk, Dv] float32 (a snapshot array [N, T, H, Dk, Dv] is N * T states,
 * state n * T + t). Forks a request (pool to pool) or restores a snapshot
 * (snapshots to pool). dst_slots must be distinct and no destination state may
 * be the source of another pair; a slot outside its array's range skips that
 * pair on the device. pairs == 0 is a no-op.
 * Errors: KDA_ERROR_INVALID_VALUE for NULL pointers, negative sizes,
 * misalignment or an unsupported head size; KDA_ERROR_NOT_SUPPORTED for more
 * than 65535 pairs; KDA_ERROR_LAUNCH if the launch fails. */
kda_status kda_state_copy(float* dst, int dst_count, const int32_t* dst_slots, const float* src,
                          int src_count, const int32_t* src_slots, int pairs, int H, int Dk,
                          int Dv, void* stream);

/* Input preparation: the raw projections of `tokens` token positions
 * (B * T, or the packed total) to the inputs the calls above take, in one
 * pass over memory:
 *
 *   q_out = scale q / |q|     k_out = k / |k|      L2 norm over the Dk channels
 *   g_out = log sigmoid(a)    (float32, one log-decay per key channel, < 0)
 *   beta_out = sigmoid(b)
 *
 * Normalised queries and keys are those of "Notes on Linear Attention"
 * (zhilingong.com), sections 4 and 5.3; beta as a sigmoid of a projection is
 * the write strength of "From Fast Weight Programmers to KDA"; the pages fix
 * g = log(alpha) with alpha in (0, 1) but not its parameterisation, and
 * alpha = sigmoid(a) is the plainest map onto that range.
 *
 *  q, k, a   [tokens, H, Dk]  dtype
 *  b         [tokens, H]      dtype
 *  q_out, k_out [tokens, H, Dk] dtype; g_out [tokens, H, Dk] float32;
 *  beta_out  [tokens, H] dtype. Outputs are rounded to nearest even when
 *  dtype is bfloat16. q_out, k_out and beta_out may alias q, k and b, and
 *  g_out may alias a when dtype is float32; a row of zeros stays zero.
 * Errors (nothing is enqueued): KDA_ERROR_INVALID_VALUE for NULL pointers,
 * non-positive sizes, an unsupported Dk or dtype, q, k, a, q_out, k_out or
 * g_out not 16-byte aligned, b or beta_out not element-aligned;
 * KDA_ERROR_NOT_SUPPORTED above 2^34 token-head rows; KDA_ERROR_LAUNCH if the
 * launch fails. */
kda_status kda_prepare_inputs(const void* q, const void* k, const void* a, const void* b,
                              float scale, void* q_out, void* k_out, float* g_out,
                              void* beta_out, long long tokens, int H, int Dk, kda_dtype dtype,
                              void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
