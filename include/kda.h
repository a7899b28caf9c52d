/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA recurrent prefill forward.
 *
 * The operation is the Kimi Delta Attention prefill forward described by the
 * FlashInfer PR #4262 summary (section 1 "A Fused Recurrent-Prefill Kernel",
 * section 2 "Chunk-32 Through Fixed-Anchor Exponent Centering", section 3
 * "Intra-Chunk and Inter-Chunk Decomposition") with the call contract of
 * FlashKDA's `fwd` ("How FlashKDA Manages Recurrent State Across Sequences and
 * Batch Modes", the Python wrapper and both modes).  Per sequence n and head h
 * the V x K state S evolves token by token as
 *
 *     lam_t = lower_bound * sigmoid(exp(A_log[h]) * (g_t + dt_bias[h]))  (per key column)
 *     S     = S * diag(exp(lam_t))
 *     S     = S + sigmoid(beta_t) * (v_t - S kh_t) kh_t^T
 *     out_t = scale * S qh_t
 *
 * with qh, kh the L2-normalised q and k rows (x / sqrt(|x|^2 + 1e-6)).  The
 * library evaluates this in chunks of 32 or 16 tokens (fewer for strongly
 * negative lower bounds) with bf16 matrix-core products and an fp32 state that
 * stays on chip for the whole sequence.
 * Within a chunk the decayed operands are centred on a fixed exponent anchor
 * (section 2 of the PR #4262 summary); the state rows' 1-norms must stay below
 * 2^25 for the centred state products to stay inside fp32, and q and k rows
 * below an L2 norm of 1.8e19 (their sums of squares are fp32).
 *
 * Conventions for every entry point:
 *   - Every pointer argument except `stream` is a caller-owned DEVICE pointer
 *     to contiguous memory; the library never frees or retains it.
 *   - Kernels launch on the calling thread's current HIP device: the pointers
 *     and `stream` must belong to it (hipSetDevice before the call).
 *   - The library allocates nothing and keeps no global state; calls on
 *     different streams may run concurrently.  The one exception is
 *     kda_fwd_split_noalloc, whose scratch is a static device array per GPU.
 *   - kda_fwd is asynchronous: it validates on the host, enqueues one kernel on
 *     `stream` and returns.  It never reads device memory on the host (in
 *     particular not cu_seqlens) and never synchronises.
 *   - Errors are returned as negative status codes; nothing aborts or throws
 *     across this ABI.  On a validation error nothing is enqueued.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define KDA_OK 0
#define KDA_ERR_NULL_ARG (-1)        /* a required pointer is NULL (q, k, v, g, beta and */
                                     /* out may be NULL when B * T == 0)                */
#define KDA_ERR_BAD_SHAPE (-2)       /* B,T,H < 1 (T may be 0 only with cu_seqlens),     */
                                     /* D not in {32, 64, 128}, H * D >= 2^25,            */
                                     /* B * T > 2^40, num_seqs * H > 2^29, an activation  */
                                     /* tensor of more than 2^62 bytes, or a launch of    */
                                     /* more than 2^32 - 1 work-items (workgroups times   */
                                     /* their 128 to 768 threads)                         */
#define KDA_ERR_BAD_DTYPE (-3)       /* unknown state dtype code                         */
#define KDA_ERR_BAD_VARLEN (-4)      /* cu_seqlens with B != 1, num_seqs < 1, or         */
                                     /* num_seqs != B without cu_seqlens                 */
#define KDA_ERR_BAD_ALIAS (-5)       /* an output overlaps an input or the other output; */
                                     /* only the exact in-place state alias is allowed   */
#define KDA_ERR_BAD_LOWER_BOUND (-6) /* lower_bound not finite, not < 0, below -2.35e38 */
                                     /* (lb log2(e) not a finite float), or too strong   */
                                     /* for a forced chunk size (see kda_fwd)            */
#define KDA_ERR_BAD_SCALE (-7)       /* scale not finite                                 */
#define KDA_ERR_BAD_SCHEDULE (-8)    /* unsupported forced chunk size or value tile      */
#define KDA_ERR_HIP (-9)             /* the HIP runtime reported an error at launch      */
#define KDA_ERR_BAD_WORKSPACE (-10)  /* kda_fwd_split: workspace smaller than required   */
#define KDA_ERR_SCRATCH_TOO_SMALL (-11) /* kda_fwd_split_noalloc: the call's workspace   */
                                        /* exceeds kda_split_noalloc_max_bytes()         */

/* State dtype codes (initial_state_dtype, final_state_dtype). */
#define KDA_DTYPE_BF16 0
#define KDA_DTYPE_FP32 1

/*
 * kda_fwd -- the prefill forward (FlashKDA `fwd` contract: q, k, v, g, beta,
 * scale, out, A_log, dt_bias, lower_bound, initial_state, final_state,
 * cu_seqlens).
 *
 *   q, k, v, g     bf16 [B, T, H, D], contiguous (D fastest).  K = V = D.
 *   beta           bf16 [B, T, H], logits (the kernel applies the sigmoid).
 *   scale          output scale, folded into the normalised q; finite.
 *   out            bf16 [B, T, H, D], written for every token (padding-free).
 *   A_log          fp32 [H].
 *   dt_bias        fp32 [H, D].
 *   lower_bound    gate lower bound lb (finite, < 0); per-token decay lies in (lb, 0).
 *   initial_state  [num_seqs, H, D(v), D(k)] of initial_state_dtype, or NULL for zeros.
 *   final_state    [num_seqs, H, D(v), D(k)] of final_state_dtype, or NULL (not written).
 *                  It may be exactly the same allocation as initial_state (same
 *                  pointer and dtype: in-place update); any other overlap between
 *                  buffers is rejected.  Each workgroup reads all state rows it
 *                  owns before it writes any of them, which makes the alias safe.
 *   cu_seqlens     int64 [num_seqs + 1] device array, or NULL.
 *                  NULL: batched mode, num_seqs == B, sequence b is tokens
 *                  [b*T, (b+1)*T) of the flattened [B*T] axis, no resets.
 *                  Non-NULL: varlen mode, B == 1, sequence n is tokens
 *                  [cu[n], cu[n+1]); the state restarts from initial_state[n]
 *                  (or zeros) at every sequence.  Preconditions (not checked on
 *                  the host, which never reads device memory): cu[0] = 0,
 *                  non-decreasing, cu[num_seqs] = T.  The kernel clamps every
 *                  index into [0, T] so a malformed array cannot make it access
 *                  memory out of bounds; results are then unspecified.
 *                  An empty sequence passes its initial state (or zeros) through.
 *   num_seqs       N (see above).
 *   B, T, H, D     sizes; D in {32, 64, 128}.
 *   stream         a hipStream_t (NULL: the null stream).
 *
 * Scheduling: a packed batch of at most 256 sequences whose workgroups (num_seqs *
 * H * D / value tile) number between one and four times the device's compute
 * units is dispatched longest first: the kernel ranks the lengths itself, so the
 * host still reads nothing.  The order never changes the results (see
 * kda_fwd_ordered for a caller-chosen order).
 *
 * Returns KDA_OK or a negative status.  The decay span of a chunk is
 * chunk * |lower_bound| * log2(e); it must not exceed 236.  The library uses the
 * longest chunk whose span allows it: 32 tokens for |lb| <= 5.112, 16 for
 * |lb| <= 10.22, then 8, 4 and 2 tokens, and one token per chunk for every
 * stronger lower bound (chunks shorter than 16 tokens run in 16-row tiles, so each
 * halving of the chunk doubles the kernel's sequential steps).  Past
 * |lb| = 163.6 one token's decay can exceed the span: the kernel then floors each
 * token's decay factor at 2^-236 (about 1e-71), which differs from the exact
 * recurrence by less than 1e-71 times the state.  See kda_chunk_anchor.
 */
int kda_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
            float scale, void* out, const float* A_log, const float* dt_bias, float lower_bound,
            const void* initial_state, int initial_state_dtype, void* final_state,
            int final_state_dtype, const int64_t* cu_seqlens, int64_t num_seqs, int64_t B,
            int64_t T, int64_t H, int64_t D, void* stream);

/*
 * kda_fwd_sched -- kda_fwd with a forced schedule, for tests and tuning.
 *   chunk_size  0 (automatic), or tokens per chunk: 32, 16, 8, 4, 2 or 1
 *               (KDA_ERR_BAD_SCHEDULE otherwise).  A chunk of 2 or more tokens
 *               whose decay span exceeds 236 (see kda_fwd) is rejected with
 *               KDA_ERR_BAD_LOWER_BOUND, e.g. 32 when |lb| > 5.112; one-token
 *               chunks take every lower bound.
 *   v_tile      0 (automatic) or the number of value rows one workgroup owns:
 *               a divisor of D that is a multiple of 16 and at least 32
 *               (KDA_ERR_BAD_SCHEDULE otherwise).  Automatic: D, or D/2 for
 *               D = 128 with 32-token chunks when twice num_seqs * H workgroups
 *               still fit one per compute unit of the current device (queried
 *               on the host; the host never synchronises).
 * Everything else is exactly as kda_fwd.
 */
int kda_fwd_sched(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  float scale, void* out, const float* A_log, const float* dt_bias,
                  float lower_bound, const void* initial_state, int initial_state_dtype,
                  void* final_state, int final_state_dtype, const int64_t* cu_seqlens,
                  int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t D, void* stream,
                  int chunk_size, int v_tile);

/*
 * kda_fwd_ordered -- kda_fwd with a caller-chosen order of the sequences over
 * the workgroups (the sequence-order option of the FlashInfer PR #4262
 * summary's integration section, where it serves tail utilisation).
 *   seq_order  int32 [num_seqs] device array, a permutation of 0 .. num_seqs-1:
 *              the workgroups of sequence seq_order[0] are dispatched first,
 *              then those of seq_order[1], and so on.  Longest first (see
 *              kda_longest_first) keeps long sequences of a packed batch from
 *              starting last.  It must not overlap any output
 *              (KDA_ERR_BAD_ALIAS); NULL is KDA_ERR_NULL_ARG.
 * The results are bitwise those of kda_fwd: the order only changes which
 * workgroup starts when.  The host never reads seq_order; entries outside
 * [0, num_seqs) are clamped (in bounds, but the results are then unspecified).
 * Everything else is exactly as kda_fwd.
 */
int kda_fwd_ordered(const void* q, const void* k, const void* v, const void* g,
                    const void* beta, float scale, void* out, const float* A_log,
                    const float* dt_bias, float lower_bound, const void* initial_state,
                    int initial_state_dtype, void* final_state, int final_state_dtype,
                    const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T, int64_t H,
                    int64_t D, void* stream, const int32_t* seq_order);

/*
 * kda_fwd_bf16_state -- kda_fwd_sched with the recurrent state held in bf16 in
 * on-chip memory (LDS) instead of fp32 registers, as the page "How FlashKDA
 * Stores On-Chip Recurrent State in BF16 for Memory Efficiency" describes (its
 * sections "The BF16 State Layout in Shared Memory" and "State Updates with FP32
 * FMA"): each chunk's update widens the stored state to fp32, applies the decay
 * and adds the chunk's term in fp32, then rounds once back to bf16.  An fp32
 * initial state is rounded to bf16 on entry; the final state is the stored bf16
 * state (exact in either output dtype).
 * Runs D = 128 with 32-token chunks (chunk_size 0 or 32; the lower bound must
 * allow them, |lb| <= 5.112) at v_tile 0, 64 or 128; other schedules return
 * KDA_ERR_BAD_SCHEDULE.  States are [num_seqs, H, D(v), D(k)] as for kda_fwd;
 * everything else, including the exact in-place alias, is exactly as kda_fwd.
 * The results differ from kda_fwd by the per-chunk rounding of the state; it is
 * an opt-in mode and never chosen automatically.
 */
int kda_fwd_bf16_state(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, float scale, void* out, const float* A_log,
                       const float* dt_bias, float lower_bound, const void* initial_state,
                       int initial_state_dtype, void* final_state, int final_state_dtype,
                       const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T,
                       int64_t H, int64_t D, void* stream, int chunk_size, int v_tile);

/*
 * kda_fwd_transposed_state -- kda_fwd with both states in the transposed,
 * key-major layout [num_seqs, H, D(k), D(v)]: element (v, k) of a head's
 * state sits at k * D + v (FlashKDA's alternative state layout, its
 * transpose-state-layout option).  Everything else, including the exact
 * in-place alias, is exactly as kda_fwd; the results equal those of kda_fwd on
 * transposed states bitwise.
 */
int kda_fwd_transposed_state(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, float scale, void* out, const float* A_log,
                             const float* dt_bias, float lower_bound, const void* initial_state,
                             int initial_state_dtype, void* final_state, int final_state_dtype,
                             const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T,
                             int64_t H, int64_t D, void* stream);

/*
 * kda_split_workspace_bytes -- bytes of the workspace kda_fwd_split needs.
 *   T_total     tokens of the flattened batch (B * T).
 *   num_seqs    N, as for kda_fwd.
 *   H, D        heads and head dimension; the split runs D = 128 only.
 *   lower_bound, chunk_size  as for kda_fwd_sched (0: automatic chunk length); pass
 *               kda_fwd_split the same chunk_size.
 * One record per slot and head: the prepared operands of one chunk (Qc, Kc, Kr,
 * the solve operands, Mqk and the decay, in the layout the recurrent kernel copies
 * into LDS; 35,840 bytes at 32-token chunks).  A head has floor(T_total / chunk)
 * + num_seqs + 1 slots.  Returns the size, or a negative status
 * (KDA_ERR_BAD_SHAPE, also when a head's records reach 2^31 bytes or the prep
 * kernel's grid of slots times heads workgroups of 512 threads exceeds 2^32 - 1
 * work-items; KDA_ERR_BAD_LOWER_BOUND; KDA_ERR_BAD_SCHEDULE).
 */
int64_t kda_split_workspace_bytes(int64_t T_total, int64_t num_seqs, int64_t H, int64_t D,
                                  float lower_bound, int chunk_size);

/*
 * kda_fwd_split -- kda_fwd as two kernels, the organisation of FlashKDA's
 * prep and recurrent kernels that the FlashInfer PR #4262 summary describes
 * (its workspace of chunk-local matrices and transformed Q and K between them).
 * A token-parallel kernel prepares every chunk of every head (gate, prefix,
 * norms, centred operands, Mqk and the inverted diagonal blocks) and writes it to
 * `workspace`.  The recurrent kernel then reads those records back in chunk order
 * and runs only the state side, on value tiles of v_tile rows.
 *   workspace        caller-owned device memory of at least
 *                    kda_split_workspace_bytes(B * T, num_seqs, H, D, lower_bound,
 *                    chunk_size) bytes (KDA_ERR_BAD_WORKSPACE otherwise,
 *                    KDA_ERR_NULL_ARG when NULL).  It must not overlap any other
 *                    argument (KDA_ERR_BAD_ALIAS).  Its contents on entry do not
 *                    matter and are scratch on return.
 *   workspace_bytes  its size in bytes.
 *   chunk_size       0 (automatic) or a forced chunk length, as for kda_fwd_sched.
 *   v_tile           0 (automatic, as for kda_fwd), 128, or 64 at 32-token chunks;
 *                    other schedules are KDA_ERR_BAD_SCHEDULE, as is D != 128.
 * The results are bitwise those of kda_fwd_sched with the same chunk length and
 * value tile: both
 * kernels run the fused kernel's own preparation and state-side code.  Both are
 * enqueued on `stream`.  Everything else is exactly as kda_fwd.
 */
int kda_fwd_split(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  float scale, void* out, const float* A_log, const float* dt_bias,
                  float lower_bound, const void* initial_state, int initial_state_dtype,
                  void* final_state, int final_state_dtype, const int64_t* cu_seqlens,
                  int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t D, void* stream,
                  void* workspace, int64_t workspace_bytes, int chunk_size, int v_tile);

/*
 * kda_fwd_split_noalloc -- kda_fwd_split for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The workspace is the library's own scratch: a static device
 * array of kda_split_noalloc_max_bytes() bytes (64 MiB) that each GPU the library
 * runs on holds until the process ends.  Its address is resolved once per device,
 * on the first call with that device current; the call allocates nothing.
 *   chunk_size, v_tile  as for kda_fwd_split.
 * A call whose kda_split_workspace_bytes(B * T, num_seqs, H, D, lower_bound,
 * chunk_size) exceeds the scratch returns KDA_ERR_SCRATCH_TOO_SMALL before
 * anything is enqueued (for example 96 heads hold 19 records of 35,840 bytes each:
 * T_total + 32 num_seqs below about 576 tokens at 32-token chunks).  Every call on a
 * GPU shares that GPU's array and leaves its records there; calls that overlap in
 * time on one GPU (concurrent streams, or threads) race on it and must be
 * serialised by the caller.  Nothing in the array needs to start at zero: every
 * record is written by the call's prep kernel before its recurrent kernel reads it.
 * The results are bitwise those of kda_fwd_split.  Returns KDA_OK, a kda_fwd_split
 * status, KDA_ERR_SCRATCH_TOO_SMALL, or KDA_ERR_HIP if the scratch address cannot
 * be resolved.
 */
int kda_fwd_split_noalloc(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, float scale, void* out, const float* A_log,
                          const float* dt_bias, float lower_bound, const void* initial_state,
                          int initial_state_dtype, void* final_state, int final_state_dtype,
                          const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T,
                          int64_t H, int64_t D, void* stream, int chunk_size, int v_tile);

/* kda_split_noalloc_max_bytes -- bytes of kda_fwd_split_noalloc's scratch (64 MiB). */
int64_t kda_split_noalloc_max_bytes(void);

/*
 * kda_longest_first -- writes the longest-first order of a packed batch for
 * kda_fwd_ordered: seq_order[i] is the index of the sequence with the i-th
 * largest length cu_seqlens[n+1] - cu_seqlens[n] (equal lengths keep their
 * index order).  One small kernel on `stream`; the host reads nothing.
 *   cu_seqlens  int64 [num_seqs + 1] device array (as for kda_fwd).
 *   num_seqs    1 .. 8192 (KDA_ERR_BAD_VARLEN otherwise).
 *   seq_order   int32 [num_seqs] device array, written; must not overlap
 *               cu_seqlens (KDA_ERR_BAD_ALIAS).
 * Returns KDA_OK, KDA_ERR_BAD_VARLEN (checked first), KDA_ERR_NULL_ARG,
 * KDA_ERR_BAD_ALIAS or KDA_ERR_HIP.  An order depends only on the lengths, so one computation can
 * serve every layer of a model that shares the batch.
 */
int kda_longest_first(const int64_t* cu_seqlens, int64_t num_seqs, int32_t* seq_order,
                      void* stream);

/*
 * kda_fwd_check -- the host-side validation of kda_fwd_sched on its own: the
 * same arguments without the stream, returns the status kda_fwd_sched would
 * return before launching.  Pure host code (pointer values are compared, never
 * dereferenced); needs no GPU.
 */
int kda_fwd_check(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  float scale, const void* out, const float* A_log, const float* dt_bias,
                  float lower_bound, const void* initial_state, int initial_state_dtype,
                  const void* final_state, int final_state_dtype, const int64_t* cu_seqlens,
                  int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t D, int chunk_size,
                  int v_tile);

/*
 * kda_chunk_anchor -- the fixed exponent anchor Ca (base 2) the library centres a
 * chunk's operands on: the middle of the chunk's decay span,
 * chunk_size * lower_bound * log2(e) / 2 (-118 for one-token chunks whose span
 * exceeds 236, where the decay is floored).  For 32-token chunks this is section 2
 * of the PR #4262 summary's 16 * lower_bound * log2(e) (about -115.42 for
 * lower_bound = -5).  The centred operands then reach 2^(-Ca) at most and keep
 * as much room above the bf16 normal minimum as below its maximum, which the
 * most strongly decayed rows of a chunk need.  Pure host function.
 */
float kda_chunk_anchor(float lower_bound, int chunk_size);

/* kda_status_string -- a static, human-readable name for a status code. */
const char* kda_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
