/*
 * lightning.h - C ABI of the MI355X (gfx950) Lightning Attention library.
 *
 * The operator is the causal linear attention with a per-head exponential
 * decay described in MiniMax Signal Lab · M1 (ailearn.mscapital.top),
 * §03 Lightning Attention. For a block t of B tokens (positions i, j = 1..B;
 * a last short block uses its real length m in place of B):
 *
 *     D_ij    = e^{-s_h (i - j)} [i >= j]
 *     O_intra = [(Q_t K_t^T) ⊙ D] V_t
 *     O_inter = (Q_t ⊙ d_q) S_{t-1},          d_q[i] = e^{-s_h i}
 *     O_t     = O_intra + O_inter              (§03 dataflow figure: the two
 *                                              outputs are added)
 *     S_t     = e^{-s_h B} S_{t-1} + (K_t ⊙ d_k)^T V_t,   d_k[j] = e^{-s_h (B - j)}
 *
 * with a fixed d x d FP32 state S per head (§03, and §04 Context Cache, whose
 * 70-layer state total fixes d x d FP32 per head for 64 heads of d = 128).
 * "⊙" with a length-B vector scales token rows. The value of O and of the final
 * state does not depend on B: the block form is an exact re-association of the
 * per-token recurrence S <- e^{-s_h} S + k^T v, o = q S (the token sees its own
 * key). The kernels may leave out a finite carried-state term once its decay
 * factor e^{-s t} is below 2^-16 (2^7 below the bf16 rounding of the state as
 * an operand of the products, the kernels' dominant rounding).
 * lt_prefill, lt_prefill_varlen and lt_decode write the raw sum; the
 * *_norm_gate variants also apply the normalisation and gate that follow the
 * sum in the §03 data-flow figure before anything is stored.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument except `stream` is a DEVICE pointer (HBM). The
 *    caller owns every buffer; the library allocates nothing, keeps no global
 *    state (lt_prefill_noalloc aside, whose static device scratch is described
 *    there), and never synchronises.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns before it runs.
 *  - Layouts are dense and row-major with head_dim innermost. Element offsets
 *    are 64-bit, so a tensor may exceed 2^31 elements.
 *  - State tensors are FP32 [units, heads, head_dim (key index), head_dim
 *    (value index)]: S[r][c] multiplies key component r into value column c.
 *  - Slopes are FP32 [heads], s_h >= 0 (0 = no decay). Their values are read on
 *    the device and are not validated.
 *  - Non-finite values. A NaN or Inf in any input (q, k, v, a carried-in
 *    state, a slope) makes non-finite every output that the exact operator
 *    makes non-finite, on every launch plan (NaN or Inf: which of the two may
 *    differ from the exact result). The cutoff of carried-state terms below
 *    2^-16 is never applied to a carried-in state that holds a NaN or Inf.
 *    Outputs the exact operator leaves finite stay finite and within rounding,
 *    with one exception: a NaN or Inf in v at token t can also make NaN, in the
 *    value columns it holds, the outputs of the earlier tokens of t's 64-token
 *    block (blocks counted from the sequence start): masked entries of the
 *    in-block product are zeros multiplied on the matrix cores, and 0 * Inf is
 *    NaN there. (The backward: non-finite gradients wherever the exact
 *    derivative is non-finite; a non-finite input can also make NaN the other
 *    gradients of its 64-token block, counted from either end.)
 *  - Arguments are validated on the host before any launch. A failed check
 *    returns its status and enqueues nothing. A failed launch returns
 *    LT_ERR_HIP. No C++ exception crosses this interface.
 *  - Supported: head_dim == 128; 0 <= heads <= LT_MAX_HEADS; in_dtype LT_BF16 or LT_F32 (bf16 inputs are
 *    multiplied on MFMA with fp32 accumulation; fp32 inputs on fp32 MFMA);
 *    out_dtype LT_F32 or LT_BF16.
 *  - Overlap: `state_in == state_out` (same address) is allowed and updates the
 *    state in place. Any other overlap between an output and any other buffer
 *    is rejected with LT_ERR_ALIAS.
 */
#ifndef LIGHTNING_H
#define LIGHTNING_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define LT_API __attribute__((visibility("default")))
#else
#define LT_API
#endif

typedef enum {
    LT_OK = 0,
    LT_ERR_NULL = 1,      /* a required pointer is NULL */
    LT_ERR_SHAPE = 2,     /* unsupported or inconsistent sizes */
    LT_ERR_BLOCK = 3,     /* block size out of range */
    LT_ERR_DTYPE = 4,     /* unsupported dtype code */
    LT_ERR_ALIAS = 5,     /* an output overlaps another buffer */
    LT_ERR_HIP = 6,       /* the HIP runtime reported an error at launch */
    LT_ERR_VALUE = 7,     /* a scalar argument is out of range (eps of the norm-gate variants) */
    LT_ERR_SCRATCH = 8    /* the call needs more scratch than lt_prefill_noalloc holds */
} lt_status;

typedef enum { LT_F32 = 0, LT_BF16 = 1 } lt_dtype;

/* Largest block size accepted by the prefill entry points. */
#define LT_MAX_BLOCK 65536
/* Largest head count accepted (keeps in-kernel token strides in 32 bits). */
#define LT_MAX_HEADS 65536

/* Human-readable name of a status code (static storage; never NULL). */
LT_API const char *lt_status_string(int status);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
LT_API int lt_version(void);

/* Build identity: a hash of the sources the library was compiled from (16 hex
 * digits; "unknown" when built without one). Static storage; never NULL. Runs
 * no HIP call, so it can be read on a machine without a GPU. */
LT_API const char *lt_build_id(void);

/*
 * lt_init - optional set-up on the calling thread's current device: loads the
 * library's GPU code there (the HIP runtime otherwise loads a kernel source's
 * code at the first launch of one of its kernels, a few milliseconds of host
 * work inside that first call) and looks up the device address of
 * lt_prefill_noalloc's scratch. Safe to call more than once and from several
 * threads; each other entry point works without it.
 *   Errors: LT_ERR_HIP (no device, or a load failed).
 */
LT_API lt_status lt_init(void);

/*
 * lt_prefill - block-wise prefill of `batch` sequences of equal length.
 *
 *   q, k, v    [batch, seqlen, heads, head_dim], in_dtype.
 *   slopes     [heads] fp32 per-head decay slopes s_h.
 *   o          [batch, seqlen, heads, head_dim], out_dtype: O_intra + O_inter.
 *   state_in   [batch, heads, head_dim, head_dim] fp32 carried-in state S_0,
 *              or NULL for a zero state. The first token decays it once
 *              (o_1 = q_1 (e^{-s} S_0 + k_1^T v_1)), as in the per-token form.
 *   state_out  same shape: the state after the last token, or NULL to skip.
 *              May equal state_in.
 *   block      the method's block length B, 1..LT_MAX_BLOCK. The result does
 *              not depend on it (see above); the kernels schedule their own
 *              sub-blocks.
 *   workspace  device scratch of workspace_bytes bytes owned by the caller (see
 *              lt_prefill_workspace_bytes), or NULL. Its contents on entry do
 *              not matter; it must not overlap any other argument.
 *   seqlen 0 writes state_out = state_in (or zeros). batch 0 or heads 0 is a
 *   no-op. Errors: LT_ERR_NULL, LT_ERR_SHAPE, LT_ERR_BLOCK, LT_ERR_DTYPE,
 *   LT_ERR_ALIAS, LT_ERR_HIP.
 */
LT_API lt_status lt_prefill(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                            const float *slopes, void *o, lt_dtype out_dtype,
                            const float *state_in, float *state_out,
                            int batch, long long seqlen, int heads, int head_dim, int block,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * lt_prefill_workspace_bytes - device workspace that lets lt_prefill split long
 * sequences across workgroups (used when batch * heads is too small to occupy
 * the GPU with one workgroup per sequence and head; holds one fp32 d x d state
 * per sequence, head and sequence piece). Returns 0 when no workspace helps or
 * the arguments are invalid. Given a smaller workspace, lt_prefill splits the
 * sequences into longer pre-pass pieces whose states fit it (the coarsest split
 * needs at most 63.75 MiB); given NULL or less than that, it still computes the
 * same result, with four workgroups per (sequence, head), one per 32 value
 * columns (the norm-gate variants, which need whole output rows, with one
 * workgroup per (sequence, head)).
 */
LT_API size_t lt_prefill_workspace_bytes(int batch, long long seqlen, int heads, int head_dim,
                                         lt_dtype in_dtype);

/*
 * lt_prefill_noalloc - lt_prefill for callers that cannot allocate device
 * memory at call time: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments, result and errors as
 * lt_prefill, without the workspace pair: the split of long sequences across
 * workgroups takes its states from a 64 MiB scratch array that the library
 * holds in each GPU's memory from the first call on that GPU (the device of
 * `stream`) until the process ends. No call allocates or frees memory.
 *   - The planner takes the finest pre-pass pieces whose states fit the
 *     scratch; every shape lt_prefill accepts fits (the coarsest plan of any
 *     of them needs at most 63.75 MiB). A plan that did not fit would return
 *     LT_ERR_SCRATCH and enqueue nothing.
 *   - Every call on one GPU uses that GPU's one scratch array. Calls whose
 *     work overlaps on one GPU (other streams, other threads, or graph
 *     replays running at the same time) race on it and give wrong results;
 *     calls ordered on one stream do not. Nothing in the scratch needs to be
 *     zero on entry, and it keeps the last call's contents.
 *   Errors: those of lt_prefill, LT_ERR_SCRATCH, and LT_ERR_HIP when the
 *   scratch address cannot be looked up.
 */
LT_API lt_status lt_prefill_noalloc(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                                    const float *slopes, void *o, lt_dtype out_dtype,
                                    const float *state_in, float *state_out,
                                    int batch, long long seqlen, int heads, int head_dim, int block,
                                    void *stream);

/*
 * lt_prefill_varlen - prefill of `num_seqs` packed sequences of different
 * lengths, each with its own carried-in state: chunked prefill, or resuming a
 * sequence whose state was kept (the §03 block form carries the state from one
 * block to the next, so a later call that starts from it continues the same
 * sequence; §04: that state is all a sequence keeps, whatever its length).
 *
 *   q, k, v     [total_tokens, heads, head_dim], in_dtype; sequence n owns rows
 *               cu_seqlens[n] .. cu_seqlens[n+1]-1.
 *   cu_seqlens  [num_seqs + 1] int32 on the device: cu[0] = 0, non-decreasing,
 *               cu[num_seqs] = total_tokens. Contents are not checked on the
 *               host; the kernels clamp every boundary into [0, total_tokens],
 *               so malformed boundaries give wrong results, never stray memory
 *               accesses.
 *   max_seqlen  length of the longest sequence, 0 <= max_seqlen <= total_tokens
 *               (0: not known, taken as total_tokens). With few (sequence,
 *               head) pairs, sequences are split across workgroups like
 *               lt_prefill's, on segments cut from max_seqlen; a value below
 *               the longest real length gives wrong results for the longer
 *               sequences (never memory accesses outside the tensors).
 *   slopes, o, state_in, state_out, block: as lt_prefill, with state tensors
 *               [num_seqs, heads, head_dim, head_dim]. Blocks restart at each
 *               sequence start; zero-length sequences pass their state through.
 *   workspace   as lt_prefill's, sized by lt_prefill_varlen_workspace_bytes
 *               (NULL or smaller: the same result from an unsplit plan or
 *               coarser pieces).
 *   Errors: as lt_prefill (LT_ERR_SHAPE also for max_seqlen outside
 *   [0, total_tokens] or total_tokens >= 2^31).
 */
LT_API lt_status lt_prefill_varlen(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                                   const int *cu_seqlens, int num_seqs, long long total_tokens,
                                   long long max_seqlen, const float *slopes, void *o,
                                   lt_dtype out_dtype, const float *state_in, float *state_out,
                                   int heads, int head_dim, int block, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * lt_prefill_varlen_workspace_bytes - the workspace lt_prefill_varlen (and its
 * norm-gate variant) uses to split the sequences of a packed batch whose
 * longest sequence has max_seqlen tokens (0 when no workspace helps or the
 * arguments are invalid).
 */
LT_API size_t lt_prefill_varlen_workspace_bytes(int num_seqs, long long max_seqlen, int heads,
                                                int head_dim, lt_dtype in_dtype);

/*
 * lt_decode - one decode step for `batch` sequences: each reads and writes its
 * fixed-size state in place (§03: the next block reads the carried state
 * directly instead of rescanning history; §04: that state does not grow):
 *
 *     S <- e^{-s_h} S + k^T v ;   o = q S   (o reads the updated state)
 *
 *   q, k, v  [batch, heads, head_dim], in_dtype (one token per sequence).
 *   state    [batch, heads, head_dim, head_dim] fp32, updated IN PLACE.
 *   o        [batch, heads, head_dim], out_dtype.
 *   A single token has no block, so there is no block argument.
 *   Errors: LT_ERR_NULL, LT_ERR_SHAPE, LT_ERR_DTYPE, LT_ERR_ALIAS, LT_ERR_HIP.
 */
LT_API lt_status lt_decode(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                           const float *slopes, float *state, void *o, lt_dtype out_dtype,
                           int batch, int heads, int head_dim, void *stream);

/*
 * lt_prefill_backward - gradients of a fixed-length prefill. For the loss
 *     l = sum_t dout_t . o_t + <d_state_out, S_final>   per (sequence, head)
 * it writes dq, dk, dv (= dl/dq, dl/dk, dl/dv) and d_state_in (= dl/dS_0).
 * The pages give no backward; this is the reverse-mode derivative of the
 * operator above. With G_t = q_t^T dout_t + e^{-s_h} G_{t+1} and
 * G_L = q_L^T dout_L + d_state_out:
 *     dq_t = dout_t S_t^T,  dk_t = G_t v_t,  dv_t = G_t^T k_t,
 *     d_state_in = e^{-s_h} G_1.
 * The slopes get no gradient.
 *
 *   q, k, v, dout  [batch, seqlen, heads, head_dim] bf16 (in_dtype must be
 *                  LT_BF16), the forward's inputs and the output gradient.
 *   state_in       the forward's S_0, or NULL for zero.
 *   d_state_out    [batch, heads, head_dim, head_dim] fp32 gradient of the
 *                  final state, or NULL for zero.
 *   dq, dk, dv     [batch, seqlen, heads, head_dim], grad_dtype (LT_F32 or
 *                  LT_BF16).
 *   d_state_in     [batch, heads, head_dim, head_dim] fp32, or NULL to skip.
 *   block, workspace: as lt_prefill (the workspace serves the dq pass and
 *                  then the reverse pass, one after the other on `stream`;
 *                  query its size with lt_prefill_workspace_bytes).
 *   No output may overlap an input or another output (LT_ERR_ALIAS).
 *   Errors: LT_ERR_NULL, LT_ERR_SHAPE, LT_ERR_BLOCK, LT_ERR_DTYPE,
 *   LT_ERR_ALIAS, LT_ERR_HIP.
 */
LT_API lt_status lt_prefill_backward(const void *q, const void *k, const void *v, const void *dout,
                                     lt_dtype in_dtype, const float *slopes, const float *state_in,
                                     const float *d_state_out, void *dq, void *dk, void *dv,
                                     lt_dtype grad_dtype, float *d_state_in, int batch,
                                     long long seqlen, int heads, int head_dim, int block,
                                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * lt_decode_slots - lt_decode for sequences whose states live in a pool, as a
 * server holding many concurrent sequences keeps them (§04: each sequence
 * carries its own fixed d x d fp32 state per head, whatever its length).
 *
 *   state_pool  [num_slots, heads, head_dim, head_dim] fp32, updated in place.
 *   slot_ids    [batch] int32 on the device: sequence b reads and updates
 *               state_pool[slot_ids[b]]. An id < 0 or >= num_slots marks a
 *               padding row: its o is zero and no state is touched. Valid ids
 *               must be distinct within one call (two rows on one slot race).
 *               Ids are read on the device only.
 *   q, k, v, o, slopes, dtypes: as lt_decode.
 *   Errors: as lt_decode (LT_ERR_SHAPE also for num_slots < 0; LT_ERR_NULL for
 *   a NULL slot_ids with batch > 0, or a NULL pool with num_slots > 0).
 */
LT_API lt_status lt_decode_slots(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                                 const float *slopes, float *state_pool, int num_slots,
                                 const int *slot_ids, void *o, lt_dtype out_dtype, int batch,
                                 int heads, int head_dim, void *stream);

/*
 * lt_prefill_norm_gate, lt_prefill_varlen_norm_gate, lt_decode_norm_gate -
 * the operator above followed, inside the same kernels, by the step the §03
 * data-flow figure places after the sum (the summed output is normalised and
 * gated). The pages give no formula; this library's reading, per (token, head):
 *
 *     y = o / sqrt(mean_d(o^2) + eps) * norm_weight[h] * sigmoid(gate)
 *
 * where o = O_intra + O_inter (never written to memory), the mean runs over
 * the head_dim features, sigmoid(x) = 1 / (1 + e^{-x}), and
 *
 *   gate         o's shape ([batch, seqlen, heads, head_dim], [total_tokens,
 *                heads, head_dim] or [batch, heads, head_dim]) in in_dtype.
 *   norm_weight  [heads, head_dim] fp32.
 *   eps          finite, >= 0; otherwise LT_ERR_VALUE. With eps = 0 a zero
 *                output row gives NaN, as the formula does.
 *   y            takes the place of o (same shape, out_dtype). A row whose
 *                sum o holds a NaN or Inf gives a row of y holding a NaN (the
 *                norm of an infinite row is infinite: its infinite columns
 *                come out NaN and the others 0, or the whole row NaN).
 *
 * Every other argument, the state handling and the workspace are those of
 * lt_prefill / lt_prefill_varlen / lt_decode. The prefill variants take bf16
 * inputs only (LT_ERR_DTYPE for LT_F32); the decode variant takes both. y must
 * not overlap gate or norm_weight, nor may state_out / state (LT_ERR_ALIAS).
 * Errors: those of the base entry point, plus LT_ERR_VALUE.
 */
LT_API lt_status lt_prefill_norm_gate(const void *q, const void *k, const void *v,
                                      lt_dtype in_dtype, const float *slopes, const void *gate,
                                      const float *norm_weight, float eps, void *y,
                                      lt_dtype out_dtype, const float *state_in, float *state_out,
                                      int batch, long long seqlen, int heads, int head_dim,
                                      int block, void *workspace, size_t workspace_bytes,
                                      void *stream);

LT_API lt_status lt_prefill_varlen_norm_gate(const void *q, const void *k, const void *v,
                                             lt_dtype in_dtype, const int *cu_seqlens,
                                             int num_seqs, long long total_tokens,
                                             long long max_seqlen, const float *slopes,
                                             const void *gate, const float *norm_weight, float eps,
                                             void *y, lt_dtype out_dtype, const float *state_in,
                                             float *state_out, int heads, int head_dim, int block,
                                             void *workspace, size_t workspace_bytes,
                                             void *stream);

LT_API lt_status lt_decode_norm_gate(const void *q, const void *k, const void *v,
                                     lt_dtype in_dtype, const float *slopes, float *state,
                                     const void *gate, const float *norm_weight, float eps,
                                     void *y, lt_dtype out_dtype, int batch, int heads,
                                     int head_dim, void *stream);

/*
 * lt_softmax_prefill - causal softmax attention of the hybrid's softmax layers
 * (MiniMax Signal Lab · M1, §02 Architecture: 64 query heads and 8 K/V heads
 * of 128, rotary position embedding on 64 of the 128 dimensions). Query head h
 * reads K/V head h / (q_heads / kv_heads). Token t sits at position pos0 + t:
 *
 *     o_t = sum_{j <= t} softmax_j(scale * rope(q_t) . rope(k_j)) v_j
 *
 * rope rotates feature pairs (m, m + rope_dims/2), m < rope_dims/2, by the
 * angle position * rope_base^(-2m/rope_dims) (rotate-half pairing); features
 * at or past rope_dims are not rotated. Angles are formed in double precision.
 * Scores, softmax and sums run in fp32 (products on bf16 MFMA; the
 * probabilities enter the value product as bf16).
 *
 *   q         [batch, seqlen, q_heads, head_dim] bf16.
 *   k, v      [batch, seqlen, kv_heads, head_dim] bf16.
 *   o         [batch, seqlen, q_heads, head_dim], out_dtype (LT_F32 or LT_BF16).
 *   k_rope    [batch, seqlen, kv_heads, head_dim] bf16 output: rope(k), the
 *             key rows a KV cache holds (lt_softmax_decode reads that form).
 *   head_dim  128; q_heads a multiple of kv_heads (both 0 = nothing to do).
 *   rope_dims a multiple of 32 in [0, head_dim].
 *   rope_base > 1 (LT_ERR_VALUE otherwise); scale > 0 and finite
 *             (LT_ERR_VALUE), usually 1/sqrt(head_dim).
 *   pos0      >= 0, position of token 0.
 *   No output may overlap an input or the other output (LT_ERR_ALIAS).
 *   Errors: LT_ERR_NULL, LT_ERR_SHAPE, LT_ERR_DTYPE, LT_ERR_VALUE,
 *   LT_ERR_ALIAS, LT_ERR_HIP.
 */
LT_API lt_status lt_softmax_prefill(const void *q, const void *k, const void *v, void *o,
                                    lt_dtype out_dtype, void *k_rope, int batch, long long seqlen,
                                    int q_heads, int kv_heads, int head_dim, int rope_dims,
                                    double rope_base, float scale, long long pos0, void *stream);

/*
 * lt_softmax_decode - one decode step of the softmax layer over a KV cache.
 * Sequence b's new token sits at position n = lengths[b]: rope(k_new) (at
 * position n) and v_new are written into row n of the caches, then rope(q)
 * attends over cache rows 0..n of its K/V head:
 *
 *     o[b, h] = sum_{j <= n} softmax_j(scale * rope(q[b, h]) . k_cache[b, j, g]) v_cache[b, j, g]
 *
 * with g = h / (q_heads / kv_heads). The same layer and conventions as
 * lt_softmax_prefill, whose k_rope rows are this cache's key rows.
 *
 *   q             [batch, q_heads, head_dim] bf16.
 *   k_new, v_new  [batch, kv_heads, head_dim] bf16.
 *   k_cache, v_cache  [batch, capacity, kv_heads, head_dim] bf16, updated in
 *                 place at row lengths[b] only.
 *   lengths       [batch] int32 on the device. A value outside [0, capacity)
 *                 marks a padding row: its o is zero and no cache row changes.
 *   o             [batch, q_heads, head_dim], out_dtype.
 *   q_heads / kv_heads at most 32.
 *   workspace     device scratch of lt_softmax_decode_workspace_bytes(...)
 *                 bytes, or NULL / smaller: then each (sequence, K/V head) is
 *                 served by one wave over all its keys (correct, much slower
 *                 at long contexts). The key range is split on `capacity`, so
 *                 a capacity near the longest length keeps every wave busy.
 *   rope_dims, rope_base, scale: as lt_softmax_prefill.
 *   No output (o, caches, workspace) may overlap an input or another output.
 *   Errors: LT_ERR_NULL, LT_ERR_SHAPE (also capacity 0 with batch > 0),
 *   LT_ERR_DTYPE, LT_ERR_VALUE, LT_ERR_ALIAS, LT_ERR_HIP.
 */
LT_API lt_status lt_softmax_decode(const void *q, const void *k_new, const void *v_new,
                                   void *k_cache, void *v_cache, const int *lengths, void *o,
                                   lt_dtype out_dtype, int batch, long long capacity, int q_heads,
                                   int kv_heads, int head_dim, int rope_dims, double rope_base,
                                   float scale, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* Workspace bytes lt_softmax_decode uses for these sizes (0 = none needed or
 * invalid sizes). */
LT_API size_t lt_softmax_decode_workspace_bytes(int batch, long long capacity, int q_heads,
                                                int kv_heads, int head_dim);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_H */
