/*
 * rattn.h -- C ABI of the MI355X (gfx950) exact ring attention: the forward
 * and its backward.
 *
 * The operation is exact attention, softmax(scale * Q K^T) V (guijiagi.com
 * "ring-attention-explained", memory-wall section, first formula), computed
 * blockwise with an online softmax: every query tile keeps a running row
 * maximum m, a running sum l and an unnormalised accumulator O while it
 * streams over key/value tiles, and divides by l once at the end (yz520gzy
 * FlashAttention chapter, FlashAttention-2 deferred normalisation).  Results
 * of separate key sets (ring steps) are combined with a log-sum-exp
 * correction (Twinkle "Sequence parallel and Ring Attention", forward-pass
 * section, update_out_and_lse).
 *
 * Conventions shared by every entry point
 *   - Layout (batch, sequence, heads, head_dim), contiguous, as in the
 *     flash-attn usage example of the yz520gzy chapter:
 *       q [B, Nq, Hq, d]     k, v [B, Nk, Hkv, d]     out [B, Nq, Hq, d]
 *       lse [B, Nq, Hq] float32, natural logarithm of sum_j exp(scale*s_j)
 *   - GQA: query head h reads key/value head h / (Hq / Hkv).
 *   - Causal: a key is visible to a query iff its global position is not
 *     after the query's (youngju.dev "Ring Attention" analysis, causal step).
 *   - scale <= 0 (or NaN) selects 1/sqrt(d).
 *   - d must be one of 16, 32, 64, 128.
 *   - Every sequence length (Nq, Nk, N, and each varlen sequence) is below
 *     2^31 rows; larger sizes return RATTN_EUNSUPPORTED.
 *   - Every pointer argument that names a tensor is a DEVICE pointer owned by
 *     the caller; it may be NULL only when that tensor has no rows.  The library allocates no memory, keeps no global state and
 *     never synchronises the host: work is enqueued on `stream` (a
 *     hipStream_t; NULL = the default stream) and completes asynchronously.
 *     Inputs must stay valid until the stream has passed the call.
 *   - Host-side argument checks run before anything is enqueued; a failed
 *     check returns a negative status and enqueues nothing.  RATTN_EHIP
 *     reports a HIP launch error (hipGetLastError after the launch).
 *   - Rows with no visible key get out = 0 and lse = -inf.
 *   - out/lse must not overlap q, k or v.
 */
#ifndef RATTN_H
#define RATTN_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define RATTN_API __attribute__((visibility("default")))
#else
#define RATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RATTN_OK = 0,
  RATTN_EINVAL = -1,       /* invalid argument (null pointer, bad size, ...) */
  RATTN_EUNSUPPORTED = -2, /* valid but not implemented (d, dtype, W > 32) */
  RATTN_EHIP = -3,         /* HIP reported an error when enqueueing */
  RATTN_ESCRATCH = -4      /* larger than the library's fixed scratch (rattn_fwd_split_noalloc) */
} rattn_status;

typedef enum { RATTN_F32 = 0, RATTN_F16 = 1, RATTN_BF16 = 2 } rattn_dtype;

/*
 * Whole ring schedule in one call.
 *
 * k, v hold all N key/value rows in natural order (row index == position).
 * n_ring_steps = W >= 1 simulated devices (at most 32).  zigzag = 0: device r
 * holds contiguous block r of N/W rows (ultralytics.com "Ring Attention", how
 * it works); zigzag = 1: device r holds chunks r and 2W-1-r of the 2W chunks
 * of N/(2W) rows (Twinkle page, ZigZag section).  Each simulated device visits
 * the key/value blocks in ring order, block (r - s) mod W at step s.
 *   rank = -1 : q holds all N rows in natural order (Nq == N) and the
 *               schedules of all W devices run in one launch.
 *   rank = r  : q holds device r's shard (Nq == N/W): block r, or for ZigZag
 *               [chunk r ; chunk 2W-1-r].
 * N must be a multiple of W (of 2W with zigzag).  out has q's dtype.
 * Without causal masking the result does not depend on W, zigzag or rank.
 *
 * Kernel choice (16-bit inputs, d = 32, 64, 128): the work items are query
 * tiles of 256 rows.  When there are few of them (at most a quarter of the
 * compute units, or half of them for causal calls, twice that at d = 32;
 * beyond a quarter only if the longest item sees at least 24 key tiles of
 * 64), the call runs instead on a kernel that gives
 * each workgroup 32 query rows and divides their key tiles among its 8
 * waves, whose partial results are merged in LDS by the log-sum-exp rule
 * (for a single head of 4096 queries: 128 workgroups instead of 16).  It
 * allocates nothing either.  The environment variable RATTN_FWD_SHORT,
 * read at every call, overrides the choice: "0" never, "1" always (for
 * every call this kernel can serve).  The same choice applies to
 * rattn_fwd_queued and the ring-step calls; results agree within the stated
 * tolerances, not bit for bit, between the two kernels.
 *
 * Debugging: with RATTN_SERIALIZE=1 (read at every call) the 256-row kernel
 * runs one key tile at a time, each tile requested and waited for right
 * before it is used and a workgroup barrier around every phase, and the
 * 32-row kernel is not chosen.  It computes the same arithmetic in the same
 * order, so its results equal those of the pipelined schedule bit for bit;
 * a difference points at an LDS buffering hazard.  It is slow: not for use
 * beyond debugging.  rattn_fwd_queued then runs one workgroup per item.
 */
RATTN_API int rattn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
              int B, int Hq, int Hkv, int64_t Nq, int64_t N, int d, int dtype,
              float scale, int causal, int n_ring_steps, int zigzag, int rank,
              void* stream);

/*
 * rattn_fwd with the work items (query tiles of every batch and head, as in
 * the blockwise loop of the yz520gzy FlashAttention chapter) handed out from
 * queues instead of one workgroup each: when the call (16-bit, d = 128) has
 * more than twice as many query tiles as the GPU runs at once, a grid of that
 * many workgroups
 * takes them from eight counters (one per XCD; a workgroup whose XCD's queue
 * is empty takes the others' remaining items), so that parts of the chip
 * that run at a higher clock take more of the work instead of waiting at the
 * end.  Smaller calls run exactly as rattn_fwd.  Results are identical to
 * rattn_fwd's (every tile is computed by the same code).
 *   queue_ws: DEVICE memory of at least RATTN_QUEUE_WS_BYTES bytes, 4-byte
 *   aligned, owned by the caller; its contents on entry do not matter (the
 *   call zeroes the counters on `stream` before the launch that uses them).
 *   Calls that share a workspace must not overlap in time (consecutive calls
 *   on one stream never do).  Other arguments, checks and status codes as
 *   rattn_fwd; a missing or short workspace returns RATTN_EINVAL.
 */
#define RATTN_QUEUE_WS_BYTES 64
RATTN_API int rattn_fwd_queued(const void* q, const void* k, const void* v, void* out,
                               float* lse, int B, int Hq, int Hkv, int64_t Nq, int64_t N, int d,
                               int dtype, float scale, int causal, int n_ring_steps, int zigzag,
                               int rank, void* queue_ws, int64_t queue_ws_bytes, void* stream);

/*
 * One ring step: the attention of a set of query rows over one received
 * key/value shard (the per-step block call of the Twinkle forward pass).
 *
 * The step reads query rows [q_off, q_off + Nq) of q [B, q_rows, Hq, d] and
 * key/value rows [k_off, k_off + Nk) of k_blk, v_blk [B, k_rows, Hkv, d], so
 * a part of a shard (the back query half, the front key chunk) needs no copy.
 * Query row q_off + i sits at position q_seg_start[0] + i for
 * i < q_seg_len[0] and at q_seg_start[1] + (i - q_seg_len[0]) after; likewise
 * for the Nk key/value rows with k_seg_*.  q_seg_len[0] + q_seg_len[1] == Nq
 * and k_seg_len[0] + k_seg_len[1] == Nk (a length may be 0); requires
 * q_off + Nq <= q_rows and k_off + Nk <= k_rows.  The four segment arrays are
 * HOST pointers to two int64 each.
 * Writes the normalised float32 partial out_part [B, Nq, Hq, d] and
 * lse_part [B, Nq, Hq] (row i for query row q_off + i); rows that see no key
 * get 0 and -inf, which the merge treats as an empty partial.
 */
RATTN_API int rattn_fwd_step(const void* q, const void* k_blk, const void* v_blk,
                   float* out_part, float* lse_part, int B, int Hq, int Hkv,
                   int64_t q_rows, int64_t q_off, int64_t Nq, int64_t k_rows, int64_t k_off,
                   int64_t Nk, int d, int dtype, float scale, int causal,
                   const int64_t* q_seg_start, const int64_t* q_seg_len,
                   const int64_t* k_seg_start, const int64_t* k_seg_len, void* stream);

/*
 * One ring step merged into the running result: rattn_fwd_step's partial for
 * query rows q_off + i, i in [0, Nq), of q, merged by the log-sum-exp
 * correction (Twinkle page, update_out_and_lse; same function as
 * rattn_merge) into
 *   (out, lse)[b, row_off + i, h],  out [B, Nq_out, Hq, d] float32,
 *   lse [B, Nq_out, Hq] float32,
 * in the kernel's epilogue (one launch instead of a step and a merge).
 * Requires row_off + Nq <= Nq_out; out/lse must not overlap q, k, v.  A row
 * that sees no key leaves (out, lse) unchanged.  Other arguments and errors
 * as rattn_fwd_step.
 */
RATTN_API int rattn_fwd_step_merge(const void* q, const void* k_blk, const void* v_blk,
                                   float* out, float* lse, int B, int Hq, int Hkv,
                                   int64_t q_rows, int64_t q_off, int64_t Nq, int64_t k_rows,
                                   int64_t k_off, int64_t Nk, int d, int dtype, float scale,
                                   int causal, const int64_t* q_seg_start,
                                   const int64_t* q_seg_len, const int64_t* k_seg_start,
                                   const int64_t* k_seg_len, int64_t Nq_out, int64_t row_off,
                                   void* stream);

/*
 * In-place log-sum-exp merge (Twinkle page, update_out_and_lse; computed as
 * lse' = logaddexp(lse, blk_lse), out' = e^(lse-lse') out + e^(blk_lse-lse') blk_out):
 *   (out, lse)[b, row_off + i, h] <- (out, lse)[b, row_off + i, h]
 *                                    (+) (blk_out, blk_lse)[b, i, h]
 * for i in [0, Nb).  out [B, Nq, H, d] float32, lse [B, Nq, H] float32,
 * blk_out [B, Nb, H, d] float32, blk_lse [B, Nb, H] float32.
 * A side with lse = -inf is empty and leaves the other unchanged; two empty
 * sides give out = 0, lse = -inf.  Requires row_off + Nb <= Nq; the block
 * buffers must not overlap out/lse.  All tensor pointers 16-byte aligned.
 */
RATTN_API int rattn_merge(float* out, float* lse, const float* blk_out, const float* blk_lse,
                int B, int H, int64_t Nq, int64_t Nb, int64_t row_off, int d,
                void* stream);

/*
 * Variable-length (packed or padded) batch: n_seq independent sequences in
 * one launch (the varlen attention of the yz520gzy flash-attn example and of
 * Twinkle's packed batches).  Sequence i owns query rows
 * [q_start[i], q_start[i] + q_len[i]) of q [Nq, Hq, d] and key/value rows
 * [k_start[i], k_start[i] + k_len[i]) of k, v [Nk, Hkv, d]; it attends only
 * to its own keys.  Packed batches pass prefix sums (start = cu[i],
 * len = cu[i+1] - cu[i]); padded ones pass each row block's start and the
 * true length, so pad rows are neither read as keys nor written.
 * Causal: key j of a sequence sits at position j and query i at
 * k_len - q_len + i (the last query aligned with the last key; the usual
 * rule when q_len == k_len).  q_start, q_len, k_start, k_len are DEVICE
 * arrays of n_seq int32; max_len_q >= every q_len (rows past it are not
 * computed).  Ranges are clamped to [0, Nq) and [0, Nk) in the kernels, so a
 * bad range yields wrong rows, never an access outside the tensors.  out
 * (q's dtype, [Nq, Hq, d]) and lse ([Nq, Hq]) are written only on rows that
 * belong to a sequence.  Other arguments and errors as rattn_fwd.
 */
RATTN_API int rattn_fwd_varlen(const void* q, const void* k, const void* v, void* out,
                               float* lse, const int32_t* q_start, const int32_t* q_len,
                               const int32_t* k_start, const int32_t* k_len, int n_seq,
                               int64_t max_len_q, int64_t Nq, int64_t Nk, int Hq, int Hkv, int d,
                               int dtype, float scale, int causal, void* stream);

/*
 * rattn_fwd with split-KV: the same schedule and result, with the live
 * key/value tiles of every query tile divided into n_splits contiguous
 * ranges, each processed by its own workgroup, and the n_splits partial
 * results combined by the n-way form of the log-sum-exp merge (Twinkle page,
 * update_out_and_lse, applied n_splits - 1 times).  For shapes whose query
 * tiles alone cannot fill the GPU (few heads, short sequences).
 * ws: caller-owned DEVICE scratch of ws_floats float32 elements, at least
 * n_splits * B * Nq * Hq * (d + 1), 16-byte aligned, not overlapping the
 * other tensors; the call overwrites it.  1 <= n_splits <= 64; n_splits = 1
 * is rattn_fwd (ws unused).  Other arguments and errors as rattn_fwd;
 * RATTN_EINVAL also when ws is null or too small.
 */
RATTN_API int rattn_fwd_split(const void* q, const void* k, const void* v, void* out,
                              float* lse, int B, int Hq, int Hkv, int64_t Nq, int64_t N, int d,
                              int dtype, float scale, int causal, int n_ring_steps, int zigzag,
                              int rank, int n_splits, float* ws, int64_t ws_floats,
                              void* stream);

/*
 * rattn_fwd_split for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and result, with the split partials in a scratch
 * array the library owns instead of caller workspace.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 *   - The scratch is a fixed array of RATTN_NOALLOC_SCRATCH_FLOATS float32
 *     (32 MiB) per GPU, resolved on the first call on that GPU and held until
 *     the process ends.  A call needs n_splits * B * Nq * Hq * (d + 1) floats
 *     when n_splits > 1; larger calls return RATTN_ESCRATCH and enqueue
 *     nothing.  n_splits = 1 is rattn_fwd and uses no scratch.
 *   - Every call on one GPU shares that GPU's array and leaves the last
 *     call's partials in it (nothing in it needs to start at zero: each call
 *     writes every entry it reads).  Calls that may overlap on one GPU (on
 *     different streams without ordering between them) race; order them on
 *     one stream.
 *   - The GPU is the current device of the calling thread, which must be
 *     the device of `stream`.
 * Other arguments and errors as rattn_fwd_split (no ws, ws_floats).
 */
#define RATTN_NOALLOC_SCRATCH_FLOATS (8LL << 20)
RATTN_API int rattn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* out,
                                      float* lse, int B, int Hq, int Hkv, int64_t Nq, int64_t N,
                                      int d, int dtype, float scale, int causal,
                                      int n_ring_steps, int zigzag, int rank, int n_splits,
                                      void* stream);

/*
 * A split count for rattn_fwd_split: 1 when the query tiles alone give at
 * least one workgroup per two compute units (n_cu compute units), else
 * enough splits to reach that, keeping at least eight 64-key tiles per split
 * and at most 64 splits.  Returns 1 for arguments rattn_fwd would reject.
 */
RATTN_API int rattn_split_hint(int B, int Hq, int64_t Nq, int64_t N, int d, int dtype,
                               int n_ring_steps, int zigzag, int rank, int n_cu);

/*
 * ---- Backward ----------------------------------------------------------
 * Gradients of sum(dout * out) with respect to q, k and v, recomputing the
 * probabilities from the forward's lse (youngju.dev "Ring Attention"
 * analysis, ring_attention_backward):
 *   P_ij = exp(scale q_i.k_j - lse_i)  (0 when key j is not visible to row i)
 *   D_i  = rowsum(dout_i * out_i)
 *   dv_j = sum_i P_ij dout_i
 *   dS_ij = P_ij (dout_i . v_j - D_i)
 *   dq_i = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i
 * With GQA, dk and dv of a key/value head sum over the query heads of its
 * group.  A row whose lse is -inf (it saw no key) contributes nothing.
 */

/*
 * D = rowsum(dout * out) for `rows` rows of d elements: out, dout of
 * dtype, contiguous [rows, d] (e.g. [B, Nq, Hq, d] with rows = B*Nq*Hq);
 * delta float32 [rows].  Pointers 16-byte aligned (delta 4-byte).
 */
RATTN_API int rattn_bwd_delta(const void* out, const void* dout, float* delta, int64_t rows,
                              int d, int dtype, void* stream);

/*
 * Backward of rattn_fwd, same layout arguments (B, Hq, Hkv, Nq, N, d, dtype,
 * scale, causal, n_ring_steps, zigzag, rank).
 *   q, out, dout [B, Nq, Hq, d] dtype; lse [B, Nq, Hq] float32 from rattn_fwd;
 *   k, v [B, N, Hkv, d] dtype.
 *   dq [B, Nq, Hq, d], dk, dv [B, N, Hkv, d] in dtype: written (not added to).
 *   delta_ws: caller scratch of B*Nq*Hq float32 (receives D).
 * With rank >= 0 the queries are device r's shard, and dk/dv are that
 * device's contribution to every key/value row (what the ring sends back to
 * each block's owner); with rank = -1 they are the full gradients.  The
 * result does not depend on the ring order.  All tensor pointers 16-byte
 * aligned; outputs must not overlap the inputs.
 */
RATTN_API int rattn_bwd(const void* q, const void* k, const void* v, const void* out,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        float* delta_ws, int B, int Hq, int Hkv, int64_t Nq, int64_t N, int d,
                        int dtype, float scale, int causal, int n_ring_steps, int zigzag,
                        int rank, void* stream);

/*
 * Backward of rattn_fwd_varlen: sequence i (query rows [q_start[i],
 * +q_len[i]) of q, out, dout [Nq, Hq, d]; key rows [k_start[i], +k_len[i])
 * of k, v [Nk, Hkv, d]; positions as rattn_fwd_varlen) gets its gradients
 * from its own pairs only.  dq [Nq, Hq, d], dk, dv [Nk, Hkv, d] in the input
 * type are written on the rows of the sequences (other rows untouched);
 * delta_ws: caller scratch of Nq*Hq float32.  q_start .. k_len are DEVICE
 * arrays of n_seq int32 (clamped as in rattn_fwd_varlen); max_len_q,
 * max_len_k bound the lengths.  Other arguments and errors as rattn_bwd.
 */
RATTN_API int rattn_bwd_varlen(const void* q, const void* k, const void* v, const void* out,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               float* delta_ws, const int32_t* q_start, const int32_t* q_len,
                               const int32_t* k_start, const int32_t* k_len, int n_seq,
                               int64_t max_len_q, int64_t max_len_k, int64_t Nq, int64_t Nk,
                               int Hq, int Hkv, int d, int dtype, float scale, int causal,
                               void* stream);

/*
 * One ring step of the backward: the pairs between query rows
 * [q_off, q_off + Nq) of a [B, q_rows, Hq, .] row space (q, dout dtype
 * [.., d]; lse, delta float32 [B, q_rows, Hq]; dq_acc float32 [.., d]) and
 * key/value rows [k_off, k_off + Nk) of a [B, k_rows, Hkv, d] row space
 * (k, v dtype; dk_acc, dv_acc float32).  The step's contributions are ADDED
 * to dq_acc, dk_acc and dv_acc (float32 accumulators the caller zeroes
 * once).  Positions as rattn_fwd_step: query row q_off + i sits at
 * q_seg_start[0] + i for i < q_seg_len[0], else at
 * q_seg_start[1] + (i - q_seg_len[0]); keys likewise (HOST arrays of two
 * int64, lengths summing to Nq and Nk).  lse and delta are those of the
 * final forward result (rattn_fwd or the merged ring steps) and
 * rattn_bwd_delta.  Accumulators must not overlap the inputs; calls that
 * add to the same accumulator rows must be ordered on one stream.
 */
RATTN_API int rattn_bwd_step(const void* q, const void* k, const void* v, const void* dout,
                             const float* lse, const float* delta, float* dq_acc, float* dk_acc,
                             float* dv_acc, int B, int Hq, int Hkv, int64_t q_rows,
                             int64_t q_off, int64_t Nq, int64_t k_rows, int64_t k_off,
                             int64_t Nk, int d, int dtype, float scale, int causal,
                             const int64_t* q_seg_start, const int64_t* q_seg_len,
                             const int64_t* k_seg_start, const int64_t* k_seg_len, void* stream);

/* Static description of a status code; never NULL. */
RATTN_API const char* rattn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* RATTN_H */
