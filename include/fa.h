/*
 * fa.h -- C ABI of the exact attention forward pass on AMD Instinct MI355X
 * (gfx950), computed with the online-softmax recurrence.
 *
 * The operation (for every batch b, head h and query row i):
 *
 *     s_j   = scale * (q_i . k_j)                      visible keys j only
 *     o_i   = sum_j exp(s_j - m) v_j / l               m = max_j s_j,
 *     lse_i = m + ln l                                 l = sum_j exp(s_j - m)
 *
 * -- "The math of FlashAttention" (aicassindra transformer-math series),
 *    section "What we must compute, and why storage is the problem" (the
 *    definition); "2.2b: FlashAttention -- Online Softmax" (hf-cn0.pages.dev),
 *    section "The Complete Online Softmax Algorithm" (its inputs: scores and
 *    values processed in blocks; its output: the softmax-weighted sum of the
 *    values).
 *
 * The library walks the keys in tiles and keeps, per query row, a running
 * maximum m, a running denominator l and an unnormalised output o~; each tile
 * rescales them by exp(m_old - m_new) and one division o~ / l comes at the
 * end ("The math of FlashAttention", sections "The running state" and "The
 * block-wise update, and the full algorithm").  The result equals the plain
 * definition up to floating-point rounding order ("Proof of exactness").
 *
 * lse is not on the pages; it is m + ln(l) in natural-log units over the
 * scaled scores, the per-row statistic a backward pass or a split-key merge
 * would need.
 *
 * Memory and ownership
 *   - Every pointer is a DEVICE pointer on the current HIP device, owned by
 *     the caller.  The library allocates nothing, copies nothing between host
 *     and device, and never synchronises: work is enqueued on `stream` and the
 *     call returns before it completes.
 *   - All tensors are dense and row-major in the order their shape is listed.
 *   - o and lse must not overlap q, k, v or the mask.
 *
 * Errors
 *   Every entry point returns 0 (FA_OK) or a negative fa_status.  Arguments
 *   are checked before anything is enqueued, so a call that returns an
 *   argument error has no effect.  FA_ERR_LAUNCH means HIP rejected the
 *   launch; fa_strerror() then includes HIP's own message.
 *
 * Thread safety: calls from several host threads are safe; calls that share
 * output buffers race like any two kernels writing the same memory.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = -1,      /* q, k, v, o or lse is NULL                          */
    FA_ERR_SHAPE = -2,     /* B, H, N_q or N_k <= 0, or an index would overflow  */
    FA_ERR_HEAD_DIM = -3,  /* d is not 64 or 128                                 */
    FA_ERR_DTYPE = -4,     /* dtype is not one of fa_dtype                       */
    FA_ERR_SCALE = -5,     /* scale is not finite and > 0                        */
    FA_ERR_TILE = -6,      /* fa_opts.block_n is not 0, 16, 32, 64 or 128        */
    FA_ERR_DEVICE = -7,    /* the current HIP device is not a gfx950 GPU         */
    FA_ERR_LAUNCH = -8,    /* HIP reported an error when the kernel was enqueued */
    FA_ERR_ALIAS = -9,     /* an output overlaps an input or another output      */
    FA_ERR_ARG = -10,      /* another argument is out of range: the traced row,
                              num_splits, n_parts                                */
    FA_ERR_WORKSPACE = -11,/* workspace NULL or smaller than required            */
    FA_ERR_ALIGN = -12,    /* a pointer is not aligned as its entry point needs:
                              16 bytes for q, k, v, o, acc and the trace, 4 bytes
                              for lse, m and l, the element size for the score
                              rows s and p of fa_softmax_rows                    */
    FA_ERR_SCRATCH = -13   /* the partial states of fa_fwd_splitkv_noalloc would
                              not fit the library's device scratch (32 MiB)      */
} fa_status;

typedef enum fa_dtype {
    FA_DTYPE_F32 = 0,      /* q, k, v, o are float (IEEE binary32)               */
    FA_DTYPE_BF16 = 1      /* q, k, v, o are bfloat16 (stored as uint16_t)       */
} fa_dtype;

/*
 * fa_fwd -- attention forward pass.
 *
 *   q            [B, H, N_q, d]   input, dtype `dtype`
 *   k, v         [B, H, N_k, d]   input, dtype `dtype`
 *   o            [B, H, N_q, d]   output, dtype `dtype`; bf16 is rounded to
 *                                 nearest-even from the fp32 result
 *   lse          [B, H, N_q]      output, float32: m + ln(l) per row
 *   B, H         batch and heads, >= 1
 *   N_q, N_k     query and key counts, >= 1, any value (no tile multiple)
 *   d            head width: 64 or 128
 *   scale        score multiplier, finite and > 0; normally 1/sqrt(d) with d
 *                the head width ("The math of FlashAttention", section "What
 *                we must compute"; the tiled-attention interview answer warns
 *                against using the model width instead)
 *   causal       nonzero: key j is visible to query i only if j <= i
 *                (top-left aligned; with N_q == N_k this is the usual mask)
 *   kv_len_mask  NULL, or a device array [B, N_k] of uint8 shared by all
 *                heads: key j of batch b is visible only if the byte is
 *                nonzero.  Per-batch key lengths are prefix masks.  Combined
 *                with `causal` by AND.  Masked keys get score -inf before the
 *                tile maximum, so they contribute exactly zero ("The math of
 *                FlashAttention", "Pitfalls in implementing the recurrence";
 *                tiled-attention interview answer, second paragraph).
 *                Key tiles before the first or after the last visible key of
 *                a batch are skipped outright (no transfer, no work): exact,
 *                since their weights are all zero.
 *   dtype        an fa_dtype.  Accumulation is float32 for both; bf16 inputs
 *                feed bf16 matrix-core products, fp32 inputs fp32 ones.
 *   stream       a hipStream_t (NULL: the default stream).
 *
 * A row with no visible key (all keys masked) gets o = 0 and lse = -inf.
 * The pages require such rows to have a defined convention instead of 0/0
 * (tiled-attention interview answer, second paragraph) without naming one;
 * this is the library's.
 *
 * Non-finite inputs.  Keys that kv_len_mask hides contribute exactly zero
 * whatever their k and v rows hold, NaN and +-inf included (padded cache
 * slots may hold anything): their scores become -inf by selection before
 * the tile maximum, and their v rows never enter a product.  Key j, which
 * the causal mask hides from the rows i < j, is visible to the rows i >= j:
 * a non-finite k or v row of it is a non-finite input of those rows, and
 * through its zero weight inside the matrix product of the key tile on the
 * diagonal it may also turn rows i < j of that tile non-finite.  Every
 * other non-finite value in q, k or v propagates as the definition makes
 * it.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int N_q, int N_k, int d, float scale, int causal,
           const uint8_t *kv_len_mask, int dtype, void *stream);

/*
 * FA_BF16_REF_LAG_LOG2 -- how far (in log2 units of the scaled scores) the
 * bfloat16 kernels let their exponent reference lag a row's running maximum.
 * A tile keeps the current reference when every weight exp2(score * scale *
 * log2 e - reference) stays within 2^FA_BF16_REF_LAG_LOG2; a larger score
 * moves the reference up to it.  Any common reference cancels in o~ / l and in
 * lse ("2.2b: FlashAttention -- Online Softmax", "Why This Algorithm is
 * Exact"), so the results are those of the running maximum; the cost is
 * headroom: o~ and l carry up to 2^FA_BF16_REF_LAG_LOG2 times the magnitudes
 * of the pages' recurrence, whose weights are at most 1 ("The math of
 * FlashAttention", "Proof of numerical stability").  With float32
 * accumulators that leaves about 2^(128 - 24) for |v| times the number of
 * keys -- far beyond any bfloat16 input -- but it is 24 bits less than the
 * pages' bound.  The float32 kernels keep the exact running maximum.
 */
#define FA_BF16_REF_LAG_LOG2 24

/*
 * Test hooks.  A zeroed struct (or a NULL pointer) gives fa_fwd's behaviour.
 *
 *   block_n     keys per tile of the recurrence: 0 (library choice, 64), 16,
 *               32, 64 or 128.  The result must not depend on it ("The math
 *               of FlashAttention", "Proof of exactness": block size never
 *               enters the result; the tiled-attention interview answer asks
 *               to vary the tile size when testing).
 *   reverse_kv  nonzero: visit the key tiles last to first.  The result must
 *               not depend on the order either ("The running state": blocks
 *               may be processed in any order).
 *   trace       NULL, or a device array of ceil(N_k / block_n) * 4 floats
 *               (block_n as used, 64 for 0) that receives the running state
 *               of ONE query row after every key tile the kernel visits --
 *               the per-block (m, l) printout the tiled-attention interview
 *               answer recommends for debugging.  Entry i (the i-th tile
 *               visited) is {tile index, m, l, 0}: l is the row's running
 *               denominator stated against the reference m, given in raw
 *               score units (q . k, before `scale`), so that after the tile
 *               m * scale + ln(l) is the log of the sum of exp(scaled score)
 *               over the keys absorbed so far (-inf and 0 while none is
 *               visible).  For float32, m is the running maximum itself.  For
 *               bfloat16, m lags it: the kernel moves its reference only when
 *               a tile's scores exceed it by more than
 *               FA_BF16_REF_LAG_LOG2 / (scale * log2 e), so running max -
 *               that bound <= m <= running max.  Tiles the
 *               kernel never visits leave their entries untouched: those
 *               above the causal diagonal of the row's query tile
 *               (fa_query_tile_rows rows) and, with kv_len_mask, those
 *               before the tile of the first or after the tile of the last
 *               visible key of the batch within the remaining range (all of
 *               them when it has none).
 *   trace_b, trace_h, trace_row
 *               the traced row: batch, head and query index, each in range
 *               (else FA_ERR_ARG).  Ignored when trace is NULL.
 */
typedef struct fa_opts {
    int block_n;
    int reverse_kv;
    float *trace;
    int trace_b;
    int trace_h;
    int trace_row;
} fa_opts;

int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int N_q, int N_k, int d, float scale, int causal,
              const uint8_t *kv_len_mask, int dtype, void *stream,
              const fa_opts *opts);

/*
 * fa_query_tile_rows -- query rows of one query tile of fa_fwd / fa_fwd_ex
 * for these arguments (block_n as in fa_opts, 0 = library choice; causal
 * nonzero or 0): the rows that share each key/value tile staged in on-chip
 * memory, since query rows are independent ("2.2b", "Scaling to Multiple
 * Queries").  128 or 256; the library takes 256 only for bfloat16, d = 128,
 * 64-key tiles, N_q > 128 and enough query tiles to fill the GPU without one
 * long causal tile deciding the run time.  (A workgroup may take two query
 * tiles of a head in turn; that does not change what a tile visits.)  Under
 * causality a query tile visits the key tiles up to the diagonal of its last
 * row, so a trace has one entry per such tile.  Returns the row
 * count, or FA_ERR_SHAPE (B, H or N_q < 1) / FA_ERR_HEAD_DIM / FA_ERR_DTYPE /
 * FA_ERR_TILE.  Besides its arguments it depends only on the current
 * device's compute-unit count ("enough workgroups"), queried once per device;
 * without a usable device it assumes the MI355X's 256.  It enqueues nothing.
 */
int fa_query_tile_rows(int dtype, int B, int H, int N_q, int d, int block_n, int causal);

/*
 * Split-key forward pass and the merge of partial states.
 *
 * The keys of every query row are cut into num_splits consecutive ranges of
 * whole key tiles (64 keys), processed by separate workgroups; each range
 * yields the row's PARTIAL STATE over its keys, and a second kernel merges
 * them.  A partial state is the pages' running state of a set of keys ("The
 * math of FlashAttention", "The running state: a max, a denominator, and an
 * output"), with its reference m given in raw score units:
 *
 *     m     a reference score (q . k, before `scale`), -inf if no key of the
 *           range is visible; in practice the range's maximum or just below
 *     l     sum_j exp(scale * (s_j - m))           over the range's visible keys
 *     acc   sum_j exp(scale * (s_j - m)) * v_j     (d floats)
 *
 * Merging rewrites every state to the common reference M = max_i m_i by the
 * rescaling identity (l_i and acc_i times exp(scale * (m_i - M)), "The
 * rescaling identity, derived") and adds them: the key sets are disjoint and
 * order does not matter ("Proof of exactness").  Then o = acc / l and
 * lse = M * scale + ln l, with o = 0 and lse = -inf when every m_i is -inf.
 * This is the step that serves few query rows over many keys (decoding), few
 * heads, and -- across devices -- keys sharded over GPUs.
 *
 * Partial-state arrays are part-major: for part i and row r (of `rows`),
 *     m[i * rows + r], l[i * rows + r], acc[(i * rows + r) * d + j].
 */

/*
 * fa_splitkv_workspace_bytes -- device bytes fa_fwd_splitkv needs for these
 * sizes: the partial states of num_splits parts of B*H*N_q rows, laid out as
 * m (float[num_splits][rows]), l (same), then acc (float[num_splits][rows][d])
 * starting at the next multiple of 256 bytes.  Returns 0 when an argument is
 * out of range (see fa_fwd_splitkv).
 */
size_t fa_splitkv_workspace_bytes(int B, int H, int N_q, int d, int num_splits);

/*
 * fa_splitkv_splits -- the library's choice of num_splits for these sizes on
 * the current device: enough workgroups to give every compute unit several,
 * and at least 4 key tiles per range; 1 when the plain pass already fills the
 * GPU.  Returns a value in [1, 256], or a negative fa_status.
 */
int fa_splitkv_splits(int B, int H, int N_q, int N_k, int d, int causal);

/*
 * fa_fwd_splitkv -- the same result as fa_fwd (all arguments as there,
 * key tiles of 64), computed as num_splits partial states per row that are
 * then merged.
 *
 *   num_splits       1 .. 256 (else FA_ERR_ARG).  Ranges may be empty when
 *                    num_splits exceeds a row's tile count; they contribute
 *                    nothing.
 *   workspace        device memory of at least workspace_bytes =
 *                    fa_splitkv_workspace_bytes(B, H, N_q, d, num_splits)
 *                    bytes, 16-byte aligned, owned by the caller, overlapping
 *                    no other argument (else FA_ERR_WORKSPACE / FA_ERR_ALIAS).
 *                    Its contents on entry do not matter; on return (once the
 *                    stream reaches that point) it holds the partial states in
 *                    the layout above.  Two calls in flight must not share it.
 *
 * Two kernels are enqueued on `stream`; nothing is allocated or synchronised.
 */
int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int N_q, int N_k, int d, float scale, int causal,
                   const uint8_t *kv_len_mask, int dtype, int num_splits,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv for callers that cannot allocate
 * device memory or pass a workspace: code recorded under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * checks and result as fa_fwd_splitkv, without workspace and
 * workspace_bytes: the partial states go to a scratch array owned by the
 * library instead.
 *
 *   scratch      32 MiB of device memory per GPU, a static array of the
 *                library that each GPU it runs on holds until the process
 *                ends.  A call needs fa_splitkv_workspace_bytes(B, H, N_q, d,
 *                num_splits) bytes of it; more gives FA_ERR_SCRATCH before
 *                anything is enqueued.  The first call on a device looks the
 *                array's address up (no allocation); later calls reuse it.
 *   allocation   none: no hipMalloc, hipFree or allocating library routine
 *                on any call.
 *   sharing      every call on one GPU uses the same array, which keeps the
 *                last call's partial states.  Nothing in it needs to start at
 *                zero (every part of every row is written before it is read),
 *                but two calls that overlap in time on one GPU -- on
 *                different streams, or from different host threads without
 *                ordering -- race on it and give undefined results.
 */
int fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int N_q, int N_k, int d, float scale, int causal,
                           const uint8_t *kv_len_mask, int dtype, int num_splits,
                           void *stream);

/*
 * fa_merge_states -- merge n_parts partial states per row (layout above) into
 * o and lse.
 *
 *   m, l         device float[n_parts * rows]
 *   acc          device float[n_parts * rows * d]
 *   n_parts      >= 1 (else FA_ERR_ARG); rows >= 1 (else FA_ERR_SHAPE)
 *   d            64 or 128
 *   scale        the score multiplier the states were formed with (> 0)
 *   o            device [rows, d] of `dtype` (bf16 rounded to nearest-even)
 *   lse          device float[rows]
 *
 * A part whose m is -inf contributes nothing; its l and acc are not read.
 * Otherwise l must be >= 0 and finite, as a real partial state's is.
 */
int fa_merge_states(const float *m, const float *l, const float *acc, int n_parts,
                    int64_t rows, int d, float scale, void *o, float *lse, int dtype,
                    void *stream);

/*
 * fa_softmax_rows -- softmax along every row of a score matrix, by the online
 * recurrence with the values removed ("2.2b: FlashAttention -- Online
 * Softmax", sections "The Challenge: Computing m and l in Blocks" through
 * "When Rescaling Actually Happens"): one pass over the row carries the
 * running maximum m and the running denominator l, rescaling l by
 * exp(m_old - m_new) whenever m grows; a second pass writes
 * p_j = exp(s_j - m) / l.  That reads the row twice where the safe softmax
 * ("The math of FlashAttention", "Safe softmax: the max-subtraction we cannot
 * give up") reads it three times.
 *
 *   s        device [rows, n] scores, `dtype`; -inf marks a masked entry
 *            (weight exactly 0).  NaN and +inf inputs are out of scope.
 *   p        device [rows, n] output, `dtype` (bf16 rounded to nearest-even).
 *            p == s (in place) is allowed; any other overlap is FA_ERR_ALIAS.
 *   m, l     NULL, or device float[rows]: the row maximum and
 *            l = sum_j exp(s_j - m)
 *   rows, n  >= 1 (else FA_ERR_SHAPE)
 *   dtype    FA_DTYPE_F32 or FA_DTYPE_BF16; arithmetic is float32
 *
 * A row whose entries are all -inf gets p = 0, m = -inf and l = 0.  One
 * workgroup handles one row; rows that are not 16-byte aligned take a slower
 * element-wise path.
 */
int fa_softmax_rows(const void *s, void *p, float *m, float *l, int64_t rows, int64_t n,
                    int dtype, void *stream);

/*
 * fa_strerror -- a NUL-terminated description of a status code, never NULL.
 * For FA_ERR_LAUNCH and FA_ERR_DEVICE it appends the last HIP error seen by
 * the calling thread; that text lives in a thread-local buffer that stays
 * valid until the thread's next fa_strerror call.  The caller frees nothing.
 */
const char *fa_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
