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
    FA_ERR_ALIAS = -9      /* o or lse overlaps an input buffer                  */
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
 *   dtype        an fa_dtype.  Accumulation is float32 for both; bf16 inputs
 *                feed bf16 matrix-core products, fp32 inputs fp32 ones.
 *   stream       a hipStream_t (NULL: the default stream).
 *
 * A row with no visible key (all keys masked) gets o = 0 and lse = -inf.
 * The pages require such rows to have a defined convention instead of 0/0
 * (tiled-attention interview answer, second paragraph) without naming one;
 * this is the library's.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int N_q, int N_k, int d, float scale, int causal,
           const uint8_t *kv_len_mask, int dtype, void *stream);

/*
 * Test hooks.  A zeroed struct (or a NULL pointer) gives fa_fwd's behaviour.
 *
 *   block_n     keys per tile of the recurrence: 0 (library choice), 16, 32,
 *               64 or 128.  The result must not depend on it ("The math of
 *               FlashAttention", "Proof of exactness": block size never enters
 *               the result; the tiled-attention interview answer asks to vary
 *               the tile size when testing).
 *   reverse_kv  nonzero: visit the key tiles last to first.  The result must
 *               not depend on the order either ("The running state": blocks
 *               may be processed in any order).
 */
typedef struct fa_opts {
    int block_n;
    int reverse_kv;
} fa_opts;

int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int N_q, int N_k, int d, float scale, int causal,
              const uint8_t *kv_len_mask, int dtype, void *stream,
              const fa_opts *opts);

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
