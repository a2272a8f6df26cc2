/*
 * fa_cpu.h -- C ABI of the exact attention forward pass on the HOST CPU,
 * computed with the same online-softmax recurrence as the GPU library, tiled
 * for the caches and vectorized.
 *
 * "The math of FlashAttention", section "Why the same math matters on a
 * CPU": a CPU has the same shape of problem as the GPU -- a small fast cache
 * in front of slow memory -- and the recurrence keeps the active score block
 * small enough to stay in cache while keys and values stream through once;
 * the update is a max and two scaled sums, which map onto SIMD lanes.
 *
 * This library is a separate CPU implementation of the method, for hosts
 * without the GPU and as a fair CPU comparison point.  It is not a fallback:
 * libfa.so never calls it, and it never calls libfa.so.
 *
 * Memory and ownership: every pointer is a HOST pointer owned by the caller;
 * tensors are dense row-major in the order their shape is listed.  The call
 * is synchronous; it allocates per-thread scratch of about 272 KiB on the
 * heap and frees it before returning.
 *
 * Errors: the same codes as include/fa.h (0 = OK, negative = fa_status);
 * arguments are checked before any work.
 */
#ifndef FA_CPU_H
#define FA_CPU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_fwd_cpu -- attention forward pass on the host; the same operation,
 * argument meaning, layouts and conventions as fa_fwd in include/fa.h
 * (o = 0 and lse = -inf for a row with no visible key; causal is top-left
 * aligned; kv_len_mask is [B, N_k] uint8 shared by all heads), except:
 *
 *   q, k, v, o, lse, kv_len_mask   host pointers
 *   d         any head width from 1 to 256
 *   dtype     FA_DTYPE_F32 (0) or FA_DTYPE_BF16 (1); bf16 inputs are widened
 *             to float exactly and o is rounded to nearest-even
 *   threads   OpenMP threads to use; 0 = the OpenMP default
 *
 * Returns the number of threads used (>= 1), or a negative fa_status:
 * NULL (-1), SHAPE (-2), HEAD_DIM (-3), DTYPE (-4), SCALE (-5), ALIAS (-9).
 *
 * Key tiles of 64 keys and query tiles of 64 rows; within a tile each row
 * takes the pages' step with its exact running maximum ("2.2b: FlashAttention
 * -- Online Softmax", "The Complete Online Softmax Algorithm").  The tile
 * routine exists for AVX-512, AVX2 + FMA and baseline x86-64; the best one
 * the CPU supports is used, and the environment variable FA_CPU_ISA ("avx2"
 * or "base"), read once per process, can lower that choice.
 */
int fa_fwd_cpu(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int H, int N_q, int N_k, int d, float scale, int causal,
               const uint8_t *kv_len_mask, int dtype, int threads);

/*
 * fa_cpu_expf -- the vectorizable exponential the CPU kernel uses, for
 * testing: exp(x) for x <= 0 by Cody-Waite range reduction
 * (x log2 e = k + f, |f| <= 1/2) and a degree-7 Taylor polynomial of
 * e^(f ln 2), scaled by 2^k through the exponent bits.  exp(-inf) = 0,
 * results below 2^-126 are flushed to 0.  Inputs > 0 are clamped to 0 (the
 * recurrence never forms one).
 */
float fa_cpu_expf(float x);

#ifdef __cplusplus
}
#endif

#endif /* FA_CPU_H */
