// fa_softmax.hip -- softmax along the rows of a score matrix with the online
// recurrence, on gfx950.
//
// Per row, pass 1 carries the running maximum m and the running denominator
// l over the row's entries: when a block of entries raises the maximum, the
// sum so far is rescaled by exp(m_old - m_new) <= 1 and the block's terms are
// added against m_new ("2.2b: FlashAttention -- Online Softmax", sections "The
// Solution: Rescaling When the Maximum Changes" and "When Rescaling Actually
// Happens").  Pass 2 writes p_j = exp(s_j - m) / l.  Two reads of the row
// instead of the safe softmax's three ("The math of FlashAttention", "Safe
// softmax: the max-subtraction we cannot give up").
//
// One workgroup of 256 threads per row.  In pass 1 every thread runs the
// recurrence over its own entries -- one 16-byte vector (4 fp32 or 8 bf16) is
// one block -- and the 256 partial states (m, l) are then combined with the
// same identity: rewrite both to the larger maximum and add.  The row is
// HBM-bound: per entry pass 1 costs about five vector instructions and pass 2
// four, far below what the SIMDs can issue while the row streams in; the
// second read of a row usually hits L2.
//
// exp(x) is computed as exp2(x * log2 e) with x = s - m formed first: the
// difference is exact or nearly so, and an exponent error of one rounding of
// x * log2 e stays below 1e-6 relative for the |x| that give weights above
// the fp32 bar.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

struct SoftmaxParams {
    const void *s;
    void *p;
    float *m;
    float *l;
    int64_t rows;
    int64_t n;
};

namespace {

constexpr float kNegInfS = -__builtin_inff();
constexpr float kLog2e = 1.44269504088896341f;

typedef float sf32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t su32x4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ float ex(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Combine state (m2, l2) into (m, l): both rewritten to the larger maximum.
__device__ __forceinline__ void combine(float &m, float &l, float m2, float l2)
{
    const float mn = fmaxf(m, m2);
    if (mn == kNegInfS) return;             // both empty
    l = (m == kNegInfS ? 0.0f : l * ex(m - mn)) + (m2 == kNegInfS ? 0.0f : l2 * ex(m2 - mn));
    m = mn;
}

// One block of E entries absorbed into the running state.
template <int E>
__device__ __forceinline__ void absorb(float &m, float &l, const float (&x)[E])
{
    float bm = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) bm = fmaxf(bm, x[e]);
    if (bm > m) {
        l = (m == kNegInfS) ? 0.0f : l * ex(m - bm);
        m = bm;
    }
    if (m == kNegInfS) return;              // every entry so far is masked
#pragma unroll
    for (int e = 0; e < E; ++e) l += ex(x[e] - m);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16)
{
    return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// 16-byte vector i of a row as E floats.
template <bool BF16>
__device__ __forceinline__ void load_vec(const void *row, int64_t i, float (&x)[BF16 ? 8 : 4])
{
    if (BF16) {
        const su32x4 u = reinterpret_cast<const su32x4 *>(row)[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_to_f32(u[e] & 0xffffu);
            x[2 * e + 1] = bf16_to_f32(u[e] >> 16);
        }
    } else {
        const sf32x4 v = reinterpret_cast<const sf32x4 *>(row)[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = v[e];
    }
}

template <bool BF16>
__device__ __forceinline__ void store_vec(void *row, int64_t i, const float (&y)[BF16 ? 8 : 4])
{
    if (BF16) {
        su32x4 u;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            u[e] = f32_to_bf16_bits(y[2 * e]) | (f32_to_bf16_bits(y[2 * e + 1]) << 16);
        reinterpret_cast<su32x4 *>(row)[i] = u;
    } else {
        const sf32x4 v = {y[0], y[1], y[2], y[3]};
        reinterpret_cast<sf32x4 *>(row)[i] = v;
    }
}

template <bool BF16>
__device__ __forceinline__ float load_one(const void *row, int64_t j)
{
    if (BF16) return bf16_to_f32(static_cast<const uint16_t *>(row)[j]);
    return static_cast<const float *>(row)[j];
}

template <bool BF16>
__device__ __forceinline__ void store_one(void *row, int64_t j, float y)
{
    if (BF16)
        static_cast<uint16_t *>(row)[j] = (uint16_t)f32_to_bf16_bits(y);
    else
        static_cast<float *>(row)[j] = y;
}

}  // namespace

// VEC: the rows are 16-byte aligned and a whole number of vectors long.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void fa_softmax_rows_kernel(const SoftmaxParams p)
{
    constexpr int E = BF16 ? 8 : 4;
    constexpr int ESZ = BF16 ? 2 : 4;
    __shared__ float red_m[4], red_l[4];
    const int tid = threadIdx.x;
    const int w = tid >> 6;

    for (int64_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
        const void *src = static_cast<const char *>(p.s) + row * p.n * ESZ;
        void *dst = static_cast<char *>(p.p) + row * p.n * ESZ;

        // pass 1: this thread's running state over its blocks
        float m = kNegInfS, l = 0.0f;
        if (VEC) {
            const int64_t nv = p.n / E;
            for (int64_t i = tid; i < nv; i += 256) {
                float x[E];
                load_vec<BF16>(src, i, x);
                absorb<E>(m, l, x);
            }
        } else {
            for (int64_t j = tid; j < p.n; j += 256) {
                const float x[1] = {load_one<BF16>(src, j)};
                absorb<1>(m, l, x);
            }
        }

        // the 256 states combined: within the wave, then across the 4 waves
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
            combine(m, l, __shfl_xor(m, off), __shfl_xor(l, off));
        if ((tid & 63) == 0) {
            red_m[w] = m;
            red_l[w] = l;
        }
        __syncthreads();
        m = red_m[0];
        l = red_l[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) combine(m, l, red_m[i], red_l[i]);
        __syncthreads();     // red_* is reused by the next row

        // pass 2: p_j = exp(s_j - m) / l; all -inf rows give 0
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        const float base = m == kNegInfS ? 0.0f : m;
        if (VEC) {
            const int64_t nv = p.n / E;
            for (int64_t i = tid; i < nv; i += 256) {
                float x[E];
                load_vec<BF16>(src, i, x);
#pragma unroll
                for (int e = 0; e < E; ++e) x[e] = ex(x[e] - base) * inv;
                store_vec<BF16>(dst, i, x);
            }
        } else {
            for (int64_t j = tid; j < p.n; j += 256)
                store_one<BF16>(dst, j, ex(load_one<BF16>(src, j) - base) * inv);
        }
        if (tid == 0) {
            if (p.m) p.m[row] = m;
            if (p.l) p.l[row] = l;
        }
    }
}

template <bool BF16, bool VEC>
static hipError_t launch_softmax_v(const SoftmaxParams &p, hipStream_t stream)
{
    const int grid = (int)(p.rows < (1 << 20) ? p.rows : (1 << 20));
    void (*fn)(SoftmaxParams) = fa_softmax_rows_kernel<BF16, VEC>;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_softmax_rows(const void *s, void *p, float *m, float *l, int64_t rows,
                               int64_t n, int dtype, hipStream_t stream)
{
    SoftmaxParams sp;
    sp.s = s;
    sp.p = p;
    sp.m = m;
    sp.l = l;
    sp.rows = rows;
    sp.n = n;
    const int esz = dtype == 1 ? 2 : 4;
    const bool vec = ((reinterpret_cast<uintptr_t>(s) | reinterpret_cast<uintptr_t>(p)) & 15) == 0 &&
                     (n * esz) % 16 == 0;
    if (dtype == 1)
        return vec ? launch_softmax_v<true, true>(sp, stream) : launch_softmax_v<true, false>(sp, stream);
    return vec ? launch_softmax_v<false, true>(sp, stream) : launch_softmax_v<false, false>(sp, stream);
}

}  // namespace fa
