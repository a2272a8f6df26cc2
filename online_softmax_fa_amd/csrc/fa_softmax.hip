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
// four, far below what the SIMDs can issue while the row streams in.
//
// Rows of at most KEEP vectors per thread (8192 fp32 or 16384 bf16 entries
// for KEEP = 8) are read from memory once: pass 1 issues all of a thread's
// loads at once and keeps the raw vectors in registers, and pass 2 computes
// from them.  Longer rows are read twice; the second read then mostly hits
// L2 or the MALL.
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

// A row vector as it is kept between the passes: four floats, or eight
// bf16 in four 32-bit words.  (Elements of an integer vector are never
// bit-cast to float one by one: that form has been compiled to read element
// 0 for every element.)
template <bool BF16>
struct RawVec {
    typedef sf32x4 type;
};
template <>
struct RawVec<true> {
    typedef su32x4 type;
};

template <bool BF16>
__device__ __forceinline__ void unpack(const typename RawVec<BF16>::type &u,
                                       float (&x)[BF16 ? 8 : 4])
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (BF16) {
            x[2 * e] = bf16_to_f32(u[e] & 0xffffu);
            x[2 * e + 1] = bf16_to_f32(u[e] >> 16);
        } else {
            x[e] = u[e];
        }
    }
}

// The 256 per-thread states (m, l) combined into the row's, in every thread:
// within the wave, then across the 4 waves through LDS.
__device__ __forceinline__ void combine_workgroup(float &m, float &l, float *red_m, float *red_l)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        combine(m, l, __shfl_xor(m, off), __shfl_xor(l, off));
    if ((tid & 63) == 0) {
        red_m[tid >> 6] = m;
        red_l[tid >> 6] = l;
    }
    __syncthreads();
    m = red_m[0];
    l = red_l[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) combine(m, l, red_m[i], red_l[i]);
    __syncthreads();     // red_* is reused by the next row
}

// VEC: the rows are 16-byte aligned and a whole number of vectors long.
// KEEP > 0 (with VEC): every row has at most KEEP * 256 vectors, held in
// registers between the passes.
template <bool BF16, bool VEC, int KEEP>
__global__ __launch_bounds__(256) void fa_softmax_rows_kernel(const SoftmaxParams p)
{
    constexpr int E = BF16 ? 8 : 4;
    constexpr int ESZ = BF16 ? 2 : 4;
    __shared__ float red_m[4], red_l[4];
    const int tid = threadIdx.x;

    for (int64_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
        const void *src = static_cast<const char *>(p.s) + row * p.n * ESZ;
        void *dst = static_cast<char *>(p.p) + row * p.n * ESZ;

        if (KEEP > 0) {
            const int nv = (int)(p.n / E);
            typedef typename RawVec<BF16>::type Raw;
            Raw raw[KEEP > 0 ? KEEP : 1];
#pragma unroll
            for (int u = 0; u < KEEP; ++u)
                if (tid + 256 * u < nv) raw[u] = reinterpret_cast<const Raw *>(src)[tid + 256 * u];
            float m = kNegInfS, l = 0.0f;
#pragma unroll
            for (int u = 0; u < KEEP; ++u)
                if (tid + 256 * u < nv) {
                    float x[E];
                    unpack<BF16>(raw[u], x);
                    absorb<E>(m, l, x);
                }
            combine_workgroup(m, l, red_m, red_l);
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            const float base = m == kNegInfS ? 0.0f : m;
#pragma unroll
            for (int u = 0; u < KEEP; ++u)
                if (tid + 256 * u < nv) {
                    float x[E];
                    unpack<BF16>(raw[u], x);
#pragma unroll
                    for (int e = 0; e < E; ++e) x[e] = ex(x[e] - base) * inv;
                    store_vec<BF16>(dst, tid + 256 * u, x);
                }
            if (tid == 0) {
                if (p.m) p.m[row] = m;
                if (p.l) p.l[row] = l;
            }
            continue;
        }

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

        combine_workgroup(m, l, red_m, red_l);

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

template <bool BF16, bool VEC, int KEEP>
static hipError_t launch_softmax_v(const SoftmaxParams &p, hipStream_t stream)
{
    const int grid = (int)(p.rows < (1 << 20) ? p.rows : (1 << 20));
    void (*fn)(SoftmaxParams) = fa_softmax_rows_kernel<BF16, VEC, KEEP>;
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
    constexpr int KEEP = 8;
    const bool keep = vec && n * esz <= (int64_t)KEEP * 256 * 16;
    if (dtype == 1) {
        if (keep) return launch_softmax_v<true, true, KEEP>(sp, stream);
        return vec ? launch_softmax_v<true, true, 0>(sp, stream)
                   : launch_softmax_v<true, false, 0>(sp, stream);
    }
    if (keep) return launch_softmax_v<false, true, KEEP>(sp, stream);
    return vec ? launch_softmax_v<false, true, 0>(sp, stream)
               : launch_softmax_v<false, false, 0>(sp, stream);
}

}  // namespace fa
