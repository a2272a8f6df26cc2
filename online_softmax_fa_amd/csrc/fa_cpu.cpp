// fa_cpu.cpp -- the online-softmax attention forward pass on the host CPU,
// tiled for the caches and vectorized (libfa_cpu.so; ABI in include/fa_cpu.h).
//
// "The math of FlashAttention", section "Why the same math matters on a
// CPU": the recurrence keeps the active score block in cache while keys and
// values stream through once, and its update -- a max and two scaled sums --
// maps onto SIMD lanes.  Per (batch, head, query tile of BQ rows) one thread:
//   - widens the query tile to float once;
//   - for every key tile of BK keys: packs K transposed (dims x keys) and V
//     (keys x dims) into its scratch, forms the score block
//     S = scale * Q . K^T vectorized across the keys (four rows share every
//     load of K), masks it (-inf before
//     the maximum: "Pitfalls in implementing the recurrence"), and takes the
//     pages' step per row with its exact running maximum:
//         m_new = max(m, max_j s_j),  alpha = exp(m - m_new),
//         p_j = exp(s_j - m_new),  l = alpha l + sum p,  o~ = alpha o~ + P.V
//     ("2.2b: FlashAttention -- Online Softmax", "The Complete Online Softmax
//     Algorithm"), the P.V sum vectorized across the head dims, four keys
//     per pass over each accumulator row;
//   - divides once: o = o~ / l, lse = m + ln l.
// A block whose keys are all masked while m is still -inf leaves the state
// unchanged (the pages never meet this case; skipping such a block is the
// reading the GPU library uses too).
//
// The tile routine is compiled three times -- AVX-512, AVX2 + FMA, and
// baseline x86-64 -- and the first one the host's CPU supports is used (a
// feature check, not a model check).

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>

#ifdef _OPENMP
#include <omp.h>
#endif

#include "fa_cpu.h"

namespace {

constexpr int BQ = 64;       // query rows per tile
constexpr int BK = 64;       // keys per tile
constexpr int DMAX = 256;    // largest head width
constexpr float kNegInf = -INFINITY;

// Per-thread working set, about 272 KiB: it stays in the core's L2 while a
// query tile streams its key tiles through.
struct Scratch {
    alignas(64) float q[BQ * DMAX];      // query tile, row-major, rows past N_q zero
    alignas(64) float kt[DMAX * BK];     // key tile transposed: [dim][key], keys past N_k zero
    alignas(64) float v[BK * DMAX];      // value tile: [key][dim], keys past N_k zero
    alignas(64) float s[BQ * BK];        // scores, then weights
    alignas(64) float acc[BQ * DMAX];    // o~ of the tile's rows
    float m[BQ], l[BQ];
};

struct Args {
    const void *q, *k, *v;
    void *o;
    float *lse;
    const uint8_t *mask;
    int B, H, Nq, Nk, d;
    float scale;
    int causal, bf16;
};

inline float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

inline uint16_t float_to_bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);   // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);                                            // round to nearest even
    return (uint16_t)(u >> 16);
}

inline float load_elem(const void *base, int64_t idx, int bf16)
{
    if (bf16) return bf16_bits_to_float(static_cast<const uint16_t *>(base)[idx]);
    return static_cast<const float *>(base)[idx];
}

// a * b + c: one fused operation where the instruction set has it (the
// baseline build would otherwise call a slow software fma).
template <bool FMA>
inline __attribute__((always_inline)) float fmadd(float a, float b, float c)
{
    if (FMA) return __builtin_fmaf(a, b, c);
    return a * b + c;
}

// exp(x) for x <= 0: Cody-Waite reduction x = k ln2 + r (ln 2 split into a
// high part exact in k * hi and a low part), e^r by a degree-7 Taylor
// polynomial (|r| <= ln2 / 2, truncation < 6e-9), 2^k through the exponent
// bits.  Branch-free, so loops over it vectorize.
template <bool FMA>
inline __attribute__((always_inline)) float exp_nonpos(float x)
{
    const float kLog2e = 1.44269504088896341f;
    const float kLn2Hi = 0.693145751953125f;        // 12 significant bits: k * hi is exact
    const float kLn2Lo = 1.42860682030941723e-6f;   // ln 2 - hi
    x = x > 0.0f ? 0.0f : x;
    x = x < -104.0f ? -104.0f : x;                  // also maps -inf into range
    // round to the nearest integer by adding and subtracting 1.5 * 2^23 (exact
    // for |x log2 e| < 2^22; the library is built without reassociation)
    const float kRound = 12582912.0f;
    const float kf = (x * kLog2e + kRound) - kRound;
    float r = fmadd<FMA>(-kf, kLn2Hi, x);             // exact: kf * hi has <= 20 bits
    r = fmadd<FMA>(-kf, kLn2Lo, r);
    float p = 1.0f / 5040.0f;
    p = fmadd<FMA>(p, r, 1.0f / 720.0f);
    p = fmadd<FMA>(p, r, 1.0f / 120.0f);
    p = fmadd<FMA>(p, r, 1.0f / 24.0f);
    p = fmadd<FMA>(p, r, 1.0f / 6.0f);
    p = fmadd<FMA>(p, r, 0.5f);
    p = fmadd<FMA>(p, r, 1.0f);
    p = fmadd<FMA>(p, r, 1.0f);
    const int ki = (int)kf;
    const int bits = (ki + 127) << 23;
    float two_k;
    memcpy(&two_k, &bits, 4);
    return ki < -126 ? 0.0f : p * two_k;
}

// One query tile of one (batch, head): rows q0 .. q0 + nq - 1.  Inlined into
// one wrapper per instruction set below, which compiles it for that set.
template <bool FMA>
inline __attribute__((always_inline)) void query_tile(const Args &a, Scratch &w, int bh, int q0,
                                                      int nq)
{
    const int d = a.d, Nk = a.Nk, Nq = a.Nq;
    const int b = bh / a.H;
    const int64_t qoff = ((int64_t)bh * Nq + q0) * d;
    const int64_t koff = (int64_t)bh * Nk * d;
    const uint8_t *mask = a.mask ? a.mask + (int64_t)b * Nk : nullptr;
    const int nq4 = (nq + 3) & ~3;                     // rows in blocks of 4, padded with zeros

    for (int i = 0; i < nq4; ++i)
        for (int c = 0; c < d; ++c)
            w.q[i * d + c] = i < nq ? load_elem(a.q, qoff + (int64_t)i * d + c, a.bf16) : 0.0f;
    for (int i = 0; i < nq4; ++i) {
        w.m[i] = kNegInf;
        w.l[i] = 0.0f;
        for (int c = 0; c < d; ++c) w.acc[i * d + c] = 0.0f;
    }

    int kend = Nk;
    if (a.causal) kend = q0 + nq < Nk ? q0 + nq : Nk;   // keys beyond the last row are masked
    for (int k0 = 0; k0 < kend; k0 += BK) {
        const int nk = kend - k0 < BK ? kend - k0 : BK;
        // pack the tile: V row by row, K transposed; keys past nk are zero
        for (int j = 0; j < BK; ++j) {
            float *vj = w.v + j * d;
            if (j < nk) {
                const int64_t e = koff + (int64_t)(k0 + j) * d;
                for (int c = 0; c < d; ++c) vj[c] = load_elem(a.v, e + c, a.bf16);
                for (int c = 0; c < d; ++c) w.kt[c * BK + j] = load_elem(a.k, e + c, a.bf16);
            } else {
                for (int c = 0; c < d; ++c) vj[c] = 0.0f;
                for (int c = 0; c < d; ++c) w.kt[c * BK + j] = 0.0f;
            }
        }

        // S = Q . K^T, four rows at a time, vectorized across the 64 keys
        for (int i0 = 0; i0 < nq4; i0 += 4) {
            float s4[4][BK];
            for (int r = 0; r < 4; ++r)
#pragma omp simd
                for (int j = 0; j < BK; ++j) s4[r][j] = 0.0f;
            const float *q4 = w.q + i0 * d;
            for (int c = 0; c < d; ++c) {
                const float *kc = w.kt + c * BK;
                const float x0 = q4[c], x1 = q4[d + c], x2 = q4[2 * d + c], x3 = q4[3 * d + c];
#pragma omp simd
                for (int j = 0; j < BK; ++j) {
                    const float kv = kc[j];
                    s4[0][j] = fmadd<FMA>(x0, kv, s4[0][j]);
                    s4[1][j] = fmadd<FMA>(x1, kv, s4[1][j]);
                    s4[2][j] = fmadd<FMA>(x2, kv, s4[2][j]);
                    s4[3][j] = fmadd<FMA>(x3, kv, s4[3][j]);
                }
            }
            for (int r = 0; r < 4; ++r)
#pragma omp simd
                for (int j = 0; j < BK; ++j) w.s[(i0 + r) * BK + j] = s4[r][j];
        }

        // the recurrence step of every row
        for (int i = 0; i < nq; ++i) {
            float *srow = w.s + i * BK;
            const int qi = q0 + i;
            float mblk = kNegInf;
#pragma omp simd reduction(max : mblk)
            for (int j = 0; j < BK; ++j) {
                const int key = k0 + j;
                bool vis = j < nk;
                if (a.causal) vis = vis && key <= qi;
                if (mask) vis = vis && mask[key < Nk ? key : Nk - 1] != 0;
                const float sv = vis ? a.scale * srow[j] : kNegInf;
                srow[j] = sv;
                mblk = sv > mblk ? sv : mblk;
            }
            const float m_old = w.m[i];
            const float m_new = m_old > mblk ? m_old : mblk;
            if (m_new == kNegInf) {                  // nothing visible yet: state unchanged
#pragma omp simd
                for (int j = 0; j < BK; ++j) srow[j] = 0.0f;
                continue;
            }
            const float alpha = exp_nonpos<FMA>(m_old - m_new);   // exp(-inf) = 0 wipes the empty state
            float psum = 0.0f;
#pragma omp simd reduction(+ : psum)
            for (int j = 0; j < BK; ++j) {
                const float p = srow[j] == kNegInf ? 0.0f : exp_nonpos<FMA>(srow[j] - m_new);
                srow[j] = p;
                psum += p;
            }
            w.l[i] = alpha * w.l[i] + psum;
            w.m[i] = m_new;
            float *ar = w.acc + i * d;
#pragma omp simd
            for (int c = 0; c < d; ++c) ar[c] *= alpha;
        }

        // o~ += P . V, four keys per pass over each accumulator row
        const int nk4 = (nk + 3) & ~3;
        for (int i = 0; i < nq; ++i) {
            const float *pr = w.s + i * BK;
            float *ar = w.acc + i * d;
            for (int j = 0; j < nk4; j += 4) {
                const float p0 = pr[j], p1 = pr[j + 1], p2 = pr[j + 2], p3 = pr[j + 3];
                const float *v0 = w.v + j * d;
#pragma omp simd
                for (int c = 0; c < d; ++c) {
                    float x = fmadd<FMA>(p0, v0[c], ar[c]);
                    x = fmadd<FMA>(p1, v0[d + c], x);
                    x = fmadd<FMA>(p2, v0[2 * d + c], x);
                    ar[c] = fmadd<FMA>(p3, v0[3 * d + c], x);
                }
            }
        }
    }

    for (int i = 0; i < nq; ++i) {
        const int64_t row = (int64_t)bh * Nq + q0 + i;
        const float l = w.l[i];
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        for (int c = 0; c < d; ++c) {
            const float x = w.acc[i * d + c] * inv;
            if (a.bf16)
                static_cast<uint16_t *>(a.o)[row * d + c] = float_to_bf16_bits(x);
            else
                static_cast<float *>(a.o)[row * d + c] = x;
        }
        a.lse[row] = l > 0.0f ? w.m[i] + std::log(l) : kNegInf;
    }
}

__attribute__((target("avx512f,avx512vl,avx512bw,avx512dq,avx2,fma")))
void query_tile_avx512(const Args &a, Scratch &w, int bh, int q0, int nq)
{
    query_tile<true>(a, w, bh, q0, nq);
}

__attribute__((target("avx2,fma")))
void query_tile_avx2(const Args &a, Scratch &w, int bh, int q0, int nq)
{
    query_tile<true>(a, w, bh, q0, nq);
}

void query_tile_base(const Args &a, Scratch &w, int bh, int q0, int nq)
{
    query_tile<false>(a, w, bh, q0, nq);
}

typedef void (*TileFn)(const Args &, Scratch &, int, int, int);

// The best build the CPU supports.  The environment variable FA_CPU_ISA
// ("avx2" or "base") can only lower the choice, so that every build can be
// tested on one machine.
TileFn pick_tile_fn()
{
    __builtin_cpu_init();
    const char *env = getenv("FA_CPU_ISA");
    const int cap = !env ? 2 : (strcmp(env, "avx2") == 0 ? 1 : (strcmp(env, "base") == 0 ? 0 : 2));
    if (cap >= 2 && __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512vl") &&
        __builtin_cpu_supports("avx512bw") && __builtin_cpu_supports("avx512dq") &&
        __builtin_cpu_supports("fma"))
        return query_tile_avx512;
    if (cap >= 1 && __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma"))
        return query_tile_avx2;
    return query_tile_base;
}

bool overlaps(const void *x, size_t nx, const void *y, size_t ny)
{
    if (!x || !y || nx == 0 || ny == 0) return false;
    const uintptr_t a0 = (uintptr_t)x, b0 = (uintptr_t)y;
    return a0 < b0 + ny && b0 < a0 + nx;
}

__attribute__((target("fma"))) float exp_fma(float x) { return exp_nonpos<true>(x); }

}  // namespace

extern "C" {

float fa_cpu_expf(float x)
{
    static const bool fma = (__builtin_cpu_init(), __builtin_cpu_supports("fma"));
    return fma ? exp_fma(x) : exp_nonpos<false>(x);
}

int fa_fwd_cpu(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
               int N_q, int N_k, int d, float scale, int causal, const uint8_t *kv_len_mask,
               int dtype, int threads)
{
    if (!q || !k || !v || !o || !lse) return -1;
    if (B <= 0 || H <= 0 || N_q <= 0 || N_k <= 0) return -2;
    if (d < 1 || d > DMAX) return -3;
    if (dtype != 0 && dtype != 1) return -4;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return -5;
    const double bh = (double)B * H;
    if (bh * N_q * d > 9.0e18 || bh * N_k * d > 9.0e18 || bh > 2.0e9) return -2;
    const size_t esz = dtype ? 2 : 4;
    const size_t qb = (size_t)B * H * N_q * d * esz, kb = (size_t)B * H * N_k * d * esz;
    const size_t lb = (size_t)B * H * N_q * 4, mb = kv_len_mask ? (size_t)B * N_k : 0;
    const void *ins[4] = {q, k, v, kv_len_mask};
    const size_t inb[4] = {qb, kb, kb, mb};
    for (int i = 0; i < 4; ++i)
        if (overlaps(o, qb, ins[i], inb[i]) || overlaps(lse, lb, ins[i], inb[i])) return -9;
    if (overlaps(o, qb, lse, lb)) return -9;

    static const TileFn tile = pick_tile_fn();
    Args a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.mask = kv_len_mask;
    a.B = B;
    a.H = H;
    a.Nq = N_q;
    a.Nk = N_k;
    a.d = d;
    a.scale = scale;
    a.causal = causal ? 1 : 0;
    a.bf16 = dtype;

    const int n_qt = (N_q + BQ - 1) / BQ;
    const int64_t items = (int64_t)B * H * n_qt;
#ifdef _OPENMP
    int nthr = threads > 0 ? threads : omp_get_max_threads();
#else
    int nthr = 1;
    (void)threads;
#endif
    if ((int64_t)nthr > items) nthr = (int)items;
    // one scratch block per thread, all allocated before any work
    Scratch **ws = static_cast<Scratch **>(calloc((size_t)nthr, sizeof(Scratch *)));
    bool ok = ws != nullptr;
    for (int t = 0; ok && t < nthr; ++t) {
        ws[t] = static_cast<Scratch *>(aligned_alloc(64, sizeof(Scratch)));
        ok = ws[t] != nullptr;
    }
    int used = 0;
    if (ok) {
#ifdef _OPENMP
#pragma omp parallel num_threads(nthr)
        {
            const int t = omp_get_thread_num();
#pragma omp single
            used = omp_get_num_threads();
            // longest causal tiles first, handed out one at a time
#pragma omp for schedule(dynamic, 1)
            for (int64_t it = 0; it < items; ++it) {
                const int bh = (int)(it / n_qt);
                const int qt = a.causal ? n_qt - 1 - (int)(it % n_qt) : (int)(it % n_qt);
                const int q0 = qt * BQ;
                tile(a, *ws[t], bh, q0, N_q - q0 < BQ ? N_q - q0 : BQ);
            }
        }
#else
        used = 1;
        for (int64_t it = 0; it < items; ++it) {
            const int bh = (int)(it / n_qt);
            const int q0 = (int)(it % n_qt) * BQ;
            tile(a, *ws[0], bh, q0, N_q - q0 < BQ ? N_q - q0 : BQ);
        }
#endif
    }
    if (ws) {
        for (int t = 0; t < nthr; ++t) free(ws[t]);
        free(ws);
    }
    if (!ok) return -2;
    return used;
}

}  // extern "C"
