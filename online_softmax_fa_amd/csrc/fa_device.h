// fa_device.h -- device-side helpers shared by the kernel files of
// libfa.so: vector types, the MFMA register layout, cross-lane reductions,
// LDS swizzles, LDS DMA and the launch helper.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fa_internal.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

static constexpr float kNegInf = -__builtin_inff();
static constexpr float kLn2 = 0.693147180559945309f;

// ---------------------------------------------------------------------------
// Grid mapping.  Workgroups are dispatched round-robin over the device's
// XCDs (workgroup g runs on XCD g % X, X = Params.xcds, queried from the
// device), and each XCD takes its share in order of g.  Work items are
// (batch-head, query tile, key range), key ranges innermost.  Every XCD gets
// a contiguous range of them, so the query tiles of one (batch, head) run on
// one XCD and share its L2 for K and V.
//
// Under causality query tile t visits t + 1 times the keys of tile 0, so item
// lengths differ, and a CU that finishes early takes the next item in
// dispatch order.  Each XCD therefore goes through its heads in groups, and
// within a group takes the items longest first across the group's heads
// (query tiles from the last to the first, the heads within each): the CUs
// then finish together.  A group is the fewest heads (a power of two) with at
// least as many items as the XCD runs workgroups at once (`slots`), which
// keeps the K/V the XCD reads at a time, and so its L2 footprint, small.
// That needs the heads to divide evenly among the XCDs; otherwise the items
// go head by head, each head's longest first.  When pairs of query tiles
// (t, n_qt - 1 - t) fill whole rounds of the device's workgroup slots, the
// bf16 launcher pairs them instead (pair_item), which needs no ordering.
// ---------------------------------------------------------------------------
// Workgroups g = 0 .. G-1 dealt to X XCDs in turn, numbered so that every
// XCD holds a contiguous range of the G items.
__device__ __forceinline__ int xcd_contiguous(int g, int G, int X)
{
    const int x = g % X, j = g / X;
    const int per = G / X, rem = G % X;
    return x * per + (x < rem ? x : rem) + j;
}

__device__ __forceinline__ int logical_tile(int g, int G, int n_qt, int n_split, bool causal,
                                            int slots, int X)
{
    const int x = g % X, j = g / X;
    const int heads = G / (n_qt * n_split);
    if (causal && heads % X == 0) {
        const int hp = heads / X;                  // heads per XCD
        const int items = n_qt * n_split;          // items per head
        int grp = 1;
        while (grp < hp && grp * items < slots) grp *= 2;
        grp = grp < hp ? grp : hp;
        const int gi = j / (grp * items), jg = j - gi * grp * items;
        const int h0 = gi * grp;
        const int gs = hp - h0 < grp ? hp - h0 : grp;   // heads in this group
        const int per_rank = gs * n_split;
        const int r = jg / per_rank, rest = jg - r * per_rank;
        const int hh = h0 + rest / n_split, sp = rest % n_split;
        return ((x * hp + hh) * n_qt + r) * n_split + sp;
    }
    return xcd_contiguous(g, G, X);
}

// Work item of workgroup g when causal query tiles go in pairs: the
// workgroup takes query tiles n_qt - 1 - t and t of one (batch, head), the
// longer first ("2.2b", "Scaling to Multiple Queries": rows are independent,
// so one workgroup may take any of them).  Every pair visits the same number
// of key tiles (an odd n_qt's middle tile is alone and shorter), so the
// workgroups are equally long and need no ordering; pairs are dealt to the
// XCDs in contiguous ranges (a head stays on one XCD).  item: 0 or 1;
// returns false when the workgroup has no such item.
__device__ __forceinline__ bool pair_item(int g, int G, int n_qt, int X, int item, int &bh,
                                          int &qt)
{
    const int np = (n_qt + 1) / 2;
    const int L = xcd_contiguous(g, G, X);
    bh = L / np;
    const int t = L - bh * np;
    qt = item == 0 ? n_qt - 1 - t : t;
    return item == 0 || t != n_qt - 1 - t;
}

// Position, inside a 32-key block, of register r of a lane with half h = l/32:
// key = 8*(r/4) + 4*h + r%4.  kpos(r) is the part that does not depend on h.
__device__ __forceinline__ constexpr int kpos(int r) { return 8 * (r >> 2) + (r & 3); }

// Visibility bits of the 32 keys of one key block, as seen by this lane: bit
// kpos(r) set <=> register r holds a visible key.
//   lim      number of leading keys (from the lane's first key) inside both
//            the causal limit and N_k, clamped to [0, 32]
//   kvbits   key-padding bits of the block, already shifted by 4*h
__device__ __forceinline__ uint32_t prefix_bits(int lim)
{
    return lim >= 32 ? 0xffffffffu : (lim <= 0 ? 0u : ((1u << lim) - 1u));
}

template <int NKB>
__device__ __forceinline__ void apply_visibility(f32x16 (&s)[NKB], const uint32_t (&vis)[NKB])
{
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s[kb][r] = ((vis[kb] >> kpos(r)) & 1u) ? s[kb][r] : kNegInf;
}

// Value of x in the lane l ^ 32 combined with x by `op`, in every lane: one
// v_permlane32_swap exchanges the two 32-lane halves, and both operands of
// the combination are the same two values in every lane (so both halves get
// bitwise the same result).
__device__ __forceinline__ float pair_max(float x)
{
    const int xi = __builtin_bit_cast(int, x);
    const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}

__device__ __forceinline__ float pair_sum(float x)
{
    const int xi = __builtin_bit_cast(int, x);
    const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// The recurrence step of the bf16 kernels, with a lagging reference, over
// NKB blocks of 32 keys (16 scores per lane each).
//
// The exponent base mc = fl(m_ref * c) (log2 units) follows the running
// maximum, but moves only when a step's maximum exceeds it by more than
// kLag.  Until then the weights exp2(s*c - mc) may exceed 1, up to
// 2^kLag = 256 here and 2^24 on the kernels' fast path that skips this step
// -- far from any fp32 or bf16 limit -- and alpha is exactly 1,
// so the rescale of o~ is skipped; when the base does move,
// alpha = exp2(mc_old - mc_new) < 2^-kLag rescales l and o~ as the pages'
// recurrence does.  l and o~ are always stated against the same base, so
// o~ / l and lse = (mc + log2 l) ln 2 are the same quantities as with the
// exact running maximum ("2.2b", "Why This Algorithm is Exact": any common
// reference cancels; "The math of FlashAttention", "Proof of numerical
// stability": here every exponent is at most 24 instead of 0).
//
// s: raw scores in (hidden keys at -inf), fp32 weights out; l_part: this
// lane's share of l, summed over the fp32 weights.  Returns whether o~ must
// be rescaled by `alpha`: some row of the wave moved its base after having
// seen a visible key.  While every key so far is hidden mc stays -inf and
// the weights are exp2(-inf) = 0.
static constexpr float kLag = 8.0f;

template <int NKB>
__device__ __forceinline__ bool lazy_step(f32x16 (&s)[NKB], float &mc, float &l_part, float c,
                                          float &alpha)
{
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = pair_max(mx);
    const float mxc = mx * c;                       // -inf when the step is all hidden
    const bool grow = mxc > mc + kLag;              // always true on the first visible step
    const float mc_new = grow ? mxc : mc;
    alpha = grow ? __builtin_amdgcn_exp2f(mc - mc_new) : 1.0f;
    const bool rescale = __any(grow && mc != kNegInf);
    mc = mc_new;
    const float base = (mc_new == kNegInf) ? 0.0f : mc_new;

    // l sums the fp32 weights (before they are rounded for the product), so
    // lse keeps fp32 accuracy; four partial sums keep the adds independent.
    float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -base));
            s[kb][r] = pv;
            sum[r & 3] += pv;
        }
    l_part = l_part * alpha + ((sum[0] + sum[1]) + (sum[2] + sum[3]));
    return rescale;
}

// LDS tiles of the bf16 kernels: BN rows of D bf16 (D*2 bytes, unpadded), K
// and V both in [key][dim] order.  Tiles
// are filled by LDS DMA (global_load_lds_dwordx4): one wave instruction
// writes 1 KiB of contiguous LDS, so rows cannot be padded; instead the
// 16-byte chunks of each row are XOR-permuted (swz_k, swz_v) and every lane
// loads the global chunk that belongs at its LDS slot.  The permutations keep
// the two LDS read patterns free of bank conflicts:
//   K (ds_read_b128): 32 consecutive rows, one 16-byte chunk each;
//   V (ds_read_b64_tr_b16): per half wave, 4 consecutive rows x 64 bytes.
template <int D>
__device__ __forceinline__ int swz_k(int r)
{
    if (D == 128) return r & 15;
    return ((r >> 1) & 7) ^ ((r & 1) << 2);
}

template <int D>
__device__ __forceinline__ int swz_v(int r)
{
    if (D == 128) return (0xAC60 >> (4 * (r & 3))) & 15;   // 0, 6, 12, 10
    return 2 * (r & 3);
}

// LDS DMA of 16 bytes per lane, global base + voff (bytes, per lane) to LDS
// lds_addr + 16 * lane (global_load_lds_dwordx4; M0 holds the LDS address).
// Written as inline assembly on purpose: the compiler then does not treat the
// transfer as a store to LDS, and does not make every later LDS read wait for
// all DMA in flight.  The kernel orders the two itself: a stage is read only
// after the s_waitcnt vmcnt(0) and barrier that end the iteration filling it,
// and refilled only after the barrier that ends the iteration reading it.
// The base address is first copied by a scalar move: gfx9 needs five wait
// states between a VALU instruction writing an SGPR (as v_readlane does when
// the compiler restores a spilled base right before the asm, whose contents
// it does not inspect) and a vector-memory instruction reading it, while a
// scalar instruction reading it waits in hardware.  The move also gives the
// one wait state after the M0 write.
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds_addr)
{
    uint64_t b;
    asm volatile("s_mov_b64 %0, %2\n\tglobal_load_lds_dwordx4 %1, %0"
                 : "=&s"(b)
                 : "v"(voff), "s"(base), "{m0}"(lds_addr));
}

// s_waitcnt vmcnt(0): every vector-memory operation of this wave, LDS DMA
// included, has completed (expcnt and lgkmcnt fields left at their maximum).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Key-padding masks: the first and the last visible key (nonzero byte) of
// row[k_lo .. k_hi), found by all T threads of the workgroup together.
// Returns false when every key of the range is masked.  Every thread of the
// workgroup must call it (it synchronises once); it reads only bytes inside
// the range: aligned 4-byte words for the interior, single bytes for up to
// three keys at either end.  The results are workgroup-uniform.
template <int T>
__device__ __forceinline__ bool visible_span(const uint8_t *row, int k_lo, int k_hi, int &first,
                                             int &last)
{
    __shared__ int red[2 * (T / 64)];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int f = 0x7fffffff, l = -1;
    const uintptr_t base = (uintptr_t)row;
    const uintptr_t p0 = base + k_lo, p1 = base + k_hi;
    const uintptr_t w0 = (p0 + 3) & ~(uintptr_t)3, w1 = p1 & ~(uintptr_t)3;
    const uintptr_t head_end = w0 < p1 ? w0 : p1;
    const uintptr_t tail_beg = w1 > head_end ? w1 : head_end;
    // edge bytes: threads 0..2 the head, 3..5 the tail
    if (tid < 3 && p0 + tid < head_end && row[k_lo + tid]) {
        f = k_lo + tid;
        l = f;
    }
    if (tid >= 3 && tid < 6 && tail_beg + (tid - 3) < p1) {
        const int k = (int)(tail_beg - base) + (tid - 3);
        if (row[k]) {
            f = f < k ? f : k;
            l = l > k ? l : k;
        }
    }
    // interior words
    const int nwd = w1 > w0 ? (int)((w1 - w0) >> 2) : 0;
    const uint32_t *wp = reinterpret_cast<const uint32_t *>(w0);
    const int k_w0 = (int)(w0 - base);
    for (int i = tid; i < nwd; i += T) {
        const uint32_t x = wp[i];
        const uint32_t nz = ((x & 0x000000ffu) ? 1u : 0u) | ((x & 0x0000ff00u) ? 2u : 0u) |
                            ((x & 0x00ff0000u) ? 4u : 0u) | ((x & 0xff000000u) ? 8u : 0u);
        if (nz) {
            const int k = k_w0 + 4 * i;
            const int kf = k + __builtin_ctz(nz), kl = k + 31 - __builtin_clz(nz);
            f = f < kf ? f : kf;
            l = l > kl ? l : kl;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int fo = __shfl_xor(f, off), lo = __shfl_xor(l, off);
        f = f < fo ? f : fo;
        l = l > lo ? l : lo;
    }
    if (lane == 0) {
        red[wv] = f;
        red[T / 64 + wv] = l;
    }
    __syncthreads();
    f = red[0];
    l = red[T / 64];
#pragma unroll
    for (int i = 1; i < T / 64; ++i) {
        f = f < red[i] ? f : red[i];
        l = l > red[T / 64 + i] ? l : red[T / 64 + i];
    }
    first = __builtin_amdgcn_readfirstlane(f);
    last = __builtin_amdgcn_readfirstlane(l);
    return last >= 0;
}

// A key-padding mask can leave whole key tiles at either end of a
// workgroup's range with no visible key.  The range shrinks to the tiles from
// the first to the last visible key, or to none when every key is masked: a
// tile without a visible key adds nothing to l or o~ (all its weights are 0),
// so leaving it out is exact, and saves its transfers and its wait.  Every
// thread of the workgroup calls this with the same arguments.
template <int BN, int T>
__device__ __forceinline__ void trim_to_visible(const uint8_t *Mg, int Nk, int &t_lo, int &n_t)
{
    if (!Mg || n_t <= 0) return;
    const int64_t end = (int64_t)(t_lo + n_t) * BN;
    const int k_hi = end < Nk ? (int)end : Nk;
    int first, last;
    if (visible_span<T>(Mg, t_lo * BN, k_hi, first, last)) {
        t_lo = first / BN;
        n_t = last / BN + 1 - t_lo;
    } else {
        n_t = 0;
    }
}

template <int N>
struct IntC {
    static constexpr int value = N;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// ---------------------------------------------------------------------------
// Launch helper
// ---------------------------------------------------------------------------
// Dynamic LDS above the default limit is opted into once per kernel and
// device; `done` is the per-kernel record of devices already set up.
inline hipError_t launch(const void *kernel, void (*fn)(Params), std::atomic<uint64_t> &done,
                         int grid, int threads, size_t lds, hipStream_t stream, const Params &p)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = 1ull << (dev & 63);
    if (!(done.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        done.fetch_or(bit, std::memory_order_acq_rel);
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), lds, stream, p);
    return hipGetLastError();
}

}  // namespace fa
