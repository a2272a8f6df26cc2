// fa_decode.hip -- the split-key partial pass for decoding: one query row per
// (batch, head), bf16, keys cut into ranges whose partial states the merge
// kernel then combines.
//
// With a single query row every key and value byte is used once, so the pass
// is bound by reading K and V from HBM, and what decides its speed is how
// many bytes are in flight.  The general kernel stages K/V through LDS, and
// LDS capacity caps that (two 32 KiB tiles per CU in flight); it also spends
// 32-row matrix products on one row.  This kernel keeps nothing in LDS:
// every wave streams its own keys straight into registers, the loads of the
// keys issued before the current ones are used, and the dot products
// run on the vector units in fp32 (bf16 widens exactly).
//
// Per wave and step of STEP keys, lane l = LPK * g + e (LPK = d / 8 lanes
// per key) loads 16 bytes -- dims 8e .. 8e+7 -- of key i * KPI + g for each
// load instruction i, for K and for V.  Its partial dot products with q are
// summed over the LPK lanes of its group, by a reduce-scatter that leaves
// lane l with the full score of one key (key (e % NI) * KPI + g: instruction
// e % NI; with NI < LPK the lanes e and e + NI hold the same key).
// The recurrence then runs per lane with the exact running maximum
// ("2.2b: FlashAttention -- Online Softmax", "The Complete Online Softmax
// Algorithm"): m_new = max(m, max of the step), alpha = exp(m - m_new),
// p = exp(s - m_new), l = alpha l + p, o~ = alpha o~ + p v.  The 4 waves of
// a workgroup take its steps in turn, and their states are merged at the end
// with the rescaling identity ("The math of
// FlashAttention", "The rescaling identity, derived").

#include "fa_device.h"

namespace fa {

template <int D>
struct DecCfg {
    static constexpr int NW = 4;            // waves per workgroup
    static constexpr int T = 64 * NW;
    static constexpr int TILE = 64;         // keys per unit of the split ranges
    // keys per step: 32, so that three K/V blocks in flight stay within the
    // register budget and every wave has an even number of steps; a key's
    // score ends up in 64 / STEP lanes
    static constexpr int STEP = 32;
    static constexpr int LPK = D / 8;       // lanes per key, 8 bf16 (16 bytes) each
    static constexpr int KPI = 64 / LPK;    // keys per load instruction
    static constexpr int NI = STEP / KPI;   // load instructions per step
};

// The two bf16 values of a 32-bit word (the lower address in the low half)
// as floats: exact.
__device__ __forceinline__ float lo_bf16(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t x)
{
    return __builtin_bit_cast(float, x & 0xffff0000u);
}

template <int D>
struct DecBuf {
    u32x4 k[DecCfg<D>::NI];
    u32x4 v[DecCfg<D>::NI];
    uint32_t mk;             // key-padding byte of this lane's key (ignored without a mask)
};

template <int D, bool CAUSAL>
struct Decode {
    using C = DecCfg<D>;

    int lane, w, g, e;
    int Nk;
    float c;
    const uint16_t *Kg, *Vg;
    const uint8_t *Mg;       // the batch's key-padding row; without a mask any readable
                             // address (the K rows), whose byte is ignored
    bool masked;
    float qf[8];             // dims 8e .. 8e+7 of the query row
    float m, l_part;         // running maximum (raw score units) and this lane's share of l
    float o[8];              // o~ for dims 8e .. 8e+7, summed over this lane's keys

    // 16 bytes of key row `key` (clamped to the last key; such scores are
    // masked).  The byte offset within the head fits 32 bits (the launcher
    // sends larger heads to the general kernel), so the load takes the
    // uniform base in scalar registers and one offset register per lane.
    __device__ __forceinline__ u32x4 row16(const uint16_t *base, int key) const
    {
        const uint32_t r = (uint32_t)(key < Nk ? key : Nk - 1);
        const uint32_t off = r * (uint32_t)(2 * D) + 16u * (uint32_t)e;
        return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(base) + off);
    }

    // K rows of the step at k0, and the padding byte of this lane's key,
    // loaded together and without a branch: every load of a step is then
    // waited for at one place.
    __device__ __forceinline__ void load_k(DecBuf<D> &b, int k0) const
    {
#pragma unroll
        for (int i = 0; i < C::NI; ++i) b.k[i] = row16(Kg, k0 + i * C::KPI + g);
        const int key = k0 + (e % C::NI) * C::KPI + g;
        b.mk = Mg[masked ? (key < Nk ? key : Nk - 1) : 0];
    }

    __device__ __forceinline__ void load_v(DecBuf<D> &b, int k0) const
    {
#pragma unroll
        for (int i = 0; i < C::NI; ++i) b.v[i] = row16(Vg, k0 + i * C::KPI + g);
    }

    // Raw score of key k0 + (e % NI) * KPI + g (this lane's key), -inf if
    // hidden or if the step is a filler (`real` false).
    __device__ __forceinline__ float scores(const DecBuf<D> &b, int k0, bool real) const
    {
        float part[C::NI];
#pragma unroll
        for (int i = 0; i < C::NI; ++i) {
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a = __builtin_fmaf(qf[2 * j], lo_bf16(b.k[i][j]), a);
                a = __builtin_fmaf(qf[2 * j + 1], hi_bf16(b.k[i][j]), a);
            }
            part[i] = a;
        }
        // Sum over the LPK lanes of the group: plain sums over the lane bits
        // at and above NI, then a reduce-scatter: at the step with lane
        // distance h, a lane keeps the half of its values whose index has bit
        // h equal to its own lane bit h and adds the other lane's.
#pragma unroll
        for (int h = C::LPK / 2; h >= C::NI; h >>= 1)
#pragma unroll
            for (int i = 0; i < C::NI; ++i) part[i] += __shfl_xor(part[i], h);
#pragma unroll
        for (int h = C::NI / 2; h >= 1; h >>= 1) {
            const bool upper = (e & h) != 0;
#pragma unroll
            for (int i = 0; i < h; ++i) {
                const float keep = upper ? part[i + h] : part[i];
                const float give = upper ? part[i] : part[i + h];
                part[i] = keep + __shfl_xor(give, h);
            }
        }
        const int key = k0 + (e % C::NI) * C::KPI + g;
        bool vis = real && key < Nk && (!masked || b.mk != 0);
        if (CAUSAL) vis = vis && key == 0;       // the only query row is row 0
        return vis ? part[0] : kNegInf;
    }

    __device__ __forceinline__ static float wave_max(float x)
    {
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) x = fmaxf(x, __shfl_xor(x, h));
        return x;
    }

    __device__ __forceinline__ static float wave_sum(float x)
    {
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) x += __shfl_xor(x, h);
        return x;
    }

    // The recurrence step over the STEP keys whose scores are s (one per lane
    // and copy) and whose V rows are in b.
    __device__ __forceinline__ void update(float s, const DecBuf<D> &b)
    {
        const float m_new = fmaxf(m, wave_max(s));
        const float m_use = m_new == kNegInf ? 0.0f : m_new;   // nothing visible yet
        const float alpha = __builtin_amdgcn_exp2f((m - m_use) * c);
        const float pv = __builtin_amdgcn_exp2f((s - m_use) * c);
        m = m_new;
        // l counts each key once: only its first copy adds
        l_part = __builtin_fmaf(l_part, alpha, e < C::NI ? pv : 0.0f);
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] *= alpha;
        // o~ += p v: instruction i holds key i * KPI + g, whose weight is in
        // lane (g, e = i) of this lane's group.  A hidden key (masked, past
        // N_k, a filler step) has weight exactly 0, but its V row may hold
        // anything (padded cache slots, repeated rows), and 0 * NaN is NaN;
        // when the step has such a weight its products are skipped instead,
        // so hidden keys contribute exactly zero whatever their values.
        if (__any(pv == 0.0f)) {
#pragma unroll
            for (int i = 0; i < C::NI; ++i) {
                const float pk = __shfl(pv, i, C::LPK);
                const bool take = pk != 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v0 = take ? lo_bf16(b.v[i][j]) : 0.0f;
                    const float v1 = take ? hi_bf16(b.v[i][j]) : 0.0f;
                    o[2 * j] = __builtin_fmaf(pk, v0, o[2 * j]);
                    o[2 * j + 1] = __builtin_fmaf(pk, v1, o[2 * j + 1]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::NI; ++i) {
                const float pk = __shfl(pv, i, C::LPK);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    o[2 * j] = __builtin_fmaf(pk, lo_bf16(b.v[i][j]), o[2 * j]);
                    o[2 * j + 1] = __builtin_fmaf(pk, hi_bf16(b.v[i][j]), o[2 * j + 1]);
                }
            }
        }
    }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fa_decode_bf16_kernel(const Params p)
{
    using C = DecCfg<D>;
    __shared__ float sm[C::NW], sl[C::NW];
    __shared__ __attribute__((aligned(16))) float so[C::NW][D];

    Decode<D, CAUSAL> k;
    k.lane = threadIdx.x & 63;
    k.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    k.g = k.lane / C::LPK;
    k.e = k.lane % C::LPK;
    const int split = blockIdx.x % p.n_split;
    const int bh = blockIdx.x / p.n_split;
    const int b = bh / p.H;
    k.Nk = p.Nk;
    k.c = p.c;
    k.Kg = static_cast<const uint16_t *>(p.k) + (size_t)bh * p.Nk * D;
    k.Vg = static_cast<const uint16_t *>(p.v) + (size_t)bh * p.Nk * D;
    k.masked = p.mask != nullptr;
    k.Mg = k.masked ? p.mask + (size_t)b * p.Nk : reinterpret_cast<const uint8_t *>(k.Kg);
    {
        const u32x4 qw = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.q) +
                                                          (size_t)bh * D + 8 * k.e);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            k.qf[2 * j] = lo_bf16(qw[j]);
            k.qf[2 * j + 1] = hi_bf16(qw[j]);
        }
    }
    k.m = kNegInf;
    k.l_part = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) k.o[j] = 0.0f;

    // This workgroup's range of 64-key tiles, cut as the general kernel cuts
    // it (under causality the only row sees key 0 alone), less the tiles
    // outside a key-padding mask's visible span.
    const int n_all = CAUSAL ? 1 : (p.Nk + C::TILE - 1) / C::TILE;
    int t_lo = (int)((int64_t)split * n_all / p.n_split);
    int n_t = (int)((int64_t)(split + 1) * n_all / p.n_split) - t_lo;
    trim_to_visible<C::TILE, C::T>(k.masked ? k.Mg : nullptr, p.Nk, t_lo, n_t);
    // The workgroup's steps of 32 keys go to its waves in turn (step i to
    // wave i % 4), so that at any time the workgroup streams one contiguous
    // stretch of K and of V.
    constexpr int SPT = C::TILE / C::STEP;     // steps per tile
    const int s0 = t_lo * SPT, s1 = (t_lo + n_t) * SPT;
    const int cnt = s1 - s0 > k.w ? (s1 - s0 - k.w + C::NW - 1) / C::NW : 0;
    const int last = cnt > 0 ? s0 + k.w + C::NW * (cnt - 1) : s0;
    auto key0 = [&](int j) {                   // first key of the wave's j-th step
        const int st = s0 + k.w + C::NW * j;
        return (st < last ? st : last) * C::STEP;
    };

    // Two buffers: the next step's K is loaded before the current scores,
    // its V once the current scores no longer need this step's K, so that at
    // most three of the four K/V blocks are live.  The loads carry no
    // condition, which keeps the load counters the compiler waits on exact:
    // past the wave's last step they re-read that step's rows (a filler step
    // when the count is odd, its scores hidden; and the unused prefetch after
    // the end).  The scheduling barriers keep every load group where it is
    // written, so that each wait covers only the loads it needs.
    DecBuf<D> b0, b1;
    k.load_k(b0, key0(0));
    k.load_v(b0, key0(0));
    for (int j = 0; j < cnt; j += 2) {
        k.load_k(b1, key0(j + 1));
        __builtin_amdgcn_sched_barrier(0);
        const float sa = k.scores(b0, key0(j), true);
        __builtin_amdgcn_sched_barrier(0);
        k.load_v(b1, key0(j + 1));
        __builtin_amdgcn_sched_barrier(0);
        k.update(sa, b0);
        __builtin_amdgcn_sched_barrier(0);
        k.load_k(b0, key0(j + 2));
        __builtin_amdgcn_sched_barrier(0);
        const float sb = k.scores(b1, key0(j + 1), j + 1 < cnt);
        __builtin_amdgcn_sched_barrier(0);
        k.load_v(b0, key0(j + 2));
        __builtin_amdgcn_sched_barrier(0);
        k.update(sb, b1);
    }

    // The wave's state: l summed over its lanes, o~ over the lane groups.
    const float l_w = Decode<D, CAUSAL>::wave_sum(k.l_part);
#pragma unroll
    for (int h = C::LPK; h < 64; h <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j) k.o[j] += __shfl_xor(k.o[j], h);
    if (k.lane < C::LPK) {
#pragma unroll
        for (int j = 0; j < 8; ++j) so[k.w][8 * k.e + j] = k.o[j];
    }
    if (k.lane == 0) {
        sm[k.w] = k.m;
        sl[k.w] = l_w;
    }
    __syncthreads();

    // Merge the waves' states: the workgroup's partial state, or, without a
    // split (all keys in this workgroup), o = o~ / l and lse = m + ln l
    // directly (o = 0 and lse = -inf when no key was visible).
    if (threadIdx.x < D) {
        float big = kNegInf;
#pragma unroll
        for (int i = 0; i < C::NW; ++i) big = fmaxf(big, sm[i]);
        float l = 0.0f, acc = 0.0f;
#pragma unroll
        for (int i = 0; i < C::NW; ++i) {
            if (sm[i] == kNegInf) continue;           // that wave saw no visible key
            const float f = __builtin_amdgcn_exp2f((sm[i] - big) * k.c);
            l = __builtin_fmaf(f, sl[i], l);
            acc = __builtin_fmaf(f, so[i][threadIdx.x], acc);
        }
        if (p.part_o) {
            const size_t row = (size_t)split * p.part_rows + bh;
            p.part_o[row * D + threadIdx.x] = acc;
            if (threadIdx.x == 0) {
                p.part_m[row] = big;
                p.part_l[row] = l;
            }
        } else {
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            static_cast<__bf16 *>(p.o)[(size_t)bh * D + threadIdx.x] = (__bf16)(acc * inv);
            if (threadIdx.x == 0)
                p.lse[bh] = l > 0.0f ? __builtin_fmaf(big, p.scale, __builtin_amdgcn_logf(l) * kLn2)
                                     : kNegInf;
        }
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_decode_dc(const Params &p, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((fa_decode_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(DecCfg<D>::T), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_decode(const Params &p, int d, int causal, int B, int H, hipStream_t stream)
{
    const int grid = B * H * p.n_split;
    if (d == 64)
        return causal ? launch_decode_dc<64, true>(p, grid, stream)
                      : launch_decode_dc<64, false>(p, grid, stream);
    return causal ? launch_decode_dc<128, true>(p, grid, stream)
                  : launch_decode_dc<128, false>(p, grid, stream);
}

}  // namespace fa
