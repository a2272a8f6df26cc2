// fa_kernels.hip -- gfx950 kernels for the exact attention forward pass with
// the online-softmax recurrence.
//
// Per query row the kernel carries the running maximum m, the running
// denominator l and the unnormalised output o~ across key tiles; every tile
// rescales them by alpha = exp(m_old - m_new) and adds its own terms measured
// against m_new; one division o~ / l comes at the end.
//   -- "2.2b: FlashAttention -- Online Softmax", section "The Complete Online
//      Softmax Algorithm"; "The math of FlashAttention", sections "The
//      rescaling identity, derived" and "The block-wise update, and the full
//      algorithm".
// Many query rows are processed at once: every row is independent ("2.2b",
// "Scaling to Multiple Queries"), so a tile of queries turns the score block
// into a small matrix and P.V into a dense product ("The math of
// FlashAttention", end of "The block-wise update").  Both products run on the
// CDNA4 matrix cores.
//
// Work decomposition (one work item = NW waves = 32*NW query rows of one
// (batch, head); a workgroup takes one item, or two when causal query tiles
// go in pairs):
//   - each wave owns 32 query rows for the whole item;
//   - key/value tiles of BN keys are staged in LDS, double-buffered, by LDS
//     DMA of 16 bytes per lane, both in [key][dim] order with XOR-permuted
//     16-byte chunks; the P.V operands come out of V through transposing LDS
//     reads;
//   - scores are formed transposed, S^T = K . Q^T, with the 32x32 MFMA: lane l
//     then holds 16 keys of ONE query row (row l % 32), so the row maximum and
//     row sum are in-lane reductions plus one exchange with lane l ^ 32, and
//     the score registers are already laid out as the B operand of
//     O^T += V^T . P^T (no data movement between the two products);
//   - exp is the hardware exp2 with log2(e) folded into the score scale.
//
// MFMA register layout used throughout (32x32 output, 16 fp32 per lane):
//   lane l, register r  ->  row 8*(r/4) + 4*(l/32) + r%4,  column l%32.
// Operand layout of v_mfma_f32_32x32x16_bf16: lane l supplies row (A) or
// column (B) l%32 and the 8 consecutive k-slots 8*(l/32) .. 8*(l/32)+7.
// Operand layout of v_mfma_f32_32x32x2_f32: lane l supplies row/column l%32
// and k-slot l/32.
// The k-slot -> key assignment of a contraction is free as long as both
// operands use the same one; the P.V products use the one the score layout
// hands them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fa.h"
#include "fa_device.h"

namespace fa {

// The fast path of the bf16 kernels keeps a tile's weights against the
// current exponent base when every lane's sum of them is at most
// 2^FA_BF16_REF_LAG_LOG2 (include/fa.h): each weight is then at most that,
// and the base lags the running maximum by less than FA_BF16_REF_LAG_LOG2
// (log2 units).
constexpr float kFastSumLimit = (float)(1u << FA_BF16_REF_LAG_LOG2);
static_assert(FA_BF16_REF_LAG_LOG2 == 24, "the lag the documentation and tests state");

// One step of the recurrence on a tile of raw scores held in s (NKB blocks of
// 16 per lane), as the fp32 kernel runs it.  m_raw: running max in raw score
// units (-inf while no visible key has been seen); l_part: this lane's share
// of the running denominator.  Turns s into the weights p and returns alpha.
// c = scale * log2(e) > 0, so the max of raw scores is the max of scaled ones.
//
// "2.2b: FlashAttention -- Online Softmax", "The Complete Online Softmax
// Algorithm": m_block, m_new = max(m, m_block), scale = exp(m - m_new),
// P = exp(S - m_new), l = l*scale + sum(P).  Weights are measured against m
// itself, (s - m)*c, so the row maximum maps to exp2(0) = 1 exactly, and
// alpha = exp2((m_old - m_new)*c), whose difference is exact.
// While every key seen so far is masked, m_new is -inf and exp(m - m_new)
// would be exp(-inf + inf).  The pages never meet this case; the reading here
// is that such a tile changes nothing: alpha = 1 on the empty state and every
// weight is exp2(-inf) = 0 (the exponent base is taken as 0 for the weights).
// The first tile with a visible key then gets alpha = exp2(-inf) = 0, as the
// pages' -inf initialisation intends.
template <int NKB>
__device__ __forceinline__ float online_step(f32x16 (&s)[NKB], float &m_raw, float &l_part,
                                             float c)
{
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = pair_max(mx);

    const float m_new = fmaxf(m_raw, mx);
    const bool empty = (m_new == kNegInf);
    const float base = empty ? 0.0f : m_new;
    const float alpha = empty ? 1.0f : __builtin_amdgcn_exp2f((m_raw - m_new) * c);

    float sum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f((s[kb][r] - base) * c);
            s[kb][r] = pv;
            sum += pv;
        }
    l_part = l_part * alpha + sum;
    m_raw = m_new;
    return alpha;
}

// The lagging-reference step (lazy_step, fa_device.h) on a whole tile, with
// the weights also written as bf16 P.V operands: k-step t16 takes registers
// 8*(t16%2) .. +7 of key block t16/2.
template <int NKB, int NT16>
__device__ __forceinline__ bool lazy_step(f32x16 (&s)[NKB], bf16x8 (&pb)[NT16], float &mc,
                                          float &l_part, float c, float &alpha)
{
    const bool rescale = lazy_step<NKB>(s, mc, l_part, c, alpha);
#pragma unroll
    for (int t16 = 0; t16 < NT16; ++t16)
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[t16][i] = (__bf16)s[t16 >> 1][8 * (t16 & 1) + i];
    return rescale;
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
// Waves per workgroup of the bf16 kernel: 4 (query tiles of 128 rows, one
// wave per SIMD and workgroup, two or more workgroups per CU), or 8 (256
// rows, two waves per SIMD, one workgroup per CU), which serves every K/V
// tile staged in LDS to twice the rows.  8 waves pay off only for d = 128
// with 64-key tiles and when there are enough workgroups that none of them
// is the critical path: causal workgroups differ in length (the last query
// tile visits every key tile), so there it takes two per CU, which the
// longest-first order packs evenly; equal-length non-causal ones need only
// fill the CUs (the device's count, cus).
inline int bf16_waves(int d, int bn, int64_t B, int64_t H, int64_t nq, bool causal, int n_split,
                      int cus)
{
    if (d != 128 || bn != 64 || nq <= 128) return 4;
    const int64_t wgs = B * H * ((nq + 255) / 256) * n_split;
    return wgs >= (causal ? 2 : 1) * (int64_t)cus ? 8 : 4;
}

template <int D, int BN, int NW>
struct Bf16Cfg {
    static constexpr int BM = 32 * NW;
    static constexpr int BNA = BN < 32 ? 32 : BN;        // key rows allocated per tile
    static constexpr int NKB = BNA / 32;                 // 32-key blocks per tile
    static constexpr int NT16 = BN / 16;                 // 16-key k-steps of P.V
    static constexpr int ROW = D * 2;                    // bytes per key row
    static constexpr int CH = ROW / 16;                  // 16-byte chunks per row
    static constexpr int TILE = BNA * ROW;               // bytes of one K or V tile
    static constexpr int STAGE = 2 * TILE;
    static constexpr int ROWS_PER_DMA = 1024 / ROW;
    static constexpr int DMA_PER_TILE = BN * ROW / 1024;  // wave instructions per matrix
    static constexpr int DMA_PER_WAVE = (DMA_PER_TILE + NW - 1) / NW;
    static constexpr int T = NW * 64;
    // Two pipeline stages: one tile in flight while the other is read.  (A
    // third stage, two tiles in flight, measured slower on MI355X.)
    static constexpr int STAGES = 2;
    static constexpr size_t LDS_BYTES = (size_t)STAGES * STAGE;
    // LDS layout: the K tiles of all stages, then the V tiles.  Reads add a
    // stage offset of at most (STAGES-1) * TILE to per-lane base addresses
    // (the V base included in them), which stays within the 16-bit offset
    // field of the LDS instructions.
    static constexpr int V_BASE = STAGES * TILE;
    // Waves per SIMD the kernel is compiled for: two (at most 256 VGPRs per
    // lane), except for d = 64, which with shallower operand prefetch fits
    // three (64-key tiles, at most 168 VGPRs) or four (shorter tiles, 128):
    // the softmax-heavy small head width gains more from the extra waves
    // than from deeper prefetch.
    static constexpr int WAVES_PER_SIMD = D == 64 ? (BN <= 32 ? 4 : (BN == 64 ? 3 : 2)) : 2;
    static constexpr bool LEAN = WAVES_PER_SIMD > 2;
};

// Workgroups per CU the kernel is compiled for: WAVES_PER_SIMD waves on each
// of the 4 SIMDs, as far as the LDS of that many workgroups (tiles plus
// 1 KiB of static LDS) fits in the CU's 160 KiB.
template <int D, int BN, int NW>
constexpr int bf16_blocks_per_cu()
{
    const int by_waves = Bf16Cfg<D, BN, NW>::WAVES_PER_SIMD * 4 / NW;
    const int by_lds = (int)((160 * 1024) / (Bf16Cfg<D, BN, NW>::LDS_BYTES + 1024));
    const int b = by_waves < by_lds ? by_waves : by_lds;
    return b < 1 ? 1 : b;
}

// Per-thread state and steps of the bf16 kernel.  The kernel body is a
// struct with device member functions (no lambdas), all inlined.  TRACE
// builds the variant that records one row's state after every tile
// (fa_opts.trace); the other variant carries no trace code at all.
template <int D, int BN, int NW, bool CAUSAL, bool TRACE>
struct Bf16Fwd {
    using C = Bf16Cfg<D, BN, NW>;

    lds_char *lds;
    int lane, w, l31, h;
    int bh, b, q0, qw0, qrow, Nq, Nk;
    int split, t_lo, n_t;   // key-range split of this workgroup: tiles t_lo .. t_lo + n_t - 1
    bool reverse;
    bool trace_on;          // this wave holds the traced row
    float c;
    float *trace;
    int trace_row;
    const uint16_t *Kg, *Vg;
    const uint8_t *Mg;

    bf16x8 qf[D / 16];
    int offk[D / 16];
    int offv[D / 32];
    int dmak[C::DMA_PER_WAVE];     // per-lane element offsets of the DMA sources
    int dmav[C::DMA_PER_WAVE];     // within a tile (row-major K / V rows)

    float mc, l_part;   // exponent base fl(m_ref * c) (log2 units), this lane's share of l
    bool started;       // a key tile has been through the recurrence (wave-uniform)
    f32x16 o[D / 32];
    uint64_t kv_lo, kv_hi;
    int mnext0, mnext1;     // key-padding bytes of the next tile

    // Work item `item` of this workgroup (0, or 1 when causal query tiles go
    // in pairs): (batch-head, query tile, key range).  False if there is none.
    static __device__ __forceinline__ bool work_item(const Params &p, int item, int &bh_, int &qt,
                                                     int &split_)
    {
        if (CAUSAL && p.pair) {
            split_ = 0;
            return pair_item(blockIdx.x, gridDim.x, p.n_qt, p.xcds, item, bh_, qt);
        }
        if (item > 0) return false;
        // L = (head, query tile, key range), key ranges innermost
        const int L = logical_tile(blockIdx.x, gridDim.x, p.n_qt, p.n_split, CAUSAL,
                                   p.cus / p.xcds * bf16_blocks_per_cu<D, BN, NW>(), p.xcds);
        split_ = L % p.n_split;
        const int L2 = L / p.n_split;
        bh_ = L2 / p.n_qt;
        qt = CAUSAL ? (p.n_qt - 1 - L2 % p.n_qt) : (L2 % p.n_qt);
        return true;
    }

    __device__ __forceinline__ void init(const Params &p, lds_char *lds_base, int bh_, int qt,
                                         int split_)
    {
        lds = lds_base;
        const int tid = threadIdx.x;
        lane = tid & 63;
        // the wave index is uniform across the wave; reading it from lane 0
        // lets the compiler keep every per-wave decision in scalar registers
        w = __builtin_amdgcn_readfirstlane(tid >> 6);
        l31 = lane & 31;
        h = lane >> 5;

        split = split_;
        bh = bh_;
        b = bh / p.H;
        q0 = qt * C::BM;
        qw0 = q0 + 32 * w;          // first query row of this wave
        qrow = qw0 + l31;           // this lane's query row
        Nq = p.Nq;
        Nk = p.Nk;
        c = p.c;
        reverse = p.reverse != 0;
        trace = p.trace;
        trace_row = p.trace_row;
        trace_on = TRACE && bh == p.trace_bh && p.trace_row >= qw0 && p.trace_row < qw0 + 32;

        const uint16_t *Qg = static_cast<const uint16_t *>(p.q) + (size_t)bh * Nq * D;
        Kg = static_cast<const uint16_t *>(p.k) + (size_t)bh * Nk * D;
        Vg = static_cast<const uint16_t *>(p.v) + (size_t)bh * Nk * D;
        Mg = p.mask ? p.mask + (size_t)b * Nk : nullptr;

        const uint32_t lbase = (uint32_t)(uintptr_t)lds;
        // Q fragments: B operand of S^T = K . Q^T.  k-step kk covers head
        // dims 16*kk .. +15; this lane supplies dims 16*kk + 8*h .. +7.
        const int qr = qrow < Nq ? qrow : Nq - 1;
        const uint16_t *src = Qg + (size_t)qr * D + 8 * h;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8 *>(src + 16 * kk);

        // Key tiles the query tile needs (under causality, up to the diagonal
        // of its last row), and this workgroup's range of them.
        int n_all = (Nk + BN - 1) / BN;
        if (CAUSAL) {
            const int last_q = (q0 + C::BM < Nq ? q0 + C::BM : Nq) - 1;
            const int need = last_q / BN + 1;
            n_all = need < n_all ? need : n_all;
        }
        t_lo = (int)((int64_t)split * n_all / p.n_split);
        n_t = (int)((int64_t)(split + 1) * n_all / p.n_split) - t_lo;
        trim_to_visible<BN, C::T>(Mg, Nk, t_lo, n_t);

        // Per-lane LDS byte addresses (stage 0) of the MFMA operands.
        //   K (A operand of S^T = K.Q^T, 16 bytes): key row 32*kb + l31,
        //   dims 16*kk + 8*h .. +7, i.e. 16-byte chunk 2*kk + h of the row.
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            offk[kk] = lbase + l31 * C::ROW + 16 * ((2 * kk + h) ^ swz_k<D>(l31));
        //   V (A operand of O^T += V^T.P^T) through the transposing read:
        //   within a group of 16 lanes, lane i receives element i%4 of the
        //   8-byte chunks addressed by lanes 4j + i/4 (j = 0..3).  Lane
        //   i + 16g therefore addresses key row 16*t + 4*h + i/4 (+8 for the
        //   second read), dims 32*db + 16*(g&1) + 4*(i&3) .. +3, and receives
        //   V[16t + 4h + j][32db + l31] for j = 0..3: exactly the k-slots the
        //   score layout gives P.
        const int g = lane >> 4, i = lane & 15;
        const int vrow = 4 * h + (i >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int e = 8 * db + 4 * (g & 1) + (i & 3);   // 8-byte chunk of the row
            offv[db] = lbase + C::V_BASE + vrow * C::ROW + 16 * ((e >> 1) ^ swz_v<D>(vrow)) +
                       8 * (e & 1);
        }

        // DMA instruction i of this wave covers rows (w + i*NW)*ROWS_PER_DMA
        // .. +ROWS_PER_DMA-1 of a tile; the lane fills 16-byte slot
        // lane % CH of row lane / CH and fetches the global chunk that the
        // row's swizzle places there.
#pragma unroll
        for (int i2 = 0; i2 < C::DMA_PER_WAVE; ++i2) {
            const int row = (w + i2 * NW) * C::ROWS_PER_DMA + lane / C::CH;
            const int pc = lane % C::CH;
            dmak[i2] = row * D + 8 * (pc ^ swz_k<D>(row));
            dmav[i2] = row * D + 8 * (pc ^ swz_v<D>(row));
        }

        mc = kNegInf;
        l_part = 0.0f;
        started = false;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
        kv_lo = ~0ull;
        kv_hi = ~0ull;
        mnext0 = 0;
        mnext1 = 0;
    }

    // LDS DMA of key tile t into stage st: wave w issues instructions w,
    // w + NW, ...; instruction j covers rows j*ROWS_PER_DMA .. +ROWS_PER_DMA-1
    // of both K and V.  Rows past N_k are clamped to the last key (their
    // scores are masked).
    __device__ __forceinline__ void issue_tile(int t, int st)
    {
        const int k0 = t * BN;
        const uint16_t *kt = Kg + (size_t)k0 * D;     // wave-uniform tile bases
        const uint16_t *vt = Vg + (size_t)k0 * D;
        const bool full = k0 + BN <= Nk;
#pragma unroll
        for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
            const int j = w + i * NW;
            if (C::DMA_PER_TILE % NW == 0 || j < C::DMA_PER_TILE) {
                int ok = dmak[i], ov = dmav[i];
                if (!full) {
                    // rows past N_k re-read the last key (their scores are masked)
                    const int row = j * C::ROWS_PER_DMA + lane / C::CH;
                    const int over = k0 + row - (Nk - 1);
                    if (over > 0) {
                        ok -= over * D;
                        ov -= over * D;
                    }
                }
                const uint32_t dst = (uint32_t)(uintptr_t)(lds + st * C::TILE + j * 1024);
                dma16(kt, 2u * (uint32_t)ok, dst);
                dma16(vt, 2u * (uint32_t)ov, dst + C::V_BASE);
            }
        }
    }

    // One key-padding byte per lane for tile t (two for 128-key tiles),
    // loaded with the tile's transfers and turned into bits after the wait
    // for them.
    __device__ __forceinline__ void load_mask(int t)
    {
        const int j0 = t * BN + lane;
        mnext0 = (lane < BN && j0 < Nk) ? Mg[j0] : 0;
        mnext1 = (BN > 64 && lane + 64 < BN && j0 + 64 < Nk) ? Mg[j0 + 64] : 0;
    }

    __device__ __forceinline__ void take_mask()
    {
        kv_lo = __ballot(mnext0 != 0);
        kv_hi = __ballot(mnext1 != 0);
    }

    // Key tile visited at step it.
    __device__ __forceinline__ int tile_at(int it) const
    {
        return t_lo + (reverse ? (n_t - 1 - it) : it);
    }

    // Transfers of the tile visited at step it, into stage `st`.
    __device__ __forceinline__ void fetch(int it, int st)
    {
        const int t = tile_at(it);
        if (Mg) load_mask(t);
        issue_tile(t, st);
    }

    // Wait until every transfer of this wave has landed, then synchronise:
    // after it the tile fetched last is readable by all waves, and the stage
    // read before it is free to be refilled.
    __device__ __forceinline__ void land()
    {
        wait_vmem();
        __syncthreads();
    }

    // One iteration: start the transfers of step it + 1 into the other
    // stage, compute step it from stage ST, then wait for step it + 1's tile
    // and synchronise.
    template <int ST>
    __device__ __forceinline__ void iteration(int it)
    {
        const int t = tile_at(it);
        const bool has_next = it + 1 < n_t;
        if (has_next) fetch(it + 1, ST ^ 1);

        const int k0 = t * BN;
        const bool tile_empty = Mg && kv_lo == 0 && (BN <= 64 || kv_hi == 0);
        // A masked key's weight is exactly 0, but the product P.V would still
        // multiply it by the key's V row, and 0 * NaN or 0 * Inf is NaN:
        // padded cache slots may hold anything.  On tiles with hidden keys
        // (key-padding mask, or keys past N_k whose rows repeat the last
        // key), those V rows are cleared in LDS first, so hidden keys
        // contribute exactly zero whatever their values ("Pitfalls in
        // implementing the recurrence"; the interview answer: masked keys
        // contribute zero).  The mask is shared by all rows of the batch,
        // so every wave can use the cleared rows.
        if (Mg && !tile_empty && !(kv_lo == ~0ull && (BN <= 64 || kv_hi == ~0ull)))
            clear_hidden_v<ST>();
        // Keys beyond this wave's last row are all masked under causality;
        // a wave whose rows all lie past N_q has nothing to compute.
        const bool wave_skip = tile_empty || (CAUSAL && k0 > qw0 + 31) || qw0 >= Nq;
        if (!wave_skip) compute<ST>(k0);
        if (TRACE && trace_on) record(it, t);

        if (has_next) {
            land();
            if (Mg) take_mask();
        }
    }

    // Zero the V rows of the keys of the tile in stage ST that the
    // key-padding bits (kv_lo, kv_hi: visible and inside N_k) hide, then
    // synchronise.  Rows are whole in LDS (the swizzle only permutes the
    // 16-byte chunks inside a row).  Every thread of the workgroup calls it.
    template <int ST>
    __device__ __forceinline__ void clear_hidden_v()
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (int idx = threadIdx.x; idx < BN * C::CH; idx += C::T) {
            const int row = idx / C::CH, ch = idx % C::CH;
            const uint64_t word = row < 64 ? kv_lo : kv_hi;
            if (!((word >> (row & 63)) & 1ull))
                *reinterpret_cast<__attribute__((address_space(3))) u32x4 *>(
                    lds + C::V_BASE + ST * C::TILE + row * C::ROW + 16 * ch) = zero;
        }
        __syncthreads();
    }

    // Raw scores S^T = K . Q^T of the tile in stage ST ("The math of
    // FlashAttention", the tiled score block).
    template <int ST>
    __device__ __forceinline__ void qk(f32x16 (&s)[C::NKB]) const
    {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
        bf16x8 kfr[D / 16][C::NKB];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
                kfr[kk][kb] = *(const lds_bf16x8 *)(uintptr_t)(offk[kk] + ST * C::TILE +
                                                                kb * 32 * C::ROW);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[kk][kb], qf[kk], s[kb], 0, 0, 0);
        // Interleave the K-fragment reads with the products, PF reads ahead
        // of their use: a bounded number of live fragments, and the LDS
        // latency is hidden behind the matrix cores.
        {
            constexpr int NM = D / 16 * C::NKB, PF = C::LEAN ? NM / 4 : NM / 2;
            __builtin_amdgcn_sched_group_barrier(0x100, PF, 5);
#pragma unroll
            for (int i = 0; i < NM - PF; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 5);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 5);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, PF, 5);
        }
    }

    __device__ __forceinline__ void mask_scores(int k0, f32x16 (&s)[C::NKB]) const
    {
        // Masks go in before the tile maximum ("The math of FlashAttention",
        // "Pitfalls in implementing the recurrence").
        const bool kv_partial = Mg && !(kv_lo == ~0ull && (BN <= 64 || kv_hi == ~0ull));
        const bool tail = k0 + C::BNA > Nk || BN < 32;
        const bool diag = CAUSAL && (k0 + BN - 1 > qw0);
        if (kv_partial || tail || diag) {
            uint32_t vis[C::NKB];
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
                const int first = k0 + 32 * kb + 4 * h;  // key of kpos 0
                int lim = (BN < 32 ? k0 + BN : Nk) - first;
                if (BN < 32 && Nk - first < lim) lim = Nk - first;
                if (CAUSAL && qrow - first + 1 < lim) lim = qrow - first + 1;
                // keys sit at kpos 0-3, 8-11, 16-19, 24-27 of the lane's bit
                // word; the key at kpos k is visible iff k < lim.
                uint32_t bits = prefix_bits(lim);
                if (Mg) {
                    const uint64_t word = (kb < 2) ? kv_lo : kv_hi;
                    bits &= (uint32_t)(word >> (32 * (kb & 1) + 4 * h));
                }
                vis[kb] = bits;
            }
            apply_visibility<C::NKB>(s, vis);
        }
    }

    // V operand of P.V product i (k-step i / (D/32), dims 32*(i % (D/32)) ..
    // +31) from the tile in stage ST, through two transposing reads: within
    // a group of 16 lanes, lane j receives element j%4 of the 8-byte chunks
    // addressed by lanes 4m + j/4, so the operand holds exactly the keys the
    // score layout gives this lane's weights.
    template <int ST>
    __device__ __forceinline__ bf16x8 load_v(int i) const
    {
        const int t16 = i / (D / 32), db = i % (D / 32);
        const uint32_t row = offv[db] + ST * C::TILE + 16 * t16 * C::ROW;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)row);
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)(row + 8 * C::ROW));
        const s16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, av);
    }

    template <int ST>
    __device__ __forceinline__ void compute(int k0)
    {
        f32x16 s[C::NKB];
        qk<ST>(s);
        mask_scores(k0, s);
        // The V operands of the first VA products are read now, so that the
        // softmax below hides their LDS latency; the product loop then keeps
        // VA products' operands in flight.
        constexpr int NPV = C::NT16 * (D / 32);
        constexpr int VA_MAX = (C::NKB >= 4 || C::LEAN) ? 2 : 4;   // fewer where registers are short
        constexpr int VA = NPV < VA_MAX ? NPV : VA_MAX;
        bf16x8 vf[NPV];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < VA; ++i) vf[i] = load_v<ST>(i);
        bf16x8 pb[C::NT16];
        // Fast path: the weights against the current base, without the tile
        // maximum.  They are kept when every lane's sum of them is at most
        // kFastSumLimit, which bounds each weight too; the base stays where it
        // is and alpha is 1.  Otherwise (a score far above the base, or a row
        // with no base yet, whose weights come out +inf or NaN and fail the
        // test) the scores are formed again from the K tile, which is still
        // in LDS, and the step with the maximum runs.  The wave's first tile
        // has no base in any row, so it goes to that step directly.
        float tot = 0.0f;
        bool done = false;
        if (started) {
            float fs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
                    fs[r & 3] += s[kb][r];
                }
            tot = (fs[0] + fs[1]) + (fs[2] + fs[3]);
            done = !__any(!(tot <= kFastSumLimit));
            // the V reads first, then the vector work
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * VA, 9);
            __builtin_amdgcn_sched_group_barrier(0x406, 512, 9);
        }
        if (done) {
#pragma unroll
            for (int t16 = 0; t16 < C::NT16; ++t16)
#pragma unroll
                for (int i = 0; i < 8; ++i) pb[t16][i] = (__bf16)s[t16 >> 1][8 * (t16 & 1) + i];
            l_part += tot;
        } else if (started) {
            qk<ST>(s);
            mask_scores(k0, s);
        }
        started = true;
        float alpha;
        if (!done && lazy_step<C::NKB, C::NT16>(s, pb, mc, l_part, c, alpha)) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }

        // o~ += P . V as O^T += V^T . P^T.  k-step t16 covers keys 16*t16 ..
        // +15; this lane's 8 weights are registers 8*(t16%2) .. +7 of key
        // block t16/2, i.e. keys 16*t16 + 4h + {0..3, 8..11}.
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            if (i + VA < NPV) vf[i + VA] = load_v<ST>(i + VA);
            const int t16 = i / (D / 32), db = i % (D / 32);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pb[t16], o[db], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            if (i + VA < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 6);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 6);
        }
    }

    // The whole pass over one work item: state, the tile loop, the epilogue.
    __device__ __forceinline__ void run(const Params &p, lds_char *lds_base, int bh_, int qt,
                                        int split_)
    {
        init(p, lds_base, bh_, qt, split_);

        if (n_t > 0) fetch(0, 0);
        land();
        if (Mg) take_mask();

        for (int it = 0; it < n_t; it += 2) {
            iteration<0>(it);
            if (it + 1 < n_t) iteration<1>(it + 1);
        }
        epilogue(p);
    }

    // The reference of the row's state in raw score units: mc / c.
    __device__ __forceinline__ float m_raw() const { return mc == kNegInf ? kNegInf : mc / c; }

    // Trace entry `it`: {tile, m, l, 0} of the traced row after tile t.
    __device__ __forceinline__ void record(int it, int t)
    {
        const float l_row = pair_sum(l_part);
        if (qrow == trace_row && h == 0) {
            const f32x4 e = {(float)t, m_raw(), l_row, 0.0f};
            *reinterpret_cast<f32x4 *>(trace + 4 * (size_t)it) = e;
        }
    }

    // Split-key mode: the row's partial state over this key range.
    __device__ __forceinline__ void write_partial(const Params &p, float l_row)
    {
        const size_t row = (size_t)split * p.part_rows + (size_t)bh * Nq + qrow;
        float *Og = p.part_o + row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 x = {o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
                *reinterpret_cast<f32x4 *>(Og + 32 * db + 8 * g + 4 * h) = x;
            }
        if (h == 0) {
            p.part_m[row] = m_raw();
            p.part_l[row] = l_row;
        }
    }

    // o = o~ / l, lse = m + ln l; a row with no visible key gets o = 0 and
    // lse = -inf.
    __device__ __forceinline__ void epilogue(const Params &p)
    {
        const float l_row = pair_sum(l_part);
        const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
        if (qrow >= Nq) return;
        if (p.part_o) {
            write_partial(p, l_row);
            return;
        }
        uint16_t *Og = static_cast<uint16_t *>(p.o) + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const __bf16 x0 = (__bf16)(o[db][4 * g + 0] * inv);
                const __bf16 x1 = (__bf16)(o[db][4 * g + 1] * inv);
                const __bf16 x2 = (__bf16)(o[db][4 * g + 2] * inv);
                const __bf16 x3 = (__bf16)(o[db][4 * g + 3] * inv);
                u32x2 pk;
                pk[0] = (uint32_t)__builtin_bit_cast(uint16_t, x0) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
                pk[1] = (uint32_t)__builtin_bit_cast(uint16_t, x2) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, x3) << 16);
                *reinterpret_cast<u32x2 *>(Og + 32 * db + 8 * g + 4 * h) = pk;
            }
        if (h == 0)
            p.lse[(size_t)bh * Nq + qrow] =
                l_row > 0.0f ? (mc + __builtin_amdgcn_logf(l_row)) * kLn2 : kNegInf;
    }
};

template <int D, int BN, int NW, bool CAUSAL, bool TRACE>
__global__ __launch_bounds__(NW * 64, (bf16_blocks_per_cu<D, BN, NW>())) void fa_fwd_bf16_kernel(
    const Params p)
{
    extern __shared__ __attribute__((aligned(1024))) char lds_raw[];
    using F = Bf16Fwd<D, BN, NW, CAUSAL, TRACE>;
    F k;
    int bh, qt, split;
    F::work_item(p, 0, bh, qt, split);
    k.run(p, (lds_char *)lds_raw, bh, qt, split);
    // The second item of a pair, after a barrier: the first item's last tile
    // may still be read from LDS.  (Written out rather than as a loop, which
    // would keep the first item's registers live across both.)
    if (CAUSAL && F::work_item(p, 1, bh, qt, split)) {
        __syncthreads();
        k.run(p, (lds_char *)lds_raw, bh, qt, split);
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel: same recurrence with fp32 MFMA products and fp32 weights.  It
// exists for exact-input checks at fp32 precision; K and V keep the
// [key][dim] layout in LDS (the fp32 operands are one element per lane, so
// no transposition is needed), single-buffered.
// ---------------------------------------------------------------------------
template <int D, int BN, int NW>
struct F32Cfg {
    static constexpr int BM = 32 * NW;
    static constexpr int BNA = BN < 32 ? 32 : BN;
    static constexpr int NKB = BNA / 32;
    static constexpr int P = D + 4;                 // row pitch, floats
    static constexpr int K_ELEMS = BNA * P;
    static constexpr int T = NW * 64;
    static constexpr int CHUNKS = BN * D / 4;       // 16-byte chunks per matrix
    static constexpr int PER_T = (CHUNKS + T - 1) / T;
    static constexpr size_t LDS_BYTES = 2 * K_ELEMS * sizeof(float);
};

// One key tile of the fp32 kernel for the 32 query rows of a wave: scores,
// masks, the recurrence step (online_step) and the P.V products.
template <int D, int BN, int NW, bool CAUSAL>
__device__ __forceinline__ void f32_tile(const float *Kl, const float *Vl, const f32x4 (&qf)[D / 8],
                                         int k0, int Nk, int qw0, int qrow, int l31, int h,
                                         const uint8_t *Mg, uint64_t kv_lo, uint64_t kv_hi,
                                         float c, float &m_raw, float &l_part,
                                         f32x16 (&o)[D / 32])
{
    using C = F32Cfg<D, BN, NW>;
    f32x16 s[C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
    for (int g = 0; g < D / 8; ++g)
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(
                Kl + (32 * kb + l31) * C::P + 8 * g + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], qf[g][i], s[kb], 0, 0, 0);
        }

    const bool kv_partial = Mg && !(kv_lo == ~0ull && (BN <= 64 || kv_hi == ~0ull));
    const bool tail = k0 + C::BNA > Nk || BN < 32;
    const bool diag = CAUSAL && (k0 + BN - 1 > qw0);
    if (kv_partial || tail || diag) {
        uint32_t vis[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            const int first = k0 + 32 * kb + 4 * h;
            int lim = (BN < 32 ? k0 + BN : Nk) - first;
            if (BN < 32 && Nk - first < lim) lim = Nk - first;
            if (CAUSAL && qrow - first + 1 < lim) lim = qrow - first + 1;
            uint32_t bits = prefix_bits(lim);
            if (Mg) {
                const uint64_t word = (kb < 2) ? kv_lo : kv_hi;
                bits &= (uint32_t)(word >> (32 * (kb & 1) + 4 * h));
            }
            vis[kb] = bits;
        }
        apply_visibility<C::NKB>(s, vis);
    }

    const float alpha = online_step<C::NKB>(s, m_raw, l_part, c);
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }

    // O^T += V^T . P^T: the MFMA fed by weight register r contracts over
    // the two keys 32kb + kpos(r) (lanes 0-31) and 32kb + kpos(r) + 4
    // (lanes 32-63); the V operand of lane l is V[that key][32db + l%32].
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // keys 16..31 of a 16-key tile are phantoms (registers 8..15)
            if (BN < 32 && r >= 8) continue;
            const int key = 32 * kb + kpos(r) + 4 * h;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const float a = Vl[key * C::P + 32 * db + l31];
                o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kb][r], o[db], 0, 0, 0);
            }
        }
}

template <int D, int BN, int NW, bool CAUSAL, bool TRACE>
__global__ __launch_bounds__(NW * 64, 1) void fa_fwd_f32_kernel(const Params p)
{
    using C = F32Cfg<D, BN, NW>;
    extern __shared__ __attribute__((aligned(16))) float ldsf[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l31 = lane & 31;
    const int h = lane >> 5;

    // work item L = (head, query tile, key range), key ranges innermost
    const int L = logical_tile(blockIdx.x, gridDim.x, p.n_qt, p.n_split, CAUSAL,
                               p.cus / p.xcds * 2, p.xcds);
    const int split = L % p.n_split;
    const int L2 = L / p.n_split;
    const int bh = L2 / p.n_qt;
    const int qt = CAUSAL ? (p.n_qt - 1 - L2 % p.n_qt) : (L2 % p.n_qt);
    const int b = bh / p.H;
    const int q0 = qt * C::BM;
    const int qw0 = q0 + 32 * w;
    const int qrow = qw0 + l31;
    const int Nq = p.Nq, Nk = p.Nk;

    const float *Qg = static_cast<const float *>(p.q) + (size_t)bh * Nq * D;
    const float *Kg = static_cast<const float *>(p.k) + (size_t)bh * Nk * D;
    const float *Vg = static_cast<const float *>(p.v) + (size_t)bh * Nk * D;
    const uint8_t *Mg = p.mask ? p.mask + (size_t)b * Nk : nullptr;

    // Q fragments: the 4 MFMAs of group g contract dims 8g + 4h + i (i = 0..3)
    // on this lane, for both operands.
    f32x4 qf[D / 8];
    {
        const int qr = qrow < Nq ? qrow : Nq - 1;
#pragma unroll
        for (int g = 0; g < D / 8; ++g)
            qf[g] = *reinterpret_cast<const f32x4 *>(Qg + (size_t)qr * D + 8 * g + 4 * h);
    }

    // Key tiles the query tile needs, and this workgroup's range of them.
    int n_all = (Nk + BN - 1) / BN;
    if (CAUSAL) {
        const int last_q = (q0 + C::BM < Nq ? q0 + C::BM : Nq) - 1;
        const int need = last_q / BN + 1;
        n_all = need < n_all ? need : n_all;
    }
    int t_lo = (int)((int64_t)split * n_all / p.n_split);
    int n_t = (int)((int64_t)(split + 1) * n_all / p.n_split) - t_lo;
    trim_to_visible<BN, C::T>(Mg, Nk, t_lo, n_t);
    const bool trace_on = TRACE && bh == p.trace_bh && p.trace_row >= qw0 && p.trace_row < qw0 + 32;

    float *Kl = ldsf;
    float *Vl = ldsf + C::K_ELEMS;
    f32x4 kreg[C::PER_T], vreg[C::PER_T];

    auto load_tile = [&](int t) {
        const int k0 = t * BN;
#pragma unroll
        for (int i = 0; i < C::PER_T; ++i) {
            const int ch = tid + i * C::T;
            if (C::CHUNKS % C::T == 0 || ch < C::CHUNKS) {
                const int row = ch / (D / 4), col = ch % (D / 4);
                int kr = k0 + row;
                kr = kr < Nk ? kr : Nk - 1;
                kreg[i] = *reinterpret_cast<const f32x4 *>(Kg + (size_t)kr * D + 4 * col);
                vreg[i] = *reinterpret_cast<const f32x4 *>(Vg + (size_t)kr * D + 4 * col);
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < C::PER_T; ++i) {
            const int ch = tid + i * C::T;
            if (C::CHUNKS % C::T == 0 || ch < C::CHUNKS) {
                const int row = ch / (D / 4), col = ch % (D / 4);
                *reinterpret_cast<f32x4 *>(Kl + row * C::P + 4 * col) = kreg[i];
                *reinterpret_cast<f32x4 *>(Vl + row * C::P + 4 * col) = vreg[i];
            }
        }
    };

    float m_raw = kNegInf, l_part = 0.0f;
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;

    const float c = p.c;

    // Phantom keys of a 16-key tile (rows 16..31 of the 32-row block) are
    // never written; zero them once so the P.V products read finite values.
    if (BN < 32) {
        for (int x = tid; x < (C::BNA - BN) * C::P; x += C::T) {
            Kl[BN * C::P + x] = 0.0f;
            Vl[BN * C::P + x] = 0.0f;
        }
    }

    if (n_t > 0) load_tile(t_lo + (p.reverse ? n_t - 1 : 0));

    for (int it = 0; it < n_t; ++it) {
        const int t = t_lo + (p.reverse ? (n_t - 1 - it) : it);
        __syncthreads();   // every wave is done with the previous tile
        store_tile();
        __syncthreads();
        if (it + 1 < n_t) load_tile(t_lo + (p.reverse ? (n_t - 2 - it) : (it + 1)));

        const int k0 = t * BN;
        uint64_t kv_lo = ~0ull, kv_hi = ~0ull;
        if (Mg) {
            const int j0 = k0 + lane;
            const bool v0 = lane < BN && j0 < Nk && Mg[j0] != 0;
            kv_lo = __ballot(v0);
            if (BN > 64) {
                const int j1 = j0 + 64;
                const bool v1 = lane + 64 < BN && j1 < Nk && Mg[j1] != 0;
                kv_hi = __ballot(v1);
            }
        }
        const bool tile_empty = Mg && kv_lo == 0 && (BN <= 64 || kv_hi == 0);
        // V rows of hidden keys are cleared before the products, so that
        // their zero weights never meet non-finite values (as in the bf16
        // kernel).
        if (Mg && !tile_empty && !(kv_lo == ~0ull && (BN <= 64 || kv_hi == ~0ull))) {
            for (int x = tid; x < BN * D; x += C::T) {
                const int row = x / D;
                const uint64_t word = row < 64 ? kv_lo : kv_hi;
                if (!((word >> (row & 63)) & 1ull)) Vl[row * C::P + x % D] = 0.0f;
            }
            __syncthreads();
        }
        if (!(tile_empty || (CAUSAL && k0 > qw0 + 31) || qw0 >= Nq))
            f32_tile<D, BN, NW, CAUSAL>(Kl, Vl, qf, k0, Nk, qw0, qrow, l31, h, Mg, kv_lo, kv_hi, c,
                                        m_raw, l_part, o);
        if (TRACE && trace_on) {
            // trace entry it: {tile, m, l, 0} of the traced row after tile t
            const float l_row = pair_sum(l_part);
            if (qrow == p.trace_row && h == 0) {
                const f32x4 e = {(float)t, m_raw, l_row, 0.0f};
                *reinterpret_cast<f32x4 *>(p.trace + 4 * (size_t)it) = e;
            }
        }
    }

    const float l_row = pair_sum(l_part);
    if (qrow >= Nq) return;
    if (p.part_o) {
        // split-key mode: the row's partial state over this key range
        const size_t row = (size_t)split * p.part_rows + (size_t)bh * Nq + qrow;
        float *Og = p.part_o + row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 x = {o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
                *reinterpret_cast<f32x4 *>(Og + 32 * db + 8 * g + 4 * h) = x;
            }
        if (h == 0) {
            p.part_m[row] = m_raw;
            p.part_l[row] = l_row;
        }
        return;
    }
    const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
    {
        float *Og = static_cast<float *>(p.o) + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x;
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = o[db][4 * g + i] * inv;
                *reinterpret_cast<f32x4 *>(Og + 32 * db + 8 * g + 4 * h) = x;
            }
        if (h == 0)
            p.lse[(size_t)bh * Nq + qrow] =
                l_row > 0.0f ? __builtin_fmaf(m_raw, p.scale, __builtin_amdgcn_logf(l_row) * kLn2)
                             : kNegInf;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, int BN, int NW, bool CAUSAL, bool TRACE, bool BF16>
static hipError_t launch_instance(int grid, int threads, size_t lds, hipStream_t stream,
                                  const Params &p)
{
    static std::atomic<uint64_t> done{0};
    void (*fn)(Params);
    if constexpr (BF16)
        fn = fa_fwd_bf16_kernel<D, BN, NW, CAUSAL, TRACE>;
    else
        fn = fa_fwd_f32_kernel<D, BN, NW, CAUSAL, TRACE>;
    return launch(reinterpret_cast<const void *>(fn), fn, done, grid, threads, lds, stream, p);
}

// The four (causal, trace) variants of one kernel configuration.
template <int D, int BN, int NW, bool BF16>
static hipError_t launch_variant(int causal, int grid, int threads, size_t lds,
                                 hipStream_t stream, const Params &p)
{
    const bool trace = p.trace != nullptr;
    if (causal)
        return trace ? launch_instance<D, BN, NW, true, true, BF16>(grid, threads, lds, stream, p)
                     : launch_instance<D, BN, NW, true, false, BF16>(grid, threads, lds, stream, p);
    return trace ? launch_instance<D, BN, NW, false, true, BF16>(grid, threads, lds, stream, p)
                 : launch_instance<D, BN, NW, false, false, BF16>(grid, threads, lds, stream, p);
}

template <int D, int BN, int NW>
static hipError_t dispatch_bf16_nw(const Params &p0, int causal, int B, int H, hipStream_t stream)
{
    using C = Bf16Cfg<D, BN, NW>;
    Params p = p0;
    p.n_qt = (p.Nq + C::BM - 1) / C::BM;
    // Under causality the query tiles of a head differ in length (tile t
    // visits t + 1 times the keys of tile 0); paired as (t, n_qt - 1 - t)
    // they make workgroups of one length, which finish together when they
    // fill whole rounds of the device's workgroup slots.  Otherwise (or when
    // a round would be only partly full) the items go singly, longest first.
    const int64_t pairs = (int64_t)B * H * ((p.n_qt + 1) / 2);
    const int64_t slots = (int64_t)p.cus * bf16_blocks_per_cu<D, BN, NW>();
    p.pair = causal && p.n_split == 1 && p.n_qt >= 2 && pairs % slots == 0;
    const int grid = p.pair ? (int)pairs : B * H * p.n_qt * p.n_split;
    return launch_variant<D, BN, NW, true>(causal, grid, C::T, C::LDS_BYTES, stream, p);
}

template <int D, int BN>
static hipError_t dispatch_bf16(const Params &p, int causal, int B, int H, hipStream_t stream)
{
    if constexpr (D == 128 && BN == 64) {
        if (bf16_waves(D, BN, B, H, p.Nq, causal != 0, p.n_split, p.cus) == 8)
            return dispatch_bf16_nw<D, BN, 8>(p, causal, B, H, stream);
    }
    return dispatch_bf16_nw<D, BN, 4>(p, causal, B, H, stream);
}

template <int D, int BN>
static hipError_t dispatch_f32(const Params &p0, int causal, int B, int H, hipStream_t stream)
{
    constexpr int NW = 4;
    using C = F32Cfg<D, BN, NW>;
    Params p = p0;
    p.n_qt = (p.Nq + C::BM - 1) / C::BM;
    const int grid = B * H * p.n_qt * p.n_split;
    return launch_variant<D, BN, NW, false>(causal, grid, C::T, C::LDS_BYTES, stream, p);
}

template <int D>
static hipError_t dispatch_d(const Params &p, int dtype, int block_n, int causal, int B, int H,
                             hipStream_t s)
{
    if (dtype == 1) {
        switch (block_n) {
        case 16: return dispatch_bf16<D, 16>(p, causal, B, H, s);
        case 32: return dispatch_bf16<D, 32>(p, causal, B, H, s);
        case 128: return dispatch_bf16<D, 128>(p, causal, B, H, s);
        default: return dispatch_bf16<D, 64>(p, causal, B, H, s);
        }
    }
    switch (block_n) {
    case 16: return dispatch_f32<D, 16>(p, causal, B, H, s);
    case 32: return dispatch_f32<D, 32>(p, causal, B, H, s);
    case 128: return dispatch_f32<D, 128>(p, causal, B, H, s);
    default: return dispatch_f32<D, 64>(p, causal, B, H, s);
    }
}

int query_tile_rows(int dtype, int d, int block_n, int B, int H, int n_q, int causal, int n_split,
                    int cus)
{
    return dtype == 1 ? 32 * bf16_waves(d, block_n, B, H, n_q, causal != 0, n_split, cus) : 32 * 4;
}

hipError_t launch_fwd(const Params &p, int dtype, int d, int block_n, int causal, int B, int H,
                      hipStream_t stream)
{
    if (d == 64) return dispatch_d<64>(p, dtype, block_n, causal, B, H, stream);
    return dispatch_d<128>(p, dtype, block_n, causal, B, H, stream);
}

// ---------------------------------------------------------------------------
// Merge of partial states.  Every state of a row is rewritten to the common
// reference M = max_i m_i by the rescaling identity -- l_i and acc_i times
// exp(scale * (m_i - M)) <= 1 -- and the rewritten sums add ("The math of
// FlashAttention", "The rescaling identity, derived"; "Proof of exactness":
// the order of the key ranges does not matter).  Then o = acc / l and
// lse = M * scale + ln l; o = 0 and lse = -inf when no part saw a visible key.
//
// D/4 threads per row, each owning 4 consecutive columns: the m and l reads
// of a row are the same addresses for all of its threads (one cache line),
// the acc reads and the o writes are 16 bytes per lane and contiguous across
// the row.  Parts are loaded 8 at a time so that few memory round trips
// remain when there are few rows (decoding); with many rows the kernel is
// bound by reading acc once.
// ---------------------------------------------------------------------------
struct MergeParams {
    const float *m;
    const float *l;
    const float *acc;
    void *o;
    float *lse;
    int64_t rows;
    int n_parts;
    float c;        // scale * log2(e)
    float scale;
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_merge_kernel(const MergeParams p)
{
    constexpr int TPR = D / 4;          // threads per row
    constexpr int RPB = 256 / TPR;      // rows per workgroup pass
    constexpr int CHUNK = 8;            // parts loaded together (one memory round trip)
    const int j = 4 * (threadIdx.x % TPR);
    for (int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR; row < p.rows;
         row += (int64_t)gridDim.x * RPB) {
        // The states are folded in CHUNK at a time with the recurrence itself:
        // the running reference M moves to the chunk's maximum when that is
        // larger, and what was accumulated is rescaled by exp(M_old - M_new).
        float big_m = kNegInf, l = 0.0f;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int i0 = 0; i0 < p.n_parts; i0 += CHUNK) {
            float mi[CHUNK], li[CHUNK];
            f32x4 ai[CHUNK];
#pragma unroll
            for (int u = 0; u < CHUNK; ++u) {
                mi[u] = kNegInf;
                if (i0 + u < p.n_parts) {
                    const size_t pr = (size_t)(i0 + u) * p.rows + row;
                    mi[u] = p.m[pr];
                    li[u] = p.l[pr];
                    ai[u] = *reinterpret_cast<const f32x4 *>(p.acc + pr * D + j);
                }
            }
            float cm = kNegInf;
#pragma unroll
            for (int u = 0; u < CHUNK; ++u) cm = fmaxf(cm, mi[u]);
            if (cm == kNegInf) continue;              // no visible key in this chunk
            if (cm > big_m) {
                const float alpha = big_m == kNegInf ? 0.0f
                                                     : __builtin_amdgcn_exp2f((big_m - cm) * p.c);
                l *= alpha;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] *= alpha;
                big_m = cm;
            }
#pragma unroll
            for (int u = 0; u < CHUNK; ++u) {
                if (mi[u] == kNegInf) continue;       // l and acc of such a part are ignored
                const float w = __builtin_amdgcn_exp2f((mi[u] - big_m) * p.c);
                l = __builtin_fmaf(w, li[u], l);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, ai[u][e], acc[e]);
            }
        }
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        if (BF16) {
            u32x2 pk;
            pk[0] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[0] * inv)) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[1] * inv)) << 16);
            pk[1] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[2] * inv)) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[3] * inv)) << 16);
            *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p.o) + (size_t)row * D + j) = pk;
        } else {
            const f32x4 x = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
            *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + (size_t)row * D + j) = x;
        }
        if (j == 0)
            p.lse[row] = l > 0.0f ? __builtin_fmaf(big_m, p.scale, __builtin_amdgcn_logf(l) * kLn2)
                                  : kNegInf;
    }
}

template <int D, bool BF16>
static hipError_t launch_merge_d(const MergeParams &p, hipStream_t stream)
{
    constexpr int RPB = 256 / (D / 4);
    const int64_t want = (p.rows + RPB - 1) / RPB;
    const int grid = (int)(want < 65536 ? want : 65536);
    void (*fn)(MergeParams) = fa_merge_kernel<D, BF16>;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_merge(const float *m, const float *l, const float *acc, int n_parts,
                        int64_t rows, int d, float scale, void *o, float *lse, int dtype,
                        hipStream_t stream)
{
    MergeParams p;
    p.m = m;
    p.l = l;
    p.acc = acc;
    p.o = o;
    p.lse = lse;
    p.rows = rows;
    p.n_parts = n_parts;
    p.c = (float)((double)scale * 1.4426950408889634073599);   // as the forward kernels
    p.scale = scale;
    if (d == 64)
        return dtype == 1 ? launch_merge_d<64, true>(p, stream) : launch_merge_d<64, false>(p, stream);
    return dtype == 1 ? launch_merge_d<128, true>(p, stream) : launch_merge_d<128, false>(p, stream);
}

}  // namespace fa
