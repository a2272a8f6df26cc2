// fa_api.cpp -- the C entry points of libfa.so: argument checks, device
// check, and the launch.  The operation and its conventions are documented in
// include/fa.h.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "fa.h"
#include "fa_internal.h"

namespace {

thread_local char g_msg[512];
thread_local hipError_t g_last_hip = hipSuccess;

// gfx950 check, cached per device: 0 = unknown, 1 = gfx950, 2 = other.
std::atomic<int> g_dev_kind[64];

int check_device()
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip = e;
        return FA_ERR_DEVICE;
    }
    if (dev < 0 || dev >= 64) return FA_ERR_DEVICE;
    int kind = g_dev_kind[dev].load(std::memory_order_acquire);
    if (kind == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            g_last_hip = e;
            return FA_ERR_DEVICE;
        }
        kind = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_dev_kind[dev].store(kind, std::memory_order_release);
    }
    return kind == 1 ? FA_OK : FA_ERR_DEVICE;
}

// Compute units and XCDs per device, queried once: 0 = not yet known.
std::atomic<int> g_dev_cus[64];
std::atomic<int> g_dev_xcds[64];

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// Sizes of the buffers of one forward call, after validation.
struct Sizes {
    size_t qb, kb, lb, mb;   // bytes of q (and o), k (and v), lse, mask
    int64_t rows;            // B * H * N_q
};

// Checks shared by the forward entry points, in the documented order.
// The decoding pass addresses a head's K and V with 32-bit byte offsets.
bool decode_fits(int N_k, int d) { return (int64_t)N_k * d * 2 < ((int64_t)1 << 31); }

bool misaligned(const void *ptr, uintptr_t bytes)
{
    return (reinterpret_cast<uintptr_t>(ptr) & (bytes - 1)) != 0;
}

int check_fwd_args(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                   int H, int N_q, int N_k, int d, float scale, const uint8_t *kv_len_mask,
                   int dtype, int n_split, Sizes &sz)
{
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || N_q <= 0 || N_k <= 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
    // The kernels move q, k, v and o in 16-byte vectors and lse in words.
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(lse, 4))
        return FA_ERR_ALIGN;

    // Index space: every element offset must fit in int64, and the grid
    // (B*H*ceil(N_q/32)*n_split workgroups at most) in int32.
    const int64_t bh = (int64_t)B * H;
    if (bh > (int64_t)1 << 31 || (double)bh * N_q * d > 9.0e18 || (double)bh * N_k * d > 9.0e18)
        return FA_ERR_SHAPE;
    if ((double)bh * (((int64_t)N_q + 31) / 32) * n_split > (double)INT32_MAX) return FA_ERR_SHAPE;

    const size_t esz = dtype == FA_DTYPE_BF16 ? 2 : 4;
    sz.qb = (size_t)(bh * N_q * d) * esz;
    sz.kb = (size_t)(bh * N_k * d) * esz;
    sz.lb = (size_t)bh * N_q * sizeof(float);
    sz.mb = kv_len_mask ? (size_t)B * N_k : 0;
    sz.rows = bh * N_q;
    const void *ins[4] = {q, k, v, kv_len_mask};
    const size_t in_bytes[4] = {sz.qb, sz.kb, sz.kb, sz.mb};
    for (int i = 0; i < 4; ++i)
        if (overlaps(o, sz.qb, ins[i], in_bytes[i]) || overlaps(lse, sz.lb, ins[i], in_bytes[i]))
            return FA_ERR_ALIAS;
    if (overlaps(o, sz.qb, lse, sz.lb)) return FA_ERR_ALIAS;
    return FA_OK;
}

// True if [p, p + n) overlaps any buffer of a forward call.
bool overlaps_fwd(const void *p, size_t n, const void *q, const void *k, const void *v,
                  const void *o, const float *lse, const uint8_t *mask, const Sizes &sz)
{
    return overlaps(p, n, q, sz.qb) || overlaps(p, n, k, sz.kb) || overlaps(p, n, v, sz.kb) ||
           overlaps(p, n, o, sz.qb) || overlaps(p, n, lse, sz.lb) || overlaps(p, n, mask, sz.mb);
}

fa::Params make_params(const void *q, const void *k, const void *v, void *o, float *lse, int H,
                       int N_q, int N_k, float scale, const uint8_t *kv_len_mask)
{
    fa::Params p;
    std::memset(&p, 0, sizeof p);
    fa::device_geometry(p.cus, p.xcds);
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.mask = kv_len_mask;
    p.H = H;
    p.Nq = N_q;
    p.Nk = N_k;
    p.c = (float)((double)scale * 1.4426950408889634073599);
    p.scale = scale;
    p.n_split = 1;
    return p;
}

int launch_status(hipError_t e)
{
    if (e != hipSuccess) {
        g_last_hip = e;
        return FA_ERR_LAUNCH;
    }
    return FA_OK;
}

constexpr int kMaxSplits = 256;
constexpr int kSplitBlockN = 64;

// Byte offset of acc in a split-key workspace, and its total size; false if
// the sizes overflow.
bool splitkv_layout(int64_t rows, int d, int num_splits, size_t &acc_off, size_t &total)
{
    const double bytes = (double)num_splits * rows * (d + 2) * sizeof(float) + 256.0;
    if (bytes > 9.0e18) return false;
    const size_t ml = (size_t)num_splits * rows * 2 * sizeof(float);
    acc_off = (ml + 255) & ~(size_t)255;
    total = acc_off + (size_t)num_splits * rows * d * sizeof(float);
    return true;
}

int fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
             int N_q, int N_k, int d, float scale, int causal, const uint8_t *kv_len_mask,
             int dtype, void *stream, const fa_opts *opts)
{
    Sizes sz;
    int rc = check_fwd_args(q, k, v, o, lse, B, H, N_q, N_k, d, scale, kv_len_mask, dtype, 1, sz);
    if (rc != FA_OK) return rc;

    int block_n = opts ? opts->block_n : 0;
    if (block_n != 0 && block_n != 16 && block_n != 32 && block_n != 64 && block_n != 128)
        return FA_ERR_TILE;
    if (block_n == 0) block_n = 64;

    float *trace = opts ? opts->trace : nullptr;
    if (trace) {
        if (opts->trace_b < 0 || opts->trace_b >= B || opts->trace_h < 0 || opts->trace_h >= H ||
            opts->trace_row < 0 || opts->trace_row >= N_q)
            return FA_ERR_ARG;
        const size_t tb = (size_t)((N_k + block_n - 1) / block_n) * 4 * sizeof(float);
        if (overlaps_fwd(trace, tb, q, k, v, o, lse, kv_len_mask, sz)) return FA_ERR_ALIAS;
        if (misaligned(trace, 16)) return FA_ERR_ALIGN;   // one 16-byte entry per tile
    }

    rc = check_device();
    if (rc != FA_OK) return rc;

    fa::Params p = make_params(q, k, v, o, lse, H, N_q, N_k, scale, kv_len_mask);
    p.reverse = (opts && opts->reverse_kv) ? 1 : 0;
    // One query row per (batch, head) in bf16, with the library's tile and
    // order and no trace: the decoding pass, all keys in one workgroup.
    if (dtype == FA_DTYPE_BF16 && N_q == 1 && !trace && !p.reverse &&
        (!opts || opts->block_n == 0) && decode_fits(N_k, d))
        return launch_status(fa::launch_decode(p, d, causal ? 1 : 0, B, H,
                                               static_cast<hipStream_t>(stream)));
    if (trace) {
        p.trace = trace;
        p.trace_bh = opts->trace_b * H + opts->trace_h;
        p.trace_row = opts->trace_row;
    }
    return launch_status(fa::launch_fwd(p, dtype, d, block_n, causal ? 1 : 0, B, H,
                                        static_cast<hipStream_t>(stream)));
}

// fa_fwd_splitkv and fa_fwd_splitkv_noalloc: the partial states go to the
// caller's workspace, or (use_scratch) to the library's own device scratch,
// whose address is looked up once per device and which is never allocated
// here.
int splitkv_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                 int N_q, int N_k, int d, float scale, int causal, const uint8_t *kv_len_mask,
                 int dtype, int num_splits, void *workspace, size_t workspace_bytes,
                 bool use_scratch, void *stream)
{
    Sizes sz;
    const int ns = (num_splits >= 1 && num_splits <= kMaxSplits) ? num_splits : 1;
    int rc = check_fwd_args(q, k, v, o, lse, B, H, N_q, N_k, d, scale, kv_len_mask, dtype, ns, sz);
    if (rc != FA_OK) return rc;
    if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_ARG;
    size_t acc_off = 0, total = 0;
    if (!splitkv_layout(sz.rows, d, num_splits, acc_off, total)) return FA_ERR_SHAPE;
    if (use_scratch) {
        if (total > fa::kScratchBytes) return FA_ERR_SCRATCH;
    } else {
        if (!workspace || workspace_bytes < total ||
            (reinterpret_cast<uintptr_t>(workspace) & 15))
            return FA_ERR_WORKSPACE;
        if (overlaps_fwd(workspace, total, q, k, v, o, lse, kv_len_mask, sz)) return FA_ERR_ALIAS;
    }

    rc = check_device();
    if (rc != FA_OK) return rc;
    if (use_scratch) {
        const hipError_t e = fa::scratch_address(&workspace);
        if (e != hipSuccess) {
            g_last_hip = e;
            return FA_ERR_DEVICE;
        }
    }

    fa::Params p = make_params(q, k, v, o, lse, H, N_q, N_k, scale, kv_len_mask);
    float *ws = static_cast<float *>(workspace);
    p.n_split = num_splits;
    p.part_rows = sz.rows;
    p.part_m = ws;
    p.part_l = ws + (size_t)num_splits * sz.rows;
    p.part_o = reinterpret_cast<float *>(static_cast<char *>(workspace) + acc_off);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // One query row per (batch, head) in bf16: the decoding pass, which streams
    // K and V through registers (its offsets within a head are 32-bit);
    // otherwise the forward kernel in split mode.  Both write every part of
    // every row, so nothing in the workspace needs clearing first.
    if (dtype == FA_DTYPE_BF16 && N_q == 1 && decode_fits(N_k, d))
        rc = launch_status(fa::launch_decode(p, d, causal ? 1 : 0, B, H, st));
    else
        rc = launch_status(fa::launch_fwd(p, dtype, d, kSplitBlockN, causal ? 1 : 0, B, H, st));
    if (rc != FA_OK) return rc;
    return launch_status(fa::launch_merge(p.part_m, p.part_l, p.part_o, num_splits, sz.rows, d,
                                          scale, o, lse, dtype, st));
}

}  // namespace

namespace fa {

void device_geometry(int &cus, int &xcds)
{
    cus = 256;
    xcds = 8;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return;
    int c = g_dev_cus[dev].load(std::memory_order_acquire);
    int x = g_dev_xcds[dev].load(std::memory_order_acquire);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            c = 256;
        if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x <= 0)
            x = 1;
        // The grid mapping deals workgroups to XCDs in turn; an XCD count it
        // cannot use that way (not a power of two, or not dividing the CUs
        // evenly) falls back to the plain order of one.
        if ((x & (x - 1)) != 0 || c % x != 0) x = 1;
        g_dev_xcds[dev].store(x, std::memory_order_release);
        g_dev_cus[dev].store(c, std::memory_order_release);
    }
    cus = c;
    xcds = x;
}

}  // namespace fa

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
           int N_q, int N_k, int d, float scale, int causal, const uint8_t *kv_len_mask,
           int dtype, void *stream)
{
    return fwd_impl(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask, dtype,
                    stream, nullptr);
}

int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
              int N_q, int N_k, int d, float scale, int causal, const uint8_t *kv_len_mask,
              int dtype, void *stream, const fa_opts *opts)
{
    return fwd_impl(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask, dtype,
                    stream, opts);
}

size_t fa_splitkv_workspace_bytes(int B, int H, int N_q, int d, int num_splits)
{
    if (B <= 0 || H <= 0 || N_q <= 0 || (d != 64 && d != 128) || num_splits < 1 ||
        num_splits > kMaxSplits)
        return 0;
    size_t acc_off = 0, total = 0;
    if (!splitkv_layout((int64_t)B * H * N_q, d, num_splits, acc_off, total)) return 0;
    return total;
}

int fa_query_tile_rows(int dtype, int B, int H, int N_q, int d, int block_n, int causal)
{
    if (B <= 0 || H <= 0 || N_q <= 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
    if (block_n != 0 && block_n != 16 && block_n != 32 && block_n != 64 && block_n != 128)
        return FA_ERR_TILE;
    int cus = 256, xcds = 8;
    fa::device_geometry(cus, xcds);
    return fa::query_tile_rows(dtype, d, block_n == 0 ? 64 : block_n, B, H, N_q, causal ? 1 : 0, 1,
                               cus);
}

int fa_splitkv_splits(int B, int H, int N_q, int N_k, int d, int causal)
{
    if (B <= 0 || H <= 0 || N_q <= 0 || N_k <= 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    int rc = check_device();
    if (rc != FA_OK) return rc;
    int cus = 256, xcds = 8;
    fa::device_geometry(cus, xcds);
    // Four workgroups per compute unit keep every unit busy with work queued
    // behind the resident ones (query tiles of the bf16 kernel).
    const double target = 4.0 * cus;
    const int64_t bm =
        fa::query_tile_rows(FA_DTYPE_BF16, d, kSplitBlockN, B, H, N_q, causal ? 1 : 0, 1, cus);
    const double wgs = (double)B * H * (((int64_t)N_q + bm - 1) / bm);
    if (wgs >= target) return 1;
    const int64_t keys = causal ? (N_q < N_k ? N_q : N_k) : N_k;
    const int64_t tiles = (keys + kSplitBlockN - 1) / kSplitBlockN;
    int64_t s = (int64_t)std::ceil(target / wgs);
    const int64_t by_tiles = tiles / 4 > 1 ? tiles / 4 : 1;   // at least 4 tiles per range
    if (s > by_tiles) s = by_tiles;
    if (s > kMaxSplits) s = kMaxSplits;
    return (int)(s < 1 ? 1 : s);
}

int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                   int H, int N_q, int N_k, int d, float scale, int causal,
                   const uint8_t *kv_len_mask, int dtype, int num_splits, void *workspace,
                   size_t workspace_bytes, void *stream)
{
    return splitkv_impl(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask, dtype,
                        num_splits, workspace, workspace_bytes, false, stream);
}

int fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int N_q, int N_k, int d, float scale, int causal,
                           const uint8_t *kv_len_mask, int dtype, int num_splits, void *stream)
{
    return splitkv_impl(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask, dtype,
                        num_splits, nullptr, 0, true, stream);
}

int fa_merge_states(const float *m, const float *l, const float *acc, int n_parts, int64_t rows,
                    int d, float scale, void *o, float *lse, int dtype, void *stream)
{
    if (!m || !l || !acc || !o || !lse) return FA_ERR_NULL;
    if (rows <= 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
    if (misaligned(acc, 16) || misaligned(o, 16) || misaligned(m, 4) || misaligned(l, 4) ||
        misaligned(lse, 4))
        return FA_ERR_ALIGN;
    if (n_parts < 1) return FA_ERR_ARG;
    if ((double)n_parts * rows * d * sizeof(float) > 9.0e18) return FA_ERR_SHAPE;
    const size_t mlb = (size_t)n_parts * rows * sizeof(float);
    const size_t ab = mlb * d;
    const size_t ob = (size_t)rows * d * (dtype == FA_DTYPE_BF16 ? 2 : 4);
    const size_t lb = (size_t)rows * sizeof(float);
    if (overlaps(o, ob, m, mlb) || overlaps(o, ob, l, mlb) || overlaps(o, ob, acc, ab) ||
        overlaps(lse, lb, m, mlb) || overlaps(lse, lb, l, mlb) || overlaps(lse, lb, acc, ab) ||
        overlaps(o, ob, lse, lb))
        return FA_ERR_ALIAS;
    int rc = check_device();
    if (rc != FA_OK) return rc;
    return launch_status(fa::launch_merge(m, l, acc, n_parts, rows, d, scale, o, lse, dtype,
                                          static_cast<hipStream_t>(stream)));
}

int fa_softmax_rows(const void *s, void *p, float *m, float *l, int64_t rows, int64_t n,
                    int dtype, void *stream)
{
    if (!s || !p) return FA_ERR_NULL;
    if (rows <= 0 || n <= 0) return FA_ERR_SHAPE;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
    const size_t esz = dtype == FA_DTYPE_BF16 ? 2 : 4;
    if ((double)rows * n * esz > 9.0e18) return FA_ERR_SHAPE;
    if (misaligned(s, esz) || misaligned(p, esz) || misaligned(m, 4) || misaligned(l, 4))
        return FA_ERR_ALIGN;
    const size_t sb = (size_t)rows * n * esz, vb = (size_t)rows * sizeof(float);
    if (p != s && overlaps(p, sb, s, sb)) return FA_ERR_ALIAS;
    const void *bufs[2] = {s, p};
    for (int i = 0; i < 2; ++i)
        if (overlaps(m, vb, bufs[i], sb) || overlaps(l, vb, bufs[i], sb)) return FA_ERR_ALIAS;
    if (overlaps(m, vb, l, vb)) return FA_ERR_ALIAS;
    int rc = check_device();
    if (rc != FA_OK) return rc;
    return launch_status(fa::launch_softmax_rows(s, p, m, l, rows, n, dtype,
                                                 static_cast<hipStream_t>(stream)));
}

const char *fa_strerror(int code)
{
    const char *base;
    switch (code) {
    case FA_OK: base = "success"; break;
    case FA_ERR_NULL: base = "a required pointer is NULL"; break;
    case FA_ERR_SHAPE: base = "B, H, N_q or N_k is not positive, or the sizes overflow"; break;
    case FA_ERR_HEAD_DIM: base = "head width d must be 64 or 128"; break;
    case FA_ERR_DTYPE: base = "dtype must be FA_DTYPE_F32 or FA_DTYPE_BF16"; break;
    case FA_ERR_SCALE: base = "scale must be finite and positive"; break;
    case FA_ERR_TILE: base = "block_n must be 0, 16, 32, 64 or 128"; break;
    case FA_ERR_DEVICE: base = "the current HIP device is not a gfx950 GPU"; break;
    case FA_ERR_LAUNCH: base = "HIP rejected the kernel launch"; break;
    case FA_ERR_ALIAS: base = "an output overlaps an input or another output"; break;
    case FA_ERR_ARG:
        base = "argument out of range (traced row, num_splits or n_parts)";
        break;
    case FA_ERR_WORKSPACE:
        base = "workspace is NULL, not 16-byte aligned, or smaller than required";
        break;
    case FA_ERR_ALIGN:
        base = "q, k, v, o, acc or the trace is not 16-byte aligned, or lse, m or l not 4-byte";
        break;
    case FA_ERR_SCRATCH:
        base = "the partial states exceed the library's device scratch (32 MiB per GPU); "
               "use fa_fwd_splitkv with a workspace, or fewer splits";
        break;
    default: base = "unknown status code"; break;
    }
    if ((code == FA_ERR_LAUNCH || code == FA_ERR_DEVICE) && g_last_hip != hipSuccess) {
        std::snprintf(g_msg, sizeof g_msg, "%s (HIP: %s)", base, hipGetErrorString(g_last_hip));
        return g_msg;
    }
    return base;
}

}  // extern "C"
