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

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

int fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
             int N_q, int N_k, int d, float scale, int causal, const uint8_t *kv_len_mask,
             int dtype, void *stream, const fa_opts *opts)
{
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || N_q <= 0 || N_k <= 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;

    int block_n = opts ? opts->block_n : 0;
    if (block_n != 0 && block_n != 16 && block_n != 32 && block_n != 64 && block_n != 128)
        return FA_ERR_TILE;
    if (block_n == 0) block_n = 64;

    // Index space: every element offset must fit in int64, and the grid
    // (B*H*ceil(N_q/32) workgroups at most) in int32.
    const int64_t bh = (int64_t)B * H;
    const int64_t nq_el = bh * N_q * d, nk_el = bh * N_k * d;
    if (bh > (int64_t)1 << 31 || (double)bh * N_q * d > 9.0e18 || (double)bh * N_k * d > 9.0e18)
        return FA_ERR_SHAPE;
    if (bh * (((int64_t)N_q + 31) / 32) > INT32_MAX) return FA_ERR_SHAPE;

    const size_t esz = dtype == FA_DTYPE_BF16 ? 2 : 4;
    const size_t qb = (size_t)nq_el * esz, kb = (size_t)nk_el * esz;
    const size_t lb = (size_t)bh * N_q * sizeof(float);
    const size_t mb = kv_len_mask ? (size_t)B * N_k : 0;
    const void *ins[4] = {q, k, v, kv_len_mask};
    const size_t in_bytes[4] = {qb, kb, kb, mb};
    for (int i = 0; i < 4; ++i)
        if (overlaps(o, qb, ins[i], in_bytes[i]) || overlaps(lse, lb, ins[i], in_bytes[i]))
            return FA_ERR_ALIAS;
    if (overlaps(o, qb, lse, lb)) return FA_ERR_ALIAS;

    int rc = check_device();
    if (rc != FA_OK) return rc;

    fa::Params p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.mask = kv_len_mask;
    p.H = H;
    p.Nq = N_q;
    p.Nk = N_k;
    p.n_qt = 0;
    p.c = (float)((double)scale * 1.4426950408889634073599);
    p.scale = scale;
    p.reverse = (opts && opts->reverse_kv) ? 1 : 0;

    hipError_t e = fa::launch_fwd(p, dtype, d, block_n, causal ? 1 : 0, B, H,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        g_last_hip = e;
        return FA_ERR_LAUNCH;
    }
    return FA_OK;
}

}  // namespace

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

const char *fa_strerror(int code)
{
    const char *base;
    switch (code) {
    case FA_OK: base = "success"; break;
    case FA_ERR_NULL: base = "q, k, v, o or lse is NULL"; break;
    case FA_ERR_SHAPE: base = "B, H, N_q or N_k is not positive, or the sizes overflow"; break;
    case FA_ERR_HEAD_DIM: base = "head width d must be 64 or 128"; break;
    case FA_ERR_DTYPE: base = "dtype must be FA_DTYPE_F32 or FA_DTYPE_BF16"; break;
    case FA_ERR_SCALE: base = "scale must be finite and positive"; break;
    case FA_ERR_TILE: base = "block_n must be 0, 16, 32, 64 or 128"; break;
    case FA_ERR_DEVICE: base = "the current HIP device is not a gfx950 GPU"; break;
    case FA_ERR_LAUNCH: base = "HIP rejected the kernel launch"; break;
    case FA_ERR_ALIAS: base = "o or lse overlaps an input buffer"; break;
    default: base = "unknown status code"; break;
    }
    if ((code == FA_ERR_LAUNCH || code == FA_ERR_DEVICE) && g_last_hip != hipSuccess) {
        std::snprintf(g_msg, sizeof g_msg, "%s (HIP: %s)", base, hipGetErrorString(g_last_hip));
        return g_msg;
    }
    return base;
}

}  // extern "C"
