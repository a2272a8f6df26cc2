// fa_internal.h -- declarations shared by the host entry points and the
// kernels of libfa.so.  Not installed; the public ABI is include/fa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Kernel arguments, passed by value.
struct Params {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;
    const uint8_t *mask;  // [B, N_k] or nullptr
    int H;
    int Nq;
    int Nk;
    int n_qt;             // query tiles per (batch, head); set by the launcher
    float c;              // scale * log2(e): scores to the exp2 domain
    float scale;
    int reverse;          // visit key tiles last to first
};

// Enqueues the forward kernel for validated arguments.  dtype: 0 = fp32,
// 1 = bf16; d: 64 or 128; block_n: 16, 32, 64 or 128.
hipError_t launch_fwd(const Params &p, int dtype, int d, int block_n, int causal, int B, int H,
                      hipStream_t stream);

}  // namespace fa
