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
    // Split-key mode: each query tile's key tiles are cut into n_split
    // consecutive ranges, one workgroup each, and every row's partial state
    // (m in raw score units, l, o~) goes to part_m / part_l / part_o
    // ([n_split][part_rows], same, [n_split][part_rows][d]) instead of o and
    // lse.  n_split = 1 and null pointers: the plain pass.
    int n_split;
    int64_t part_rows;    // B * H * N_q
    float *part_m;
    float *part_l;
    float *part_o;
    // Per-tile state of one row (fa_opts.trace), or nullptr.
    float *trace;
    int trace_bh;         // b * H + h of the traced row
    int trace_row;        // its query index
    // Shape of the device, queried once per device by the entry points:
    // compute units, and XCDs the dispatcher deals workgroups to in turn.
    int cus;
    int xcds;
    // Causal query tiles go in pairs (t, n_qt - 1 - t), two work items per
    // workgroup; set by the launcher of the bf16 kernel.
    int pair;
};

// Compute units and XCDs of the current device (cached per device); 256 and
// 8 when no device can be queried.  xcds is 1 unless it is a power of two
// that divides cus (then workgroups are dealt to XCDs in turn).
void device_geometry(int &cus, int &xcds);

// Query rows per workgroup of the forward kernel for validated arguments
// (dtype 0 = fp32, 1 = bf16; d 64 or 128; block_n 16, 32, 64 or 128; B, H,
// n_q >= 1; n_split key ranges per query tile, 1 for the plain pass; cus the
// device's compute units).
int query_tile_rows(int dtype, int d, int block_n, int B, int H, int n_q, int causal, int n_split,
                    int cus);

// Enqueues the forward kernel for validated arguments.  dtype: 0 = fp32,
// 1 = bf16; d: 64 or 128; block_n: 16, 32, 64 or 128.
hipError_t launch_fwd(const Params &p, int dtype, int d, int block_n, int causal, int B, int H,
                      hipStream_t stream);

// Enqueues the pass for N_q = 1 and bf16 (decoding): the workgroup of
// (b, h, split) writes the partial state of row b*H + h over its key range,
// as the forward kernel does in split-key mode, or, with n_split = 1 and no
// partial-state buffers, o and lse of the row.
hipError_t launch_decode(const Params &p, int d, int causal, int B, int H, hipStream_t stream);

// Enqueues the merge of n_parts partial states per row (part-major layout of
// fa_merge_states) into o (dtype 0 = fp32, 1 = bf16) and lse.
hipError_t launch_merge(const float *m, const float *l, const float *acc, int n_parts,
                        int64_t rows, int d, float scale, void *o, float *lse, int dtype,
                        hipStream_t stream);

// Bytes of the library's own device scratch (fa_fwd_splitkv_noalloc), one
// array per GPU, held until the process ends.
constexpr size_t kScratchBytes = (size_t)32 << 20;

// Device address of that scratch on the current device, looked up once per
// device (hipGetSymbolAddress) and cached.
hipError_t scratch_address(void **ptr);

// Enqueues the row softmax (fa_softmax_rows) for validated arguments.
hipError_t launch_softmax_rows(const void *s, void *p, float *m, float *l, int64_t rows,
                               int64_t n, int dtype, hipStream_t stream);

}  // namespace fa
