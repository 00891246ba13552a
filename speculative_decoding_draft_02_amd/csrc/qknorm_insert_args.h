// Kernel-argument block of the draft block's fused QK-norm / RoPE / KV
// insert, shared by the host side (qknorm_insert.cpp) and the kernels
// (qknorm_insert_kernel.hip).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace dspark {

struct InsertArgs {
    uint16_t *qkv;               // bf16 [T, (H + 2 nkv) * 128], in place
    const uint16_t *q_w;         // bf16 [128]
    const uint16_t *k_w;         // bf16 [128]
    const uint16_t *cos_sin;     // bf16 [rows, R] = [cos | sin]
    const int64_t *positions;    // [T]
    const int64_t *slots;        // [T] (insert only)
    void *cache;                 // [num_blocks, nkv, bs, 256] (insert only)
    uint8_t *q_fp8;              // [T, H * 128] (q fp8 output only)
    const float *k_scale;        // device scalar or NULL (1.0)
    const float *v_scale;        // device scalar or NULL (1.0)
    float q_scale;
    float eps;
    uint32_t num_rows;           // T * (H + 2 nkv): one 128-dim head each
    int32_t heads_per_token;     // H + 2 nkv
    int32_t num_heads;           // H
    int32_t nkv;
    int32_t bs_log2;             // log2(block_size)
};

// Cache kinds of a launch.
enum InsertCache { kNoInsert = 0, kInsertBf16 = 1, kInsertFp8 = 2 };

// Enqueue one launch.  Returns the hipError_t of the launch.
hipError_t launch_qknorm_insert(const InsertArgs &args, int rotary_dim, InsertCache cache,
                                bool q_fp8, hipStream_t stream);

// Record `fmt` as this thread's last error and return `status` (defined with
// the context writer, which owns the last-error string).
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace dspark
