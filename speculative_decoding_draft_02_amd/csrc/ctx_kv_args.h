// Kernel-argument block of the fused context-KV write, shared by the host
// side (ctx_kv_writer.cpp) and the kernels (ctx_kv_kernel.hip).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "dspark_ctx_kv.h"

namespace dspark {

// Passed by value in the kernel-argument segment: the per-layer offset tables
// travel with every launch (and are frozen into a captured HIP graph node), so
// no device-side table exists and a write never copies host to device.
struct CtxKvArgs {
    const void *all_kv;          // bf16 [num_ctx, L, 2, nkv, 128]
    const void *k_norm_weight;   // bf16 [L, 128]
    const uint16_t *cos_sin;     // bf16 [rows, R] = [cos | sin]
    const int64_t *positions;    // [num_ctx]
    const int64_t *slots;        // [num_ctx], < 0 = padding
    void *cache0;                // layer 0's cache (bf16 or uint8 elements)
    const float *scale0;         // layer 0's k scale
    uint32_t num_units;          // num_ctx * nkv: one (token, kv head) row each
    int32_t num_layers;
    int32_t nkv;
    int32_t bs_log2;             // log2(block_size)
    float eps;
    // reciprocal multipliers ceil(2^32 / d) for the wave -> (row group, layer
    // group) split (d = layer groups) and, with 4 heads of one token per
    // wave, for wave -> token (d = nkv / 4); 0 = divide (see fast_div)
    uint32_t split_magic;
    uint32_t token_magic;
    int64_t cache_off[DSPARK_MAX_LAYERS];  // elements from cache0
    int64_t kscale_off[DSPARK_MAX_LAYERS]; // floats from scale0
    int64_t vscale_off[DSPARK_MAX_LAYERS]; // floats from scale0
    // per-layer slot mappings (layer l's [num_ctx] mapping), used instead of
    // `slots` when layer_slots_on is set
    const int64_t *layer_slots[DSPARK_MAX_LAYERS];
    int32_t layer_slots_on;
};

// Enqueue one launch.  Returns the hipError_t of the launch.
hipError_t launch_ctx_kv(const CtxKvArgs &args, int rotary_dim, bool fp8, hipStream_t stream);

}  // namespace dspark
