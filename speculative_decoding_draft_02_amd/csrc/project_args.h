// Kernel arguments of the step before the context write: the Gemma hidden
// norm of the context states, and the token-major K/V projection with the
// context write in its epilogue.  Shared by project.cpp and
// project_kernel.hip.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "dspark_ctx_kv.h"

namespace dspark {

struct ProjArgs {
    const uint16_t *z;             // bf16 [num_ctx, hidden]: the hidden-norm output
    const uint16_t *W;             // bf16 [cols, hidden]: the projection, [out, in]
                                   // (or its fragment-major packing)
    const uint16_t *k_norm_weight; // bf16 [L, 128]
    const uint16_t *cos_sin;       // bf16 [rows, R] = [cos | sin]
    const int64_t *positions;      // [num_ctx]
    const int64_t *slots;          // [num_ctx], < 0 = padding
    void *cache0;                  // layer 0's cache (bf16 or uint8 elements)
    const float *scale0;           // layer 0's k scale
    uint16_t *all_kv_out;          // bf16 [num_ctx, cols]: the projection's output,
                                   // also stored when not NULL
    uint32_t num_ctx;
    int32_t hidden;                // multiple of 64
    uint32_t cols;                 // L * 2 * nkv * 128
    int32_t num_layers;
    int32_t nkv;
    int32_t bs_log2;
    float eps;
    uint32_t big_tiles;            // 128 x 512 tiles of a launch whose other
                                   // workgroups take 64-token halves (set by
                                   // the launcher)
    int64_t cache_off[DSPARK_MAX_LAYERS];   // elements from cache0
    int64_t kscale_off[DSPARK_MAX_LAYERS];  // floats from scale0
    int64_t vscale_off[DSPARK_MAX_LAYERS];  // floats from scale0
};

// Gemma RMSNorm of `rows` rows of `dim` bf16 values (dim % 8 == 0).
hipError_t launch_hidden_norm(const uint16_t *x, const uint16_t *w, uint16_t *out, uint32_t rows,
                              int32_t dim, float eps, hipStream_t stream);

// The projection z @ W^T with the context write of every (layer, kv, head)
// column block in the epilogue; `packed`: W is in the fragment-major layout
// of launch_pack_kv_weight.
hipError_t launch_project_write(const ProjArgs &args, int rotary_dim, bool fp8, bool packed,
                                hipStream_t stream);

// W [cols, hidden] (row-major) -> its fragment-major layout (same size):
// element (c, k) at fragment (c / 32) * hidden / 16 + k / 16 (512 elements
// each), position 8 (c % 32 + 32 ((k % 16) / 8)) + k % 8.  cols % 32 == 0,
// hidden % 16 == 0.
hipError_t launch_pack_kv_weight(const uint16_t *w, uint16_t *out, uint32_t cols, int32_t hidden,
                                 hipStream_t stream);

}  // namespace dspark
