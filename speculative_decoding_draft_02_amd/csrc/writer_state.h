// The context writer's host state: the layout it was built for and the
// per-layer offset tables (elements from layer 0's cache, floats from layer
// 0's k scale).  Private to the library's host files.
#pragma once

#include <stdint.h>

#include "dspark_ctx_kv.h"

struct dspark_ctx_kv_writer {

    int32_t num_layers;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t bs_log2;
    int64_t num_blocks;
    int32_t kv_cache_dtype;
    void *cache0;
    const float *scale0;
    int64_t cache_off[DSPARK_MAX_LAYERS];
    int64_t kscale_off[DSPARK_MAX_LAYERS];
    int64_t vscale_off[DSPARK_MAX_LAYERS];
};
