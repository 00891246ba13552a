// Host side of the draft block's fused QK-norm / RoPE / KV insert: argument
// checks and the launch.
//
// Follows dspark_qknorm_rope_kv_insert on the vLLM API page
// "vllm.models.minimax_m3.common.dspark": the insert happens only when a slot
// mapping is given (and then the cache is required), the block size is
// kv_cache.size(2), the cache is fp8 when its storage is uint8, and the query
// fp8 output is optional with a host-side scale.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "dspark_qknorm_insert.h"
#include "qknorm_insert_args.h"

namespace {

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int log2_exact(int64_t v) {
    int k = 0;
    while ((int64_t{1} << k) < v) ++k;
    return k;
}

}  // namespace

using dspark::fail;

extern "C" int dspark_qknorm_rope_kv_insert(void *qkv, int64_t num_tokens,
                                            const void *q_norm_weight, const void *k_norm_weight,
                                            const void *cos_sin_cache, int64_t cos_sin_rows,
                                            const int64_t *positions,
                                            int32_t num_heads, int32_t num_kv_heads,
                                            int32_t rotary_dim, float eps,
                                            const int64_t *slot_mapping, void *kv_cache,
                                            int64_t num_blocks, int32_t block_size,
                                            int32_t kv_cache_dtype,
                                            const float *k_scale, const float *v_scale,
                                            void *q_fp8_out, float q_fp8_scale,
                                            void *stream) {
    if (rotary_dim != 16 && rotary_dim != 32 && rotary_dim != 64)
        return fail(DSPARK_E_ARG, "rotary_dim %d is not 16, 32 or 64", rotary_dim);
    if (num_tokens < 0)
        return fail(DSPARK_E_ARG, "num_tokens %lld is negative", (long long)num_tokens);
    if (num_heads <= 0 || num_kv_heads <= 0)
        return fail(DSPARK_E_ARG, "num_heads %d and num_kv_heads %d must be positive", num_heads,
                    num_kv_heads);
    const int64_t heads = int64_t{num_heads} + 2 * int64_t{num_kv_heads};
    if (num_tokens > 0 && heads > (int64_t{1} << 31) / num_tokens)
        return fail(DSPARK_E_ARG, "num_tokens * (num_heads + 2 num_kv_heads) exceeds 2^31");
    if (!qkv || !q_norm_weight || !k_norm_weight || !cos_sin_cache || !positions)
        return fail(DSPARK_E_ARG, "a device pointer is NULL");
    if (!aligned(qkv, 16) || !aligned(q_norm_weight, 16) || !aligned(k_norm_weight, 16) ||
        !aligned(cos_sin_cache, 16))
        return fail(DSPARK_E_ARG, "qkv, the norm weights and cos_sin_cache must be 16-byte aligned");
    if (!aligned(positions, 8))
        return fail(DSPARK_E_ARG, "positions must be 8-byte aligned");
    if (cos_sin_rows <= 0)
        return fail(DSPARK_E_ARG, "cos_sin_cache has no rows");

    dspark::InsertCache cache_kind = dspark::kNoInsert;
    int bs_log2 = 0;
    if (slot_mapping) {
        if (!kv_cache)
            return fail(DSPARK_E_ARG, "a slot mapping was given without a KV cache");
        if (!aligned(slot_mapping, 8))
            return fail(DSPARK_E_ARG, "slot_mapping must be 8-byte aligned");
        if (!aligned(kv_cache, 16))
            return fail(DSPARK_E_ARG, "kv_cache must be 16-byte aligned");
        if (num_blocks <= 0)
            return fail(DSPARK_E_ARG, "kv_cache has no blocks");
        if (block_size <= 0 || (block_size & (block_size - 1)))
            return fail(DSPARK_E_ARG, "block size %d is not a power of two", block_size);
        if (kv_cache_dtype == DSPARK_KV_AUTO)
            cache_kind = dspark::kInsertBf16;
        else if (kv_cache_dtype == DSPARK_KV_FP8_E4M3)
            cache_kind = dspark::kInsertFp8;
        else
            return fail(DSPARK_E_ARG, "kv_cache_dtype %d", kv_cache_dtype);
        if ((k_scale && !aligned(k_scale, 4)) || (v_scale && !aligned(v_scale, 4)))
            return fail(DSPARK_E_ARG, "k_scale and v_scale must be 4-byte aligned");
        bs_log2 = log2_exact(block_size);
    }
    if (q_fp8_out) {
        if (!aligned(q_fp8_out, 8))
            return fail(DSPARK_E_ARG, "q_fp8_out must be 8-byte aligned");
        if (!(q_fp8_scale > 0.0f) || !isfinite(q_fp8_scale))
            return fail(DSPARK_E_ARG, "q_fp8_scale %g must be finite and > 0", (double)q_fp8_scale);
    }
    if (num_tokens == 0)
        return DSPARK_OK;

    dspark::InsertArgs a{};
    a.qkv = static_cast<uint16_t *>(qkv);
    a.q_w = static_cast<const uint16_t *>(q_norm_weight);
    a.k_w = static_cast<const uint16_t *>(k_norm_weight);
    a.cos_sin = static_cast<const uint16_t *>(cos_sin_cache);
    a.positions = positions;
    const bool insert = cache_kind != dspark::kNoInsert;
    a.slots = insert ? slot_mapping : nullptr;
    a.cache = insert ? kv_cache : nullptr;
    a.k_scale = insert ? k_scale : nullptr;
    a.v_scale = insert ? v_scale : nullptr;
    a.q_fp8 = static_cast<uint8_t *>(q_fp8_out);
    a.q_scale = q_fp8_out ? q_fp8_scale : 1.0f;
    a.eps = eps;
    a.num_rows = static_cast<uint32_t>(num_tokens * heads);
    a.heads_per_token = static_cast<int32_t>(heads);
    a.num_heads = num_heads;
    a.nkv = num_kv_heads;
    a.bs_log2 = bs_log2;
    const hipError_t e = dspark::launch_qknorm_insert(a, rotary_dim, cache_kind, q_fp8_out != nullptr,
                                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DSPARK_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return DSPARK_OK;
}
