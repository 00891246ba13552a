// Host side of the step before the context write: argument checks and the
// launches of the hidden norm and of the projection with the write in its
// epilogue (vLLM API page "vllm.models.minimax_m3.common.dspark",
// MiniMaxM3DSparkModel.precompute_and_store_context_kv).
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dspark_project.h"
#include "project_args.h"
#include "qknorm_insert_args.h"
#include "writer_state.h"

using dspark::fail;

namespace {
bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
}  // namespace

extern "C" int dspark_hidden_norm(const void *x, int64_t rows, int32_t dim, const void *weight,
                                  float eps, void *out, void *stream) {
    if (rows < 0)
        return fail(DSPARK_E_ARG, "rows %lld is negative", (long long)rows);
    if (dim <= 0 || dim % 8)
        return fail(DSPARK_E_ARG, "dim %d is not a positive multiple of 8", dim);
    if (rows >= (int64_t{1} << 31))
        return fail(DSPARK_E_ARG, "rows %lld exceeds 2^31 - 1", (long long)rows);
    if (!x || !weight || !out)
        return fail(DSPARK_E_ARG, "a device pointer is NULL");
    if (!aligned(x, 16) || !aligned(weight, 16) || !aligned(out, 16))
        return fail(DSPARK_E_ARG, "x, weight and out must be 16-byte aligned");
    if (rows == 0)
        return DSPARK_OK;
    const hipError_t e = dspark::launch_hidden_norm(
        static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(weight),
        static_cast<uint16_t *>(out), static_cast<uint32_t>(rows), dim, eps,
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DSPARK_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return DSPARK_OK;
}

namespace {

// Checks and launch shared by the two projection entry points (kv_weight
// row-major, or in the fragment-major packing).
int project_write(dspark_ctx_kv_writer *w, const void *states, int64_t num_ctx, int32_t hidden,
                  const void *kv_weight, int32_t num_layers, int32_t num_kv_heads,
                  const void *k_norm_weight, float eps, const int64_t *positions,
                  const void *cos_sin_cache, int64_t cos_sin_rows, int32_t rotary_dim,
                  const int64_t *slot_mapping, void *stream, bool packed,
                  void *all_kv_out = nullptr) {
    if (w == nullptr)
        return fail(DSPARK_E_ARG, "writer is NULL");
    if (num_layers != w->num_layers || num_kv_heads != w->num_kv_heads)
        return fail(DSPARK_E_ARG,
                    "the projection has %d layers and %d kv heads; the writer was built for %d and %d",
                    num_layers, num_kv_heads, w->num_layers, w->num_kv_heads);
    if (!dspark_rotary_dims_supported(rotary_dim, DSPARK_HEAD_DIM))
        return fail(DSPARK_E_ARG, "rotary_dim %d is not 16, 32 or 64", rotary_dim);
    if (hidden <= 0 || hidden % 64)
        return fail(DSPARK_E_ARG, "hidden %d is not a positive multiple of 64", hidden);
    if (num_ctx < 0)
        return fail(DSPARK_E_ARG, "num_ctx %lld is negative", (long long)num_ctx);
    if (num_ctx >= (int64_t{1} << 31))
        return fail(DSPARK_E_ARG, "num_ctx %lld exceeds 2^31 - 1", (long long)num_ctx);
    if (!states || !kv_weight || !k_norm_weight || !positions || !cos_sin_cache || !slot_mapping)
        return fail(DSPARK_E_ARG, "a device pointer is NULL");
    if (!aligned(states, 16) || !aligned(kv_weight, 16) || !aligned(k_norm_weight, 16) ||
        !aligned(cos_sin_cache, 16))
        return fail(DSPARK_E_ARG,
                    "states, kv_weight, k_norm_weight and cos_sin_cache must be 16-byte aligned");
    if (!aligned(positions, 8) || !aligned(slot_mapping, 8))
        return fail(DSPARK_E_ARG, "positions and slot_mapping must be 8-byte aligned");
    if (cos_sin_rows <= 0)
        return fail(DSPARK_E_ARG, "cos_sin_cache has no rows");
    // the kernels address states and kv_weight with 32-bit byte offsets
    // (one tile of 256 rows past the end included)
    const int64_t cols = int64_t{num_layers} * 2 * num_kv_heads * DSPARK_HEAD_DIM;
    if ((num_ctx + 256) * hidden * 2 >= (int64_t{1} << 31) || cols * hidden * 2 >= (int64_t{1} << 31))
        return fail(DSPARK_E_ARG, "states or kv_weight exceed 2 GiB (num_ctx %lld, hidden %d)",
                    (long long)num_ctx, hidden);
    if (all_kv_out != nullptr && !aligned(all_kv_out, 16))
        return fail(DSPARK_E_ARG, "all_kv_out must be 16-byte aligned");
    if (num_ctx == 0)
        return DSPARK_OK;

    dspark::ProjArgs a;
    memset(&a, 0, sizeof a);
    a.z = static_cast<const uint16_t *>(states);
    a.W = static_cast<const uint16_t *>(kv_weight);
    a.k_norm_weight = static_cast<const uint16_t *>(k_norm_weight);
    a.cos_sin = static_cast<const uint16_t *>(cos_sin_cache);
    a.positions = positions;
    a.slots = slot_mapping;
    a.cache0 = w->cache0;
    a.scale0 = w->scale0;
    a.all_kv_out = static_cast<uint16_t *>(all_kv_out);
    a.num_ctx = static_cast<uint32_t>(num_ctx);
    a.hidden = hidden;
    a.cols = static_cast<uint32_t>(cols);
    a.num_layers = w->num_layers;
    a.nkv = w->num_kv_heads;
    a.bs_log2 = w->bs_log2;
    a.eps = eps;
    memcpy(a.cache_off, w->cache_off, sizeof a.cache_off);
    memcpy(a.kscale_off, w->kscale_off, sizeof a.kscale_off);
    memcpy(a.vscale_off, w->vscale_off, sizeof a.vscale_off);
    const hipError_t e = dspark::launch_project_write(
        a, rotary_dim, w->kv_cache_dtype == DSPARK_KV_FP8_E4M3, packed,
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DSPARK_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return DSPARK_OK;
}

}  // namespace

extern "C" int dspark_ctx_kv_writer_project_write(
    dspark_ctx_kv_writer *w, const void *states, int64_t num_ctx, int32_t hidden,
    const void *kv_weight, int32_t num_layers, int32_t num_kv_heads, const void *k_norm_weight,
    float eps, const int64_t *positions, const void *cos_sin_cache, int64_t cos_sin_rows,
    int32_t rotary_dim, const int64_t *slot_mapping, void *stream) {
    return project_write(w, states, num_ctx, hidden, kv_weight, num_layers, num_kv_heads,
                         k_norm_weight, eps, positions, cos_sin_cache, cos_sin_rows, rotary_dim,
                         slot_mapping, stream, false);
}

extern "C" int dspark_ctx_kv_writer_project_write_packed(
    dspark_ctx_kv_writer *w, const void *states, int64_t num_ctx, int32_t hidden,
    const void *packed_kv_weight, int32_t num_layers, int32_t num_kv_heads,
    const void *k_norm_weight, float eps, const int64_t *positions, const void *cos_sin_cache,
    int64_t cos_sin_rows, int32_t rotary_dim, const int64_t *slot_mapping, void *stream) {
    return project_write(w, states, num_ctx, hidden, packed_kv_weight, num_layers, num_kv_heads,
                         k_norm_weight, eps, positions, cos_sin_cache, cos_sin_rows, rotary_dim,
                         slot_mapping, stream, true);
}

extern "C" int dspark_ctx_kv_writer_project_write_all_kv(
    dspark_ctx_kv_writer *w, const void *states, int64_t num_ctx, int32_t hidden,
    const void *kv_weight, int32_t weight_packed, int32_t num_layers, int32_t num_kv_heads,
    const void *k_norm_weight, float eps, const int64_t *positions, const void *cos_sin_cache,
    int64_t cos_sin_rows, int32_t rotary_dim, const int64_t *slot_mapping, void *all_kv_out,
    void *stream) {
    if (weight_packed != 0 && weight_packed != 1)
        return fail(DSPARK_E_ARG, "weight_packed must be 0 or 1, not %d", weight_packed);
    if (all_kv_out == nullptr && num_ctx > 0)
        return fail(DSPARK_E_ARG, "all_kv_out is NULL");
    return project_write(w, states, num_ctx, hidden, kv_weight, num_layers, num_kv_heads,
                         k_norm_weight, eps, positions, cos_sin_cache, cos_sin_rows, rotary_dim,
                         slot_mapping, stream, weight_packed == 1, all_kv_out);
}

extern "C" int dspark_kv_weight_pack(const void *kv_weight, int64_t cols, int32_t hidden,
                                     void *packed, void *stream) {
    if (cols <= 0 || cols % 32)
        return fail(DSPARK_E_ARG, "cols %lld is not a positive multiple of 32", (long long)cols);
    if (hidden <= 0 || hidden % 16)
        return fail(DSPARK_E_ARG, "hidden %d is not a positive multiple of 16", hidden);
    if (cols * hidden * 2 >= (int64_t{1} << 31))
        return fail(DSPARK_E_ARG, "kv_weight exceeds 2 GiB (cols %lld, hidden %d)",
                    (long long)cols, hidden);
    if (!kv_weight || !packed)
        return fail(DSPARK_E_ARG, "a device pointer is NULL");
    if (!aligned(kv_weight, 16) || !aligned(packed, 16))
        return fail(DSPARK_E_ARG, "kv_weight and packed must be 16-byte aligned");
    const uintptr_t src = reinterpret_cast<uintptr_t>(kv_weight);
    const uintptr_t dst = reinterpret_cast<uintptr_t>(packed);
    const uintptr_t bytes = static_cast<uintptr_t>(cols * hidden * 2);
    if (src < dst + bytes && dst < src + bytes)
        return fail(DSPARK_E_ARG, "packed overlaps kv_weight");
    const hipError_t e = dspark::launch_pack_kv_weight(
        static_cast<const uint16_t *>(kv_weight), static_cast<uint16_t *>(packed),
        static_cast<uint32_t>(cols), hidden, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DSPARK_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return DSPARK_OK;
}
