// Host side of the fused DSpark context-KV write: layout validation, the
// writer object with its per-layer offset tables, and the launch.
//
// Mirrors class DSparkContextKVWriter on the vLLM API page
// "vllm.models.minimax_m3.common.ops.dspark_context_kv": _validate (the
// layout rules and their reason strings), _ensure_tables (cache offsets in
// elements from layer 0's cache, scale offsets in floats from layer 0's k
// scale, [2, L]: k scales then v scales) and __call__ (L / nkv must match,
// num_ctx == 0 is a no-op, one launch).
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <string>

#include <hip/hip_runtime_api.h>

#include "ctx_kv_args.h"
#include "qknorm_insert_args.h"
#include "writer_state.h"
#include "dspark_ctx_kv.h"


namespace {
thread_local std::string g_last_error;
}  // namespace

// The last-error string of every entry point of the library.
int dspark::fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

namespace {

using dspark::fail;

int ok() { return DSPARK_OK; }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int element_size(int32_t kv_cache_dtype) { return kv_cache_dtype == DSPARK_KV_FP8_E4M3 ? 1 : 2; }

int validate(int32_t num_layers, void *const *kv_caches, const float *const *k_scales,
             const float *const *v_scales, int64_t num_blocks, int32_t num_kv_heads,
             int32_t block_size, int32_t head_dim, int32_t kv_cache_dtype) {
    if (num_layers <= 0 || kv_caches == nullptr)
        return fail(DSPARK_E_LAYOUT, "no layers");
    if (num_layers > DSPARK_MAX_LAYERS)
        return fail(DSPARK_E_LAYOUT, "%d layers exceed the supported %d", num_layers,
                    DSPARK_MAX_LAYERS);
    if (kv_cache_dtype != DSPARK_KV_AUTO && kv_cache_dtype != DSPARK_KV_FP8_E4M3)
        return fail(DSPARK_E_LAYOUT, "kv_cache_dtype %d", kv_cache_dtype);
    for (int l = 0; l < num_layers; ++l)
        if (kv_caches[l] == nullptr)
            return fail(DSPARK_E_LAYOUT, "KV cache not bound");
    if (num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0)
        return fail(DSPARK_E_LAYOUT, "KV cache not bound");
    if (head_dim != DSPARK_HEAD_DIM)
        return fail(DSPARK_E_LAYOUT, "unexpected cache shape (%lld, %d, %d, %d)",
                    (long long)num_blocks, num_kv_heads, block_size, 2 * head_dim);
    if (!is_pow2(block_size))
        return fail(DSPARK_E_LAYOUT, "block size %d is not a power of two", block_size);
    if (k_scales == nullptr || v_scales == nullptr)
        return fail(DSPARK_E_LAYOUT, "_k_scale is not a device fp32 pointer");
    for (int l = 0; l < num_layers; ++l) {
        if (k_scales[l] == nullptr || (reinterpret_cast<uintptr_t>(k_scales[l]) & 3))
            return fail(DSPARK_E_LAYOUT, "_k_scale is not a device fp32 pointer");
        if (v_scales[l] == nullptr || (reinterpret_cast<uintptr_t>(v_scales[l]) & 3))
            return fail(DSPARK_E_LAYOUT, "_v_scale is not a device fp32 pointer");
    }
    const int esize = element_size(kv_cache_dtype);
    const char *base = static_cast<const char *>(kv_caches[0]);
    if (reinterpret_cast<uintptr_t>(base) & 15)
        return fail(DSPARK_E_LAYOUT, "layer 0 cache is not 16-byte aligned");
    for (int l = 1; l < num_layers; ++l) {
        const int64_t delta = static_cast<const char *>(kv_caches[l]) - base;
        if (delta % (16 * esize))
            return fail(DSPARK_E_LAYOUT, "layer caches are not 16-element aligned to each other");
    }
    return ok();
}

int write_impl(dspark_ctx_kv_writer *w, const void *all_kv, int64_t num_ctx, int32_t num_layers,
               int32_t num_kv_heads, const void *k_norm_weight, float eps,
               const int64_t *positions, const void *cos_sin_cache, int64_t cos_sin_rows,
               int32_t rotary_dim, const int64_t *slot_mapping,
               const int64_t *const *layer_slot_mappings, void *stream) {
    if (w == nullptr)
        return fail(DSPARK_E_ARG, "writer is NULL");
    if (num_layers != w->num_layers || num_kv_heads != w->num_kv_heads)
        return fail(DSPARK_E_ARG,
                    "all_kv has %d layers and %d kv heads; the writer was built for %d and %d",
                    num_layers, num_kv_heads, w->num_layers, w->num_kv_heads);
    if (!dspark_rotary_dims_supported(rotary_dim, DSPARK_HEAD_DIM))
        return fail(DSPARK_E_ARG, "rotary_dim %d is not 16, 32 or 64", rotary_dim);
    if (num_ctx < 0)
        return fail(DSPARK_E_ARG, "num_ctx %lld is negative", (long long)num_ctx);
    if (num_ctx == 0)
        return ok();
    if (num_ctx * num_kv_heads >= (int64_t{1} << 31))
        return fail(DSPARK_E_ARG, "num_ctx * num_kv_heads = %lld exceeds 2^31 - 1",
                    (long long)(num_ctx * num_kv_heads));
    if (all_kv == nullptr || k_norm_weight == nullptr || positions == nullptr ||
        cos_sin_cache == nullptr || (slot_mapping == nullptr && layer_slot_mappings == nullptr))
        return fail(DSPARK_E_ARG, "a device pointer is NULL");
    if (layer_slot_mappings != nullptr) {
        for (int l = 0; l < num_layers; ++l) {
            if (layer_slot_mappings[l] == nullptr)
                return fail(DSPARK_E_ARG, "slot mapping of layer %d is NULL", l);
            if (reinterpret_cast<uintptr_t>(layer_slot_mappings[l]) & 7)
                return fail(DSPARK_E_ARG, "slot mapping of layer %d is not 8-byte aligned", l);
        }
    }
    if ((reinterpret_cast<uintptr_t>(all_kv) | reinterpret_cast<uintptr_t>(k_norm_weight) |
         reinterpret_cast<uintptr_t>(cos_sin_cache)) & 15)
        return fail(DSPARK_E_ARG, "all_kv, k_norm_weight and cos_sin_cache must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(positions) | reinterpret_cast<uintptr_t>(slot_mapping)) & 7)
        return fail(DSPARK_E_ARG, "positions and slot_mapping must be 8-byte aligned");
    if (cos_sin_rows <= 0)
        return fail(DSPARK_E_ARG, "cos_sin_cache has no rows");

    dspark::CtxKvArgs a;
    memset(&a, 0, sizeof a);
    a.all_kv = all_kv;
    a.k_norm_weight = k_norm_weight;
    a.cos_sin = static_cast<const uint16_t *>(cos_sin_cache);
    a.positions = positions;
    a.slots = slot_mapping;
    a.cache0 = w->cache0;
    a.scale0 = w->scale0;
    a.num_units = static_cast<uint32_t>(num_ctx * num_kv_heads);
    a.num_layers = w->num_layers;
    a.nkv = w->num_kv_heads;
    a.bs_log2 = w->bs_log2;
    a.eps = eps;
    memcpy(a.cache_off, w->cache_off, sizeof a.cache_off);
    memcpy(a.kscale_off, w->kscale_off, sizeof a.kscale_off);
    memcpy(a.vscale_off, w->vscale_off, sizeof a.vscale_off);
    if (layer_slot_mappings != nullptr) {
        a.layer_slots_on = 1;
        for (int l = 0; l < num_layers; ++l) a.layer_slots[l] = layer_slot_mappings[l];
    }

    const hipError_t e = dspark::launch_ctx_kv(a, rotary_dim, w->kv_cache_dtype == DSPARK_KV_FP8_E4M3,
                                               static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DSPARK_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int dspark_ctx_kv_validate(int32_t num_layers, void *const *kv_caches,
                           const float *const *k_scales, const float *const *v_scales,
                           int64_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                           int32_t head_dim, int32_t kv_cache_dtype) {
    return validate(num_layers, kv_caches, k_scales, v_scales, num_blocks, num_kv_heads,
                    block_size, head_dim, kv_cache_dtype);
}

int dspark_ctx_kv_writer_create(int32_t num_layers, void *const *kv_caches,
                                const float *const *k_scales, const float *const *v_scales,
                                int64_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                                int32_t head_dim, int32_t kv_cache_dtype,
                                dspark_ctx_kv_writer **out) {
    if (out == nullptr)
        return fail(DSPARK_E_ARG, "out is NULL");
    *out = nullptr;
    const int st = validate(num_layers, kv_caches, k_scales, v_scales, num_blocks,
                            num_kv_heads, block_size, head_dim, kv_cache_dtype);
    if (st != DSPARK_OK)
        return st;
    dspark_ctx_kv_writer *w = new (std::nothrow) dspark_ctx_kv_writer();
    if (w == nullptr)
        return fail(DSPARK_E_ARG, "out of host memory");
    w->num_layers = num_layers;
    w->num_kv_heads = num_kv_heads;
    w->block_size = block_size;
    w->bs_log2 = __builtin_ctz(static_cast<unsigned>(block_size));
    w->num_blocks = num_blocks;
    w->kv_cache_dtype = kv_cache_dtype;
    w->cache0 = kv_caches[0];
    w->scale0 = k_scales[0];
    const int esize = element_size(kv_cache_dtype);
    const char *c0 = static_cast<const char *>(kv_caches[0]);
    const char *s0 = reinterpret_cast<const char *>(k_scales[0]);
    for (int l = 0; l < num_layers; ++l) {
        w->cache_off[l] = (static_cast<const char *>(kv_caches[l]) - c0) / esize;
        w->kscale_off[l] = (reinterpret_cast<const char *>(k_scales[l]) - s0) / 4;
        w->vscale_off[l] = (reinterpret_cast<const char *>(v_scales[l]) - s0) / 4;
    }
    *out = w;
    return ok();
}

int dspark_ctx_kv_writer_write(dspark_ctx_kv_writer *w, const void *all_kv, int64_t num_ctx,
                               int32_t num_layers, int32_t num_kv_heads,
                               const void *k_norm_weight, float eps, const int64_t *positions,
                               const void *cos_sin_cache, int64_t cos_sin_rows,
                               int32_t rotary_dim, const int64_t *slot_mapping, void *stream) {
    if (slot_mapping == nullptr && num_ctx > 0)
        return fail(DSPARK_E_ARG, "a device pointer is NULL");
    return write_impl(w, all_kv, num_ctx, num_layers, num_kv_heads, k_norm_weight, eps, positions,
                      cos_sin_cache, cos_sin_rows, rotary_dim, slot_mapping, nullptr, stream);
}

int dspark_ctx_kv_writer_write_layer_slots(dspark_ctx_kv_writer *w, const void *all_kv,
                                           int64_t num_ctx, int32_t num_layers,
                                           int32_t num_kv_heads, const void *k_norm_weight,
                                           float eps, const int64_t *positions,
                                           const void *cos_sin_cache, int64_t cos_sin_rows,
                                           int32_t rotary_dim,
                                           const int64_t *const *slot_mappings, void *stream) {
    if (slot_mappings == nullptr && num_ctx > 0)
        return fail(DSPARK_E_ARG, "slot_mappings is NULL");
    return write_impl(w, all_kv, num_ctx, num_layers, num_kv_heads, k_norm_weight, eps, positions,
                      cos_sin_cache, cos_sin_rows, rotary_dim, nullptr, slot_mappings, stream);
}

void dspark_ctx_kv_writer_destroy(dspark_ctx_kv_writer *w) { delete w; }

int dspark_rotary_dims_supported(int32_t rotary_dim, int32_t head_dim) {
    return head_dim == DSPARK_HEAD_DIM && (rotary_dim == 16 || rotary_dim == 32 || rotary_dim == 64);
}

const char *dspark_ctx_kv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
