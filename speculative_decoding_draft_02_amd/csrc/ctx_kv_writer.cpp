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

#include <climits>
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

// ------------------------------------------------------- layout rules --
//
// The layouts a writer accepts are the rules of DSparkContextKVWriter._validate
// on the vLLM API page "vllm.models.minimax_m3.common.ops.dspark_context_kv",
// held here as a table: every layer is checked in order, each against the
// rules in table order, and the first rule that fails names the reason (the
// page's wording).  A rule sees one layer and layer 0 (for the rules that
// compare layers).

// The kv_cache_dtype names the page accepts, and the cache kind each means.
struct KvDtypeName {
    const char *name;
    int32_t kind;
};
constexpr KvDtypeName kKvDtypeNames[] = {
    {"auto", DSPARK_KV_AUTO}, {"fp8", DSPARK_KV_FP8_E4M3}, {"fp8_e4m3", DSPARK_KV_FP8_E4M3}};

// DSPARK_KV_* for a supported name, else -1.
int32_t kv_kind(const char *name) {
    if (name == nullptr) return -1;
    for (const KvDtypeName &k : kKvDtypeNames)
        if (strcmp(name, k.name) == 0) return k.kind;
    return -1;
}

int64_t numel(const dspark_tensor_info &t) {
    if (t.data == nullptr || t.ndim < 0 || t.ndim > DSPARK_MAX_DIMS) return 0;
    int64_t n = 1;
    for (int d = 0; d < t.ndim; ++d) n *= t.shape[d];
    return n;
}

// Row-major strides, ignoring those of dims of size 1.
bool contiguous(const dspark_tensor_info &t) {
    int64_t expect = 1;
    for (int d = t.ndim - 1; d >= 0; --d) {
        if (t.shape[d] != 1 && t.strides[d] != expect) return false;
        expect *= t.shape[d];
    }
    return true;
}

std::string shape_text(const dspark_tensor_info &t) {
    std::string s = "(";
    const int nd = t.ndim < 0 ? 0 : (t.ndim > DSPARK_MAX_DIMS ? DSPARK_MAX_DIMS : t.ndim);
    for (int d = 0; d < nd; ++d) {
        s += std::to_string(static_cast<long long>(t.shape[d]));
        if (d + 1 < nd || nd == 1) s += ",";
        if (d + 1 < nd) s += " ";
    }
    return s + ")";
}

const char *type_text(const dspark_tensor_info &t) {
    if (t.dtype_name != nullptr) return t.dtype_name;
    switch (t.dtype) {
    case DSPARK_DTYPE_BF16: return "bfloat16";
    case DSPARK_DTYPE_UINT8: return "uint8";
    case DSPARK_DTYPE_FP32: return "float32";
    default: return "an unsupported type";
    }
}

bool is_gpu_fp32(const dspark_tensor_info &t) {
    return t.data != nullptr && t.dtype == DSPARK_DTYPE_FP32 && t.on_gpu;
}

using Layer = dspark_layer_info;
// true if the rule holds; else false with the reason in `why`
using LayerRule = bool (*)(const Layer &a, const Layer &first, std::string &why);

bool kv_dtype_supported(const Layer &a, const Layer &, std::string &why) {
    if (kv_kind(a.kv_cache_dtype) >= 0) return true;
    why = a.kv_cache_dtype ? std::string("kv_cache_dtype '") + a.kv_cache_dtype + "'"
                           : std::string("kv_cache_dtype None");
    return false;
}

bool cache_bound(const Layer &a, const Layer &, std::string &why) {
    if (numel(a.kv_cache) > 0) return true;
    why = "KV cache not bound";
    return false;
}

bool cache_shape(const Layer &a, const Layer &, std::string &why) {
    if (a.kv_cache.ndim == 4 && a.kv_cache.shape[3] == 2 * DSPARK_HEAD_DIM) return true;
    why = "unexpected cache shape " + shape_text(a.kv_cache);
    return false;
}

bool block_size_pow2(const Layer &a, const Layer &, std::string &why) {
    if (is_pow2(a.kv_cache.shape[2])) return true;
    why = "block size " + std::to_string(static_cast<long long>(a.kv_cache.shape[2])) +
          " is not a power of two";
    return false;
}

bool cache_contiguous(const Layer &a, const Layer &, std::string &why) {
    if (contiguous(a.kv_cache)) return true;
    why = "cache is not contiguous";
    return false;
}

bool cache_element_type(const Layer &a, const Layer &, std::string &why) {
    const bool fp8 = kv_kind(a.kv_cache_dtype) == DSPARK_KV_FP8_E4M3;
    if (a.kv_cache.dtype == (fp8 ? DSPARK_DTYPE_UINT8 : DSPARK_DTYPE_BF16)) return true;
    why = std::string(fp8 ? "fp8 cache has dtype " : "cache has dtype ") + type_text(a.kv_cache);
    return false;
}

bool scales_on_gpu(const Layer &a, const Layer &, std::string &why) {
    if (!is_gpu_fp32(a.k_scale)) {
        why = "_k_scale is not a CUDA fp32 tensor";
        return false;
    }
    if (!is_gpu_fp32(a.v_scale)) {
        why = "_v_scale is not a CUDA fp32 tensor";
        return false;
    }
    return true;
}

bool same_layout_as_first(const Layer &a, const Layer &f, std::string &why) {
    bool same = a.kv_cache.ndim == f.kv_cache.ndim && a.kv_cache.dtype == f.kv_cache.dtype &&
                strcmp(a.kv_cache_dtype, f.kv_cache_dtype) == 0;
    for (int d = 0; same && d < a.kv_cache.ndim; ++d)
        same = a.kv_cache.shape[d] == f.kv_cache.shape[d] &&
               a.kv_cache.strides[d] == f.kv_cache.strides[d];
    if (same) return true;
    why = "layers do not share cache shape/stride/dtype";
    return false;
}

bool same_device_as_first(const Layer &a, const Layer &f, std::string &why) {
    if (a.kv_cache.on_gpu == f.kv_cache.on_gpu &&
        a.kv_cache.device_index == f.kv_cache.device_index)
        return true;
    why = "layers are on different devices";
    return false;
}

bool aligned_to_first(const Layer &a, const Layer &f, std::string &why) {
    const int esize = a.kv_cache.dtype == DSPARK_DTYPE_UINT8 ? 1 : 2;
    const int64_t delta = static_cast<const char *>(a.kv_cache.data) -
                          static_cast<const char *>(f.kv_cache.data);
    if (delta % (16 * esize) == 0) return true;
    why = "layer caches are not 16-element aligned to each other";
    return false;
}

constexpr LayerRule kLayerRules[] = {
    kv_dtype_supported, cache_bound,   cache_shape,          block_size_pow2,
    cache_contiguous,   cache_element_type, scales_on_gpu,   same_layout_as_first,
    same_device_as_first, aligned_to_first};

int validate(int32_t num_layers, const dspark_layer_info *layers) {
    if (num_layers <= 0 || layers == nullptr)
        return fail(DSPARK_E_LAYOUT, "no layers");
    if (num_layers > DSPARK_MAX_LAYERS)
        return fail(DSPARK_E_LAYOUT, "%d layers exceed the supported %d", num_layers,
                    DSPARK_MAX_LAYERS);
    std::string why;
    for (int l = 0; l < num_layers; ++l)
        for (LayerRule rule : kLayerRules)
            if (!rule(layers[l], layers[0], why))
                return fail(DSPARK_E_LAYOUT, "%s", why.c_str());
    // the library's own limits
    if (reinterpret_cast<uintptr_t>(layers[0].kv_cache.data) & 15)
        return fail(DSPARK_E_LAYOUT, "layer 0 cache is not 16-byte aligned");
    for (int l = 0; l < num_layers; ++l) {
        if (reinterpret_cast<uintptr_t>(layers[l].k_scale.data) & 3)
            return fail(DSPARK_E_LAYOUT, "_k_scale of layer %d is not 4-byte aligned", l);
        if (reinterpret_cast<uintptr_t>(layers[l].v_scale.data) & 3)
            return fail(DSPARK_E_LAYOUT, "_v_scale of layer %d is not 4-byte aligned", l);
    }
    if (layers[0].kv_cache.shape[1] > INT32_MAX || layers[0].kv_cache.shape[2] > INT32_MAX)
        return fail(DSPARK_E_LAYOUT, "unexpected cache shape %s",
                    shape_text(layers[0].kv_cache).c_str());
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

int dspark_ctx_kv_validate(int32_t num_layers, const dspark_layer_info *layers) {
    return validate(num_layers, layers);
}

int dspark_ctx_kv_writer_create(int32_t num_layers, const dspark_layer_info *layers,
                                dspark_ctx_kv_writer **out) {
    if (out == nullptr)
        return fail(DSPARK_E_ARG, "out is NULL");
    *out = nullptr;
    const int st = validate(num_layers, layers);
    if (st != DSPARK_OK)
        return st;
    dspark_ctx_kv_writer *w = new (std::nothrow) dspark_ctx_kv_writer();
    if (w == nullptr)
        return fail(DSPARK_E_ARG, "out of host memory");
    const dspark_tensor_info &c0 = layers[0].kv_cache;
    w->num_layers = num_layers;
    w->num_blocks = c0.shape[0];
    w->num_kv_heads = static_cast<int32_t>(c0.shape[1]);
    w->block_size = static_cast<int32_t>(c0.shape[2]);
    w->bs_log2 = __builtin_ctz(static_cast<unsigned>(w->block_size));
    w->kv_cache_dtype = kv_kind(layers[0].kv_cache_dtype);
    w->cache0 = const_cast<void *>(c0.data);
    w->scale0 = static_cast<const float *>(layers[0].k_scale.data);
    const int esize = element_size(w->kv_cache_dtype);
    const char *base = static_cast<const char *>(c0.data);
    const char *s0 = static_cast<const char *>(layers[0].k_scale.data);
    for (int l = 0; l < num_layers; ++l) {
        w->cache_off[l] = (static_cast<const char *>(layers[l].kv_cache.data) - base) / esize;
        w->kscale_off[l] = (static_cast<const char *>(layers[l].k_scale.data) - s0) / 4;
        w->vscale_off[l] = (static_cast<const char *>(layers[l].v_scale.data) - s0) / 4;
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
