/*
 * dspark_ctx_kv.h - C ABI of the DSpark fused context-KV write for MI355X
 * (gfx950).
 *
 * The operation is the one the vLLM API page
 * "vllm.models.minimax_m3.common.ops.dspark_context_kv" defines in its module
 * docstring and in class DSparkContextKVWriter: from the fused projection
 * output all_kv [num_ctx, L, 2, nkv, 128] (bf16), every draft layer l gets
 *
 *   K = partial NeoX RoPE( bf16( x * rsqrt(mean(x^2) + eps) * (1 + w_l) ) )
 *       (the norm in fp32, its output rounded to bf16; RoPE on the leading
 *        rotary_dim dims at the token's position, each result rounded to bf16)
 *   V = all_kv[t, l, 1, h, :] unchanged
 *
 * stored at cache_l[slot / block_size, h, slot % block_size, 0:128] (K) and
 * [..., 128:256] (V) of layer l's separately allocated paged cache
 * [num_blocks, nkv, block_size, 256], as raw bf16 or as OCP fp8 e4m3 of
 * (fp32 value) / (fp32 per-layer scale), saturating at +-448.  A token whose
 * slot is < 0 is padding: nothing is written for it and its position is not
 * used (its all_kv rows may still be read, ahead of the slot).
 *
 * The writer is built once from the layers' caches and scales (class
 * DSparkContextKVWriter.__init__ and _validate on that page).  Layer l's cache
 * is addressed as layer 0's cache plus a per-layer element offset, and each
 * scale as layer 0's k scale plus a float offset (_ensure_tables); the offsets
 * are computed at creation and travel by value in every launch, so a call
 * captured in a HIP graph keeps addressing the same memory and never needs a
 * host-to-device copy.
 *
 * Ownership: the caller owns every device buffer and stream; the library owns
 * only the writer object (host memory).  All entry points are thread-safe for
 * distinct writers; the last-error string is per thread.
 */
#ifndef DSPARK_CTX_KV_H
#define DSPARK_CTX_KV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Head size the write supports ("2 * 128" cache rows; rotary_dims_supported). */
#define DSPARK_HEAD_DIM 128
/* Most draft layers one writer handles (a draft has a handful; the offsets
 * ride in the kernel-argument segment). */
#define DSPARK_MAX_LAYERS 32

/* kv_cache_dtype: "auto" (raw bf16 cache) or "fp8" / "fp8_e4m3" (uint8
 * storage holding OCP e4m3), as accepted by DSparkContextKVWriter. */
enum {
    DSPARK_KV_AUTO = 0,
    DSPARK_KV_FP8_E4M3 = 1
};

/* Status codes.  On any non-zero status dspark_ctx_kv_last_error() gives the
 * reason. */
enum {
    DSPARK_OK = 0,
    DSPARK_E_LAYOUT = -1, /* cache layout the writer does not support (_validate) */
    DSPARK_E_ARG = -2,    /* bad argument to write (shape mismatch, rotary dim, pointer) */
    DSPARK_E_HIP = -4     /* the HIP runtime reported an error */
};

typedef struct dspark_ctx_kv_writer dspark_ctx_kv_writer; /* opaque */

/* Element types of a tensor, as the caller's framework reports them. */
enum {
    DSPARK_DTYPE_OTHER = 0, /* any type the write does not take */
    DSPARK_DTYPE_BF16 = 1,
    DSPARK_DTYPE_UINT8 = 2,
    DSPARK_DTYPE_FP32 = 3
};

/* Most dimensions a tensor description carries. */
#define DSPARK_MAX_DIMS 8

/* What the library needs to know of one tensor to check a layout without a
 * framework: its address, element type, where it lives, and its shape and
 * strides (in elements).  A zeroed record (data NULL) means "no tensor". */
typedef struct dspark_tensor_info {
    const void *data;                  /* NULL: the attribute is absent or not a tensor */
    int32_t dtype;                     /* DSPARK_DTYPE_* */
    const char *dtype_name;            /* the framework's name of the type, quoted in
                                          reasons (e.g. "torch.int16"); may be NULL */
    int32_t on_gpu;                    /* 1: GPU device memory; 0: anything else */
    int32_t device_index;              /* which GPU, when on_gpu */
    int32_t ndim;                      /* 0 .. DSPARK_MAX_DIMS */
    int64_t shape[DSPARK_MAX_DIMS];
    int64_t strides[DSPARK_MAX_DIMS];  /* elements */
} dspark_tensor_info;

/* One draft attention layer as the writer sees it: the attributes
 * DSparkContextKVWriter reads from each layer on the vLLM API page
 * "vllm.models.minimax_m3.common.ops.dspark_context_kv" (kv_cache,
 * _k_scale, _v_scale, kv_cache_dtype). */
typedef struct dspark_layer_info {
    const char *kv_cache_dtype;  /* "auto", "fp8" or "fp8_e4m3"; NULL: the layer has none */
    dspark_tensor_info kv_cache; /* [num_blocks, num_kv_heads, block_size, 256] */
    dspark_tensor_info k_scale;  /* fp32 on the GPU, one value read at every write */
    dspark_tensor_info v_scale;
} dspark_layer_info;

/* Host-only check of the layers' cache layout: the rules of
 * DSparkContextKVWriter._validate on the page above, in its order (layers in
 * order, and for each layer the rules in this order; the first rule that
 * fails gives the reason, the page's text):
 *   num_layers >= 1 and layers non-NULL ("no layers");
 *   num_layers <= DSPARK_MAX_LAYERS (a limit of this library);
 *   per layer l:
 *     kv_cache_dtype is "auto", "fp8" or "fp8_e4m3" ("kv_cache_dtype 'x'");
 *     the cache is a tensor with elements ("KV cache not bound");
 *     4 dims, the last 256 = 2 * 128 ("unexpected cache shape (...)");
 *     block_size = shape[2] a power of two;
 *     contiguous (strides of a row-major tensor; dims of size 1 free);
 *     uint8 elements for fp8, bf16 for "auto" ("fp8 cache has dtype ..." /
 *       "cache has dtype ...");
 *     _k_scale then _v_scale each an fp32 tensor on a GPU;
 *     the same shape, strides, element type and kv_cache_dtype as layer 0's
 *       cache ("layers do not share cache shape/stride/dtype");
 *     on layer 0's GPU ("layers are on different devices");
 *     a multiple of 16 elements away from layer 0's cache;
 *   then the library's own limits: layer 0's cache 16-byte aligned, every
 *   scale 4-byte aligned, num_kv_heads and block_size below 2^31.
 * Touches no device.  Returns DSPARK_OK or DSPARK_E_LAYOUT (reason in
 * dspark_ctx_kv_last_error()). */
int dspark_ctx_kv_validate(int32_t num_layers, const dspark_layer_info *layers);

/* Build a writer for the layers' caches: validates as
 * dspark_ctx_kv_validate, then computes the per-layer cache offsets
 * (elements from layer 0's cache) and scale offsets (floats from layer 0's k
 * scale) of _ensure_tables.  num_blocks, num_kv_heads and block_size are the
 * caches' shape[0..2].  The scale VALUES are read on the device at every
 * write, so they may change between calls or graph replays; the cache and
 * scale ADDRESSES may not (destroy and create again to re-bind).  Allocates
 * host memory only.  On success *out receives the writer and the return is
 * DSPARK_OK; otherwise *out is NULL (when out is not) and the return is
 * DSPARK_E_LAYOUT, or DSPARK_E_ARG for out == NULL. */
int dspark_ctx_kv_writer_create(int32_t num_layers, const dspark_layer_info *layers,
                                dspark_ctx_kv_writer **out);

/* Enqueue the fused write on `stream` (a hipStream_t; NULL = the null
 * stream).  One kernel launch; no allocation, synchronisation or copy, so the
 * call can be captured in a HIP graph.  Arguments (device pointers):
 *   all_kv         bf16 [num_ctx, num_layers, 2, num_kv_heads, 128],
 *                  contiguous, 16-byte aligned; axis 2: 0 = K, 1 = V
 *   k_norm_weight  bf16 [num_layers, 128], row l = layer l's K-norm weight w
 *                  (the norm multiplies by 1 + w), 16-byte aligned
 *   eps            the norm's epsilon (used as fp32)
 *   positions      int64 [num_ctx], the row of cos_sin_cache for each token
 *   cos_sin_cache  bf16 [cos_sin_rows, rotary_dim], row p = [cos | sin] of
 *                  the rotary_dim/2 frequencies, 16-byte aligned
 *   rotary_dim     16, 32 or 64 (dspark_rotary_dims_supported)
 *   slot_mapping   int64 [num_ctx]; < 0 = padding, else the cache slot
 * num_layers and num_kv_heads must equal the writer's (the assert in
 * DSparkContextKVWriter.__call__).  num_ctx == 0 returns DSPARK_OK without a
 * launch.  Preconditions NOT checked on the device (as on the page): the
 * position of every token with a slot >= 0 is in [0, cos_sin_rows) (a
 * padding token's position is never used as an index, so it may hold any
 * value), every slot is < num_blocks * block_size, and no two non-padding
 * tokens share a slot (with duplicates either token's values may land).  The buffers must not be
 * written by other work while the kernel runs.  Returns DSPARK_OK,
 * DSPARK_E_ARG or DSPARK_E_HIP (launch failure). */
int dspark_ctx_kv_writer_write(dspark_ctx_kv_writer *w,
                               const void *all_kv, int64_t num_ctx,
                               int32_t num_layers, int32_t num_kv_heads,
                               const void *k_norm_weight, float eps,
                               const int64_t *positions,
                               const void *cos_sin_cache, int64_t cos_sin_rows,
                               int32_t rotary_dim,
                               const int64_t *slot_mapping,
                               void *stream);

/* The same write when every draft layer has its own slot mapping (layers in
 * different KV-cache groups): the case the vLLM API page
 * "vllm.models.minimax_m3.common.dspark" (_shared_slot_mapping) sends to the
 * unfused path, because its fused kernel takes one mapping for all layers.
 * slot_mappings is a host array of num_layers device pointers, each int64
 * [num_ctx], 8-byte aligned; layer l's K and V rows of token t go to
 * slot_mappings[l][t], and a slot < 0 skips that layer only (the token's rows
 * are still read).  Everything else, including the preconditions, is as for
 * dspark_ctx_kv_writer_write; the pointers are taken by value into the
 * launch, so the host array may be reused after the call.  A token's
 * position is used as an index only if its slot is >= 0 in at least one
 * layer.  Returns DSPARK_OK,
 * DSPARK_E_ARG (also for a NULL or misaligned mapping) or DSPARK_E_HIP. */
int dspark_ctx_kv_writer_write_layer_slots(dspark_ctx_kv_writer *w,
                                           const void *all_kv, int64_t num_ctx,
                                           int32_t num_layers, int32_t num_kv_heads,
                                           const void *k_norm_weight, float eps,
                                           const int64_t *positions,
                                           const void *cos_sin_cache,
                                           int64_t cos_sin_rows, int32_t rotary_dim,
                                           const int64_t *const *slot_mappings,
                                           void *stream);

/* Free a writer (host memory only).  No graph that captured a write through
 * it may be replayed afterwards.  NULL is ignored. */
void dspark_ctx_kv_writer_destroy(dspark_ctx_kv_writer *w);

/* 1 if the write supports this rotary dim and head size (rotary_dims_supported:
 * the leading 16, 32 or 64 dims of a 128-dim head), else 0. */
int dspark_rotary_dims_supported(int32_t rotary_dim, int32_t head_dim);

/* The reason for the last non-zero status returned on this thread ("" if
 * none).  Valid until the next call on this thread. */
const char *dspark_ctx_kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_CTX_KV_H */
