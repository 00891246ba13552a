/*
 * dspark_qknorm_insert.h - C ABI of the draft block's fused QK-norm / RoPE /
 * KV insert for MI355X (gfx950).
 *
 * The operation is ops.fused_minimax_m3_qknorm_rope_kv_insert as the vLLM API
 * page "vllm.models.minimax_m3.common.dspark" calls it from
 * dspark_qknorm_rope_kv_insert: on the draft block's fused projection output
 * qkv [num_tokens, (H + 2 nkv) * 128] (bf16; H query heads, then nkv key
 * heads, then nkv value heads, 128 dims each), every query and key head is
 * replaced in place by
 *
 *   partial NeoX RoPE( bf16( x * rsqrt(mean(x^2) + eps) * (1 + w) ) )
 *
 * (the Gemma RMSNorm of the head in fp32 with q_norm_weight for query heads
 * and k_norm_weight for key heads, its output rounded to bf16; RoPE on the
 * leading rotary_dim dims, pairs (i, i + rotary_dim/2), at the token's
 * cos_sin_cache row, each result rounded to bf16), exactly as the context
 * write of dspark_ctx_kv.h treats K.  Value heads are not changed.  When a
 * slot mapping is given (the attention context has one), the token's key and
 * value heads are also stored at kv_cache[slot / block_size, h, slot %
 * block_size, 0:128] (K, after norm and RoPE) and [..., 128:256] (V), as raw
 * bf16 or as OCP fp8 e4m3 of (fp32 value) / (fp32 scale); slots < 0 are not
 * stored.  When q_fp8_out is given it receives e4m3 of every rotated query
 * value divided by q_fp8_scale (the layer's _q_scale_float), saturating at
 * +-448, in addition to the in-place bf16 query.
 *
 * One kernel launch, no allocation, synchronisation or copy: the call can be
 * captured in a HIP graph.  The caller owns every buffer and the stream.
 */
#ifndef DSPARK_QKNORM_INSERT_H
#define DSPARK_QKNORM_INSERT_H

#include <stdint.h>

#include "dspark_ctx_kv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue the fused QK-norm / RoPE / KV insert on `stream` (a hipStream_t;
 * NULL = the null stream).  Device pointers:
 *   qkv             bf16 [num_tokens, (num_heads + 2 num_kv_heads) * 128],
 *                   contiguous, 16-byte aligned; read and written in place
 *   q_norm_weight   bf16 [128], the query heads' norm weight w (the norm
 *                   multiplies by 1 + w), 16-byte aligned
 *   k_norm_weight   bf16 [128], the key heads' norm weight, 16-byte aligned
 *   cos_sin_cache   bf16 [cos_sin_rows, rotary_dim] = [cos | sin] rows,
 *                   16-byte aligned
 *   positions       int64 [num_tokens], the cos_sin_cache row of each token
 *   slot_mapping    int64 [num_tokens] or NULL.  NULL: no insert (kv_cache,
 *                   num_blocks, block_size, kv_cache_dtype and the scales are
 *                   then ignored).  Else < 0 = not stored, otherwise the slot
 *   kv_cache        [num_blocks, num_kv_heads, block_size, 256] of bf16
 *                   (DSPARK_KV_AUTO) or uint8 holding e4m3
 *                   (DSPARK_KV_FP8_E4M3), contiguous, 16-byte aligned
 *   block_size      a power of two (kv_cache.size(2))
 *   k_scale,v_scale fp32 scalars on the device, read at every call, or NULL
 *                   for 1.0 (the page's call passes no scale; see the design
 *                   notes); used by an fp8 cache only
 *   q_fp8_out       uint8 [num_tokens, num_heads * 128] or NULL, 8-byte aligned
 *   q_fp8_scale     the query fp8 scale (host value, finite and > 0 when
 *                   q_fp8_out is given)
 * rotary_dim is 16, 32 or 64 (dspark_rotary_dims_supported).  num_tokens == 0
 * returns DSPARK_OK without a launch.  Preconditions NOT checked on the
 * device: every position is in [0, cos_sin_rows) (query and key heads are
 * rotated for every token, stored or not), every slot is < num_blocks *
 * block_size, no two stored tokens share a slot, device scales are finite and
 * > 0, and q_fp8_out does not overlap qkv.  Returns DSPARK_OK, DSPARK_E_ARG
 * (the reason in dspark_ctx_kv_last_error()) or DSPARK_E_HIP. */
int dspark_qknorm_rope_kv_insert(void *qkv, int64_t num_tokens,
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
                                 void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_QKNORM_INSERT_H */
