/*
 * dspark_project.h - C ABI of the step before the DSpark context-KV write on
 * MI355X (gfx950): the Gemma hidden norm of the context states and the
 * token-major K/V projection, with the context write fused into the
 * projection's epilogue.
 *
 * What is computed follows the vLLM API page
 * "vllm.models.minimax_m3.common.dspark" (MiniMaxM3DSparkModel):
 * _normalize_context_states applies the draft's Gemma hidden_norm
 * (_gemma_rms_norm) to the target's context states,
 * _project_context_kv_token_major multiplies them by the stacked K/V
 * projection of every draft layer into all_kv [num_ctx, L, 2, nkv, 128], and
 * precompute_and_store_context_kv hands all_kv to the fused context write
 * (dspark_ctx_kv.h).  Here the write runs inside the projection kernel, so
 * all_kv is never stored.
 */
#ifndef DSPARK_PROJECT_H
#define DSPARK_PROJECT_H

#include <stdint.h>

#include "dspark_ctx_kv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Gemma RMSNorm of every row: out[r, i] = bf16( x[r, i] * rsqrt(mean_i
 * x[r, i]^2 + eps) * (1 + weight[i]) ), the norm in fp32.  x and out are bf16
 * [rows, dim] (they may be the same buffer), weight bf16 [dim]; all three
 * 16-byte aligned; dim a positive multiple of 8.  One launch on `stream` (a
 * hipStream_t, NULL = null stream), no allocation; rows == 0 returns DSPARK_OK
 * without a launch.  Returns DSPARK_OK, DSPARK_E_ARG (reason in
 * dspark_ctx_kv_last_error()) or DSPARK_E_HIP. */
int dspark_hidden_norm(const void *x, int64_t rows, int32_t dim, const void *weight, float eps,
                       void *out, void *stream);

/* The projection all_kv = bf16(states @ kv_weight^T) with the context write
 * of dspark_ctx_kv_writer_write applied to it in the same kernel:
 *   states     bf16 [num_ctx, hidden], the hidden-norm output, contiguous,
 *              16-byte aligned; hidden a positive multiple of 64;
 *              (num_ctx + 256) * hidden * 2 below 2^31 bytes
 *   kv_weight  bf16 [num_layers * 2 * num_kv_heads * 128, hidden], a linear
 *              layer's [out, in] weight whose output row is ordered as
 *              all_kv's (layer, K/V, kv head, dim), 16-byte aligned, below
 *              2^31 bytes
 * and the remaining arguments exactly as for dspark_ctx_kv_writer_write
 * (the writer's layers, kv heads, caches and scales; k_norm_weight, eps,
 * positions, cos_sin_cache, rotary_dim, slot_mapping, and its
 * preconditions).  The projection accumulates in fp32 on the matrix cores
 * and rounds each all_kv value to bf16 before the write's norm and RoPE, as
 * the unfused projection's bf16 output would be.  One kernel launch, no
 * allocation, synchronisation or copy (graph-capturable).  num_ctx == 0
 * returns DSPARK_OK without a launch.  Returns DSPARK_OK, DSPARK_E_ARG or
 * DSPARK_E_HIP. */
int dspark_ctx_kv_writer_project_write(dspark_ctx_kv_writer *w, const void *states,
                                       int64_t num_ctx, int32_t hidden, const void *kv_weight,
                                       int32_t num_layers, int32_t num_kv_heads,
                                       const void *k_norm_weight, float eps,
                                       const int64_t *positions, const void *cos_sin_cache,
                                       int64_t cos_sin_rows, int32_t rotary_dim,
                                       const int64_t *slot_mapping, void *stream);

/* The projection's weight in its fragment-major layout, for
 * dspark_ctx_kv_writer_project_write_packed.  kv_weight is bf16 [cols, hidden]
 * (row-major, as above); packed receives the same cols * hidden bf16
 * values, element (c, k) at index
 *     ((c / 32) * (hidden / 16) + k / 16) * 512 + 8 * (c % 32 + 32 * ((k % 16) / 8)) + k % 8,
 * so that each 32 x 16 operand fragment of the matrix cores (32 output
 * columns by 16 inputs, in the lane order the MFMA reads it) is 1 KB
 * contiguous.  A weight is static, so it is packed once (a permutation:
 * no arithmetic, no rounding).  cols a positive multiple of 32, hidden of
 * 16, cols * hidden * 2 below 2^31 bytes; both buffers device memory,
 * 16-byte aligned, not overlapping; the caller owns both.  One launch on
 * `stream`, no allocation.  Returns DSPARK_OK, DSPARK_E_ARG or
 * DSPARK_E_HIP. */
int dspark_kv_weight_pack(const void *kv_weight, int64_t cols, int32_t hidden, void *packed,
                          void *stream);

/* dspark_ctx_kv_writer_project_write with the weight packed by
 * dspark_kv_weight_pack (same hidden and cols = num_layers * 2 *
 * num_kv_heads * 128); every other argument, precondition, return value and
 * result as there, bit for bit: the same products are accumulated in the
 * same order.  The kernel loads the packed weight straight into registers
 * instead of staging it in LDS. */
int dspark_ctx_kv_writer_project_write_packed(dspark_ctx_kv_writer *w, const void *states,
                                              int64_t num_ctx, int32_t hidden,
                                              const void *packed_kv_weight, int32_t num_layers,
                                              int32_t num_kv_heads, const void *k_norm_weight,
                                              float eps, const int64_t *positions,
                                              const void *cos_sin_cache, int64_t cos_sin_rows,
                                              int32_t rotary_dim, const int64_t *slot_mapping,
                                              void *stream);

/* dspark_ctx_kv_writer_project_write (weight_packed == 0, kv_weight
 * row-major) or dspark_ctx_kv_writer_project_write_packed (weight_packed ==
 * 1, kv_weight from dspark_kv_weight_pack) that also stores the projection's
 * bf16 output all_kv [num_ctx, num_layers, 2, num_kv_heads, 128] to
 * all_kv_out: exactly the values the write's norm, RoPE and conversion were
 * applied to (the token-major projection's output on the vLLM API page
 * "vllm.models.minimax_m3.common.dspark", _project_context_kv_token_major).
 * For callers that need all_kv itself besides the caches, and for checking
 * the fused kernel; the store adds num_ctx * cols * 2 bytes of traffic.
 * all_kv_out: device memory, contiguous, 16-byte aligned, not overlapping any
 * other argument, owned by the caller.  Every other argument, precondition,
 * cache byte and return value as for those entry points; DSPARK_E_ARG also
 * for a NULL or misaligned all_kv_out (num_ctx > 0) or weight_packed other
 * than 0 or 1. */
int dspark_ctx_kv_writer_project_write_all_kv(dspark_ctx_kv_writer *w, const void *states,
                                              int64_t num_ctx, int32_t hidden,
                                              const void *kv_weight, int32_t weight_packed,
                                              int32_t num_layers, int32_t num_kv_heads,
                                              const void *k_norm_weight, float eps,
                                              const int64_t *positions,
                                              const void *cos_sin_cache, int64_t cos_sin_rows,
                                              int32_t rotary_dim, const int64_t *slot_mapping,
                                              void *all_kv_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_PROJECT_H */
