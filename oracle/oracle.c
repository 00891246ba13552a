/*
 * Exact-value CPU oracle for the DSpark fused context-KV write.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code, header or table with the HIP path.
 *
 * What it computes follows the vLLM API page
 * "vllm.models.minimax_m3.common.ops.dspark_context_kv" (module docstring and
 * class DSparkContextKVWriter), which defines the fused write as exactly the
 * result of the unfused chain it replaces (permute copy, per-layer K norm +
 * stack, positions.repeat, rotary_embedding, per-layer reshape_and_cache_flash):
 *
 *   for every context token t whose slot is >= 0, every draft layer l and
 *   every kv head h:
 *     K row  = all_kv[t, l, 0, h, :]   (bf16, 128 values)
 *     V row  = all_kv[t, l, 1, h, :]
 *     y      = bf16( x * rsqrt(mean(x^2) + eps) * (1 + w_l) )   Gemma RMSNorm
 *     k'     = partial NeoX RoPE of y at positions[t], leading R dims
 *              (pairs (i, i + R/2), cos_sin_cache row = [cos | sin]),
 *              each result rounded to bf16 as the unfused rotary writes it
 *     store  = cache_l[slot / bs, h, slot % bs, 0:128] = k', [128:256] = V
 *              raw bf16, or fp8 e4m3 of (fp32 value) / (fp32 scale)
 *   every other cache byte stays as it was.
 *
 * Precision.  The page fixes "fp32" for the norm but not the summation
 * order or the rsqrt accuracy, so different correct fp32 programs can round
 * the norm output to different bf16 neighbours.  This oracle evaluates every
 * quantity in fp64, where the squares, the sum, the products of bf16 values
 * and the RoPE products are exact for the workloads here (the only rounding
 * before the bf16 step is the ~2^-52 relative error of sqrt and divide), and
 * rounds once.  A norm output whose fp64 value lies within `near_delta`
 * (relative) of a bf16 rounding midpoint is a near tie: both neighbours are
 * correct answers, and every K code that can follow from either neighbour is
 * reported as an alternate for that element (at most 2 x 2 combinations per
 * RoPE pair).  The fp8 step is fixed by reshape_and_cache_flash semantics:
 * fp32 value divided by the fp32 scale with IEEE division, then e4m3.
 *
 * Codecs are written from the format definitions:
 *   bf16: IEEE-754 binary32 truncated to 8 significand bits (1 sign, 8
 *         exponent, 7 fraction bits), round to nearest, ties to even;
 *   e4m3: OCP 8-bit floating point (OFP8) E4M3: bias 7, no infinities,
 *         S.1111.111 is NaN, largest finite 448 (0x7E), smallest normal 2^-6,
 *         subnormal step 2^-9; round to nearest even, |x| > 448 saturates
 *         to +-448 (the store is a saturating one); zero keeps its sign.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC (x86-64, SSE
 * arithmetic, so float division is the IEEE correctly rounded one).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 --- */

double dspark_oracle_bf16_decode(uint16_t code)
{
    uint32_t u = (uint32_t)code << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a finite double to bf16, ties to even, in one step.
 * If `near_delta` > 0 and |z| lies within near_delta*|z| of the midpoint
 * between its two bf16 neighbours, *near_tie is set and *other receives the
 * neighbour that was not chosen. */
uint16_t dspark_oracle_bf16_round(double z, double near_delta, int *near_tie,
                                  uint16_t *other)
{
    if (near_tie)
        *near_tie = 0;
    uint16_t sign = signbit(z) ? 0x8000u : 0u;
    double a = fabs(z);
    if (a == 0.0) {
        if (other)
            *other = sign;
        return sign;
    }
    int e;
    frexp(a, &e);            /* a = m * 2^e, m in [0.5, 1): binade 2^(e-1) */
    int binade = e - 1;
    if (binade < -126)       /* subnormal range: fixed quantum 2^-133 */
        binade = -126;
    double quantum = ldexp(1.0, binade - 7);   /* one bf16 ulp in this binade */
    double n = a / quantum;                    /* exact: power-of-two scaling */
    double lo = floor(n);
    double frac = n - lo;                      /* exact */
    double k;
    if (frac > 0.5)
        k = lo + 1.0;
    else if (frac < 0.5)
        k = lo;
    else
        k = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;

    /* the chosen value is a bf16 number, hence an fp32 number; fp32 overflow
     * (k * quantum = 2^128) gives infinity, which is the IEEE result */
    float fv = (float)(k * quantum);
    uint32_t u;
    memcpy(&u, &fv, sizeof u);
    uint16_t code = (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFFu));

    if (near_delta > 0.0 && near_tie) {
        double mid = (lo + 0.5) * quantum;
        if (fabs(a - mid) <= near_delta * a) {
            double ko = (k == lo) ? lo + 1.0 : lo;
            float fo = (float)(ko * quantum);
            uint32_t uo;
            memcpy(&uo, &fo, sizeof uo);
            *near_tie = 1;
            if (other)
                *other = (uint16_t)(sign | (uint16_t)((uo >> 16) & 0x7FFFu));
        }
    }
    return code;
}

/* ---------------------------------------------------------------- e4m3 --- */

/* Value of an OCP E4M3 code, from the format definition; NaN for S.1111.111. */
double dspark_oracle_e4m3_decode(uint8_t code)
{
    int s = code >> 7;
    int ex = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (ex == 0xF && m == 0x7)
        return NAN;
    if (ex == 0)
        v = ldexp((double)m, -9);                     /* subnormal: m * 2^-9 */
    else
        v = ldexp(1.0 + (double)m / 8.0, ex - 7);     /* normal */
    return s ? -v : v;
}

/* Saturating round-to-nearest-even encode.  The non-negative finite codes
 * 0x00..0x7E are in increasing order of value, so the nearest code is found
 * by binary search over their decoded values; a tie goes to the even code,
 * which is the code whose significand ends in 0. */
uint8_t dspark_oracle_e4m3_encode(float f)
{
    uint8_t sign = signbit(f) ? 0x80u : 0u;
    if (isnan(f))
        return (uint8_t)(sign | 0x7Fu);
    double a = fabs((double)f);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7Eu);
    int lo = 0, hi = 0x7E;             /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (dspark_oracle_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double vlo = dspark_oracle_e4m3_decode((uint8_t)lo);
    double vhi = dspark_oracle_e4m3_decode((uint8_t)hi);
    int code;
    if (a - vlo < vhi - a)
        code = lo;
    else if (a - vlo > vhi - a)
        code = hi;
    else
        code = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | (uint8_t)code);
}

/* The cache store of an fp8 element: e4m3 of (fp32 value / fp32 scale). */
uint8_t dspark_oracle_fp8_store(uint16_t bf16_value, float scale)
{
    float x = (float)dspark_oracle_bf16_decode(bf16_value);   /* exact */
    float q = x / scale;                                        /* IEEE fp32 */
    return dspark_oracle_e4m3_encode(q);
}

/* --------------------------------------------------------- context-KV --- */

#define HEAD_DIM 128
#define MAX_CAND 4

static int add_candidate(uint16_t *set, int n, uint16_t c)
{
    for (int i = 0; i < n; ++i)
        if (set[i] == c)
            return n;
    set[n] = c;
    return n + 1;
}

/* Gemma RMSNorm of one 128-value bf16 row followed by partial NeoX RoPE, as
 * the unfused chain computes it: the norm x * rsqrt(mean(x^2) + eps) * (1 + w)
 * evaluated exactly (fp64) and rounded once to bf16, then the rotation of the
 * pairs (i, i + R/2) of that bf16 output by the table row [cos | sin], each
 * result rounded once to bf16; dims R..127 keep the norm output.
 * kcode receives the codes; kcand[i][0..ncand[i]) every code that a near tie
 * of the norm output can lead to (kcand[i][0] == kcode[i]). */
static void norm_rope_row(const uint16_t *row, const uint16_t *w, float eps,
                          const uint16_t *cs_row, int R, double near_delta,
                          uint16_t kcode[HEAD_DIM], uint16_t kcand[HEAD_DIM][MAX_CAND],
                          int ncand_k[HEAD_DIM])
{
    double x[HEAD_DIM];
    uint16_t ycode[HEAD_DIM];
    uint16_t ycand[HEAD_DIM][2];
    int ncand_y[HEAD_DIM];

    double ss = 0.0;
    for (int i = 0; i < HEAD_DIM; ++i) {
        x[i] = dspark_oracle_bf16_decode(row[i]);
        ss += x[i] * x[i];
    }
    double r = 1.0 / sqrt(ss / HEAD_DIM + (double)eps);
    for (int i = 0; i < HEAD_DIM; ++i) {
        double wi = dspark_oracle_bf16_decode(w[i]);
        double z = x[i] * r * (1.0 + wi);
        int near = 0;
        uint16_t other = 0;
        ycode[i] = dspark_oracle_bf16_round(z, near_delta, &near, &other);
        ycand[i][0] = ycode[i];
        ncand_y[i] = 1;
        if (near) {
            ycand[i][1] = other;
            ncand_y[i] = 2;
        }
    }
    for (int i = 0; i < HEAD_DIM; ++i) {
        kcode[i] = ycode[i];
        ncand_k[i] = 0;
    }
    for (int i = 0; i < R / 2; ++i) {
        int j = i + R / 2;
        double c = dspark_oracle_bf16_decode(cs_row[i]);
        double s = dspark_oracle_bf16_decode(cs_row[R / 2 + i]);
        double a0 = dspark_oracle_bf16_decode(ycode[i]);
        double b0 = dspark_oracle_bf16_decode(ycode[j]);
        kcode[i] = dspark_oracle_bf16_round(a0 * c - b0 * s, 0.0, NULL, NULL);
        kcode[j] = dspark_oracle_bf16_round(b0 * c + a0 * s, 0.0, NULL, NULL);
        for (int ia = 0; ia < ncand_y[i]; ++ia) {
            for (int ib = 0; ib < ncand_y[j]; ++ib) {
                double a = dspark_oracle_bf16_decode(ycand[i][ia]);
                double b = dspark_oracle_bf16_decode(ycand[j][ib]);
                ncand_k[i] = add_candidate(kcand[i], ncand_k[i],
                    dspark_oracle_bf16_round(a * c - b * s, 0.0, NULL, NULL));
                ncand_k[j] = add_candidate(kcand[j], ncand_k[j],
                    dspark_oracle_bf16_round(b * c + a * s, 0.0, NULL, NULL));
            }
        }
    }
    for (int i = R; i < HEAD_DIM; ++i) {
        ncand_k[i] = 0;
        for (int ia = 0; ia < ncand_y[i]; ++ia)
            ncand_k[i] = add_candidate(kcand[i], ncand_k[i], ycand[i][ia]);
    }
}

/* Record an element with more than one correct code. */
static void record_alternates(int64_t *n_alt, int64_t capacity, int64_t tag, int64_t index,
                              const uint16_t *codes, int nc, int64_t *alt_tag,
                              int64_t *alt_index, int32_t *alt_count, uint16_t *alt_codes)
{
    if (nc <= 1)
        return;
    if (*n_alt < capacity) {
        alt_tag[*n_alt] = tag;
        alt_index[*n_alt] = index;
        alt_count[*n_alt] = nc;
        for (int q = 0; q < MAX_CAND; ++q)
            alt_codes[*n_alt * MAX_CAND + q] = q < nc ? codes[q] : 0;
    }
    ++*n_alt;
}

/*
 * The whole write, on host buffers.
 *
 * all_kv         bf16 bits [num_ctx, L, 2, nkv, 128] (axis 2: 0 = K, 1 = V)
 * k_norm_weight  bf16 bits [L, 128], row l is layer l's K-norm weight w
 * eps            the norm epsilon, as fp32
 * positions      int64 [num_ctx]
 * cos_sin        bf16 bits [cs_rows, R], row p = [cos(p*theta_i) | sin(...)]
 * slot_mapping   int64; layer l uses slot_mapping[l * slot_layer_stride + t]:
 *                stride 0 = one mapping [num_ctx] shared by every layer, stride
 *                num_ctx = one mapping per layer [L, num_ctx] (draft layers in
 *                different KV-cache groups); < 0 is padding for that layer
 * caches         L host pointers, each [num_blocks, nkv, bs, 256] of uint16
 *                (bf16 cache) or uint8 (fp8 cache)
 * k_scales, v_scales  fp32 [L] (read only for fp8 caches)
 * near_delta     relative distance to a bf16 midpoint that makes a near tie
 * alt_*          receive K elements with more than one correct code:
 *                layer, element index in that layer's cache, the number of
 *                codes and up to 4 codes each; at most alt_capacity entries
 * t_begin, t_end the token range to process
 *
 * Returns the number of K elements with alternates (may exceed
 * alt_capacity; only the first alt_capacity are recorded), or a negative
 * value when a precondition fails: -1 rotary dim, -2 block size, -3 position
 * out of the cos/sin table, -4 slot out of the cache, -5 sizes.
 */
int64_t dspark_oracle_ctx_kv_write(
    const uint16_t *all_kv, int64_t num_ctx, int32_t num_layers, int32_t nkv,
    const uint16_t *k_norm_weight, float eps,
    const int64_t *positions, const uint16_t *cos_sin, int64_t cs_rows,
    int32_t rotary_dim,
    const int64_t *slot_mapping, int64_t slot_layer_stride,
    int64_t num_blocks, int32_t block_size,
    int32_t fp8, const float *k_scales, const float *v_scales,
    void *const *caches,
    double near_delta,
    int64_t *alt_layer, int64_t *alt_index, int32_t *alt_count,
    uint16_t *alt_codes, int64_t alt_capacity,
    int64_t t_begin, int64_t t_end)
{
    const int R = rotary_dim;
    if (R != 16 && R != 32 && R != 64)
        return -1;
    if (block_size <= 0 || (block_size & (block_size - 1)))
        return -2;
    if (num_layers <= 0 || nkv <= 0 || num_ctx < 0 || t_begin < 0 ||
        t_end > num_ctx || t_begin > t_end)
        return -5;

    int64_t n_alt = 0;
    uint16_t kcand[HEAD_DIM][MAX_CAND];
    int ncand_k[HEAD_DIM];
    uint16_t kcode[HEAD_DIM];

    for (int64_t t = t_begin; t < t_end; ++t) {
        for (int l = 0; l < num_layers; ++l) {
            int64_t slot = slot_mapping[l * slot_layer_stride + t];
            if (slot < 0)
                continue;                           /* padding: not written */
            if (slot >= num_blocks * (int64_t)block_size)
                return -4;
            int64_t blk = slot / block_size;
            int64_t off = slot % block_size;
            int64_t p = positions[t];
            if (p < 0 || p >= cs_rows)
                return -3;
            const uint16_t *cs_row = cos_sin + p * R;   /* same row for every layer */

            for (int h = 0; h < nkv; ++h) {
                const uint16_t *krow =
                    all_kv + (((t * num_layers + l) * 2 + 0) * nkv + h) * HEAD_DIM;
                const uint16_t *vrow =
                    all_kv + (((t * num_layers + l) * 2 + 1) * nkv + h) * HEAD_DIM;

                norm_rope_row(krow, k_norm_weight + l * HEAD_DIM, eps, cs_row, R, near_delta,
                              kcode, kcand, ncand_k);

                /* store into layer l's cache at [blk, h, off, :] */
                int64_t row = ((blk * nkv + h) * block_size + off) * (2 * HEAD_DIM);
                for (int i = 0; i < HEAD_DIM; ++i) {
                    uint16_t codes[MAX_CAND];
                    int nc = 0;
                    if (fp8) {
                        uint8_t *cache = (uint8_t *)caches[l];
                        cache[row + i] = dspark_oracle_fp8_store(kcode[i], k_scales[l]);
                        cache[row + HEAD_DIM + i] = dspark_oracle_fp8_store(vrow[i], v_scales[l]);
                        for (int q = 0; q < ncand_k[i]; ++q)
                            nc = add_candidate(codes, nc,
                                dspark_oracle_fp8_store(kcand[i][q], k_scales[l]));
                    } else {
                        uint16_t *cache = (uint16_t *)caches[l];
                        cache[row + i] = kcode[i];
                        cache[row + HEAD_DIM + i] = vrow[i];     /* bit copy */
                        for (int q = 0; q < ncand_k[i]; ++q)
                            nc = add_candidate(codes, nc, kcand[i][q]);
                    }
                    record_alternates(&n_alt, alt_capacity, l, row + i, codes, nc,
                                      alt_layer, alt_index, alt_count, alt_codes);
                }
            }
        }
    }
    return n_alt;
}

/* ------------------------------------------- draft-block QK norm + RoPE --- */

/*
 * The fused QK-norm / RoPE on the draft block's qkv, also storing the draft
 * tokens' K/V (vLLM API page "vllm.models.minimax_m3.common.dspark",
 * dspark_qknorm_rope_kv_insert; the per-head Gemma RMSNorm on Q and K before
 * partial RoPE is the NeMo page's description of the same draft attention).
 *
 * qkv            bf16 bits [num_tokens, (H + 2 nkv) * 128]: H q heads, then
 *                nkv k heads, then nkv v heads; rewritten in place: every q
 *                and k head is replaced by its normed and rotated bf16 value,
 *                v heads are left as they are
 * q_norm_weight, k_norm_weight  bf16 bits [128], shared by the heads
 * positions      int64 [num_tokens]; cos_sin bf16 bits [cs_rows, R]
 * slot_mapping   NULL (no insert) or int64 [num_tokens], < 0 = not stored
 * cache          NULL or [num_blocks, nkv, bs, 256] of uint16 (bf16) or uint8
 *                (fp8): K at [..., :128], V at [..., 128:]
 * k_scale, v_scale  fp32 scales of an fp8 cache
 * q_fp8          NULL or uint8 [num_tokens, H * 128]: e4m3 of q / q_scale
 * alt_tag        which output an alternate belongs to: 0 qkv, 1 cache, 2 q_fp8
 *
 * Returns the number of alternates, or -1 rotary dim, -2 block size,
 * -3 position, -4 slot, -5 sizes.
 */
int64_t dspark_oracle_qknorm_rope_kv_insert(
    uint16_t *qkv, int64_t num_tokens, int32_t num_heads, int32_t nkv,
    const uint16_t *q_norm_weight, const uint16_t *k_norm_weight, float eps,
    const int64_t *positions, const uint16_t *cos_sin, int64_t cs_rows, int32_t rotary_dim,
    const int64_t *slot_mapping, void *cache, int64_t num_blocks, int32_t block_size,
    int32_t fp8, float k_scale, float v_scale,
    uint8_t *q_fp8, float q_scale,
    double near_delta,
    int64_t *alt_tag, int64_t *alt_index, int32_t *alt_count, uint16_t *alt_codes,
    int64_t alt_capacity)
{
    const int R = rotary_dim;
    if (R != 16 && R != 32 && R != 64)
        return -1;
    if (slot_mapping != NULL && (block_size <= 0 || (block_size & (block_size - 1))))
        return -2;
    if (num_tokens < 0 || num_heads <= 0 || nkv <= 0)
        return -5;
    const int64_t row_len = (int64_t)(num_heads + 2 * nkv) * HEAD_DIM;
    int64_t n_alt = 0;
    uint16_t kcand[HEAD_DIM][MAX_CAND];
    int ncand_k[HEAD_DIM];
    uint16_t kcode[HEAD_DIM];
    uint16_t src[HEAD_DIM];

    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t p = positions[t];
        if (p < 0 || p >= cs_rows)
            return -3;
        const uint16_t *cs_row = cos_sin + p * R;
        int64_t slot = -1;
        if (slot_mapping != NULL && cache != NULL) {
            slot = slot_mapping[t];
            if (slot >= num_blocks * (int64_t)block_size)
                return -4;
        }
        uint16_t *tok = qkv + t * row_len;

        /* q heads, then k heads: norm + RoPE, written back in place */
        for (int hh = 0; hh < num_heads + nkv; ++hh) {
            const int is_k = hh >= num_heads;
            uint16_t *row = tok + (int64_t)hh * HEAD_DIM;
            memcpy(src, row, sizeof src);
            norm_rope_row(src, is_k ? k_norm_weight : q_norm_weight, eps, cs_row, R,
                          near_delta, kcode, kcand, ncand_k);
            for (int i = 0; i < HEAD_DIM; ++i) {
                row[i] = kcode[i];
                record_alternates(&n_alt, alt_capacity, 0, t * row_len + hh * HEAD_DIM + i,
                                  kcand[i], ncand_k[i], alt_tag, alt_index, alt_count,
                                  alt_codes);
            }
            if (!is_k && q_fp8 != NULL) {
                uint8_t *out = q_fp8 + (t * num_heads + hh) * HEAD_DIM;
                for (int i = 0; i < HEAD_DIM; ++i) {
                    uint16_t codes[MAX_CAND];
                    int nc = 0;
                    out[i] = dspark_oracle_fp8_store(kcode[i], q_scale);
                    for (int q = 0; q < ncand_k[i]; ++q)
                        nc = add_candidate(codes, nc, dspark_oracle_fp8_store(kcand[i][q], q_scale));
                    record_alternates(&n_alt, alt_capacity, 2,
                                      (t * num_heads + hh) * HEAD_DIM + i, codes, nc,
                                      alt_tag, alt_index, alt_count, alt_codes);
                }
            }
            if (is_k && slot >= 0) {
                int h = hh - num_heads;
                int64_t crow = ((slot / block_size * nkv + h) * block_size + slot % block_size) *
                               (2 * HEAD_DIM);
                for (int i = 0; i < HEAD_DIM; ++i) {
                    uint16_t codes[MAX_CAND];
                    int nc = 0;
                    if (fp8) {
                        ((uint8_t *)cache)[crow + i] = dspark_oracle_fp8_store(kcode[i], k_scale);
                        for (int q = 0; q < ncand_k[i]; ++q)
                            nc = add_candidate(codes, nc, dspark_oracle_fp8_store(kcand[i][q], k_scale));
                    } else {
                        ((uint16_t *)cache)[crow + i] = kcode[i];
                        for (int q = 0; q < ncand_k[i]; ++q)
                            nc = add_candidate(codes, nc, kcand[i][q]);
                    }
                    record_alternates(&n_alt, alt_capacity, 1, crow + i, codes, nc, alt_tag,
                                      alt_index, alt_count, alt_codes);
                }
            }
        }
        /* v heads: stored as they are */
        if (slot >= 0) {
            for (int h = 0; h < nkv; ++h) {
                const uint16_t *vrow = tok + (int64_t)(num_heads + nkv + h) * HEAD_DIM;
                int64_t crow = ((slot / block_size * nkv + h) * block_size + slot % block_size) *
                               (2 * HEAD_DIM) + HEAD_DIM;
                for (int i = 0; i < HEAD_DIM; ++i) {
                    if (fp8)
                        ((uint8_t *)cache)[crow + i] = dspark_oracle_fp8_store(vrow[i], v_scale);
                    else
                        ((uint16_t *)cache)[crow + i] = vrow[i];
                }
            }
        }
    }
    return n_alt;
}

/* ------------------------------------------- the step before the write --- */

/*
 * Gemma RMSNorm of `rows` rows of `dim` bf16 values (the draft's hidden_norm
 * on the context states, vLLM API page "vllm.models.minimax_m3.common.dspark":
 * _gemma_rms_norm, _normalize_context_states):
 *
 *   out[r, i] = bf16( x[r, i] * rsqrt(mean_i(x[r, i]^2) + eps) * (1 + w[i]) )
 *
 * evaluated in fp64 and rounded once (the same reading of "fp32" as for the
 * K norm).  An element within near_delta (relative) of a bf16 midpoint is a
 * near tie: its flat index and the other neighbour are recorded (at most
 * alt_capacity of them).  Returns the number of near ties.
 */
int64_t dspark_oracle_gemma_rms_norm(const uint16_t *x, int64_t rows, int32_t dim,
                                     const uint16_t *w, float eps, uint16_t *out,
                                     double near_delta, int64_t *alt_index,
                                     uint16_t *alt_other, int64_t alt_capacity)
{
    int64_t n_alt = 0;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * dim;
        double ss = 0.0;
        for (int i = 0; i < dim; ++i) {
            double v = dspark_oracle_bf16_decode(xr[i]);
            ss += v * v;
        }
        double rs = 1.0 / sqrt(ss / dim + (double)eps);
        for (int i = 0; i < dim; ++i) {
            double z = dspark_oracle_bf16_decode(xr[i]) * rs * (1.0 + dspark_oracle_bf16_decode(w[i]));
            int near = 0;
            uint16_t other = 0;
            out[r * dim + i] = dspark_oracle_bf16_round(z, near_delta, &near, &other);
            if (near) {
                if (n_alt < alt_capacity) {
                    alt_index[n_alt] = r * dim + i;
                    alt_other[n_alt] = other;
                }
                ++n_alt;
            }
        }
    }
    return n_alt;
}

/*
 * The token-major K/V projection (_project_context_kv_token_major on the same
 * page): all_kv[t, c] = bf16( sum_k z[t, k] * W[c, k] ) for the rows
 * [r_begin, r_end) and columns [c_begin, c_end) of the output, where z is
 * [rows, hidden] (the hidden_norm output) and W is [cols, hidden] (a linear
 * layer's [out, in] weight); column c = ((l * 2 + kv) * nkv + h) * 128 + d,
 * so the output read as [rows, L, 2, nkv, 128] is all_kv.
 *
 * Products of bf16 values are exact in fp64 and the sum's rounding error is
 * below hidden * 2^-53 of sum |z W|, so the value rounded to bf16 is the
 * exactly rounded sum (a tie decided by that error is not possible unless
 * the sum lies within ~2^-40 relative of a midpoint).  out, and exact /
 * abs_sum when not NULL, are the selected block [r_end - r_begin,
 * c_end - c_begin], row-major: the bf16 code, the fp64 sum and sum |z W| (for
 * error bounds of fp32 accumulation).
 */
void dspark_oracle_kv_project(const uint16_t *z, int32_t hidden, const uint16_t *W,
                              int64_t r_begin, int64_t r_end, int64_t c_begin, int64_t c_end,
                              uint16_t *out, double *exact, double *abs_sum)
{
    const int64_t bc = c_end - c_begin;
    const int64_t br = r_end - r_begin;
    /* the block's z rows and one W row at a time, decoded to fp64 */
    double *zd = (double *)malloc(sizeof(double) * (size_t)(br * hidden + 1));
    double *wc = (double *)malloc(sizeof(double) * (size_t)hidden);
    if (!zd || !wc) {
        free(zd);
        free(wc);
        return;
    }
    for (int64_t r = r_begin; r < r_end; ++r)
        for (int k = 0; k < hidden; ++k)
            zd[(r - r_begin) * hidden + k] = dspark_oracle_bf16_decode(z[r * hidden + k]);
    for (int64_t c = c_begin; c < c_end; ++c) {
        for (int k = 0; k < hidden; ++k)
            wc[k] = dspark_oracle_bf16_decode(W[c * hidden + k]);
        for (int64_t r = r_begin; r < r_end; ++r) {
            const double *zp = zd + (r - r_begin) * hidden;
            double s = 0.0, a = 0.0;
            for (int k = 0; k < hidden; ++k) {
                double p = zp[k] * wc[k];
                s += p;
                a += fabs(p);
            }
            const int64_t o = (r - r_begin) * bc + (c - c_begin);
            out[o] = dspark_oracle_bf16_round(s, 0.0, NULL, NULL);
            if (exact)
                exact[o] = s;
            if (abs_sum)
                abs_sum[o] = a;
        }
    }
    free(zd);
    free(wc);
}
