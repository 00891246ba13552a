// Fused DSpark context-KV write for CDNA4 (gfx950).
//
// Computes what the vLLM API page
// "vllm.models.minimax_m3.common.ops.dspark_context_kv" defines (module
// docstring, DSparkContextKVWriter): per (token, layer, kv head), K gets the
// layer's Gemma RMSNorm x * rsqrt(mean(x^2) + eps) * (1 + w) in fp32, rounded
// to bf16, then partial NeoX RoPE on the leading R dims (pairs (i, i + R/2),
// table row [cos | sin] at the token's position), each result rounded to
// bf16; V passes unchanged.  Both land in layer l's paged cache row
// [slot / bs, h, slot % bs, :] (K at 0..127, V at 128..255), as bf16 bits or
// as OCP e4m3 of value / scale.  Padding slots (< 0) read and write nothing.
//
// Work decomposition (HBM-bound: about one flop per byte, no contraction, so
// no MFMA):
//   * one wavefront per (token, kv head) unit, covering all L layers;
//   * the wave's 4 quarters (16 lanes, one DPP row each) hold 4 rows of 128
//     bf16 at 8 values (16 bytes) per lane: K of layer l, V of layer l,
//     K of layer l+1, V of layer l+1.  A quarter pair's store is one
//     contiguous 512-byte (bf16) or 256-byte (fp8) cache row segment;
//   * every row load of the unit is issued before any arithmetic;
//   * the 128-wide sum of squares is reduced inside the 16-lane row with four
//     DPP adds (no LDS), leaving the identical sum in all 16 lanes;
//   * the RoPE partner of element i (i + R/2) sits in the same register of
//     lane c ^ (R/16), fetched with one DPP move;
//   * the token's cos/sin values are loaded once per wave into registers and
//     reused for every layer;
//   * fp8: division by the fp32 scale (IEEE), clamp to +-448, then the
//     hardware pack conversion v_cvt_pk_fp8_f32 (OCP e4m3 on gfx950).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ctx_kv_args.h"

namespace dspark {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = 64 * kWavesPerBlock;

// DPP control codes (CDNA3/CDNA4 ISA, DPP_CTRL field).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowShl4 = 0x104;       // lane i <- lane i + 4 within the row
constexpr int kRowShr4 = 0x114;       // lane i <- lane i - 4 within the row
constexpr int kRowMirror = 0x140;     // lane i <- lane 15 - i
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7 - i within each half row

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xF, 0xF, true));
}

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, dpp_u32<kCtrl>(__builtin_bit_cast(uint32_t, v)));
}

// Sum over the 16 lanes of a DPP row; every lane ends with the same bits
// (each step adds two equal-valued operands in commuted order).
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp_f32<kQuadXor1>(v);
    v += dpp_f32<kQuadXor2>(v);
    v += dpp_f32<kRowHalfMirror>(v);
    v += dpp_f32<kRowMirror>(v);
    return v;
}

// Value of lane (c ^ (R / 16)) of the same 16-lane row.
template <int R>
__device__ __forceinline__ uint32_t rope_partner(uint32_t v, int c) {
    if constexpr (R == 16) {
        return dpp_u32<kQuadXor1>(v);
    } else if constexpr (R == 32) {
        return dpp_u32<kQuadXor2>(v);
    } else {
        const uint32_t up = dpp_u32<kRowShl4>(v);
        const uint32_t dn = dpp_u32<kRowShr4>(v);
        return (c & 4) ? dn : up;
    }
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// Two fp32 -> packed bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 b = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float clamp448(float x) {
    return __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f);
}

// 8 floats -> 8 OCP e4m3 bytes of x / scale.
__device__ __forceinline__ uint2 pack_fp8(const float (&v)[8], float scale) {
    int w0 = 0, w1 = 0;
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v[0] / scale), clamp448(v[1] / scale), w0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v[2] / scale), clamp448(v[3] / scale), w0, true);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v[4] / scale), clamp448(v[5] / scale), w1, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v[6] / scale), clamp448(v[7] / scale), w1, true);
    return make_uint2(static_cast<uint32_t>(w0), static_cast<uint32_t>(w1));
}

// kGroups = number of 4-row groups (2 layers each) loaded before any math.
template <int R, bool kFp8, int kGroups>
__global__ __launch_bounds__(kBlockThreads) void ctx_kv_write_kernel(const CtxKvArgs a) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4;        // row slot of this quarter: 0 K_l, 1 V_l, 2 K_l+1, 3 V_l+1
    const int c = lane & 15;        // 16-byte chunk: elements 8c .. 8c+7
    const int kv = q & 1;
    const int lhalf = q >> 1;

    const uint32_t unit = blockIdx.x * kWavesPerBlock +
                          __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (unit >= a.num_units) return;
    const int L = a.num_layers;
    const int nkv = a.nkv;
    const uint32_t t = unit / static_cast<uint32_t>(nkv);
    const int h = static_cast<int>(unit - t * static_cast<uint32_t>(nkv));

    const int64_t slot = a.slots[t];
    if (slot < 0) return;           // padding: nothing read, nothing written
    const int64_t pos = a.positions[t];
    const int64_t blk = slot >> a.bs_log2;
    const int64_t off = slot & ((int64_t{1} << a.bs_log2) - 1);
    // element index of this unit's row inside any layer's cache
    const int64_t row = (((blk * nkv + h) << a.bs_log2) + off) * (2 * DSPARK_HEAD_DIM);

    // this token's cos/sin for the 8 pair indices of this lane (rotated dims only)
    constexpr int kRotLanes = R / 8;
    float cs_c[8], cs_s[8];
    if (c < kRotLanes) {
        const int i0 = (c * 8) % (R / 2);
        const uint16_t *cs_row = a.cos_sin + pos * R;
        const uint4 cv = *reinterpret_cast<const uint4 *>(cs_row + i0);
        const uint4 sv = *reinterpret_cast<const uint4 *>(cs_row + R / 2 + i0);
        const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
        const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            cs_c[2 * k] = bf16_lo(cw[k]);
            cs_c[2 * k + 1] = bf16_hi(cw[k]);
            cs_s[2 * k] = bf16_lo(sw[k]);
            cs_s[2 * k + 1] = bf16_hi(sw[k]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            cs_c[k] = 1.0f;
            cs_s[k] = 0.0f;
        }
    }
    // first half of the rotated dims: k = y c - y' s; second half: k = y c + y' s
    const float sin_sign = (c < kRotLanes / 2) ? -1.0f : 1.0f;

    const uint4 *kv_base = reinterpret_cast<const uint4 *>(a.all_kv) +
                           static_cast<int64_t>(t) * L * 2 * nkv * 16 + h * 16 + c;
    const uint4 *w_base = reinterpret_cast<const uint4 *>(a.k_norm_weight) + c;

    for (int lb = 0; lb < L; lb += 2 * kGroups) {
        uint4 d[kGroups];
        uint4 wv[kGroups];
#pragma unroll
        for (int j = 0; j < kGroups; ++j) {
            const int l = lb + 2 * j + lhalf;
            d[j] = make_uint4(0, 0, 0, 0);
            wv[j] = make_uint4(0, 0, 0, 0);
            if (l < L) {
                d[j] = kv_base[(l * 2 + kv) * nkv * 16];
                wv[j] = w_base[l * 16];
            }
        }
#pragma unroll
        for (int j = 0; j < kGroups; ++j) {
            const int l0 = lb + 2 * j;
            if (l0 >= L) break;
            const int l = l0 + lhalf;

            const uint32_t dw[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
            const uint32_t ww[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
            float x[8], w1[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[2 * k] = bf16_lo(dw[k]);
                x[2 * k + 1] = bf16_hi(dw[k]);
                w1[2 * k] = 1.0f + bf16_lo(ww[k]);
                w1[2 * k + 1] = 1.0f + bf16_hi(ww[k]);
            }
            // Gemma RMSNorm in fp32 (computed by every quarter; V quarters
            // discard it)
            float ss = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) ss = __builtin_fmaf(x[k], x[k], ss);
            ss = row_sum16(ss);
            const float r = __builtin_amdgcn_rsqf(ss * (1.0f / DSPARK_HEAD_DIM) + a.eps);
            uint32_t yb[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                yb[k] = pack_bf16((x[2 * k] * r) * w1[2 * k], (x[2 * k + 1] * r) * w1[2 * k + 1]);

            // partial NeoX RoPE on the bf16 norm output
            uint32_t pb[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) pb[k] = rope_partner<R>(yb[k], c);
            float kf[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float y0 = bf16_lo(yb[k]), y1 = bf16_hi(yb[k]);
                const float p0 = bf16_lo(pb[k]), p1 = bf16_hi(pb[k]);
                // p * s is exact in fp32 (two 8-bit significands); the fma
                // rounds the exact y c +- p s once to fp32.  Dims past R keep y.
                kf[2 * k] = (c < kRotLanes)
                    ? __builtin_fmaf(y0, cs_c[2 * k], sin_sign * (p0 * cs_s[2 * k])) : y0;
                kf[2 * k + 1] = (c < kRotLanes)
                    ? __builtin_fmaf(y1, cs_c[2 * k + 1], sin_sign * (p1 * cs_s[2 * k + 1])) : y1;
            }

            // layers of the lower (l0) and upper (l1) half-wave: uniform scalars
            const int l1 = (l0 + 1 < L) ? l0 + 1 : l0;
            const int64_t cache_off = lhalf ? a.cache_off[l1] : a.cache_off[l0];
            if (l < L) {
                if constexpr (!kFp8) {
                    uint4 out;
                    if (kv == 0) {
                        out = make_uint4(pack_bf16(kf[0], kf[1]), pack_bf16(kf[2], kf[3]),
                                         pack_bf16(kf[4], kf[5]), pack_bf16(kf[6], kf[7]));
                    } else {
                        out = d[j];
                    }
                    uint4 *dst = reinterpret_cast<uint4 *>(
                        static_cast<uint16_t *>(a.cache0) + cache_off + row + kv * DSPARK_HEAD_DIM + c * 8);
                    *dst = out;
                } else {
                    const float ks0 = a.scale0[a.kscale_off[l0]], ks1 = a.scale0[a.kscale_off[l1]];
                    const float vs0 = a.scale0[a.vscale_off[l0]], vs1 = a.scale0[a.vscale_off[l1]];
                    const float ks = lhalf ? ks1 : ks0;
                    const float vs = lhalf ? vs1 : vs0;
                    float v[8];
                    if (kv == 0) {
                        // the K cached is the bf16 RoPE output
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const uint32_t kb = pack_bf16(kf[2 * k], kf[2 * k + 1]);
                            v[2 * k] = bf16_lo(kb);
                            v[2 * k + 1] = bf16_hi(kb);
                        }
                    } else {
#pragma unroll
                        for (int k = 0; k < 8; ++k) v[k] = x[k];
                    }
                    const uint2 out = pack_fp8(v, kv ? vs : ks);
                    uint2 *dst = reinterpret_cast<uint2 *>(
                        static_cast<uint8_t *>(a.cache0) + cache_off + row + kv * DSPARK_HEAD_DIM + c * 8);
                    *dst = out;
                }
            }
        }
    }
}

template <int R, bool kFp8>
hipError_t launch_r(const CtxKvArgs &a, hipStream_t stream) {
    const dim3 grid((a.num_units + kWavesPerBlock - 1) / kWavesPerBlock);
    const dim3 block(kBlockThreads);
    const int groups = (a.num_layers + 1) / 2;
    if (groups <= 1)
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, 1>), grid, block, 0, stream, a);
    else if (groups == 2)
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, 2>), grid, block, 0, stream, a);
    else if (groups == 3)
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, 3>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, 4>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ctx_kv(const CtxKvArgs &a, int rotary_dim, bool fp8, hipStream_t stream) {
    switch (rotary_dim) {
    case 16: return fp8 ? launch_r<16, true>(a, stream) : launch_r<16, false>(a, stream);
    case 32: return fp8 ? launch_r<32, true>(a, stream) : launch_r<32, false>(a, stream);
    case 64: return fp8 ? launch_r<64, true>(a, stream) : launch_r<64, false>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dspark
