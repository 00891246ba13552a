// Device helpers shared by the DSpark kernels for CDNA4 (gfx950): DPP row
// reductions and moves, streaming 16- and 8-byte row accesses, bf16 and OCP
// e4m3 packing, the correctly rounded division by a scale, and the Gemma
// RMSNorm + partial NeoX RoPE of one 128-dim head held as 16 lanes x 8 bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dspark_ctx_kv.h"

namespace dspark {
namespace {

// Cache policy of the streams: inputs are read once and go through the
// nontemporal (streaming) path; so do the stores of store_row16/store_row8
// (the context write's scattered cache rows use the sc1 stores below where
// it can).
constexpr bool kStreamLoads = true;
constexpr bool kStreamStores = true;
// DPP control codes (CDNA3/CDNA4 ISA, DPP_CTRL field).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;     // lane i <- lane 15 - i
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7 - i within each half row
constexpr int kRowRor4 = 0x124;       // lane i <- lane (i - 4) mod 16 of its row
constexpr int kRowRor12 = 0x12C;      // lane i <- lane (i + 4) mod 16 of its row

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
        // lane c ^ 4: row_ror:12 brings lane c + 4 (for c & 4 == 0), row_ror:4
        // lane c - 4 (for c & 4 != 0); two DPP moves and a select measured 2%
        // faster on the fp8 prefill than one ds_swizzle (an LDS round trip
        // that the RoPE then waits for)
        const uint32_t up = dpp_u32<kRowRor12>(v), down = dpp_u32<kRowRor4>(v);
        return (c & 4) ? down : up;
    }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_row16(const uint4 *p) {
    if constexpr (kStreamLoads) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

__device__ __forceinline__ void store_row16(void *p, const uint4 &v) {
    if constexpr (kStreamStores) {
        const u32x4 w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, static_cast<u32x4 *>(p));
    } else {
        *static_cast<uint4 *>(p) = v;
    }
}

__device__ __forceinline__ void store_row8(void *p, const uint2 &v) {
    if constexpr (kStreamStores) {
        const u32x2 w = {v.x, v.y};
        __builtin_nontemporal_store(w, static_cast<u32x2 *>(p));
    } else {
        *static_cast<uint2 *>(p) = v;
    }
}

// Stores with the sc1 cache policy (device scope) through a buffer resource
// whose base is a wave-uniform address: the lanes add byte offsets below
// 2^31.  On the write's scattered rows this measured 9% more HBM throughput
// than nontemporal stores (a copy of the same address pattern: 6.1 vs 5.6
// TB/s).  The resource has no range limit: offsets are the caller's to bound.
constexpr int kStoreSc1 = 16;   // cache-policy bit sc1 of a buffer store

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void *wave_base) {
    const uint64_t a = reinterpret_cast<uint64_t>(wave_base);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)));
    const uint32_t hi =
        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)));
    void *p = reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, -1, 0x00020000);
}

__device__ __forceinline__ void store16_sc1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                            const uint4 &v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, static_cast<int>(byte_off), 0, kStoreSc1);
}

__device__ __forceinline__ void store8_sc1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                           const uint2 &v) {
    const u32x2 w = {v.x, v.y};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, static_cast<int>(byte_off), 0, kStoreSc1);
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

// a.lo * b.lo + a.hi * b.hi + acc over packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
}

// The 64-bit value v holds in lane `lane` (wave-uniform result).
__device__ __forceinline__ int64_t read_lane64(int64_t v, int lane) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), lane));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The value register v holds in lane `lane` (wave-uniform result).
__device__ __forceinline__ float lane_value(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// fp32 quotient x / s rounded as IEEE division would, given y = RN(1 / s)
// (Markstein's correction step, residual negated so that +-0 keep their
// sign).  x is first clamped to +-lim = +-460 s: a quotient at or beyond that
// stores 448 either way, the clamped quotient stays below 464 so the e4m3
// conversion cannot overflow (no separate saturation needed), and x y cannot
// reach infinity.
__device__ __forceinline__ float div_by_scale(float x, float s, float y, float lim) {
    const float xc = __builtin_amdgcn_fmed3f(x, -lim, lim);
    const float q0 = xc * y;
    const float rn = __builtin_fmaf(q0, s, -xc);
    return __builtin_fmaf(-rn, y, q0);
}

// 8 bf16 (packed in 4 words) -> 8 OCP e4m3 bytes of value / s.
__device__ __forceinline__ uint2 pack_fp8(const uint32_t (&b)[4], float s, float y, float lim) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = div_by_scale(bf16_lo(b[k]), s, y, lim);
        v[2 * k + 1] = div_by_scale(bf16_hi(b[k]), s, y, lim);
    }
    // the first conversion of each word sets its low half; the high half it
    // keeps from `old` is overwritten by the second, so `old` is any value
    // already in a register (no zeroing move)
    int w0 = __builtin_bit_cast(int, v[0]), w1 = __builtin_bit_cast(int, v[4]);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], w0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], w1, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
    return make_uint2(static_cast<uint32_t>(w0), static_cast<uint32_t>(w1));
}

// Norm + RoPE of one K row chunk (8 values in this lane) -> 4 packed bf16.
// cs[e] packs element e's (cos, +-sin) as bf16 (sin negated on the first
// half of the rotated dims), or (1, 0) on lanes past the rotated dims.
template <int R>
__device__ __forceinline__ void norm_rope(const uint4 &d, const uint4 &w, float eps, int c,
                                          const uint32_t (&cs)[8], uint32_t (&out)[4]) {
    constexpr int kRotLanes = R / 8;   // lanes holding rotated dims
    const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    // sum of squares: bf16 x bf16 products are exact in fp32
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) ss = dot2_bf16(dw[k], dw[k], ss);
    ss = row_sum16(ss);
    const float r = __builtin_amdgcn_rsqf(ss * (1.0f / DSPARK_HEAD_DIM) + eps);
    // y = (x r)(1 + w) = fma(x r, w, x r): 1 + w is exact in fp32, so both
    // forms round the same product once
    uint32_t yb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float xr0 = bf16_lo(dw[k]) * r, xr1 = bf16_hi(dw[k]) * r;
        yb[k] = pack_bf16(__builtin_fmaf(xr0, bf16_lo(ww[k]), xr0),
                          __builtin_fmaf(xr1, bf16_hi(ww[k]), xr1));
    }
    // partial NeoX RoPE on the bf16 norm output: k = y c + p s' as one bf16
    // dot product of (y, p) with (c, s'): both products are exact in fp32
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t pb = rope_partner<R>(yb[k], c);
        const float r0 = dot2_bf16(__builtin_amdgcn_perm(pb, yb[k], 0x05040100u), cs[2 * k], 0.0f);
        const float r1 = dot2_bf16(__builtin_amdgcn_perm(pb, yb[k], 0x07060302u), cs[2 * k + 1], 0.0f);
        out[k] = (c < kRotLanes) ? pack_bf16(r0, r1) : yb[k];
    }
}

// This lane's RoPE operands for the token whose [cos | sin] row is cs_row:
// cs[e] packs element e's (cos, +-sin) as bf16, sin negated on the first half
// of the rotated dims (k = y c - p s there, y c + p s on the second half).
// Lanes past the rotated dims get the values of lane c % (R / 8), which
// norm_rope ignores.
template <int R>
__device__ __forceinline__ void rope_operands(const uint16_t *cs_row, int c, uint32_t (&cs)[8]) {
    constexpr int kRotLanes = R / 8;
    const int cr = c % kRotLanes;
    const int i0 = (cr * 8) % (R / 2);
    const uint4 cv = *reinterpret_cast<const uint4 *>(cs_row + i0);
    const uint4 sv = *reinterpret_cast<const uint4 *>(cs_row + R / 2 + i0);
    const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
    const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
    const uint32_t sign = (c < kRotLanes / 2) ? 0x80000000u : 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        cs[2 * k] = __builtin_amdgcn_perm(sw[k], cw[k], 0x05040100u) ^ sign;
        cs[2 * k + 1] = __builtin_amdgcn_perm(sw[k], cw[k], 0x07060302u) ^ sign;
    }
}

}  // namespace
}  // namespace dspark
