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
// Work decomposition.  The write moves about 8 KB per token per layer group
// and does about one flop per byte: it is bound by HBM bandwidth, nothing in
// it is a dense contraction (no MFMA), and its vector-ALU work must stay well
// under the bandwidth budget (a wave64 fp32 instruction costs 4 cycles of a
// 16-lane SIMD).  So:
//   * a wavefront owns 4 (token, kv head) rows, one per quarter (16 lanes =
//     one DPP row), each lane holding 8 bf16 (16 bytes) of a 128-dim row;
//   * the wave walks the L layers; per layer one instruction covers the 4
//     K rows and one the 4 V rows, so every lane of a K instruction does
//     useful norm/RoPE work and V rows are a plain copy (bf16) or a scaled
//     conversion (fp8);
//   * every K and V load of the wave's layers is issued before any math;
//   * the 128-wide sum of squares is reduced inside the 16-lane row with four
//     DPP adds (no LDS); every lane ends with the same bits;
//   * the RoPE partner of element i (i + R/2) sits in the same register of
//     lane c ^ (R/16), fetched with one DPP move (R = 16, 32) or ds_swizzle
//     (R = 64);
//   * the token's cos/sin values are loaded once per row into registers and
//     reused for every layer;
//   * fp8: x / scale is formed from y = RN(1/scale) (one IEEE division per
//     wave gives every layer's reciprocals, one per lane) as q0 = x y,
//     r = fma(q0, scale, -x), q = fma(-r, y, q0), which is the correctly
//     rounded quotient for every finite bf16 x at the e4m3 resolution
//     (Markstein's correction step) on x clamped to +-460 scale, which also
//     keeps the result inside the e4m3 range; then the hardware pack
//     conversion v_cvt_pk_fp8_f32 (OCP e4m3 on gfx950).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ctx_kv_args.h"

namespace dspark {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = 64 * kWavesPerBlock;
constexpr int kRowsPerWave = 4;
constexpr int kMaxChunk = 8;   // layers held in registers at once
// Cache policy of the streams: all_kv is read once and the cache rows are
// written once, so both go through the nontemporal (streaming) path.
constexpr bool kStreamLoads = true;
constexpr bool kStreamStores = true;
// Workgroup i runs on XCD i % 8; remapping gives each XCD a contiguous range
// of rows.
constexpr bool kXcdRemap = true;
constexpr int kNumXcds = 8;

// DPP control codes (CDNA3/CDNA4 ISA, DPP_CTRL field).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
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
        // lane ^ 4 within 32 lanes: ds_swizzle bit mode (and 0x1f, or 0,
        // xor 4); it runs in the LDS crossbar, not the VALU
        (void)c;
        return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x101F));
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
    int w0 = 0, w1 = 0;
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

// kChunk = layers held in registers per pass; kSinglePass: L == kChunk (the
// whole write is one straight-line pass), else L > kChunk and the layers go
// in chunks of kChunk.
// kUniform: nkv % 4 == 0, so a wave's 4 rows are 4 heads of one token and the
// token's slot and position are wave-uniform (scalar loads, scalar exit).
// kLayerSlots: every layer has its own slot mapping (layers in different KV
// cache groups); always with the general row mapping.
template <int R, bool kFp8, int kChunk, bool kSinglePass, bool kUniform, bool kLayerSlots>
__global__ __launch_bounds__(kBlockThreads) void ctx_kv_write_kernel(const CtxKvArgs a) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4;        // quarter: which of the wave's 4 rows
    const int c = lane & 15;        // 16-byte chunk: elements 8c .. 8c+7
    const int L = kSinglePass ? kChunk : a.num_layers;
    const int nkv = a.nkv;

    uint32_t block = blockIdx.x;
    if constexpr (kXcdRemap) {
        // blocks [0, full) are remapped so that XCD x owns one contiguous run
        const uint32_t full = gridDim.x - gridDim.x % kNumXcds;
        if (block < full) block = (block % kNumXcds) * (full / kNumXcds) + block / kNumXcds;
    }
    const uint32_t wave = block * kWavesPerBlock +
                          static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    const uint32_t unit0 = wave * kRowsPerWave;             // first row of the wave
    if (unit0 >= a.num_units) return;

    uint32_t t;
    int h;
    int64_t slot, pos;
    uint4 dk[kChunk], dv[kChunk], wv[kChunk];
    int64_t lslot[kChunk];          // per-layer slots (kLayerSlots only)
    bool in_range = true;
    const int64_t kv_stride = static_cast<int64_t>(nkv) * 16;    // K_l -> V_l (uint4 units)
    const uint4 *w_base = reinterpret_cast<const uint4 *>(a.k_norm_weight) + c;
    const uint4 *kv_base;
    // every K, V and weight load of the chunk goes out before any arithmetic;
    // all_kv[t, l, kv, h, 8c..8c+7] = kv_base + (l * 2 + kv) * nkv * 16
    auto load_chunk = [&](int lb) {
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const int l = (lb + j < L) ? lb + j : L - 1;   // a short last chunk repeats a row
            dk[j] = load_row16(kv_base + (2 * l) * kv_stride);
            dv[j] = load_row16(kv_base + (2 * l + 1) * kv_stride);
            wv[j] = w_base[l * 16];
            if constexpr (kLayerSlots) lslot[j] = a.layer_slots[l][t];
        }
    };
    if constexpr (kUniform) {
        t = unit0 / static_cast<uint32_t>(nkv);
        h = static_cast<int>(unit0 - t * static_cast<uint32_t>(nkv)) + q;
        kv_base = reinterpret_cast<const uint4 *>(a.all_kv) +
                  (static_cast<int64_t>(t) * L * 2 * nkv + h) * 16 + c;
        slot = a.slots[t];
        pos = a.positions[t];
        // The row loads do not depend on the slot: they go out together with
        // the slot load, so the slot's latency overlaps theirs (a padding
        // token's rows are then read for nothing).  The barrier keeps the
        // compiler from sinking them below the padding exit.
        load_chunk(0);
        asm volatile("" ::: "memory");
        // padding: nothing written (a negative position never occurs; testing
        // it keeps both scalar loads ahead of the branch)
        if (slot < 0 || pos < 0) return;
    } else if constexpr (kLayerSlots) {
        // Each layer's store has its own slot: every in-range quarter reads
        // its rows (a quarter past the end reads the wave's first row) and
        // each layer's stores are predicated on that layer's slot.
        const uint32_t unit = unit0 + q;                    // (token, kv head) row
        in_range = unit < a.num_units;
        t = (in_range ? unit : unit0) / static_cast<uint32_t>(nkv);
        h = static_cast<int>((in_range ? unit : unit0) - t * static_cast<uint32_t>(nkv));
        slot = 0;
        pos = a.positions[t];
        kv_base = reinterpret_cast<const uint4 *>(a.all_kv) +
                  (static_cast<int64_t>(t) * L * 2 * nkv + h) * 16 + c;
        load_chunk(0);
        asm volatile("" ::: "memory");   // keep the loads ahead of the predicated stores
    } else {
        const uint32_t unit = unit0 + q;                    // (token, kv head) row
        in_range = unit < a.num_units;
        t = (in_range ? unit : unit0) / static_cast<uint32_t>(nkv);
        h = static_cast<int>((in_range ? unit : unit0) - t * static_cast<uint32_t>(nkv));
        slot = a.slots[t];
        pos = a.positions[t];
        const bool valid = in_range && slot >= 0;
        const uint64_t valid_mask = __ballot(valid);
        if (valid_mask == 0) return;
        // A quarter without a row of its own mirrors the first valid quarter:
        // it reads the same rows, computes the same bytes and stores them to
        // the same place.  Identical addresses in one instruction move no
        // extra bytes, and every load and store stays unconditional (no branch
        // for the compiler to sink a load into).
        const int src = static_cast<int>(__builtin_ctzll(valid_mask));
        if (!valid) {
            t = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(t), src));
            h = __builtin_amdgcn_readlane(h, src);
            pos = read_lane64(pos, src);
            slot = read_lane64(slot, src);
        }
        kv_base = reinterpret_cast<const uint4 *>(a.all_kv) +
                  (static_cast<int64_t>(t) * L * 2 * nkv + h) * 16 + c;
        load_chunk(0);
    }

    // this token's (cos, sin) for the 8 pair indices of this lane
    constexpr int kRotLanes = R / 8;
    uint32_t cs[8];
    {
        const int cr = c % kRotLanes;                 // lanes past R re-read lane cr's chunk
        const int i0 = (cr * 8) % (R / 2);
        const uint16_t *cs_row = a.cos_sin + pos * R;
        const uint4 cv = *reinterpret_cast<const uint4 *>(cs_row + i0);
        const uint4 sv = *reinterpret_cast<const uint4 *>(cs_row + R / 2 + i0);
        const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
        const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
        // first half of the rotated dims: k = y c - p s; second half: y c + p s
        const uint32_t sign = (c < kRotLanes / 2) ? 0x80000000u : 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            cs[2 * k] = __builtin_amdgcn_perm(sw[k], cw[k], 0x05040100u) ^ sign;
            cs[2 * k + 1] = __builtin_amdgcn_perm(sw[k], cw[k], 0x07060302u) ^ sign;
        }
    }

    const int64_t blk = slot >> a.bs_log2;
    const int64_t off = slot & ((int64_t{1} << a.bs_log2) - 1);
    // element index of this row inside any layer's cache, plus this lane's chunk
    const int64_t row = ((((blk * nkv + h) << a.bs_log2) + off) * (2 * DSPARK_HEAD_DIM)) + c * 8;

    for (int lb = 0;;) {
        // fp8: lane 2j holds layer lb+j's k scale, lane 2j+1 its v scale, and
        // one IEEE division gives every reciprocal of the chunk
        float my_scale = 1.0f, my_rcp = 1.0f;
        if constexpr (kFp8) {
            int64_t soff = 0;
            bool has = false;
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                if (lb + j < L) {
                    if (lane == 2 * j) { soff = a.kscale_off[lb + j]; has = true; }
                    if (lane == 2 * j + 1) { soff = a.vscale_off[lb + j]; has = true; }
                }
            }
            if (has) my_scale = a.scale0[soff];
            my_rcp = 1.0f / my_scale;
        }
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const int l = lb + j;
            if (l >= L) break;
            uint32_t kb[4];
            norm_rope<R>(dk[j], wv[j], a.eps, c, cs, kb);
            int64_t base = a.cache_off[l] + row;
            bool store = true;
            if constexpr (kLayerSlots) {
                const int64_t s = lslot[j];
                store = in_range && s >= 0;
                const int64_t lb_blk = s >> a.bs_log2;
                const int64_t lb_off = s & ((int64_t{1} << a.bs_log2) - 1);
                base = a.cache_off[l] +
                       ((((lb_blk * nkv + h) << a.bs_log2) + lb_off) * (2 * DSPARK_HEAD_DIM)) + c * 8;
            }
            if constexpr (!kFp8) {
                uint16_t *cache = static_cast<uint16_t *>(a.cache0) + base;
                if (store) {
                    store_row16(cache, make_uint4(kb[0], kb[1], kb[2], kb[3]));
                    store_row16(cache + DSPARK_HEAD_DIM, dv[j]);
                }
            } else {
                const float ks = lane_value(my_scale, 2 * j), kr = lane_value(my_rcp, 2 * j);
                const float vs = lane_value(my_scale, 2 * j + 1), vr = lane_value(my_rcp, 2 * j + 1);
                const uint32_t vb[4] = {dv[j].x, dv[j].y, dv[j].z, dv[j].w};
                const uint2 ko = pack_fp8(kb, ks, kr, 460.0f * ks);
                const uint2 vo = pack_fp8(vb, vs, vr, 460.0f * vs);
                uint8_t *cache = static_cast<uint8_t *>(a.cache0) + base;
                if (store) {
                    store_row8(cache, ko);
                    store_row8(cache + DSPARK_HEAD_DIM, vo);
                }
            }
        }
        if constexpr (kSinglePass) {
            break;
        } else {
            lb += kChunk;
            if (lb >= L) break;
            load_chunk(lb);
        }
    }
}

template <int R, bool kFp8, int kChunk, bool kSinglePass>
void launch_one(const CtxKvArgs &a, hipStream_t stream) {
    const uint32_t waves = (a.num_units + kRowsPerWave - 1) / kRowsPerWave;
    const dim3 grid((waves + kWavesPerBlock - 1) / kWavesPerBlock);
    if (a.layer_slots_on)
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, kChunk, kSinglePass, false, true>), grid,
                           dim3(kBlockThreads), 0, stream, a);
    else if (a.nkv % kRowsPerWave == 0)
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, kChunk, kSinglePass, true, false>), grid,
                           dim3(kBlockThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, kChunk, kSinglePass, false, false>), grid,
                           dim3(kBlockThreads), 0, stream, a);
}

template <int R, bool kFp8>
hipError_t launch_r(const CtxKvArgs &a, hipStream_t stream) {
    switch (a.num_layers) {
    case 1: launch_one<R, kFp8, 1, true>(a, stream); break;
    case 2: launch_one<R, kFp8, 2, true>(a, stream); break;
    case 3: launch_one<R, kFp8, 3, true>(a, stream); break;
    case 4: launch_one<R, kFp8, 4, true>(a, stream); break;
    case 5: launch_one<R, kFp8, 5, true>(a, stream); break;
    case 6: launch_one<R, kFp8, 6, true>(a, stream); break;
    case 7: launch_one<R, kFp8, 7, true>(a, stream); break;
    case 8: launch_one<R, kFp8, 8, true>(a, stream); break;
    default: launch_one<R, kFp8, kMaxChunk, false>(a, stream); break;
    }
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
