// Fused QK-norm / partial RoPE / KV insert on the draft block's qkv, for
// CDNA4 (gfx950).
//
// Computes what ops.fused_minimax_m3_qknorm_rope_kv_insert does when the vLLM
// API page "vllm.models.minimax_m3.common.dspark" calls it from
// dspark_qknorm_rope_kv_insert: each query and key head of qkv
// [T, (H + 2 nkv) * 128] is replaced in place by the Gemma RMSNorm of the head
// (fp32, rounded to bf16) followed by partial NeoX RoPE at the token's
// position (each result rounded to bf16), the same per-row arithmetic as the
// context write; with a slot mapping, every token with slot >= 0 also has its
// key heads (after RoPE) and value heads (as they are) stored into the paged
// cache row [slot / bs, h, slot % bs, :] (K at 0..127, V at 128..255) as bf16
// or OCP e4m3 of value / scale; with a q fp8 output, the rotated query heads
// are also written as e4m3 of value / q_scale.
//
// Work decomposition.  The op streams the draft block once: about 1 flop per
// byte, so it is HBM-bound and nothing here is a dense contraction (no MFMA).
// A wavefront owns 4 consecutive 128-dim heads of the flattened
// [T * (H + 2 nkv)] head list, one per quarter (16 lanes = one DPP row, 8 bf16
// per lane), so one instruction normalises and rotates 4 heads, whatever mix
// of query, key and value heads the 4 are: each quarter picks its own norm
// weight and its own destinations, and stores are predicated per quarter.
// When H + 2 nkv is a multiple of 4 the wave's heads share one token and its
// position and slot are wave-uniform.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "qknorm_insert_args.h"

namespace dspark {
namespace {

constexpr int kInsWavesPerBlock = 4;
constexpr int kInsBlockThreads = 64 * kInsWavesPerBlock;
constexpr int kInsRowsPerWave = 4;
constexpr int kInsNumXcds = 8;

// kCache: what the insert stores (kNoInsert, kInsertBf16, kInsertFp8);
// kQFp8: the e4m3 query output is written; kUniform: (H + 2 nkv) % 4 == 0.
template <int R, int kCache, bool kQFp8, bool kUniform>
__global__ __launch_bounds__(kInsBlockThreads) void qknorm_insert_kernel(const InsertArgs a) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4;        // quarter: which of the wave's 4 heads
    const int c = lane & 15;        // 16-byte chunk: elements 8c .. 8c+7

    // Workgroup i runs on XCD i % 8: give each XCD a contiguous run of heads
    uint32_t block = blockIdx.x;
    const uint32_t full = gridDim.x - gridDim.x % kInsNumXcds;
    if (block < full) block = (block % kInsNumXcds) * (full / kInsNumXcds) + block / kInsNumXcds;
    const uint32_t wave = block * kInsWavesPerBlock +
                          static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    const uint32_t unit0 = wave * kInsRowsPerWave;
    if (unit0 >= a.num_rows) return;

    const uint32_t nh = static_cast<uint32_t>(a.heads_per_token);
    const int H = a.num_heads;
    const int nkv = a.nkv;
    // a quarter past the last head reads the last head and stores nothing
    const bool in_range = unit0 + q < a.num_rows;
    const uint32_t u = in_range ? unit0 + q : a.num_rows - 1;
    uint32_t t;
    int hh;
    if constexpr (kUniform) {
        t = unit0 / nh;
        hh = static_cast<int>(unit0 - t * nh) + q;
    } else {
        t = u / nh;
        hh = static_cast<int>(u - t * nh);
    }
    const bool is_q = hh < H;
    const bool is_v = hh >= H + nkv;

    // qkv[t, hh, 8c .. 8c+7]: the flat head index u addresses it directly
    uint4 *row = reinterpret_cast<uint4 *>(a.qkv) + static_cast<int64_t>(u) * 16 + c;
    const uint4 d = load_row16(row);
    const uint4 w = *(reinterpret_cast<const uint4 *>(is_q ? a.q_w : a.k_w) + c);
    const int64_t pos = a.positions[t];
    int64_t slot = -1;
    if constexpr (kCache != kNoInsert) slot = a.slots[t];

    uint32_t cs[8];
    rope_operands<R>(a.cos_sin + pos * R, c, cs);
    uint32_t out[4];
    norm_rope<R>(d, w, a.eps, c, cs, out);

    // query and key heads go back in place; value heads are left alone
    if (in_range && !is_v) store_row16(row, make_uint4(out[0], out[1], out[2], out[3]));

    if constexpr (kCache != kNoInsert || kQFp8) {
        // what a key or value head stores: K after RoPE, V as read
        const uint32_t res[4] = {is_v ? d.x : out[0], is_v ? d.y : out[1],
                                 is_v ? d.z : out[2], is_v ? d.w : out[3]};
        const bool to_cache = kCache != kNoInsert && in_range && !is_q && slot >= 0;
        // kv head index and element offset of this lane's chunk in the cache
        const int h = hh - H - (is_v ? nkv : 0);
        const int64_t blk = slot >> a.bs_log2;
        const int64_t off = slot & ((int64_t{1} << a.bs_log2) - 1);
        const int64_t crow = ((((blk * nkv + h) << a.bs_log2) + off) * (2 * DSPARK_HEAD_DIM)) +
                             (is_v ? DSPARK_HEAD_DIM : 0) + c * 8;
        if constexpr (kCache == kInsertBf16) {
            if (to_cache)
                store_row16(static_cast<uint16_t *>(a.cache) + crow,
                            make_uint4(res[0], res[1], res[2], res[3]));
        }
        if constexpr (kCache == kInsertFp8 || kQFp8) {
            // per quarter: q_scale for a query head, the k or v scale otherwise
            float s = a.q_scale;
            if (!is_q) {
                const float *p = is_v ? a.v_scale : a.k_scale;
                s = p ? *p : 1.0f;
            }
            const float y = 1.0f / s;
            const uint2 f8 = pack_fp8(res, s, y, 460.0f * s);
            if constexpr (kQFp8) {
                if (in_range && is_q)
                    store_row8(a.q_fp8 + (static_cast<int64_t>(t) * H + hh) * DSPARK_HEAD_DIM + c * 8,
                               f8);
            }
            if constexpr (kCache == kInsertFp8) {
                if (to_cache) store_row8(static_cast<uint8_t *>(a.cache) + crow, f8);
            }
        }
    }
}

template <int R, int kCache, bool kQFp8>
void launch_c(const InsertArgs &a, hipStream_t stream) {
    const uint32_t waves = (a.num_rows + kInsRowsPerWave - 1) / kInsRowsPerWave;
    const dim3 grid((waves + kInsWavesPerBlock - 1) / kInsWavesPerBlock);
    if (a.heads_per_token % kInsRowsPerWave == 0)
        hipLaunchKernelGGL((qknorm_insert_kernel<R, kCache, kQFp8, true>), grid,
                           dim3(kInsBlockThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((qknorm_insert_kernel<R, kCache, kQFp8, false>), grid,
                           dim3(kInsBlockThreads), 0, stream, a);
}

template <int R>
void launch_r(const InsertArgs &a, InsertCache cache, bool q_fp8, hipStream_t stream) {
    switch (cache) {
    case kNoInsert:
        q_fp8 ? launch_c<R, kNoInsert, true>(a, stream) : launch_c<R, kNoInsert, false>(a, stream);
        break;
    case kInsertBf16:
        q_fp8 ? launch_c<R, kInsertBf16, true>(a, stream) : launch_c<R, kInsertBf16, false>(a, stream);
        break;
    case kInsertFp8:
        q_fp8 ? launch_c<R, kInsertFp8, true>(a, stream) : launch_c<R, kInsertFp8, false>(a, stream);
        break;
    }
}

}  // namespace

hipError_t launch_qknorm_insert(const InsertArgs &a, int rotary_dim, InsertCache cache,
                                bool q_fp8, hipStream_t stream) {
    switch (rotary_dim) {
    case 16: launch_r<16>(a, cache, q_fp8, stream); break;
    case 32: launch_r<32>(a, cache, q_fp8, stream); break;
    case 64: launch_r<64>(a, cache, q_fp8, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dspark
