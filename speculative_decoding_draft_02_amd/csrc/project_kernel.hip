// The step before the context write, for CDNA4 (gfx950): the Gemma hidden
// norm of the context states, and the token-major K/V projection with the
// write in its epilogue, so that all_kv never goes through HBM.
//
// What it computes follows the vLLM API page
// "vllm.models.minimax_m3.common.dspark" (MiniMaxM3DSparkModel:
// _normalize_context_states with the Gemma hidden_norm,
// _project_context_kv_token_major, then the fused write of
// precompute_and_store_context_kv): z = bf16(GemmaRMSNorm(states)),
// all_kv = bf16(z @ W^T) read as [N, L, 2, nkv, 128], then for every
// (token, layer, kv head) the context write (K: norm, RoPE; V as is) into
// layer l's paged cache at the token's slot.
//
// The projection is a dense contraction, so it runs on the matrix cores:
// v_mfma_f32_32x32x16_bf16 (lane l holds A[l % 32][8 (l / 32) + i] and
// B[8 (l / 32) + i][l % 32], i < 8; accumulator register i holds
// D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32]).  A workgroup of 4 waves (one per
// SIMD) owns a 256-token x 256-column tile (with a packed weight, mostly
// 128 tokens x 512 columns); each wave computes 128 tokens x 128 columns,
// and 128 columns are exactly one (layer, kv, head) row of
// all_kv, so the write's per-row norm, RoPE and store happen on data the wave
// holds.  The weight is the MFMA's first operand, so a lane ends with one
// token's values in runs of 4 consecutive columns (half of the head; lane
// l ^ 32 holds the other half): the norm's sum of squares is local adds and
// one exchange, and every RoPE partner column is in the same lane.  Operands
// go from memory straight into a ring of LDS stages (buffer loads with the
// lds bit; rows past num_ctx read as zero), whose 16-byte chunks are
// XOR-swizzled so that the MFMA operand reads are free of bank conflicts.
// The epilogue stages the tile's cos/sin rows in LDS, writes the finished
// rows to LDS and stores whole 256-byte (bf16) or 128-byte (e4m3) cache half
// rows per 16 lanes.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "device_common.h"
#include "project_args.h"

namespace dspark {
namespace {

// ------------------------------------------------------------ hidden norm --

// One wave per row: the sum of squares over the row (each lane adds its
// chunks c = lane, lane + 64, ... in that order with bf16 dot2, then DPP row
// sums and the four 16-lane partials added in a fixed order), then
// y = (x r)(1 + w) rounded to bf16.  Rows of up to 64 kPer chunks stay in
// registers between the two steps (one read of the row); longer rows are read
// again (from L2).  Both give the same sums in the same order.
constexpr int kNormPer = 16;    // chunks per lane held in registers: dim <= 8192

__global__ __launch_bounds__(256) void hidden_norm_resident_kernel(
    const uint16_t *x, const uint16_t *w, uint16_t *out, uint32_t rows, int32_t dim, float eps) {
    const int lane = threadIdx.x & 63;
    const uint32_t row = blockIdx.x * 4 +
                         static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    if (row >= rows) return;
    const int chunks = dim / 8;
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + static_cast<int64_t>(row) * dim);
    uint4 d[kNormPer];
#pragma unroll
    for (int j = 0; j < kNormPer; ++j)
        if (64 * j < chunks) d[j] = lane + 64 * j < chunks ? load_row16(xr + lane + 64 * j)
                                                           : make_uint4(0, 0, 0, 0);
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < kNormPer; ++j)
        if (64 * j < chunks && lane + 64 * j < chunks) {
            ss = dot2_bf16(d[j].x, d[j].x, ss);
            ss = dot2_bf16(d[j].y, d[j].y, ss);
            ss = dot2_bf16(d[j].z, d[j].z, ss);
            ss = dot2_bf16(d[j].w, d[j].w, ss);
        }
    ss = row_sum16(ss);
    ss = lane_value(ss, 0) + lane_value(ss, 16) + lane_value(ss, 32) + lane_value(ss, 48);
    const float r = __builtin_amdgcn_rsqf(ss / static_cast<float>(dim) + eps);
    const uint4 *wr = reinterpret_cast<const uint4 *>(w);
    uint4 *orow = reinterpret_cast<uint4 *>(out + static_cast<int64_t>(row) * dim);
#pragma unroll
    for (int j = 0; j < kNormPer; ++j) {
        const int c = lane + 64 * j;
        if (64 * j < chunks && c < chunks) {
            const uint4 wv = wr[c];
            const uint32_t dw[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
            const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float x0 = bf16_lo(dw[k]) * r, x1 = bf16_hi(dw[k]) * r;
                o[k] = pack_bf16(__builtin_fmaf(x0, bf16_lo(ww[k]), x0),
                                 __builtin_fmaf(x1, bf16_hi(ww[k]), x1));
            }
            store_row16(orow + c, make_uint4(o[0], o[1], o[2], o[3]));
        }
    }
}

__global__ __launch_bounds__(256) void hidden_norm_kernel(const uint16_t *x, const uint16_t *w,
                                                          uint16_t *out, uint32_t rows,
                                                          int32_t dim, float eps) {
    const int lane = threadIdx.x & 63;
    const uint32_t row = blockIdx.x * 4 +
                         static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    if (row >= rows) return;
    const int chunks = dim / 8;
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + static_cast<int64_t>(row) * dim);
    float ss = 0.0f;
    for (int c = lane; c < chunks; c += 64) {
        const uint4 d = xr[c];
        ss = dot2_bf16(d.x, d.x, ss);
        ss = dot2_bf16(d.y, d.y, ss);
        ss = dot2_bf16(d.z, d.z, ss);
        ss = dot2_bf16(d.w, d.w, ss);
    }
    ss = row_sum16(ss);
    ss = lane_value(ss, 0) + lane_value(ss, 16) + lane_value(ss, 32) + lane_value(ss, 48);
    const float r = __builtin_amdgcn_rsqf(ss / static_cast<float>(dim) + eps);
    const uint4 *wr = reinterpret_cast<const uint4 *>(w);
    uint4 *orow = reinterpret_cast<uint4 *>(out + static_cast<int64_t>(row) * dim);
    for (int c = lane; c < chunks; c += 64) {
        const uint4 d = xr[c];
        const uint4 wv = wr[c];
        const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
        const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float x0 = bf16_lo(dw[k]) * r, x1 = bf16_hi(dw[k]) * r;
            o[k] = pack_bf16(__builtin_fmaf(x0, bf16_lo(ww[k]), x0),
                             __builtin_fmaf(x1, bf16_hi(ww[k]), x1));
        }
        store_row16(orow + c, make_uint4(o[0], o[1], o[2], o[3]));
    }
}

// --------------------------------------------- projection + write epilogue --

constexpr int kPNumXcds = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float round_bf16(float v) { return bf16_lo(pack_bf16(v, 0.0f)); }


// The epilogue: this wave's 128 columns are one (layer, kv, head) row of
// all_kv for its TI * 32 tokens; it normalises and rotates K, converts, and
// stores whole cache half rows.  cs_lds holds kBM * R bf16 for the tile's
// cos/sin rows; tile_row(r) is the LDS address of row r (of WN * kBM) of the
// finished tile, 128 elements of the cache type each.  Every operand read of
// the main loop must be complete before the call.
template <int R, bool kFp8, int WM, int WN, int TI, int kBM, class TileRow>
__device__ __forceinline__ void project_epilogue(const ProjArgs &a, f32x16 (&acc)[TI][4],
                                                 int64_t m0, uint32_t nb, int wn, int wrow,
                                                 int tid, int lane, int64_t my_pos,
                                                 const int64_t (&my_slot)[TI / 2],
                                                 uint16_t *cs_lds, TileRow tile_row) {
    // this wave's 128 columns are all_kv's (layer, kv, head) = a row of the write
    const int head = static_cast<int>(nb) * WN + wn;
    const int hi = lane >> 5;
    const int cl = lane & 31;
    const int layer = head / (2 * a.nkv);
    const int kv = (head / a.nkv) & 1;
    const int h = head % a.nkv;
    // the tile's [cos | sin] rows, [kBM][R]; row r's 16-byte chunk c sits at
    // c ^ (r % (R / 8)) so that lanes reading one chunk of consecutive rows
    // spread over the banks
    constexpr int kCsMask = R / 8 - 1;
    static_assert(64 * WM * WN >= kBM, "one staging thread per token row");
    if (tid < kBM) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(a.cos_sin + my_pos * R);
        u32x4 *dst = reinterpret_cast<u32x4 *>(cs_lds + tid * R);
#pragma unroll
        for (int q = 0; q < R / 8; ++q) dst[q ^ (tid & kCsMask)] = src[q];
    }
    __syncthreads();

    // The MFMAs ran with the weight as the first operand, so acc[i][n][e]
    // holds column 32 n + 8 (e / 4) + 4 hi + e % 4 of token wrow + 32 i + cl:
    // a lane owns one token per i and half of its head (lane l ^ 32 the other
    // half), in runs of 4 consecutive columns.  The norm's sum is 64 local
    // adds and one exchange with lane l ^ 32; every RoPE partner column is in
    // the same lane.
    float wv2[4][4][4];   // the K norm weight at this lane's columns [n][q][rr]
    if (kv == 0) {
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint2 wp = *reinterpret_cast<const uint2 *>(
                    a.k_norm_weight + layer * 128 + 32 * n + 8 * q + 4 * hi);
                wv2[n][q][0] = bf16_lo(wp.x);
                wv2[n][q][1] = bf16_hi(wp.x);
                wv2[n][q][2] = bf16_lo(wp.y);
                wv2[n][q][3] = bf16_hi(wp.y);
            }
    }
    float fs = 1.0f, fy = 1.0f, flim = 460.0f;
    if constexpr (kFp8) {
        fs = a.scale0[kv == 0 ? a.kscale_off[layer] : a.vscale_off[layer]];
        fy = 1.0f / fs;
        flim = 460.0f * fs;
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        const int rho = wrow + 32 * i + cl;           // this lane's token row in the tile
        float y[4][16];
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int e = 0; e < 16; ++e) y[n][e] = round_bf16(acc[i][n][e]);
        if (a.all_kv_out != nullptr && m0 + rho < a.num_ctx) {
            // the projection's bf16 output itself: runs of 4 columns
            uint16_t *orow = a.all_kv_out + (m0 + rho) * a.cols + head * DSPARK_HEAD_DIM + 4 * hi;
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<uint2 *>(orow + 32 * n + 8 * q) =
                        make_uint2(pack_bf16(y[n][4 * q], y[n][4 * q + 1]),
                                   pack_bf16(y[n][4 * q + 2], y[n][4 * q + 3]));
        }
        if (kv == 0) {
            float ss = 0.0f;
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int e = 0; e < 16; ++e) ss = __builtin_fmaf(y[n][e], y[n][e], ss);
            ss += __shfl_xor(ss, 32);
            const float r = __builtin_amdgcn_rsqf(ss * (1.0f / DSPARK_HEAD_DIM) + a.eps);
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float xr = y[n][e] * r;
                    y[n][e] = round_bf16(__builtin_fmaf(xr, wv2[n][e >> 2][e & 3], xr));
                }
            // partial NeoX RoPE: column c < R / 2 pairs with c + R / 2
            const uint16_t *cs = cs_lds + rho * R;
            constexpr int kQ = (R / 2) / 8;            // 8-column groups in the first half
#pragma unroll
            for (int q = 0; q < kQ; ++q) {
                const int cq = (q ^ (rho & kCsMask)) * 8 + 4 * hi;
                const int sq = ((kQ + q) ^ (rho & kCsMask)) * 8 + 4 * hi;
                const uint2 cw = *reinterpret_cast<const uint2 *>(cs + cq);
                const uint2 sw2 = *reinterpret_cast<const uint2 *>(cs + sq);
                const float c4[4] = {bf16_lo(cw.x), bf16_hi(cw.x), bf16_lo(cw.y), bf16_hi(cw.y)};
                const float s4[4] = {bf16_lo(sw2.x), bf16_hi(sw2.x), bf16_lo(sw2.y), bf16_hi(sw2.y)};
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    // first-half column 8 q + 4 hi + rr and its partner
                    float &ya = (R == 64) ? y[0][4 * q + rr] : y[0][4 * q + rr];
                    float &yb = (R == 64) ? y[1][4 * q + rr] : y[0][4 * (q + kQ) + rr];
                    const float a0 = ya, b0 = yb;
                    ya = round_bf16(__builtin_fmaf(a0, c4[rr], -(b0 * s4[rr])));
                    yb = round_bf16(__builtin_fmaf(b0, c4[rr], a0 * s4[rr]));
                }
            }
        }
        // the finished values of this token into the head's row-major
        // [kBM][128] tile over the operand stages (every wave is past its
        // last operand read): runs of 4 columns, 8 (bf16) or 4 (e4m3) bytes.
        // Row rho's 8-column units are permuted by unit ^ (rho % 16), so the
        // 32 lanes writing one unit of 32 consecutive rows hit 16 bank groups.
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = ((4 * n + q) ^ (rho & 15)) * 8 + 4 * hi;
                const float *v = &y[n][4 * q];
                if constexpr (!kFp8) {
                    uint2 *dst = reinterpret_cast<uint2 *>(
                        reinterpret_cast<uint16_t *>(tile_row(wn * kBM + rho)) + col);
                    *dst = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
                } else {
                    int code = 0;
                    code = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_scale(v[0], fs, fy, flim),
                                                          div_by_scale(v[1], fs, fy, flim), code, false);
                    code = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_scale(v[2], fs, fy, flim),
                                                          div_by_scale(v[3], fs, fy, flim), code, true);
                    *reinterpret_cast<int *>(tile_row(wn * kBM + rho) + col) = code;
                }
            }
    }
    __syncthreads();

    // stores: 16 lanes per token row, 4 rows per wave instruction, each wave
    // its own rows of its own head
    const int q4 = lane >> 4;
    const int c16 = lane & 15;
    const int64_t bmask = (int64_t{1} << a.bs_log2) - 1;
#pragma unroll
    for (int u = 0; u < TI / 2; ++u)
#pragma unroll 4
    for (int it = 16 * u; it < 16 * u + 16; ++it) {
        const int rho = wrow + 4 * it + q4;
        // < 0: padding or past num_ctx
        const int64_t slot = __shfl(my_slot[u], 4 * (it - 16 * u) + q4);
        if (slot < 0) continue;
        const int64_t base = a.cache_off[layer] +
                             ((((slot >> a.bs_log2) * a.nkv + h) << a.bs_log2) + (slot & bmask)) *
                                 (2 * DSPARK_HEAD_DIM) +
                             kv * DSPARK_HEAD_DIM + c16 * 8;
        const int unit = c16 ^ (rho & 15);                   // the row's permuted 8-column unit
        if constexpr (!kFp8) {
            const u32x4 v = reinterpret_cast<const u32x4 *>(tile_row(wn * kBM + rho))[unit];
            store_row16(static_cast<uint16_t *>(a.cache0) + base, make_uint4(v.x, v.y, v.z, v.w));
        } else {
            store_row8(static_cast<uint8_t *>(a.cache0) + base,
                       reinterpret_cast<const uint2 *>(tile_row(wn * kBM + rho))[unit]);
        }
    }
}

// ------------------------------------------------ the projection kernel --
//
// Four waves, each 128 tokens x 128 columns (4 x 4 MFMA tiles, accumulators in
// the AGPRs): per 16-wide k step a wave reads 8 KB of operands from LDS for
// 16 MFMAs (two waves per SIMD at 64 x 128 each would read 12 KB for the same
// work, and the CU's LDS would then run at its limit).  The operands go from
// memory straight into LDS (buffer loads with the lds bit: no registers, no
// LDS store instructions), into a ring of five stages of 32 k each, issued
// four stages ahead.  Each stage is a separate LDS array and the barriers
// carry no memory fence, so the compiler's wait counts track each stage's
// loads on their own and never drain the ring; every stage's own loads are
// awaited by hand (vmcnt) before the barrier that publishes it.
constexpr int kDK = 32;                  // k per stage
constexpr int kDRows = 256;              // tile rows of each operand
constexpr int kDStage = 2 * kDRows * kDK / 8;   // 16-byte chunks: A then B
constexpr int kDLoads = 8;               // DMA instructions per thread per stage
constexpr int kNSt = 5;                  // stages in the ring
// tiles in groups of kGroupTokens / kBM token blocks (columns vary between
// groups): the 32 tiles an XCD runs at once span 1024 tokens and 2048 weight
// columns (4 x 8 tiles of 256 x 256, or 8 x 4 of 128 x 512), so its L2 serves
// 12 operand slices of 256 rows per k stage (18 in token-block-first order)
constexpr uint32_t kGroupTokens = 1024;
// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at their maxima).  A stage's loads go out in two halves of kDLoads / 2
// (token rows, then weight rows a half stage later); a stage waits for its
// successor with the loads of kNSt - 2 later stages in flight, the prologue
// for stage 0 with kNSt - 2 later stages and one half in flight.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitStage = vmcnt_imm((kNSt - 2) * kDLoads);
constexpr int kWaitPrologue = vmcnt_imm((kNSt - 2) * kDLoads + kDLoads / 2);

typedef __attribute__((address_space(3))) void lds_void;

// Tiles of kBM tokens (block mb) x kBN columns (block nb), in a grouped
// order: kGroupTokens / kBM token blocks per group, columns varying between
// groups.
struct Tile {
    uint32_t mb, nb;
};

template <int kBM, int kBN>
__device__ __forceinline__ Tile tile_at(uint32_t p, uint32_t num_ctx, uint32_t cols) {
    constexpr uint32_t kGm = kGroupTokens / kBM;
    const uint32_t mblocks = (num_ctx + kBM - 1) / kBM;
    const uint32_t gsz = kGm * (cols / kBN);
    const uint32_t gm0 = (p / gsz) * kGm;
    const uint32_t gm = mblocks - gm0 < kGm ? mblocks - gm0 : kGm;
    const uint32_t rem = p % gsz;
    return Tile{gm0 + rem % gm, rem / gm};
}

// Workgroup i of a run of n runs on XCD i % 8; its position in the order is
// chosen so that each XCD takes a contiguous part of the run (the last n % 8
// keep theirs).
__device__ __forceinline__ uint32_t xcd_run(uint32_t i, uint32_t n) {
    const uint32_t full = n - n % kPNumXcds;
    return i < full ? (i % kPNumXcds) * (full / kPNumXcds) + i / kPNumXcds : i;
}

template <int kBM, int kBN>
__device__ __forceinline__ Tile tile_of(uint32_t num_ctx, uint32_t cols) {
    return tile_at<kBM, kBN>(xcd_run(blockIdx.x, gridDim.x), num_ctx, cols);
}

// 16 bytes per lane from a buffer resource (voff per lane, soff per wave)
// into LDS at lds + 16 lane (lds wave-uniform)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t res, u32x4 *lds, int voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_void *)lds, 16, voff, soff, 0, 0);
#endif
}

// LDS layout of a stage: operand row r (of 256; A rows, then B rows) is 4
// chunks of 16 bytes (32 k), logical chunk j stored at position
// j ^ ((r / 4) % 4): the 16 consecutive rows that one operand read touches
// at one logical chunk land in 16 distinct bank groups.

template <int R, bool kFp8>
__global__ __launch_bounds__(256, 1) void project_write_kernel(const ProjArgs a) {
    constexpr int WM = 2, WN = 2, TI = 4, kBM = kDRows;
    // the ring; after the main loop stages 0-3 hold the finished tile and
    // stage 4 the tile's cos/sin rows
    __shared__ u32x4 st0[kDStage], st1[kDStage], st2[kDStage], st3[kDStage], st4[kDStage];
    static_assert(kBM * 64 * 2 <= kDStage * 16, "cos/sin rows fit one stage");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv % WM;
    const int wn = wv / WM;
    const Tile tile = tile_of<kBM, 128 * WN>(a.num_ctx, a.cols);
    const uint32_t nb = tile.nb;
    const int64_t m0 = static_cast<int64_t>(tile.mb) * kBM;
    const int64_t n0 = static_cast<int64_t>(nb) * (128 * WN);

    // DMA roles: instruction p of wave wv fills rows 64 p + 16 wv .. + 15 of
    // an operand (1 KB of LDS, 16 bytes per lane in lane order); lane l holds
    // physical chunk l % 4 of row 16 wv + l / 4, i.e. logical chunk
    // (l % 4) ^ ((l / 16) % 4).  Rows past num_ctx read as zero.
    const __amdgpu_buffer_rsrc_t zres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.z), 0, static_cast<int>(a.num_ctx * 2u * a.hidden), 0x00020000);
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.W), 0, static_cast<int>(a.cols * 2u * a.hidden), 0x00020000);
    const int row_bytes = 2 * a.hidden;
    const int drow = 16 * wv + (lane >> 2);
    const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
    const int zoff = (static_cast<int>(m0) + drow) * row_bytes + dchunk * 16;
    const int woff = (static_cast<int>(n0) + drow) * row_bytes + dchunk * 16;
    const int pstep = 64 * row_bytes;
    const int nk = a.hidden / kDK;
    auto issue_a = [&](u32x4 *st, int kt) {
        const int ko = kt * (kDK * 2);
#pragma unroll
        for (int p = 0; p < 4; ++p)
            dma16(zres, st + (64 * p + 16 * wv) * 4, zoff, p * pstep + ko);
    };
    auto issue_b = [&](u32x4 *st, int kt) {
        const int ko = kt * (kDK * 2);
#pragma unroll
        for (int p = 0; p < 4; ++p)
            dma16(wres, st + kDRows * 4 + (64 * p + 16 * wv) * 4, woff, p * pstep + ko);
    };

    // operand reads: rows wrow + 32 i + cl of A and 128 wn + 32 n + cl of B,
    // logical chunk 2 s + hi of the k step s (0, 1) of a stage
    const int hi = lane >> 5;
    const int cl = lane & 31;
    const int wrow = 32 * TI * wm;
    const int arow = (wrow + cl) * 4;
    const int brow = kDRows * 4 + (128 * wn + cl) * 4;
    const int xs0 = hi ^ ((cl >> 2) & 3);
    const int xs1 = (2 + hi) ^ ((cl >> 2) & 3);

    // tile row tid's position, for the epilogue's cos/sin staging; a row that
    // stores nothing (a padding slot, or past num_ctx) stages table row 0, so
    // a padding token's position is never used as an index
    int64_t my_pos = 0;
    if (tid < kBM) {
        int64_t t = m0 + tid;
        const bool inside = t < a.num_ctx;
        if (!inside) t = a.num_ctx - 1;
        const int64_t pos = a.positions[t];
        const int64_t slot = a.slots[t];
        my_pos = inside && slot >= 0 ? pos : 0;
    }
    int64_t my_slot[TI / 2];
#pragma unroll
    for (int u = 0; u < TI / 2; ++u) {
        const int64_t t = m0 + wrow + 64 * u + lane;
        my_slot[u] = t < a.num_ctx ? a.slots[t] : -1;
    }

    f32x16 acc[TI][4];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n] = f32x16{};

    bf16x8 fa[2][TI], fb[2][4];
    auto read_frags = [&](int buf, const u32x4 *st, int xs) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
            fa[buf][i] = __builtin_bit_cast(bf16x8, st[arow + 128 * i + xs]);
#pragma unroll
        for (int n = 0; n < 4; ++n)
            fb[buf][n] = __builtin_bit_cast(bf16x8, st[brow + 128 * n + xs]);
    };
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int n = 0; n < 4; ++n)
                acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][n], fa[buf][i],
                                                                    acc[i][n], 0, 0, 0);
    };
    // Instruction schedule of a half stage (one 16-wide k step): 16 MFMAs
    // with the next step's 8 LDS operand reads and 4 of the loads in between,
    // per group of four MFMAs two reads and one load, so that their latency
    // and issue sit behind the MFMAs.  sched_group_barrier masks: 0x008 MFMA,
    // 0x020 VMEM read, 0x100 LDS read.
    auto interleave_half = [&]() {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    };
    // Stage kt (array cur; prev holds stage kt - 1, nxt stage kt + 1):
    // the MFMAs of k step 0 run while step 1's operands are read and the
    // weight half of stage kt + 4 goes into prev (retired at the last
    // barrier); then this wave's loads of stage kt + 1 are awaited (three
    // later stages may still be in flight), its LDS reads drained, and the
    // barrier publishes stage kt + 1 and retires stage kt, whose refill with
    // stage kt + 5 starts with its token half while the MFMAs of step 1 run
    // and step 0 of stage kt + 1 is read.  Refills past the last stage load
    // the last stage again (clamped), so that every stage issues the same
    // number of loads and the hand-written wait counts stay exact.
    auto clamp = [&](int k) { return k < nk ? k : nk - 1; };
    auto stage = [&](u32x4 *prev, u32x4 *cur, u32x4 *nxt, int kt) {
        read_frags(1, cur, xs1);
        issue_b(prev, clamp(kt + kNSt - 1));
        mfmas(0);
        interleave_half();
        __builtin_amdgcn_s_waitcnt(kWaitStage);
        __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        issue_a(cur, clamp(kt + kNSt));
        read_frags(0, nxt, xs0);
        mfmas(1);
        interleave_half();
    };

    // prologue: the first kNSt - 1 stages and the token half of the last
    // (its weight half goes out in stage 0), then stage 0 awaited
    u32x4 *const stp[5] = {st0, st1, st2, st3, st4};
#pragma unroll
    for (int j = 0; j < kNSt - 1; ++j) {
        issue_a(stp[j], clamp(j));
        issue_b(stp[j], clamp(j));
    }
    issue_a(stp[kNSt - 1], clamp(kNSt - 1));
    __builtin_amdgcn_s_waitcnt(kWaitPrologue);
    __builtin_amdgcn_s_barrier();
    read_frags(0, st0, xs0);
    int kt = 0;
    for (; kt + kNSt <= nk; kt += kNSt) {
#pragma unroll
        for (int j = 0; j < kNSt; ++j)
            stage(stp[(j + kNSt - 1) % kNSt], stp[j], stp[(j + 1) % kNSt], kt + j);
    }
    // the last nk % kNSt stages start the ring again at stage array 0
#pragma unroll
    for (int j = 0; j < kNSt - 1; ++j)
        if (kt + j < nk) stage(stp[(j + kNSt - 1) % kNSt], stp[j], stp[j + 1], kt + j);
    // every load (the tail's reloads too) has landed before the stages are
    // reused for the finished tile
    __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0)
    __syncthreads();

    project_epilogue<R, kFp8, WM, WN, TI, kBM>(
        a, acc, m0, nb, wn, wrow, tid, lane, my_pos, my_slot, reinterpret_cast<uint16_t *>(st4),
        [&](int row) {
            constexpr int kRowBytes = kFp8 ? 128 : 256;
            constexpr int kRowsPerStage = kDStage * 16 / kRowBytes;
            const int q = row / kRowsPerStage;
            u32x4 *base = q == 0 ? st0 : q == 1 ? st1 : q == 2 ? st2 : st3;
            return reinterpret_cast<uint8_t *>(base) + (row % kRowsPerStage) * kRowBytes;
        });
}

// ------------------------------ the projection with a pre-packed weight --
//
// The same waves, MFMAs and epilogue as above, with the weight in the
// fragment-major layout that pack_kv_weight_kernel writes: every 32 x 16
// weight fragment of the MFMA is 1 KB contiguous, lane l's 16 bytes at
// 16 l.  A wave then loads its weight fragments straight into registers,
// 1 KB per instruction in whole cache lines, and the weight never passes
// through LDS; the L2 serves it in 128-byte lines instead of 64-byte halves.
// The token rows still go through LDS by DMA, in a ring of four stages; the
// weight goes through a ring of four register stages (32 registers each).
// Two arrangements of the four waves (WM x WN, each wave 128 tokens, or 64
// in the halves of the last round, x 128 columns):
//   1 x 4: 128 tokens x 512 columns (four heads) per workgroup; the token
//          rows (8 KB per stage) are shared by the four waves, and each wave
//          loads its own head's weight, so no fragment is fetched twice: per
//          stage the CU moves 40 KB from L2 and 40 KB through LDS;
//   2 x 2: 256 tokens x 256 columns, for column counts that are not a
//          multiple of 512; the two waves that share a column block both
//          load it (48 KB from L2 and 48 KB through LDS per stage).
constexpr int kLdsChunks = 160 * 1024 / 16;   // the CU's LDS in 16-byte chunks
constexpr int kPkRing = 4;                   // stages in flight, in LDS and in registers
// Per stage a wave issues kPkBLoads weight loads, then (after the barrier)
// kALoads token loads; with a ring of n stages the token loads of stage
// j + 1 are followed in issue order by the weight loads of stages j + 1 ..
// j + n - 1 and the token loads of j + 2 .. j + n - 1 (the steady-state
// wait).  The prologue waits for stage 0 with one more token stage in
// flight; the last stages wait as if every weight load after the awaited
// token loads were gone (they are dead there, and the compiler may drop
// them).
constexpr int kPkBLoads = 8;

// One tile: kBM = 32 TI WM tokens from m0 by 128 WN columns of column block
// nb.  sa0 .. sa3 are the workgroup's token stages (kStageAlloc chunks each,
// of which a stage uses kBM * kDK / 8) and rest the remainder of its 160 KB
// of LDS: a fifth stage (for a ring of five) and the epilogue's spare area.
template <int R, bool kFp8, int WM, int TI, int kStageAlloc>
__device__ __forceinline__ void packed_tile(const ProjArgs &a, int64_t m0, uint32_t nb,
                                            u32x4 *sa0, u32x4 *sa1, u32x4 *sa2, u32x4 *sa3,
                                            u32x4 *rest) {
    constexpr int WN = 4 / WM, kBM = 32 * TI * WM;
    static_assert(TI == 2 || TI == 4, "32 TI tokens per wave");
    constexpr int kStage = kBM * kDK / 8;        // 16-byte chunks of a token stage
    static_assert(kStage <= kStageAlloc, "a stage fits its array");
    constexpr int kALoads = kBM / 64;            // token DMA instructions per wave and stage
    constexpr int kWaitStage = vmcnt_imm((kPkRing - 1) * kPkBLoads + (kPkRing - 2) * kALoads);
    constexpr int kWaitPrologue = vmcnt_imm((kPkRing - 1) * (kPkBLoads + kALoads));
    constexpr int kWaitTail = vmcnt_imm((kPkRing - 2) * kALoads);
    static_assert((kPkRing - 1) * (kPkBLoads + kALoads) <= 63, "vmcnt holds at most 63");
    constexpr int kSpare = kLdsChunks - kPkRing * kStageAlloc;
    static_assert(kPkRing == 4 || kPkRing == 5, "the ring's arrays");
    u32x4 *const sa4 = rest;
    u32x4 *const spare = rest + (kPkRing - 4) * kStageAlloc;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv % WM;
    const int wn = wv / WM;
    const int64_t n0 = static_cast<int64_t>(nb) * (128 * WN);

    const __amdgpu_buffer_rsrc_t zres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.z), 0, static_cast<int>(a.num_ctx * 2u * a.hidden), 0x00020000);
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.W), 0, static_cast<int>(a.cols * 2u * a.hidden), 0x00020000);
    const int row_bytes = 2 * a.hidden;
    const int nk = a.hidden / kDK;
    auto clamp = [&](int k) { return k < nk ? k : nk - 1; };

    // token rows into LDS as in the kernel above (rows past num_ctx read as zero)
    const int drow = 16 * wv + (lane >> 2);
    const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
    const int zoff = (static_cast<int>(m0) + drow) * row_bytes + dchunk * 16;
    const int pstep = 64 * row_bytes;
    auto issue_a = [&](u32x4 *st, int kt) {
        const int ko = kt * (kDK * 2);
#pragma unroll
        for (int p = 0; p < kALoads; ++p)
            dma16(zres, st + (64 * p + 16 * wv) * 4, zoff, p * pstep + ko);
    };

    // weight fragments into registers: fragment (column block cb, k block
    // kb) sits at byte (cb * hidden / 16 + kb) * 1024; this wave's column
    // blocks are (n0 + 128 wn) / 32 + n, and stage kt holds k blocks 2 kt + s
    const int boff = (static_cast<int>(n0) + 128 * wn) * row_bytes + 16 * lane;
    const int nstep = 32 * row_bytes;            // one column block of fragments
    bf16x8 fb[kPkRing][2][4];
    auto issue_b = [&](int slot, int kt) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int n = 0; n < 4; ++n)
                fb[slot][s][n] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(wres, boff + 1024 * s,
                                                                  kt * 2048 + n * nstep, 0));
    };

    const int hi = lane >> 5;
    const int cl = lane & 31;
    const int wrow = 32 * TI * wm;
    const int arow = (wrow + cl) * 4;
    const int xs0 = hi ^ ((cl >> 2) & 3);
    const int xs1 = (2 + hi) ^ ((cl >> 2) & 3);

    // tile row tid's position, for the epilogue's cos/sin staging; a row that
    // stores nothing (a padding slot, or past num_ctx) stages table row 0, so
    // a padding token's position is never used as an index
    int64_t my_pos = 0;
    if (tid < kBM) {
        int64_t t = m0 + tid;
        const bool inside = t < a.num_ctx;
        if (!inside) t = a.num_ctx - 1;
        const int64_t pos = a.positions[t];
        const int64_t slot = a.slots[t];
        my_pos = inside && slot >= 0 ? pos : 0;
    }
    int64_t my_slot[TI / 2];
#pragma unroll
    for (int u = 0; u < TI / 2; ++u) {
        const int64_t t = m0 + wrow + 64 * u + lane;
        my_slot[u] = t < a.num_ctx ? a.slots[t] : -1;
    }

    f32x16 acc[TI][4];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n] = f32x16{};

    bf16x8 fa[2][TI];
    auto read_frags = [&](int buf, const u32x4 *st, int xs) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
            fa[buf][i] = __builtin_bit_cast(bf16x8, st[arow + 128 * i + xs]);
    };
    auto mfmas = [&](int slot, int s) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int n = 0; n < 4; ++n)
                acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][s][n], fa[s][i],
                                                                    acc[i][n], 0, 0, 0);
    };
    // per group of TI MFMAs (a quarter of a k step): one LDS read (in TI of
    // the four groups) and two (k step 0: the weight loads) or, in kALoads
    // of the four groups, one (k step 1: the token loads) memory loads
    auto interleave = [&](bool step0) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (g < TI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (step0)
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
            else if (g % (4 / kALoads) == 0)
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            if (TI > 2) __builtin_amdgcn_sched_group_barrier(0x008, TI - 2, 0);
        }
    };
    // Stage kt (token stage cur, weight slot `slot`): k step 0's MFMAs run
    // while step 1's token operands are read and the weight of stage kt + 3
    // is requested; then the token rows of stage kt + 1 are awaited, this
    // wave's LDS reads drained, and the barrier publishes stage kt + 1 and
    // retires cur, whose refill with stage kt + 4 goes out during step 1.
    auto stage = [&](u32x4 *cur, u32x4 *nxt, int slot, int kt, bool last) {
        read_frags(1, cur, xs1);
        issue_b((slot + kPkRing - 1) % kPkRing, clamp(kt + kPkRing - 1));
        mfmas(slot, 0);
        interleave(true);
        if (last)
            __builtin_amdgcn_s_waitcnt(kWaitTail);
        else
            __builtin_amdgcn_s_waitcnt(kWaitStage);
        __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        issue_a(cur, clamp(kt + kPkRing));
        read_frags(0, nxt, xs0);
        mfmas(slot, 1);
        interleave(false);
    };

    u32x4 *const stp[5] = {sa0, sa1, sa2, sa3, sa4};
    // prologue, in issue order: tokens 0, weight 0, tokens 1, weight 1, ...,
    // weight n - 2, tokens n - 1
#pragma unroll
    for (int j = 0; j < kPkRing - 1; ++j) {
        issue_a(stp[j], clamp(j));
        issue_b(j, clamp(j));
    }
    issue_a(stp[kPkRing - 1], clamp(kPkRing - 1));
    __builtin_amdgcn_s_waitcnt(kWaitPrologue);
    __builtin_amdgcn_s_barrier();
    read_frags(0, sa0, xs0);
    // whole rounds of the rings while more than one round is left, then the
    // last ones (at most a round)
    int kt = 0;
    for (; kt + kPkRing < nk; kt += kPkRing) {
#pragma unroll
        for (int j = 0; j < kPkRing; ++j)
            stage(stp[j], stp[(j + 1) % kPkRing], j, kt + j, false);
    }
#pragma unroll
    for (int j = 0; j < kPkRing; ++j)
        if (kt + j < nk) stage(stp[j], stp[(j + 1) % kPkRing], j, kt + j, true);
    // every load (the clamped reloads too) has landed before the LDS is
    // reused for the finished tile
    __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0)
    __syncthreads();

    // the epilogue's LDS: the tile's cos/sin rows at the start of the spare
    // area, the finished tile's rows over the rest of it, then the token
    // stages
    uint8_t *const sp = reinterpret_cast<uint8_t *>(spare);
    project_epilogue<R, kFp8, WM, WN, TI, kBM>(
        a, acc, m0, nb, wn, wrow, tid, lane, my_pos, my_slot, reinterpret_cast<uint16_t *>(spare),
        [&](int row) {
            constexpr int kRowBytes = kFp8 ? 128 : 256;
            constexpr int kCsBytes = kBM * 64 * 2;
            constexpr int kSpareRows = (kSpare * 16 - kCsBytes) / kRowBytes;
            constexpr int kStageRows = kStageAlloc * 16 / kRowBytes;
            static_assert(kCsBytes <= kSpare * 16, "the cos/sin rows fit the spare area");
            static_assert(kSpareRows + kPkRing * kStageRows >= WN * kBM, "the finished tile fits");
            if (row < kSpareRows) return sp + kCsBytes + row * kRowBytes;
            const int r = row - kSpareRows;
            const int q = r / kStageRows;
            u32x4 *base = q == 0 ? sa0 : q == 1 ? sa1 : q == 2 ? sa2 : q == 3 ? sa3 : sa4;
            return reinterpret_cast<uint8_t *>(base) + (r % kStageRows) * kRowBytes;
        });
}

// 2 x 2 waves on 256 x 256 tiles, for column counts that are not a multiple
// of 512.
template <int R, bool kFp8>
__global__ __launch_bounds__(256, 1) void project_write_packed_kernel(const ProjArgs a) {
    constexpr int kStage = 256 * kDK / 8;
    __shared__ u32x4 sa0[kStage], sa1[kStage], sa2[kStage], sa3[kStage],
        rest[kLdsChunks - 4 * kStage];
    const Tile tile = tile_of<256, 256>(a.num_ctx, a.cols);
    packed_tile<R, kFp8, 2, 4, kStage>(a, static_cast<int64_t>(tile.mb) * 256, tile.nb, sa0, sa1,
                                       sa2, sa3, rest);
}

// 1 x 4 waves on 128 x 512 tiles.  The tile count rarely divides into whole
// rounds of the CUs, and a last round that fills few of them takes as long
// as a full one; so when the last round would fill at most half of the CUs,
// its tiles are run as twice as many 64-token halves (the workgroups from
// big_tiles on), one round of about half the time.
template <int R, bool kFp8>
__global__ __launch_bounds__(256, 1) void project_write_packed_wide_kernel(const ProjArgs a) {
    constexpr int kStage = 128 * kDK / 8;
    __shared__ u32x4 sa0[kStage], sa1[kStage], sa2[kStage], sa3[kStage],
        rest[kLdsChunks - 4 * kStage];
    const uint32_t big = a.big_tiles;
    if (blockIdx.x < big) {
        const Tile t = tile_at<128, 512>(xcd_run(blockIdx.x, big), a.num_ctx, a.cols);
        packed_tile<R, kFp8, 1, 4, kStage>(a, static_cast<int64_t>(t.mb) * 128, t.nb, sa0, sa1,
                                           sa2, sa3, rest);
    } else {
        // halves 2 j and 2 j + 1 of tile big + j (in the grouped order)
        const uint32_t h = xcd_run(blockIdx.x - big, gridDim.x - big);
        const Tile t = tile_at<128, 512>(big + h / 2, a.num_ctx, a.cols);
        const int64_t m0 = static_cast<int64_t>(t.mb) * 128 + 64 * (h % 2);
        if (m0 >= a.num_ctx) return;             // a half wholly past the last token
        packed_tile<R, kFp8, 1, 2, kStage>(a, m0, t.nb, sa0, sa1, sa2, sa3, rest);
    }
}

// The weight's fragment-major layout: element (c, k) of the [cols, hidden]
// weight goes to fragment (c / 32) * hidden / 16 + k / 16 (1 KB each), lane
// c % 32 + 32 ((k % 16) / 8), element k % 8 of that lane's 16 bytes.  One
// thread per 16-byte output chunk (writes contiguous, reads 16 bytes per
// weight row).
__global__ __launch_bounds__(256) void pack_kv_weight_kernel(const u32x4 *w, u32x4 *out,
                                                             uint32_t chunks, int32_t hidden) {
    const uint32_t q = blockIdx.x * 256u + threadIdx.x;
    if (q >= chunks) return;
    const uint32_t frag = q / 64, lane = q % 64;
    const uint32_t kblocks = static_cast<uint32_t>(hidden) / 16;
    const uint32_t c = (frag / kblocks) * 32 + lane % 32;
    const uint32_t k = (frag % kblocks) * 16 + (lane / 32) * 8;
    out[q] = w[(static_cast<uint64_t>(c) * hidden + k) / 8];
}

// The number of compute units of the current device (read once per device).
int cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// One workgroup per tile: 256 tokens x 256 columns, or with a packed weight
// and a column count that is a multiple of 512, 128 tokens x 512 columns
// (the last round's tiles, when they fill at most half of the CUs, in
// 64-token halves).
template <int R, bool kFp8>
void launch_pw(const ProjArgs &a, bool packed, hipStream_t stream) {
    const dim3 grid((a.num_ctx + kDRows - 1) / kDRows * (a.cols / 256));
    if (packed && a.cols % 512 == 0) {
        const uint32_t tiles = (a.num_ctx + 127) / 128 * (a.cols / 512);
        const uint32_t cus = static_cast<uint32_t>(cu_count());
        const uint32_t last = tiles % cus;
        ProjArgs b = a;
        b.big_tiles = last != 0 && 2 * last <= cus ? tiles - last : tiles;
        const uint32_t groups = b.big_tiles + 2 * (tiles - b.big_tiles);
        hipLaunchKernelGGL((project_write_packed_wide_kernel<R, kFp8>), dim3(groups), dim3(256), 0,
                           stream, b);
    } else if (packed) {
        hipLaunchKernelGGL((project_write_packed_kernel<R, kFp8>), grid, dim3(256), 0, stream, a);
    } else {
        hipLaunchKernelGGL((project_write_kernel<R, kFp8>), grid, dim3(256), 0, stream, a);
    }
}

}  // namespace

hipError_t launch_hidden_norm(const uint16_t *x, const uint16_t *w, uint16_t *out, uint32_t rows,
                              int32_t dim, float eps, hipStream_t stream) {
    if (dim <= 8 * 64 * kNormPer)
        hipLaunchKernelGGL(hidden_norm_resident_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream,
                           x, w, out, rows, dim, eps);
    else
        hipLaunchKernelGGL(hidden_norm_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, x, w,
                           out, rows, dim, eps);
    return hipGetLastError();
}

hipError_t launch_project_write(const ProjArgs &a, int rotary_dim, bool fp8, bool packed,
                                hipStream_t stream) {
    switch (rotary_dim) {
    case 16: fp8 ? launch_pw<16, true>(a, packed, stream) : launch_pw<16, false>(a, packed, stream); break;
    case 32: fp8 ? launch_pw<32, true>(a, packed, stream) : launch_pw<32, false>(a, packed, stream); break;
    case 64: fp8 ? launch_pw<64, true>(a, packed, stream) : launch_pw<64, false>(a, packed, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_pack_kv_weight(const uint16_t *w, uint16_t *out, uint32_t cols, int32_t hidden,
                                 hipStream_t stream) {
    const uint32_t chunks = cols * static_cast<uint32_t>(hidden) / 8;
    hipLaunchKernelGGL(pack_kv_weight_kernel, dim3((chunks + 255) / 256), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4 *>(w), reinterpret_cast<u32x4 *>(out), chunks,
                       hidden);
    return hipGetLastError();
}

}  // namespace dspark
