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
// D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32]).  A workgroup of 8 waves (two per
// SIMD) owns a 256-token x 256-column tile; each wave computes 64 tokens x 128
// columns, and 128 columns are exactly one (layer, kv, head) row of all_kv, so
// the write's per-row norm, RoPE and store happen on data the wave holds.  The
// weight is the MFMA's first operand, so a lane ends with one token's values
// in runs of 4 consecutive columns (half of the head; lane l ^ 32 holds the
// other half): the norm's sum of squares is local adds and one exchange, and
// every RoPE partner column is in the same lane.  Operands are read through
// buffer resources (rows past num_ctx read as zero) into registers two k
// slices ahead, then into double-buffered LDS whose 16-byte chunks are
// XOR-swizzled so that the stores and the MFMA operand reads are free of
// bank conflicts.  The epilogue stages the tile's cos/sin rows in LDS, writes
// the finished rows to LDS and stores whole 256-byte (bf16) or 128-byte
// (e4m3) cache half rows per 16 lanes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "project_args.h"

namespace dspark {
namespace {

// ------------------------------------------------------------ hidden norm --

// One wave per row: the sum of squares over the row (bf16 dot2, DPP row sums,
// then the four 16-lane partials added in a fixed order), then the row again
// (from L2) for y = (x r)(1 + w) rounded to bf16.
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

// Tile geometry: WM x WN waves; a wave computes 4 x TI MFMA tiles of 32 x 32,
// i.e. 128 columns = exactly one (layer, kv, head) row of all_kv for 32 TI
// tokens.  A workgroup tile is (32 TI WM) tokens x (128 WN) columns, k slices
// of 64; DEPTH k slices are in flight in registers.
constexpr int kPK = 64;
constexpr int kPNumXcds = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// position of 16-byte chunk j (of 8) of LDS row r: XOR with (r / 2) % 8 makes
// 16 consecutive rows at one logical chunk hit 16 distinct bank groups
__device__ __forceinline__ int swz(int r, int j) { return (r << 3) + (j ^ ((r >> 1) & 7)); }

__device__ __forceinline__ float round_bf16(float v) { return bf16_lo(pack_bf16(v, 0.0f)); }


template <int WM, int WN, int TI>
struct Tile {
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int kBM = 32 * TI * WM;        // tokens
    static constexpr int kBN = 128 * WN;            // columns
    static constexpr int kA = kBM * kPK / 8;        // 16-byte chunks of an A slice
    static constexpr int kB = kBN * kPK / 8;
    static constexpr int kStage = kA + kB;
    static constexpr int kPA = kA / kThreads;       // A chunks per thread per slice
    static constexpr int kPB = kB / kThreads;
    static constexpr int kRowStep = kThreads / 8;   // rows covered by one pass of the threads
    // LDS: two stages, then the staged cos/sin rows (up to R = 64)
    static constexpr int kCsOff = 2 * kStage;       // in 16-byte chunks
    static constexpr int kLds = kCsOff + kBM * 64 * 2 / 16;
    static_assert(kBM * kBN * 2 <= 2 * kStage * 16, "the finished tile must fit the stages");
};

template <int R, bool kFp8, int WM, int WN, int TI, int DEPTH>
__global__ __launch_bounds__(64 * WM * WN, 1) void project_write_kernel(const ProjArgs a) {
    using T = Tile<WM, WN, TI>;
    __shared__ u32x4 lds[T::kLds];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv % WM;
    const int wn = wv / WM;
    const uint32_t mblocks = (a.num_ctx + T::kBM - 1) / T::kBM;

    // XCD-aware tile order: XCD x (workgroup i runs on XCD i % 8) takes a
    // contiguous run of tiles; tiles are M-fastest, so an XCD works through a
    // few heads' weight slices while all token tiles pass through its L2
    uint32_t bid = blockIdx.x;
    const uint32_t full = gridDim.x - gridDim.x % kPNumXcds;
    if (bid < full) bid = (bid % kPNumXcds) * (full / kPNumXcds) + bid / kPNumXcds;
    const uint32_t mb = bid % mblocks;
    const uint32_t nb = bid / mblocks;
    const int64_t m0 = static_cast<int64_t>(mb) * T::kBM;
    const int64_t n0 = static_cast<int64_t>(nb) * T::kBN;

    // global -> LDS copy roles: chunk j of rows r0 + kRowStep p.  Operands
    // are read through buffer resources: one per-lane byte offset, the row
    // step and the k slice in scalar offsets, and token rows past num_ctx
    // fall outside the resource's range and read as zero (computed, never
    // stored).  kRowStep is a multiple of 16, so every row a thread copies
    // has the same chunk swizzle and its LDS slots are constant offsets.
    static_assert(T::kRowStep % 16 == 0, "one swizzle per copying thread");
    const int j = tid & 7;
    const int r0 = tid >> 3;
    const __amdgpu_buffer_rsrc_t zres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.z), 0, static_cast<int>(a.num_ctx * 2u * a.hidden), 0x00020000);
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.W), 0, static_cast<int>(a.cols * 2u * a.hidden), 0x00020000);
    const int row_bytes = 2 * a.hidden;
    const int zoff = (static_cast<int>(m0) + r0) * row_bytes + j * 16;
    const int woff = (static_cast<int>(n0) + r0) * row_bytes + j * 16;
    const int step_bytes = T::kRowStep * row_bytes;
    const int aw0 = swz(r0, j);
    const int bw0 = T::kA + swz(r0, j);
    // MFMA operand reads: rows wrow + 32 i + cl of A and 128 wn + 32 n + cl
    // of B, chunk 2 s + hi of the 16-wide k step s; all these rows share the
    // swizzle (cl / 2) % 8
    const int hi = lane >> 5;
    const int cl = lane & 31;
    const int wrow = 32 * TI * wm;                    // this wave's first token row
    const int sw = (cl >> 1) & 7;
    const int arow = (wrow + cl) * 8;
    const int brow = T::kA + (128 * wn + cl) * 8;
    int xs[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) xs[s4] = (2 * s4 + hi) ^ sw;

    // the epilogue's per-token inputs, requested now so that their latency
    // hides behind the main loop: the position of token row tid (for the
    // cos/sin staging) and the slot of this wave's store row wrow + lane
    static_assert(32 * TI == 64, "one store row of the wave band per lane");
    int64_t my_pos = 0;
    if (tid < T::kBM) {
        int64_t t = m0 + tid;
        if (t >= a.num_ctx) t = a.num_ctx - 1;
        my_pos = a.positions[t];
    }
    const int64_t my_slot = (m0 + wrow + lane < a.num_ctx) ? a.slots[m0 + wrow + lane] : -1;

    f32x16 acc[TI][4];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n] = f32x16{};

    // Two register sets keep two k slices in flight: while the matrix cores
    // work on slice kt (LDS stage kt % 2), slice kt + 1 is arriving in one
    // set and slice kt + 2 is requested into the other; slice kt + 1 goes to
    // LDS after the MFMAs (its stage was last read before the previous
    // barrier).  The loop is unrolled by two so that both sets are named
    // statically and stay in registers.  A wave raises its issue priority
    // while it runs its MFMAs, so that the other wave of its SIMD issues its
    // loads and LDS traffic in the gaps rather than competing for the
    // matrix core.
    constexpr int kP = T::kPA + T::kPB;
    u32x4 ra[kP], rb[kP];
    const int nk = a.hidden / kPK;
#define DSPARK_FETCH(r, kt)                                                              \
    do {                                                                                 \
        const int o_ = (kt) * (kPK * 2);                                                 \
        _Pragma("unroll") for (int p = 0; p < T::kPA; ++p)                               \
            r[p] = __builtin_amdgcn_raw_buffer_load_b128(zres, zoff, p * step_bytes + o_, 0); \
        _Pragma("unroll") for (int p = 0; p < T::kPB; ++p)                               \
            r[T::kPA + p] =                                                              \
                __builtin_amdgcn_raw_buffer_load_b128(wres, woff, p * step_bytes + o_, 0); \
    } while (0)
#define DSPARK_PUT(r, stage)                                                             \
    do {                                                                                 \
        _Pragma("unroll") for (int p = 0; p < T::kPA; ++p)                               \
            lds[(stage) + aw0 + p * T::kRowStep * 8] = r[p];                             \
        _Pragma("unroll") for (int p = 0; p < T::kPB; ++p)                               \
            lds[(stage) + bw0 + p * T::kRowStep * 8] = r[T::kPA + p];                    \
    } while (0)
    // one k slice: `next` holds slice kt + 1 (arriving), `spare` receives kt + 2
#define DSPARK_STEP(kt, next, spare)                                                     \
    do {                                                                                 \
        const int cur_ = ((kt) & 1) * T::kStage;                                         \
        if ((kt) + 2 < nk) DSPARK_FETCH(spare, (kt) + 2);                                \
        __builtin_amdgcn_s_setprio(1);                                                   \
        _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                  \
            bf16x8 af[TI], bfr[4];                                                       \
            _Pragma("unroll") for (int i = 0; i < TI; ++i)                               \
                af[i] = __builtin_bit_cast(bf16x8, lds[cur_ + arow + 256 * i + xs[s]]);  \
            _Pragma("unroll") for (int n = 0; n < 4; ++n)                                \
                bfr[n] = __builtin_bit_cast(bf16x8, lds[cur_ + brow + 256 * n + xs[s]]); \
            _Pragma("unroll") for (int i = 0; i < TI; ++i)                               \
                _Pragma("unroll") for (int n = 0; n < 4; ++n)                            \
                    acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                 \
                        bfr[n], af[i], acc[i][n], 0, 0, 0);                              \
        }                                                                                \
        __builtin_amdgcn_s_setprio(0);                                                   \
        if ((kt) + 1 < nk) DSPARK_PUT(next, T::kStage - cur_);                           \
        __syncthreads();                                                                 \
    } while (0)
    DSPARK_FETCH(ra, 0);
    DSPARK_PUT(ra, 0);
    if constexpr (DEPTH == 2) {
        if (nk > 1) DSPARK_FETCH(ra, 1);
        __syncthreads();
        for (int kt = 0; kt < nk; kt += 2) {
            DSPARK_STEP(kt, ra, rb);
            if (kt + 1 < nk) DSPARK_STEP(kt + 1, rb, ra);
        }
    } else {
        // one slice in flight: slice kt + 1 is requested into the one set
        // at the top of step kt and stored after its MFMAs
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur_ = (kt & 1) * T::kStage;
            if (kt + 1 < nk) DSPARK_FETCH(ra, kt + 1);
            __builtin_amdgcn_s_setprio(1);
            _Pragma("unroll") for (int s = 0; s < 4; ++s) {
                bf16x8 af[TI], bfr[4];
                _Pragma("unroll") for (int i = 0; i < TI; ++i)
                    af[i] = __builtin_bit_cast(bf16x8, lds[cur_ + arow + 256 * i + xs[s]]);
                _Pragma("unroll") for (int n = 0; n < 4; ++n)
                    bfr[n] = __builtin_bit_cast(bf16x8, lds[cur_ + brow + 256 * n + xs[s]]);
                _Pragma("unroll") for (int i = 0; i < TI; ++i)
                    _Pragma("unroll") for (int n = 0; n < 4; ++n)
                        acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[n], af[i], acc[i][n],
                                                                            0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
            if (kt + 1 < nk) DSPARK_PUT(ra, T::kStage - cur_);
            __syncthreads();
        }
    }
#undef DSPARK_STEP
#undef DSPARK_PUT
#undef DSPARK_FETCH

    // ---------------------------------------------------------- epilogue --
    // this wave's 128 columns are all_kv's (layer, kv, head) = a row of the write
    const int head = static_cast<int>(nb) * WN + wn;
    const int layer = head / (2 * a.nkv);
    const int kv = (head / a.nkv) & 1;
    const int h = head % a.nkv;
    // the tile's [cos | sin] rows, [kBM][R]; row r's 16-byte chunk c sits at
    // c ^ (r % (R / 8)) so that lanes reading one chunk of consecutive rows
    // spread over the banks
    constexpr int kCsMask = R / 8 - 1;
    uint16_t *cs_lds = reinterpret_cast<uint16_t *>(lds + T::kCsOff);
    static_assert(T::kThreads >= T::kBM, "one staging thread per token row");
    if (tid < T::kBM) {
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
                        reinterpret_cast<uint16_t *>(lds) + (wn * T::kBM + rho) * 128 + col);
                    *dst = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
                } else {
                    int code = 0;
                    code = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_scale(v[0], fs, fy, flim),
                                                          div_by_scale(v[1], fs, fy, flim), code, false);
                    code = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_scale(v[2], fs, fy, flim),
                                                          div_by_scale(v[3], fs, fy, flim), code, true);
                    *reinterpret_cast<int *>(reinterpret_cast<uint8_t *>(lds) +
                                             (wn * T::kBM + rho) * 128 + col) = code;
                }
            }
    }
    __syncthreads();

    // stores: 16 lanes per token row, 4 rows per wave instruction, each wave
    // its own rows of its own head
    const int q4 = lane >> 4;
    const int c16 = lane & 15;
    const int64_t bmask = (int64_t{1} << a.bs_log2) - 1;
#pragma unroll 4
    for (int it = 0; it < 8 * TI; ++it) {
        const int rho = wrow + 4 * it + q4;
        const int64_t slot = __shfl(my_slot, 4 * it + q4);   // < 0: padding or past num_ctx
        if (slot < 0) continue;
        const int64_t base = a.cache_off[layer] +
                             ((((slot >> a.bs_log2) * a.nkv + h) << a.bs_log2) + (slot & bmask)) *
                                 (2 * DSPARK_HEAD_DIM) +
                             kv * DSPARK_HEAD_DIM + c16 * 8;
        const int unit = c16 ^ (rho & 15);                   // the row's permuted 8-column unit
        if constexpr (!kFp8) {
            const u32x4 v = lds[(wn * T::kBM + rho) * 16 + unit];
            store_row16(static_cast<uint16_t *>(a.cache0) + base, make_uint4(v.x, v.y, v.z, v.w));
        } else {
            store_row8(static_cast<uint8_t *>(a.cache0) + base,
                       reinterpret_cast<const uint2 *>(lds)[(wn * T::kBM + rho) * 16 + unit]);
        }
    }
}

// the tile geometry in use: 8 waves (two per SIMD), 256-token x 256-column
// tiles, two k slices in flight
constexpr int kWM = 4, kWN = 2, kTI = 2, kDepth = 2;

template <int R, bool kFp8>
void launch_pw(const ProjArgs &a, hipStream_t stream) {
    using T = Tile<kWM, kWN, kTI>;
    const uint32_t mblocks = (a.num_ctx + T::kBM - 1) / T::kBM;
    hipLaunchKernelGGL((project_write_kernel<R, kFp8, kWM, kWN, kTI, kDepth>),
                       dim3(mblocks * (a.cols / T::kBN)), dim3(T::kThreads), 0, stream, a);
}

}  // namespace

hipError_t launch_hidden_norm(const uint16_t *x, const uint16_t *w, uint16_t *out, uint32_t rows,
                              int32_t dim, float eps, hipStream_t stream) {
    hipLaunchKernelGGL(hidden_norm_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, x, w, out,
                       rows, dim, eps);
    return hipGetLastError();
}

hipError_t launch_project_write(const ProjArgs &a, int rotary_dim, bool fp8, hipStream_t stream) {
    switch (rotary_dim) {
    case 16: fp8 ? launch_pw<16, true>(a, stream) : launch_pw<16, false>(a, stream); break;
    case 32: fp8 ? launch_pw<32, true>(a, stream) : launch_pw<32, false>(a, stream); break;
    case 64: fp8 ? launch_pw<64, true>(a, stream) : launch_pw<64, false>(a, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dspark
