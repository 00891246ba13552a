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
// as OCP e4m3 of value / scale.  Nothing is written for a padding slot
// (< 0), and the position of a token stored in no layer is never used as a
// table index (its rows may still be read, ahead of its slot).
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
//     lane c ^ (R/16), fetched with one DPP move (R = 16, 32) or two DPP
//     row rotations and a select (R = 64);
//   * the token's cos/sin values are loaded once per row into registers and
//     reused for every layer;
//   * fp8: x / scale is formed from y = RN(1/scale) (one IEEE division per
//     wave gives every layer's reciprocals, one per lane) as q0 = x y,
//     r = fma(q0, scale, -x), q = fma(-r, y, q0), which is the correctly
//     rounded quotient for every finite bf16 x at the e4m3 resolution
//     (Markstein's correction step) on x clamped to +-460 scale, which also
//     keeps the result inside the e4m3 range; then the hardware pack
//     conversion v_cvt_pk_fp8_f32 (OCP e4m3 on gfx950);
//   * loads are nontemporal; the cache stores carry the sc1 policy through a
//     buffer resource on a wave-uniform base (uniform-token rows and
//     per-layer slots), which moves the scattered 512-byte rows faster than
//     nontemporal stores; the general row mapping keeps nontemporal stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ctx_kv_args.h"
#include "device_common.h"

namespace dspark {
namespace {

// Waves per workgroup: 4.  (Eight-wave workgroups were about 1% faster on
// the bf16 prefill while its stores were nontemporal; with the sc1 stores
// four waves are 0.8% faster, and they are faster on small and fp8 writes.)
constexpr int kWavesPerGroup = 4;
// Writes of at most this many 4-row waves give each layer its own wave, by
// row mapping (a wave's rows are heads of one token, or the general mapping)
// and cache type.  Measured at L = 5 (medians of 5-9 rounds, prefill token
// subsets, head shards and the long layout as bf16):
//   * one token per wave, bf16: the split saves 3.9% at 8192 waves (the
//     4096-token prefill), 7% at 4096, 3.6% at 16384, nothing at 32768 and
//     loses 1.8% at 65536;
//   * one token per wave, fp8: it saves 0.7 us of 3.2 on a 300-wave write
//     and beats groups of three layers at 1024 waves (5.22 vs 5.42 us), but
//     groups of three are faster from 2048 waves (7.81 vs 8.70 us) on;
//   * the general mapping (nkv = 2): bf16 gains at 1024 waves (5.85 vs 6.31
//     us) and is even at 2048; fp8 gains at 1536 (7.86 vs 8.47 us) and loses
//     12% at 2048 (10.0 vs 8.8 us);
//   * per-layer slot mappings (nkv = 8): bf16 gains 9% at 1024 waves, 8% at
//     4096 and 5.8% at 8192; fp8 one layer per wave beats groups of three
//     at 1024 waves (5.41 vs 6.21 us), groups of three win from 2048 on.
#ifndef DSPARK_SPLIT_MAX_WAVES_BF16
#define DSPARK_SPLIT_MAX_WAVES_BF16 16384
#endif
#ifndef DSPARK_SPLIT_MAX_WAVES_FP8
#define DSPARK_SPLIT_MAX_WAVES_FP8 1536
#endif
#ifndef DSPARK_SPLIT_MAX_WAVES_GENERAL_BF16
#define DSPARK_SPLIT_MAX_WAVES_GENERAL_BF16 1536
#endif
#ifndef DSPARK_SPLIT_MAX_WAVES_GENERAL_FP8
#define DSPARK_SPLIT_MAX_WAVES_GENERAL_FP8 1536
#endif
#ifndef DSPARK_SPLIT_MAX_WAVES_LAYER_SLOTS_BF16
#define DSPARK_SPLIT_MAX_WAVES_LAYER_SLOTS_BF16 16384
#endif
#ifndef DSPARK_SPLIT_MAX_WAVES_LAYER_SLOTS_FP8
#define DSPARK_SPLIT_MAX_WAVES_LAYER_SLOTS_FP8 1536
#endif
constexpr uint32_t kSplitMaxWavesBf16 = DSPARK_SPLIT_MAX_WAVES_BF16;
constexpr uint32_t kSplitMaxWavesFp8 = DSPARK_SPLIT_MAX_WAVES_FP8;
constexpr uint32_t kSplitMaxWavesGeneralBf16 = DSPARK_SPLIT_MAX_WAVES_GENERAL_BF16;
constexpr uint32_t kSplitMaxWavesGeneralFp8 = DSPARK_SPLIT_MAX_WAVES_GENERAL_FP8;
constexpr uint32_t kSplitMaxWavesLayerSlotsBf16 = DSPARK_SPLIT_MAX_WAVES_LAYER_SLOTS_BF16;
constexpr uint32_t kSplitMaxWavesLayerSlotsFp8 = DSPARK_SPLIT_MAX_WAVES_LAYER_SLOTS_FP8;
// Writes above those thresholds give each wave a group of this many layers
// (1: every layer of the row group in one wave), when L is larger.  Groups of
// three, measured at L = 5 (groups {0,1,2}, {3,4}) against whole row groups:
// fp8 prefill 25.0 -> 23.8 us at 8192 waves, -4.2% at 6144, -1.6% at 4096,
// long fp8 181.8 -> 176.7 us, per-layer slots fp8 -3.4%; bf16 -2.4% at 65536
// waves and even at 32768; the general mapping 6% slower (bf16, nkv = 2,
// 2048 waves) and even for fp8.  fp8 takes groups of two ({0,1}, {2,3},
// {4}): measured while the XCD remap applied to large launches only, the fp8
// prefill 23.59 -> 23.12 us against groups of three, long fp8 even (177.0 vs
// 176.4).
#ifndef DSPARK_GROUP_LAYERS_BF16
#define DSPARK_GROUP_LAYERS_BF16 3
#endif
#ifndef DSPARK_GROUP_LAYERS_FP8
#define DSPARK_GROUP_LAYERS_FP8 2
#endif
#ifndef DSPARK_GROUP_LAYERS_GENERAL
#define DSPARK_GROUP_LAYERS_GENERAL 1
#endif
constexpr int kGroupLayersBf16 = DSPARK_GROUP_LAYERS_BF16;
constexpr int kGroupLayersFp8 = DSPARK_GROUP_LAYERS_FP8;
constexpr int kGroupLayersGeneral = DSPARK_GROUP_LAYERS_GENERAL;
#ifndef DSPARK_FASTDIV
#define DSPARK_FASTDIV 1
#endif
#ifndef DSPARK_SLOT_FIRST
#define DSPARK_SLOT_FIRST 1
#endif
// Split launches with one token per wave test the token's slot (or its
// slots, with per-layer mappings) before issuing the row loads, so a
// padding token's rows are not read; other launches issue the loads ahead
// of the slot.
constexpr bool kSlotFirst = DSPARK_SLOT_FIRST;
constexpr int kRowsPerWave = 4;
constexpr int kMaxChunk = 8;   // layers held in registers at once
// Workgroup i runs on XCD i % 8; every launch remaps block ids so that each
// XCD takes a contiguous range of rows.  The waves of one token's layers then
// share one XCD's L2, which fetches the token's cos/sin row, slot and
// position once instead of once per XCD (decode: 1.016x its algorithmic
// bytes against 1.037x in round-robin order); long fp8 2.6% and the bf16
// prefill 0.8% faster, the smaller launches even (decode -0.4%, TP-4 shard
// -0.8%, fp8 prefill -0.3%, medians of 15 alternating rounds, twice).
#ifndef DSPARK_XCD_REMAP
#define DSPARK_XCD_REMAP 1
#endif
constexpr bool kXcdRemap = DSPARK_XCD_REMAP;
constexpr int kNumXcds = 8;

// kChunk = layers held in registers per pass; kSinglePass: L == kChunk (the
// whole write is one straight-line pass), else L > kChunk and the layers go
// in chunks of kChunk.
// kUniform: nkv % 4 == 0, so a wave's 4 rows are 4 heads of one token and the
// token's slot and position are wave-uniform (scalar loads, scalar exit).
// kLayerSlots: every layer has its own slot mapping (layers in different KV
// cache groups); with the uniform-token mapping each layer's slot is
// wave-uniform, else every quarter reads its own.
// kLayerSplit (single pass): each wave writes one group of kChunk layers of
// its 4 rows (the last group shorter); wave w takes layer group w % ng of row
// group w / ng.  The write then spreads over ng times more waves, each with
// an ng-th of the loads and arithmetic, so more of them are in flight at
// different phases.  One layer per wave up to the thresholds below, groups
// of three beyond.
// n / d for the wave-uniform index n: one multiply-high by the host's
// ceil(2^32 / d) when it is exact for every n of the launch (the host
// checks n d < 2^32), else a division.
__device__ __forceinline__ uint32_t fast_div(uint32_t n, uint32_t d, uint32_t magic) {
    if (DSPARK_FASTDIV && magic != 0) return __umulhi(n, magic);
    return d == 1 ? n : n / d;
}

template <int R, bool kFp8, int kChunk, bool kSinglePass, bool kUniform, bool kLayerSlots,
          bool kLayerSplit, int kWavesPerBlock>
__global__ __launch_bounds__(64 * kWavesPerBlock) void ctx_kv_write_kernel(const CtxKvArgs a) {
    static_assert(!kLayerSplit || kSinglePass, "a split wave holds one group of layers");
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4;        // quarter: which of the wave's 4 rows
    const int c = lane & 15;        // 16-byte chunk: elements 8c .. 8c+7
    int L = kSinglePass ? kChunk : a.num_layers;             // layers this wave writes
    const int Lrow = kLayerSplit ? a.num_layers : L;         // layers per all_kv token row
    const int nkv = a.nkv;
    // The kernel arguments the prologue branches on, and the pointers of its
    // first loads, are read in one batch before the first branch: the empty
    // instruction below takes them as inputs and yields the zero added to
    // the block index, so the compiler issues their scalar loads together
    // and waits once, instead of loading and waiting for each one where a
    // branch needs it (decode -1.2%, the TP-4 shard -1.9%, the large writes
    // even).  It touches no memory, so the slot and position reads stay
    // scalar loads.
    uint32_t zero_after_args;
    {
        const uint32_t nu = a.num_units, sm = a.split_magic, tm = a.token_magic, gd = gridDim.x;
        const int32_t nl = a.num_layers, bl = a.bs_log2;
        const int64_t *ps = a.positions, *ss = a.slots;
        const void *kv = a.all_kv, *kw = a.k_norm_weight, *cs = a.cos_sin;
        asm("s_mov_b32 %0, 0"
            : "=s"(zero_after_args)
            : "s"(nu), "s"(sm), "s"(tm), "s"(gd), "s"(nl), "s"(nkv), "s"(bl), "s"(ps), "s"(ss),
              "s"(kv), "s"(kw), "s"(cs));
    }

    uint32_t block = blockIdx.x + zero_after_args;
    if constexpr (kXcdRemap) {
        // blocks [0, full) are remapped so that XCD x owns one contiguous run
        const uint32_t full = gridDim.x - gridDim.x % kNumXcds;
        if (block < full) block = (block % kNumXcds) * (full / kNumXcds) + block / kNumXcds;
    }
    uint32_t wave = block * kWavesPerBlock +
                    static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    int l0 = 0;                     // first layer this wave writes
    if constexpr (kLayerSplit) {
        // wave w writes layer group w % ng (kChunk layers, the last one
        // shorter) of row group w / ng
        const uint32_t ng = (static_cast<uint32_t>(a.num_layers) + kChunk - 1) / kChunk;
        const uint32_t rg = fast_div(wave, ng, a.split_magic);
        l0 = static_cast<int>(wave - rg * ng) * kChunk;
        wave = rg;
        L = a.num_layers - l0 < kChunk ? a.num_layers - l0 : kChunk;
    }
    const uint32_t unit0 = wave * kRowsPerWave;             // first row of the wave
    if (unit0 >= a.num_units) return;

    uint32_t t;
    int h;
    int hu = 0;                     // uniform path: the head of quarter 0
    int64_t slot, pos;
    uint4 dk[kChunk], dv[kChunk], wv[kChunk];
    int64_t lslot[kChunk];          // per-layer slots (kLayerSlots only)
    // the slots are read and tested before the rows (split, one token per wave)
    constexpr bool kSlotsFirst = kSlotFirst && kLayerSplit && kUniform;
    bool in_range = true;
    const int64_t kv_stride = static_cast<int64_t>(nkv) * 16;    // K_l -> V_l (uint4 units)
    const uint4 *w_base = reinterpret_cast<const uint4 *>(a.k_norm_weight) + l0 * 16 + c;
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
            if constexpr (kLayerSlots && !kSlotsFirst) lslot[j] = a.layer_slots[l0 + l][t];
        }
    };
    // per-layer mappings: whether token t has a slot >= 0 in any of the
    // wave's layers.  Only such a token's cos/sin row is read, so a token
    // stored in no layer may carry any position.
    auto stored_in_any_layer = [&]() {
        bool any = false;
        if constexpr (kSinglePass) {
#pragma unroll
            for (int j = 0; j < kChunk; ++j) any |= (j < L) & (lslot[j] >= 0);
        } else {
            for (int l = 0; l < L; ++l) any |= a.layer_slots[l0 + l][t] >= 0;
        }
        return any;
    };
    if constexpr (kUniform) {
        t = fast_div(wave, static_cast<uint32_t>(nkv) / kRowsPerWave, a.token_magic);
        hu = static_cast<int>(unit0 - t * static_cast<uint32_t>(nkv));
        h = hu + q;
        kv_base = reinterpret_cast<const uint4 *>(a.all_kv) +
                  ((static_cast<int64_t>(t) * Lrow + l0) * 2 * nkv + h) * 16 + c;
        slot = kLayerSlots ? 0 : a.slots[t];    // per-layer slots: read per layer
        pos = a.positions[t];
        if constexpr (kSlotsFirst) {
            // one layer group per wave: the slot (read by every layer group's
            // wave of this row group, mostly from L2) is tested before any
            // row is read
            if constexpr (kLayerSlots) {
#pragma unroll
                for (int j = 0; j < kChunk; ++j)
                    lslot[j] = a.layer_slots[l0 + (j < L ? j : L - 1)][t];
                if (!stored_in_any_layer()) return;
            } else if (slot < 0 || pos < 0) {
                return;
            }
        }
        // Otherwise the row loads go out together with the slot load, so the
        // slot's latency overlaps theirs (a padding token's rows are then
        // read for nothing).  The barrier keeps the compiler from sinking
        // them below the padding exit.
        load_chunk(0);
        asm volatile("" ::: "memory");
        // padding: nothing written (a negative position never occurs; testing
        // it keeps both scalar loads ahead of the branch); with per-layer
        // slots each layer's store tests its own slot, and a token stored in
        // no layer of the wave ends here, before its cos/sin row is read
        if constexpr (kLayerSlots) {
            if (!stored_in_any_layer()) return;
        } else if (slot < 0 || pos < 0) {
            return;
        }
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
                  ((static_cast<int64_t>(t) * Lrow + l0) * 2 * nkv + h) * 16 + c;
        load_chunk(0);
        asm volatile("" ::: "memory");   // keep the loads ahead of the predicated stores
        // a quarter whose token is stored in no layer (or past the end) reads
        // cos/sin row 0 instead of its position's row; its stores are off
        const bool stores = in_range && stored_in_any_layer();
        if (__ballot(stores) == 0) return;
        if (!stores) pos = 0;
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
                  ((static_cast<int64_t>(t) * Lrow + l0) * 2 * nkv + h) * 16 + c;
        load_chunk(0);
    }

    // this token's (cos, sin) for the 8 pair indices of this lane
    uint32_t cs[8];
    rope_operands<R>(a.cos_sin + pos * R, c, cs);

    const int64_t blk = slot >> a.bs_log2;
    const int64_t off = slot & ((int64_t{1} << a.bs_log2) - 1);
    // element index of this row inside any layer's cache, plus this lane's chunk
    const int64_t row = ((((blk * nkv + h) << a.bs_log2) + off) * (2 * DSPARK_HEAD_DIM)) + c * 8;
    // uniform path: quarter q's row lies (q << bs_log2) rows after quarter 0's,
    // whose address is the same for the whole wave, so the stores go through
    // a buffer resource on that address with the sc1 policy (lane offsets
    // below 2^31 bytes while block_size <= 2^20)
    const int64_t row0 = (((blk * nkv + hu) << a.bs_log2) + off) * (2 * DSPARK_HEAD_DIM);
    const uint32_t lane_elem =
        (static_cast<uint32_t>(q) << a.bs_log2) * (2 * DSPARK_HEAD_DIM) + static_cast<uint32_t>(c) * 8;
    const bool sc1 = !kUniform || a.bs_log2 <= 20;   // the other paths check per layer

    for (int lb = 0;;) {
        // fp8: lane 2j holds layer lb+j's k scale, lane 2j+1 its v scale, and
        // one IEEE division gives every reciprocal of the chunk
        float my_scale = 1.0f, my_rcp = 1.0f;
        if constexpr (kFp8) {
            // The chunk's scale offsets are wave-uniform: all of them are
            // read as one batch of scalar loads, and the empty instruction
            // below keeps the compiler from moving each load into a branch
            // of its own lane's select (which waited once per offset: the
            // fp8 prefill 2.6-5.4% slower, per-layer fp8 6%).
            int64_t ko[kChunk], vo[kChunk];
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                const int l = l0 + (lb + j < L ? lb + j : L - 1);
                ko[j] = a.kscale_off[l];
                vo[j] = a.vscale_off[l];
            }
#pragma unroll
            for (int j = 0; j < kChunk; ++j) asm("" : "+s"(ko[j]), "+s"(vo[j]));
            int64_t soff = 0;
#pragma unroll
            for (int j = 0; j < kChunk; ++j)
                soff = lane == 2 * j ? ko[j] : lane == 2 * j + 1 ? vo[j] : soff;
            if (lane < 2 * (L - lb < kChunk ? L - lb : kChunk)) my_scale = a.scale0[soff];
            my_rcp = 1.0f / my_scale;
        }
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const int l = lb + j;
            if (l >= L) break;
            uint32_t kb[4];
            norm_rope<R>(dk[j], wv[j], a.eps, c, cs, kb);
            // element index of this lane's row start (chunk excluded) in layer l
            int64_t rbase = a.cache_off[l0 + l] + row - c * 8;
            bool store = true;
            int64_t lrow0 = row0;          // uniform path: quarter 0's row in layer l
            if constexpr (kLayerSlots) {
                const int64_t s = lslot[j];
                store = in_range && s >= 0;
                const int64_t lb_blk = s >> a.bs_log2;
                const int64_t lb_off = s & ((int64_t{1} << a.bs_log2) - 1);
                rbase = a.cache_off[l0 + l] +
                        ((((lb_blk * nkv + h) << a.bs_log2) + lb_off) * (2 * DSPARK_HEAD_DIM));
                if constexpr (kUniform) {
                    // the token's slot in this layer is wave-uniform
                    if (!store) continue;
                    lrow0 = (((lb_blk * nkv + hu) << a.bs_log2) + lb_off) * (2 * DSPARK_HEAD_DIM);
                }
            }
            // the stores go through a buffer resource on a wave-uniform base
            // with the sc1 policy when every lane's offset fits in 31 bits,
            // else as nontemporal stores to the lane's address
            constexpr int kEsz = kFp8 ? 1 : 2;
            bool use_sc1 = sc1;
            __amdgpu_buffer_rsrc_t r;
            uint32_t loff;
            if constexpr (kUniform) {
                r = wave_rsrc(static_cast<char *>(a.cache0) + (a.cache_off[l0 + l] + lrow0) * kEsz);
                loff = lane_elem * kEsz;
            } else if constexpr (!kLayerSlots) {
                // the general row mapping (quarters of different tokens, nkv
                // not a multiple of 4) measured slower with sc1 stores (the
                // 4096-token prefill at nkv = 2: 10.2 vs 9.3 us)
                use_sc1 = false;
                r = wave_rsrc(a.cache0);
                loff = 0;
            } else {
                // per-layer slots: the base is the lowest of the four row
                // starts (a row this layer does not store takes the first
                // stored one's address)
                int64_t qa = reinterpret_cast<int64_t>(static_cast<char *>(a.cache0) + rbase * kEsz);
                const uint64_t sm = __ballot(store);
                if (sm == 0) continue;
                if (!store) qa = read_lane64(qa, static_cast<int>(__builtin_ctzll(sm)));
                const int64_t a0 = read_lane64(qa, 0), a1 = read_lane64(qa, 16);
                const int64_t a2 = read_lane64(qa, 32), a3 = read_lane64(qa, 48);
                const int64_t lo = a0 < a1 ? (a0 < a2 ? (a0 < a3 ? a0 : a3) : (a2 < a3 ? a2 : a3))
                                           : (a1 < a2 ? (a1 < a3 ? a1 : a3) : (a2 < a3 ? a2 : a3));
                const int64_t hi = a0 > a1 ? (a0 > a2 ? (a0 > a3 ? a0 : a3) : (a2 > a3 ? a2 : a3))
                                           : (a1 > a2 ? (a1 > a3 ? a1 : a3) : (a2 > a3 ? a2 : a3));
                use_sc1 = hi - lo < (int64_t{1} << 31) - 1024;
                r = wave_rsrc(reinterpret_cast<void *>(lo));
                loff = static_cast<uint32_t>(qa - lo) + static_cast<uint32_t>(c) * 8 * kEsz;
            }
            const int64_t base = rbase + c * 8;
            if constexpr (!kFp8) {
                if (use_sc1) {
                    if (store) {
                        store16_sc1(r, loff, make_uint4(kb[0], kb[1], kb[2], kb[3]));
                        store16_sc1(r, loff + DSPARK_HEAD_DIM * 2, dv[j]);
                    }
                } else {
                    uint16_t *cache = static_cast<uint16_t *>(a.cache0) + base;
                    if (store) {
                        store_row16(cache, make_uint4(kb[0], kb[1], kb[2], kb[3]));
                        store_row16(cache + DSPARK_HEAD_DIM, dv[j]);
                    }
                }
            } else {
                const float ks = lane_value(my_scale, 2 * j), kr = lane_value(my_rcp, 2 * j);
                const float vs = lane_value(my_scale, 2 * j + 1), vr = lane_value(my_rcp, 2 * j + 1);
                const uint32_t vb[4] = {dv[j].x, dv[j].y, dv[j].z, dv[j].w};
                const uint2 ko = pack_fp8(kb, ks, kr, 460.0f * ks);
                const uint2 vo = pack_fp8(vb, vs, vr, 460.0f * vs);
                if (use_sc1) {
                    if (store) {
                        store8_sc1(r, loff, ko);
                        store8_sc1(r, loff + DSPARK_HEAD_DIM, vo);
                    }
                } else {
                    uint8_t *cache = static_cast<uint8_t *>(a.cache0) + base;
                    if (store) {
                        store_row8(cache, ko);
                        store_row8(cache + DSPARK_HEAD_DIM, vo);
                    }
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

template <int R, bool kFp8, int kChunk, bool kSinglePass, int kWavesPerBlock>
void launch_wpb(const CtxKvArgs &args, uint32_t waves, hipStream_t stream) {
    const dim3 grid((waves + kWavesPerBlock - 1) / kWavesPerBlock);
    const dim3 block(64 * kWavesPerBlock);
    CtxKvArgs a = args;
    if (a.layer_slots_on && a.nkv % kRowsPerWave == 0)
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, kChunk, kSinglePass, true, true, false,
                                                kWavesPerBlock>), grid, block, 0, stream, a);
    else if (a.layer_slots_on)
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, kChunk, kSinglePass, false, true, false,
                                                kWavesPerBlock>), grid, block, 0, stream, a);
    else if (a.nkv % kRowsPerWave == 0)
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, kChunk, kSinglePass, true, false, false,
                                                kWavesPerBlock>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, kChunk, kSinglePass, false, false, false,
                                                kWavesPerBlock>), grid, block, 0, stream, a);
}

// ceil(2^32 / d) if n_max * d < 2^32 (then n / d == umulhi(n, magic) for
// every n <= n_max), else 0.
uint32_t div_magic(uint64_t n_max, uint64_t d) {
    if (d < 2 || (n_max + 1) * d >= (uint64_t{1} << 32)) return 0;
    return static_cast<uint32_t>(((uint64_t{1} << 32) + d - 1) / d);
}

// One wave per (row group, group of kGroup layers), four waves per workgroup.
template <int R, bool kFp8, int kGroup>
void launch_split(const CtxKvArgs &args, uint32_t waves, hipStream_t stream) {
    CtxKvArgs a = args;
    const uint32_t ng = (static_cast<uint32_t>(a.num_layers) + kGroup - 1) / kGroup;
    const uint32_t split = waves * ng;
    a.split_magic = div_magic(uint64_t{split} + 3, ng);
    const dim3 grid((split + 3) / 4);
    const dim3 block(256);
    if (a.layer_slots_on && a.nkv % kRowsPerWave == 0)
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, kGroup, true, true, true, true, 4>),
                           grid, block, 0, stream, a);
    else if (a.layer_slots_on)
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, kGroup, true, false, true, true, 4>),
                           grid, block, 0, stream, a);
    else if (a.nkv % kRowsPerWave == 0)
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, kGroup, true, true, false, true, 4>),
                           grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((ctx_kv_write_kernel<R, kFp8, kGroup, true, false, false, true, 4>),
                           grid, block, 0, stream, a);
}

template <int R, bool kFp8, int kChunk, bool kSinglePass>
void launch_one(const CtxKvArgs &args, hipStream_t stream) {
    CtxKvArgs a = args;
    const uint32_t waves = (a.num_units + kRowsPerWave - 1) / kRowsPerWave;
    if (a.nkv % kRowsPerWave == 0)
        a.token_magic = div_magic(waves, static_cast<uint32_t>(a.nkv) / kRowsPerWave);
    const bool general = !a.layer_slots_on && a.nkv % kRowsPerWave != 0;
    const uint32_t max_split =
        a.layer_slots_on ? (kFp8 ? kSplitMaxWavesLayerSlotsFp8 : kSplitMaxWavesLayerSlotsBf16)
        : !general       ? (kFp8 ? kSplitMaxWavesFp8 : kSplitMaxWavesBf16)
                         : (kFp8 ? kSplitMaxWavesGeneralFp8 : kSplitMaxWavesGeneralBf16);
    if (a.num_layers > 1 && waves <= max_split) {
        launch_split<R, kFp8, 1>(a, waves, stream);
        return;
    }
    // a split launch numbers its waves in 32 bits (wave count times layer
    // groups); a write too large for that keeps whole row groups per wave
    auto split_fits = [&](int group) {
        const uint64_t ng = (static_cast<uint64_t>(a.num_layers) + group - 1) / group;
        return uint64_t{waves} * ng + 4 < (uint64_t{1} << 32);
    };
    constexpr int kGroup = kFp8 ? kGroupLayersFp8 : kGroupLayersBf16;
    if (kGroup > 1 && !general && a.num_layers > kGroup && split_fits(kGroup)) {
        launch_split<R, kFp8, kGroup>(a, waves, stream);
        return;
    }
    if (kGroupLayersGeneral > 1 && general && a.num_layers > kGroupLayersGeneral &&
        split_fits(kGroupLayersGeneral)) {
        launch_split<R, kFp8, kGroupLayersGeneral>(a, waves, stream);
        return;
    }
    launch_wpb<R, kFp8, kChunk, kSinglePass, kWavesPerGroup>(a, waves, stream);
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
