// csa2_attn.hip -- CSA2 sparse attention over the FP4 global KV plus the FP8
// sliding window.
//
// "DeepSeek V4.1 Flash: architecture study notes", section 2: each query
// attends to at most 512 selected global records together with its local
// window; section 1: the window is 128 tokens and every layer keeps its own;
// section 4: the FP4 cache is dequantised on read and fed to ordinary
// attention (the saving is storage, not FP4 arithmetic); the SWA KV stays FP8.
//
// Design (gfx950).  A query's entries (selected records, then window tokens)
// are cut into tiles of 32.  One workgroup of W waves serves one (query, group
// of 16 heads); wave w takes tiles w, w + W, w + 2W, ..., keeps its own online
// softmax state, and the W states are merged through LDS at the end, so one
// launch produces the output.  All heads share one KV head (MQA), so per tile
// the logits are a dense [32 entries x 16 heads] contraction on MFMA
// (v_mfma_f32_16x16x32_f16):
//   - S^T = K Q^T: lane (entry c, quarter g) of row block blk holds channels
//     [32g, 32g + 32) of entry 16 blk + c (16 bytes of E2M1 codes, or 32 bytes
//     of E4M3 for a window token); MFMA step ks consumes channels
//     32g + 8ks .. +8 of that lane group, and q is laid out with the same
//     channel permutation, which leaves every dot product unchanged.  The lane
//     loads the two E4M3 group scales of exactly those channels itself (one
//     2-byte load), so no scale is moved between lanes.
//   - O^T += V^T P^T: P comes straight from the S^T registers (a lane holds
//     entries 4g..4g+3 and 16+4g..16+4g+3 of its head); V is dequantised by
//     the lane that loaded it, written row-major into a wave-private LDS tile
//     and read back transposed (ds_read_b64_tr_b16) as the A operand.
//   - the softmax denominator of the selected records is one more MFMA per
//     tile with an all-ones A operand: it sums exactly the fp16 probabilities
//     that weight the values.
//   - dequantised E2M1 x E4M3 values have at most 6 significant bits in
//     [2^-10, 2688], so they are exact in fp16; E4M3 window codes are exact in
//     fp16 and their fp32 row scales are applied to the logit (K) and to the
//     probability (V) in fp32.  A window tile's probabilities times V scales
//     are brought into [128, 256) per head by a power of two before the fp16
//     cast, and its PV product is scaled back in fp32, so small window scales
//     do not fall into fp16 subnormals.
//   - q * sm_scale * log2(e) is split into fp16 hi + lo (22 significant bits)
//     after a per-head power-of-two scaling that puts the head's largest
//     magnitude into [2^14, 2^15); logits are scaled back in fp32.
//   - softmax is online in fp32 with base-2 exponentials; a wave's reference
//     maximum moves only when a tile's maximum passes it by more than 8
//     (log2 units), so most tiles skip the rescale.
// Absent entries (slots past top-K, positions outside [0, cap), window tokens
// past the window length) are read from a valid row and masked to -inf, so
// the loads need no per-entry branches.  Workgroups are numbered so that the
// head groups of one query land on the same XCD (consecutive workgroup ids go
// round-robin over the 8 XCDs), sharing its L2 for the gathered rows.
#include <hip/hip_ext.h>

#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;           // entries per tile
// waves per workgroup: 8, or 4 when there are enough (query, head group)
// workgroups for two of them to share each CU, so that they all run in one
// round
constexpr int kWavesWide = 8, kWavesNarrow = 4;
constexpr int kGroupHeads = 16;     // heads per workgroup (one MFMA column block)
constexpr int kVPitch = 144;        // fp16 per V row in LDS (128 + 16)
constexpr int kMergePitch = kHeadDim + 4;  // fp32 per merged output row in LDS
constexpr int kXcds = 8;
constexpr int kCusPerChip = 256;
constexpr int kMaxWindow = 128;     // window tokens a query attends to
constexpr int kPosRegs = 4;         // position registers per wave: 2 tiles each
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag the true max
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS: per-wave V tiles, then the merge area (each wave's output rows,
// reference maxima and sums), so a wave can store its state as soon as its
// own tiles are done
constexpr int kWaveBytes = kTile * kVPitch * 2;
// a wave's merge rows (16 heads x 128 fp32, its running max and sum per
// head) go into its own V-tile area once it is done with its tiles
constexpr int kWaveMergeBytes = (kGroupHeads * kMergePitch + 2 * kGroupHeads) * 4;
// q of the workgroup's 16 heads as fp16 hi and lo rows, and each head's scale
constexpr int kQPitch = kHeadDim + 8;  // fp16 per q row
constexpr int kQBytes = 2 * kGroupHeads * kQPitch * 2 + kGroupHeads * 4;
constexpr int lds_bytes(int W) { return W * kWaveBytes + kQBytes; }
static_assert(kWaveMergeBytes <= kWaveBytes, "a wave's merge rows fit its tile area");
static_assert(lds_bytes(kWavesWide) <= 160 * 1024, "LDS");
static_assert(3 * lds_bytes(kWavesNarrow) <= 160 * 1024, "three narrow workgroups per CU");

// Stage of a layer group (raw bytes of the selected records as the lanes hold
// them): per tile four 1 KiB planes of 16 bytes per lane (K block 0, K block
// 1, V half 0, V half 1), two 256-byte planes of one dword per lane (K scale
// pairs, V scale pairs) and the 32-bit presence mask.
constexpr int kStageK0 = 0, kStageK1 = 1024, kStageV0 = 2048, kStageV1 = 3072;
constexpr int kStageKs = 4096, kStageVs = 4352, kStageValid = 4608;
static_assert(kStageValid + 4 <= kStageTileBytes, "stage tile");

size_t attn_workspace_bytes(int64_t, int, int, int) { return 0; }

// Where one workgroup finds its entries.
struct SeqView {
    const uint8_t* kvc;    // this sequence's code rows
    const uint8_t* kvs;    // this sequence's scale rows
    const uint8_t* swk;    // this query's first window row (K codes)
    const uint8_t* swv;
    const float* swks;     // this query's first window row scale
    const float* swvs;
    const int32_t* idx;    // this query's top-K row
    uint8_t* stage;        // this query's staged tiles, or null
    int stage_rem, stage_mod;  // a writing workgroup writes the tiles t with t % mod == rem
    int64_t cap;
    int topk;
    int swa_len;   // window tokens attended (known at process time)
    int win_rows;  // window rows readable from swk / swv (known at entry)
    int n_tiles_global;
};

// Raw bytes of one tile of selected records held by one lane (c = lane & 15,
// g = lane >> 4, q4 = lane & 3):
//   k[blk]  E2M1 codes of entry 16 blk + c, channels [32g, 32g + 32)
//   v[j]    E2M1 codes of entry 16j + lane/4, channels [32 q4, +32)
//   ks      E4M3 scales of the lane's K channels: bits 0..15 for block 0
//           (groups 2g, 2g + 1), bits 16..31 for block 1
//   vs      the same for the lane's V channels (groups 2 q4, 2 q4 + 1)
//   valid   bit e: entry e of the tile is present (equal in every lane)
struct GTile {
    u32x4_t k[2];
    u32x4_t v[2];
    uint32_t ks, vs;
    uint32_t valid;
};

// Raw bytes of one tile of window tokens held by one lane (q8 = lane & 7):
//   k[blk][h]  E4M3 codes of token 16 blk + c, channels [32g + 16h, +16)
//   v[j]       E4M3 codes of token 8j + lane/8, channels [16 q8, +16)
//   sc         lanes 0..31: fp32 K row scale of token `lane`; lanes 32..63:
//              V row scale of token `lane - 32`
struct WTile {
    u32x4_t k[2][2];
    u32x4_t v[4];
    float sc;
};

__device__ __forceinline__ u32x4_t ld16(const uint8_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ uint32_t ld2(const uint8_t* p) {
    return *reinterpret_cast<const uint16_t*>(p);
}

// position of entry e held by lane `src` of a position register
__device__ __forceinline__ int32_t lane_value(int32_t v, int src) {
    return __builtin_amdgcn_ds_bpermute(src << 2, v);
}

// Issue the loads of global tile t.  P: the position register holding the
// tile (entry e in lane 32 * half + e); STAGE_READ ignores it.
template <int STAGE>
__device__ __forceinline__ void fetch_global(const SeqView& s, int t, int32_t P, int half,
                                             int lane, GTile& r) {
    const int c = lane & 15, g = lane >> 4, q4 = lane & 3;
    if (STAGE == kStageRead) {
        const uint8_t* src = s.stage + (int64_t)t * kStageTileBytes;
        r.k[0] = ld16(src + kStageK0 + 16 * lane);
        r.k[1] = ld16(src + kStageK1 + 16 * lane);
        r.v[0] = ld16(src + kStageV0 + 16 * lane);
        r.v[1] = ld16(src + kStageV1 + 16 * lane);
        r.ks = *reinterpret_cast<const uint32_t*>(src + kStageKs + 4 * lane);
        r.vs = *reinterpret_cast<const uint32_t*>(src + kStageVs + 4 * lane);
        r.valid = *reinterpret_cast<const uint32_t*>(src + kStageValid);  // same in every lane
        return;
    }
    // P holds -1 for absent entries; they read row 0 and are masked later
    const int base = 32 * half;
    const int32_t pk0 = lane_value(P, base + c), pk1 = lane_value(P, base + 16 + c);
    const int32_t pv0 = lane_value(P, base + (lane >> 2)), pv1 = lane_value(P, base + 16 + (lane >> 2));
    const int64_t rk0 = pk0 < 0 ? 0 : pk0, rk1 = pk1 < 0 ? 0 : pk1;
    const int64_t rv0 = pv0 < 0 ? 0 : pv0, rv1 = pv1 < 0 ? 0 : pv1;
    r.k[0] = ld16(s.kvc + rk0 * 128 + 16 * g);
    r.k[1] = ld16(s.kvc + rk1 * 128 + 16 * g);
    r.v[0] = ld16(s.kvc + rv0 * 128 + 64 + 16 * q4);
    r.v[1] = ld16(s.kvc + rv1 * 128 + 64 + 16 * q4);
    const uint32_t ks0 = ld2(s.kvs + rk0 * 16 + 2 * g), ks1 = ld2(s.kvs + rk1 * 16 + 2 * g);
    const uint32_t vs0 = ld2(s.kvs + rv0 * 16 + 8 + 2 * q4), vs1 = ld2(s.kvs + rv1 * 16 + 8 + 2 * q4);
    r.ks = ks0 | (ks1 << 16);
    r.vs = vs0 | (vs1 << 16);
    r.valid = (uint32_t)(__builtin_amdgcn_ballot_w64(P >= 0) >> base);
}

// Issue the loads of window tile j (tokens [32j, 32j + 32) of the query's
// window).  Rows past the readable window rows read its first row; which
// tokens count is decided when the tile is processed.
__device__ __forceinline__ void fetch_window(const SeqView& s, int j, int lane, WTile& r) {
    const int c = lane & 15, g = lane >> 4;
    const int tok0 = j * kTile;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int tok = tok0 + 16 * blk + c;
        const uint8_t* src = s.swk + (int64_t)(tok < s.win_rows ? tok : 0) * kHeadDim + 32 * g;
        r.k[blk][0] = ld16(src);
        r.k[blk][1] = ld16(src + 16);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int tok = tok0 + 8 * jj + (lane >> 3);
        r.v[jj] = ld16(s.swv + (int64_t)(tok < s.win_rows ? tok : 0) * kHeadDim + 16 * (lane & 7));
    }
    const int tok = tok0 + (lane & 31);
    const int row = tok < s.win_rows ? tok : 0;
    r.sc = lane < 32 ? s.swks[row] : s.swvs[row];
}

// IEEE 754-2019 maximum (v_maximum3_f32 on gfx950): the same value as fmaxf
// for every input but NaN, without the NaN-quieting instruction fmaxf costs
// per operand here (MFMA results and lane swaps are not known to be quiet)
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max / sum over the four lanes c, c+16, c+32, c+48 (v_permlane*_swap: each
// call hands every lane its partner's value 32 resp. 16 lanes away)
// max over each half wave (lanes 0..31, 32..63; every lane active), in every
// lane: DPP within each 16-lane row, then the row pair through a lane swap
__device__ __forceinline__ float half_wave_max(float v) {
    v = fmaxf(v, dppf<0xB1>(v));
    v = fmaxf(v, dppf<0x4E>(v));
    v = fmaxf(v, dppf<0x141>(v));
    v = fmaxf(v, dppf<0x140>(v));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float xmax4(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float xsum4(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Eight E2M1 codes times an fp16 scale pair element (SEL 0: low, 1: high), as
// one MFMA operand.
template <int SEL>
__device__ __forceinline__ half8_t fp4x8_h8(uint32_t w, half2_t s) {
    const half2_t s2 = __builtin_shufflevector(s, s, SEL, SEL);
    const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    const half4_t a = __builtin_shufflevector(h0, h1, 0, 1, 2, 3);
    const half4_t b = __builtin_shufflevector(h2, h3, 0, 1, 2, 3);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Eight E4M3 codes (two dwords), exact in fp16, as one MFMA operand.
__device__ __forceinline__ half8_t fp8x8_h8(uint32_t w0, uint32_t w1) {
    const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    const half4_t a = __builtin_shufflevector(h0, h1, 0, 1, 2, 3);
    const half4_t b = __builtin_shufflevector(h2, h3, 0, 1, 2, 3);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

struct WaveState {
    float4_t o[8];  // O^T[dim 16 dt + 4g + r][head c], relative to m
    float4_t lsum;  // sum of the fp16 probabilities of selected records (all four equal)
    float lwin;     // this lane's share of the window tokens' probabilities
    float m;        // reference (base-2 logit) of head c; lags its running max by < 8
};

// The lane's C entries: 4g + i (i < 4) and 16 + 4g + i - 4 (i >= 4).
__device__ __forceinline__ int c_entry(int i, int g) { return i < 4 ? 4 * g + i : 12 + 4 * g + i; }

// Raise the reference maximum when this tile's maximum passes it by more than
// the slack (uniform branch over the wave).
__device__ __forceinline__ void online_rescale(float tmax, WaveState& st) {
    const bool move = tmax > st.m + kRescaleSlack || (st.m == -INFINITY && tmax != -INFINITY);
    if (__builtin_amdgcn_ballot_w64(move)) {
        const float m_new = move ? tmax : st.m;
        // a head whose maximum is still -inf has accumulated nothing (every
        // tile has a present entry, so its first one sets the maximum): the
        // scaling is skipped while that holds for the whole wave
        if (__builtin_amdgcn_ballot_w64(st.m != -INFINITY)) {
            const float alpha = (st.m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(st.m - m_new);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) st.o[dt] *= alpha;
            st.lsum *= alpha;
            st.lwin *= alpha;
        }
        st.m = m_new;
    }
}

// Transposed V operands from the wave's row-major V tile: in each 16-lane
// group, lane 4j + i/4 supplies channels [16dt + 4(i/4), +4) of the entry at
// k slot j, and lane i receives channel 16dt + i of the four entries.
__device__ __forceinline__ half8_t v_operand(const _Float16* vtile, int lane, int dt) {
    const int sq = lane & 15, g = lane >> 4;
    const int ent0 = 4 * g + (sq >> 2), ent1 = 16 + 4 * g + (sq >> 2);
    const int col = 16 * dt + 4 * (sq & 3);
    const half4_t v0 = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4_t*)(vtile + ent0 * kVPitch + col)));
    const half4_t v1 = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4_t*)(vtile + ent1 * kVPitch + col)));
    return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The MFMA B operands of the wave's q (head c, MFMA step ks: channels
// 32g + 8ks .. +8, fp16 hi and lo parts): held in registers for the whole
// kernel (QRegs), or read from the workgroup's LDS rows at each use (QLds,
// 32 registers fewer).
struct QRegs {
    half8_t h[4], l[4];
    __device__ __forceinline__ half8_t hi(int ks) const { return h[ks]; }
    __device__ __forceinline__ half8_t lo(int ks) const { return l[ks]; }
};
struct QLds {
    const _Float16* h;  // q_hi + c * kQPitch + 32 g
    const _Float16* l;
    __device__ __forceinline__ half8_t hi(int ks) const { return *reinterpret_cast<const half8_t*>(h + 8 * ks); }
    __device__ __forceinline__ half8_t lo(int ks) const { return *reinterpret_cast<const half8_t*>(l + 8 * ks); }
};

// One tile of selected FP4 records.
template <int STAGE, class QOps>
__device__ __forceinline__ void process_global(const SeqView& s, int t, const GTile& r,
                                               const QOps& q, float qmul,
                                               _Float16* __restrict__ vtile, int lane,
                                               WaveState& st) {
    const int g = lane >> 4;
    if (STAGE == kStageWrite && t % s.stage_mod == s.stage_rem) {
        // hand the gathered bytes on to the layers that reuse this selection
        uint8_t* dst = s.stage + (int64_t)t * kStageTileBytes;
        *reinterpret_cast<u32x4_t*>(dst + kStageK0 + 16 * lane) = r.k[0];
        *reinterpret_cast<u32x4_t*>(dst + kStageK1 + 16 * lane) = r.k[1];
        *reinterpret_cast<u32x4_t*>(dst + kStageV0 + 16 * lane) = r.v[0];
        *reinterpret_cast<u32x4_t*>(dst + kStageV1 + 16 * lane) = r.v[1];
        *reinterpret_cast<uint32_t*>(dst + kStageKs + 4 * lane) = r.ks;
        *reinterpret_cast<uint32_t*>(dst + kStageVs + 4 * lane) = r.vs;
        if (lane == 0) *reinterpret_cast<uint32_t*>(dst + kStageValid) = r.valid;
    }
    const uint32_t valid = __builtin_amdgcn_readfirstlane(r.valid);
    if (valid == 0u) return;  // uniform: nothing present (padding)

    // ---- V: dequantised row-major into the wave's V tile ----
    {
        const int q4 = lane & 3;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            half8_t* dst = reinterpret_cast<half8_t*>(vtile + (16 * j + (lane >> 2)) * kVPitch + 32 * q4);
            const half2_t sv = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.vs >> (16 * j), 1.0f, false);
            dst[0] = fp4x8_h8<0>(r.v[j][0], sv);
            dst[1] = fp4x8_h8<0>(r.v[j][1], sv);
            dst[2] = fp4x8_h8<1>(r.v[j][2], sv);
            dst[3] = fp4x8_h8<1>(r.v[j][3], sv);
        }
    }

    // ---- S^T = K Q^T (scaled base-2 logits) ----
    float4_t sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const half2_t sk = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.ks >> (16 * blk), 1.0f, false);
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const half8_t ka = ks < 2 ? fp4x8_h8<0>(r.k[blk][ks], sk) : fp4x8_h8<1>(r.k[blk][ks], sk);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, q.hi(ks), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, q.lo(ks), acc, 0, 0, 0);
        }
        sacc[blk] = acc;
    }

    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = sacc[i >> 2][i & 3];
    if (valid != 0xFFFFFFFFu) {  // uniform: mask the absent entries
        const uint32_t vb = ((valid >> (4 * g)) & 0xFu) | (((valid >> (16 + 4 * g)) & 0xFu) << 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (vb >> i) & 1u ? x[i] : -INFINITY;
    }
    float tmax = vmax(vmax(vmax(x[0], x[1]), vmax(x[2], x[3])),
                      vmax(vmax(x[4], x[5]), vmax(x[6], x[7])));
    tmax = xmax4(tmax) * qmul;
    online_rescale(tmax, st);
    half8_t pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(x[i], qmul, -st.m));

    wave_lds_sync();
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v_operand(vtile, lane, dt), pb, st.o[dt], 0, 0, 0);
    const half8_t ones = {1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16};
    st.lsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb, st.lsum, 0, 0, 0);
    wave_lds_sync();  // the next tile rewrites the V tile
}

// One tile of FP8 window tokens, of which the first n (>= 1) are attended.
template <class QOps>
__device__ __forceinline__ void process_window(const WTile& r, int n, const QOps& q, float qmul,
                                               _Float16* __restrict__ vtile, int lane,
                                               WaveState& st) {
    const int g = lane >> 4;
    const uint32_t valid = n >= kTile ? 0xFFFFFFFFu : ((1u << n) - 1u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        half8_t* dst = reinterpret_cast<half8_t*>(vtile + (8 * j + (lane >> 3)) * kVPitch + 16 * (lane & 7));
        dst[0] = fp8x8_h8(r.v[j][0], r.v[j][1]);
        dst[1] = fp8x8_h8(r.v[j][2], r.v[j][3]);
    }
    float4_t sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const half8_t ka = fp8x8_h8(r.k[blk][ks >> 1][2 * (ks & 1)], r.k[blk][ks >> 1][2 * (ks & 1) + 1]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, q.hi(ks), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, q.lo(ks), acc, 0, 0, 0);
        }
        sacc[blk] = acc;
    }
    float ksc[8], vsc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = c_entry(i, g);
        ksc[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(e << 2, __float_as_int(r.sc)));
        vsc[i] = __int_as_float(__builtin_amdgcn_ds_bpermute((32 + e) << 2, __float_as_int(r.sc)));
    }
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = sacc[i >> 2][i & 3] * qmul * ksc[i];
    if (valid != 0xFFFFFFFFu) {
        const uint32_t vb = ((valid >> (4 * g)) & 0xFu) | (((valid >> (16 + 4 * g)) & 0xFu) << 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (vb >> i) & 1u ? x[i] : -INFINITY;
    }
    float tmax = vmax(vmax(vmax(x[0], x[1]), vmax(x[2], x[3])),
                      vmax(vmax(x[4], x[5]), vmax(x[6], x[7])));
    tmax = xmax4(tmax);
    online_rescale(tmax, st);
    float w[8], wmax = 0.0f, psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(x[i] - st.m);
        psum += p;
        w[i] = p * vsc[i];
        wmax = vmax(wmax, w[i]);
    }
    st.lwin += psum;
    wmax = xmax4(wmax);
    // p * V scale of the head, brought into [128, 256) by a power of two; the
    // exponent is clamped so that both factors stay normal fp32 numbers (a
    // head whose window weights are all below 2^-100 keeps them as they are,
    // scaled by 2^108: still far inside the fp16 range)
    int e = wmax > 0.0f ? __builtin_amdgcn_frexp_expf(wmax) : 0;
    e = e < -100 ? -100 : (e > 120 ? 120 : e);
    const float up = __builtin_amdgcn_ldexpf(1.0f, 8 - e), down = __builtin_amdgcn_ldexpf(1.0f, e - 8);
    half8_t pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = (_Float16)(w[i] * up);

    wave_lds_sync();
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const float4_t zero = {0.f, 0.f, 0.f, 0.f};
        const float4_t pv = __builtin_amdgcn_mfma_f32_16x16x32_f16(v_operand(vtile, lane, dt), pb, zero, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.o[dt][i] = fmaf(pv[i], down, st.o[dt][i]);
    }
    wave_lds_sync();
}

// Every argument is needed before the first gather; touching them all at
// kernel entry makes the compiler fetch them in one batch of scalar loads
// instead of one dependent batch per first use.
template <class T>
__device__ __forceinline__ void touch(const T& v) {
    asm volatile("" ::"s"(v));
}

// grid = ceil(n_q / 8) * 8 * (H / 16) workgroups of W waves.
// Workgroup id -> (query bq, head group hg): ids with the same id % 8 share an
// XCD, and all head groups of one query get ids with the same id % 8.
template <int STAGE, int kWaves>
__global__ __launch_bounds__(kWaves * 64, kWaves == kWavesNarrow ? 3 : 2) void k_attn(AttnArgs a, int n_tiles_global) {
    constexpr int kThreads = kWaves * 64;
    __shared__ __attribute__((aligned(16))) unsigned char smem[lds_bytes(kWaves)];
    touch(a.q); touch(a.H); touch(a.Q); touch(a.kvc); touch(a.kvs); touch(a.cap);
    touch(a.idx); touch(a.topk); touch(a.swk); touch(a.swv); touch(a.swks); touch(a.swvs);
    touch(a.swa_len); touch(a.swa_rows); touch(a.sm_scale); touch(a.out); touch(a.lse);
    touch(a.n_q); touch(n_tiles_global); touch(a.stage);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int G = a.H / kGroupHeads;
    const int id = blockIdx.x;
    const int round = (id / kXcds) / G;
    const int hg = (id / kXcds) - round * G;
    const int64_t bq = (int64_t)round * kXcds + (id % kXcds);
    if (bq >= a.n_q) return;  // uniform over the workgroup
    const int64_t b = bq / a.Q;
    // the decode window length is loaded first: loads complete in issue
    // order, so one issued after the tiles would hold back the q set-up
    int sl = 0;
    if (a.swa_len != nullptr) sl = a.swa_len[b];

    SeqView s;
    s.kvc = a.kvc + b * a.cap * 128;
    s.kvs = a.kvs + b * a.cap * 16;
    s.idx = a.idx + bq * a.topk;
    // in a gathering launch the head groups' workgroups share the stage writes
    s.stage = STAGE != 0 ? a.stage + bq * n_tiles_global * kStageTileBytes : nullptr;
    s.stage_rem = hg;
    s.stage_mod = G;
    s.cap = a.cap;
    s.topk = a.topk;
    s.n_tiles_global = n_tiles_global;
    int64_t w0;
    if (a.swa_len != nullptr) {
        // decode: the sequence's window rows; how many count is read below
        w0 = b * a.swa_rows;
        s.win_rows = a.swa_rows;
    } else {
        // chunk query i sees the window tokens [max(0, i - 127), i]
        const int i = (int)(bq % a.Q);
        const int start = i + 1 > kMaxWindow ? i + 1 - kMaxWindow : 0;
        w0 = b * a.swa_rows + start;
        s.win_rows = i + 1 - start;
    }
    s.swk = a.swk + w0 * kHeadDim;
    s.swv = a.swv + w0 * kHeadDim;
    s.swks = a.swks + w0;
    s.swvs = a.swvs + w0;

    // The wave's tiles: selected-record tiles wave, wave + W, ... (two in
    // flight), and at most one window tile: window tile j is the
    // (n_tiles_global + j)-th tile of the query, dealt round robin like the
    // others.  Every load the wave's first tiles need is issued before
    // anything waits, and the window tile, whose rows do not wait for the
    // positions, is attended first, while the selected records are on their
    // way.  Narrow workgroups run three to a CU, so a wave has 168 registers:
    // it reads its q operands from LDS at each tile.
    constexpr bool kLean = kWaves == kWavesNarrow;
    const int n_win_max = (s.win_rows + kTile - 1) / kTile;
    const int jw = ((wave - n_tiles_global) % kWaves + kWaves) % kWaves;
    const bool has_win = jw < n_win_max;
    const int t0 = wave, t1 = wave + kWaves;
    GTile ra, rb;
    WTile rw;
    // positions of the wave's tiles: tile wave + kW in lanes 32 (k & 1) ..
    // + 31 of register k / 2 (-1: absent; unused by a stage-reading launch).
    // Every lane loads (a slot past top-K reads a valid word and takes -1),
    // so the waits count exactly the loads issued after these.
    int32_t P[kPosRegs] = {};
    if (STAGE != kStageRead) {
        const int32_t* any = s.topk > 0 ? s.idx : reinterpret_cast<const int32_t*>(a.q);
#pragma unroll
        for (int k = 0; k < kPosRegs; ++k) {
            const int slot = (wave + kWaves * (2 * k + (lane >> 5))) * kTile + (lane & 31);
            P[k] = *(slot < s.topk ? s.idx + slot : any);
        }
    }
    // this wave's share of q: heads wave * HPW .. + HPW, 4 channels per lane
    // and load (lane: head + (lane >> 5), channels 4 (lane & 31) .. + 4)
    constexpr int kHPW = kGroupHeads / kWaves;
    float4 xq[kHPW / 2];
#pragma unroll
    for (int i = 0; i < kHPW / 2; ++i)
        xq[i] = reinterpret_cast<const float4*>(
            a.q + (bq * a.H + hg * kGroupHeads + wave * kHPW + 2 * i + (lane >> 5)) * kHeadDim)[lane & 31];
    // Loads complete in issue order: q, then the window tile, then the
    // selected-record tiles, in the order the wave consumes them.  They are
    // issued unconditionally, so that each wait counts exactly the loads
    // behind it: a wave without a window tile reads rows clamped to the
    // window's first row, and one past the last selected tile reads stage
    // tile 0 (a staging launch always has one) or, through positions of -1,
    // cache row 0; neither tile is processed.
    fetch_window(s, jw, lane, rw);
    if (STAGE != kStageRead) {
        // the q and window loads stay ahead of the wait for the positions
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kPosRegs; ++k) {
            const int slot = (wave + kWaves * (2 * k + (lane >> 5))) * kTile + (lane & 31);
            P[k] = (slot < s.topk && P[k] >= 0 && P[k] < s.cap) ? P[k] : -1;
        }
    }
    fetch_global<STAGE>(s, t0 < n_tiles_global ? t0 : 0, P[0], 0, lane, ra);
    fetch_global<STAGE>(s, t1 < n_tiles_global ? t1 : 0, P[0], 1, lane, rb);
    s.swa_len = a.swa_len != nullptr ? (sl < 0 ? 0 : (sl > a.swa_rows ? a.swa_rows : sl))
                                     : s.win_rows;
    // the position register of the wave's k-th selected tile, loaded now when
    // it is past the preloaded ones
    auto tile_pos = [&](int k) -> int32_t {
        if (k < 2 * kPosRegs) return P[k >> 1];
        const int t = wave + kWaves * k;
        const int slot = t * kTile + (lane & 31);
        int32_t p = slot < s.topk ? s.idx[slot] : -1;
        return (p >= 0 && p < s.cap) ? p : -1;
    };

    // q * sm_scale * log2(e), scaled per head by a power of two into
    // [2^14, 2^15), as fp16 hi + lo rows in LDS; then every wave reads its
    // B operands: head c, MFMA step ks takes channels 32g + 8ks .. +8
    _Float16* q_hi = reinterpret_cast<_Float16*>(smem + kWaves * kWaveBytes);
    _Float16* q_lo = q_hi + kGroupHeads * kQPitch;
    float* q_mul = reinterpret_cast<float*>(q_lo + kGroupHeads * kQPitch);
    {
        const float logit_mul = a.sm_scale * kLog2e;
#pragma unroll
        for (int i = 0; i < kHPW / 2; ++i) {
            const float x[4] = {xq[i].x * logit_mul, xq[i].y * logit_mul, xq[i].z * logit_mul,
                                xq[i].w * logit_mul};
            float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
            amax = half_wave_max(amax);
            int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 0;  // amax in [2^(e-1), 2^e)
            e = e < -100 ? -100 : (e > 100 ? 100 : e);
            const int head = wave * kHPW + 2 * i + (lane >> 5);
            half4_t hv, lv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = __builtin_amdgcn_ldexpf(x[j], 15 - e);
                hv[j] = (_Float16)v;
                lv[j] = (_Float16)(v - (float)hv[j]);
            }
            *reinterpret_cast<half4_t*>(q_hi + head * kQPitch + 4 * (lane & 31)) = hv;
            *reinterpret_cast<half4_t*>(q_lo + head * kQPitch + 4 * (lane & 31)) = lv;
            if ((lane & 31) == 0) q_mul[head] = __builtin_amdgcn_ldexpf(1.0f, e - 15);
        }
    }
    __syncthreads();
    typename std::conditional<kLean, QLds, QRegs>::type qo;
    if constexpr (kLean) {
        qo.h = q_hi + c * kQPitch + 32 * g;
        qo.l = q_lo + c * kQPitch + 32 * g;
    } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            qo.h[ks] = *reinterpret_cast<const half8_t*>(q_hi + c * kQPitch + 32 * g + 8 * ks);
            qo.l[ks] = *reinterpret_cast<const half8_t*>(q_lo + c * kQPitch + 32 * g + 8 * ks);
        }
    }
    const float qmul = q_mul[c];

    WaveState st;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    st.lsum = float4_t{0.f, 0.f, 0.f, 0.f};
    st.lwin = 0.0f;
    st.m = -INFINITY;
    _Float16* vtile = reinterpret_cast<_Float16*>(smem + wave * kWaveBytes);

    if (has_win && jw * kTile < s.swa_len)
        process_window(rw, s.swa_len - jw * kTile, qo, qmul, vtile, lane, st);
    int k = 0;  // index of tile t among the wave's selected-record tiles
    for (int t = t0; t < n_tiles_global; t += 2 * kWaves, k += 2) {
        process_global<STAGE>(s, t, ra, qo, qmul, vtile, lane, st);
        if (t + 2 * kWaves < n_tiles_global)
            fetch_global<STAGE>(s, t + 2 * kWaves, tile_pos(k + 2), (k + 2) & 1, lane, ra);
        const int u = t + kWaves;
        if (u < n_tiles_global) {
            process_global<STAGE>(s, u, rb, qo, qmul, vtile, lane, st);
            if (u + 2 * kWaves < n_tiles_global)
                fetch_global<STAGE>(s, u + 2 * kWaves, tile_pos(k + 3), (k + 3) & 1, lane, rb);
        }
    }

    // ---- merge the waves' states through LDS: each wave's rows, max and
    // sum in its own tile area (m_rows(w)), which only it has used so far ----
    const float l_wave = st.lsum[0] + xsum4(st.lwin);
    auto m_rows = [&](int w) { return reinterpret_cast<float*>(smem + w * kWaveBytes); };
    constexpr int kMaxOff = kGroupHeads * kMergePitch, kSumOff = kMaxOff + kGroupHeads;
    {
        float* orow = m_rows(wave) + c * kMergePitch + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            *reinterpret_cast<float4*>(orow + 16 * dt) =
                make_float4(st.o[dt][0], st.o[dt][1], st.o[dt][2], st.o[dt][3]);
        if (g == 0) {
            m_rows(wave)[kMaxOff + c] = st.m;
            m_rows(wave)[kSumOff + c] = l_wave;
        }
    }
    __syncthreads();
    for (int item = tid; item < kGroupHeads * (kHeadDim / 4); item += kThreads) {
        const int hh = item / (kHeadDim / 4), d4 = item % (kHeadDim / 4);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_rows(w)[kMaxOff + hh]);
        float L = 0.0f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float mw = m_rows(w)[kMaxOff + hh];
                const float wt = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
                L += wt * m_rows(w)[kSumOff + hh];
                const float4 ow = *reinterpret_cast<const float4*>(m_rows(w) + hh * kMergePitch + 4 * d4);
                acc.x += wt * ow.x;
                acc.y += wt * ow.y;
                acc.z += wt * ow.z;
                acc.w += wt * ow.w;
            }
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        const int64_t oh = bq * a.H + hg * kGroupHeads + hh;
        *reinterpret_cast<float4*>(a.out + oh * kHeadDim + 4 * d4) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
        if (d4 == 0) a.lse[oh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// Large launches with H a multiple of 32: one workgroup of 4 waves per (query,
// group of 32 heads), two 16-head MFMA column blocks per wave, so each tile of
// records is dequantised once for 32 heads (the 16-head workgroups above
// dequantise it once per 16 heads).  Two workgroups per CU (54.4 KB of LDS,
// up to 256 registers per wave).  The lane layouts, q scaling, softmax and
// window handling of k_attn; the window tile first; the merge in two rounds
// of one column block through each wave's own tile area.
// ---------------------------------------------------------------------------
constexpr int kPairCB = 2;                         // 16-head column blocks per wave
constexpr int kPairHeads = kPairCB * kGroupHeads;  // 32
constexpr int kPairWaves = 4;
constexpr int kPairQBytes = 2 * kPairHeads * kQPitch * 2 + kPairHeads * 4;
constexpr int kPairLds = kPairWaves * kWaveBytes + kPairQBytes;
static_assert(2 * kPairLds <= 160 * 1024, "two pair workgroups per CU");

struct PairState {
    float4_t o[kPairCB][8];
    float4_t lsum[kPairCB];
    float lwin[kPairCB];
    float m[kPairCB];
};

__device__ __forceinline__ void pair_rescale(float tmax, PairState& st, int cb) {
    const bool move = tmax > st.m[cb] + kRescaleSlack || (st.m[cb] == -INFINITY && tmax != -INFINITY);
    if (__builtin_amdgcn_ballot_w64(move)) {
        const float m_new = move ? tmax : st.m[cb];
        if (__builtin_amdgcn_ballot_w64(st.m[cb] != -INFINITY)) {  // as in online_rescale
            const float alpha = (st.m[cb] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(st.m[cb] - m_new);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) st.o[cb][dt] *= alpha;
            st.lsum[cb] *= alpha;
            st.lwin[cb] *= alpha;
        }
        st.m[cb] = m_new;
    }
}

// S^T = K Q^T of both column blocks, channel step ks outer: the MFMAs of one
// step for every (column block, row block) pair are issued before the next
// step, four independent accumulations; q is read from the workgroup's LDS
// rows (head cb*16 + c, channels 32g + 8ks .. +8).
__device__ __forceinline__ void pair_scores(const half8_t (&ka)[2][4], const _Float16* q_hi,
                                            const _Float16* q_lo, int c, int g,
                                            float4_t (&sacc)[kPairCB][2]) {
#pragma unroll
    for (int cb = 0; cb < kPairCB; ++cb)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) sacc[cb][blk] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int cb = 0; cb < kPairCB; ++cb) {
            const int off = (cb * kGroupHeads + c) * kQPitch + 32 * g + 8 * ks;
            const half8_t qh = *reinterpret_cast<const half8_t*>(q_hi + off);
            const half8_t ql = *reinterpret_cast<const half8_t*>(q_lo + off);
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
                sacc[cb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[blk][ks], qh, sacc[cb][blk], 0, 0, 0);
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
                sacc[cb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[blk][ks], ql, sacc[cb][blk], 0, 0, 0);
        }
    }
}

__device__ __forceinline__ void pair_global(const GTile& r, const _Float16* q_hi,
                                            const _Float16* q_lo, const float (&qmul)[kPairCB],
                                            _Float16* __restrict__ vtile, int lane, PairState& st) {
    const int c = lane & 15, g = lane >> 4;
    const uint32_t valid = __builtin_amdgcn_readfirstlane(r.valid);
    if (valid == 0u) return;
    {
        const int q4 = lane & 3;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            half8_t* dst = reinterpret_cast<half8_t*>(vtile + (16 * j + (lane >> 2)) * kVPitch + 32 * q4);
            const half2_t sv = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.vs >> (16 * j), 1.0f, false);
            dst[0] = fp4x8_h8<0>(r.v[j][0], sv);
            dst[1] = fp4x8_h8<0>(r.v[j][1], sv);
            dst[2] = fp4x8_h8<1>(r.v[j][2], sv);
            dst[3] = fp4x8_h8<1>(r.v[j][3], sv);
        }
    }
    half8_t ka[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const half2_t sk = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.ks >> (16 * blk), 1.0f, false);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            ka[blk][ks] = ks < 2 ? fp4x8_h8<0>(r.k[blk][ks], sk) : fp4x8_h8<1>(r.k[blk][ks], sk);
    }
    const uint32_t vb = ((valid >> (4 * g)) & 0xFu) | (((valid >> (16 + 4 * g)) & 0xFu) << 4);
    // S for every column block at once, channel steps outer: eight
    // independent accumulation chains keep the MFMA pipe busy
    float4_t sacc[kPairCB][2];
    pair_scores(ka, q_hi, q_lo, c, g, sacc);
    half8_t pb[kPairCB];
#pragma unroll
    for (int cb = 0; cb < kPairCB; ++cb) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = sacc[cb][i >> 2][i & 3];
        if (valid != 0xFFFFFFFFu) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = (vb >> i) & 1u ? x[i] : -INFINITY;
        }
        float tmax = vmax(vmax(vmax(x[0], x[1]), vmax(x[2], x[3])),
                          vmax(vmax(x[4], x[5]), vmax(x[6], x[7])));
        tmax = xmax4(tmax) * qmul[cb];
        pair_rescale(tmax, st, cb);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            pb[cb][i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(x[i], qmul[cb], -st.m[cb]));
    }
    wave_lds_sync();
    const half8_t ones = {1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const half8_t va = v_operand(vtile, lane, dt);
#pragma unroll
        for (int cb = 0; cb < kPairCB; ++cb)
            st.o[cb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[cb], st.o[cb][dt], 0, 0, 0);
    }
#pragma unroll
    for (int cb = 0; cb < kPairCB; ++cb)
        st.lsum[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[cb], st.lsum[cb], 0, 0, 0);
    wave_lds_sync();
}

__device__ __forceinline__ void pair_window(const WTile& r, int n, const _Float16* q_hi,
                                            const _Float16* q_lo, const float (&qmul)[kPairCB],
                                            _Float16* __restrict__ vtile, int lane, PairState& st) {
    const int c = lane & 15, g = lane >> 4;
    const uint32_t valid = n >= kTile ? 0xFFFFFFFFu : ((1u << n) - 1u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        half8_t* dst = reinterpret_cast<half8_t*>(vtile + (8 * j + (lane >> 3)) * kVPitch + 16 * (lane & 7));
        dst[0] = fp8x8_h8(r.v[j][0], r.v[j][1]);
        dst[1] = fp8x8_h8(r.v[j][2], r.v[j][3]);
    }
    half8_t ka[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            ka[blk][ks] = fp8x8_h8(r.k[blk][ks >> 1][2 * (ks & 1)], r.k[blk][ks >> 1][2 * (ks & 1) + 1]);
    float ksc[8], vsc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = c_entry(i, g);
        ksc[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(e << 2, __float_as_int(r.sc)));
        vsc[i] = __int_as_float(__builtin_amdgcn_ds_bpermute((32 + e) << 2, __float_as_int(r.sc)));
    }
    const uint32_t vb = ((valid >> (4 * g)) & 0xFu) | (((valid >> (16 + 4 * g)) & 0xFu) << 4);
    float4_t sacc[kPairCB][2];
    pair_scores(ka, q_hi, q_lo, c, g, sacc);
    half8_t pb[kPairCB];
    float down[kPairCB];
#pragma unroll
    for (int cb = 0; cb < kPairCB; ++cb) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = sacc[cb][i >> 2][i & 3] * qmul[cb] * ksc[i];
        if (valid != 0xFFFFFFFFu) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = (vb >> i) & 1u ? x[i] : -INFINITY;
        }
        float tmax = vmax(vmax(vmax(x[0], x[1]), vmax(x[2], x[3])),
                          vmax(vmax(x[4], x[5]), vmax(x[6], x[7])));
        tmax = xmax4(tmax);
        pair_rescale(tmax, st, cb);
        float w[8], wmax = 0.0f, psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(x[i] - st.m[cb]);
            psum += p;
            w[i] = p * vsc[i];
            wmax = vmax(wmax, w[i]);
        }
        st.lwin[cb] += psum;
        wmax = xmax4(wmax);
        int e = wmax > 0.0f ? __builtin_amdgcn_frexp_expf(wmax) : 0;
        e = e < -100 ? -100 : (e > 120 ? 120 : e);
        const float up = __builtin_amdgcn_ldexpf(1.0f, 8 - e);
        down[cb] = __builtin_amdgcn_ldexpf(1.0f, e - 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[cb][i] = (_Float16)(w[i] * up);
    }
    wave_lds_sync();
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const half8_t va = v_operand(vtile, lane, dt);
#pragma unroll
        for (int cb = 0; cb < kPairCB; ++cb) {
            const float4_t zero = {0.f, 0.f, 0.f, 0.f};
            const float4_t pv = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[cb], zero, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) st.o[cb][dt][i] = fmaf(pv[i], down[cb], st.o[cb][dt][i]);
        }
    }
    wave_lds_sync();
}

// grid = ceil(n_q / 8) * 8 * (H / 32) workgroups of 4 waves; the head groups
// of one query share an XCD, as in k_attn.
__global__ __launch_bounds__(kPairWaves * 64, 2) void k_attn_pair(AttnArgs a, int n_tiles_global) {
    constexpr int kWaves = kPairWaves, kThreads = kWaves * 64;
    __shared__ __attribute__((aligned(16))) unsigned char smem[kPairLds];
    touch(a.q); touch(a.H); touch(a.Q); touch(a.kvc); touch(a.kvs); touch(a.cap);
    touch(a.idx); touch(a.topk); touch(a.swk); touch(a.swv); touch(a.swks); touch(a.swvs);
    touch(a.swa_len); touch(a.swa_rows); touch(a.sm_scale); touch(a.out); touch(a.lse);
    touch(a.n_q); touch(n_tiles_global);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int G = a.H / kPairHeads;
    const int id = blockIdx.x;
    const int round = (id / kXcds) / G;
    const int hg = (id / kXcds) - round * G;
    const int64_t bq = (int64_t)round * kXcds + (id % kXcds);
    if (bq >= a.n_q) return;  // uniform over the workgroup
    const int64_t b = bq / a.Q;
    // the decode window length is loaded first: loads complete in issue
    // order, so one issued after the tiles would hold back the q set-up
    int sl = 0;
    if (a.swa_len != nullptr) sl = a.swa_len[b];

    SeqView s;
    s.kvc = a.kvc + b * a.cap * 128;
    s.kvs = a.kvs + b * a.cap * 16;
    s.idx = a.idx + bq * a.topk;
    s.stage = nullptr;
    s.stage_rem = 0;
    s.stage_mod = 1;
    s.cap = a.cap;
    s.topk = a.topk;
    s.n_tiles_global = n_tiles_global;
    int64_t w0;
    if (a.swa_len != nullptr) {
        w0 = b * a.swa_rows;
        s.win_rows = a.swa_rows;
    } else {
        const int i = (int)(bq % a.Q);
        const int start = i + 1 > kMaxWindow ? i + 1 - kMaxWindow : 0;
        w0 = b * a.swa_rows + start;
        s.win_rows = i + 1 - start;
    }
    s.swk = a.swk + w0 * kHeadDim;
    s.swv = a.swv + w0 * kHeadDim;
    s.swks = a.swks + w0;
    s.swvs = a.swvs + w0;

    const int n_win_max = (s.win_rows + kTile - 1) / kTile;
    const int jw = ((wave - n_tiles_global) % kWaves + kWaves) % kWaves;
    const int t0 = wave, t1 = wave + kWaves;
    GTile ra, rb;
    WTile rw;
    // positions loaded by every lane, range-checked after the q and window
    // loads are issued, as in k_attn
    int32_t P[kPosRegs];
    const int32_t* any = s.topk > 0 ? s.idx : reinterpret_cast<const int32_t*>(a.q);
#pragma unroll
    for (int k = 0; k < kPosRegs; ++k) {
        const int slot = (wave + kWaves * (2 * k + (lane >> 5))) * kTile + (lane & 31);
        P[k] = *(slot < s.topk ? s.idx + slot : any);
    }
    // this wave's share of q: 8 heads, 32 channels per lane and head pair
    constexpr int kHPW = kPairHeads / kWaves;
    float4 xq[kHPW / 2];
#pragma unroll
    for (int i = 0; i < kHPW / 2; ++i)
        xq[i] = reinterpret_cast<const float4*>(
            a.q + (bq * a.H + hg * kPairHeads + wave * kHPW + 2 * i + (lane >> 5)) * kHeadDim)[lane & 31];
    // at most one window tile a wave (at most 128 window rows, 4 waves)
    const bool has_win = jw < n_win_max;
    // issued unconditionally, as in k_attn (absent tiles read valid rows)
    fetch_window(s, jw, lane, rw);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kPosRegs; ++k) {
        const int slot = (wave + kWaves * (2 * k + (lane >> 5))) * kTile + (lane & 31);
        P[k] = (slot < s.topk && P[k] >= 0 && P[k] < s.cap) ? P[k] : -1;
    }
    fetch_global<0>(s, t0, P[0], 0, lane, ra);
    fetch_global<0>(s, t1, P[0], 1, lane, rb);
    s.swa_len = a.swa_len != nullptr ? (sl < 0 ? 0 : (sl > a.swa_rows ? a.swa_rows : sl))
                                     : s.win_rows;
    auto tile_pos = [&](int k) -> int32_t {
        if (k < 2 * kPosRegs) return P[k >> 1];
        const int t = wave + kWaves * k;
        const int slot = t * kTile + (lane & 31);
        int32_t p = slot < s.topk ? s.idx[slot] : -1;
        return (p >= 0 && p < s.cap) ? p : -1;
    };

    _Float16* q_hi = reinterpret_cast<_Float16*>(smem + kWaves * kWaveBytes);
    _Float16* q_lo = q_hi + kPairHeads * kQPitch;
    float* q_mul = reinterpret_cast<float*>(q_lo + kPairHeads * kQPitch);
    {
        const float logit_mul = a.sm_scale * kLog2e;
#pragma unroll
        for (int i = 0; i < kHPW / 2; ++i) {
            const float x[4] = {xq[i].x * logit_mul, xq[i].y * logit_mul, xq[i].z * logit_mul,
                                xq[i].w * logit_mul};
            float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
            amax = half_wave_max(amax);
            int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 0;
            e = e < -100 ? -100 : (e > 100 ? 100 : e);
            const int head = wave * kHPW + 2 * i + (lane >> 5);
            half4_t hv, lv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = __builtin_amdgcn_ldexpf(x[j], 15 - e);
                hv[j] = (_Float16)v;
                lv[j] = (_Float16)(v - (float)hv[j]);
            }
            *reinterpret_cast<half4_t*>(q_hi + head * kQPitch + 4 * (lane & 31)) = hv;
            *reinterpret_cast<half4_t*>(q_lo + head * kQPitch + 4 * (lane & 31)) = lv;
            if ((lane & 31) == 0) q_mul[head] = __builtin_amdgcn_ldexpf(1.0f, e - 15);
        }
    }
    __syncthreads();
    float qmul[kPairCB];
#pragma unroll
    for (int cb = 0; cb < kPairCB; ++cb) qmul[cb] = q_mul[cb * kGroupHeads + c];

    PairState st;
#pragma unroll
    for (int cb = 0; cb < kPairCB; ++cb) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.o[cb][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
        st.lsum[cb] = float4_t{0.f, 0.f, 0.f, 0.f};
        st.lwin[cb] = 0.0f;
        st.m[cb] = -INFINITY;
    }
    _Float16* vtile = reinterpret_cast<_Float16*>(smem + wave * kWaveBytes);

    // the window tile first: its rows do not wait for the positions
    if (has_win && jw * kTile < s.swa_len)
        pair_window(rw, s.swa_len - jw * kTile, q_hi, q_lo, qmul, vtile, lane, st);
    int k = 0;
    for (int t = t0; t < n_tiles_global; t += 2 * kWaves, k += 2) {
        pair_global(ra, q_hi, q_lo, qmul, vtile, lane, st);
        if (t + 2 * kWaves < n_tiles_global)
            fetch_global<0>(s, t + 2 * kWaves, tile_pos(k + 2), (k + 2) & 1, lane, ra);
        const int u = t + kWaves;
        if (u < n_tiles_global) {
            pair_global(rb, q_hi, q_lo, qmul, vtile, lane, st);
            if (u + 2 * kWaves < n_tiles_global)
                fetch_global<0>(s, u + 2 * kWaves, tile_pos(k + 3), (k + 3) & 1, lane, rb);
        }
    }

    // ---- merge, one column block per round, each wave's rows, max and sum
    // in its own tile area (m_rows(w)); the first round's writes need no
    // barrier, since only this wave has used its area ----
    float lw[kPairCB];
#pragma unroll
    for (int cb = 0; cb < kPairCB; ++cb) lw[cb] = st.lsum[cb][0] + xsum4(st.lwin[cb]);
    auto m_rows = [&](int w) { return reinterpret_cast<float*>(smem + w * kWaveBytes); };
    constexpr int kMaxOff = kGroupHeads * kMergePitch, kSumOff = kMaxOff + kGroupHeads;
#pragma unroll
    for (int cb = 0; cb < kPairCB; ++cb) {
        if (cb > 0) __syncthreads();  // the previous round's readers are done
        {
            float* orow = m_rows(wave) + c * kMergePitch + 4 * g;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                *reinterpret_cast<float4*>(orow + 16 * dt) =
                    make_float4(st.o[cb][dt][0], st.o[cb][dt][1], st.o[cb][dt][2], st.o[cb][dt][3]);
            if (g == 0) {
                m_rows(wave)[kMaxOff + c] = st.m[cb];
                m_rows(wave)[kSumOff + c] = lw[cb];
            }
        }
        __syncthreads();
        for (int item = tid; item < kGroupHeads * (kHeadDim / 4); item += kThreads) {
            const int hh = item / (kHeadDim / 4), d4 = item % (kHeadDim / 4);
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_rows(w)[kMaxOff + hh]);
            float L = 0.0f;
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            if (M != -INFINITY) {
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    const float mw = m_rows(w)[kMaxOff + hh];
                    const float wt = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
                    L += wt * m_rows(w)[kSumOff + hh];
                    const float4 ow = *reinterpret_cast<const float4*>(m_rows(w) + hh * kMergePitch + 4 * d4);
                    acc.x += wt * ow.x;
                    acc.y += wt * ow.y;
                    acc.z += wt * ow.z;
                    acc.w += wt * ow.w;
                }
            }
            const float inv = L > 0.0f ? 1.0f / L : 0.0f;
            const int64_t oh = bq * a.H + hg * kPairHeads + cb * kGroupHeads + hh;
            *reinterpret_cast<float4*>(a.out + oh * kHeadDim + 4 * d4) =
                make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
            if (d4 == 0) a.lse[oh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
        }
    }
}

hipError_t launch_attn(const AttnArgs& a, void* /*ws*/, size_t /*ws_bytes*/, hipStream_t stream,
                       hipEvent_t start, hipEvent_t stop) {
    if (a.n_q <= 0) return hipSuccess;
    // decode: the window length is clamped to swa_rows, so at most 128 rows;
    // chunk: swa_rows is the chunk length, each query reads at most 128 rows
    if (a.topk > kMaxTopk || (a.swa_len != nullptr && a.swa_rows > kMaxWindow) ||
        a.H % kGroupHeads != 0)
        return hipErrorInvalidValue;
    const int n_tiles_global = (a.topk + kTile - 1) / kTile;
    const int G = a.H / kGroupHeads;
    const int64_t rounds = (a.n_q + kXcds - 1) / kXcds;
    const unsigned grid = (unsigned)(rounds * kXcds * G);
    if (a.stage_mode != 0 && (a.stage == nullptr || a.Q != 1)) return hipErrorInvalidValue;
    // enough (query, 16-head group) pairs to fill the chip twice and H a
    // multiple of 32: workgroups of 32 heads, each tile dequantised once for
    // all of them
    if (a.stage_mode == 0 && a.H % kPairHeads == 0 && (int64_t)grid >= 2 * kCusPerChip) {
        const unsigned pgrid = (unsigned)(rounds * kXcds * (a.H / kPairHeads));
        if (start != nullptr && stop != nullptr)
            hipExtLaunchKernelGGL(k_attn_pair, dim3(pgrid), dim3(kPairWaves * 64), 0, stream, start,
                                  stop, 0, a, n_tiles_global);
        else
            hipLaunchKernelGGL(k_attn_pair, dim3(pgrid), dim3(kPairWaves * 64), 0, stream, a,
                               n_tiles_global);
        return hipGetLastError();
    }
    // narrow workgroups once two rounds of wide ones would be needed
    const bool narrow = a.stage_mode == 0 && (int64_t)grid >= 2 * kCusPerChip;
    void (*kern)(AttnArgs, int) = a.stage_mode == kStageWrite  ? k_attn<kStageWrite, kWavesWide>
                                  : a.stage_mode == kStageRead ? k_attn<kStageRead, kWavesWide>
                                  : narrow                     ? k_attn<0, kWavesNarrow>
                                                               : k_attn<0, kWavesWide>;
    const dim3 block((narrow ? kWavesNarrow : kWavesWide) * 64);
    if (start != nullptr && stop != nullptr) {
        // the runtime records `start` / `stop` immediately around this dispatch
        hipExtLaunchKernelGGL(kern, dim3(grid), block, 0, stream, start, stop, 0, a,
                              n_tiles_global);
    } else {
        hipLaunchKernelGGL(kern, dim3(grid), block, 0, stream, a, n_tiles_global);
    }
    return hipGetLastError();
}

}  // namespace csa2
