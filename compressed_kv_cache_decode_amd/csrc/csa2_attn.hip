// csa2_attn.hip -- CSA2 sparse attention over the FP4 global KV plus the FP8
// sliding window.
//
// "DeepSeek V4.1 Flash: architecture study notes", section 2: each query
// attends to at most 512 selected global records together with its local
// window; section 1: the window is 128 tokens and every layer keeps its own;
// section 4: the FP4 cache is dequantised on read and fed to ordinary
// attention (the saving is storage, not FP4 arithmetic); the SWA KV stays FP8.
//
// Design (gfx950).  The entry list of a query (selected records, then window
// tokens) is cut into tiles of 32 entries.  One workgroup of 8 waves serves
// one (query, group of 16 heads); wave w takes tiles w, w + 8, w + 16, ... and
// keeps its own online softmax; the 8 partial states are merged through LDS at
// the end, so one launch produces the output (no partials in HBM, no second
// kernel).  All heads share one KV head (MQA), so per tile the logits are a
// dense [16 heads x 32 entries] contraction on MFMA (v_mfma_f32_16x16x32_f16):
//   - S^T = K Q^T: the K operand is dequantised straight from the gathered
//     bytes into registers.  Lane (entry e, quarter g) loads channels
//     [32g, 32g + 32) of its record, and MFMA step ks consumes channels
//     32g + 8ks .. +8 from that lane group; q is laid out with the same
//     channel permutation, which leaves the dot products unchanged.
//   - O^T += V^T P^T: P comes straight from the S^T registers (each lane holds
//     entries 4g..4g+3 and 16+4g..16+4g+3 of its head); V is dequantised by the
//     lanes that own those entries and transposed through a wave-private LDS
//     tile, so no workgroup barrier sits inside the tile loop.
//   - dequantised E2M1 x E4M3 values have at most 6 significant bits and lie
//     in [2^-10, 2688], so they are exact in fp16; E4M3 window codes are exact
//     in fp16 and their fp32 row scale is applied to the logit (K) or to the
//     probability (V) in fp32;
//   - q is split into fp16 hi + lo parts, so q.k carries ~22 bits;
//   - accumulation is fp32, softmax is online in fp32 (base-2 exponentials).
// Memory instructions, not bytes, bound a gather this small: every vector load
// costs the address unit about the same time whatever its width.  So the
// workgroup reads q, the top-K row and the window scales once into LDS, and
// each wave gathers a tile's rows with 16-byte loads only: the K operand
// directly, the V codes and the scale bytes through a wave-private LDS stage
// from which the lanes pick their operand bytes.  Each wave keeps two tiles'
// bytes in flight.  Workgroups are numbered so that the head groups of one
// query land on the same XCD (consecutive workgroup ids go round-robin over
// the 8 XCDs), sharing its L2 for the gathered rows.
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
// workgroups for two of them to share each CU (its LDS holds two 4-wave
// workgroups, not two 8-wave ones), so that they all run in one round
constexpr int kWavesWide = 8, kWavesNarrow = 4;
constexpr int kGroupHeads = 16;     // heads per workgroup (one MFMA column block)
constexpr int kVPitch = 144;        // fp16 per V row in LDS (128 + 16)
constexpr int kMergePitch = kHeadDim + 4;  // fp32 per merged output row in LDS
constexpr int kXcds = 8;
constexpr int kCusPerChip = 256;
constexpr int kMaxWindow = 128;     // window tokens a query attends to
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag the true max
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS map (bytes)
constexpr int kWaveBytes = kTile * kVPitch * 2;              // one wave's V tile
constexpr int kOffQ = 0;                                     // q [16][128] fp32
constexpr int kOffWin = kOffQ + kGroupHeads * kHeadDim * 4;  // window K scales [128], V scales [128]
constexpr int kOffWave = kOffWin + 2 * kMaxWindow * 4;       // per-wave V tiles
constexpr int lds_bytes(int W) { return kOffWave + W * kWaveBytes; }
constexpr int merge_bytes(int W) {
    return (W * kGroupHeads * kMergePitch + 2 * W * kGroupHeads) * 4;
}
static_assert(merge_bytes(kWavesWide) <= kWavesWide * kWaveBytes, "merge area aliases the wave areas");
static_assert(merge_bytes(kWavesNarrow) <= kWavesNarrow * kWaveBytes, "merge area aliases the wave areas");
static_assert(lds_bytes(kWavesWide) <= 160 * 1024, "LDS");
static_assert(2 * lds_bytes(kWavesNarrow) <= 160 * 1024, "two narrow workgroups per CU");

size_t attn_workspace_bytes(int64_t, int, int, int) { return 0; }

// What one workgroup needs to locate its entries.
struct SeqView {
    const uint8_t* kvc;
    const uint8_t* kvs;
    const uint8_t* swk;
    const uint8_t* swv;
    const int32_t* idx;    // this query's top-K row
    uint8_t* stage;        // this query's staged tiles (stage mode), or null
    int stage_rem, stage_mod;  // a writing workgroup writes the tiles t with t % mod == rem
    int64_t cap;
    int64_t b;
    int topk;
    int swa_rows;
    int swa_start;  // first window row of this query (chunk: the last 128 tokens up to it)
    int swa_len;
    int n_tiles_global;
};

// Position of entry lane % 32 of global tile t, or -1 when absent (slot past
// topk, or a position outside [0, cap)); lanes 32..63 repeat lanes 0..31.
__device__ __forceinline__ int32_t tile_position(const SeqView& s, int t, int lane) {
    const int slot = t * kTile + (lane & (kTile - 1));
    const int32_t p = slot < s.topk ? s.idx[slot] : -1;
    return (p >= 0 && p < s.cap) ? p : -1;
}

// position of entry e of the tile, from the lane that loaded it (or -1)
__device__ __forceinline__ int32_t entry_position(int32_t pos, int e) {
    return __builtin_amdgcn_ds_bpermute(e << 2, pos);
}

// window row of token e of window tile t, or -1
__device__ __forceinline__ int64_t window_row(const SeqView& s, int t, int e) {
    const int tok = (t - s.n_tiles_global) * kTile + e;
    return tok < s.swa_len ? s.b * s.swa_rows + s.swa_start + tok : -1;
}

// Raw bytes of one tile held by one lane (c = lane & 15, g = lane >> 4).
// Absent rows load nothing and read as zero.
//   k[blk]  K operand of entry 16 blk + c, channels [32g, 32g + 32):
//           global 16 B of E2M1 codes (k[blk][0]); window 32 B of E4M3 (k[blk][0..1])
//   v       V codes, whole 64-byte sectors per group of lanes: global v[j] = channels
//           [32q, 32q + 32) of entry 16j + lane/4 (q = lane & 3); window v[j] =
//           channels [16q8, 16q8 + 16) of token 8j + lane/8 (q8 = lane & 7)
//   sc      global, lanes 0..31: the 16 scale bytes (K 0..7, V 8..15) of entry `lane`
//   valid   bit e: entry e of the tile is present (same in every lane)
struct TileRegs {
    u32x4_t k[2][2];
    u32x4_t v[4];
    u32x4_t sc;
    uint32_t valid;
};

__device__ __forceinline__ u32x4_t ld16(const uint8_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}

// Issue the loads of tile t.  pos: tile_position(s, t, lane) for a global
// tile (unused for a window tile, or when the tile comes from the stage).
template <int STAGE>
__device__ __forceinline__ void fetch_tile(const SeqView& s, int t, int32_t pos, int lane,
                                           TileRegs& r) {
    const int c = lane & 15, g = lane >> 4;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    if (STAGE == kStageRead && t < s.n_tiles_global) {
        // the lanes' bytes as the gathering layer held them: 16 coalesced bytes
        // per lane and register
        const uint8_t* src = s.stage + (int64_t)t * kStageTileBytes + 16 * lane;
        r.k[0][0] = ld16(src);
        r.k[1][0] = ld16(src + 1024);
        r.v[0] = ld16(src + 2048);
        r.v[1] = ld16(src + 3072);
        r.sc = lane < kTile ? ld16(src + 4096) : z;
        r.valid = *reinterpret_cast<const uint32_t*>(s.stage + (int64_t)t * kStageTileBytes + 4608);
        r.k[0][1] = z;
        r.k[1][1] = z;
        r.v[2] = z;
        r.v[3] = z;
    } else if (t < s.n_tiles_global) {
        const int64_t base = s.b * s.cap;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int32_t p = entry_position(pos, 16 * blk + c);
            r.k[blk][0] = p >= 0 ? ld16(s.kvc + (base + (p >= 0 ? p : 0)) * 128 + 16 * g) : z;
            r.k[blk][1] = z;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int32_t p = entry_position(pos, 16 * j + (lane >> 2));
            r.v[j] = p >= 0 ? ld16(s.kvc + (base + (p >= 0 ? p : 0)) * 128 + 64 + 16 * (lane & 3)) : z;
        }
        r.v[2] = z;
        r.v[3] = z;
        const bool has = lane < kTile && pos >= 0;
        r.sc = has ? ld16(s.kvs + (base + (has ? pos : 0)) * 16) : z;
        r.valid = (uint32_t)__builtin_amdgcn_ballot_w64(has);
    } else {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int64_t row = window_row(s, t, 16 * blk + c);
            const uint8_t* src = s.swk + (row >= 0 ? row : 0) * kHeadDim + 32 * g;
            r.k[blk][0] = row >= 0 ? ld16(src) : z;
            r.k[blk][1] = row >= 0 ? ld16(src + 16) : z;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t vrow = window_row(s, t, 8 * j + (lane >> 3));
            r.v[j] = vrow >= 0 ? ld16(s.swv + (vrow >= 0 ? vrow : 0) * kHeadDim + 16 * (lane & 7)) : z;
        }
        r.sc = z;
        const int tok0 = (t - s.n_tiles_global) * kTile;
        const int nv = s.swa_len - tok0;  // >= 1: window tiles end at swa_len
        r.valid = nv >= kTile ? 0xFFFFFFFFu : ((1u << nv) - 1u);
    }
}

// max / sum over the four lanes c, c+16, c+32, c+48 (v_permlane*_swap: each
// call hands every lane its partner's value 32 resp. 16 lanes away)
__device__ __forceinline__ float xmax4(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
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

// Eight E2M1 codes times an fp16 scale, as one MFMA operand.
__device__ __forceinline__ half8_t fp4x8_h8(uint32_t w, _Float16 sc) {
    const half2_t s2 = {sc, sc};
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
    float m;        // reference (base-2 logit) of head c; lags its running max by < 8
    float l;        // this lane's share of the running sum, relative to m
};

// The lane's C entries: 4g + i (i < 4) and 16 + 4g + i - 4 (i >= 4).
__device__ __forceinline__ int c_entry(int i, int g) { return i < 4 ? 4 * g + i : 12 + 4 * g + i; }

// One tile: V into LDS, logits, online softmax, PV.  GLOBAL: a tile of
// selected FP4 records, else a tile of FP8 window tokens.
template <bool GLOBAL, int STAGE>
__device__ __forceinline__ void process_tile(const SeqView& s, int t, const TileRegs& r,
                                             const float* __restrict__ win_l,
                                             const half8_t (&qhi)[4], const half8_t (&qlo)[4],
                                             _Float16* __restrict__ vtile, int lane,
                                             WaveState& st) {
    const int c = lane & 15, g = lane >> 4;
    constexpr bool global = GLOBAL;

    if (global && STAGE == kStageWrite && t % s.stage_mod == s.stage_rem) {
        // hand the gathered bytes on to the layers that reuse this selection
        uint8_t* dst = s.stage + (int64_t)t * kStageTileBytes;
        u32x4_t* d = reinterpret_cast<u32x4_t*>(dst + 16 * lane);
        d[0] = r.k[0][0];
        d[64] = r.k[1][0];
        d[128] = r.v[0];
        d[192] = r.v[1];
        if (lane < kTile) d[256] = r.sc;
        if (lane == 0) *reinterpret_cast<uint32_t*>(dst + 4608) = r.valid;
    }

    // scale bytes come from the lane that loaded the entry's 16-byte chunk:
    // K scales 2g, 2g + 1 of entries c and 16 + c; V scales 2q, 2q + 1 of
    // entries lane/4 and 16 + lane/4
    const int q4 = lane & 3;
    uint32_t ksc[2] = {0u, 0u}, vsc[2] = {0u, 0u};
    if (global) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int src = (16 * blk + c) << 2;
            const uint32_t d0 = __builtin_amdgcn_ds_bpermute(src, r.sc[0]);
            const uint32_t d1 = __builtin_amdgcn_ds_bpermute(src, r.sc[1]);
            ksc[blk] = ((g >> 1) ? d1 : d0) >> (16 * (g & 1));
            const int vsrc = (16 * blk + (lane >> 2)) << 2;
            const uint32_t d2 = __builtin_amdgcn_ds_bpermute(vsrc, r.sc[2]);
            const uint32_t d3 = __builtin_amdgcn_ds_bpermute(vsrc, r.sc[3]);
            vsc[blk] = ((q4 >> 1) ? d3 : d2) >> (16 * (q4 & 1));
        }
    }

    // ---- V codes of the lane, dequantised, row-major into the wave's V tile ----
    if (global) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            half8_t* dst = reinterpret_cast<half8_t*>(vtile + (16 * j + (lane >> 2)) * kVPitch + 32 * q4);
            const _Float16 s0 = e4m3_to_f16(vsc[j] & 0xFFu), s1 = e4m3_to_f16((vsc[j] >> 8) & 0xFFu);
#pragma unroll
            for (int m = 0; m < 4; ++m) dst[m] = fp4x8_h8(r.v[j][m], m < 2 ? s0 : s1);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            half8_t* dst = reinterpret_cast<half8_t*>(vtile + (8 * j + (lane >> 3)) * kVPitch + 16 * (lane & 7));
            dst[0] = fp8x8_h8(r.v[j][0], r.v[j][1]);
            dst[1] = fp8x8_h8(r.v[j][2], r.v[j][3]);
        }
    }

    // ---- S^T = K Q^T (base-2 logits up to the window row scale) ----
    float4_t sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        half8_t ka[4];
        if (global) {
            const uint32_t sb = ksc[blk];
            const _Float16 s0 = e4m3_to_f16(sb & 0xFFu), s1 = e4m3_to_f16((sb >> 8) & 0xFFu);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) ka[ks] = fp4x8_h8(r.k[blk][0][ks], ks < 2 ? s0 : s1);
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                ka[ks] = fp8x8_h8(r.k[blk][ks >> 1][2 * (ks & 1)], r.k[blk][ks >> 1][2 * (ks & 1) + 1]);
        }
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[ks], qhi[ks], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[ks], qlo[ks], acc, 0, 0, 0);
        }
        sacc[blk] = acc;
    }

    // ---- logits of the lane's C entries; absent entries are -inf ----
    float x[8], vmul[8];
    const uint32_t vbits = ((r.valid >> (4 * g)) & 0xFu) | (((r.valid >> (16 + 4 * g)) & 0xFu) << 4);
    if (global) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = (vbits >> i & 1u) ? sacc[i >> 2][i & 3] : -INFINITY;
            vmul[i] = 1.0f;
        }
    } else {
        const int tok0 = (t - s.n_tiles_global) * kTile;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tok = tok0 + c_entry(i, g);
            x[i] = (vbits >> i & 1u) ? sacc[i >> 2][i & 3] * win_l[tok] : -INFINITY;
            vmul[i] = win_l[kMaxWindow + tok];
        }
    }

    // ---- online softmax; the reference m moves only when the tile max passes
    // it by more than the slack, so most tiles skip the rescale ----
    float tmax = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, x[i]);
    tmax = xmax4(tmax);
    const bool move = tmax > st.m + kRescaleSlack || (st.m == -INFINITY && tmax != -INFINITY);
    if (__builtin_amdgcn_ballot_w64(move)) {  // uniform branch
        const float m_new = move ? tmax : st.m;
        const float alpha = (st.m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(st.m - m_new);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.o[dt] *= alpha;
        st.l *= alpha;
        st.m = m_new;
    }
    half8_t pb;
    float psum = 0.0f;
    if (st.m == -INFINITY) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (_Float16)0.0f;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(x[i] - st.m);  // x - m <= 8; -inf -> 0
            psum += p;
            pb[i] = (_Float16)(p * vmul[i]);
        }
    }
    st.l += psum;

    wave_lds_sync();
    // ---- O^T += V^T P^T; the A operand is read transposed from the row-major
    // V tile: in each 16-lane group, lane 4j + i/4 supplies channels
    // [16dt + 4(i/4), +4) of the entry at k slot j, and lane i receives channel
    // 16dt + i of the four entries ----
    const int sq = lane & 15;
    const int ent0 = 4 * g + (sq >> 2), ent1 = 16 + 4 * g + (sq >> 2);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const int col = 16 * dt + 4 * (sq & 3);
        const half4_t v0 = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t*)(vtile + ent0 * kVPitch + col)));
        const half4_t v1 = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t*)(vtile + ent1 * kVPitch + col)));
        const half8_t va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, st.o[dt], 0, 0, 0);
    }
    wave_lds_sync();  // the next tile rewrites the V tile
}

// grid = ceil(n_q / 8) * 8 * (H / 16) workgroups of 512 threads.
// Workgroup id -> (query bq, head group hg): ids with the same id % 8 share an
// XCD, and all head groups of one query get ids with the same id % 8.
// Every argument is needed before the first gather; touching them all at
// kernel entry makes the compiler fetch them in one batch of scalar loads
// instead of one dependent batch per first use.
template <class T>
__device__ __forceinline__ void touch(const T& v) {
    asm volatile("" ::"s"(v));
}

template <int STAGE, int kWaves>
__global__ __launch_bounds__(kWaves * 64) void k_attn(AttnArgs a, int n_tiles_global) {
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

    float* q_l = reinterpret_cast<float*>(smem + kOffQ);
    float* win_l = reinterpret_cast<float*>(smem + kOffWin);

    SeqView s;
    s.kvc = a.kvc; s.kvs = a.kvs; s.swk = a.swk; s.swv = a.swv;
    s.idx = a.idx + bq * a.topk;
    // in a gathering launch the head groups' workgroups share the stage writes
    s.stage = STAGE != 0 ? a.stage + bq * n_tiles_global * kStageTileBytes : nullptr;
    s.stage_rem = hg;
    s.stage_mod = G;
    s.cap = a.cap;
    s.b = bq / a.Q;
    s.topk = a.topk;
    s.swa_rows = a.swa_rows;
    s.n_tiles_global = n_tiles_global;
    const float logit_mul = a.sm_scale * kLog2e;

    // ---- each wave starts gathering its first two tiles at once; tiles of
    // selected records do not wait for the window length ----
    const int t0 = wave, t1 = wave + kWaves;
    TileRegs ra, rb;
    {
        const bool pos = STAGE != kStageRead;  // positions needed
        const int32_t p0 = pos && t0 < n_tiles_global ? tile_position(s, t0, lane) : -1;
        const int32_t p1 = pos && t1 < n_tiles_global ? tile_position(s, t1, lane) : -1;
        s.swa_len = 0;  // not read on the path of selected records
        if (t0 < n_tiles_global) fetch_tile<STAGE>(s, t0, p0, lane, ra);
        if (t1 < n_tiles_global) fetch_tile<STAGE>(s, t1, p1, lane, rb);
    }
    if (a.swa_len != nullptr) {
        const int sl = a.swa_len[s.b];
        s.swa_start = 0;
        s.swa_len = sl < 0 ? 0 : (sl > a.swa_rows ? a.swa_rows : sl);
    } else {
        // chunk query i sees the window tokens [max(0, i - 127), i]
        const int i = (int)(bq % a.Q);
        s.swa_start = i + 1 > kMaxWindow ? i + 1 - kMaxWindow : 0;
        s.swa_len = i + 1 - s.swa_start;
    }
    const int n_tiles = n_tiles_global + (s.swa_len + kTile - 1) / kTile;
    if (t0 >= n_tiles_global && t0 < n_tiles) fetch_tile<STAGE>(s, t0, -1, lane, ra);
    if (t1 >= n_tiles_global && t1 < n_tiles) fetch_tile<STAGE>(s, t1, -1, lane, rb);

    // ---- meanwhile, once per workgroup: q of the 16 heads, window scales ----
    {
        static_assert(kGroupHeads * kHeadDim / 4 % kThreads == 0, "q staging");
        static_assert(2 * kMaxWindow <= kThreads, "window scales staging");
#pragma unroll
        for (int i = tid; i < kGroupHeads * kHeadDim / 4; i += kThreads)
            reinterpret_cast<float4*>(q_l)[i] = reinterpret_cast<const float4*>(
                a.q + (bq * a.H + hg * kGroupHeads) * kHeadDim)[i];
        float wv = 0.0f;
        const int tok = tid & (kMaxWindow - 1);
        if (tid < 2 * kMaxWindow && tok < s.swa_len)
            wv = (tid < kMaxWindow ? a.swks : a.swvs)[s.b * s.swa_rows + s.swa_start + tok];
        if (tid < 2 * kMaxWindow) win_l[tid] = wv;
    }
    __syncthreads();

    // q * sm_scale * log2(e) (so that logits come out in base-2 units) as fp16
    // hi + lo, B-operand layout: head c, MFMA step ks takes channels 32g + 8ks .. +8
    half8_t qhi[4], qlo[4];
    {
        const float4* qrow = reinterpret_cast<const float4*>(q_l + c * kHeadDim + 32 * g);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const float4 x0 = qrow[2 * ks], x1 = qrow[2 * ks + 1];
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float xq = xs[i] * logit_mul;
                const _Float16 hq = (_Float16)xq;
                qhi[ks][i] = hq;
                qlo[ks][i] = (_Float16)(xq - (float)hq);
            }
        }
    }

    WaveState st;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.0f;
    _Float16* vtile = reinterpret_cast<_Float16*>(smem + kOffWave + wave * kWaveBytes);

    for (int t = t0; t < n_tiles; t += 2 * kWaves) {
        if (t < n_tiles_global)
            process_tile<true, STAGE>(s, t, ra, win_l, qhi, qlo, vtile, lane, st);
        else
            process_tile<false, STAGE>(s, t, ra, win_l, qhi, qlo, vtile, lane, st);
        const int ta = t + 2 * kWaves;
        if (ta < n_tiles)
            fetch_tile<STAGE>(s, ta,
                              STAGE != kStageRead && ta < n_tiles_global ? tile_position(s, ta, lane) : -1,
                              lane, ra);
        const int u = t + kWaves;
        if (u < n_tiles) {
            if (u < n_tiles_global)
                process_tile<true, STAGE>(s, u, rb, win_l, qhi, qlo, vtile, lane, st);
            else
                process_tile<false, STAGE>(s, u, rb, win_l, qhi, qlo, vtile, lane, st);
            const int ub = u + 2 * kWaves;
            if (ub < n_tiles)
                fetch_tile<STAGE>(s, ub,
                                  STAGE != kStageRead && ub < n_tiles_global ? tile_position(s, ub, lane) : -1,
                                  lane, rb);
        }
    }

    // ---- merge the 8 waves' states through LDS (aliases the wave areas) ----
    const float l_wave = xsum4(st.l);
    __syncthreads();
    float* mo = reinterpret_cast<float*>(smem + kOffWave);
    float* mm = mo + kWaves * kGroupHeads * kMergePitch;
    float* ml = mm + kWaves * kGroupHeads;
    {
        float* orow = mo + (wave * kGroupHeads + c) * kMergePitch + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            *reinterpret_cast<float4*>(orow + 16 * dt) =
                make_float4(st.o[dt][0], st.o[dt][1], st.o[dt][2], st.o[dt][3]);
        if (g == 0) {
            mm[wave * kGroupHeads + c] = st.m;
            ml[wave * kGroupHeads + c] = l_wave;
        }
    }
    __syncthreads();
    for (int item = tid; item < kGroupHeads * (kHeadDim / 4); item += kThreads) {
        const int hh = item / (kHeadDim / 4), d4 = item % (kHeadDim / 4);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mm[w * kGroupHeads + hh]);
        float L = 0.0f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float mw = mm[w * kGroupHeads + hh];
                const float wt = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
                L += wt * ml[w * kGroupHeads + hh];
                const float4 ow = *reinterpret_cast<const float4*>(
                    mo + (w * kGroupHeads + hh) * kMergePitch + 4 * d4);
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
