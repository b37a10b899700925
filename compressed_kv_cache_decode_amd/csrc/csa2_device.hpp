// csa2_device.hpp -- device-side number formats and wave helpers for gfx950.
//
// Formats ("DeepSeek V4.1 Flash: architecture study notes", section 4; "DeepSeek
// V4.1 Flash is live", "cache precision and persistence tiers"): main KV is
// E2M1 with one E4M3 scale per 16 channels; the SWA window and the indexer key
// are E4M3 with one fp32 scale per row.  E4M3 is the OCP 8-bit format (bias 7,
// max 448, no infinities); E2M1 is the OCP MX 4-bit format.
//
// Everything in this library is compiled with -ffp-contract=off: a float
// expression is the sequence of IEEE operations it reads as, and fused
// multiply-adds appear only where fmaf() is written.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kHeadDim = 128;
constexpr int kIdxHeads = 4;
constexpr int kIdxDim = 64;
constexpr int kIdxTile = 64;
constexpr int kBlock = 8;

// ---------------------------------------------------------------------------
// E4M3 encode: round to nearest, ties to even, saturate to +-448.
// Normal range: round the fp32 bit pattern to 3 mantissa bits with the usual
// add-half-minus-one-plus-lsb trick (the carry walks into the exponent), then
// rebias the exponent from 127 to 7.  Subnormal range (|x| < 2^-6): the code
// is rint(|x| * 2^9), which is exact scaling followed by one RNE rounding;
// a result of 8 is the smallest normal 2^-6, whose code is also 8.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x43E00000u) {                 // |x| >= 448 (also inf / nan)
        code = 0x7Eu;
    } else if (a < 0x3C800000u) {           // |x| < 2^-6
        code = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
    } else {
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        code = r - (120u << 3);
        if (code > 0x7Eu) code = 0x7Eu;
    }
    return sign | code;
}

// E4M3 decode from bits (used outside hot loops and as the cross-check of
// the hardware converter).
__device__ __forceinline__ float e4m3_decode_bits(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * (1.0f / 512.0f);
    return (c & 0x80u) ? -mag : mag;
}

// Hardware conversion of two E4M3 bytes (gfx950 uses the OCP encoding).
// WORD = false converts bytes 0,1 of `packed`; WORD = true converts bytes 2,3.
template <bool WORD>
__device__ __forceinline__ float2 e4m3x2_to_f32(uint32_t packed) {
    auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)packed, WORD);
    return make_float2(v[0], v[1]);
}

// ---------------------------------------------------------------------------
// E2M1 encode of t = x / scale: ladder of the midpoints between the eight
// magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; a value exactly on a midpoint goes
// to the even code; anything above 5 saturates to 6.  Sign in bit 3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e2m1_encode(float t) {
    const uint32_t sign = (__float_as_uint(t) >> 28) & 8u;
    const float a = fabsf(t);
    uint32_t c;
    if (a <= 0.25f) c = 0;
    else if (a < 0.75f) c = 1;
    else if (a <= 1.25f) c = 2;
    else if (a < 1.75f) c = 3;
    else if (a <= 2.5f) c = 4;
    else if (a < 3.5f) c = 5;
    else if (a <= 5.0f) c = 6;
    else c = 7;
    return sign | c;
}

// E2M1 code -> fp16 bit pattern (exact): exponent field e (bias 1) and
// mantissa bit m map to fp16 exponent e - 1 + 15; code 1 is 0.5 (0x3800).
__device__ __forceinline__ uint32_t e2m1_to_f16_bits(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    uint32_t mag = e ? (((e + 14u) << 10) | (m << 9)) : (m ? 0x3800u : 0u);
    return ((c & 8u) << 12) | mag;
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    float mag = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : (m ? 0.5f : 0.0f);
    return (c & 8u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// Ranking keys: an order-preserving map from fp32 scores to uint32 where a
// larger score gives a larger key.  -0 is first folded onto +0 (x + 0.0f),
// so equal scores always give equal keys.  Every non-NaN float maps to a key
// >= 0x00800000, which leaves 0 free to mean "not visible".
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float s) {
    const uint32_t u = __float_as_uint(s + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).  DPP controls: quad_perm [1,0,3,2] = 0xB1,
// quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141 (lane i <-> 7-i within
// each group of 8), row_mirror = 0x140 (lane i <-> 15-i within each row of 16).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// max over each aligned group of 8 lanes, result in every lane of the group
__device__ __forceinline__ uint32_t max8_u32(uint32_t v) {
    v = max(v, dpp<0xB1>(v));
    v = max(v, dpp<0x4E>(v));
    v = max(v, dpp<0x141>(v));
    return v;
}

// max over the wave of a value whose aligned 8-lane groups already hold their
// group max (max8_u32): scalar reads of the eight groups
__device__ __forceinline__ uint32_t wave_max_of_groups8(uint32_t g8) {
    uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)g8, 0);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = max(m, (uint32_t)__builtin_amdgcn_readlane((int)g8, 8 * i));
    return m;
}

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __uint_as_float(dpp<CTRL>(__float_as_uint(v)));
}

// max over the wave (every lane active): DPP within each 16-lane row
// (quad_perm, row_half_mirror, row_mirror = 0x140), then the four rows'
// results read as scalars; the result is the same in every lane
__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, dppf<0xB1>(v));
    v = fmaxf(v, dppf<0x4E>(v));
    v = fmaxf(v, dppf<0x141>(v));
    v = fmaxf(v, dppf<0x140>(v));
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Indexer query of one head, lane = channel (a whole wave): sq = fl(amax /
// 448), code = RNE_E4M3(fl(x / sq)) (a zero head keeps its signs as +-0
// codes); returns the code's exact fp32 value.  The caller folds sq into the
// head weight, w' = fl(w * sq).
__device__ __forceinline__ float quantise_query_channel(float x, float& sq) {
    sq = wave_max_f32(fabsf(x)) / 448.0f;
    const uint32_t c = (sq == 0.0f) ? ((__float_as_uint(x) >> 24) & 0x80u) : e4m3_encode(x / sq);
    return e4m3_decode_bits(c);
}

// max over each aligned group of 8 lanes (every lane active), in every lane
// of the group
__device__ __forceinline__ float group8_max_f32(float v) {
    v = fmaxf(v, dppf<0xB1>(v));
    v = fmaxf(v, dppf<0x4E>(v));
    v = fmaxf(v, dppf<0x141>(v));
    return v;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// fp16 value of an E4M3 byte (exact), through the hardware converter
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t byte) {
    const half2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(byte, 1.0f, false);
    return h[0];
}

// Eight E2M1 codes (one dword) -> eight fp16 values times an fp16 scale.
// The converter runs with scale 1 (exact); the E4M3 scale is applied by an
// fp16 multiply, exact because the product has at most 6 significant bits and
// lies in [2^-10, 2688].
__device__ __forceinline__ void fp4x8_to_f16(uint32_t w, _Float16 sc, _Float16* out) {
    const half2_t s2 = {sc, sc};
    const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    out[0] = h0[0]; out[1] = h0[1]; out[2] = h1[0]; out[3] = h1[1];
    out[4] = h2[0]; out[5] = h2[1]; out[6] = h3[0]; out[7] = h3[1];
}

// Eight E4M3 codes (two dwords) -> eight fp16 values (exact).
__device__ __forceinline__ void fp8x8_to_f16(uint32_t w0, uint32_t w1, _Float16* out) {
    const uint32_t w[2] = {w0, w1};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false);
        const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true);
        out[4 * i + 0] = lo[0];
        out[4 * i + 1] = lo[1];
        out[4 * i + 2] = hi[0];
        out[4 * i + 3] = hi[1];
    }
}

__device__ __forceinline__ int clamp_nvis(int32_t n, int64_t cap) {
    return n < 0 ? 0 : (n > cap ? (int)cap : n);
}

// Largest visible count over the Q queries of sequence b, read by the
// workgroup's threads in parallel and reduced through LDS.  Call from every
// thread.
__device__ __forceinline__ int workgroup_nv_max(const int32_t* __restrict__ n_vis, int b, int Q,
                                                int64_t cap, int* red) {
    int m = 0;
    for (int q = threadIdx.x; q < Q; q += blockDim.x)
        m = max(m, clamp_nvis(n_vis[(int64_t)b * Q + q], cap));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    int r = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r = max(r, red[w]);
    __syncthreads();  // red may be reused
    return r;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load that is not expected to be reused (nontemporal hint)
__device__ __forceinline__ uint4 load16_stream(const uint8_t* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// byte offset of (row, channel group g) in the tiled indexer-K layout
__device__ __forceinline__ int64_t ik_offset(int64_t row, int g) {
    return (((row >> 6) * 4 + g) * 64 + (row & 63)) * 16;
}

// FP4 indexer key, tiled the same way: per 64 positions two 1 KB planes,
// plane h holding the 16 code bytes of channels 32h..32h+31 of each position
// (low nibble = even channel); byte offset of (row, plane h)
__device__ __forceinline__ int64_t ik4_offset(int64_t row, int h) {
    return (((row >> 6) * 2 + h) * 64 + (row & 63)) * 16;
}

}  // namespace csa2
