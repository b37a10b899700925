// csa2_chunk.hip -- Full-layer indexer for a multi-query chunk on MFMA, with a
// guard band and an exact rescore.
//
// "DeepSeek V4.1 Flash: architecture study notes", section 5: a decoder whose
// window state is gone replays the last 128 tokens; each replayed query runs
// the Full layer's indexer over every position it can see.  With 128 queries
// the scores form a dense [positions x queries x 4 heads x 64 channels]
// contraction, so they are computed on v_mfma_f32_16x16x32_f16.  E4M3 values
// (keys and quantised queries) are exact in fp16 and their products exact in
// fp32, so each MFMA dot product is within a small, bounded distance of the
// score the indexer defines (the sequential fp32 FMA chain over the channels):
//
//   |dot_mfma - dot_exact| <= 2^-18 S  (fp32 accumulation; measured <= 2^-22 S)
//   |dot_seq  - dot_exact| <= 63 * 2^-24 * (1 + 2^-18) S < 2^-18 S
//   S = sum_c |q_c k_c| <= 448 ||q_h||_1       (every E4M3 key value <= 448)
//
// so per head |dot_mfma - dot_seq| <= D_h = 2^-16 * 448 * ||q_h||_1 (twice the
// sum above).  ReLU does not widen it.  The head combine t = sum_h w'_h r_h
// and the scale s = sigma * t are fp32 operations on both sides; their
// rounding is at most a few 2^-24 T (T = sum_h |w'_h| r_h, and every r_h is at
// most (1 + 2^-18) 448 ||q_h||_1), covered by 2^-18 T, plus 2^-24 |s| per
// operation on s, covered by 2^-20 |s|.  So each visible position's score lies
// within
//
//   d = sigma * C'_q + 2^-20 |s|,  C'_q = (1 + 2^-10) (2^-16 + 2^-18) 448 sum_h |w'_h| ||q_h||_1
//
// of the exact one (the factor 1 + 2^-10 absorbs the rounding of the bound
// arithmetic itself).  A lane holds 4 positions of a block of 8; with
// m = max s, a = max |s| and g = max sigma over its visible ones,
// M = g C'_q + 2^-20 a bounds every d there, so m - M is at most the exact
// score of the position that attains m, and m + M at least every exact score
// of the four.  The kernel writes, per block of 8, the key of the larger lower
// bound of its two lanes (lo: some position's exact score reaches it), and per
// half-block of 4, the key of the lane's upper bound (hi: no exact score of
// the four exceeds it); 0 where no position is visible.
//
// If x is the K-th largest block lo, K distinct blocks each hold a position
// with exact score >= x, so the K-th largest exact score t is >= x, and every
// position with score >= t (every position the exact top-K can take, ties
// included) lies in a half-block whose hi reaches x.  Those half-blocks hold
// the exact top-K; k_chunk_select (csa2_index.hip) lists them in ascending
// order, scores their positions exactly (the VALU scan's arithmetic, same keys
// bit for bit) and selects there, so ties still go to the lowest position.  A
// query whose candidates do not fit its list is scored over all its visible
// positions instead.
#include <hip/hip_ext.h>

#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kMmaQ = 128;        // queries staged in LDS per pass
constexpr int kMmaPitch = 264;    // fp16 per staged query: 4 heads x 64 + 8 (bank spread)
constexpr int kMmaThreads = 512;  // 8 waves, 32 positions each
constexpr int kMmaPos = 256;      // positions per workgroup

// Eight E4M3 codes (two dwords), exact in fp16.
__device__ __forceinline__ half8_t e4m3x8_h8(uint32_t w0, uint32_t w1) {
    const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    const half4_t a = __builtin_shufflevector(h0, h1, 0, 1, 2, 3);
    const half4_t b = __builtin_shufflevector(h2, h3, 0, 1, 2, 3);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// max(x, 0) as one signed integer max of the bits: every float with the sign
// bit set (-0 included) becomes +0, the rest stay (an fmaxf would also quiet
// its operand first)
__device__ __forceinline__ float relu(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// grid = (ceil(cap / 256), B), 512 threads.  Wave w scores positions
// p0 + 32w .. +32 (two MFMA row tiles of 16) against every query of sequence
// b, 16 queries per MFMA column tile, one accumulator per head:
// S_h^T[16 positions x 16 queries] += K[16 x 32 channels] Q_h^T[32 x 16], two
// channel steps per head.  Lane l holds rows 4(l/16) .. +4 of column l % 16;
// lanes l and l ^ 16 share a block of 8 positions.
// FMT kIdxFp4: FP4 keys (E2M1 codes, one E4M3 scale per 16 channels, no
// per-position scale): the A operands are the keys' exact values e2m1 x scale
// in fp16 and the score is not scaled (sigma 1); the guard band, derived for
// keys |k| <= 448 sigma, takes for a row the factor g = 6 max_g scale_g / 448,
// since its values satisfy |k| <= 6 max_g scale_g.
template <int FMT>
__global__ __launch_bounds__(kMmaThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_scan_mma(
    const uint8_t* __restrict__ ikc, const float* __restrict__ iks, int64_t cap, int Q,
    const _Float16* __restrict__ qh, const float* __restrict__ wq, const float* __restrict__ cq,
    const int32_t* __restrict__ n_vis, uint32_t* __restrict__ bkeys_lo,
    uint32_t* __restrict__ hkeys_hi) {
    __shared__ __attribute__((aligned(16))) _Float16 sq[kMmaQ * kMmaPitch];
    __shared__ __attribute__((aligned(16))) float sw[kMmaQ * kIdxHeads];
    __shared__ float sc[kMmaQ];
    __shared__ int snv[kMmaQ];
    __shared__ int red[kMmaThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * kMmaPos;
    const int nv_max = workgroup_nv_max(n_vis, b, Q, cap, red);
    if (p0 >= nv_max) return;  // uniform over the workgroup
    const int64_t nb = cap / kBlock;

    // A operands of the wave's two row tiles: lane l holds position
    // base + l % 16, channels 32 ks + 8 (l / 16) .. +8 (channel group
    // 2 ks + l / 32, bytes 8 ((l / 16) & 1) of its 16); and sigma of the four
    // output rows 4 (l / 16) + i
    half8_t a[2][2];
    float4 sig[2];
    float gmax[2];  // the guard-band factor of the lane's four output rows
    bool inside[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const int64_t base = p0 + 32 * wave + 16 * st;
        inside[st] = base < cap;  // cap is a multiple of 64: a row tile is wholly in or out
        if (inside[st]) {
            const int64_t row = (int64_t)b * cap + base + (lane & 15);
            if constexpr (FMT == kIdxFp8) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const uint2 raw = *reinterpret_cast<const uint2*>(
                        ikc + ik_offset(row, 2 * ks + (lane >> 5)) + 8 * ((lane >> 4) & 1));
                    a[st][ks] = e4m3x8_h8(raw.x, raw.y);
                }
                sig[st] = *reinterpret_cast<const float4*>(iks + (int64_t)b * cap + base +
                                                          4 * (lane >> 4));
            } else {
                // channels 32 ks + 8 (l / 16) .. +8: plane ks, code bytes
                // 4 (l / 16) .. +4, scale byte 2 ks + l / 32
                const uint32_t sc4 = reinterpret_cast<const uint32_t*>(iks)[row];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(
                        ikc + ik4_offset(row, ks) + 4 * (lane >> 4));
                    const uint32_t sb = (sc4 >> (8 * (2 * ks + (lane >> 5)))) & 0xFFu;
                    const _Float16 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false)[0];
                    _Float16 v[8];
                    fp4x8_to_f16(w, sc, v);
                    a[st][ks] = half8_t{v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
                }
                sig[st] = make_float4(1.f, 1.f, 1.f, 1.f);
            }
        } else {
            const half8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
            a[st][0] = z;
            a[st][1] = z;
            sig[st] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        gmax[st] = fmaxf(fmaxf(sig[st].x, sig[st].y), fmaxf(sig[st].z, sig[st].w));
        if constexpr (FMT == kIdxFp4) {
            // largest E4M3 scale of the four output rows 4 (l / 16) + i
            float smax = 0.0f;
            if (inside[st]) {
                const uint4 w4 = *reinterpret_cast<const uint4*>(
                    reinterpret_cast<const uint32_t*>(iks) + (int64_t)b * cap + base +
                    4 * (lane >> 4));
                const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
                    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
                    smax = fmaxf(smax, fmaxf(fmaxf(lo[0], lo[1]), fmaxf(hi[0], hi[1])));
                }
            }
            gmax[st] = smax * (6.0f / 448.0f);
        }
    }

    for (int q0 = 0; q0 < Q; q0 += kMmaQ) {
        const int nqp = min(kMmaQ, Q - q0);
        const int64_t bq0 = (int64_t)b * Q + q0;
        __syncthreads();  // the previous pass's readers are done
        {
            // the pass's queries, 16 bytes a lane, every load in flight at once
            constexpr int kPer = kMmaQ * kIdxHeads * kIdxDim / 8 / kMmaThreads;
            const int n16 = nqp * (kIdxHeads * kIdxDim / 8);
            const uint4* src = reinterpret_cast<const uint4*>(qh + bq0 * kIdxHeads * kIdxDim);
            uint4 v[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int i = tid + k * kMmaThreads;
                v[k] = i < n16 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int i = tid + k * kMmaThreads;
                if (i < n16)
                    *reinterpret_cast<uint4*>(sq + (i >> 5) * kMmaPitch + 8 * (i & 31)) = v[k];
            }
        }
        for (int i = tid; i < nqp * kIdxHeads; i += kMmaThreads) sw[i] = wq[bq0 * kIdxHeads + i];
        for (int j = tid; j < nqp; j += kMmaThreads) {
            sc[j] = cq[bq0 + j];
            snv[j] = clamp_nvis(n_vis[bq0 + j], cap);
        }
        __syncthreads();

        for (int qt = 0; qt < nqp; qt += 16) {
            const int j = qt + (lane & 15);  // this lane's query (column)
            const bool qok = j < nqp;
            const int jj = qok ? j : 0;  // columns past the pass read query 0, unused
            half8_t bop[kIdxHeads][2];
#pragma unroll
            for (int h = 0; h < kIdxHeads; ++h)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    bop[h][ks] = *reinterpret_cast<const half8_t*>(
                        sq + jj * kMmaPitch + h * kIdxDim + 32 * ks + 8 * (lane >> 4));
            const float4 w = *reinterpret_cast<const float4*>(sw + jj * 4);
            const float cqj = sc[jj];
            const int nv = snv[jj];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                if (!inside[st]) continue;  // uniform over the wave
                const int64_t base = p0 + 32 * wave + 16 * st;
                const int64_t pos0 = base + 4 * (lane >> 4);  // this lane's four rows
                float4_t acc[kIdxHeads];
#pragma unroll
                for (int h = 0; h < kIdxHeads; ++h) {
                    acc[h] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[st][ks], bop[h][ks],
                                                                       acc[h], 0, 0, 0);
                }
                const float sg[4] = {sig[st].x, sig[st].y, sig[st].z, sig[st].w};
                float s[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float r0 = relu(acc[0][i]), r1 = relu(acc[1][i]);
                    const float r2 = relu(acc[2][i]), r3 = relu(acc[3][i]);
                    float t = w.x * r0;
                    t = fmaf(w.y, r1, t);
                    t = fmaf(w.z, r2, t);
                    t = fmaf(w.w, r3, t);
                    s[i] = sg[i] * t;
                }
                float m, a_abs;
                if (pos0 + 3 < nv) {
                    m = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
                    const float lo4 = fminf(fminf(s[0], s[1]), fminf(s[2], s[3]));
                    a_abs = fmaxf(m, -lo4);
                } else {  // the query's visible range ends in these four rows
                    m = -INFINITY;
                    float lo4 = INFINITY;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (pos0 + i < nv) {
                            m = fmaxf(m, s[i]);
                            lo4 = fminf(lo4, s[i]);
                        }
                    a_abs = m >= lo4 ? fmaxf(m, -lo4) : 0.0f;  // m = -inf: none visible
                }
                const float M = fmaf(a_abs, 0x1p-20f, gmax[st] * cqj);
                const float hi = m + M;  // -inf when no row is visible
                float lo = m - M;
                if (qok)  // half-block (base + 4 (l / 16)) / 4
                    hkeys_hi[(bq0 + j) * (2 * nb) + (base >> 2) + (lane >> 4)] =
                        hi != -INFINITY ? score_key(hi) : 0u;
                lo = fmaxf(lo, __shfl_xor(lo, 16, 64));
                if (qok && ((lane >> 4) & 1) == 0)
                    bkeys_lo[(bq0 + j) * nb + (base >> 3) + (lane >> 5)] =
                        lo != -INFINITY ? score_key(lo) : 0u;
            }
        }
    }
}

hipError_t launch_scan_mma(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                           const _Float16* qh, const float* wq, const float* cq,
                           const int32_t* n_vis, uint32_t* bkeys_lo, uint32_t* hkeys_hi,
                           hipStream_t stream, hipEvent_t start, hipEvent_t stop, int fmt) {
    dim3 grid((unsigned)((cap + kMmaPos - 1) / kMmaPos), (unsigned)B);
    auto kern = fmt == kIdxFp4 ? k_scan_mma<kIdxFp4> : k_scan_mma<kIdxFp8>;
    if (start != nullptr && stop != nullptr) {
        hipExtLaunchKernelGGL(kern, grid, dim3(kMmaThreads), 0, stream, start, stop, 0, ikc, iks,
                              cap, Q, qh, wq, cq, n_vis, bkeys_lo, hkeys_hi);
    } else {
        hipLaunchKernelGGL(kern, grid, dim3(kMmaThreads), 0, stream, ikc, iks, cap, Q, qh, wq, cq,
                           n_vis, bkeys_lo, hkeys_hi);
    }
    return hipGetLastError();
}


}  // namespace csa2
