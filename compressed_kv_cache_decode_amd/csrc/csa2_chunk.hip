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
// sum above).  ReLU does not widen it; the head combine t = sum_h w'_h r_h and
// the scale s = sigma * t are the same IEEE operations on both sides, whose
// roundings are covered by the terms 2^-18 T (T = sum_h |w'_h| r_h) and
// 2^-20 |s| below.  Every visible position has a lower bound lo <= s and an
// upper bound hi >= s:
//
//   d = sigma * (C_q + 2^-18 T) + 2^-20 |s|,  C_q = (1 + 2^-10) sum_h |w'_h| D_h
//   lo = s - d,  hi = s + d,
//
// and the kernel writes, per block of 8 positions, the largest key of each.
// If x is the K-th largest block maximum of lo, K distinct blocks each hold a
// position with s >= lo >= x, so the K-th largest exact score t is >= x, and
// every position with s >= t (every position the exact top-K can take, ties
// included) has hi >= x.  The blocks whose largest hi reaches x thus hold the
// exact top-K (k_cand_pool); rescoring their positions exactly (the Reindex
// kernels: same scores, bit for bit, as the VALU scan) and selecting there
// gives the exact top-K with its tie rule, as the candidate blocks are listed
// in ascending order.  A query whose candidate blocks do not fit the pool is
// flagged and recomputed by the exact VALU scan.
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

// grid = (ceil(cap / 256), B), 512 threads.  Wave w scores positions
// p0 + 32w .. +32 (two MFMA row tiles of 16) against every query of sequence
// b, 16 queries per MFMA column tile, one accumulator per head:
// S_h^T[16 positions x 16 queries] += K[16 x 32 channels] Q_h^T[32 x 16], two
// channel steps per head.  Lane l holds rows 4(l/16) .. +4 of column l % 16.
__global__ __launch_bounds__(kMmaThreads) void k_scan_mma(
    const uint8_t* __restrict__ ikc, const float* __restrict__ iks, int64_t cap, int Q,
    const float* __restrict__ qd, const float* __restrict__ wq, const float* __restrict__ cq,
    const int32_t* __restrict__ n_vis, uint32_t* __restrict__ bkeys_lo,
    uint32_t* __restrict__ bkeys_hi) {
    __shared__ __attribute__((aligned(16))) _Float16 sq[kMmaQ * kMmaPitch];
    __shared__ float sw[kMmaQ * kIdxHeads];
    __shared__ float sc[kMmaQ];
    __shared__ int snv[kMmaQ];
    __shared__ int red[kMmaThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * kMmaPos;
    const int nv_max = workgroup_nv_max(n_vis, nullptr, b, Q, cap, red);
    if (p0 >= nv_max) return;  // uniform over the workgroup
    const int64_t nb = cap / kBlock;

    // A operands of the wave's two row tiles: lane l holds position
    // base + l % 16, channels 32 ks + 8 (l / 16) .. +8 (channel group
    // 2 ks + l / 32, bytes 8 ((l / 16) & 1) of its 16); and sigma of the four
    // output rows 4 (l / 16) + i
    half8_t a[2][2];
    float4 sig[2];
    bool inside[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const int64_t base = p0 + 32 * wave + 16 * st;
        inside[st] = base < cap;  // cap is a multiple of 64: a row tile is wholly in or out
        if (inside[st]) {
            const int64_t row = (int64_t)b * cap + base + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint2 raw = *reinterpret_cast<const uint2*>(
                    ikc + ik_offset(row, 2 * ks + (lane >> 5)) + 8 * ((lane >> 4) & 1));
                a[st][ks] = e4m3x8_h8(raw.x, raw.y);
            }
            sig[st] = *reinterpret_cast<const float4*>(iks + (int64_t)b * cap + base + 4 * (lane >> 4));
        } else {
            const half8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
            a[st][0] = z;
            a[st][1] = z;
            sig[st] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }

    for (int q0 = 0; q0 < Q; q0 += kMmaQ) {
        const int nqp = min(kMmaQ, Q - q0);
        const int64_t bq0 = (int64_t)b * Q + q0;
        __syncthreads();  // the previous pass's readers are done
        for (int i = tid; i < nqp * kIdxHeads * kIdxDim; i += kMmaThreads) {
            const int j = i >> 8, hc = i & 255;
            sq[j * kMmaPitch + hc] = (_Float16)qd[(bq0 + j) * kIdxHeads * kIdxDim + hc];  // exact
        }
        for (int i = tid; i < nqp * kIdxHeads; i += kMmaThreads) sw[i] = wq[bq0 * kIdxHeads + i];
        for (int j = tid; j < nqp; j += kMmaThreads) {
            sc[j] = cq[bq0 + j];
            snv[j] = clamp_nvis(n_vis[bq0 + j], cap);
        }
        __syncthreads();

#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (!inside[st]) continue;  // uniform over the wave
            const int64_t base = p0 + 32 * wave + 16 * st;
            const int64_t pos0 = base + 4 * (lane >> 4);  // this lane's four rows
            const float sg[4] = {sig[st].x, sig[st].y, sig[st].z, sig[st].w};
            for (int qt = 0; qt < nqp; qt += 16) {
                const int j = qt + (lane & 15);  // this lane's query (column)
                float4_t acc[kIdxHeads];
#pragma unroll
                for (int h = 0; h < kIdxHeads; ++h) {
                    acc[h] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const int jj = j < nqp ? j : 0;  // columns past the pass read query 0, unused
                        const half8_t bop = *reinterpret_cast<const half8_t*>(
                            sq + jj * kMmaPitch + h * kIdxDim + 32 * ks + 8 * (lane >> 4));
                        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[st][ks], bop, acc[h], 0, 0, 0);
                    }
                }
                const bool qok = j < nqp;
                const int jj = qok ? j : 0;
                const float w0 = sw[jj * 4 + 0], w1 = sw[jj * 4 + 1], w2 = sw[jj * 4 + 2], w3 = sw[jj * 4 + 3];
                const float cqj = sc[jj];
                const int nv = snv[jj];
                uint32_t klo[4], khi[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float r0 = acc[0][i] > 0.0f ? acc[0][i] : 0.0f;
                    const float r1 = acc[1][i] > 0.0f ? acc[1][i] : 0.0f;
                    const float r2 = acc[2][i] > 0.0f ? acc[2][i] : 0.0f;
                    const float r3 = acc[3][i] > 0.0f ? acc[3][i] : 0.0f;
                    // the head combine of the score, operation by operation
                    float t = w0 * r0;
                    t = t + w1 * r1;
                    t = t + w2 * r2;
                    t = t + w3 * r3;
                    const float s = sg[i] * t;
                    const float T = fabsf(w0) * r0 + fabsf(w1) * r1 + fabsf(w2) * r2 + fabsf(w3) * r3;
                    const float d = sg[i] * (cqj + 0x1p-18f * T) + 0x1p-20f * fabsf(s);
                    const bool vis = pos0 + i < nv;
                    klo[i] = vis ? score_key(s - d) : 0u;
                    khi[i] = vis ? score_key(s + d) : 0u;
                }
                // block of 8 = rows 0..7 (lanes l / 16 = 0, 1) or 8..15 (2, 3)
                uint32_t mlo = max(max(klo[0], klo[1]), max(klo[2], klo[3]));
                uint32_t mhi = max(max(khi[0], khi[1]), max(khi[2], khi[3]));
                mlo = max(mlo, (uint32_t)__shfl_xor((int)mlo, 16, 64));
                mhi = max(mhi, (uint32_t)__shfl_xor((int)mhi, 16, 64));
                if (qok && ((lane >> 4) & 1) == 0) {
                    const int64_t blk = (base >> 3) + (lane >> 5);
                    bkeys_lo[(bq0 + j) * nb + blk] = mlo;
                    bkeys_hi[(bq0 + j) * nb + blk] = mhi;
                }
            }
        }
    }
}

hipError_t launch_scan_mma(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                           const float* qd, const float* wq, const float* cq,
                           const int32_t* n_vis, uint32_t* bkeys_lo, uint32_t* bkeys_hi,
                           hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    dim3 grid((unsigned)((cap + kMmaPos - 1) / kMmaPos), (unsigned)B);
    if (start != nullptr && stop != nullptr) {
        hipExtLaunchKernelGGL(k_scan_mma, grid, dim3(kMmaThreads), 0, stream, start, stop, 0, ikc,
                              iks, cap, Q, qd, wq, cq, n_vis, bkeys_lo, bkeys_hi);
    } else {
        hipLaunchKernelGGL(k_scan_mma, grid, dim3(kMmaThreads), 0, stream, ikc, iks, cap, Q, qd,
                           wq, cq, n_vis, bkeys_lo, bkeys_hi);
    }
    return hipGetLastError();
}


}  // namespace csa2
