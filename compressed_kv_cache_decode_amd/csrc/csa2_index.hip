// csa2_index.hip -- CSA2 indexer: Full-layer scan, Reindex pool rescoring and
// exact top-K selection.
//
// "DeepSeek V4.1 Flash: architecture study notes", section 2: a Full layer
// picks this step's positions, at most 512 per query; the decoder's first
// Full layer scans every causally visible position and scores blocks to build
// a shared candidate pool of at most 2048 blocks x 8 positions (Figure 5);
// Reindex layers pick their own top-512 inside the pool with their own
// indexer query; Reuse layers take the indices as they are.  "DeepSeek V4.1
// Flash is live", "CSA2 attention": the pool makes the deeper indexers' cost
// independent of context, the first scan still grows with it.
//
// Score of position s for one query (all IEEE fp32, in this order):
//   dot_h = sum over channels c = 0..63 ascending of E4M3(q_hc) * E4M3(k_sc)
//           (each product is exact in fp32, so fmaf(q, k, dot) is that sum);
//   r_h   = dot_h > 0 ? dot_h : +0;
//   t     = w'_0 r_0, then t = t + w'_h r_h for h = 1, 2, 3;
//   score = sigma_s * t.
// Scores become order-preserving uint32 keys (score_key); 0 = not visible.
//
// Memory layout of the indexer K (per 64 positions: four 1 KB planes, plane g
// holding channels 16g..16g+15 of the 64 positions, 16 bytes each) makes every
// wave-wide load a contiguous 1 KB: lane i reads its position's 16 bytes.
#include <hip/hip_ext.h>

#include <utility>

#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

// Score of one indexer-K row from its four 16-byte channel groups.
// qd: the query's decoded E4M3 values [4][64] (uniform across the wave, read
// through the scalar cache); wq: the 4 folded head weights.
__device__ __forceinline__ void decode_fp8_row(const uint4 (&raw)[4], float (&kf)[kIdxDim]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t w[4] = {raw[g].x, raw[g].y, raw[g].z, raw[g].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float2 lo = e4m3x2_to_f32<false>(w[i]);
            const float2 hi = e4m3x2_to_f32<true>(w[i]);
            kf[16 * g + 4 * i + 0] = lo.x;
            kf[16 * g + 4 * i + 1] = lo.y;
            kf[16 * g + 4 * i + 2] = hi.x;
            kf[16 * g + 4 * i + 3] = hi.y;
        }
    }
}

__device__ __forceinline__ float score_row(const uint4 (&raw)[4], float sigma,
                                           const float* __restrict__ qd,
                                           const float* __restrict__ wq) {
    float kf[kIdxDim];
    decode_fp8_row(raw, kf);
    float t = 0.0f;
#pragma unroll
    for (int h = 0; h < kIdxHeads; ++h) {
        float dot = 0.0f;
#pragma unroll
        for (int c = 0; c < kIdxDim; ++c) dot = fmaf(qd[h * kIdxDim + c], kf[c], dot);
        const float r = dot > 0.0f ? dot : 0.0f;
        const float wr = wq[h] * r;
        t = (h == 0) ? wr : t + wr;
    }
    return sigma * t;
}

__device__ __forceinline__ void load_ik_row(const uint8_t* __restrict__ ikc, int64_t row,
                                            uint4 (&raw)[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
        raw[g] = load16_stream(ikc + ik_offset(row, g));
}

// FP4 indexer key (36 bytes: 32 bytes of E2M1 codes, low nibble = even
// channel, and one E4M3 scale per 16 channels, no per-position scale).
// Block-scaled score, in this order:
//   inner_hg = fp32 sum over the 16 channels of group g ascending of
//              E4M3(q_hc) * E2M1(k_c) (each product exact), from +0;
//   dot_h    = fused multiply-add chain over g = 0..3 of scale_g * inner_hg;
//   r_h, t as for the FP8 key; score = t.
__device__ __forceinline__ void decode_fp4_row(const uint4 (&raw)[2], float (&kf)[kIdxDim]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w[4] = {raw[h].x, raw[h].y, raw[h].z, raw[h].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // byte b of the word: channels 2b (low nibble) and 2b + 1
            const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 0);
            const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 1);
            const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 2);
            const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 3);
            float* o = kf + 32 * h + 8 * i;
            o[0] = v0[0]; o[1] = v0[1]; o[2] = v1[0]; o[3] = v1[1];
            o[4] = v2[0]; o[5] = v2[1]; o[6] = v3[0]; o[7] = v3[1];
        }
    }
}

__device__ __forceinline__ float score_row4(const uint4 (&raw)[2], uint32_t sc4,
                                            const float* __restrict__ qd,
                                            const float* __restrict__ wq) {
    float kf[kIdxDim];  // E2M1 values, unscaled
    decode_fp4_row(raw, kf);
    const float2 s01 = e4m3x2_to_f32<false>(sc4);
    const float2 s23 = e4m3x2_to_f32<true>(sc4);
    const float sg[4] = {s01.x, s01.y, s23.x, s23.y};
    float t = 0.0f;
#pragma unroll
    for (int h = 0; h < kIdxHeads; ++h) {
        float dot = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float inner = 0.0f;
#pragma unroll
            for (int c = 16 * g; c < 16 * g + 16; ++c)
                inner = fmaf(qd[h * kIdxDim + c], kf[c], inner);
            dot = fmaf(sg[g], inner, dot);
        }
        const float r = dot > 0.0f ? dot : 0.0f;
        const float wr = wq[h] * r;
        t = (h == 0) ? wr : t + wr;
    }
    return t;
}

// ---------------------------------------------------------------------------
// The same scores with the query held in registers instead of read through
// the scalar cache at every step.  Lane l holds q_h[4 (l % 16) + r] in
// v[h][r], so channel c of head h sits in register c % 4 of lane c / 4 of
// every 16-lane row, and a DPP row_newbcast operand hands it to all lanes
// inside the multiply-add itself (v_fmac_f32_dpp: acc + q * k, one rounding,
// the fmaf of the scalar versions).  The operations and their order are
// those of score_row and score_row4.  DPP reads other lanes: these run with
// every lane of the wave active.
// ---------------------------------------------------------------------------
struct QQuad {
    float v[kIdxHeads][4];
    // q: one query's decoded values [4][64], in global memory or LDS
    __device__ __forceinline__ void load(const float* q) {
#pragma unroll
        for (int h = 0; h < kIdxHeads; ++h) {
            const float4 x = reinterpret_cast<const float4*>(q + h * kIdxDim)[threadIdx.x & 15];
            v[h][0] = x.x; v[h][1] = x.y; v[h][2] = x.z; v[h][3] = x.w;
        }
    }
};

// acc + (q of lane N of this 16-lane row) * k.  Volatile, so that the
// compiler keeps it where the whole wave is active.
template <int N>
__device__ __forceinline__ float fmac_bcast(float acc, float q, float k) {
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(acc) : "v"(q), "v"(k), "i"(N));
    return acc;
}

// channel C of every head: acc[h] += q_hC * k
template <int C>
__device__ __forceinline__ void fmac_heads(float (&acc)[kIdxHeads], const QQuad& q, float k) {
#pragma unroll
    for (int h = 0; h < kIdxHeads; ++h) acc[h] = fmac_bcast<(C >> 2)>(acc[h], q.v[h][C & 3], k);
}

// channels 16g .. 16g + 15 of group g = G (words 2 (G % 2) and 2 (G % 2) + 1
// of plane G / 2), decoded right before their multiply-adds: the group sums,
// then the scaled add into each head's dot (the scheduling barrier keeps the
// next group's decode below these)
template <int G, int... J>
__device__ __forceinline__ void fp4_group(float (&dot)[kIdxHeads], const QQuad& q,
                                          const uint4& plane, float sg,
                                          std::integer_sequence<int, J...>) {
    const uint32_t w[2] = {(G & 1) ? plane.z : plane.x, (G & 1) ? plane.w : plane.y};
    float kf[16];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        // byte b of the word: channels 2b (low nibble) and 2b + 1
        const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 0);
        const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 1);
        const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 2);
        const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 3);
        float* o = kf + 8 * i;
        o[0] = v0[0]; o[1] = v0[1]; o[2] = v1[0]; o[3] = v1[1];
        o[4] = v2[0]; o[5] = v2[1]; o[6] = v3[0]; o[7] = v3[1];
    }
    float inner[kIdxHeads] = {0.0f, 0.0f, 0.0f, 0.0f};
    (fmac_heads<16 * G + J>(inner, q, kf[J]), ...);
#pragma unroll
    for (int h = 0; h < kIdxHeads; ++h) dot[h] = fmaf(sg, inner[h], dot[h]);
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float weigh_heads(const float (&dot)[kIdxHeads],
                                             const float* __restrict__ wq) {
    float t = 0.0f;
#pragma unroll
    for (int h = 0; h < kIdxHeads; ++h) {
        const float r = dot[h] > 0.0f ? dot[h] : 0.0f;
        const float wr = wq[h] * r;
        t = (h == 0) ? wr : t + wr;
    }
    return t;
}

// channels 16G .. 16G + 15 (plane G of the row), decoded right before their
// multiply-adds: the plane waits for its own load only, and at most 16
// decoded values are live (the scheduling barrier keeps the next plane's
// decode from being hoisted above these)
template <int G, int... J>
__device__ __forceinline__ void fp8_plane(float (&dot)[kIdxHeads], const QQuad& q, const uint4& raw,
                                          std::integer_sequence<int, J...>) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float kf[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float2 lo = e4m3x2_to_f32<false>(w[i]);
        const float2 hi = e4m3x2_to_f32<true>(w[i]);
        kf[4 * i + 0] = lo.x;
        kf[4 * i + 1] = lo.y;
        kf[4 * i + 2] = hi.x;
        kf[4 * i + 3] = hi.y;
    }
    (fmac_heads<16 * G + J>(dot, q, kf[J]), ...);
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float score_row_q(const uint4 (&raw)[4], float sigma, const QQuad& q,
                                             const float* __restrict__ wq) {
    float dot[kIdxHeads] = {0.0f, 0.0f, 0.0f, 0.0f};
    constexpr auto kP = std::make_integer_sequence<int, 16>{};
    fp8_plane<0>(dot, q, raw[0], kP);
    fp8_plane<1>(dot, q, raw[1], kP);
    fp8_plane<2>(dot, q, raw[2], kP);
    fp8_plane<3>(dot, q, raw[3], kP);
    return sigma * weigh_heads(dot, wq);
}

__device__ __forceinline__ float score_row4_q(const uint4 (&raw)[2], uint32_t sc4, const QQuad& q,
                                              const float* __restrict__ wq) {
    const float2 s01 = e4m3x2_to_f32<false>(sc4);
    const float2 s23 = e4m3x2_to_f32<true>(sc4);
    float dot[kIdxHeads] = {0.0f, 0.0f, 0.0f, 0.0f};
    constexpr auto kG = std::make_integer_sequence<int, 16>{};
    fp4_group<0>(dot, q, raw[0], s01.x, kG);
    fp4_group<1>(dot, q, raw[0], s01.y, kG);
    fp4_group<2>(dot, q, raw[1], s23.x, kG);
    fp4_group<3>(dot, q, raw[1], s23.y, kG);
    return weigh_heads(dot, wq);
}

// One position's key in either format: FP8 (codes in the 4-plane tiles, fp32
// sigma per row in `aux`) or FP4 (codes in the 2-plane tiles, the four E4M3
// scale bytes of the row as one 32-bit word of `aux`).
template <int FMT>
struct IdxRow {
    uint4 raw[FMT == 0 ? 4 : 2];
    uint32_t aux;
    __device__ __forceinline__ void load(const uint8_t* __restrict__ ikc,
                                         const float* __restrict__ iks, int64_t row) {
        if constexpr (FMT == 0) {
            load_ik_row(ikc, row, raw);
            aux = __float_as_uint(iks[row]);
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) raw[h] = load16_stream(ikc + ik4_offset(row, h));
            aux = reinterpret_cast<const uint32_t*>(iks)[row];
        }
    }
    __device__ __forceinline__ float score(const float* __restrict__ qd,
                                           const float* __restrict__ wq) const {
        if constexpr (FMT == 0) return score_row(raw, __uint_as_float(aux), qd, wq);
        else return score_row4(raw, aux, qd, wq);
    }
    // the same score, query in registers (whole wave active)
    __device__ __forceinline__ float score(const QQuad& q, const float* __restrict__ wq) const {
        if constexpr (FMT == 0) return score_row_q(raw, __uint_as_float(aux), q, wq);
        else return score_row4_q(raw, aux, q, wq);
    }
};

// Keys of one query over its nv visible positions (and the block keys of the
// blocks they fill), computed by a whole workgroup of `nthreads` threads with
// k_scan's arithmetic: the replay chunk's fallback for a query whose MFMA
// candidates overflowed.  Positions past nv in the last block get key 0.
template <int FMT>
__device__ __forceinline__ void scan_query_exact(const uint8_t* __restrict__ ikc,
                                                 const float* __restrict__ iks, int64_t row0,
                                                 const float* __restrict__ qd,
                                                 const float* __restrict__ wq, int nv, int nthreads,
                                                 uint32_t* __restrict__ keys,
                                                 uint32_t* __restrict__ bkeys) {
    const int64_t nv8 = ((int64_t)nv + kBlock - 1) / kBlock * kBlock;
    for (int64_t p0 = 0; p0 < nv8; p0 += nthreads) {  // uniform trip count
        const int64_t p = p0 + threadIdx.x;
        uint32_t key = 0u;
        if (p < nv) {
            IdxRow<FMT> r;
            r.load(ikc, iks, row0 + p);
            key = score_key(r.score(qd, wq));
        }
        const uint32_t bk = max8_u32(key);  // every lane of the wave takes part
        if (p < nv8) {
            keys[p] = key;
            if ((threadIdx.x & 7) == 0) bkeys[p >> 3] = bk;
        }
    }
}

// ---------------------------------------------------------------------------
// Full-layer scan.  grid = (ceil(cap / 256), B); 256 threads, one position each.
// Each workgroup quantises the query itself (wave h: head h, the E4M3 codes'
// fp32 values and the folded weights w' = w * sq in LDS, as k_prep_iq
// computes them) while its key rows are in flight, and every lane then holds
// its quad of query values in registers (QQuad).
// For every query of the sequence: key of each position, the max key of each
// 8-position block (DPP max over 8 adjacent lanes) and, when sbkeys is set,
// of each 64-position superblock (one wave).  Tiles that no query of the
// sequence can see are skipped entirely.
// ---------------------------------------------------------------------------
// FMT 0: FP8 keys (iks = fp32 sigma per row); FMT 1: FP4 keys (iks = the
// rows' four E4M3 scale bytes, read as one 32-bit word per row).
// iq [B*Q][4][64], iw [B*Q][4]: the queries and head weights as given.
// ONE: one query per sequence (Q == 1), which then needs no loop: the query
// channel, loaded before the key row, is waited for alone.
template <int FMT, bool ONE>
__global__ __launch_bounds__(256) void k_scan(const uint8_t* __restrict__ ikc,
                                              const float* __restrict__ iks, int64_t cap, int Q,
                                              const float* __restrict__ iq,
                                              const float* __restrict__ iw,
                                              const int32_t* __restrict__ n_vis,
                                              uint32_t* __restrict__ keys,
                                              uint32_t* __restrict__ bkeys,
                                              uint32_t* __restrict__ sbkeys) {
    __shared__ __attribute__((aligned(16))) float sq[kIdxHeads * kIdxDim];
    __shared__ float sw[kIdxHeads];
    const int b = blockIdx.y;
    // h is the wave's index: taken as wave-uniform, the head weights load
    // through the scalar cache and no vector wait orders them
    const int lane = threadIdx.x & 63, h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t p0 = (int64_t)blockIdx.x * 256;
    const int64_t p = p0 + threadIdx.x;
    int nv_max = 0;
    for (int q = 0; q < Q; ++q) nv_max = max(nv_max, clamp_nvis(n_vis[(int64_t)b * Q + q], cap));
    if (p0 >= nv_max) return;  // uniform over the block
    // cap is a multiple of 64, so a wave is either wholly inside or wholly
    // past it; a wave past it takes part in the query set-up only
    const bool live = p0 + (threadIdx.x & ~63) < cap;

    // loads complete in issue order: the first query's channel and weight
    // (from L2), then the key row (a wave past cap reads the sequence's first
    // rows and scores nothing)
    float x = iq[((int64_t)b * Q * kIdxHeads + h) * kIdxDim + lane];
    float wh = iw[(int64_t)b * Q * kIdxHeads + h];
    __builtin_amdgcn_sched_barrier(0);  // keep the channel's load ahead of the row's
    IdxRow<FMT> r;
    r.load(ikc, iks, (int64_t)b * cap + (live ? p : lane));
    const int64_t nb = cap / kBlock;
    // one query: quantise it in the workgroup, score the row, write the keys
    const auto one_query = [&](int64_t bq, int nv, float xq, float wq) {
        float sqh;
        sq[h * kIdxDim + lane] = quantise_query_channel(xq, sqh);
        if (lane == 0) sw[h] = wq * sqh;
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);  // the row is decoded after the barrier
        if (!live) return;  // uniform over the wave
        QQuad qq;
        qq.load(sq);
        const float s = r.score(qq, sw);  // every lane of the wave is active
        const uint32_t key = (p < nv) ? score_key(s) : 0u;
        keys[bq * cap + p] = key;
        const uint32_t bk = max8_u32(key);
        if ((threadIdx.x & 7) == 0) bkeys[bq * nb + (p >> 3)] = bk;
        if (sbkeys != nullptr) {
            const uint32_t sk = wave_max_of_groups8(bk);
            if ((threadIdx.x & 63) == 0) sbkeys[bq * (cap / kSuper) + (p / kSuper)] = sk;
        }
    };
    if constexpr (ONE) {
        one_query(b, nv_max, x, wh);  // p0 < nv_max, the one query's count
        return;
    }
    for (int q = 0; q < Q; ++q) {
        const int64_t bq = (int64_t)b * Q + q;
        const int nv = clamp_nvis(n_vis[bq], cap);
        if (p0 >= nv) continue;  // uniform over the block
        if (q > 0) {
            x = iq[(bq * kIdxHeads + h) * kIdxDim + lane];
            wh = iw[bq * kIdxHeads + h];
            __syncthreads();  // the previous query's readers are done
        }
        one_query(bq, nv, x, wh);
    }
}

// ---------------------------------------------------------------------------
// Full-layer scan for many queries per sequence (the replay chunk).  Same
// scores, bit for bit, as k_scan; the position's key row is converted to fp32
// once and the queries are staged in LDS, 32 at a time, so every lane reads the
// query values as LDS broadcasts.  grid = (ceil(cap / 256), B), 256 threads.
// ---------------------------------------------------------------------------
constexpr int kScanQChunk = 32;

__global__ __launch_bounds__(256) void k_scan_multi(const uint8_t* __restrict__ ikc,
                                                    const float* __restrict__ iks, int64_t cap,
                                                    int Q, const float* __restrict__ qd,
                                                    const float* __restrict__ wq,
                                                    const int32_t* __restrict__ n_vis,
                                                    uint32_t* __restrict__ keys,
                                                    uint32_t* __restrict__ bkeys,
                                                    uint32_t* __restrict__ sbkeys) {
    __shared__ __attribute__((aligned(16))) float sq[kScanQChunk * kIdxHeads * kIdxDim];
    __shared__ float sw[kScanQChunk * kIdxHeads];
    __shared__ int red[4];
    const int b = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * 256;
    const int64_t p = p0 + threadIdx.x;
    const int nv_max = workgroup_nv_max(n_vis, b, Q, cap, red);
    if (p0 >= nv_max) return;  // uniform over the block
    // cap is a multiple of 64: a wave is wholly inside or wholly past it; waves
    // past it still take part in the barriers below
    const bool live = p0 + (threadIdx.x & ~63) < cap;

    float kf[kIdxDim];
    float sigma = 0.0f;
    if (live) {
        const int64_t row = (int64_t)b * cap + p;
        uint4 raw[4];
        load_ik_row(ikc, row, raw);
        sigma = iks[row];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t w[4] = {raw[g].x, raw[g].y, raw[g].z, raw[g].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float2 lo = e4m3x2_to_f32<false>(w[i]);
                const float2 hi = e4m3x2_to_f32<true>(w[i]);
                kf[16 * g + 4 * i + 0] = lo.x;
                kf[16 * g + 4 * i + 1] = lo.y;
                kf[16 * g + 4 * i + 2] = hi.x;
                kf[16 * g + 4 * i + 3] = hi.y;
            }
        }
    }
    const int64_t nb = cap / kBlock;
    for (int q0 = 0; q0 < Q; q0 += kScanQChunk) {
        const int nq = min(kScanQChunk, Q - q0);
        __syncthreads();  // the previous chunk's readers are done
        const float* src = qd + ((int64_t)b * Q + q0) * kIdxHeads * kIdxDim;
        for (int i = threadIdx.x; i < nq * kIdxHeads * kIdxDim / 4; i += 256)
            reinterpret_cast<float4*>(sq)[i] = reinterpret_cast<const float4*>(src)[i];
        if (threadIdx.x < nq * kIdxHeads)
            sw[threadIdx.x] = wq[((int64_t)b * Q + q0) * kIdxHeads + threadIdx.x];
        __syncthreads();
        if (!live) continue;
        for (int j = 0; j < nq; ++j) {
            const int64_t bq = (int64_t)b * Q + q0 + j;
            const int nv = clamp_nvis(n_vis[bq], cap);
            if (p0 >= nv) continue;  // uniform
            // the sequence of IEEE operations of score_row
            float t = 0.0f;
#pragma unroll
            for (int h = 0; h < kIdxHeads; ++h) {
                const float4* qh = reinterpret_cast<const float4*>(sq + (j * kIdxHeads + h) * kIdxDim);
                float dot = 0.0f;
#pragma unroll
                for (int c4 = 0; c4 < kIdxDim / 4; ++c4) {
                    const float4 qv = qh[c4];
                    dot = fmaf(qv.x, kf[4 * c4 + 0], dot);
                    dot = fmaf(qv.y, kf[4 * c4 + 1], dot);
                    dot = fmaf(qv.z, kf[4 * c4 + 2], dot);
                    dot = fmaf(qv.w, kf[4 * c4 + 3], dot);
                }
                const float r = dot > 0.0f ? dot : 0.0f;
                const float wr = sw[j * kIdxHeads + h] * r;
                t = (h == 0) ? wr : t + wr;
            }
            const float score = sigma * t;
            const uint32_t key = (p < nv) ? score_key(score) : 0u;
            keys[bq * cap + p] = key;
            const uint32_t bk = max8_u32(key);
            if ((threadIdx.x & 7) == 0) bkeys[bq * nb + (p >> 3)] = bk;
            if (sbkeys != nullptr) {
                const uint32_t sk = wave_max_of_groups8(bk);
                if ((threadIdx.x & 63) == 0) sbkeys[bq * (cap / kSuper) + (p / kSuper)] = sk;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Wave-wide scans and reductions of uint32 values (whole wave active).
// ---------------------------------------------------------------------------
// inclusive prefix sum over the 64 lanes (DPP row shifts, then row broadcasts)
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row_bcast:31
    return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v), 63);
}

template <class OP>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, OP op) {
    v = op(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    v = op(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    v = op(v, dpp<0x141>(v));  // row_half_mirror
    v = op(v, dpp<0x140>(v));  // row_mirror
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return op(op(r0, r1), op(r2, r3));
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// ---------------------------------------------------------------------------
// Reindex: score the positions of the pool blocks with the layer's own query.
// grid = (ceil(P*8 / 256), B*Q), 256 threads.  Slot s of query bq is position
// pool[j]*8 + (s & 7) with j = s / 8; invisible or empty slots get key 0.
// The eight lanes of one block read 8 x 16 contiguous bytes per plane.
// Each workgroup quantises its query itself (wave h: head h, E4M3 codes
// decoded back to fp32 in LDS, w' = w * sq), while its row loads are in
// flight; every lane then takes its quad of q values from LDS into registers.
// With `parts`, each wave also writes a summary of its 64 keys for the
// selection that follows: the largest key of each of its four groups of 16
// slots (0: none visible) at parts[bq * nw + s / 64], nw = ceil(P*8 / 64).
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(256) void k_pool_score(const uint8_t* __restrict__ ikc,
                                                    const float* __restrict__ iks, int64_t cap,
                                                    int Q, const float* __restrict__ iq,
                                                    const float* __restrict__ iw,
                                                    const int32_t* __restrict__ n_vis,
                                                    const int32_t* __restrict__ pool, int P,
                                                    uint32_t* __restrict__ ckeys,
                                                    uint4* __restrict__ parts) {
    __shared__ __attribute__((aligned(16))) float sq[kIdxHeads * kIdxDim];
    __shared__ float sw[kIdxHeads];
    const int64_t bq = blockIdx.y;
    const int64_t b = bq / Q;
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n_slots = (int64_t)P * kBlock;
    // Loads complete in issue order.  The query's values and weight go out
    // with the slot's block, and every lane then loads a key row (a slot past
    // the pool or outside the visible positions reads the sequence's first
    // row and is not scored), so the quantisation below waits for nothing
    // and runs while the rows are in flight.
    const int lane = threadIdx.x & 63, h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float x = iq[(bq * kIdxHeads + h) * kIdxDim + lane];
    const float wh = iw[bq * kIdxHeads + h];
    const int nv = clamp_nvis(n_vis[bq], cap);
    const int32_t blk = pool[bq * P + (s < n_slots ? (s >> 3) : 0)];
    const int64_t pos = (int64_t)blk * kBlock + (s & 7);
    const bool valid = s < n_slots && blk >= 0 && pos < nv;
    IdxRow<FMT> r;
    r.load(ikc, iks, b * cap + (valid ? pos : 0));
    {   // the query's E4M3 codes (exact fp32 values) and folded weights
        float sqh;
        sq[h * kIdxDim + lane] = quantise_query_channel(x, sqh);
        if (lane == 0) sw[h] = wh * sqh;
    }
    __syncthreads();
    // nothing of the row is decoded before the barrier: a wave waits for its
    // own rows only, not for the slowest wave's
    __builtin_amdgcn_sched_barrier(0);
    // every lane scores (with the whole wave active), the absent ones are dropped
    QQuad qq;
    qq.load(sq);
    const float sc = r.score(qq, sw);
    const uint32_t key = valid ? score_key(sc) : 0u;
    if (s < n_slots) ckeys[bq * n_slots + s] = key;
    if (parts != nullptr) {  // every lane of a 16-lane row ends with the row's maximum
        uint32_t m = max(key, dpp<0xB1>(key));
        m = max(m, dpp<0x4E>(m));
        m = max(m, dpp<0x141>(m));
        m = max(m, dpp<0x140>(m));
        const int64_t nw = (n_slots + 63) / 64, wv = (int64_t)blockIdx.x * 4 + h;
        if ((lane & 15) == 0 && wv < nw)
            reinterpret_cast<uint32_t*>(parts)[(bq * nw + wv) * 4 + (lane >> 4)] = m;
    }
}

// ---------------------------------------------------------------------------
// Exact top-K selection, one workgroup of 1024 threads per query.
//
// Slots are numbered in ascending index order; key 0 marks an empty slot.
// The K-th largest key T is found by range refinement: a min/max pass, then
// up to three histogram passes, each splitting the current key interval
// [lo, hi] into at most 2048 equal bins (bins follow the keys' actual range,
// so a narrow score distribution does not pile every key into one LDS bin)
// and keeping the bin that holds the K-th largest.  Output: every slot with
// key > T, then the lowest-numbered slots with key == T until K are taken,
// written in ascending slot order (ties go to the lowest position or block);
// fewer than K non-empty slots: all of them; the rest of the row is -1.
//
// Up to 16384 slots are held in registers (16 per thread); larger counts are
// streamed: wave w owns a contiguous range, lane l the slots range_begin +
// 64 i + l, re-read from memory on every pass.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelRegSlots = 16384;             // slots held in registers
constexpr int kSelBins = 2048;
static_assert(kSelBins >= kMaxTopk, "the histogram area stages a top-K row");

struct SelShared {
    // also holds the register path's state (SelRegShared)
    alignas(16) uint32_t hist[kSelBins + 5 * kSelWaves + 4];
    uint32_t keys[1];  // unused by the streaming path (keys are re-read)
    int32_t pool[kMaxPoolBlocks];
    uint32_t red[3][kSelWaves];
    uint32_t wgt[kSelWaves], weq[kSelWaves];
    uint32_t pick[2];
};

// key of slot s: block keys, position keys gathered through the pool, or a
// compact pool-ordered array
struct KeySrc {
    const uint32_t* src;
    const int32_t* pool;  // LDS, sanitised (-1 = empty)
    int64_t n;
    int nv;
    int kind;             // 0 direct, 1 gather through pool, 2 compact (pool order)
    __device__ __forceinline__ uint32_t key(int64_t s) const {
        if (kind == 1) {
            const int32_t blk = pool[s >> 3];
            const int64_t pos = (int64_t)blk * kBlock + (s & 7);
            return (blk >= 0 && pos < nv) ? src[pos] : 0u;
        }
        return src[s];
    }
    __device__ __forceinline__ int32_t index(int64_t s) const {
        return kind == 0 ? (int32_t)s : pool[s >> 3] * kBlock + (int32_t)(s & 7);
    }
    // keys of the 16 slots s0 .. s0 + 15 (s0 a multiple of 16; 0 past n)
    __device__ __forceinline__ void load16(int64_t s0, uint32_t (&k)[16]) const {
        if (kind == 1) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t sb = s0 + 8 * j;
                const int32_t blk = sb < n ? pool[sb >> 3] : -1;
                const int64_t pos = (int64_t)blk * kBlock;
                if (blk >= 0 && pos + kBlock <= nv) {
                    const uint4 a = *reinterpret_cast<const uint4*>(src + pos);
                    const uint4 b = *reinterpret_cast<const uint4*>(src + pos + 4);
                    k[8 * j + 0] = a.x; k[8 * j + 1] = a.y; k[8 * j + 2] = a.z; k[8 * j + 3] = a.w;
                    k[8 * j + 4] = b.x; k[8 * j + 5] = b.y; k[8 * j + 6] = b.z; k[8 * j + 7] = b.w;
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        k[8 * j + i] = (blk >= 0 && pos + i < nv) ? src[pos + i] : 0u;
                }
            }
        } else if (s0 + 16 <= n) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 a = *reinterpret_cast<const uint4*>(src + s0 + 4 * j);
                k[4 * j + 0] = a.x; k[4 * j + 1] = a.y; k[4 * j + 2] = a.z; k[4 * j + 3] = a.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) k[i] = s0 + i < n ? src[s0 + i] : 0u;
        }
    }
};

struct SelRange {
    int64_t beg, end;  // this wave's slots
};

__device__ __forceinline__ SelRange wave_range(int64_t n, int wave) {
    const int64_t chunk = ((n + kSelWaves - 1) / kSelWaves + 63) / 64 * 64;
    SelRange r;
    r.beg = min(n, (int64_t)wave * chunk);
    r.end = min(n, r.beg + chunk);
    return r;
}

// Visit this thread's keys in ascending slot order, the same trip count in
// every lane of a wave: f(key, slot, in_range).  CACHED: keys come from LDS.
template <bool CACHED, class F>
__device__ __forceinline__ void for_keys(const KeySrc& ks, const uint32_t* cache,
                                         const SelRange& r, int lane, F f) {
    for (int64_t base = r.beg; base < r.end; base += 64) {
        const int64_t s = base + lane;
        const bool in = s < r.end;
        f(in ? (CACHED ? cache[s] : ks.key(s)) : 0u, s, in);
    }
}

struct Threshold {
    uint32_t t_ge;   // every key >= t_ge is taken
    uint32_t t_eq;   // plus the first `quota` keys equal to t_eq
    uint32_t quota;
    uint32_t total;  // number taken
};

// What a selection may know of its keys beforehand: at least K non-zero keys
// lie at or above lo and none lies above hi.  lo == 0: nothing is known.
struct KeyBound {
    uint32_t lo, hi;
};

template <bool REG>
__device__ __forceinline__ Threshold find_threshold(const KeySrc& ks, const uint32_t* reg,
                                    const SelRange& r, int K, SelShared& sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // count, min and max of the non-empty keys
    uint32_t cnt = 0, kmin = 0xFFFFFFFFu, kmax = 0;
    for_keys<REG>(ks, reg, r, lane, [&](uint32_t k, int64_t, bool) {
        if (k) { ++cnt; kmin = min(kmin, k); kmax = max(kmax, k); }
    });
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        cnt += __shfl_xor(cnt, off, 64);
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off, 64));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off, 64));
    }
    if (lane == 0) { sh.red[0][wave] = cnt; sh.red[1][wave] = kmin; sh.red[2][wave] = kmax; }
    __syncthreads();
    cnt = 0; kmin = 0xFFFFFFFFu; kmax = 0;
    for (int w = 0; w < kSelWaves; ++w) {
        cnt += sh.red[0][w];
        kmin = min(kmin, sh.red[1][w]);
        kmax = max(kmax, sh.red[2][w]);
    }
    if (cnt <= (uint32_t)K) return Threshold{1u, 0u, 0u, cnt};

    uint32_t lo = kmin, hi = kmax, remaining = (uint32_t)K;
    for (int pass = 0; pass < 4; ++pass) {
        const uint32_t width = hi - lo;
        if (width == 0) return Threshold{lo + 1, lo, remaining, (uint32_t)K};
        const int bits = 32 - __clz((int)width);
        const int shift = bits > 11 ? bits - 11 : 0;
        const int nbins = (int)(width >> shift) + 1;
        __syncthreads();  // previous readers of hist are done
        for (int i = tid; i < nbins; i += kSelThreads) sh.hist[i] = 0;
        __syncthreads();
        for_keys<REG>(ks, reg, r, lane, [&](uint32_t k, int64_t, bool) {
            if (k >= lo && k <= hi) atomicAdd(&sh.hist[(k - lo) >> shift], 1u);
        });
        __syncthreads();
        if (wave == 0) {
            // lane l scans bins nbins-1-32l .. nbins-32-32l (descending)
            uint32_t loc = 0;
            for (int j = 0; j < 32; ++j) {
                const int bin = nbins - 1 - 32 * lane - j;
                loc += bin >= 0 ? sh.hist[bin] : 0u;
            }
            uint32_t incl = loc;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_up(incl, off, 64);
                if (lane >= off) incl += y;
            }
            uint32_t above = incl - loc;
            if (above < remaining && incl >= remaining) {  // the bin is in this lane's run
                for (int j = 0; j < 32; ++j) {
                    const int bin = nbins - 1 - 32 * lane - j;
                    const uint32_t h = sh.hist[bin];
                    if (above + h >= remaining) {
                        sh.pick[0] = (uint32_t)bin;
                        sh.pick[1] = above;
                        break;
                    }
                    above += h;
                }
            }
        }
        __syncthreads();
        const uint32_t d = sh.pick[0], above = sh.pick[1];
        const uint32_t in_bin = sh.hist[d];
        remaining -= above;
        const uint32_t new_lo = lo + (d << shift);
        const uint32_t span = (shift == 0) ? 0u : ((1u << shift) - 1u);
        const uint32_t new_hi = (hi - new_lo > span) ? new_lo + span : hi;
        if (in_bin == remaining) return Threshold{new_lo, 0u, 0u, (uint32_t)K};
        lo = new_lo;
        hi = new_hi;
    }
    return Threshold{lo + 1, lo, remaining, (uint32_t)K};  // not reached: width hits 0
}

// Write the selected indices of this query in ascending slot order; the
// rest of out[0, K) becomes -1.  When `lds_out` is set, also mirror them there.
template <bool REG>
__device__ __forceinline__ void compact(const KeySrc& ks, const uint32_t* reg, const SelRange& r,
                        const Threshold& th, int K, int32_t* out, int32_t* lds_out,
                        SelShared& sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t c_gt = 0, c_eq = 0;
    for_keys<REG>(ks, reg, r, lane, [&](uint32_t k, int64_t, bool) {
        c_gt += __popcll(__ballot(k != 0 && k >= th.t_ge));
        c_eq += __popcll(__ballot(k != 0 && th.quota != 0 && k == th.t_eq));
    });
    __syncthreads();
    if (lane == 0) { sh.wgt[wave] = c_gt; sh.weq[wave] = c_eq; }
    __syncthreads();
    uint32_t eq_before = 0, out_before = 0, total = 0, eb = 0;
    for (int w = 0; w < kSelWaves; ++w) {
        const uint32_t take_eq = th.quota > eb ? min(th.quota - eb, sh.weq[w]) : 0u;
        if (w == wave) { eq_before = eb; out_before = total; }
        total += sh.wgt[w] + take_eq;
        eb += sh.weq[w];
    }
    uint32_t eq_seen = 0, taken = 0;
    for_keys<REG>(ks, reg, r, lane, [&](uint32_t k, int64_t s, bool) {
        const bool gt = k != 0 && k >= th.t_ge;
        const bool eq = k != 0 && th.quota != 0 && k == th.t_eq;
        const uint64_t eq_mask = __ballot(eq);
        const uint32_t eq_rank = eq_before + eq_seen +
            __builtin_amdgcn_mbcnt_hi((uint32_t)(eq_mask >> 32),
                                      __builtin_amdgcn_mbcnt_lo((uint32_t)eq_mask, 0));
        const bool take = gt || (eq && eq_rank < th.quota);
        const uint64_t tk_mask = __ballot(take);
        const uint32_t rank = out_before + taken +
            __builtin_amdgcn_mbcnt_hi((uint32_t)(tk_mask >> 32),
                                      __builtin_amdgcn_mbcnt_lo((uint32_t)tk_mask, 0));
        if (take && rank < (uint32_t)K) {
            const int32_t idx = ks.index(s);
            if (out) out[rank] = idx;
            if (lds_out) lds_out[rank] = idx;
        }
        eq_seen += __popcll(eq_mask);
        taken += __popcll(tk_mask);
    });
    for (int64_t i = (int64_t)total + tid; i < K; i += kSelThreads) {
        if (out) out[i] = -1;
        if (lds_out) lds_out[i] = -1;
    }
}

// ---------------------------------------------------------------------------
// Register path (at most 16384 slots): lane l of wave w holds the keys of the
// 16 consecutive slots w*1024 + 16 l .. +15, so its keys load as 16-byte
// vectors, wave-wide sums are DPP scans, the bin search is spread over all
// 1024 threads, and output ranks follow from per-lane prefix counts (slot
// order is lane order within a wave).
// ---------------------------------------------------------------------------
constexpr int kSelKpt = 16;

// One counter per bin.  (Spreading a bin over four counters picked by lane,
// so that lanes of one atomic instruction landing in one bin hit different
// words, cost more in clearing and summing than it saved: 25.2 against
// 24.3 us per Full-layer selection.)
struct SelRegShared {
    alignas(16) uint32_t hist[kSelBins];
    alignas(16) uint32_t part[5][kSelWaves];
    uint32_t pick[4];
};
static_assert(sizeof(SelRegShared) <= sizeof(SelShared::hist), "register state fits the histogram area");

// One range-refinement pass: the N values per thread that lie in [lo, hi]
// are counted into at most 2048 equal bins (with skip_lowest, values in the
// lowest bin are not counted: the caller knows in_range, the number of values
// in [lo, hi], so that bin's count is in_range minus the others), and the bin
// that holds the remaining-th largest is picked: its index, the count above
// it and its own count.  With second != 0 (and skip_lowest false), the bin
// that holds the second-th largest is picked as well (bin2; second <=
// remaining, so it exists whenever the first does).
struct BinPick {
    uint32_t bin, before, in_bin, bin2;
    int shift;
};

template <int N>
__device__ __forceinline__ BinPick hist_pick(const uint32_t (&v)[N], uint32_t lo, uint32_t hi,
                                             uint32_t remaining, bool skip_lowest,
                                             uint32_t in_range, SelRegShared& sh,
                                             uint32_t second = 0u) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t width = hi - lo;  // > 0
    const int bits = 32 - __clz((int)width);
    const int shift = bits > 11 ? bits - 11 : 0;
    const int nbins = (int)(width >> shift) + 1;
    const uint32_t first = skip_lowest ? lo + (1u << shift) : lo;  // smallest value counted
    __syncthreads();  // earlier readers of hist / part / pick are done
    static_assert(kSelBins == 2 * kSelThreads, "one 8-byte clear per thread");
    reinterpret_cast<uint2*>(sh.hist)[tid] = make_uint2(0u, 0u);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (v[i] >= first && v[i] <= hi && v[i] != 0)
            atomicAdd(&sh.hist[(v[i] - lo) >> shift], 1u);
    __syncthreads();
    // thread t owns bins nbins-1-2t and nbins-2-2t (descending order)
    const int b0 = nbins - 1 - 2 * tid, b1 = b0 - 1;
    uint32_t h0 = b0 >= 0 ? sh.hist[b0] : 0u, h1 = b1 >= 0 ? sh.hist[b1] : 0u;
    uint32_t mine = h0 + h1;  // a skipped lowest bin counts 0 here: it is last in the order
    const uint32_t incl = wave_incl_scan(mine);
    if (lane == 63) sh.part[0][wave] = incl;
    __syncthreads();
    uint32_t above = incl - mine;
    {
        static_assert(kSelWaves == 16, "per-wave totals read as four uint4");
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 x = reinterpret_cast<const uint4*>(sh.part[0])[j];
            above += (4 * j + 0 < wave ? x.x : 0u) + (4 * j + 1 < wave ? x.y : 0u) +
                     (4 * j + 2 < wave ? x.z : 0u) + (4 * j + 3 < wave ? x.w : 0u);
        }
    }
    if (skip_lowest) {  // the lowest bin's count: the values in range not in any other bin
        if (b0 == 0) h0 = in_range - above;
        if (b1 == 0) h1 = in_range - above - h0;
        mine = h0 + h1;
    }
    if (above < remaining && above + mine >= remaining) {
        if (above + h0 >= remaining) { sh.pick[0] = (uint32_t)b0; sh.pick[1] = above; sh.pick[2] = h0; }
        else { sh.pick[0] = (uint32_t)b1; sh.pick[1] = above + h0; sh.pick[2] = h1; }
    }
    if (second != 0u && above < second && above + mine >= second)
        sh.pick[3] = above + h0 >= second ? (uint32_t)b0 : (uint32_t)b1;
    __syncthreads();
    return BinPick{sh.pick[0], sh.pick[1], sh.pick[2], second != 0u ? sh.pick[3] : 0u, shift};
}

// The K-th largest of the workgroup's register keys (16 per thread), as the
// take rule of a Threshold.  The non-zero keys' range [kmin, kmax] is refined
// by 2048-bin histogram passes.  Before them, a pass over group maxima (each
// thread's maximum when K <= 1024, else the maxima of its four groups of four
// keys) finds a lower bound: the lower edge of the bin holding the K-th
// largest group maximum has at least K group maxima, hence at least K keys, at
// or above it, so the K-th largest key is at or above it, and the key passes
// only count keys from there up (a few hundred instead of every key).
// A caller that already holds such a bound (kb.lo != 0) skips the range and
// group-maxima passes.  With second != 0 (second <= K) and `next`, the
// group-maxima pass also yields a bound for the second-th largest key: the
// lower edge of the bin holding the second-th largest group maximum, with
// hi = kmax (next->lo == 0 when that pass did not run).
__device__ __forceinline__ Threshold threshold_reg(const uint32_t (&k)[kSelKpt], int K,
                                                   SelRegShared& sh, KeyBound kb = {0u, 0u},
                                                   uint32_t second = 0u,
                                                   KeyBound* next = nullptr) {
    if (next != nullptr) *next = KeyBound{0u, 0u};
    uint32_t lo = kb.lo, hi = kb.hi;
    bool known = false;  // in_range is the count of keys in [lo, hi]
    uint32_t in_range = 0;
    if (kb.lo == 0u) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        uint32_t cnt = 0, kmin = 0xFFFFFFFFu, kmax = 0;
        uint32_t gm[4];  // maxima of the four groups of four keys
#pragma unroll
        for (int j = 0; j < 4; ++j) gm[j] = max(max(k[4 * j], k[4 * j + 1]), max(k[4 * j + 2], k[4 * j + 3]));
#pragma unroll
        for (int i = 0; i < kSelKpt; ++i) {
            cnt += k[i] != 0;
            kmin = k[i] ? min(kmin, k[i]) : kmin;
        }
        kmax = max(max(gm[0], gm[1]), max(gm[2], gm[3]));
        uint32_t ngm1 = kmax != 0, ngm4 = (gm[0] != 0) + (gm[1] != 0) + (gm[2] != 0) + (gm[3] != 0);
        cnt = wave_sum(cnt);
        ngm1 = wave_sum(ngm1);
        ngm4 = wave_sum(ngm4);
        kmin = wave_reduce(kmin, [](uint32_t x, uint32_t y) { return min(x, y); });
        kmax = wave_reduce(kmax, [](uint32_t x, uint32_t y) { return max(x, y); });
        __syncthreads();  // earlier readers of part are done
        if (lane == 0) {
            sh.part[0][wave] = cnt; sh.part[1][wave] = kmin; sh.part[2][wave] = kmax;
            sh.part[3][wave] = ngm1; sh.part[4][wave] = ngm4;
        }
        __syncthreads();
        cnt = 0; kmin = 0xFFFFFFFFu; kmax = 0; ngm1 = 0; ngm4 = 0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) {
            cnt += sh.part[0][w];
            kmin = min(kmin, sh.part[1][w]);
            kmax = max(kmax, sh.part[2][w]);
            ngm1 += sh.part[3][w];
            ngm4 += sh.part[4][w];
        }
        if (cnt <= (uint32_t)K) return Threshold{1u, 0u, 0u, cnt};

        lo = kmin;
        hi = kmax;
        known = true;
        in_range = cnt;
        if (kmax > kmin && (K <= 1024 ? ngm1 : ngm4) >= (uint32_t)K) {
            BinPick bp;
            if (K <= 1024) {
                const uint32_t t1[1] = {max(max(gm[0], gm[1]), max(gm[2], gm[3]))};
                bp = hist_pick(t1, lo, hi, (uint32_t)K, false, 0u, sh, second);
            } else {
                bp = hist_pick(gm, lo, hi, (uint32_t)K, false, 0u, sh, second);
            }
            if (second != 0u && next != nullptr) *next = KeyBound{lo + (bp.bin2 << bp.shift), hi};
            lo = lo + (bp.bin << bp.shift);
            known = lo == kmin;
        }
    }
    uint32_t remaining = (uint32_t)K;
    for (int pass = 0; pass < 4; ++pass) {
        const uint32_t width = hi - lo;
        if (width == 0) return Threshold{lo + 1, lo, remaining, (uint32_t)K};
        const BinPick bp = hist_pick(k, lo, hi, remaining, known, in_range, sh);
        remaining -= bp.before;
        const uint32_t new_lo = lo + (bp.bin << bp.shift);
        const uint32_t span = (bp.shift == 0) ? 0u : ((1u << bp.shift) - 1u);
        const uint32_t new_hi = (hi - new_lo > span) ? new_lo + span : hi;
        if (bp.in_bin == remaining) return Threshold{new_lo, 0u, 0u, (uint32_t)K};
        lo = new_lo;
        hi = new_hi;
        in_range = bp.in_bin;
        known = true;
    }
    return Threshold{lo + 1, lo, remaining, (uint32_t)K};  // not reached: width hits 0
}

// unsigned minimum the optimiser cannot reason about (see compact_reg)
__device__ __forceinline__ uint32_t umin_opaque(uint32_t a, uint32_t b) {
    uint32_t r;
    asm volatile("v_min_u32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// exclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v) { return wave_incl_scan(v) - v; }

// Keys above the threshold are all taken; keys equal to it are taken in slot
// order until the quota is met.  With an LDS copy requested (`lds_out`), the
// indices are ranked into it and then written out in one coalesced pass;
// otherwise each lane writes its ranks straight to `out`.
template <class IDX>
__device__ __forceinline__ void compact_reg(const uint32_t (&k)[kSelKpt], const Threshold& th,
                                            int K, IDX index_of, int32_t* out, int32_t* lds_out,
                                            SelRegShared& sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int32_t* stage = lds_out ? lds_out : reinterpret_cast<int32_t*>(sh.hist);
    uint32_t gtm = 0, eqm = 0;
#pragma unroll
    for (int i = 0; i < kSelKpt; ++i) {
        gtm |= (k[i] != 0 && k[i] >= th.t_ge) ? (1u << i) : 0u;
        eqm |= (k[i] != 0 && th.quota != 0 && k[i] == th.t_eq) ? (1u << i) : 0u;
    }
    const uint32_t n_gt = __popc(gtm), n_eq = __popc(eqm);
    const uint32_t gt_lane = wave_excl_scan(n_gt), eq_lane = wave_excl_scan(n_eq);
    __syncthreads();  // the threshold search is done with hist / part
    if (lane == 63) { sh.part[0][wave] = gt_lane + n_gt; sh.part[1][wave] = eq_lane + n_eq; }
    __syncthreads();
    uint32_t gt_before = 0, eq_before = 0, gt_total = 0, eq_total = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const uint32_t a = sh.part[0][w], b = sh.part[1][w];
        gt_before += w < wave ? a : 0u;
        eq_before += w < wave ? b : 0u;
        gt_total += a;
        eq_total += b;
    }
    const uint32_t eq_off = eq_before + eq_lane;  // equal keys in earlier slots
    // Equal keys are taken in slot order until the quota is met: this lane
    // takes min(q, eq_off + n_eq) - min(q, eq_off) of them, after
    // min(q, eq_off) taken in earlier slots.  The minima are explicit
    // v_min_u32: with plain min() and a comparison here, this compiler
    // (ROCm 7.2 clang, gfx950) folded both as if eq_off <= q always held,
    // which mis-ranks the keys after an untaken tie.
    const uint32_t eq_taken_before = umin_opaque(th.quota, eq_off);
    uint32_t eq_take = umin_opaque(th.quota, eq_off + n_eq) - eq_taken_before;
    uint32_t rank = gt_before + gt_lane + eq_taken_before;
    const uint32_t total = gt_total + umin_opaque(th.quota, eq_total);
    // taken slots: every key above the threshold plus the first eq_take
    // equal ones; visit only the set bits (a wave loops as often as its
    // busiest lane takes keys)
    uint32_t takem = gtm, em = eqm;
    for (; eq_take != 0 && em != 0; --eq_take) {
        takem |= em & (0u - em);
        em &= em - 1u;
    }
    if (lds_out == nullptr) {  // global row only: write each rank where it goes
        while (takem != 0) {
            const int i = __builtin_ctz(takem);
            if (rank < (uint32_t)K) out[rank] = index_of(wave * 1024 + 16 * lane + i);
            ++rank;
            takem &= takem - 1u;
        }
        for (int i = (int)total + tid; i < K; i += kSelThreads) out[i] = -1;
        return;
    }
    while (takem != 0) {
        const int i = __builtin_ctz(takem);
        if (rank < (uint32_t)K) stage[rank] = index_of(wave * 1024 + 16 * lane + i);
        ++rank;
        takem &= takem - 1u;
    }
    // one coalesced pass writes the row
    __syncthreads();
    for (int i = tid; i < K; i += kSelThreads) {
        const int32_t v = i < (int)total ? stage[i] : -1;
        if (out) out[i] = v;
        if (lds_out) lds_out[i] = v;
    }
}

// The K-th largest of the workgroup's register keys (threshold_reg's result
// th): the tie value, else the smallest key at or above the cut; 1 when fewer
// than K keys are non-zero.  red: kSelWaves words of LDS.
__device__ __forceinline__ uint32_t kth_key_reg(const uint32_t (&k)[kSelKpt], const Threshold& th,
                                                int K, uint32_t* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t m = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < kSelKpt; ++i) m = (k[i] != 0 && k[i] >= th.t_ge) ? min(m, k[i]) : m;
    m = wave_reduce(m, [](uint32_t a, uint32_t b) { return min(a, b); });
    __syncthreads();  // earlier readers of red are done
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) m = min(m, red[w]);
    return th.total < (uint32_t)K ? 1u : (th.quota != 0 ? th.t_eq : m);
}

// Select through the register path when the slot count allows it, else the
// streaming path.  `ks` gives keys and indices of slots; kb, second and next
// as for threshold_reg (the streaming path takes no bound and yields none).
__device__ __forceinline__ void select_into(const KeySrc& ks, int K, int32_t* out, int32_t* lds_out,
                                            SelShared& sh, KeyBound kb = {0u, 0u},
                                            uint32_t second = 0u, KeyBound* next = nullptr) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (ks.n <= kSelRegSlots) {
        uint32_t k[kSelKpt];
        ks.load16((int64_t)wave * 1024 + 16 * lane, k);
        SelRegShared& rs = *reinterpret_cast<SelRegShared*>(&sh.hist[0]);
        const Threshold th = threshold_reg(k, K, rs, kb, second, next);
        compact_reg(k, th, K, [&](int64_t s) { return ks.index(s); }, out, lds_out, rs);
    } else {
        if (next != nullptr) *next = KeyBound{0u, 0u};
        const SelRange r = wave_range(ks.n, wave);
        const Threshold th = find_threshold<false>(ks, sh.keys, r, K, sh);
        compact<false>(ks, sh.keys, r, th, K, out, lds_out, sh);
    }
}

// Blocks too many for the register path (more than 16384, e.g. a 1M-position
// context): with x the P-th largest superblock key (max over 8 blocks), P
// distinct superblocks each hold a block whose key is >= x, so the P-th
// largest block key is >= x and every block of the pool lies in a superblock
// whose key reaches x.  Those superblocks, in ascending order (at most 2048,
// so their 16384 block keys fit the register path), give the pool with the
// same ranking and tie rule.  Returns false (nothing selected) when more than
// 2048 superblocks qualify (heavy ties): the caller then streams the blocks.
constexpr int kSuperCand = 2048;
static_assert(2 * kSuperCand <= kMaxPoolBlocks, "pool and superblock list share sh.pool");

__device__ __forceinline__ bool select_blocks_super(const uint32_t* __restrict__ bkeys,
                                                    const uint32_t* __restrict__ sbkeys,
                                                    int64_t nbv, int64_t nsv, int P,
                                                    int32_t* pool_out, SelShared& sh,
                                                    uint32_t second, KeyBound* next) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    SelRegShared& rs = *reinterpret_cast<SelRegShared*>(&sh.hist[0]);
    const KeySrc sup{sbkeys, nullptr, nsv, (int)nsv, 0};
    uint32_t k[kSelKpt];
    sup.load16((int64_t)wave * 1024 + 16 * lane, k);
    const Threshold th = threshold_reg(k, P, rs);
    const uint32_t x = kth_key_reg(k, th, P, sh.red[0]);
    // ordered compaction of the qualifying superblocks (this thread's 16 are
    // consecutive) into the upper half of sh.pool
    uint32_t mask = 0;
#pragma unroll
    for (int i = 0; i < kSelKpt; ++i) mask |= (k[i] != 0 && k[i] >= x) ? (1u << i) : 0u;
    const uint32_t cnt = __popc(mask);
    const uint32_t excl = wave_excl_scan(cnt);
    if (lane == 63) sh.wgt[wave] = excl + cnt;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        before += w < wave ? sh.wgt[w] : 0u;
        total += sh.wgt[w];
    }
    if (total > (uint32_t)kSuperCand) return false;  // uniform
    int32_t* list = sh.pool + kSuperCand;
    uint32_t r = before + excl;
    for (uint32_t mm = mask; mm != 0; mm &= mm - 1u, ++r)
        list[r] = 16 * tid + __builtin_ctz(mm);
    __syncthreads();  // the list is complete
    // block s of the candidates is block 8 list[s / 8] + s % 8 (absent past nbv)
    const KeySrc cand{bkeys, list, (int64_t)total * kBlock, (int)nbv, 1};
    select_into(cand, P, pool_out, sh.pool, sh, KeyBound{0u, 0u}, second, next);
    return true;
}

// Full layer for query bq: best P blocks (pool), then the best K positions
// inside it.  pool_out may be null (internal pool).  sbkeys: null, or the
// scan's superblock keys, used when the blocks do not fit the register path.
// With K <= P, the block selection's group-maxima pass bounds the K-th
// largest block key x from below by some y; the pool holds K blocks whose
// keys are >= x (the P best include the K best), each block key is the key of
// one of its positions, so K positions of the pool have keys >= y, and no
// position key exceeds the largest block key: the position selection starts
// from that bound.
__device__ __forceinline__ void select_full_query(const uint32_t* __restrict__ keys,
                                                  const uint32_t* __restrict__ bkeys, int64_t cap,
                                                  int64_t bq, int nv, int P, int K,
                                                  int32_t* pool_out, int32_t* topk_out,
                                                  SelShared& sh,
                                                  const uint32_t* __restrict__ sbkeys = nullptr) {
    const int64_t nbv = ((int64_t)nv + kBlock - 1) / kBlock;
    const int64_t nsv = ((int64_t)nv + kSuper - 1) / kSuper;
    int32_t* prow = pool_out ? pool_out + bq * P : nullptr;
    bool done = false;
    const uint32_t second = K <= P ? (uint32_t)K : 0u;
    KeyBound nb{0u, 0u};
    if (sbkeys != nullptr && nbv > kSelRegSlots && nsv <= kSelRegSlots && P <= kSuperCand)
        done = select_blocks_super(bkeys + bq * (cap / kBlock), sbkeys + bq * (cap / kSuper), nbv,
                                   nsv, P, prow, sh, second, &nb);
    if (!done) {
        __syncthreads();
        KeySrc blocks{bkeys + bq * (cap / kBlock), nullptr, nbv, nv, 0};
        select_into(blocks, P, prow, sh.pool, sh, KeyBound{0u, 0u}, second, &nb);
    }
    __syncthreads();
    KeySrc pos{keys + bq * cap, sh.pool, (int64_t)P * kBlock, nv, 1};
    select_into(pos, K, topk_out + bq * K, nullptr, sh, nb);
}

__global__ __launch_bounds__(kSelThreads) void k_select_full(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ bkeys, int64_t cap,
    const int32_t* __restrict__ n_vis, int P, int K, int32_t* __restrict__ pool_out,
    int32_t* __restrict__ topk_out, const uint32_t* __restrict__ sbkeys) {
    __shared__ SelShared sh;
    const int64_t bq = blockIdx.x;
    select_full_query(keys, bkeys, cap, bq, clamp_nvis(n_vis[bq], cap), P, K, pool_out, topk_out,
                      sh, sbkeys);
}

// Lower bound of the K-th largest pool key from k_pool_score's wave summaries
// (p: this lane's summaries of waves lane + 64 j, j < 4, valid below nw <=
// 256; each the maxima of four disjoint groups of slots).  A wave whose
// second-largest group maximum is non-zero holds two keys at or above it;
// when such waves number at least K / 2, at least K keys lie at or above the
// smallest of those values, and none above the largest maximum.  Every wave
// reduces all summaries itself (no barrier).
__device__ __forceinline__ KeyBound pool_bound(const uint4 (&p)[4], int nw, int K) {
    const int lane = threadIdx.x & 63;
    uint32_t n2 = 0, lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool in = lane + 64 * j < nw;
        const uint32_t a = max(p[j].x, p[j].y), b = min(p[j].x, p[j].y);
        const uint32_t c = max(p[j].z, p[j].w), d = min(p[j].z, p[j].w);
        const uint32_t second = max(min(a, c), max(b, d));
        const bool two = in && second != 0u;
        n2 += two;
        lo = two ? min(lo, second) : lo;
        hi = in ? max(hi, max(a, c)) : hi;
    }
    n2 = wave_sum(n2);
    lo = wave_reduce(lo, [](uint32_t a, uint32_t b) { return min(a, b); });
    hi = wave_reduce(hi, [](uint32_t a, uint32_t b) { return max(a, b); });
    return 2u * n2 >= (uint32_t)K ? KeyBound{lo, hi} : KeyBound{0u, 0u};
}

// Reindex: best K positions of the compact pool-ordered keys; parts: the
// scoring launch's wave summaries (ceil(P*8 / 64) per query).
__global__ __launch_bounds__(kSelThreads) void k_select_pool(
    const uint32_t* __restrict__ ckeys, const uint4* __restrict__ parts, const int32_t* __restrict__ pool, int P,
    const int32_t* __restrict__ n_vis, int64_t cap, int K, int32_t* __restrict__ topk_out) {
    __shared__ SelShared sh;
    const int64_t bq = blockIdx.x;
    const int nv = clamp_nvis(n_vis[bq], cap);
    const int64_t nbv = ((int64_t)nv + kBlock - 1) / kBlock;
    const KeySrc ks{ckeys + bq * (int64_t)P * kBlock, sh.pool, (int64_t)P * kBlock, nv, 2};
    auto stage_pool = [&]() {
        for (int j = threadIdx.x; j < P; j += kSelThreads) {
            const int32_t blk = pool[bq * P + j];
            sh.pool[j] = (blk >= 0 && blk < nbv) ? blk : -1;
        }
    };
    if (ks.n <= kSelRegSlots) {
        // the wave summaries and the compact keys (which do not go through
        // the pool) are loaded first, and the pool (needed only to name the
        // selected positions) is staged meanwhile; the threshold search's
        // first barrier orders it before compact_reg reads it
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int nw = (P * kBlock + 63) / 64;
        uint4 pw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) pw[j] = parts[bq * nw + (lane + 64 * j < nw ? lane + 64 * j : 0)];
        uint32_t k[kSelKpt];
        ks.load16((int64_t)wave * 1024 + 16 * lane, k);
        stage_pool();
        const KeyBound kb = pool_bound(pw, nw, K);
        SelRegShared& rs = *reinterpret_cast<SelRegShared*>(&sh.hist[0]);
        const Threshold th = threshold_reg(k, K, rs, kb);
        compact_reg(k, th, K, [&](int64_t s) { return ks.index(s); }, topk_out + bq * K, nullptr,
                    rs);
    } else {
        stage_pool();
        __syncthreads();
        select_into(ks, K, topk_out + bq * K, nullptr, sh);
    }
}

// Top-K of one query of the multi-query MFMA scan (csa2_chunk.hip), one
// workgroup per query, from the scan's lower-bound keys per block of 8 and
// upper-bound keys per half-block of 4:
//   1. x = the K-th largest lower-bound block key (1 when fewer than K blocks
//      hold a visible position).  K distinct blocks each hold a position whose
//      exact score is >= x, so every position the exact top-K can take lies
//      in a half-block whose upper-bound key reaches x;
//   2. those candidate half-blocks, in ascending order, are listed in LDS;
//   3. their positions are scored exactly (k_scan's arithmetic, so the keys
//      are bit-identical) into LDS;
//   4. the register-path selection takes the top K there, ties to the lowest
//      position since the slots are in ascending position order.
// A query with more than Pc candidate half-blocks (heavy ties) is scored over
// all its visible positions instead (into keys / bkeys, its own rows) and
// takes the Full layer's selection, K blocks then K positions.
constexpr int kHalf = 4;                               // positions per half-block
constexpr int kChunkMaxCand = 3072;                    // candidate half-blocks held in LDS
constexpr int kChunkSlots = kChunkMaxCand * kHalf;     // 12288 keys
static_assert(kChunkSlots <= kSelRegSlots, "the candidates' keys fit the register path");
static_assert(kChunkMaxCand <= kMaxPoolBlocks, "the candidate list fits sh.pool");

// Ordered compaction: this thread's first rank among the items the threads
// before it hold (`cnt` of its own) and, in `total`, the workgroup's count.
// part: kSelWaves words of LDS (earlier readers are waited for).
__device__ __forceinline__ uint32_t rank_of_count(uint32_t cnt, uint32_t* part, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t excl = wave_excl_scan(cnt);
    __syncthreads();
    if (lane == 63) part[wave] = excl + cnt;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        before += w < wave ? part[w] : 0u;
        total += part[w];
    }
    return before + excl;
}

// Exact keys of the n_c candidate half-blocks listed (ascending) in `list`,
// scored with k_scan's arithmetic into ck, then their top K into out (ties to
// the lowest position, since the slots ascend).  Two slots per thread in
// flight; consecutive threads take the 4 positions of a half-block.
template <int FMT>
__device__ __forceinline__ void topk_of_halves(const uint8_t* __restrict__ ikc,
                                               const float* __restrict__ iks, int64_t row0,
                                               const float* qrow, const float* wrow, int nv,
                                               uint32_t n_c, const int32_t* list, uint32_t* ck,
                                               int K, int32_t* out, SelRegShared& rs) {
    const int tid = threadIdx.x;
    const int n_slots = (int)n_c * kHalf;
    // the query's values held in registers and broadcast by DPP, as in k_scan
    QQuad qq;
    qq.load(qrow);
    const float w4[kIdxHeads] = {wrow[0], wrow[1], wrow[2], wrow[3]};
    for (int s0 = 0; s0 < n_slots; s0 += 2 * kSelThreads) {
        IdxRow<FMT> r[2];
        bool vis[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int s = s0 + u * kSelThreads + tid;
            const int64_t pos = s < n_slots ? (int64_t)list[s >> 2] * kHalf + (s & 3) : nv;
            vis[u] = pos < nv;
            r[u].load(ikc, iks, row0 + (vis[u] ? pos : 0));  // an absent slot reads row 0
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int s = s0 + u * kSelThreads + tid;
            // a wave with no slot left skips the round; otherwise every lane
            // scores (DPP reads other lanes) and the absent ones are dropped
            if (__ballot(s < n_slots) == 0) continue;
            const float sc = r[u].score(qq, w4);
            if (s < n_slots) ck[s] = vis[u] ? score_key(sc) : 0u;
        }
    }
    __syncthreads();
    // register path: 16 consecutive slots a lane
    uint32_t k[kSelKpt];
#pragma unroll
    for (int i = 0; i < kSelKpt; ++i) {
        const int s = 16 * tid + i;
        k[i] = s < n_slots ? ck[s] : 0u;
    }
    const Threshold tk = threshold_reg(k, K, rs);
    compact_reg(k, tk, K, [&](int64_t s) { return list[s >> 2] * kHalf + (int32_t)(s & 3); }, out,
                nullptr, rs);
}

template <int FMT>
__global__ __launch_bounds__(kSelThreads) void k_chunk_select(
    const uint8_t* __restrict__ ikc, const float* __restrict__ iks, int64_t cap, int Q,
    const float* __restrict__ qd, const float* __restrict__ wq,
    const uint32_t* __restrict__ hkeys_hi, const int32_t* __restrict__ n_vis, int K, int Pc,
    uint32_t* __restrict__ keys, uint32_t* __restrict__ bkeys, int32_t* __restrict__ topk_out) {
    __shared__ SelShared sh;
    __shared__ uint32_t ck[kChunkSlots];
    __shared__ uint32_t part[kSelWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bq = blockIdx.x;
    const int64_t row0 = (bq / Q) * cap;
    const int nv = clamp_nvis(n_vis[bq], cap);
    const int64_t nb = cap / kBlock, nbv = ((int64_t)nv + kBlock - 1) / kBlock;
    const int64_t nhv = ((int64_t)nv + kHalf - 1) / kHalf;
    const KeySrc lo{bkeys + bq * nb, nullptr, nbv, nv, 0};  // the scan's lower bounds
    const KeySrc hi{hkeys_hi + bq * (cap / kHalf), nullptr, nhv, nv, 0};
    const float* qrow = qd + bq * kIdxHeads * kIdxDim;
    const float* wrow = wq + bq * kIdxHeads;
    SelRegShared& rs = *reinterpret_cast<SelRegShared*>(&sh.hist[0]);

    // 1. the K-th largest lower-bound key: the threshold's tie value, else the
    // smallest key at or above its cut
    Threshold th;
    uint32_t m = 0xFFFFFFFFu;
    if (nbv <= kSelRegSlots) {
        uint32_t k[kSelKpt];
        lo.load16((int64_t)wave * 1024 + 16 * lane, k);
        th = threshold_reg(k, K, rs);
#pragma unroll
        for (int i = 0; i < kSelKpt; ++i)
            m = (k[i] != 0 && k[i] >= th.t_ge) ? min(m, k[i]) : m;
    } else {
        const SelRange r = wave_range(nbv, wave);
        th = find_threshold<false>(lo, sh.keys, r, K, sh);
        for_keys<false>(lo, sh.keys, r, lane, [&](uint32_t k, int64_t, bool) {
            m = (k != 0 && k >= th.t_ge) ? min(m, k) : m;
        });
    }
    m = wave_reduce(m, [](uint32_t a, uint32_t b) { return min(a, b); });
    if (lane == 0) part[wave] = m;
    __syncthreads();
    m = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) m = min(m, part[w]);
    const uint32_t x = th.total < (uint32_t)K ? 1u : (th.quota != 0 ? th.t_eq : m);

    // 2. ordered compaction of the candidate half-blocks into sh.pool, 16
    // per thread per sweep
    uint32_t n_c = 0;
    for (int64_t b0 = 0; b0 < nhv; b0 += (int64_t)kSelThreads * kSelKpt) {
        const int64_t first = b0 + (int64_t)tid * kSelKpt;
        uint32_t h[kSelKpt];
        hi.load16(first, h);  // 0 past the visible half-blocks, and x >= 1
        uint32_t mask = 0;
#pragma unroll
        for (int i = 0; i < kSelKpt; ++i) mask |= h[i] >= x ? (1u << i) : 0u;
        uint32_t total;
        uint32_t r = n_c + rank_of_count(__popc(mask), part, total);
        for (uint32_t mm = mask; mm != 0; mm &= mm - 1u, ++r)
            if (r < (uint32_t)Pc) sh.pool[r] = (int32_t)(first + __builtin_ctz(mm));
        n_c += total;  // uniform
    }

    if (n_c > (uint32_t)Pc) {  // uniform: the exact fallback
        scan_query_exact<FMT>(ikc, iks, row0, qrow, wrow, nv, kSelThreads, keys + bq * cap,
                         bkeys + bq * nb);
        __syncthreads();  // the keys are the workgroup's own global writes
        select_full_query(keys, bkeys, cap, bq, nv, K, K, nullptr, topk_out, sh);
        return;
    }
    __syncthreads();  // the candidate list is complete

    // 3-4. exact keys of the candidates' positions, and their top-K
    topk_of_halves<FMT>(ikc, iks, row0, qrow, wrow, nv, n_c, sh.pool, ck, K, topk_out + bq * K, rs);
}

// Full layer with a pool of P blocks, for one query of the multi-query MFMA
// scan (one workgroup per query, at most 16384 blocks: each thread holds the
// bound keys of 16 consecutive blocks in registers).  lo and hi are the
// scan's bound keys; a block's upper bound ub is the larger hi of its halves.
//   1. x = the P-th largest lo: as for positions, every block the exact pool
//      can take (ties included) has ub >= x;
//   2. y = the (P+1)-th largest ub: a block with lo > y is in the pool, since
//      only blocks with ub > y (at most P, itself among them) can rank above
//      it; with at most P visible blocks, all of them are;
//   3. the other blocks with ub >= x are undecided (a few near the cut).  When
//      more of them remain than the pool has room for, their positions are
//      scored exactly and the best of them by exact block key (the maximum
//      over its positions), ties to the lowest block, fill the pool;
//   4. the pool is written in ascending block order.  x' = the K-th largest
//      lo among its blocks bounds the K-th largest exact score inside it, so
//      the top-K lies in the pool's half-blocks whose hi reaches x'; those are
//      scored exactly and the top-K taken as in k_chunk_select.
// When a list overflows (heavy ties) the query is scored over all its
// visible positions instead and takes the Full selection.
constexpr int kPoolUndecided = 1024;  // undecided blocks held in LDS
static_assert(kMaxPoolBlocks >= kChunkMaxCand, "sh.pool holds either list");

template <int FMT>
__global__ __launch_bounds__(kSelThreads) void k_chunk_select_pool(
    const uint8_t* __restrict__ ikc, const float* __restrict__ iks, int64_t cap, int Q,
    const float* __restrict__ qd, const float* __restrict__ wq,
    const uint32_t* __restrict__ hkeys_hi, const int32_t* __restrict__ n_vis, int P, int K, int Pc,
    uint32_t* __restrict__ keys, uint32_t* __restrict__ bkeys, int32_t* __restrict__ pool_out,
    int32_t* __restrict__ topk_out) {
    __shared__ SelShared sh;
    __shared__ uint32_t ck[kChunkSlots];
    __shared__ uint32_t part[kSelWaves];
    __shared__ int32_t ulist[kPoolUndecided];
    __shared__ uint32_t ukey[kPoolUndecided];
    __shared__ uint32_t taken[kSelRegSlots / 32];  // undecided blocks the pool takes
    const int tid = threadIdx.x;
    const int64_t bq = blockIdx.x;
    const int64_t row0 = (bq / Q) * cap;
    const int nv = clamp_nvis(n_vis[bq], cap);
    const int64_t nb = cap / kBlock, nbv = ((int64_t)nv + kBlock - 1) / kBlock;
    const int64_t nhv = ((int64_t)nv + kHalf - 1) / kHalf;
    const KeySrc lo_src{bkeys + bq * nb, nullptr, nbv, nv, 0};  // the scan's lower bounds
    const KeySrc hi_src{hkeys_hi + bq * (cap / kHalf), nullptr, nhv, nv, 0};
    const float* qrow = qd + bq * kIdxHeads * kIdxDim;
    const float* wrow = wq + bq * kIdxHeads;
    SelRegShared& rs = *reinterpret_cast<SelRegShared*>(&sh.hist[0]);
    const int32_t b0 = tid * kSelKpt;  // this thread's first block

    for (int i = tid; i < kSelRegSlots / 32; i += kSelThreads) taken[i] = 0u;
    uint32_t lo[kSelKpt], ub[kSelKpt];
    lo_src.load16(b0, lo);  // 0 where no position is visible
    {
        uint32_t h[kSelKpt];
        hi_src.load16(2 * b0, h);
#pragma unroll
        for (int i = 0; i < kSelKpt / 2; ++i) ub[i] = max(h[2 * i], h[2 * i + 1]);
        hi_src.load16(2 * b0 + kSelKpt, h);
#pragma unroll
        for (int i = 0; i < kSelKpt / 2; ++i) ub[kSelKpt / 2 + i] = max(h[2 * i], h[2 * i + 1]);
    }

    // 1-2. x and y
    const Threshold tx = threshold_reg(lo, P, rs);
    const uint32_t x = kth_key_reg(lo, tx, P, part);
    const Threshold ty = threshold_reg(ub, P + 1, rs);
    const uint32_t y = kth_key_reg(ub, ty, P + 1, part);
    const bool all_in = ty.total <= (uint32_t)P;
    uint32_t sure = 0, und = 0;
#pragma unroll
    for (int i = 0; i < kSelKpt; ++i) {
        if (lo[i] != 0 && (all_in || lo[i] > y)) sure |= 1u << i;
        else if (lo[i] != 0 && ub[i] >= x) und |= 1u << i;
    }
    // both counts at once: sure in the high half-word (each total <= 16384)
    uint32_t tot;
    const uint32_t rk = rank_of_count(__popc(und) | (__popc(sure) << 16), part, tot);
    const uint32_t n_und = tot & 0xFFFFu, n_sure = tot >> 16;
    const uint32_t need = (uint32_t)P - n_sure;  // n_sure <= P

    auto fallback = [&]() {
        scan_query_exact<FMT>(ikc, iks, row0, qrow, wrow, nv, kSelThreads, keys + bq * cap,
                         bkeys + bq * nb);
        __syncthreads();  // the keys are the workgroup's own global writes
        select_full_query(keys, bkeys, cap, bq, nv, P, K, pool_out, topk_out, sh);
    };

    // 3. the undecided blocks, when the pool cannot take them all
    uint32_t in_pool = sure | und;
    if (n_und > need) {  // uniform
        if (n_und > (uint32_t)kPoolUndecided) {
            fallback();
            return;
        }
        uint32_t r = rk & 0xFFFFu;
        for (uint32_t mm = und; mm != 0; mm &= mm - 1u, ++r) ulist[r] = b0 + __builtin_ctz(mm);
        __syncthreads();
        // exact block keys: a block's 8 positions on 8 consecutive lanes (the
        // trip count is uniform, so every lane takes part in the group max)
        // (the query in registers, broadcast by DPP: every lane of a wave
        // scores, an absent position reads row 0 and is dropped)
        const int n_pos = (int)n_und * kBlock;
        QQuad qq;
        qq.load(qrow);
        const float w4[kIdxHeads] = {wrow[0], wrow[1], wrow[2], wrow[3]};
        for (int s0 = 0; s0 < n_pos; s0 += kSelThreads) {
            const int s = s0 + tid;
            const int64_t pos = s < n_pos ? (int64_t)ulist[s >> 3] * kBlock + (s & 7) : nv;
            if (__ballot(s < n_pos) == 0) continue;  // uniform over the wave
            IdxRow<FMT> r;
            r.load(ikc, iks, row0 + (pos < nv ? pos : 0));
            const float sc = r.score(qq, w4);
            const uint32_t key = max8_u32(pos < nv ? score_key(sc) : 0u);
            if (s < n_pos && (s & 7) == 0) ukey[s >> 3] = key;
        }
        __syncthreads();
        uint32_t k[kSelKpt];
#pragma unroll
        for (int i = 0; i < kSelKpt; ++i) {
            const int s = 16 * tid + i;
            k[i] = s < (int)n_und ? ukey[s] : 0u;
        }
        const Threshold tu = threshold_reg(k, (int)need, rs);
        compact_reg(k, tu, (int)need, [&](int64_t s) { return ulist[s]; }, nullptr, sh.pool, rs);
        __syncthreads();
        for (int j = tid; j < (int)need; j += kSelThreads) {
            const int32_t blk = sh.pool[j];
            if (blk >= 0) atomicOr(&taken[blk >> 5], 1u << (blk & 31));
        }
        __syncthreads();
        in_pool = sure | ((taken[tid >> 1] >> (16 * (tid & 1))) & 0xFFFFu);
    }

    // 4. the pool, ascending
    uint32_t n_pool;
    {
        uint32_t r = rank_of_count(__popc(in_pool), part, n_pool);
        int32_t* prow = pool_out + bq * P;
        for (uint32_t mm = in_pool; mm != 0; mm &= mm - 1u, ++r)
            if (r < (uint32_t)P) prow[r] = b0 + __builtin_ctz(mm);  // n_pool <= P
        for (int i = (int)n_pool + tid; i < P; i += kSelThreads) prow[i] = -1;
    }
    uint32_t kp[kSelKpt];
#pragma unroll
    for (int i = 0; i < kSelKpt; ++i) kp[i] = (in_pool >> i) & 1u ? lo[i] : 0u;
    const Threshold tk = threshold_reg(kp, K, rs);
    const uint32_t xk = kth_key_reg(kp, tk, K, part);
    // candidate half-blocks of the pool: half 2 b0 + j of this thread
    uint32_t cmask = 0;
    {
        uint32_t h[kSelKpt];
        hi_src.load16(2 * b0, h);
#pragma unroll
        for (int j = 0; j < kSelKpt; ++j)
            cmask |= ((in_pool >> (j >> 1)) & 1u) && h[j] >= xk ? (1u << j) : 0u;
        hi_src.load16(2 * b0 + kSelKpt, h);
#pragma unroll
        for (int j = 0; j < kSelKpt; ++j)
            cmask |= ((in_pool >> (8 + (j >> 1))) & 1u) && h[j] >= xk ? (1u << (16 + j)) : 0u;
    }
    uint32_t n_c;
    uint32_t r = rank_of_count(__popc(cmask), part, n_c);
    if (n_c > (uint32_t)Pc) {  // uniform
        fallback();
        return;
    }
    for (uint32_t mm = cmask; mm != 0; mm &= mm - 1u, ++r)
        sh.pool[r] = 2 * b0 + __builtin_ctz(mm);
    __syncthreads();  // the candidate list is complete
    topk_of_halves<FMT>(ikc, iks, row0, qrow, wrow, nv, n_c, sh.pool, ck, K, topk_out + bq * K, rs);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_scan(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                       const float* iq, const float* iw, float* qd, float* wq,
                       const int32_t* n_vis, uint32_t* keys, uint32_t* bkeys, hipStream_t stream,
                       hipEvent_t start, hipEvent_t stop, uint32_t* sbkeys, int fmt) {
    dim3 grid((unsigned)((cap + 255) / 256), (unsigned)B);
    // a few queries per sequence (FP4 keys: any number): k_scan quantises
    // them itself; many (the replay chunk, FP8 keys): k_prep_iq writes them
    // to qd / wq once and k_scan_multi stages them in LDS
    const bool multi = fmt == 0 && Q >= 4;
    if (multi) {
        const hipError_t e = launch_prep_iq(iq, iw, (int64_t)B * Q, qd, wq, stream);
        if (e != hipSuccess) return e;
    }
    auto kern = fmt == 1 ? (Q == 1 ? k_scan<1, true> : k_scan<1, false>)
                         : (multi ? k_scan_multi : (Q == 1 ? k_scan<0, true> : k_scan<0, false>));
    const float* qa = multi ? qd : iq;
    const float* wa = multi ? wq : iw;
    if (start != nullptr && stop != nullptr) {
        // the runtime records `start` / `stop` immediately around this dispatch
        hipExtLaunchKernelGGL(kern, grid, dim3(256), 0, stream, start, stop, 0, ikc, iks, cap, Q,
                              qa, wa, n_vis, keys, bkeys, sbkeys);
    } else {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, ikc, iks, cap, Q, qa, wa, n_vis,
                           keys, bkeys, sbkeys);
    }
    return hipGetLastError();
}

hipError_t launch_pool_score(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                             const float* iq, const float* iw, const int32_t* n_vis,
                             const int32_t* pool, int P, uint32_t* ckeys, uint4* parts,
                             hipStream_t stream, int fmt) {
    const int64_t n_slots = (int64_t)P * kBlock;
    dim3 grid((unsigned)((n_slots + 255) / 256), (unsigned)(B * Q));
    hipLaunchKernelGGL(fmt == 1 ? k_pool_score<1> : k_pool_score<0>, grid, dim3(256), 0, stream,
                       ikc, iks, cap, Q, iq, iw, n_vis, pool, P, ckeys, parts);
    return hipGetLastError();
}

hipError_t launch_select_full(const uint32_t* keys, const uint32_t* bkeys, int64_t cap,
                              const int32_t* n_vis, int64_t n_queries, int P, int K,
                              int32_t* pool_out, int32_t* topk_out, hipStream_t stream,
                              const uint32_t* sbkeys) {
    hipLaunchKernelGGL(k_select_full, dim3((unsigned)n_queries), dim3(kSelThreads), 0, stream, keys,
                       bkeys, cap, n_vis, P, K, pool_out, topk_out, sbkeys);
    return hipGetLastError();
}

hipError_t launch_select_pool(const uint32_t* ckeys, const uint4* parts, const int32_t* pool,
                              int P, const int32_t* n_vis, int64_t cap, int64_t n_queries, int K,
                              int32_t* topk_out, hipStream_t stream) {
    hipLaunchKernelGGL(k_select_pool, dim3((unsigned)n_queries), dim3(kSelThreads), 0, stream,
                       ckeys, parts, pool, P, n_vis, cap, K, topk_out);
    return hipGetLastError();
}

hipError_t launch_chunk_select(const uint8_t* ikc, const float* iks, int64_t cap, int Q,
                               const float* qd, const float* wq, const uint32_t* hkeys_hi,
                               const int32_t* n_vis, int64_t n_queries, int K, uint32_t* keys,
                               uint32_t* bkeys, int32_t* topk_out, hipStream_t stream, int P,
                               int32_t* pool_out, int fmt) {
    const int Pc = chunk_cand_halves(K);
    if (Pc > kChunkMaxCand) return hipErrorInvalidValue;
    if (P > 0) {
        if (cap / kBlock > kSelRegSlots || P > kMaxPoolBlocks || pool_out == nullptr)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(fmt == kIdxFp4 ? k_chunk_select_pool<kIdxFp4>
                                          : k_chunk_select_pool<kIdxFp8>,
                           dim3((unsigned)n_queries), dim3(kSelThreads), 0,
                           stream, ikc, iks, cap, Q, qd, wq, hkeys_hi, n_vis, P, K, Pc, keys,
                           bkeys, pool_out, topk_out);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(fmt == kIdxFp4 ? k_chunk_select<kIdxFp4> : k_chunk_select<kIdxFp8>,
                       dim3((unsigned)n_queries), dim3(kSelThreads), 0, stream,
                       ikc, iks, cap, Q, qd, wq, hkeys_hi, n_vis, K, Pc, keys, bkeys, topk_out);
    return hipGetLastError();
}

}  // namespace csa2
