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
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

// Score of one indexer-K row from its four 16-byte channel groups.
// qd: the query's decoded E4M3 values [4][64] (uniform across the wave, read
// through the scalar cache); wq: the 4 folded head weights.
__device__ __forceinline__ float score_row(const uint4 (&raw)[4], float sigma,
                                           const float* __restrict__ qd,
                                           const float* __restrict__ wq) {
    float kf[kIdxDim];
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

// ---------------------------------------------------------------------------
// Full-layer scan.  grid = (ceil(cap / 256), B); 256 threads, one position each.
// For every query of the sequence: key of each position, and the max key of
// each 8-position block (DPP max over 8 adjacent lanes).  Tiles that no
// query of the sequence can see are skipped entirely.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_scan(const uint8_t* __restrict__ ikc,
                                              const float* __restrict__ iks, int64_t cap, int Q,
                                              const float* __restrict__ qd,
                                              const float* __restrict__ wq,
                                              const int32_t* __restrict__ n_vis,
                                              uint32_t* __restrict__ keys,
                                              uint32_t* __restrict__ bkeys) {
    const int b = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * 256;
    const int64_t p = p0 + threadIdx.x;
    int nv_max = 0;
    for (int q = 0; q < Q; ++q) nv_max = max(nv_max, clamp_nvis(n_vis[(int64_t)b * Q + q], cap));
    if (p0 >= nv_max) return;  // uniform over the block
    // cap is a multiple of 64, so a wave is either wholly inside or wholly past it
    if (p0 + (threadIdx.x & ~63) >= cap) return;

    const int64_t row = (int64_t)b * cap + p;
    uint4 raw[4];
    load_ik_row(ikc, row, raw);
    const float sigma = iks[row];
    const int64_t nb = cap / kBlock;
    for (int q = 0; q < Q; ++q) {
        const int64_t bq = (int64_t)b * Q + q;
        const int nv = clamp_nvis(n_vis[bq], cap);
        if (p0 >= nv) continue;  // uniform
        const float s = score_row(raw, sigma, qd + bq * kIdxHeads * kIdxDim, wq + bq * kIdxHeads);
        const uint32_t key = (p < nv) ? score_key(s) : 0u;
        keys[bq * cap + p] = key;
        const uint32_t bk = max8_u32(key);
        if ((threadIdx.x & 7) == 0) bkeys[bq * nb + (p >> 3)] = bk;
    }
}

// ---------------------------------------------------------------------------
// Reindex: score the positions of the pool blocks with the layer's own query.
// grid = (ceil(P*8 / 256), B*Q).  Slot s of query bq is position
// pool[j]*8 + (s & 7) with j = s / 8; invisible or empty slots get key 0.
// The eight lanes of one block read 8 x 16 contiguous bytes per plane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pool_score(const uint8_t* __restrict__ ikc,
                                                    const float* __restrict__ iks, int64_t cap,
                                                    int Q, const float* __restrict__ qd,
                                                    const float* __restrict__ wq,
                                                    const int32_t* __restrict__ n_vis,
                                                    const int32_t* __restrict__ pool, int P,
                                                    uint32_t* __restrict__ ckeys) {
    const int64_t bq = blockIdx.y;
    const int64_t b = bq / Q;
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n_slots = (int64_t)P * kBlock;
    if (s >= n_slots) return;
    const int nv = clamp_nvis(n_vis[bq], cap);
    const int32_t blk = pool[bq * P + (s >> 3)];
    const int64_t pos = (int64_t)blk * kBlock + (s & 7);
    uint32_t key = 0;
    if (blk >= 0 && pos < nv) {
        const int64_t row = b * cap + pos;
        uint4 raw[4];
        load_ik_row(ikc, row, raw);
        key = score_key(score_row(raw, iks[row], qd + bq * kIdxHeads * kIdxDim, wq + bq * kIdxHeads));
    }
    ckeys[bq * n_slots + s] = key;
}

// ---------------------------------------------------------------------------
// Exact top-K select, one workgroup of 1024 threads per query.
//
// Slots are numbered in ascending index order; key 0 marks an empty slot.
// The K-th largest key T is found by a 4-pass MSB-first radix select (8-bit
// digits, LDS histogram).  The output is every slot with key > T plus the
// lowest-numbered slots with key == T until K are taken, written in
// ascending slot order (so ties go to the lowest position / block).
// Fewer than K non-empty slots: all are output.  The rest is -1.
//
//   MODE_BLOCKS  slots = blocks [0, ceil(n_vis/8)), key = block max key,
//                index = block id.
//   MODE_GATHER  slots = pool positions (P*8), key read from the full
//                per-position key array, index = position.
//   MODE_COMPACT slots = pool positions, key from a compact [P*8] array.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelLdsKeys = 16384;

template <int MODE>
struct SlotSource {
    const uint32_t* src;
    const int32_t* pool;  // LDS copy of the query's pool (MODE_GATHER / MODE_COMPACT)
    int nv;
    __device__ __forceinline__ uint32_t key(int64_t s) const {
        if (MODE == kModeGather) {
            const int32_t blk = pool[s >> 3];
            const int64_t pos = (int64_t)blk * kBlock + (s & 7);
            return (blk >= 0 && pos < nv) ? src[pos] : 0u;
        }
        return src[s];
    }
    __device__ __forceinline__ int32_t index(int64_t s) const {
        if (MODE == kModeBlocks) return (int32_t)s;
        return pool[s >> 3] * kBlock + (int32_t)(s & 7);
    }
};

template <int MODE>
__global__ __launch_bounds__(kSelThreads) void k_select(
    const uint32_t* __restrict__ src, int64_t src_stride, const int32_t* __restrict__ pool, int P,
    const int32_t* __restrict__ n_vis, int64_t cap, int K, int32_t* __restrict__ out,
    int64_t out_stride) {
    __shared__ uint32_t s_keys[kSelLdsKeys];
    __shared__ int32_t s_pool[kMaxPoolBlocks];
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_wgt[kSelWaves], s_weq[kSelWaves];
    __shared__ uint32_t s_state[3];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bq = blockIdx.x;
    const int nv = clamp_nvis(n_vis[bq], cap);
    int64_t n;
    if (MODE == kModeBlocks) {
        n = ((int64_t)nv + kBlock - 1) / kBlock;
    } else {
        n = (int64_t)P * kBlock;
        const int64_t nbv = ((int64_t)nv + kBlock - 1) / kBlock;
        for (int j = tid; j < P; j += kSelThreads) {
            int32_t blk = pool[bq * P + j];
            s_pool[j] = (blk >= 0 && blk < nbv) ? blk : -1;  // out-of-range ids are ignored
        }
        __syncthreads();
    }
    SlotSource<MODE> srcv{src + bq * src_stride, s_pool, nv};
    const bool cached = n <= kSelLdsKeys;
    if (cached) {
        for (int64_t s = tid; s < n; s += kSelThreads) s_keys[s] = srcv.key(s);
        __syncthreads();
    }
    auto key_at = [&](int64_t s) -> uint32_t { return cached ? s_keys[s] : srcv.key(s); };

    // ---- radix select of the K-th largest key ----
    uint32_t prefix = 0, mask = 0;
    uint32_t remaining = (uint32_t)K;
    uint32_t t_ge = 1, t_eq = 0, quota = 0;  // default: take every non-empty slot
    bool resolved = false;
    for (int pass = 0; pass < 4 && !resolved; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) s_hist[tid] = 0;
        __syncthreads();
        for (int64_t s = tid; s < n; s += kSelThreads) {
            const uint32_t k = key_at(s);
            if (k != 0 && (k & mask) == prefix) atomicAdd(&s_hist[(k >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds digits 255-4l .. 252-4l (descending)
            uint32_t h[4], loc = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) { h[i] = s_hist[255 - 4 * lane - i]; loc += h[i]; }
            uint32_t incl = loc;  // inclusive scan over lanes
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_up(incl, off, 64);
                if (lane >= off) incl += y;
            }
            const uint32_t total = __shfl(incl, 63, 64);
            uint32_t above = incl - loc;
            if (lane == 0) { s_state[0] = 0xFFFFFFFFu; s_state[2] = total; }
            // exactly one (lane, i) satisfies above < remaining <= above + h
            if (pass > 0 || total > remaining) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (above < remaining && above + h[i] >= remaining) {
                        s_state[0] = (uint32_t)(255 - 4 * lane - i);
                        s_state[1] = above;
                    }
                    above += h[i];
                }
            }
        }
        __syncthreads();
        const uint32_t d = s_state[0];
        if (pass == 0 && s_state[2] <= remaining) {  // K or fewer non-empty slots: take all
            resolved = true;
        } else {
            const uint32_t above = s_state[1];
            const uint32_t cnt = s_hist[d];
            remaining -= above;
            prefix |= d << shift;
            mask |= 0xFFu << shift;
            if (cnt == remaining) {  // the whole bin is taken: threshold is its lowest key
                t_ge = prefix;
                quota = 0;
                resolved = true;
            } else if (pass == 3) {  // T = prefix exactly; take `remaining` of the ties
                t_ge = prefix + 1;
                t_eq = prefix;
                quota = remaining;
                resolved = true;
            }
        }
        __syncthreads();
    }

    // ---- compaction in ascending slot order (each wave owns a contiguous range) ----
    const int64_t chunk = ((n + kSelWaves - 1) / kSelWaves + 63) / 64 * 64;
    const int64_t beg = (int64_t)wave * chunk;
    const int64_t end = min(n, beg + chunk);
    uint32_t c_gt = 0, c_eq = 0;
    for (int64_t base = beg; base < end; base += 64) {
        const int64_t s = base + lane;
        const uint32_t k = s < end ? key_at(s) : 0u;
        const bool gt = k != 0 && k >= t_ge;
        const bool eq = k != 0 && quota != 0 && k == t_eq;
        c_gt += __popcll(__ballot(gt));
        c_eq += __popcll(__ballot(eq));
    }
    if (lane == 0) { s_wgt[wave] = c_gt; s_weq[wave] = c_eq; }
    __syncthreads();
    // per-wave prefix of ties and of outputs (16 values, every thread)
    uint32_t eq_before = 0, out_before = 0, total_sel = 0, eb = 0;
    for (int w = 0; w < kSelWaves; ++w) {
        const uint32_t take_eq = quota > eb ? min(quota - eb, s_weq[w]) : 0u;
        if (w == wave) { eq_before = eb; out_before = total_sel; }
        total_sel += s_wgt[w] + take_eq;
        eb += s_weq[w];
    }
    int32_t* o = out + bq * out_stride;
    uint32_t eq_seen = 0, taken = 0;
    for (int64_t base = beg; base < end; base += 64) {
        const int64_t s = base + lane;
        const uint32_t k = s < end ? key_at(s) : 0u;
        const bool gt = k != 0 && k >= t_ge;
        const bool eq = k != 0 && quota != 0 && k == t_eq;
        const uint64_t eq_mask = __ballot(eq);
        const uint32_t eq_rank = eq_before + eq_seen +
            __builtin_amdgcn_mbcnt_hi((uint32_t)(eq_mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eq_mask, 0));
        const bool take = gt || (eq && eq_rank < quota);
        const uint64_t tk_mask = __ballot(take);
        const uint32_t rank = out_before + taken +
            __builtin_amdgcn_mbcnt_hi((uint32_t)(tk_mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)tk_mask, 0));
        if (take && rank < (uint32_t)K) o[rank] = srcv.index(s);
        eq_seen += __popcll(eq_mask);
        taken += __popcll(tk_mask);
    }
    for (int64_t i = (int64_t)total_sel + tid; i < K; i += kSelThreads) o[i] = -1;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_scan(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                       const float* qd, const float* wq, const int32_t* n_vis, uint32_t* keys,
                       uint32_t* bkeys, hipStream_t stream) {
    dim3 grid((unsigned)((cap + 255) / 256), (unsigned)B);
    hipLaunchKernelGGL(k_scan, grid, dim3(256), 0, stream, ikc, iks, cap, Q, qd, wq, n_vis, keys,
                       bkeys);
    return hipGetLastError();
}

hipError_t launch_pool_score(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                             const float* qd, const float* wq, const int32_t* n_vis,
                             const int32_t* pool, int P, uint32_t* ckeys, hipStream_t stream) {
    const int64_t n_slots = (int64_t)P * kBlock;
    dim3 grid((unsigned)((n_slots + 255) / 256), (unsigned)(B * Q));
    hipLaunchKernelGGL(k_pool_score, grid, dim3(256), 0, stream, ikc, iks, cap, Q, qd, wq, n_vis,
                       pool, P, ckeys);
    return hipGetLastError();
}

hipError_t launch_select(int mode, const uint32_t* src, int64_t src_stride, const int32_t* pool,
                         int P, const int32_t* n_vis, int64_t cap, int64_t n_queries, int K,
                         int32_t* out, int64_t out_stride, hipStream_t stream) {
    dim3 grid((unsigned)n_queries);
    switch (mode) {
        case kModeBlocks:
            hipLaunchKernelGGL(k_select<kModeBlocks>, grid, dim3(kSelThreads), 0, stream, src,
                               src_stride, pool, P, n_vis, cap, K, out, out_stride);
            break;
        case kModeGather:
            hipLaunchKernelGGL(k_select<kModeGather>, grid, dim3(kSelThreads), 0, stream, src,
                               src_stride, pool, P, n_vis, cap, K, out, out_stride);
            break;
        default:
            hipLaunchKernelGGL(k_select<kModeCompact>, grid, dim3(kSelThreads), 0, stream, src,
                               src_stride, pool, P, n_vis, cap, K, out, out_stride);
            break;
    }
    return hipGetLastError();
}

}  // namespace csa2
