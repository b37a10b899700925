// csa2_attn.hip -- CSA2 sparse attention over the FP4 global KV plus the FP8
// sliding window.
//
// "DeepSeek V4.1 Flash: architecture study notes", section 2: each query
// attends to at most 512 selected global records together with its local
// window; section 1: the window is 128 tokens and every layer keeps its own;
// section 4: the FP4 cache is dequantised on read and fed to ordinary
// attention (the saving is storage, not FP4 arithmetic); the SWA KV stays FP8.
//
// Design (gfx950).  A decode batch is small (16 queries) while every query
// gathers ~108 KB from random rows, so the latency of the dependent
// index -> row loads dominates.  The entry list of each query (selected
// records, then window tokens) is cut into tiles of 32 entries and the work is
// split over (query, run of tiles) workgroups -- 320 of them for 16 queries --
// so all gathers are in flight at once; a second small kernel merges the
// per-split softmax partials (one wave per query and head, one load round).
// Within a workgroup, one wave per 16 heads: all heads share one KV head (MQA),
// so the logits are a dense [heads x entries] contraction on MFMA
// (v_mfma_f32_16x16x32_f16):
//   - dequantised E2M1 x E4M3 values have at most 6 significant bits and lie
//     in [2^-10, 2688], so they are exact in fp16; E4M3 window codes are exact
//     in fp16 and their fp32 row scale is applied to the logit (K) or to the
//     probability (V) in fp32;
//   - q is split into fp16 hi + lo parts, so q.k carries ~22 bits;
//   - accumulation is fp32, softmax is online in fp32 (base-2 exponentials).
// Per tile the workgroup dequantises the gathered bytes into LDS (K row-major,
// V transposed); each wave computes S^T = K Q^T, rescales its running output
// and accumulates O^T += V^T P^T with P taken straight from the S^T registers
// (entry order inside the k dimension is permuted consistently).  With more
// than one tile per split, the next tile's bytes are loaded while the current
// one is used.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;          // entries per tile
constexpr int kKPitch = 136;       // fp16 per K row in LDS (128 + 8)
constexpr int kVPitch = 36;        // fp16 per V^T row in LDS (32 + 4)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct SplitPlan {
    int n_tiles_global;  // ceil(topk / 32)
    int n_tiles;         // global + window tiles
    int n_splits;
    int tiles_per_split;
};

// Aim for about 512 workgroups: a decode batch of 16 queries spreads its 20
// tiles over 20 workgroups per query; a 128-query chunk takes 4 per query.
// At most 64 splits (the merge kernel gives one lane to each).
static SplitPlan plan_splits(int64_t n_q, int topk, int swa_rows) {
    SplitPlan p;
    p.n_tiles_global = (topk + kTile - 1) / kTile;
    p.n_tiles = p.n_tiles_global + (swa_rows + kTile - 1) / kTile;
    if (p.n_tiles == 0) p.n_tiles = 1;
    int64_t ns = (512 + n_q - 1) / n_q;
    if (ns > p.n_tiles) ns = p.n_tiles;
    if (ns > 64) ns = 64;
    if (ns < 1) ns = 1;
    p.tiles_per_split = (int)((p.n_tiles + ns - 1) / ns);
    p.n_splits = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
    return p;
}

size_t attn_workspace_bytes(int64_t n_q, int H, int topk, int swa_rows) {
    const SplitPlan p = plan_splits(n_q, topk, swa_rows);
    if (p.n_splits <= 1) return 0;
    return (size_t)n_q * p.n_splits * H * (kHeadDim + 2) * sizeof(float);
}

// One tile (32 entries) is loaded as 256 tasks:
//   task <  128  K task: entry e = task/4, channels [32c, 32c+32), c = task%4
//   task >= 128  V task: entries 4q..4q+3, channels [8o, 8o+8) (q, o from task-128)
// The raw bytes of a task fit in 8 dwords; `flag` carries validity bits.
struct TaskRegs {
    uint32_t w[8];
    uint32_t flag;
    float mul[4];
};

struct TileCtx {
    const uint8_t* kvc;
    const uint8_t* kvs;
    const uint8_t* swk;
    const uint8_t* swv;
    const float* swks;
    const float* swvs;
    const int32_t* idx;  // this query's top-K row
    int64_t cap;
    int64_t b;
    int topk;
    int swa_rows;
    int swa_len;
    int n_tiles_global;
};

// global entry `slot` of this query -> cache row, or -1
__device__ __forceinline__ int64_t entry_row(const TileCtx& c, int slot) {
    if (slot >= c.topk) return -1;
    const int32_t pos = c.idx[slot];
    return (pos >= 0 && pos < c.cap) ? c.b * c.cap + pos : -1;
}

// window token t of this query -> window row, or -1
__device__ __forceinline__ int64_t window_row(const TileCtx& c, int t) {
    return t < c.swa_len ? c.b * c.swa_rows + t : -1;
}

__device__ __forceinline__ void load_task(const TileCtx& c, int tile, int task, TaskRegs& r) {
    const bool global = tile < c.n_tiles_global;
    r.flag = 0;
    if (task < 128) {
        const int e = task >> 2, q4 = task & 3;
        const int64_t row = global ? entry_row(c, tile * kTile + e)
                                   : window_row(c, (tile - c.n_tiles_global) * kTile + e);
        if (row < 0) return;
        r.flag = 1;
        if (global) {
            const uint4 v = *reinterpret_cast<const uint4*>(c.kvc + row * 128 + 16 * q4);
            r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
            r.w[4] = *reinterpret_cast<const uint16_t*>(c.kvs + row * 16 + 2 * q4);
        } else {
            const uint4 v0 = *reinterpret_cast<const uint4*>(c.swk + row * kHeadDim + 32 * q4);
            const uint4 v1 = *reinterpret_cast<const uint4*>(c.swk + row * kHeadDim + 32 * q4 + 16);
            r.w[0] = v0.x; r.w[1] = v0.y; r.w[2] = v0.z; r.w[3] = v0.w;
            r.w[4] = v1.x; r.w[5] = v1.y; r.w[6] = v1.z; r.w[7] = v1.w;
            r.mul[0] = c.swks[row];
        }
    } else {
        const int u = task - 128, q = u >> 4, o = u & 15;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * q + j;
            const int64_t row = global ? entry_row(c, tile * kTile + e)
                                       : window_row(c, (tile - c.n_tiles_global) * kTile + e);
            if (row < 0) continue;
            r.flag |= 1u << j;
            if (global) {
                r.w[2 * j] = *reinterpret_cast<const uint32_t*>(c.kvc + row * 128 + 64 + 4 * o);
                r.w[2 * j + 1] = c.kvs[row * 16 + 8 + (o >> 1)];
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(c.swv + row * kHeadDim + 8 * o);
                r.w[2 * j] = v.x;
                r.w[2 * j + 1] = v.y;
                r.mul[j] = c.swvs[row];
            }
        }
    }
}

__device__ __forceinline__ void store_task(const TileCtx& c, int tile, int task,
                                           const TaskRegs& r, _Float16* sK, _Float16* sVt,
                                           float* sKmul, float* sVmul, float logit_mul) {
    const bool global = tile < c.n_tiles_global;
    if (task < 128) {
        const int e = task >> 2, q4 = task & 3;
        _Float16 v[32];
        if (!r.flag) {
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] = (_Float16)0.0f;
        } else if (global) {
            const _Float16 s0 = e4m3_to_f16(r.w[4] & 0xFFu), s1 = e4m3_to_f16(r.w[4] >> 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) fp4x8_to_f16(r.w[i], i < 2 ? s0 : s1, v + 8 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) fp8x8_to_f16(r.w[2 * i], r.w[2 * i + 1], v + 8 * i);
        }
        half8_t* dst = reinterpret_cast<half8_t*>(sK + e * kKPitch + 32 * q4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            half8_t h;
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = v[8 * j + i];
            dst[j] = h;
        }
        if (q4 == 0)
            sKmul[e] = !r.flag ? -INFINITY : (global ? logit_mul : r.mul[0] * logit_mul);
    } else {
        const int u = task - 128, q = u >> 4, o = u & 15;
        _Float16 v[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (!(r.flag >> j & 1u)) {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[j][i] = (_Float16)0.0f;
            } else if (global) {
                fp4x8_to_f16(r.w[2 * j], e4m3_to_f16(r.w[2 * j + 1]), v[j]);
            } else {
                fp8x8_to_f16(r.w[2 * j], r.w[2 * j + 1], v[j]);
            }
        }
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const half4_t h = {v[0][d], v[1][d], v[2][d], v[3][d]};
            *reinterpret_cast<half4_t*>(sVt + (8 * o + d) * kVPitch + 4 * q) = h;
        }
        if (o == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sVmul[4 * q + j] = (r.flag >> j & 1u) ? (global ? 1.0f : r.mul[j]) : 0.0f;
        }
    }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void k_attn(AttnArgs a, SplitPlan plan,
                                                  float* __restrict__ part) {
    constexpr int kThreads = NW * 64;
    constexpr int kTasksPerThread = (256 + kThreads - 1) / kThreads;
    __shared__ __attribute__((aligned(16))) _Float16 sK[kTile * kKPitch];
    __shared__ __attribute__((aligned(16))) _Float16 sVt[kHeadDim * kVPitch];
    __shared__ __attribute__((aligned(16))) float sKmul[kTile];
    __shared__ __attribute__((aligned(16))) float sVmul[kTile];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bq = blockIdx.y;
    const int split = blockIdx.x;
    const int H = a.H;
    const int head = wave * 16 + (lane & 15);
    const int g = lane >> 4;
    const float logit_mul = a.sm_scale * kLog2e;

    TileCtx ctx;
    ctx.kvc = a.kvc; ctx.kvs = a.kvs; ctx.swk = a.swk; ctx.swv = a.swv;
    ctx.swks = a.swks; ctx.swvs = a.swvs;
    ctx.idx = a.idx + bq * a.topk;
    ctx.cap = a.cap;
    ctx.b = bq / a.Q;
    ctx.topk = a.topk;
    ctx.swa_rows = a.swa_rows;
    ctx.n_tiles_global = plan.n_tiles_global;
    if (a.swa_len != nullptr) {
        const int sl = a.swa_len[ctx.b];
        ctx.swa_len = sl < 0 ? 0 : (sl > a.swa_rows ? a.swa_rows : sl);
    } else {
        ctx.swa_len = (int)(bq % a.Q) + 1;
    }

    const int t_beg = split * plan.tiles_per_split;
    const int t_end = min(plan.n_tiles, t_beg + plan.tiles_per_split);

    // q loads go out first (they depend on nothing), then the index -> row
    // chain of the first tile; q is converted while the rows travel
    float4 qraw[8];
    {
        const float* qrow = a.q + (bq * H + min(head, H - 1)) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            qraw[2 * ks] = *reinterpret_cast<const float4*>(qrow + 32 * ks + 8 * g);
            qraw[2 * ks + 1] = *reinterpret_cast<const float4*>(qrow + 32 * ks + 8 * g + 4);
        }
    }
    TaskRegs regs[kTasksPerThread];
#pragma unroll
    for (int k = 0; k < kTasksPerThread; ++k) {
        const int task = tid + k * kThreads;
        if (task < 256 && t_beg < t_end) load_task(ctx, t_beg, task, regs[k]);
    }

    // ---- q as fp16 hi/lo in B-operand layout: head, dims 32ks + 8g .. +8 ----
    half8_t qhi[4], qlo[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const float4 x0 = qraw[2 * ks], x1 = qraw[2 * ks + 1];
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const _Float16 h = (_Float16)xs[i];
            qhi[ks][i] = h;
            qlo[ks][i] = (_Float16)(xs[i] - (float)h);
        }
    }

    float4_t o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    for (int tile = t_beg; tile < t_end; ++tile) {
#pragma unroll
        for (int k = 0; k < kTasksPerThread; ++k) {
            const int task = tid + k * kThreads;
            if (task < 256) store_task(ctx, tile, task, regs[k], sK, sVt, sKmul, sVmul, logit_mul);
        }
        if (tile + 1 < t_end) {  // next tile's bytes travel during this tile's math
#pragma unroll
            for (int k = 0; k < kTasksPerThread; ++k) {
                const int task = tid + k * kThreads;
                if (task < 256) load_task(ctx, tile + 1, task, regs[k]);
            }
        }
        __syncthreads();

        if (head < H) {
            // ---- S^T = K Q^T for entries [16 sub, +16), this wave's 16 heads ----
            float4_t s[2];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const half8_t kv = *reinterpret_cast<const half8_t*>(
                        sK + (16 * sub + (lane & 15)) * kKPitch + 32 * ks + 8 * g);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, qhi[ks], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, qlo[ks], acc, 0, 0, 0);
                }
                s[sub] = acc;
            }
            // lane holds entries 16 sub + 4g + r for its head
            const float4 km0 = *reinterpret_cast<const float4*>(sKmul + 4 * g);
            const float4 km1 = *reinterpret_cast<const float4*>(sKmul + 16 + 4 * g);
            const float km[8] = {km0.x, km0.y, km0.z, km0.w, km1.x, km1.y, km1.z, km1.w};
            const float4 vm0 = *reinterpret_cast<const float4*>(sVmul + 4 * g);
            const float4 vm1 = *reinterpret_cast<const float4*>(sVmul + 16 + 4 * g);
            const float vm[8] = {vm0.x, vm0.y, vm0.z, vm0.w, vm1.x, vm1.y, vm1.z, vm1.w};
            float x[8];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = (km[i] == -INFINITY) ? -INFINITY : s[i >> 2][i & 3] * km[i];
                x[i] = v;
                tmax = fmaxf(tmax, v);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float m_new = fmaxf(m_run, tmax);
            float alpha, psum = 0.0f;
            half8_t pb;
            if (m_new == -INFINITY) {
                alpha = 1.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) pb[i] = (_Float16)0.0f;
            } else {
                alpha = exp2f(m_run - m_new);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p = exp2f(x[i] - m_new);
                    psum += p;
                    pb[i] = (_Float16)(p * vm[i]);
                }
            }
            psum += __shfl_xor(psum, 16, 64);
            psum += __shfl_xor(psum, 32, 64);
            l_run = l_run * alpha + psum;
            m_run = m_new;
            // ---- O^T = O^T * alpha + V^T P^T ----
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const _Float16* vrow = sVt + (16 * dt + (lane & 15)) * kVPitch;
                const half4_t v0 = *reinterpret_cast<const half4_t*>(vrow + 4 * g);
                const half4_t v1 = *reinterpret_cast<const half4_t*>(vrow + 16 + 4 * g);
                const half8_t va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                float4_t acc = o[dt] * alpha;
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, acc, 0, 0, 0);
            }
        }
        __syncthreads();
    }

    if (head >= H) return;
    // lane holds O^T[dim 16 dt + 4g + r][head]
    if (plan.n_splits == 1) {
        const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
        float* orow = a.out + (bq * H + head) * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            float4 v = make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
            *reinterpret_cast<float4*>(orow + 16 * dt + 4 * g) = v;
        }
        if (g == 0) a.lse[bq * H + head] = l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    } else {
        float* prow = part + ((bq * plan.n_splits + split) * H + head) * (kHeadDim + 2);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            float4 v = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
            *reinterpret_cast<float4*>(prow + 16 * dt + 4 * g) = v;
        }
        if (g == 0) {
            prow[kHeadDim] = m_run;
            prow[kHeadDim + 1] = l_run;
        }
    }
}

// Merge the per-split partials: one wave per (query, head).  Every load is
// issued in one round (lane s reads split s's (m, l); each lane reads its two
// channels of every split), then the weights exp2(m_s - M) are formed with
// DPP reductions and broadcast with readlane.  grid (n_q, H/4), 256 threads.
// n_splits <= 64.
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part, int n_splits,
                                                      int H, float* __restrict__ out,
                                                      float* __restrict__ lse) {
    constexpr int kChunk = 16;  // splits whose channels are loaded per round
    const int lane = threadIdx.x & 63;
    const int64_t bq = blockIdx.x;
    const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int64_t sstride = (int64_t)H * (kHeadDim + 2);
    const float* base = part + (bq * n_splits * H + h) * (kHeadDim + 2);
    float m = -INFINITY, l = 0.0f;
    if (lane < n_splits) {
        m = base[lane * sstride + kHeadDim];
        l = base[lane * sstride + kHeadDim + 1];
    }
    float2 v[kChunk];
#pragma unroll
    for (int s = 0; s < kChunk; ++s)
        v[s] = s < n_splits ? *reinterpret_cast<const float2*>(base + s * sstride + 2 * lane)
                            : make_float2(0.0f, 0.0f);
    const float M = wave_max_dpp(m);
    const float w = (M != -INFINITY && lane < n_splits) ? exp2f(m - M) : 0.0f;  // m = -inf -> 0
    const float L = wave_sum_dpp(l * w);
    float2 acc = make_float2(0.0f, 0.0f);
    for (int s0 = 0; s0 < n_splits; s0 += kChunk) {
        if (s0 > 0) {
#pragma unroll
            for (int s = 0; s < kChunk; ++s)
                v[s] = s0 + s < n_splits
                           ? *reinterpret_cast<const float2*>(base + (s0 + s) * sstride + 2 * lane)
                           : make_float2(0.0f, 0.0f);
        }
#pragma unroll
        for (int s = 0; s < kChunk; ++s) {
            const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s0 + s));
            acc.x += v[s].x * ws;
            acc.y += v[s].y * ws;
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    *reinterpret_cast<float2*>(out + (bq * H + h) * kHeadDim + 2 * lane) =
        make_float2(acc.x * inv, acc.y * inv);
    if (lane == 0) lse[bq * H + h] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

hipError_t launch_attn(const AttnArgs& a, void* ws, size_t, hipStream_t stream) {
    const SplitPlan plan = plan_splits(a.n_q, a.topk, a.swa_rows);
    float* part = static_cast<float*>(ws);
    dim3 grid((unsigned)plan.n_splits, (unsigned)a.n_q);
    const int nw = (a.H + 15) / 16;
    switch (nw) {
        case 1: hipLaunchKernelGGL(k_attn<1>, grid, dim3(64), 0, stream, a, plan, part); break;
        case 2: hipLaunchKernelGGL(k_attn<2>, grid, dim3(128), 0, stream, a, plan, part); break;
        case 3: hipLaunchKernelGGL(k_attn<3>, grid, dim3(192), 0, stream, a, plan, part); break;
        case 4: hipLaunchKernelGGL(k_attn<4>, grid, dim3(256), 0, stream, a, plan, part); break;
        case 5: hipLaunchKernelGGL(k_attn<5>, grid, dim3(320), 0, stream, a, plan, part); break;
        case 6: hipLaunchKernelGGL(k_attn<6>, grid, dim3(384), 0, stream, a, plan, part); break;
        case 7: hipLaunchKernelGGL(k_attn<7>, grid, dim3(448), 0, stream, a, plan, part); break;
        default: hipLaunchKernelGGL(k_attn<8>, grid, dim3(512), 0, stream, a, plan, part); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || plan.n_splits == 1) return err;
    hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)a.n_q, (unsigned)(a.H / 4)), dim3(256), 0,
                       stream, part, plan.n_splits, a.H, a.out, a.lse);
    return hipGetLastError();
}

}  // namespace csa2
