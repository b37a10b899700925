// csa2_attn.hip -- CSA2 sparse attention over the FP4 global KV plus the FP8
// sliding window.
//
// "DeepSeek V4.1 Flash: architecture study notes", section 2: each query
// attends to at most 512 selected global records together with its local
// window; section 1: the window is 128 tokens and every layer keeps its own;
// section 4: the FP4 cache is dequantised on read and fed to ordinary
// attention (the saving is storage, not FP4 arithmetic); the SWA KV stays FP8.
//
// Design (gfx950): one workgroup per (query, split of the entry list), one
// wave per 16 heads.  All heads of a query share one KV head (MQA), so the
// logits are a dense [heads x entries] contraction and go to MFMA
// (v_mfma_f32_16x16x32_f16):
//   - dequantised E2M1 x E4M3 values have at most 6 significant bits and lie
//     in [2^-10, 2688], so they are exact in fp16; E4M3 window codes are exact
//     in fp16 and their fp32 row scale is applied to the logit (K) or to the
//     probability (V) in fp32;
//   - q is split into fp16 hi + lo parts, so q.k carries ~22 bits;
//   - accumulation is fp32, softmax is online in fp32 (base-2 exponentials).
// Per 32-entry tile the workgroup gathers the selected records (128 code
// bytes + 16 scale bytes each), dequantises them into LDS (K row-major, V
// transposed), and each wave computes S^T = K Q^T, rescales its running
// output, and accumulates O^T += V^T P^T with P taken straight from the S^T
// registers (entry order inside the k dimension is permuted consistently).
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;          // entries per tile
constexpr int kKPitch = 136;       // fp16 per K row in LDS (128 + 8)
constexpr int kVPitch = 40;        // fp16 per V^T row in LDS (32 + 8)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct SplitPlan {
    int n_tiles_global;  // ceil(topk / 32)
    int n_tiles;         // global + window tiles
    int n_splits;
    int tiles_per_split;
};

static SplitPlan plan_splits(int64_t n_q, int topk, int swa_rows) {
    SplitPlan p;
    p.n_tiles_global = (topk + kTile - 1) / kTile;
    p.n_tiles = p.n_tiles_global + (swa_rows + kTile - 1) / kTile;
    int64_t want = (512 + n_q - 1) / n_q;  // aim for >= 512 workgroups
    int64_t max_splits = p.n_tiles / 2 > 0 ? p.n_tiles / 2 : 1;
    int64_t ns = want < max_splits ? want : max_splits;
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

template <int NW>
__global__ __launch_bounds__(NW * 64) void k_attn(AttnArgs a, SplitPlan plan,
                                                  float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) _Float16 sK[kTile * kKPitch];
    __shared__ __attribute__((aligned(16))) _Float16 sVt[kHeadDim * kVPitch];
    __shared__ float sKmul[kTile];
    __shared__ float sVmul[kTile];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bq = blockIdx.y;
    const int split = blockIdx.x;
    const int64_t b = bq / a.Q;
    const int H = a.H;
    const int head = wave * 16 + (lane & 15);
    const int g = lane >> 4;
    const float logit_mul = a.sm_scale * kLog2e;

    int swa_len;
    if (a.swa_len != nullptr) {
        swa_len = a.swa_len[b];
        swa_len = swa_len < 0 ? 0 : (swa_len > a.swa_rows ? a.swa_rows : swa_len);
    } else {
        swa_len = (int)(bq % a.Q) + 1;
    }

    // ---- q as fp16 hi/lo in B-operand layout: head, dims 32ks + 8g .. +8 ----
    half8_t qhi[4], qlo[4];
    {
        const float* qrow = a.q + (bq * H + head) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const float4 x0 = *reinterpret_cast<const float4*>(qrow + 32 * ks + 8 * g);
            const float4 x1 = *reinterpret_cast<const float4*>(qrow + 32 * ks + 8 * g + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const _Float16 h = (_Float16)xs[i];
                qhi[ks][i] = h;
                qlo[ks][i] = (_Float16)(xs[i] - (float)h);
            }
        }
    }

    float4_t o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    const int t_beg = split * plan.tiles_per_split;
    const int t_end = min(plan.n_tiles, t_beg + plan.tiles_per_split);
    const int32_t* idx = a.idx + bq * a.topk;

    for (int tile = t_beg; tile < t_end; ++tile) {
        // ---- gather + dequantise 32 entries into LDS ----
        for (int task = tid; task < kTile * 8; task += NW * 64) {
            const int e = task >> 3, part = task & 7;
            const bool is_v = part >= 4;
            const int cpart = part & 3;  // 32-channel quarter
            _Float16 vals[32];
            bool valid = false;
            float kmul = 0.0f, vmul = 0.0f;
            if (tile < plan.n_tiles_global) {
                const int slot = tile * kTile + e;
                const int32_t pos = slot < a.topk ? idx[slot] : -1;
                valid = pos >= 0 && pos < a.cap;
                if (valid) {
                    const int64_t row = b * a.cap + pos;
                    const uint4 c = *reinterpret_cast<const uint4*>(a.kvc + row * 128 + (is_v ? 64 : 0) + 16 * cpart);
                    const uint16_t sc = *reinterpret_cast<const uint16_t*>(a.kvs + row * 16 + (is_v ? 8 : 0) + 2 * cpart);
                    const float s0 = e4m3_decode_bits(sc & 0xFFu), s1 = e4m3_decode_bits(sc >> 8);
                    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const uint32_t byte = (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;
                        const float s = j < 8 ? s0 : s1;
                        vals[2 * j] = (_Float16)(e2m1_to_f32(byte & 0xFu) * s);
                        vals[2 * j + 1] = (_Float16)(e2m1_to_f32(byte >> 4) * s);
                    }
                    kmul = logit_mul;
                    vmul = 1.0f;
                }
            } else {
                const int t = (tile - plan.n_tiles_global) * kTile + e;
                valid = t < swa_len;
                if (valid) {
                    const int64_t row = b * a.swa_rows + t;
                    const uint8_t* src = (is_v ? a.swv : a.swk) + row * kHeadDim + 32 * cpart;
                    const uint4 c0 = *reinterpret_cast<const uint4*>(src);
                    const uint4 c1 = *reinterpret_cast<const uint4*>(src + 16);
                    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float2 lo = e4m3x2_to_f32<false>(w[j]);
                        const float2 hi = e4m3x2_to_f32<true>(w[j]);
                        vals[4 * j + 0] = (_Float16)lo.x;
                        vals[4 * j + 1] = (_Float16)lo.y;
                        vals[4 * j + 2] = (_Float16)hi.x;
                        vals[4 * j + 3] = (_Float16)hi.y;
                    }
                    kmul = a.swks[row] * logit_mul;
                    vmul = a.swvs[row];
                }
            }
            if (!valid) {
#pragma unroll
                for (int j = 0; j < 32; ++j) vals[j] = (_Float16)0.0f;
            }
            if (!is_v) {
                half8_t* dst = reinterpret_cast<half8_t*>(sK + e * kKPitch + 32 * cpart);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    half8_t h;
#pragma unroll
                    for (int i = 0; i < 8; ++i) h[i] = vals[8 * j + i];
                    dst[j] = h;
                }
                if (cpart == 0) sKmul[e] = valid ? kmul : -INFINITY;
            } else {
#pragma unroll
                for (int j = 0; j < 32; ++j) sVt[(32 * cpart + j) * kVPitch + e] = vals[j];
                if (cpart == 0) sVmul[e] = vmul;
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
            float x[8];
            float tmax = -INFINITY;
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = 16 * sub + 4 * g + r;
                    const float km = sKmul[e];
                    const float v = (km == -INFINITY) ? -INFINITY : s[sub][r] * km;
                    x[4 * sub + r] = v;
                    tmax = fmaxf(tmax, v);
                }
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
                    const int e = (i < 4) ? (4 * g + i) : (16 + 4 * g + i - 4);
                    pb[i] = (_Float16)(p * sVmul[e]);
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

// Combine the per-split partials of one query: grid n_q, 128 threads (one
// per channel), loop over heads.
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ part, int n_splits,
                                                      int H, float* __restrict__ out,
                                                      float* __restrict__ lse) {
    const int64_t bq = blockIdx.x;
    const int d = threadIdx.x;
    for (int h = 0; h < H; ++h) {
        const float* base = part + (bq * n_splits * H + h) * (kHeadDim + 2);
        const int64_t sstride = (int64_t)H * (kHeadDim + 2);
        float M = -INFINITY;
        for (int s = 0; s < n_splits; ++s) M = fmaxf(M, base[s * sstride + kHeadDim]);
        float L = 0.0f, acc = 0.0f;
        if (M != -INFINITY) {
            for (int s = 0; s < n_splits; ++s) {
                const float m = base[s * sstride + kHeadDim];
                const float w = exp2f(m - M);  // m = -inf -> 0
                L += base[s * sstride + kHeadDim + 1] * w;
                acc += base[s * sstride + d] * w;
            }
        }
        out[(bq * H + h) * kHeadDim + d] = L > 0.0f ? acc / L : 0.0f;
        if (d == 0) lse[bq * H + h] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
}

hipError_t launch_attn(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
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
    hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)a.n_q), dim3(128), 0, stream, part,
                       plan.n_splits, a.H, a.out, a.lse);
    return hipGetLastError();
}

}  // namespace csa2
