// csa2_quant.hip -- write path: FP4 main KV, FP8 rows (SWA / indexer K), the
// per-call indexer-query quantisation, and the codec probe.
//
// FP4 main KV: "DeepSeek V4.1 Flash: architecture study notes", section 4 (E2M1
// values, one 8-bit E4M3 scale per 16 channels, 4.5 bits per value) and section
// 3 (encoder groups average 2 tokens into 1 entry); "DeepSeek V4.1 Flash is
// live", "CSA2 attention" (compressed entries do not overlap) and "cache
// precision and persistence tiers" (quantise after RoPE, no global scale).
//
// These kernels are bandwidth-trivial (one entry per sequence per decode step,
// 128 per replay chunk); they are written for exactness: every division is an
// IEEE fp32 division and every rounding is spelled out.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

// Entry e by one wave; lane l owns channels 2l and 2l+1 of K and of V, so a
// 16-channel scale group is 8 adjacent lanes and one code byte per lane.
// Indexer key of the entry being written, on the lane that owns output
// channel j = lane: key_j = fp32 chain over input channels c = 0..127 of
// proj[j][c] * x[c], one fused multiply-add per channel, from +0; x[c] is
// read from lane c/2 (k0 for even c, k1 for odd c), wave-uniform.
// The projection, row j at proj[j * kProjPitch]: staged in LDS by the
// workgroup (a pitch of 129 floats keeps the lanes' rows in distinct banks).
constexpr int kProjPitch = kHeadDim + 1;

__device__ __forceinline__ float project_idx_key(const float* proj, float k0, float k1,
                                                 int lane) {
    const float* wr = proj + lane * kProjPitch;
    float acc = 0.0f;
#pragma unroll
    for (int c4 = 0; c4 < kHeadDim / 4; ++c4) {
        const float4 w = make_float4(wr[4 * c4], wr[4 * c4 + 1], wr[4 * c4 + 2], wr[4 * c4 + 3]);
        const float x0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k0), 2 * c4));
        const float x1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k1), 2 * c4));
        const float x2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k0), 2 * c4 + 1));
        const float x3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k1), 2 * c4 + 1));
        acc = __builtin_fmaf(w.x, x0, acc);
        acc = __builtin_fmaf(w.y, x1, acc);
        acc = __builtin_fmaf(w.z, x2, acc);
        acc = __builtin_fmaf(w.w, x3, acc);
    }
    return acc;
}

// FP8 row values already in registers (per = 1 or 2 channels per lane):
// sigma = fl(amax / 448), code = RNE_E4M3(fl(x / sigma)).
__device__ __forceinline__ void quant_fp8_vals(const float* xv, int per, int layout, int64_t row,
                                               uint8_t* __restrict__ codes,
                                               float* __restrict__ sigma, int lane) {
    float amax = fabsf(xv[0]);
    if (per == 2) amax = fmaxf(amax, fabsf(xv[1]));
    amax = wave_max_f32(amax);
    const float s = amax / 448.0f;
    const int dim = per * 64;
    for (int i = 0; i < per; ++i) {
        const uint32_t c = (s == 0.0f) ? ((__float_as_uint(xv[i]) >> 24) & 0x80u)
                                       : e4m3_encode(xv[i] / s);
        const int ch = lane * per + i;
        if (layout == 1) {
            codes[ik_offset(row, ch >> 4) + (ch & 15)] = (uint8_t)c;
        } else {
            codes[row * dim + ch] = (uint8_t)c;
        }
    }
    if (lane == 0) sigma[row] = s;
}

// FP4 indexer key of one row, one channel per lane (lane c = channel c):
// per 16-channel group scale = RNE_E4M3(fl(amax/6)), code = RNE_E2M1(fl(x/scale))
// (signed zero when the scale is 0), the main KV's FP4 rule over 64 channels.
__device__ __forceinline__ void quant_idx4_val(float x, int64_t row, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales, int lane) {
    float amax = fabsf(x);
    amax = fmaxf(amax, dppf<0x128>(amax));  // row_ror:8, the other half of the 16-lane group
    amax = group8_max_f32(amax);
    const uint32_t sc = e4m3_encode(amax / 6.0f);
    const float sd = e4m3_decode_bits(sc);
    const uint32_t code = (sd == 0.0f) ? ((__float_as_uint(x) >> 28) & 8u) : e2m1_encode(x / sd);
    const uint32_t odd = dpp<0xB1>(code);  // the neighbouring lane's code
    if ((lane & 1) == 0)
        codes[ik4_offset(row, lane >> 5) + ((lane & 31) >> 1)] = (uint8_t)(code | (odd << 4));
    if ((lane & 15) == 0) scales[row * 4 + (lane >> 4)] = (uint8_t)sc;
}

// proj (may be null): also the entry's indexer key, projected from its fp32 K
// (after averaging and RoPE) and written in FP8 to ik_codes (tile layout) /
// ik_sigma at the entry's row.
// The inputs of entry e as lane `lane` needs them: its K and V channel pair
// (of both tokens of the pair when ratio is 2), its rotation pair (lanes
// 32..63 load lane - 32's and ignore it) and the destination row.  Every load
// is issued whatever the arguments (an unused one reads a valid word of the
// entry's K row), so that a caller's later waits count them exactly.
struct EntryIn {
    float2 ka, kb, va, vb;  // kb, vb: second token (ratio 2)
    float2 cs;
    int64_t r, e;  // the loaded destination row (used when has_rows), the entry
    bool has_rows;
    __device__ __forceinline__ int64_t row() const { return has_rows ? r : e; }
};

__device__ __forceinline__ EntryIn load_fp4_entry(const float* __restrict__ k,
                                                  const float* __restrict__ v, int64_t e,
                                                  int ratio, const float* __restrict__ rope_cs,
                                                  const int64_t* __restrict__ dst_rows, int lane) {
    EntryIn in;
    const int64_t t0 = ratio == 1 ? e : 2 * e, t1 = ratio == 1 ? t0 : t0 + 1;
    const float* krow = k + t0 * kHeadDim;
    in.ka = reinterpret_cast<const float2*>(krow)[lane];
    in.va = reinterpret_cast<const float2*>(v + t0 * kHeadDim)[lane];
    in.kb = reinterpret_cast<const float2*>(k + t1 * kHeadDim)[lane];
    in.vb = reinterpret_cast<const float2*>(v + t1 * kHeadDim)[lane];
    in.cs = reinterpret_cast<const float2*>(rope_cs != nullptr ? rope_cs + e * 64 : krow)[lane & 31];
    in.r = *(dst_rows != nullptr ? dst_rows + e : reinterpret_cast<const int64_t*>(krow));
    in.e = e;
    in.has_rows = dst_rows != nullptr;
    return in;
}

__device__ __forceinline__ void quant_fp4_entry(const EntryIn& in, int ratio, bool rope,
                                                uint8_t* __restrict__ codes,
                                                uint8_t* __restrict__ scales, int lane,
                                                const float* __restrict__ proj = nullptr,
                                                uint8_t* __restrict__ ik_codes = nullptr,
                                                float* __restrict__ ik_sigma = nullptr,
                                                uint8_t* __restrict__ ik_scales4 = nullptr) {
    float k0, k1, v0, v1;
    if (ratio == 1) {
        k0 = in.ka.x; k1 = in.ka.y; v0 = in.va.x; v1 = in.va.y;
    } else {
        // mean of tokens 2e and 2e+1: fl(fl(a + b) * 0.5)
        k0 = (in.ka.x + in.kb.x) * 0.5f; k1 = (in.ka.y + in.kb.y) * 0.5f;
        v0 = (in.va.x + in.vb.x) * 0.5f; v1 = (in.va.y + in.vb.y) * 0.5f;
    }
    if (rope && lane < 32) {
        // rotate the interleaved pair (2l, 2l+1) of the first 64 K channels
        const float a = k0 * in.cs.x, b = k1 * in.cs.y, c = k0 * in.cs.y, d = k1 * in.cs.x;
        k0 = a - b;
        k1 = c + d;
    }

    // per-group absolute maximum over 8 lanes x 2 channels
    const float kmax = group8_max_f32(fmaxf(fabsf(k0), fabsf(k1)));
    const float vmax = group8_max_f32(fmaxf(fabsf(v0), fabsf(v1)));
    const uint32_t ksc = e4m3_encode(kmax / 6.0f);
    const uint32_t vsc = e4m3_encode(vmax / 6.0f);
    const float ksd = e4m3_decode_bits(ksc);
    const float vsd = e4m3_decode_bits(vsc);

    auto code = [](float x, float sd) -> uint32_t {
        if (sd == 0.0f) return (__float_as_uint(x) >> 28) & 8u;  // signed zero
        return e2m1_encode(x / sd);
    };
    const uint32_t kb = code(k0, ksd) | (code(k1, ksd) << 4);
    const uint32_t vb = code(v0, vsd) | (code(v1, vsd) << 4);

    const int64_t row = in.row();
    if (proj != nullptr) {
        const float key[1] = {project_idx_key(proj, k0, k1, lane)};
        if (ik_scales4 != nullptr) quant_idx4_val(key[0], row, ik_codes, ik_scales4, lane);
        else quant_fp8_vals(key, 1, 1, row, ik_codes, ik_sigma, lane);
    }
    codes[row * 128 + lane] = (uint8_t)kb;
    codes[row * 128 + 64 + lane] = (uint8_t)vb;
    if ((lane & 7) == 0) {
        scales[row * 16 + (lane >> 3)] = (uint8_t)ksc;
        scales[row * 16 + 8 + (lane >> 3)] = (uint8_t)vsc;
    }
}

__global__ __launch_bounds__(256) void k_quant_fp4(const float* __restrict__ k,
                                                   const float* __restrict__ v, int64_t n_ent,
                                                   int ratio, const float* __restrict__ rope_cs,
                                                   const int64_t* __restrict__ dst_rows,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales) {
    const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= n_ent) return;  // uniform over the wave
    const int lane = threadIdx.x & 63;
    quant_fp4_entry(load_fp4_entry(k, v, e, ratio, rope_cs, dst_rows, lane), ratio,
                    rope_cs != nullptr, codes, scales, lane);
}

// Row r of 64 or 128 values by one wave.
__device__ __forceinline__ void quant_fp8_row(const float* __restrict__ x, int64_t r, int dim,
                                              int layout, const int64_t* __restrict__ dst_rows,
                                              uint8_t* __restrict__ codes,
                                              float* __restrict__ sigma, int lane) {
    const int per = dim / 64;  // channels per lane: 1 or 2
    float xv[2] = {0.0f, 0.0f};
    for (int i = 0; i < per; ++i) xv[i] = x[r * dim + lane * per + i];
    const int64_t row = dst_rows ? dst_rows[r] : r;
    quant_fp8_vals(xv, per, layout, row, codes, sigma, lane);
}

__global__ __launch_bounds__(256) void k_quant_fp8(const float* __restrict__ x, int64_t n_rows,
                                                   int dim, int layout,
                                                   const int64_t* __restrict__ dst_rows,
                                                   uint8_t* __restrict__ codes,
                                                   float* __restrict__ sigma) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n_rows) return;  // uniform over the wave
    quant_fp8_row(x, r, dim, layout, dst_rows, codes, sigma, threadIdx.x & 63);
}

__global__ __launch_bounds__(256) void k_quant_idx4(const float* __restrict__ x, int64_t n_rows,
                                                    const int64_t* __restrict__ dst_rows,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n_rows) return;  // uniform over the wave
    const int lane = threadIdx.x & 63;
    quant_idx4_val(x[r * 64 + lane], dst_rows ? dst_rows[r] : r, codes, scales, lane);
}

// The write path of new entries in one launch: wave w < n_ent quantises entry
// w as k_quant_fp4 does, the following waves the rows of the FP8 jobs in
// order, each as k_quant_fp8 does.
__global__ __launch_bounds__(256) void k_write_entries(Fp4Job f, Fp8Jobs j) {
    __shared__ float proj_l[kIdxDim * kProjPitch];
    const int lane = threadIdx.x & 63;
    int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    // a workgroup holding entry waves stages the projection once, with every
    // thread (uniform over the workgroup, before any wave leaves)
    const bool stage = f.proj != nullptr && (int64_t)blockIdx.x * 4 < f.n_ent;
    // the projection rows (all eight 16-byte loads of each thread at once)
    // and an entry wave's own inputs go out together, before any wait
    constexpr int kPer = kIdxDim * kHeadDim / 4 / 256;
    static_assert(kPer * 256 * 4 == kIdxDim * kHeadDim, "the projection splits evenly");
    float4 pv[kPer];
    if (stage) {
#pragma unroll
        for (int r = 0; r < kPer; ++r)
            pv[r] = reinterpret_cast<const float4*>(f.proj)[threadIdx.x + 256 * r];
    }
    EntryIn in;
    if (w < f.n_ent) in = load_fp4_entry(f.k, f.v, w, f.ratio, f.rope_cs, f.dst_rows, lane);
    if (stage) {
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int i = threadIdx.x + 256 * r;
            float* d = proj_l + (i / (kHeadDim / 4)) * kProjPitch + 4 * (i % (kHeadDim / 4));
            d[0] = pv[r].x; d[1] = pv[r].y; d[2] = pv[r].z; d[3] = pv[r].w;
        }
        __syncthreads();
    }
    if (w < f.n_ent) {
        quant_fp4_entry(in, f.ratio, f.rope_cs != nullptr, f.codes, f.scales, lane,
                        stage ? proj_l : nullptr, f.ik_codes, f.ik_sigma, f.ik_scales4);
        return;
    }
    w -= f.n_ent;
#pragma unroll
    for (int i = 0; i < kMaxFp8Jobs; ++i) {
        if (i < j.n && w < j.job[i].n_rows) {
            const Fp8Job& b = j.job[i];
            quant_fp8_row(b.x, w, b.dim, b.layout, b.dst_rows, b.codes, b.sigma, lane);
            return;
        }
        if (i < j.n) w -= j.job[i].n_rows;
    }
}

// Indexer query per (sequence, query): per head sq = fl(amax/448), codes
// RNE_E4M3(fl(q/sq)) stored back as their exact fp32 values, and the head
// weight with the scale folded in, w' = fl(w * sq).  One workgroup per query,
// one wave per head, lane = channel.
__global__ __launch_bounds__(256) void k_prep_iq(const float* __restrict__ iq,
                                                 const float* __restrict__ iw, int64_t n_q,
                                                 float* __restrict__ qd, float* __restrict__ wq,
                                                 float* __restrict__ cq,
                                                 _Float16* __restrict__ qh) {
    __shared__ float sd[kIdxHeads];
    const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
    const int64_t bq = blockIdx.x;
    if (bq >= n_q) return;
    const float x = iq[(bq * kIdxHeads + h) * kIdxDim + lane];
    const float wh = iw[bq * kIdxHeads + h];  // loaded with the query, not after it
    float sq;
    const float v = quantise_query_channel(x, sq);
    qd[(bq * kIdxHeads + h) * kIdxDim + lane] = v;
    if (qh != nullptr) qh[(bq * kIdxHeads + h) * kIdxDim + lane] = (_Float16)v;  // exact
    const float w = wh * sq;
    if (lane == 0) wq[bq * kIdxHeads + h] = w;
    if (cq != nullptr) {
        // guard-band constant of the MFMA scan (csa2_chunk.hip):
        // C'_q = (1 + 2^-10) (2^-16 + 2^-18) 448 sum_h |w'_h| ||q_h||_1
        float l1 = fabsf(v);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) l1 += __shfl_xor(l1, o, 64);
        if (lane == 0) sd[h] = fabsf(w) * ((0x1p-16f + 0x1p-18f) * 448.0f * l1);
        __syncthreads();
        if (threadIdx.x == 0) cq[bq] = (sd[0] + sd[1] + sd[2] + sd[3]) * (1.0f + 0x1p-10f);
    }
}

// Codec probe: decode every E4M3 code with the fp32 converter of the scan and
// the fp16 converter of the attention, every (E2M1 code, E4M3 scale) pair
// with the attention's FP4 path, and run both encoders on caller values.
__global__ __launch_bounds__(256) void k_codec_probe(float* __restrict__ e4m3_dec,
                                                     float* __restrict__ e4m3_dec16,
                                                     float* __restrict__ fp4_dec16,
                                                     const float* __restrict__ x, int64_t n,
                                                     uint8_t* __restrict__ e4m3_enc,
                                                     uint8_t* __restrict__ e2m1_enc) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < 128) {
        const uint32_t packed = (uint32_t)(2 * t) | ((uint32_t)(2 * t + 1) << 8);
        const float2 f = e4m3x2_to_f32<false>(packed);
        e4m3_dec[2 * t] = f.x;
        e4m3_dec[2 * t + 1] = f.y;
    }
    if (t < 256) {
        e4m3_dec16[t] = (float)e4m3_to_f16((uint32_t)t);
        // scale byte t, all 16 codes: dword 0x76543210 and 0xFEDCBA98 hold codes 0..15
        _Float16 v[16];
        const _Float16 sc = e4m3_to_f16((uint32_t)t);
        fp4x8_to_f16(0x76543210u, sc, v);
        fp4x8_to_f16(0xFEDCBA98u, sc, v + 8);
        for (int c = 0; c < 16; ++c) fp4_dec16[t * 16 + c] = (float)v[c];
    }
    if (t < n) {
        e4m3_enc[t] = (uint8_t)e4m3_encode(x[t]);
        e2m1_enc[t] = (uint8_t)e2m1_encode(x[t]);
    }
}

hipError_t launch_quant_fp4(const float* k, const float* v, int64_t n_ent, int ratio,
                            const float* rope_cs, const int64_t* dst_rows, uint8_t* codes,
                            uint8_t* scales, hipStream_t stream) {
    if (n_ent == 0) return hipSuccess;
    const unsigned grid = (unsigned)((n_ent + 3) / 4);
    hipLaunchKernelGGL(k_quant_fp4, dim3(grid), dim3(256), 0, stream, k, v, n_ent, ratio, rope_cs,
                       dst_rows, codes, scales);
    return hipGetLastError();
}

hipError_t launch_quant_fp8(const float* x, int64_t n_rows, int dim, int layout,
                            const int64_t* dst_rows, uint8_t* codes, float* sigma,
                            hipStream_t stream) {
    if (n_rows == 0) return hipSuccess;
    const unsigned grid = (unsigned)((n_rows + 3) / 4);
    hipLaunchKernelGGL(k_quant_fp8, dim3(grid), dim3(256), 0, stream, x, n_rows, dim, layout,
                       dst_rows, codes, sigma);
    return hipGetLastError();
}

hipError_t launch_quant_idx4(const float* x, int64_t n_rows, const int64_t* dst_rows,
                             uint8_t* codes, uint8_t* scales, hipStream_t stream) {
    if (n_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(k_quant_idx4, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, stream, x,
                       n_rows, dst_rows, codes, scales);
    return hipGetLastError();
}

hipError_t launch_write_entries(const Fp4Job& f, const Fp8Jobs& j, hipStream_t stream) {
    int64_t waves = f.n_ent;
    for (int i = 0; i < j.n; ++i) waves += j.job[i].n_rows;
    if (waves == 0) return hipSuccess;
    const unsigned grid = (unsigned)((waves + 3) / 4);
    hipLaunchKernelGGL(k_write_entries, dim3(grid), dim3(256), 0, stream, f, j);
    return hipGetLastError();
}

hipError_t launch_prep_iq(const float* iq, const float* iw, int64_t n_q, float* qd, float* wq,
                          hipStream_t stream, float* cq, _Float16* qh) {
    hipLaunchKernelGGL(k_prep_iq, dim3((unsigned)n_q), dim3(256), 0, stream, iq, iw, n_q, qd, wq,
                       cq, qh);
    return hipGetLastError();
}

hipError_t launch_codec_probe(float* e4m3_dec, float* e4m3_dec16, float* fp4_dec16,
                              const float* x, int64_t n, uint8_t* e4m3_enc, uint8_t* e2m1_enc,
                              hipStream_t stream) {
    const int64_t threads = n > 256 ? n : 256;
    const unsigned grid = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(k_codec_probe, dim3(grid), dim3(256), 0, stream, e4m3_dec, e4m3_dec16,
                       fp4_dec16, x, n, e4m3_enc, e2m1_enc);
    return hipGetLastError();
}

}  // namespace csa2
