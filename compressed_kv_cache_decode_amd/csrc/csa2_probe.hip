// csa2_probe.hip -- bandwidth probes for measurement: a read-only pass and a
// copy over a device buffer, and a memory-only pass with the gathering
// attention's access pattern, the ceilings the hot path's kernels are
// compared with in the same run.  Not part of the attention or indexer
// arithmetic.
//
// Modes 0 (read) and 1 (copy): each thread keeps four 16-byte non-temporal
// loads in flight per step of a grid-stride loop over n_blocks workgroups;
// the read pass folds what it loads into one XOR per thread and writes one
// word per workgroup, so the loads cannot be dropped.  Mode 2 (read): one
// 16-byte load per thread over a grid that covers the buffer.  Mode 3 (read):
// one 16 KB chunk per workgroup, four 16-byte loads per thread 4 KB apart (the
// indexer scan's access: a 256-position tile of 64-byte rows), a grid that
// covers the buffer.
#include <hip/hip_ext.h>

#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const u32x4_t* __restrict__ src,
                                                               int64_t n16, uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4_t v = __builtin_nontemporal_load(src + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    __shared__ uint32_t red[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(kProbeThreads) void k_stream_copy(const u32x4_t* __restrict__ src,
                                                               u32x4_t* __restrict__ dst,
                                                               int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// one 16-byte load per thread, a grid that covers the whole buffer
__global__ __launch_bounds__(kProbeThreads) void k_stream_read1(const u32x4_t* __restrict__ src,
                                                                int64_t n16, uint32_t* sink) {
    const int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t acc = 0;
    if (i < n16) {
        const u32x4_t v = __builtin_nontemporal_load(src + i);
        acc = v[0] ^ v[1] ^ v[2] ^ v[3];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if ((threadIdx.x & 63) == 0 && acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads
}

// one 16 KB chunk per workgroup, four 16-byte loads per thread, a grid that
// covers the whole buffer
__global__ __launch_bounds__(kProbeThreads) void k_stream_read_chunk(const u32x4_t* __restrict__ src,
                                                                     int64_t n16, uint32_t* sink) {
    const int64_t i0 = (int64_t)blockIdx.x * (kProbeUnroll * kProbeThreads) + threadIdx.x;
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
        const int64_t i = i0 + u * kProbeThreads;
        v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if ((threadIdx.x & 63) == 0 && acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads
}

// Memory-only pass with the gathering decode attention's access pattern: per
// query, the topk selected records (128 code bytes and 16 scale bytes at each
// position of idx; -1 or past cap: skipped), the 128-row FP8 window (K and V
// codes, fp32 scales) and the H x 128 fp32 query are read, and an H x 128
// row written.  One workgroup of 256 threads per query; the positions first,
// then the window, then the records, 512 per round: eight lanes take the 128
// code bytes of a record, one lane its 16 scale bytes.  Every word of the
// output row holds word (i mod 4) of the XOR of every 16-byte unit read for
// the query, so a test can tell that nothing was skipped.
constexpr int kGatherThreads = 256;

__global__ __launch_bounds__(kGatherThreads) void k_gather_probe(
    const uint8_t* __restrict__ kvc, const uint8_t* __restrict__ kvs,
    const int32_t* __restrict__ idx, int topk, int64_t cap, const uint8_t* __restrict__ swk,
    const uint8_t* __restrict__ swv, const float* __restrict__ swks,
    const float* __restrict__ swvs, const float* __restrict__ q, int H, float* __restrict__ out) {
    const int64_t bq = blockIdx.x;
    const int t = threadIdx.x;
    const uint8_t* codes = kvc + bq * cap * 128;
    const uint8_t* scales = kvs + bq * cap * 16;
    const int32_t* row = idx + bq * topk;
    auto sanitize = [&](int slot) -> int64_t {
        const int32_t p = slot < topk ? row[slot] : -1;
        return (p >= 0 && p < cap) ? p : -1;
    };
    u32x4_t acc = {0u, 0u, 0u, 0u};
    const u32x4_t* wk = reinterpret_cast<const u32x4_t*>(swk + bq * 128 * 128);
    const u32x4_t* wv = reinterpret_cast<const u32x4_t*>(swv + bq * 128 * 128);
    for (int c0 = 0; c0 < topk; c0 += 512) {
        int64_t pos[16], ps[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) pos[i] = sanitize(c0 + 32 * i + (t >> 3));
#pragma unroll
        for (int j = 0; j < 2; ++j) ps[j] = sanitize(c0 + 256 * j + t);
        if (c0 == 0) {  // the window's 2 x 1024 units, 8 per thread
#pragma unroll
            for (int i = 0; i < 4; ++i) acc ^= wk[i * kGatherThreads + t] ^ wv[i * kGatherThreads + t];
        }
        u32x4_t r[16], sc[2];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            r[i] = pos[i] >= 0 ? *reinterpret_cast<const u32x4_t*>(codes + pos[i] * 128 + 16 * (t & 7))
                               : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 2; ++j)
            sc[j] = ps[j] >= 0 ? *reinterpret_cast<const u32x4_t*>(scales + ps[j] * 16)
                               : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) acc ^= r[i];
        acc ^= sc[0] ^ sc[1];
    }
    if (topk <= 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc ^= wk[i * kGatherThreads + t] ^ wv[i * kGatherThreads + t];
    }
    if (t < 32) acc ^= reinterpret_cast<const u32x4_t*>(swks + bq * 128)[t];
    else if (t < 64) acc ^= reinterpret_cast<const u32x4_t*>(swvs + bq * 128)[t - 32];
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(q + bq * H * 128);
    for (int j = t; j < H * 32; j += kGatherThreads) acc ^= qp[j];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w] ^= (uint32_t)__shfl_xor((int)acc[w], o, 64);
    __shared__ u32x4_t red[kGatherThreads / 64];
    if ((t & 63) == 0) red[t >> 6] = acc;
    __syncthreads();
    acc = red[0] ^ red[1] ^ red[2] ^ red[3];
    u32x4_t* op = reinterpret_cast<u32x4_t*>(out + bq * H * 128);
    for (int j = t; j < H * 32; j += kGatherThreads) op[j] = acc;
}

hipError_t launch_gather_probe(const uint8_t* kvc, const uint8_t* kvs, const int32_t* idx,
                               int n_q, int topk, int64_t cap, const uint8_t* swk,
                               const uint8_t* swv, const float* swks, const float* swvs,
                               const float* q, int H, float* out, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop) {
    if (n_q <= 0) return hipSuccess;
    if (start != nullptr && stop != nullptr)
        hipExtLaunchKernelGGL(k_gather_probe, dim3((unsigned)n_q), dim3(kGatherThreads), 0, stream,
                              start, stop, 0, kvc, kvs, idx, topk, cap, swk, swv, swks, swvs, q,
                              H, out);
    else
        hipLaunchKernelGGL(k_gather_probe, dim3((unsigned)n_q), dim3(kGatherThreads), 0, stream,
                           kvc, kvs, idx, topk, cap, swk, swv, swks, swvs, q, H, out);
    return hipGetLastError();
}

hipError_t launch_stream_probe(int mode, const void* src, void* dst, size_t n_bytes,
                               uint32_t* sink, int n_blocks, hipStream_t stream) {
    const int64_t n16 = (int64_t)(n_bytes / 16);
    if (mode == 2 || mode == 3) {
        const int64_t per = mode == 2 ? kProbeThreads : kProbeUnroll * kProbeThreads;
        const int64_t blocks = (n16 + per - 1) / per;
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL(mode == 2 ? k_stream_read1 : k_stream_read_chunk, dim3((unsigned)blocks),
                           dim3(kProbeThreads), 0, stream, static_cast<const u32x4_t*>(src), n16,
                           sink);
        return hipGetLastError();
    }
    if (mode == 0)
        hipLaunchKernelGGL(k_stream_read, dim3(n_blocks), dim3(kProbeThreads), 0, stream,
                           static_cast<const u32x4_t*>(src), n16, sink);
    else
        hipLaunchKernelGGL(k_stream_copy, dim3(n_blocks), dim3(kProbeThreads), 0, stream,
                           static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
    return hipGetLastError();
}

}  // namespace csa2
