// csa2_abi.cpp -- the extern "C" boundary of libcsa2 (declared in include/csa2.h).
//
// Every entry point validates its scalar arguments on the host first and
// returns a status without touching the HIP runtime when they are invalid;
// only then are kernels enqueued on the caller's stream.  No entry point
// allocates, frees, synchronises or keeps state.
#include <stdint.h>
#include <string.h>

#include <cmath>
#include <mutex>

#include <hip/hip_runtime.h>

#include "csa2.h"
#include "csa2_internal.hpp"

using namespace csa2;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct IndexLayout {
    size_t qd, wq, keys, bkeys, sbkeys, parts, total;
    // MFMA chunk path only
    size_t cq, qh, hkeys_hi;
};

// A multi-query Full layer without a pool output (the replay chunk) scores on
// MFMA with guard bands (csa2_chunk.hip); otherwise the exact VALU scan.
bool mma_path(int Q, int64_t cap, int pool_blocks, int topk) {
    return Q >= 4 && topk <= kChunkMaxTopk &&
           (pool_blocks == 0 || cap / 8 <= kChunkPoolMaxBlocks);
}

// workspace of csa2_index_full: decoded query, folded weights, per-position
// keys, per-block keys, per-superblock keys; on the MFMA path also the guard constants, the fp16
// queries and the upper-bound keys per half-block of 4 (the lower bounds use
// the per-block keys; the per-position keys serve the exact fallback)
IndexLayout full_layout(int B, int Q, int64_t cap, int topk, int pool_blocks) {
    IndexLayout L{};
    const size_t nq = (size_t)B * Q;
    size_t off = 0;
    L.qd = off; off += align_up(nq * 256 * sizeof(float));
    L.wq = off; off += align_up(nq * 4 * sizeof(float));
    L.keys = off; off += align_up(nq * (size_t)cap * sizeof(uint32_t));
    L.bkeys = off; off += align_up(nq * (size_t)(cap / 8) * sizeof(uint32_t));
    L.sbkeys = off; off += align_up(nq * (size_t)(cap / kSuper) * sizeof(uint32_t));
    if (mma_path(Q, cap, pool_blocks, topk)) {
        L.cq = off; off += align_up(nq * sizeof(float));
        L.qh = off; off += align_up(nq * 256 * sizeof(uint16_t));
        L.hkeys_hi = off; off += align_up(nq * (size_t)(cap / 4) * sizeof(uint32_t));
    }
    L.total = off;
    return L;
}

// workspace of csa2_index_reindex: pool keys, and a 16-byte summary per 64
// of them
IndexLayout reindex_layout(int B, int Q, int pool_blocks) {
    IndexLayout L{};
    const size_t nq = (size_t)B * Q;
    size_t off = 0;
    L.keys = off; off += align_up(nq * (size_t)pool_blocks * 8 * sizeof(uint32_t));
    L.parts = off; off += align_up(nq * (size_t)((pool_blocks * 8 + 63) / 64) * 16);
    L.total = off;
    return L;
}

int check_cache_dims(int64_t cap, int B, int Q) {
    if (cap <= 0 || B <= 0 || Q <= 0) return CSA2_E_ARG;
    if (cap % CSA2_IDX_TILE != 0) return CSA2_E_ARG;
    if (cap > (int64_t)INT32_MAX) return CSA2_E_UNSUPPORTED;  // positions are int32
    if (B > 65535) return CSA2_E_UNSUPPORTED;                 // grid.y
    if ((int64_t)B * Q > (int64_t)INT32_MAX) return CSA2_E_UNSUPPORTED;
    return CSA2_OK;
}

int validate_index_full(const void* ikc, const void* iks, int64_t cap, int B, int Q,
                        const void* iq, const void* iw, const void* n_vis, int topk,
                        int pool_blocks, const void* topk_idx, const void* pool_idx) {
    if (!ikc || !iks || !iq || !iw || !n_vis || !topk_idx) return CSA2_E_ARG;
    if (pool_blocks < 0) return CSA2_E_ARG;
    if (pool_blocks > 0 && !pool_idx) return CSA2_E_ARG;
    int rc = check_cache_dims(cap, B, Q);
    if (rc) return rc;
    if (topk < 1) return CSA2_E_ARG;
    if (topk > CSA2_MAX_TOPK) return CSA2_E_UNSUPPORTED;
    if (pool_blocks > CSA2_MAX_POOL_BLOCKS) return CSA2_E_UNSUPPORTED;
    if (pool_blocks > 0 && pool_blocks < topk) return CSA2_E_UNSUPPORTED;
    return CSA2_OK;
}

int validate_index_reindex(const void* ikc, const void* iks, int64_t cap, int B, int Q,
                           const void* iq, const void* iw, const void* n_vis, const void* pool,
                           int pool_blocks, int topk, const void* topk_idx) {
    if (!ikc || !iks || !iq || !iw || !n_vis || !pool || !topk_idx) return CSA2_E_ARG;
    int rc = check_cache_dims(cap, B, Q);
    if (rc) return rc;
    if (pool_blocks < 1 || topk < 1) return CSA2_E_ARG;
    if (pool_blocks > CSA2_MAX_POOL_BLOCKS || topk > CSA2_MAX_TOPK) return CSA2_E_UNSUPPORTED;
    if ((int64_t)B * Q > 65535) return CSA2_E_UNSUPPORTED;  // one grid row per query
    return CSA2_OK;
}

int validate_attn(const void* q, int B, int Q, int H, const void* kvc, const void* kvs,
                  int64_t cap, const void* idx, int topk, const void* swk, const void* swv,
                  const void* swks, const void* swvs, float sm_scale, const void* out,
                  const void* lse) {
    if (!q || !kvc || !kvs || !swk || !swv || !swks || !swvs || !out || !lse) return CSA2_E_ARG;
    if (topk < 0) return CSA2_E_ARG;
    if (topk > 0 && !idx) return CSA2_E_ARG;
    if (topk > CSA2_MAX_TOPK) return CSA2_E_UNSUPPORTED;
    if (B <= 0 || Q <= 0 || H <= 0 || cap <= 0) return CSA2_E_ARG;
    if (H % 16 != 0) return CSA2_E_UNSUPPORTED;
    if (H > CSA2_MAX_HEADS) return CSA2_E_UNSUPPORTED;
    if ((int64_t)B * Q > 65535) return CSA2_E_UNSUPPORTED;  // grid.y
    if (!(sm_scale == sm_scale) || sm_scale > 3.0e38f || sm_scale < -3.0e38f) return CSA2_E_ARG;
    return CSA2_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_E_HIP; }

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int csa2_abi_version(void) { return CSA2_ABI_VERSION; }

// Rotation table of the write path: entries are quantised after RoPE.  For
// each position p and channel pair j < 32 the angle is p * base^(-j/32),
// formed in double precision; its cosine and sine are rounded once to fp32.
__attribute__((visibility("default"))) int csa2_rope_table(const int64_t* positions, int64_t n,
                                                           double base, float* cs) {
    if (n < 0 || !(base > 1.0) || !(base < 1.0e300)) return CSA2_E_ARG;
    if (n == 0) return CSA2_OK;
    if (!positions || !cs) return CSA2_E_ARG;
    double freq[32];
    for (int j = 0; j < 32; ++j) freq[j] = std::pow(base, -(double)j / 32.0);
    for (int64_t i = 0; i < n; ++i) {
        const double pos = (double)positions[i];
        float* row = cs + i * 64;
        for (int j = 0; j < 32; ++j) {
            const double angle = pos * freq[j];
            row[2 * j] = (float)std::cos(angle);
            row[2 * j + 1] = (float)std::sin(angle);
        }
    }
    return CSA2_OK;
}

__attribute__((visibility("default"))) const char* csa2_status_str(int status) {
    switch (status) {
        case CSA2_OK: return "ok";
        case CSA2_E_ARG: return "invalid argument (null pointer or bad dimension)";
        case CSA2_E_UNSUPPORTED: return "unsupported argument value";
        case CSA2_E_WORKSPACE: return "workspace missing or too small";
        case CSA2_E_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

__attribute__((visibility("default"))) size_t csa2_workspace_size(int op, int B, int Q,
                                                                 int64_t cap, int topk,
                                                                 int pool_blocks, int H) {
    switch (op) {
        case CSA2_OP_INDEX_FULL:
            if (check_cache_dims(cap, B, Q) || topk < 1 || topk > CSA2_MAX_TOPK ||
                pool_blocks < 0 || pool_blocks > CSA2_MAX_POOL_BLOCKS)
                return SIZE_MAX;
            return full_layout(B, Q, cap, topk, pool_blocks).total;
        case CSA2_OP_INDEX_REINDEX:
            if (check_cache_dims(cap, B, Q) || pool_blocks < 1 ||
                pool_blocks > CSA2_MAX_POOL_BLOCKS)
                return SIZE_MAX;
            return reindex_layout(B, Q, pool_blocks).total;
        case CSA2_OP_ATTN_DECODE:
            if (B <= 0 || H <= 0 || topk < 0) return SIZE_MAX;
            return attn_workspace_bytes(B, H, topk, CSA2_WINDOW);
        case CSA2_OP_ATTN_CHUNK:
            if (B <= 0 || Q <= 0 || H <= 0 || topk < 0) return SIZE_MAX;
            return attn_workspace_bytes((int64_t)B * Q, H, topk, Q);
        case CSA2_OP_ATTN_STAGE:
            if (B <= 0 || topk < 0 || topk > CSA2_MAX_TOPK) return SIZE_MAX;
            return attn_stage_bytes(B, topk);
        default:
            return SIZE_MAX;
    }
}

static_assert(CSA2_MAX_FP8_JOBS == kMaxFp8Jobs, "FP8 jobs per write launch");

namespace {

int validate_quant_fp4(const float* k_tok, const float* v_tok, int64_t n_tok, int ratio,
                       const float* rope_cs, const uint8_t* kv_codes, const uint8_t* kv_scales) {
    if (n_tok < 0) return CSA2_E_ARG;
    if (ratio != 1 && ratio != 2) return CSA2_E_UNSUPPORTED;
    if (ratio == 2 && rope_cs) return CSA2_E_UNSUPPORTED;
    if (n_tok % ratio != 0) return CSA2_E_ARG;
    if (n_tok == 0) return CSA2_OK;
    if (!k_tok || !v_tok || !kv_codes || !kv_scales) return CSA2_E_ARG;
    return CSA2_OK;
}

int validate_quant_fp8(const float* x, int64_t n_rows, int dim, int layout, const uint8_t* codes,
                       const float* sigma) {
    if (n_rows < 0) return CSA2_E_ARG;
    if (dim != 64 && dim != 128) return CSA2_E_UNSUPPORTED;
    if (layout != CSA2_FP8_ROWS && layout != CSA2_FP8_IDX_TILED) return CSA2_E_ARG;
    if (layout == CSA2_FP8_IDX_TILED && dim != 64) return CSA2_E_UNSUPPORTED;
    if (n_rows == 0) return CSA2_OK;
    if (!x || !codes || !sigma) return CSA2_E_ARG;
    return CSA2_OK;
}

}  // namespace

__attribute__((visibility("default"))) int csa2_quant_fp4(const float* k_tok, const float* v_tok,
                                                         int64_t n_tok, int ratio,
                                                         const float* rope_cs,
                                                         const int64_t* dst_rows,
                                                         uint8_t* kv_codes, uint8_t* kv_scales,
                                                         hipStream_t stream) {
    const int rc = validate_quant_fp4(k_tok, v_tok, n_tok, ratio, rope_cs, kv_codes, kv_scales);
    if (rc != CSA2_OK || n_tok == 0) return rc;
    return hip_status(launch_quant_fp4(k_tok, v_tok, n_tok / ratio, ratio, rope_cs, dst_rows,
                                       kv_codes, kv_scales, stream));
}

__attribute__((visibility("default"))) int csa2_quant_fp8(const float* x, int64_t n_rows, int dim,
                                                         int layout, const int64_t* dst_rows,
                                                         uint8_t* codes, float* sigma,
                                                         hipStream_t stream) {
    const int rc = validate_quant_fp8(x, n_rows, dim, layout, codes, sigma);
    if (rc != CSA2_OK || n_rows == 0) return rc;
    return hip_status(launch_quant_fp8(x, n_rows, dim, layout, dst_rows, codes, sigma, stream));
}

__attribute__((visibility("default"))) int csa2_write_entries(
    const float* k_tok, const float* v_tok, int64_t n_tok, int ratio, const float* rope_cs,
    const int64_t* dst_rows, uint8_t* kv_codes, uint8_t* kv_scales, const csa2_fp8_job* jobs,
    int n_jobs, hipStream_t stream) {
    if (n_jobs < 0 || n_jobs > CSA2_MAX_FP8_JOBS || (n_jobs > 0 && !jobs)) return CSA2_E_ARG;
    int rc = validate_quant_fp4(k_tok, v_tok, n_tok, ratio, rope_cs, kv_codes, kv_scales);
    if (rc != CSA2_OK) return rc;
    Fp8Jobs j{};
    for (int i = 0; i < n_jobs; ++i) {
        const csa2_fp8_job& b = jobs[i];
        rc = validate_quant_fp8(b.x, b.n_rows, b.dim, b.layout, b.codes, b.sigma);
        if (rc != CSA2_OK) return rc;
        if (b.n_rows == 0) continue;
        j.job[j.n++] = Fp8Job{b.x, b.n_rows, b.dim, b.layout, b.dst_rows, b.codes, b.sigma};
    }
    const Fp4Job f{k_tok, v_tok, n_tok / ratio, ratio, rope_cs, dst_rows, kv_codes, kv_scales};
    return hip_status(launch_write_entries(f, j, stream));
}

__attribute__((visibility("default"))) int csa2_write_entries_proj(
    const float* k_tok, const float* v_tok, int64_t n_tok, int ratio, const float* rope_cs,
    const int64_t* dst_rows, uint8_t* kv_codes, uint8_t* kv_scales, const float* idx_proj,
    uint8_t* ik_codes, float* ik_sigma, const csa2_fp8_job* jobs, int n_jobs,
    hipStream_t stream) {
    if (n_jobs < 0 || n_jobs > CSA2_MAX_FP8_JOBS || (n_jobs > 0 && !jobs)) return CSA2_E_ARG;
    int rc = validate_quant_fp4(k_tok, v_tok, n_tok, ratio, rope_cs, kv_codes, kv_scales);
    if (rc != CSA2_OK) return rc;
    if (n_tok > 0 && (!idx_proj || !ik_codes || !ik_sigma)) return CSA2_E_ARG;
    Fp8Jobs j{};
    for (int i = 0; i < n_jobs; ++i) {
        const csa2_fp8_job& b = jobs[i];
        rc = validate_quant_fp8(b.x, b.n_rows, b.dim, b.layout, b.codes, b.sigma);
        if (rc != CSA2_OK) return rc;
        if (b.n_rows == 0) continue;
        j.job[j.n++] = Fp8Job{b.x, b.n_rows, b.dim, b.layout, b.dst_rows, b.codes, b.sigma};
    }
    const Fp4Job f{k_tok,    v_tok,     n_tok / ratio, ratio,   rope_cs, dst_rows,
                   kv_codes, kv_scales, idx_proj,      ik_codes, ik_sigma};
    return hip_status(launch_write_entries(f, j, stream));
}

namespace {
// The Full layer on the VALU scan: query prep, exact keys of every visible
// position (and block / superblock maxima), then the pool and top-K
// selection.  Arguments validated and the workspace checked by the caller.
int index_full_valu(int fmt, const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                    const float* iq, const float* iw, const int32_t* n_vis, int topk,
                    int pool_blocks, int32_t* topk_idx, int32_t* pool_idx, void* ws,
                    hipStream_t stream, hipEvent_t scan_start, hipEvent_t scan_stop) {
    const IndexLayout L = full_layout(B, Q, cap, topk, pool_blocks);
    char* w = static_cast<char*>(ws);
    float* qd = reinterpret_cast<float*>(w + L.qd);
    float* wq = reinterpret_cast<float*>(w + L.wq);
    uint32_t* keys = reinterpret_cast<uint32_t*>(w + L.keys);
    uint32_t* bkeys = reinterpret_cast<uint32_t*>(w + L.bkeys);
    uint32_t* sbkeys = reinterpret_cast<uint32_t*>(w + L.sbkeys);
    const int64_t nq = (int64_t)B * Q;
    // The Full layer's own top-K over every visible position equals the top-K
    // inside its best P >= K blocks (ties to the lower index on both levels),
    // so the position select only ever looks at P*8 candidates.  Without a
    // requested pool, P = K blocks are kept internally.
    const int P = pool_blocks > 0 ? pool_blocks : topk;
    // the scan quantises the queries itself (with many FP8 queries a
    // separate pass writes them to qd / wq first)
    hipError_t e = launch_scan(ikc, iks, cap, B, Q, iq, iw, qd, wq, n_vis, keys, bkeys, stream,
                               scan_start, scan_stop, sbkeys, fmt);
    if (e == hipSuccess)
        e = launch_select_full(keys, bkeys, cap, n_vis, nq, P, topk,
                               pool_blocks > 0 ? pool_idx : nullptr, topk_idx, stream, sbkeys);
    return hip_status(e);
}

// The Full layer of a multi-query chunk on MFMA: bounds on MFMA, then per
// query, in one workgroup: with a pool, the blocks the bounds decide plus the
// best undecided ones by exact block key; then the candidate half-blocks
// (upper bound reaches the K-th largest lower bound of a block, of the pool's
// blocks with a pool), their exact keys and the top-K.  A query whose
// candidates overflow is rescored over all its positions there and takes the
// Full selection.  Arguments validated and the workspace checked by the caller.
int index_full_mma(int fmt, const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                   const float* iq, const float* iw, const int32_t* n_vis, int topk,
                   int pool_blocks, int32_t* topk_idx, int32_t* pool_idx, void* ws,
                   hipStream_t stream, hipEvent_t scan_start, hipEvent_t scan_stop) {
    const IndexLayout L = full_layout(B, Q, cap, topk, pool_blocks);
    char* w = static_cast<char*>(ws);
    float* qd = reinterpret_cast<float*>(w + L.qd);
    float* wq = reinterpret_cast<float*>(w + L.wq);
    uint32_t* keys = reinterpret_cast<uint32_t*>(w + L.keys);
    uint32_t* bkeys = reinterpret_cast<uint32_t*>(w + L.bkeys);
    float* cq = reinterpret_cast<float*>(w + L.cq);
    _Float16* qh = reinterpret_cast<_Float16*>(w + L.qh);
    uint32_t* hkeys_hi = reinterpret_cast<uint32_t*>(w + L.hkeys_hi);
    const int64_t nq = (int64_t)B * Q;
    hipError_t e = launch_prep_iq(iq, iw, nq, qd, wq, stream, cq, qh);
    if (e == hipSuccess)
        e = launch_scan_mma(ikc, iks, cap, B, Q, qh, wq, cq, n_vis, bkeys, hkeys_hi, stream,
                            scan_start, scan_stop, fmt);
    if (e == hipSuccess)
        e = launch_chunk_select(ikc, iks, cap, Q, qd, wq, hkeys_hi, n_vis, nq, topk, keys, bkeys,
                                topk_idx, stream, pool_blocks, pool_blocks > 0 ? pool_idx : nullptr,
                                fmt);
    return hip_status(e);
}
}  // namespace

__attribute__((visibility("default"))) int csa2_index_full_timed(
    const uint8_t* ik_codes, const float* ik_sigma, int64_t cap, int B, int Q, const float* iq,
    const float* iw, const int32_t* n_vis, int topk, int pool_blocks, int32_t* topk_idx,
    int32_t* pool_idx, void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t scan_start,
    hipEvent_t scan_stop) {
    int rc = validate_index_full(ik_codes, ik_sigma, cap, B, Q, iq, iw, n_vis, topk, pool_blocks,
                                 topk_idx, pool_idx);
    if (rc) return rc;
    if (!ws || ws_bytes < full_layout(B, Q, cap, topk, pool_blocks).total)
        return CSA2_E_WORKSPACE;
    if (mma_path(Q, cap, pool_blocks, topk))
        return index_full_mma(kIdxFp8, ik_codes, ik_sigma, cap, B, Q, iq, iw, n_vis, topk,
                              pool_blocks, topk_idx, pool_idx, ws, stream, scan_start, scan_stop);
    return index_full_valu(kIdxFp8, ik_codes, ik_sigma, cap, B, Q, iq, iw, n_vis, topk,
                           pool_blocks, topk_idx, pool_idx, ws, stream, scan_start, scan_stop);
}

__attribute__((visibility("default"))) int csa2_index_full(
    const uint8_t* ik_codes, const float* ik_sigma, int64_t cap, int B, int Q, const float* iq,
    const float* iw, const int32_t* n_vis, int topk, int pool_blocks, int32_t* topk_idx,
    int32_t* pool_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
    return csa2_index_full_timed(ik_codes, ik_sigma, cap, B, Q, iq, iw, n_vis, topk, pool_blocks,
                                 topk_idx, pool_idx, ws, ws_bytes, stream, nullptr, nullptr);
}

__attribute__((visibility("default"))) int csa2_stream_probe(int mode, const void* src, void* dst,
                                                             size_t n_bytes, uint32_t* sink,
                                                             int n_blocks, hipStream_t stream) {
    if (mode < 0 || mode > 3 || !src || n_bytes % 16 != 0 || n_blocks < 1 || n_blocks > 65535)
        return CSA2_E_ARG;
    if ((mode != 1 && !sink) || (mode == 1 && !dst)) return CSA2_E_ARG;
    if (n_bytes == 0) return CSA2_OK;
    return hip_status(launch_stream_probe(mode, src, dst, n_bytes, sink, n_blocks, stream));
}

__attribute__((visibility("default"))) int csa2_gather_probe(
    const uint8_t* kv_codes, const uint8_t* kv_scales, const int32_t* topk_idx, int n_q, int topk,
    int64_t cap, const uint8_t* swa_k, const uint8_t* swa_v, const float* swa_ks,
    const float* swa_vs, const float* q, int H, float* out, hipStream_t stream, hipEvent_t start,
    hipEvent_t stop) {
    if (n_q < 0 || topk < 0 || topk > 2048 || cap <= 0 || H < 1 || H > 1024) return CSA2_E_ARG;
    if (n_q == 0) return CSA2_OK;
    const void* ptrs[] = {kv_codes, kv_scales, swa_k, swa_v, swa_ks, swa_vs, q, out};
    for (const void* p : ptrs)
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 16 != 0) return CSA2_E_ARG;
    if (topk > 0 && topk_idx == nullptr) return CSA2_E_ARG;
    return hip_status(launch_gather_probe(kv_codes, kv_scales, topk_idx, n_q, topk, cap, swa_k,
                                          swa_v, swa_ks, swa_vs, q, H, out, stream, start,
                                          stop));
}

// ---------------------------------------------------------------------------
// csa2_index_full without a caller workspace: the scratch is a fixed device
// array of this library (one copy per GPU, loaded with the library's code and
// kept until the process ends).  Host code never passes the array's name to a
// kernel: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = CSA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `dev`'s copy of the scratch array (null on error).
void* scratch_on(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || ptr == nullptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

__attribute__((visibility("default"))) int csa2_index_full_noalloc(
    const uint8_t* ik_codes, const float* ik_sigma, int64_t cap, int B, int Q, const float* iq,
    const float* iw, const int32_t* n_vis, int topk, int pool_blocks, int32_t* topk_idx,
    int32_t* pool_idx, hipStream_t stream) {
    int rc = validate_index_full(ik_codes, ik_sigma, cap, B, Q, iq, iw, n_vis, topk, pool_blocks,
                                 topk_idx, pool_idx);
    if (rc) return rc;
    if (full_layout(B, Q, cap, topk, pool_blocks).total > kNoAllocScratchBytes)
        return CSA2_E_WORKSPACE;
    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return CSA2_E_HIP;
    void* ws = scratch_on(dev);
    if (ws == nullptr) return CSA2_E_HIP;
    if (mma_path(Q, cap, pool_blocks, topk))
        return index_full_mma(kIdxFp8, ik_codes, ik_sigma, cap, B, Q, iq, iw, n_vis, topk,
                              pool_blocks, topk_idx, pool_idx, ws, stream, nullptr, nullptr);
    return index_full_valu(kIdxFp8, ik_codes, ik_sigma, cap, B, Q, iq, iw, n_vis, topk,
                           pool_blocks, topk_idx, pool_idx, ws, stream, nullptr, nullptr);
}

__attribute__((visibility("default"))) int csa2_index_reindex(
    const uint8_t* ik_codes, const float* ik_sigma, int64_t cap, int B, int Q, const float* iq,
    const float* iw, const int32_t* n_vis, const int32_t* pool_idx, int pool_blocks, int topk,
    int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = validate_index_reindex(ik_codes, ik_sigma, cap, B, Q, iq, iw, n_vis, pool_idx,
                                    pool_blocks, topk, topk_idx);
    if (rc) return rc;
    const IndexLayout L = reindex_layout(B, Q, pool_blocks);
    if (!ws || ws_bytes < L.total) return CSA2_E_WORKSPACE;
    char* w = static_cast<char*>(ws);
    uint32_t* ckeys = reinterpret_cast<uint32_t*>(w + L.keys);
    uint4* parts = reinterpret_cast<uint4*>(w + L.parts);
    const int64_t nq = (int64_t)B * Q;
    hipError_t e = launch_pool_score(ik_codes, ik_sigma, cap, B, Q, iq, iw, n_vis, pool_idx,
                                     pool_blocks, ckeys, parts, stream);
    if (e == hipSuccess)
        e = launch_select_pool(ckeys, parts, pool_idx, pool_blocks, n_vis, cap, nq, topk,
                               topk_idx, stream);
    return hip_status(e);
}

__attribute__((visibility("default"))) int csa2_quant_idx_fp4(const float* x, int64_t n_rows,
                                                              const int64_t* dst_rows,
                                                              uint8_t* codes, uint8_t* scales,
                                                              hipStream_t stream) {
    if (n_rows < 0) return CSA2_E_ARG;
    if (n_rows == 0) return CSA2_OK;
    if (!x || !codes || !scales) return CSA2_E_ARG;
    return hip_status(launch_quant_idx4(x, n_rows, dst_rows, codes, scales, stream));
}

__attribute__((visibility("default"))) int csa2_write_entries_proj_fp4(
    const float* k_tok, const float* v_tok, int64_t n_tok, int ratio, const float* rope_cs,
    const int64_t* dst_rows, uint8_t* kv_codes, uint8_t* kv_scales, const float* idx_proj,
    uint8_t* ik4_codes, uint8_t* ik4_scales, const csa2_fp8_job* jobs, int n_jobs,
    hipStream_t stream) {
    if (n_jobs < 0 || n_jobs > CSA2_MAX_FP8_JOBS || (n_jobs > 0 && !jobs)) return CSA2_E_ARG;
    int rc = validate_quant_fp4(k_tok, v_tok, n_tok, ratio, rope_cs, kv_codes, kv_scales);
    if (rc != CSA2_OK) return rc;
    if (n_tok > 0 && (!idx_proj || !ik4_codes || !ik4_scales)) return CSA2_E_ARG;
    Fp8Jobs j{};
    for (int i = 0; i < n_jobs; ++i) {
        const csa2_fp8_job& b = jobs[i];
        rc = validate_quant_fp8(b.x, b.n_rows, b.dim, b.layout, b.codes, b.sigma);
        if (rc != CSA2_OK) return rc;
        if (b.n_rows == 0) continue;
        j.job[j.n++] = Fp8Job{b.x, b.n_rows, b.dim, b.layout, b.dst_rows, b.codes, b.sigma};
    }
    const Fp4Job f{k_tok,    v_tok,     n_tok / ratio, ratio,     rope_cs, dst_rows,
                   kv_codes, kv_scales, idx_proj,      ik4_codes, nullptr, ik4_scales};
    return hip_status(launch_write_entries(f, j, stream));
}

__attribute__((visibility("default"))) int csa2_index_full_fp4_timed(
    const uint8_t* ik4_codes, const uint8_t* ik4_scales, int64_t cap, int B, int Q,
    const float* iq, const float* iw, const int32_t* n_vis, int topk, int pool_blocks,
    int32_t* topk_idx, int32_t* pool_idx, void* ws, size_t ws_bytes, hipStream_t stream,
    hipEvent_t scan_start, hipEvent_t scan_stop) {
    int rc = validate_index_full(ik4_codes, ik4_scales, cap, B, Q, iq, iw, n_vis, topk,
                                 pool_blocks, topk_idx, pool_idx);
    if (rc) return rc;
    if (!ws || ws_bytes < full_layout(B, Q, cap, topk, pool_blocks).total) return CSA2_E_WORKSPACE;
    const float* scales = reinterpret_cast<const float*>(ik4_scales);  // read as 32-bit words
    if (mma_path(Q, cap, pool_blocks, topk))
        return index_full_mma(kIdxFp4, ik4_codes, scales, cap, B, Q, iq, iw, n_vis, topk,
                              pool_blocks, topk_idx, pool_idx, ws, stream, scan_start, scan_stop);
    return index_full_valu(kIdxFp4, ik4_codes, scales, cap, B, Q, iq, iw, n_vis, topk,
                           pool_blocks, topk_idx, pool_idx, ws, stream, scan_start, scan_stop);
}

__attribute__((visibility("default"))) int csa2_index_full_fp4(
    const uint8_t* ik4_codes, const uint8_t* ik4_scales, int64_t cap, int B, int Q,
    const float* iq, const float* iw, const int32_t* n_vis, int topk, int pool_blocks,
    int32_t* topk_idx, int32_t* pool_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
    return csa2_index_full_fp4_timed(ik4_codes, ik4_scales, cap, B, Q, iq, iw, n_vis, topk,
                                     pool_blocks, topk_idx, pool_idx, ws, ws_bytes, stream,
                                     nullptr, nullptr);
}

__attribute__((visibility("default"))) int csa2_index_reindex_fp4(
    const uint8_t* ik4_codes, const uint8_t* ik4_scales, int64_t cap, int B, int Q,
    const float* iq, const float* iw, const int32_t* n_vis, const int32_t* pool_idx,
    int pool_blocks, int topk, int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = validate_index_reindex(ik4_codes, ik4_scales, cap, B, Q, iq, iw, n_vis, pool_idx,
                                    pool_blocks, topk, topk_idx);
    if (rc) return rc;
    const IndexLayout L = reindex_layout(B, Q, pool_blocks);
    if (!ws || ws_bytes < L.total) return CSA2_E_WORKSPACE;
    uint32_t* ckeys = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + L.keys);
    uint4* parts = reinterpret_cast<uint4*>(static_cast<char*>(ws) + L.parts);
    hipError_t e = launch_pool_score(ik4_codes, reinterpret_cast<const float*>(ik4_scales), cap,
                                     B, Q, iq, iw, n_vis, pool_idx, pool_blocks, ckeys, parts,
                                     stream, kIdxFp4);
    if (e == hipSuccess)
        e = launch_select_pool(ckeys, parts, pool_idx, pool_blocks, n_vis, cap, (int64_t)B * Q,
                               topk, topk_idx, stream);
    return hip_status(e);
}

__attribute__((visibility("default"))) int csa2_sparse_attn_decode_timed(
    const float* q, int B, int H, const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t cap,
    const int32_t* topk_idx, int topk, const uint8_t* swa_k, const uint8_t* swa_v,
    const float* swa_ks, const float* swa_vs, const int32_t* swa_len, float sm_scale, float* out,
    float* lse, void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t start,
    hipEvent_t stop) {
    int rc = validate_attn(q, B, 1, H, kv_codes, kv_scales, cap, topk_idx, topk, swa_k, swa_v,
                           swa_ks, swa_vs, sm_scale, out, lse);
    if (rc) return rc;
    if (!swa_len) return CSA2_E_ARG;
    const size_t need = attn_workspace_bytes(B, H, topk, CSA2_WINDOW);
    if (need > 0 && (!ws || ws_bytes < need)) return CSA2_E_WORKSPACE;
    AttnArgs a{q, H, 1, kv_codes, kv_scales, cap, topk_idx, topk, swa_k, swa_v, swa_ks, swa_vs,
               swa_len, CSA2_WINDOW, sm_scale, out, lse, (int64_t)B};
    return hip_status(launch_attn(a, ws, ws_bytes, stream, start, stop));
}

__attribute__((visibility("default"))) int csa2_sparse_attn_decode(
    const float* q, int B, int H, const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t cap,
    const int32_t* topk_idx, int topk, const uint8_t* swa_k, const uint8_t* swa_v,
    const float* swa_ks, const float* swa_vs, const int32_t* swa_len, float sm_scale, float* out,
    float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
    return csa2_sparse_attn_decode_timed(q, B, H, kv_codes, kv_scales, cap, topk_idx, topk, swa_k,
                                         swa_v, swa_ks, swa_vs, swa_len, sm_scale, out, lse, ws,
                                         ws_bytes, stream, nullptr, nullptr);
}

__attribute__((visibility("default"))) int csa2_sparse_attn_decode_reuse(
    const float* q, int B, int H, const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t cap,
    const int32_t* topk_idx, int topk, uint8_t* stage, size_t stage_bytes, int stage_mode,
    const uint8_t* swa_k, const uint8_t* swa_v, const float* swa_ks, const float* swa_vs,
    const int32_t* swa_len, float sm_scale, float* out, float* lse, void* ws, size_t ws_bytes,
    hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    if (stage_mode != CSA2_STAGE_WRITE && stage_mode != CSA2_STAGE_READ) return CSA2_E_ARG;
    if (topk > 0 && !stage) return CSA2_E_ARG;
    const bool read = stage_mode == CSA2_STAGE_READ;
    // a reading call takes the records from the stage: cache and positions unused
    const uint8_t* kvc = read ? stage : kv_codes;
    const uint8_t* kvs = read ? stage : kv_scales;
    const int32_t* idx = read ? reinterpret_cast<const int32_t*>(stage) : topk_idx;
    int rc = validate_attn(q, B, 1, H, kvc, kvs, read ? 1 : cap, idx, topk, swa_k, swa_v, swa_ks,
                           swa_vs, sm_scale, out, lse);
    if (rc) return rc;
    if (!swa_len) return CSA2_E_ARG;
    if (topk > 0 && stage_bytes < attn_stage_bytes(B, topk)) return CSA2_E_WORKSPACE;
    const size_t need = attn_workspace_bytes(B, H, topk, CSA2_WINDOW);
    if (need > 0 && (!ws || ws_bytes < need)) return CSA2_E_WORKSPACE;
    AttnArgs a{q, H, 1, read ? nullptr : kv_codes, read ? nullptr : kv_scales, read ? 1 : cap,
               read ? nullptr : topk_idx, topk, swa_k, swa_v, swa_ks, swa_vs, swa_len,
               CSA2_WINDOW, sm_scale, out, lse, (int64_t)B, topk > 0 ? stage : nullptr,
               topk > 0 ? (read ? kStageRead : kStageWrite) : 0};
    return hip_status(launch_attn(a, ws, ws_bytes, stream, start, stop));
}

__attribute__((visibility("default"))) int csa2_sparse_attn_chunk(
    const float* q, int B, int Q, int H, const uint8_t* kv_codes, const uint8_t* kv_scales,
    int64_t cap, const int32_t* topk_idx, int topk, const uint8_t* swa_k, const uint8_t* swa_v,
    const float* swa_ks, const float* swa_vs, float sm_scale, float* out, float* lse, void* ws,
    size_t ws_bytes, hipStream_t stream) {
    int rc = validate_attn(q, B, Q, H, kv_codes, kv_scales, cap, topk_idx, topk, swa_k, swa_v,
                           swa_ks, swa_vs, sm_scale, out, lse);
    if (rc) return rc;
    const int64_t nq = (int64_t)B * Q;
    const size_t need = attn_workspace_bytes(nq, H, topk, Q);
    if (need > 0 && (!ws || ws_bytes < need)) return CSA2_E_WORKSPACE;
    AttnArgs a{q, H, Q, kv_codes, kv_scales, cap, topk_idx, topk, swa_k, swa_v, swa_ks, swa_vs,
               nullptr, Q, sm_scale, out, lse, nq};
    return hip_status(launch_attn(a, ws, ws_bytes, stream));
}

__attribute__((visibility("default"))) int csa2_codec_probe(float* e4m3_dec, float* e4m3_dec16,
                                                           float* fp4_dec16, const float* x,
                                                           int64_t n, uint8_t* e4m3_enc,
                                                           uint8_t* e2m1_enc, hipStream_t stream) {
    if (!e4m3_dec || !e4m3_dec16 || !fp4_dec16 || n < 0) return CSA2_E_ARG;
    if (n > 0 && (!x || !e4m3_enc || !e2m1_enc)) return CSA2_E_ARG;
    return hip_status(launch_codec_probe(e4m3_dec, e4m3_dec16, fp4_dec16, x, n, e4m3_enc,
                                         e2m1_enc, stream));
}

}  // extern "C"
