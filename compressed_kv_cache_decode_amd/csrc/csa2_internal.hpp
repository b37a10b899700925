// csa2_internal.hpp -- launchers shared between the kernel files and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kMaxPoolBlocks = 4096;
constexpr int kMaxTopk = 2048;

hipError_t launch_quant_fp4(const float* k, const float* v, int64_t n_ent, int ratio,
                            const float* rope_cs, const int64_t* dst_rows, uint8_t* codes,
                            uint8_t* scales, hipStream_t stream);
hipError_t launch_quant_fp8(const float* x, int64_t n_rows, int dim, int layout,
                            const int64_t* dst_rows, uint8_t* codes, float* sigma,
                            hipStream_t stream);
// one-launch write path: FP4 entries (as launch_quant_fp4, n_ent entries) and
// up to kMaxFp8Jobs FP8 row sets (each as launch_quant_fp8)
struct Fp4Job {
    const float* k;
    const float* v;
    int64_t n_ent;
    int ratio;
    const float* rope_cs;
    const int64_t* dst_rows;
    uint8_t* codes;
    uint8_t* scales;
    // optional: the entries' indexer keys projected on the device from their
    // fp32 K, proj [64][128], written to ik_codes (tile layout) / ik_sigma
    // (FP8), or to ik_codes / ik_scales4 (FP4, when ik_scales4 is set)
    const float* proj = nullptr;
    uint8_t* ik_codes = nullptr;
    float* ik_sigma = nullptr;
    uint8_t* ik_scales4 = nullptr;
};
struct Fp8Job {
    const float* x;
    int64_t n_rows;
    int dim;
    int layout;
    const int64_t* dst_rows;
    uint8_t* codes;
    float* sigma;
};
constexpr int kMaxFp8Jobs = 3;
struct Fp8Jobs {
    Fp8Job job[kMaxFp8Jobs];
    int n;
};
hipError_t launch_write_entries(const Fp4Job& f, const Fp8Jobs& j, hipStream_t stream);
// cq, qh: the MFMA scan's guard constants and fp16 queries (null: not written)
hipError_t launch_prep_iq(const float* iq, const float* iw, int64_t n_q, float* qd, float* wq,
                          hipStream_t stream, float* cq = nullptr, _Float16* qh = nullptr);
hipError_t launch_codec_probe(float* e4m3_dec, float* e4m3_dec16, float* fp4_dec16,
                              const float* x, int64_t n, uint8_t* e4m3_enc, uint8_t* e2m1_enc,
                              hipStream_t stream);

// indexer-key formats: kIdxFp8 (4-plane tiles + fp32 sigma per row) and
// kIdxFp4 (2-plane tiles of E2M1 codes + 4 E4M3 scale bytes per row, passed
// where the sigma array goes)
constexpr int kIdxFp8 = 0;
constexpr int kIdxFp4 = 1;
// sbkeys (may be null): also the max key per superblock of kSuper positions
constexpr int kSuper = 64;
hipError_t launch_scan(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                       const float* iq, const float* iw, float* qd, float* wq,
                       const int32_t* n_vis, uint32_t* keys, uint32_t* bkeys, hipStream_t stream,
                       hipEvent_t start = nullptr, hipEvent_t stop = nullptr,
                       uint32_t* sbkeys = nullptr, int fmt = kIdxFp8);
// MFMA scan of a multi-query chunk with guard-band bounds (csa2_chunk.hip):
// the largest lower-bound score key per block of 8 positions [nq][cap / 8]
// and the upper-bound key per half-block of 4 [nq][cap / 4]
hipError_t launch_scan_mma(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                           const _Float16* qh, const float* wq, const float* cq,
                           const int32_t* n_vis, uint32_t* bkeys_lo, uint32_t* hkeys_hi,
                           hipStream_t stream, hipEvent_t start = nullptr,
                           hipEvent_t stop = nullptr, int fmt = kIdxFp8);
// top-K of each query of the MFMA scan from its bounds (csa2_index.hip):
// candidate half-blocks, their exact keys and the selection in one workgroup
// per query; keys / bkeys: scratch rows of the exact fallback (bkeys holds the
// scan's lower bounds on entry).  P > 0: the pool of P blocks first (into
// pool_out), then the top-K inside it; needs cap / 8 <= kChunkPoolMaxBlocks.
hipError_t launch_chunk_select(const uint8_t* ikc, const float* iks, int64_t cap, int Q,
                               const float* qd, const float* wq, const uint32_t* hkeys_hi,
                               const int32_t* n_vis, int64_t n_queries, int K, uint32_t* keys,
                               uint32_t* bkeys, int32_t* topk_out, hipStream_t stream, int P = 0,
                               int32_t* pool_out = nullptr, int fmt = kIdxFp8);
// blocks per sequence up to which the MFMA path also selects pools (their
// bound keys are held in registers, 16 per thread of a 1024-thread workgroup)
constexpr int64_t kChunkPoolMaxBlocks = 16384;
// candidate half-blocks per chunk query before the exact fallback: 3 K, at
// least 512
inline int chunk_cand_halves(int K) { return 3 * K < 512 ? 512 : 3 * K; }
// the MFMA scan path takes top-K up to this (its candidates' keys stay in LDS)
constexpr int kChunkMaxTopk = 1024;
// parts: [B*Q][ceil(P*8 / 64)] wave summaries of the keys for the selection
hipError_t launch_pool_score(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                             const float* iq, const float* iw, const int32_t* n_vis,
                             const int32_t* pool, int P, uint32_t* ckeys, uint4* parts,
                             hipStream_t stream, int fmt = kIdxFp8);
// FP4 indexer keys of n_rows fp32 rows [n_rows][64] into the 2-plane tiles and
// the per-row scale bytes (row dst_rows[r], or r)
hipError_t launch_quant_idx4(const float* x, int64_t n_rows, const int64_t* dst_rows,
                             uint8_t* codes, uint8_t* scales, hipStream_t stream);
// sbkeys: null, or the scan's superblock keys (used when the blocks do not
// fit the register path)
hipError_t launch_select_full(const uint32_t* keys, const uint32_t* bkeys, int64_t cap,
                              const int32_t* n_vis, int64_t n_queries, int P, int K,
                              int32_t* pool_out, int32_t* topk_out, hipStream_t stream,
                              const uint32_t* sbkeys = nullptr);
hipError_t launch_select_pool(const uint32_t* ckeys, const uint4* parts, const int32_t* pool,
                              int P, const int32_t* n_vis, int64_t cap, int64_t n_queries, int K,
                              int32_t* topk_out, hipStream_t stream);

// streaming probes (csa2_probe.hip): mode 0 reads n_bytes of src (one word
// per workgroup to sink), mode 1 copies src to dst; n_bytes a multiple of 16
hipError_t launch_gather_probe(const uint8_t* kvc, const uint8_t* kvs, const int32_t* idx,
                               int n_q, int topk, int64_t cap, const uint8_t* swk,
                               const uint8_t* swv, const float* swks, const float* swvs,
                               const float* q, int H, float* out, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop);
hipError_t launch_stream_probe(int mode, const void* src, void* dst, size_t n_bytes,
                               uint32_t* sink, int n_blocks, hipStream_t stream);

struct AttnArgs {
    const float* q;          // [n_q][H][128]
    int H;
    int Q;                   // queries per sequence (query bq belongs to sequence bq / Q)
    const uint8_t* kvc;      // [B*cap][128]
    const uint8_t* kvs;      // [B*cap][16]
    int64_t cap;
    const int32_t* idx;      // [n_q][topk]
    int topk;
    const uint8_t* swk;      // window K codes
    const uint8_t* swv;
    const float* swks;
    const float* swvs;
    const int32_t* swa_len;  // decode: [B]; chunk: nullptr (query i sees tokens [0, i])
    int swa_rows;            // rows per sequence in the window arrays (128 or Q)
    float sm_scale;
    float* out;              // [n_q][H][128]
    float* lse;              // [n_q][H]
    int64_t n_q;
    uint8_t* stage;          // staged selected records (stage_mode != 0), [n_q][tiles][kStageTileBytes]
    int stage_mode;          // 0 none, kStageWrite, kStageRead
};

// Staged records: the raw bytes of one tile of 32 selected records exactly as
// the attention lanes hold them, so that a layer that reuses a selection reads
// them with coalesced loads instead of gathering through the positions again.
constexpr int kStageWrite = 1;  // gather through the positions, also write the stage
constexpr int kStageRead = 2;   // read the records from the stage (no positions, no cache)
constexpr int kStageTileBytes = 4672;  // 4 x 1024 (K0, K1, V0, V1) + 512 (scales) + 4 (valid), padded
inline size_t attn_stage_bytes(int64_t n_q, int topk) {
    return (size_t)n_q * ((topk + 31) / 32) * kStageTileBytes;
}

size_t attn_workspace_bytes(int64_t n_q, int H, int topk, int swa_rows);
hipError_t launch_attn(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t stream,
                       hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

}  // namespace csa2
