/*
 * csa2.h -- C ABI of libcsa2: the CSA2 decode hot path on AMD Instinct MI355X
 * (gfx950).
 *
 * CSA2 ("Compressed Sparse Attention 2") keeps one global KV cache that many
 * layers share.  Its main KV is stored in FP4 (E2M1 values, one E4M3 scale
 * per 16 channels, no second-level scale); a per-position FP8 indexer key
 * drives retrieval.  Layers run in one of three modes:
 *   Full    scans every causally visible position with its own indexer query,
 *           keeps a top-K and (in the decoder) a pool of the best blocks of
 *           8 positions, at most 2048 blocks = 16384 positions;
 *   Reindex rescores only the pool with its own indexer query -> own top-K;
 *   Reuse   takes the most recent top-K unchanged (no call needed).
 * Every layer then attends to its top-K global entries (dequantised on read)
 * together with its own 128-token FP8 sliding window.
 * Sources: "DeepSeek V4.1 Flash: architecture study notes" (macin.top),
 * sections 1-4 and Figure 5; "DeepSeek V4.1 Flash is live" (myzaker.com),
 * sections "CSA2 attention" and "cache precision and persistence tiers".
 *
 * Conventions for every call
 *   - Array arguments are DEVICE pointers (hipMalloc'd, caller-owned); scalars
 *     are passed by value.  The library never allocates, frees or keeps a
 *     pointer after a call returns, and has no global mutable state.
 *   - A call validates its scalar arguments on the host, then enqueues its
 *     kernels on `stream` and returns without synchronising.  Calls on one
 *     stream are ordered; calls on different streams that share an output or
 *     workspace race.
 *   - Return value: CSA2_OK (0) or a negative status (csa2_status_str()).
 *     On a non-zero status nothing was enqueued, except CSA2_E_HIP, which
 *     reports a launch error from the HIP runtime.
 *   - Device data is not read to validate.  Out-of-range device values are
 *     clamped or skipped by the kernels (visible counts are clamped to
 *     [0, cap]; indices outside [0, cap) or [0, cap/8) are ignored), never
 *     dereferenced.  NaN or infinite inputs give unspecified (but memory-safe)
 *     results.
 *
 * Cache layouts (B independent sequences, each with capacity `cap` entries,
 * cap a multiple of 64; row r = b*cap + position)
 *   main KV codes   [B*cap][128] uint8: bytes 0..63 K, 64..127 V; byte j holds
 *                   channel 2j in its low nibble and 2j+1 in its high nibble;
 *                   a nibble is sign(bit 3) | E2M1 magnitude code (bits 0..2).
 *   main KV scales  [B*cap][16] uint8: bytes 0..7 K, 8..15 V; byte g is the
 *                   E4M3 scale of channels 16g..16g+15.
 *                   128 + 16 = 144 bytes per entry = 4.5 bits per value.
 *   indexer K codes tiled by 64 positions: position p of row r = b*cap + p
 *                   lives in tile t = r/64 at lane i = r%64; its channels
 *                   16g..16g+15 (g = 0..3) are the 16 bytes at offset
 *                   ((t*4 + g)*64 + i)*16.  E4M3 codes.
 *   indexer K sigma [B*cap] fp32 per-position scale (value = sigma * E4M3).
 *   SWA K / V       [rows][128] uint8 E4M3, per-row fp32 scale [rows].
 *   E4M3 is the OCP 8-bit format (bias 7, max 448, S.1111.111 = NaN);
 *   E2M1 is the OCP MX 4-bit format (magnitudes 0,.5,1,1.5,2,3,4,6).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 4: the Reindex workspace also holds the pool scoring's per-wave summaries
 * (csa2_workspace_size reports the size); csa2_stream_probe mode 3. */
#define CSA2_ABI_VERSION 4

#define CSA2_HEAD_DIM 128        /* main K and V width */
#define CSA2_KV_CODE_BYTES 128   /* per entry: K 64 B | V 64 B */
#define CSA2_KV_SCALE_BYTES 16   /* per entry: K 8 | V 8 E4M3 scales */
#define CSA2_IDX_HEADS 4         /* indexer heads */
#define CSA2_IDX_DIM 64          /* indexer width per head */
#define CSA2_IDX_TILE 64         /* positions per indexer-K tile */
#define CSA2_BLOCK 8             /* positions per pool block */
#define CSA2_WINDOW 128          /* SWA window */
#define CSA2_DEFAULT_TOPK 512
#define CSA2_DEFAULT_POOL_BLOCKS 2048
#define CSA2_MAX_TOPK 2048
#define CSA2_MAX_POOL_BLOCKS 4096
#define CSA2_MAX_HEADS 128       /* attention heads, multiple of 16 */

/* status codes */
#define CSA2_OK 0
#define CSA2_E_ARG (-1)          /* null pointer or bad dimension */
#define CSA2_E_UNSUPPORTED (-2)  /* valid but not supported (ratio, sizes) */
#define CSA2_E_WORKSPACE (-3)    /* workspace missing or too small */
#define CSA2_E_HIP (-4)          /* HIP runtime reported a launch error */

/* csa2_quant_fp8 layouts */
#define CSA2_IDX4_CODE_BYTES 32  /* FP4 indexer key: E2M1 codes per position */
#define CSA2_IDX4_SCALE_BYTES 4  /* FP4 indexer key: E4M3 scales per position */
#define CSA2_FP8_ROWS 0          /* codes [row][dim] */
#define CSA2_FP8_IDX_TILED 1     /* dim == 64, indexer-K tile layout above */

/* csa2_workspace_size ops */
#define CSA2_OP_INDEX_FULL 1
#define CSA2_OP_INDEX_REINDEX 2
#define CSA2_OP_ATTN_DECODE 3
#define CSA2_OP_ATTN_CHUNK 4
#define CSA2_OP_ATTN_STAGE 5     /* staged-records buffer of csa2_sparse_attn_decode_reuse */

/* stage_mode of csa2_sparse_attn_decode_reuse */
#define CSA2_STAGE_WRITE 1       /* gather through topk_idx and write the stage */
#define CSA2_STAGE_READ 2        /* take the selected records from the stage */

/*
 * csa2_quant_fp4 -- write path of the main KV.
 * "DeepSeek V4.1 Flash: architecture study notes" section 4 (E2M1 with one
 * 8-bit scale per 16 channels, 4 + 8/16 = 4.5 bits) and section 3 (encoder
 * groups merge 2 tokens into 1 entry); "DeepSeek V4.1 Flash is live",
 * "CSA2 attention" (no overlap between compressed entries) and "cache
 * precision" (quantise after RoPE, no global scale).
 *   k_tok, v_tok  [n_tok][128] fp32 token K and V.
 *   ratio         1, or 2: entry e is the mean fl(fl(a+b)*0.5) of tokens
 *                 2e and 2e+1 (n_tok must be even).
 *   rope_cs       NULL, or [n_ent][32][2] fp32 (cos, sin): K channels
 *                 (2j, 2j+1), j < 32, are rotated as
 *                 (fl(fl(x0 c) - fl(x1 s)), fl(fl(x0 s) + fl(x1 c))) before
 *                 quantisation.  Only with ratio 1.
 *   dst_rows      NULL (entry e -> row e) or [n_ent] int64 destination rows;
 *                 every row must lie inside kv_codes / kv_scales (not checked).
 *   kv_codes, kv_scales  main KV arrays (layout above); rows written only.
 * Per 16-channel group: scale = RNE_E4M3(amax/6) (saturating at 448); a zero
 * scale gives signed-zero codes; code = RNE_E2M1(x/scale), ties to the even
 * code, saturating at 6.  Divisions are IEEE fp32.
 */
int csa2_quant_fp4(const float* k_tok, const float* v_tok, int64_t n_tok, int ratio,
                   const float* rope_cs, const int64_t* dst_rows, uint8_t* kv_codes,
                   uint8_t* kv_scales, hipStream_t stream);

/*
 * csa2_quant_fp8 -- FP8 rows for the SWA K/V and the indexer K
 * ("DeepSeek V4.1 Flash: architecture study notes" section 4: the local SWA KV
 * stays FP8; the indexer key is the retrieval half of the global KV, section 1).
 *   x         [n_rows][dim] fp32; dim 64 or 128 (64 for CSA2_FP8_IDX_TILED).
 *   dst_rows  NULL (row r -> r) or [n_rows] int64 destination rows inside
 *             codes / sigma (not checked).
 *   codes     CSA2_FP8_ROWS: [rows][dim]; CSA2_FP8_IDX_TILED: tile layout.
 *   sigma     [rows] fp32.
 * sigma = fl(amax/448); code = RNE_E4M3(fl(x/sigma)); sigma == 0 gives
 * signed-zero codes.
 */
int csa2_quant_fp8(const float* x, int64_t n_rows, int dim, int layout, const int64_t* dst_rows,
                   uint8_t* codes, float* sigma, hipStream_t stream);

/* One FP8 row set of csa2_write_entries: the arguments of csa2_quant_fp8. */
typedef struct csa2_fp8_job {
    const float* x;
    int64_t n_rows;
    int dim;
    int layout;
    const int64_t* dst_rows;
    uint8_t* codes;
    float* sigma;
} csa2_fp8_job;

#define CSA2_MAX_FP8_JOBS 3

/*
 * csa2_write_entries -- the write path of new entries in one launch (the
 * same pages and sections as csa2_quant_fp4 and csa2_quant_fp8): writes
 * exactly what csa2_quant_fp4(k_tok, v_tok, n_tok, ratio, rope_cs, dst_rows,
 * kv_codes, kv_scales) and then csa2_quant_fp8 of each job would write, byte
 * for byte; e.g. a decode step's new entry and its indexer key, or a replay
 * chunk's 128 entries, their indexer keys and the window's K and V.
 *   n_tok        may be 0 (FP8 jobs only); the other FP4 arguments as in
 *                csa2_quant_fp4.
 *   jobs         host array of n_jobs (0..CSA2_MAX_FP8_JOBS) descriptors,
 *                read during the call only; jobs with n_rows 0 are skipped.
 * The rows written by the FP4 part and by the jobs must not overlap (not
 * checked).  Errors: CSA2_E_ARG for n_jobs out of range or jobs NULL with
 * n_jobs > 0; otherwise the first error csa2_quant_fp4 or csa2_quant_fp8
 * would return for its part.  Nothing is launched on an error.
 */
int csa2_write_entries(const float* k_tok, const float* v_tok, int64_t n_tok, int ratio,
                       const float* rope_cs, const int64_t* dst_rows, uint8_t* kv_codes,
                       uint8_t* kv_scales, const csa2_fp8_job* jobs, int n_jobs,
                       hipStream_t stream);

/*
 * csa2_write_entries_proj -- csa2_write_entries that also computes each new
 * entry's indexer key on the device ("DeepSeek V4.1 Flash is live", "CSA2
 * attention": the indexer key is projected from the main-KV entry instead of
 * being compressed from hidden states on its own; "DeepSeek V4.1 Flash:
 * architecture study notes" section 1: the global KV is the main KV plus the
 * indexer key).
 *   idx_proj   [64][128] fp32, row-major, device: the 128 -> 64 projection.
 *   ik_codes, ik_sigma  indexer K arrays (tile layout, fp32 sigma): the key of
 *              entry e is written at row dst_rows[e] (or e), as
 *              csa2_quant_fp8(..., dim 64, CSA2_FP8_IDX_TILED) would write the
 *              fp32 key vector.
 * Key of an entry: x = the entry's fp32 K exactly as the FP4 part quantises
 * it (after the 2:1 mean and RoPE, before quantisation);
 * key[j] = fp32 sum over c = 0..127 in order of idx_proj[j][c] * x[c], each
 * step one fused multiply-add (one rounding), starting from +0.
 * The other arguments, the launch and the errors are those of
 * csa2_write_entries; in addition CSA2_E_ARG when n_tok > 0 and idx_proj,
 * ik_codes or ik_sigma is NULL.  The FP8 jobs must not write the rows the
 * keys go to (not checked).  idx_proj is read during the launch only.
 */
int csa2_write_entries_proj(const float* k_tok, const float* v_tok, int64_t n_tok, int ratio,
                            const float* rope_cs, const int64_t* dst_rows, uint8_t* kv_codes,
                            uint8_t* kv_scales, const float* idx_proj, uint8_t* ik_codes,
                            float* ik_sigma, const csa2_fp8_job* jobs, int n_jobs,
                            hipStream_t stream);

/*
 * csa2_index_full -- Full-layer indexer ("DeepSeek V4.1 Flash: architecture
 * study notes" section 2: Full picks this step's positions, at most 512 per
 * query; the decoder's first Full layer scans every causally visible position
 * and builds a pool of at most 2048 blocks x 8 positions, Figure 5).
 *   ik_codes, ik_sigma  indexer K (tile layout), capacity cap per sequence.
 *   B, Q        sequences, queries per sequence (Q = 1 decode; Q > 1 e.g. a
 *               128-token replay chunk).
 *   iq          [B][Q][4][64] fp32 indexer queries; iw [B][Q][4] head weights.
 *   n_vis       [B][Q] int32: query (b,q) sees positions [0, n_vis).
 *   topk        1..2048; pool_blocks 0 (no pool) or topk/8 .. 4096 rounded
 *               as given (pool_blocks*8 >= topk required when > 0).
 *   topk_idx    [B][Q][topk] int32 out: the min(topk, n_vis) best positions,
 *               ascending, then -1.
 *   pool_idx    [B][Q][pool_blocks] int32 out (ignored when pool_blocks == 0):
 *               the best min(pool_blocks, ceil(n_vis/8)) blocks, ascending,
 *               then -1.
 * Score of position s: the query is quantised per head to E4M3 with
 * sq = fl(amax/448), w'_h = fl(w_h*sq); dot_h = fp32 sum over channels
 * 0..63 in order of E4M3(q) * E4M3(k); r_h = max(dot_h, +0);
 * t = w'_0 r_0 + w'_1 r_1 + w'_2 r_2 + w'_3 r_3 (left to right, each product
 * rounded); score = fl(sigma_s * t).  Block score = max over its visible
 * positions.  Ranking: larger score first, equal scores -> lower position
 * (block) first; -0 == +0.
 * ws / ws_bytes: device workspace of at least
 *   csa2_workspace_size(CSA2_OP_INDEX_FULL, B, Q, cap, topk, pool_blocks, 0).
 */
int csa2_index_full(const uint8_t* ik_codes, const float* ik_sigma, int64_t cap, int B, int Q,
                    const float* iq, const float* iw, const int32_t* n_vis, int topk,
                    int pool_blocks, int32_t* topk_idx, int32_t* pool_idx, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/*
 * csa2_index_full_timed -- csa2_index_full with the Full-layer scan kernel
 * (the only kernel of the path whose work grows with context) bracketed by two
 * caller-created HIP events: the runtime records scan_start immediately before
 * and scan_stop immediately after that dispatch (hipExtLaunchKernel), so
 * hipEventElapsedTime(scan_start, scan_stop) is the scan's duration.  Both
 * NULL: identical to csa2_index_full.  Not for use under stream capture.
 */
int csa2_index_full_timed(const uint8_t* ik_codes, const float* ik_sigma, int64_t cap, int B,
                          int Q, const float* iq, const float* iw, const int32_t* n_vis, int topk,
                          int pool_blocks, int32_t* topk_idx, int32_t* pool_idx, void* ws,
                          size_t ws_bytes, hipStream_t stream, hipEvent_t scan_start,
                          hipEvent_t scan_stop);

/*
 * csa2_index_reindex -- Reindex layer ("DeepSeek V4.1 Flash: architecture
 * study notes" section 2: reuses the Full layer's indexer K, rescores with its
 * own indexer query, only inside the pool).
 *   pool_idx   [B][Q][pool_blocks] as written by csa2_index_full (-1 ignored).
 *   topk_idx   [B][Q][topk] out: best min(topk, #visible pool positions)
 *              positions inside the pool, ascending, then -1.
 * Same score and ranking as csa2_index_full.  B*Q <= 65535 (else
 * CSA2_E_UNSUPPORTED).  ws: at least
 *   csa2_workspace_size(CSA2_OP_INDEX_REINDEX, B, Q, cap, topk, pool_blocks, 0).
 */
int csa2_index_reindex(const uint8_t* ik_codes, const float* ik_sigma, int64_t cap, int B, int Q,
                       const float* iq, const float* iw, const int32_t* n_vis,
                       const int32_t* pool_idx, int pool_blocks, int topk, int32_t* topk_idx,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * FP4 indexer key -- a second format for the indexer K ("DeepSeek V4.1
 * Flash: architecture study notes" section 4: the FP4 main KV builds on the
 * previous generation's FP4 indexer key).  The key is stored in the main KV's
 * FP4 format: E2M1 codes (low nibble = even channel) with one E4M3 scale per
 * 16 channels and no per-position scale, 32 + 4 = 36 bytes per position
 * against 68 for the FP8 key.  Layout, row r = b*cap + p:
 *   ik4_codes   tiles of 64 positions, two 1 KB planes per tile: plane h holds
 *               the 16 code bytes of channels 32h..32h+31 of each of the 64
 *               positions, at byte ((r/64)*2 + h)*1024 + (r%64)*16;
 *   ik4_scales  [B*cap][4] E4M3 bytes, byte g scaling channels 16g..16g+15.
 * Quantisation of a 64-channel key: per group scale = RNE_E4M3(fl(amax/6))
 * (saturating), code = RNE_E2M1(fl(x/scale)), ties to the even code, a zero
 * scale giving signed-zero codes (the rule of csa2_quant_fp4).
 * Score of position s (the query quantised as in csa2_index_full):
 *   inner_hg = fp32 sum over the 16 channels of group g, ascending, of
 *              E4M3(q_hc) * E2M1(k_sc) (each product exact), from +0;
 *   dot_h    = fused multiply-add chain over g = 0..3 of scale_g * inner_hg,
 *              from +0;
 *   score    = w'_0 r_0 + w'_1 r_1 + w'_2 r_2 + w'_3 r_3 (left to right, each
 *              product rounded), r_h = max(dot_h, +0).
 * Blocks, pools, ranking, ties and outputs are those of the FP8 calls.
 */

/* csa2_quant_idx_fp4 -- FP4 indexer keys of x [n_rows][64] fp32, written at
 * rows dst_rows[r] (or r) of ik4_codes / ik4_scales (not checked).
 * CSA2_E_ARG for n_rows < 0 or a NULL array with n_rows > 0. */
int csa2_quant_idx_fp4(const float* x, int64_t n_rows, const int64_t* dst_rows,
                       uint8_t* ik4_codes, uint8_t* ik4_scales, hipStream_t stream);

/* csa2_write_entries_proj_fp4 -- csa2_write_entries_proj with the projected
 * keys written as FP4 indexer keys to ik4_codes / ik4_scales. */
int csa2_write_entries_proj_fp4(const float* k_tok, const float* v_tok, int64_t n_tok, int ratio,
                                const float* rope_cs, const int64_t* dst_rows, uint8_t* kv_codes,
                                uint8_t* kv_scales, const float* idx_proj, uint8_t* ik4_codes,
                                uint8_t* ik4_scales, const csa2_fp8_job* jobs, int n_jobs,
                                hipStream_t stream);

/* csa2_index_full_fp4 -- csa2_index_full over FP4 indexer keys, with the
 * same two paths (the exact scan; for many queries per sequence the MFMA
 * bounds with exact rescoring, whose guard band allows for keys up to
 * 6 x 448).  Arguments, outputs, workspace and errors as csa2_index_full;
 * _timed brackets the scan as csa2_index_full_timed does. */
int csa2_index_full_fp4(const uint8_t* ik4_codes, const uint8_t* ik4_scales, int64_t cap, int B,
                        int Q, const float* iq, const float* iw, const int32_t* n_vis, int topk,
                        int pool_blocks, int32_t* topk_idx, int32_t* pool_idx, void* ws,
                        size_t ws_bytes, hipStream_t stream);
int csa2_index_full_fp4_timed(const uint8_t* ik4_codes, const uint8_t* ik4_scales, int64_t cap,
                              int B, int Q, const float* iq, const float* iw,
                              const int32_t* n_vis, int topk, int pool_blocks, int32_t* topk_idx,
                              int32_t* pool_idx, void* ws, size_t ws_bytes, hipStream_t stream,
                              hipEvent_t scan_start, hipEvent_t scan_stop);

/* csa2_index_reindex_fp4 -- csa2_index_reindex over FP4 indexer keys. */
int csa2_index_reindex_fp4(const uint8_t* ik4_codes, const uint8_t* ik4_scales, int64_t cap,
                           int B, int Q, const float* iq, const float* iw, const int32_t* n_vis,
                           const int32_t* pool_idx, int pool_blocks, int topk, int32_t* topk_idx,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa2_sparse_attn_decode -- sparse attention of one decode query per
 * sequence ("DeepSeek V4.1 Flash: architecture study notes" section 2: at most
 * 512 selected global records together with the local window; section 4:
 * dequantise on read, then ordinary attention).
 *   q          [B][H][128] fp32, H a multiple of 16, <= 128.
 *   kv_codes, kv_scales, cap  the shared main KV (one cache per sequence).
 *   topk_idx   [B][topk] int32 positions (-1 = none), e.g. from a Full,
 *              Reindex or (reused) earlier layer.
 *   swa_k, swa_v    [B][128][128] E4M3; swa_ks, swa_vs [B][128] fp32;
 *   swa_len    [B] int32, tokens [0, swa_len) of the window are used.
 *   out        [B][H][128] fp32; lse [B][H] fp32 = ln(sum exp(logit)).
 * logit = sm_scale * q . k over the union of selected entries
 * (k = E2M1 * E4M3 scale) and window tokens (k = sigma * E4M3); one softmax
 * over the union; out = sum p v / sum p.  No keys -> out 0, lse -inf.
 * ws: csa2_workspace_size(CSA2_OP_ATTN_DECODE, B, 1, cap, topk, 0, H) bytes,
 * currently 0 (ws may then be NULL); kept so that a later kernel may use one.
 */
int csa2_sparse_attn_decode(const float* q, int B, int H, const uint8_t* kv_codes,
                            const uint8_t* kv_scales, int64_t cap, const int32_t* topk_idx,
                            int topk, const uint8_t* swa_k, const uint8_t* swa_v,
                            const float* swa_ks, const float* swa_vs, const int32_t* swa_len,
                            float sm_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * csa2_sparse_attn_decode_timed -- csa2_sparse_attn_decode, with the HIP
 * events `start` and `stop` (created by the caller, hipEventDefault) recorded
 * by the runtime immediately before and after the attention kernel's own
 * dispatch, so hipEventElapsedTime(start, stop) is that kernel's duration.
 * NULL events: identical to csa2_sparse_attn_decode.
 */
int csa2_sparse_attn_decode_timed(const float* q, int B, int H, const uint8_t* kv_codes,
                                  const uint8_t* kv_scales, int64_t cap, const int32_t* topk_idx,
                                  int topk, const uint8_t* swa_k, const uint8_t* swa_v,
                                  const float* swa_ks, const float* swa_vs,
                                  const int32_t* swa_len, float sm_scale, float* out, float* lse,
                                  void* ws, size_t ws_bytes, hipStream_t stream,
                                  hipEvent_t start, hipEvent_t stop);

/*
 * csa2_sparse_attn_decode_reuse -- csa2_sparse_attn_decode for a stack of
 * layers that share one selection ("DeepSeek V4.1 Flash: architecture study
 * notes" section 2: a Reuse layer keeps the shared global KV and the latest
 * top-K positions and has only its own query and window; with one cache
 * shared by every layer, the selected records themselves are identical
 * across those layers).
 *   stage_mode CSA2_STAGE_WRITE: as csa2_sparse_attn_decode, and the raw bytes
 *              of every selected record (codes, scales, presence) are also
 *              written to `stage`, laid out as the attention kernel's lanes
 *              hold them.
 *   stage_mode CSA2_STAGE_READ: the records come from `stage` as written by
 *              an earlier CSA2_STAGE_WRITE call with the same B and topk (and
 *              the cache unchanged since); kv_codes, kv_scales, cap and
 *              topk_idx are not read (may be NULL / 0).
 * Outputs are bit-identical to csa2_sparse_attn_decode with the source
 * layer's topk_idx.  stage: device memory owned by the caller, at least
 * csa2_workspace_size(CSA2_OP_ATTN_STAGE, B, 1, cap, topk, 0, H) =
 * B * ceil(topk / 32) * 4672 bytes (smaller -> CSA2_E_WORKSPACE; NULL allowed
 * when topk == 0).  A reading call must not overlap the writing call in time.
 * start / stop: as csa2_sparse_attn_decode_timed (NULL: not recorded).
 */
int csa2_sparse_attn_decode_reuse(const float* q, int B, int H, const uint8_t* kv_codes,
                                  const uint8_t* kv_scales, int64_t cap, const int32_t* topk_idx,
                                  int topk, uint8_t* stage, size_t stage_bytes, int stage_mode,
                                  const uint8_t* swa_k, const uint8_t* swa_v,
                                  const float* swa_ks, const float* swa_vs,
                                  const int32_t* swa_len, float sm_scale, float* out, float* lse,
                                  void* ws, size_t ws_bytes, hipStream_t stream,
                                  hipEvent_t start, hipEvent_t stop);

/*
 * csa2_sparse_attn_chunk -- attention of a Q-token bounded-replay chunk
 * ("DeepSeek V4.1 Flash: architecture study notes" section 5: the decoder
 * replays only the last 128 tokens of the prompt to rebuild its SWA state;
 * earlier local dependencies are cut off).
 *   q          [B][Q][H][128] fp32, B*Q <= 65535; topk_idx [B][Q][topk].
 *   swa_k, swa_v    [B][Q][128] E4M3, the chunk's own tokens; swa_ks,
 *              swa_vs [B][Q].  Query i attends to the chunk tokens
 *              [max(0, i - 127), i]: the last 128 up to itself (all of
 *              [0, i] in a chunk of at most 128 tokens).
 *   out [B][Q][H][128], lse [B][Q][H].  Otherwise as the decode call.
 * ws: csa2_workspace_size(CSA2_OP_ATTN_CHUNK, B, Q, cap, topk, 0, H) bytes
 * (currently 0; ws may then be NULL).
 */
int csa2_sparse_attn_chunk(const float* q, int B, int Q, int H, const uint8_t* kv_codes,
                           const uint8_t* kv_scales, int64_t cap, const int32_t* topk_idx,
                           int topk, const uint8_t* swa_k, const uint8_t* swa_v,
                           const float* swa_ks, const float* swa_vs, float sm_scale, float* out,
                           float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes needed by `op` for these sizes (0 if none; SIZE_MAX if the
 * sizes are invalid).  Pure host function. */
size_t csa2_workspace_size(int op, int B, int Q, int64_t cap, int topk, int pool_blocks, int H);

/* Static description of a status code. */
const char* csa2_status_str(int status);

/* CSA2_ABI_VERSION of the built library. */
int csa2_abi_version(void);

/*
 * csa2_stream_probe -- diagnostics: the streaming ceilings of this GPU, for
 * comparing the kernels above against in the same run (not part of the
 * method).  mode 0 reads n_bytes of src with 16-byte non-temporal loads and
 * writes one word per workgroup to sink [n_blocks]; mode 1 copies n_bytes of
 * src to dst; both grid-stride over n_blocks workgroups of 256 threads, four
 * loads in flight per thread.  mode 2 reads src with one 16-byte load per
 * thread over a grid covering it; mode 3 reads it in 16 KB chunks, one per
 * workgroup of 256 threads, four 16-byte loads per thread 4 KB apart (the
 * indexer scan's access), over a grid covering it (modes 2 and 3: n_blocks
 * unused; sink [1] is written only by a data-dependent test that keeps the
 * loads).  n_bytes a multiple of 16;
 * device pointers; enqueued on `stream`.  CSA2_E_ARG for a bad mode, size or
 * null pointer.
 */
int csa2_stream_probe(int mode, const void* src, void* dst, size_t n_bytes, uint32_t* sink,
                      int n_blocks, hipStream_t stream);

/*
 * csa2_gather_probe -- diagnostics: the memory-side ceiling of the gathering
 * decode attention's access pattern (not part of the method).  For each of
 * the n_q queries it reads exactly what csa2_sparse_attn_decode reads for a
 * full window: the topk selected records (kv_codes [n_q][cap][128] and
 * kv_scales [n_q][cap][16] at the positions of topk_idx [n_q][topk]; -1 or a
 * position past cap is skipped), the 128 window rows swa_k / swa_v
 * [n_q][128][128] with swa_ks / swa_vs [n_q][128], and q [n_q][H][128] fp32,
 * and writes out [n_q][H][128]; no arithmetic.  Each 32-bit word i of a
 * query's output row holds word i mod 4 of the XOR of all the 16-byte units
 * read for that query.  One workgroup of 256 threads per query.  Device
 * pointers, 16-byte aligned; enqueued on `stream`; start / stop (both or
 * neither) are recorded immediately around the dispatch.  CSA2_E_ARG for
 * topk outside [0, 2048], H outside [1, 1024], cap <= 0, a null or
 * misaligned pointer.
 */
int csa2_gather_probe(const uint8_t* kv_codes, const uint8_t* kv_scales, const int32_t* topk_idx,
                      int n_q, int topk, int64_t cap, const uint8_t* swa_k, const uint8_t* swa_v,
                      const float* swa_ks, const float* swa_vs, const float* q, int H, float* out,
                      hipStream_t stream, hipEvent_t start, hipEvent_t stop);

/*
 * csa2_index_full_noalloc -- csa2_index_full for callers that cannot allocate
 * device memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument; the call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 *   Arguments, results and errors as csa2_index_full, without ws / ws_bytes.
 *   Its scratch is a fixed array of CSA2_NOALLOC_SCRATCH_BYTES bytes inside
 *   the library, one copy per GPU, held until the process ends.  A call whose
 *   csa2_workspace_size(CSA2_OP_INDEX_FULL, ...) exceeds that limit returns
 *   CSA2_E_WORKSPACE before touching the GPU (16 queries over 131072 positions
 *   need 9.2 MiB, 4 queries over 1048576 positions 18.3 MiB).  The device is
 *   the one `stream` belongs to; the first call on a device looks up that
 *   device's copy (CSA2_E_HIP if the lookup fails).
 *   Every call on one GPU shares that GPU's copy, which keeps the last call's
 *   contents: calls that overlap on one GPU (other streams, other threads)
 *   race and must be serialised by the caller.  No part of the scratch needs
 *   to start at zero (every value read is written earlier in the same call).
 */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int csa2_index_full_noalloc(const uint8_t* ik_codes, const float* ik_sigma, int64_t cap, int B,
                            int Q, const float* iq, const float* iw, const int32_t* n_vis,
                            int topk, int pool_blocks, int32_t* topk_idx, int32_t* pool_idx,
                            hipStream_t stream);

/*
 * csa2_rope_table -- HOST function: the rotation table that csa2_quant_fp4 and
 * the write-entry calls take as `rope_cs` ("DeepSeek V4.1 Flash is live",
 * section "cache precision and persistence tiers": entries are quantised after
 * RoPE; RoPE on K channels 0..63 in interleaved pairs, base 10000).
 *   positions  [n] int64 HOST array: absolute position of each entry.
 *   n          number of positions (0: nothing is written).
 *   base       rotation base (10000 for CSA2), > 1.
 *   cs         [n][32][2] fp32 HOST array, caller-owned, written only:
 *              cs[i][j] = (cos a, sin a) with a = positions[i] * base^(-j/32)
 *              evaluated in double precision and rounded once to fp32.
 * Returns CSA2_E_ARG for n < 0, base <= 1 or a null array with n > 0.  Runs on
 * the calling thread; touches no HIP state.
 */
int csa2_rope_table(const int64_t* positions, int64_t n, double base, float* cs);

/*
 * csa2_codec_probe -- diagnostics: runs the library's own device codecs.
 *   e4m3_dec   [256] fp32 out: every E4M3 code through the scan's converter.
 *   e4m3_dec16 [256] fp32 out: every E4M3 code through the attention's fp16
 *              converter.
 *   fp4_dec16  [256*16] fp32 out: [s*16 + c] = E2M1 code c (sign in bit 3)
 *              times E4M3 scale byte s, through the attention's FP4 path.
 *   x [n] fp32 in -> e4m3_enc [n], e2m1_enc [n] uint8 out (the write path's
 *   encoders).  Enqueued on `stream` like every call.
 */
int csa2_codec_probe(float* e4m3_dec, float* e4m3_dec16, float* fp4_dec16, const float* x,
                     int64_t n, uint8_t* e4m3_enc, uint8_t* e2m1_enc, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
