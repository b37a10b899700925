/*
 * csa2_oracle.h -- plain, slow CPU oracle for the CSA2 decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only tests/, the smoke check and the bench's CPU-baseline
 * leg do.  It shares no code, tables or headers with the HIP path.
 *
 * Sources (web pages summarising the DeepSeek V4.1 Flash technical report):
 *   [notes]  "DeepSeek V4.1 Flash: architecture study notes" (macin.top),
 *            section 1 (global KV vs local SWA KV), section 2 (CSA2 Full /
 *            Reindex / Reuse, top-512, hierarchical indexer, Figure 5 pool),
 *            section 3 (sequence compression), section 4 (FP4 main KV).
 *   [digest] "DeepSeek V4.1 Flash is live" (myzaker.com), section
 *            "CSA2 attention" (modes, indexer K projected from main KV,
 *            no overlap between compressed entries) and section
 *            "cache precision and persistence tiers" (FP4 after RoPE,
 *            SWA stays FP8, bounded replay).
 *
 * Where the pages leave a numeric step open, the oracle takes one fixed
 * reading (listed in the design notes of the repository):
 *   - FP4 group scale s = RNE_E4M3(amax/6), E2M1 code = RNE(x/s), saturating.
 *   - FP8 rows (indexer K, SWA K/V, indexer query): sigma = amax/448 in fp32,
 *     code = RNE_E4M3(x/sigma).
 *   - indexer score = sigma_s * sum_h w'_h * ReLU(q_h . k_s), every step one
 *     IEEE fp32 operation in a fixed order (channels ascending, heads
 *     ascending, sigma last).
 *   - ties in any ranking go to the lower position / block index.
 *   - attention is one softmax over selected global entries plus the SWA
 *     tokens, computed in fp64 from exactly dequantised values.
 *
 * Parity pins: every function here is pinned by the CPU test-suite against
 * library routines, closed forms or brute force (see tests/test_oracle_*.py).
 */
#ifndef CSA2_ORACLE_H
#define CSA2_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats (OCP 8-bit FP E4M3 "FN", OCP MX E2M1) ---- */
double  csa2o_e4m3_decode(uint8_t code);
uint8_t csa2o_e4m3_encode(float x);          /* RNE, ties to even code, saturate to +-448 */
double  csa2o_e2m1_decode(uint8_t code);     /* low 4 bits used */
uint8_t csa2o_e2m1_encode(float t);          /* RNE, ties to even code, saturate to +-6 */

/* ---- write path ---- */
/* out[c] = fl(fl(a[c]+b[c]) * 0.5) */
void csa2o_average_pair(const float* a, const float* b, int n, float* out);
/* cs[i][j][0..1] = (cos, sin)(pos[i] * base^(-j/32)), fp64 rounded to fp32, j<32 */
void csa2o_rope_table(const int64_t* pos, int64_t n, double base, float* cs);
/* rotate interleaved pairs (2j, 2j+1), j < 32, of x in place */
void csa2o_rope_apply(float* x, const float* cs_row);
/* one 128-channel vector -> 64 code bytes (low nibble = even channel) + 8 E4M3 scales */
void csa2o_fp4_quant_vec(const float* x, uint8_t* codes, uint8_t* scales);
/* the same for n_groups groups of 16 channels */
void csa2o_fp4_quant_groups(const float* x, int n_groups, uint8_t* codes, uint8_t* scales);
/* write-path batch: n_tok tokens of K and V [n_tok][128]; ratio 1 or 2;
 * rope_cs NULL or [n_ent][32][2]; out codes [n_ent][128] (K 64 B | V 64 B),
 * scales [n_ent][16] (K 8 | V 8). Returns 0 or -1 on bad arguments. */
int  csa2o_quant_fp4(const float* k, const float* v, int64_t n_tok, int ratio,
                     const float* rope_cs, uint8_t* codes, uint8_t* scales);
/* the fp32 K of each entry as the write path quantises it: pair mean
 * (ratio 2) or the token itself, then RoPE when rope_cs is given; out
 * [n_tok/ratio][128].  Returns 0 or -1 on bad arguments. */
int  csa2o_entry_k(const float* k, int64_t n_tok, int ratio, const float* rope_cs, float* out);
/* indexer key of one entry: key[j] = fused multiply-add chain over input
 * channels 0..127 in order of W[j][c] * x[c], from +0; W [64][128] */
void csa2o_project_idx(const float* x, const float* W, float* key);
void csa2o_project_idx_rows(const float* x, int64_t n, const float* W, float* keys);
/* one row of `dim` values -> E4M3 codes and fp32 sigma */
void csa2o_fp8_quant_row(const float* x, int dim, uint8_t* codes, float* sigma);
void csa2o_quant_fp8_rows(const float* x, int64_t n_rows, int dim,
                          uint8_t* codes, float* sigma);

/* ---- indexer ---- */
/* indexer query [4][64] fp32 and weights [4] -> E4M3 codes [4][64] and w' [4] */
void  csa2o_quant_iq(const float* iq, const float* iw, uint8_t* qc, float* wq);
/* score of one indexer-K row (64 E4M3 codes, fp32 sigma) */
float csa2o_score(const uint8_t* qc, const float* wq, const uint8_t* kc, float sigma);
/* Full layer, one query.  ikc [>=n_vis][64], iks [>=n_vis].
 * topk_idx [topk] ascending, -1 padded.  pool_idx [pool_blocks] ascending,
 * -1 padded (skipped when pool_blocks == 0).  scores (optional) [n_vis]. */
int csa2o_index_full(const uint8_t* ikc, const float* iks, int64_t n_vis,
                     const float* iq, const float* iw, int topk, int pool_blocks,
                     int32_t* topk_idx, int32_t* pool_idx, float* scores);
/* Reindex layer, one query: own query over the visible positions inside pool_idx. */
int csa2o_index_reindex(const uint8_t* ikc, const float* iks, int64_t n_vis,
                        const float* iq, const float* iw, const int32_t* pool_idx,
                        int pool_blocks, int topk, int32_t* topk_idx);
/* batched over B sequences x Q queries (OpenMP over queries; same per-query arithmetic).
 * ikc [B][cap][64], iks [B][cap], iq [B][Q][4][64], iw [B][Q][4], n_vis [B][Q],
 * topk_idx [B][Q][topk], pool_idx [B][Q][pool_blocks] (may be NULL if pool_blocks==0). */
int csa2o_index_full_batch(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                           const float* iq, const float* iw, const int32_t* n_vis,
                           int topk, int pool_blocks, int32_t* topk_idx, int32_t* pool_idx);
int csa2o_index_reindex_batch(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                              const float* iq, const float* iw, const int32_t* n_vis,
                              const int32_t* pool_idx, int pool_blocks, int topk,
                              int32_t* topk_idx);

/* ---- sparse attention (fp64) ----
 * q [H][128]; global codes [*][128], scales [*][16]; idx [topk] (-1 = none);
 * swa_k, swa_v [*][128] E4M3, swa_ks, swa_vs [*] fp32, tokens [0, swa_len).
 * out [H][128], lse [H] (natural log of the softmax denominator incl. max). */
void csa2o_attn(const float* q, int H, const uint8_t* codes, const uint8_t* scales,
                const int32_t* idx, int topk, const uint8_t* swa_k, const uint8_t* swa_v,
                const float* swa_ks, const float* swa_vs, int swa_len, float sm_scale,
                float* out, float* lse);
/* batched decode: B sequences each with its own cache [B][cap]; SWA [B][128]. */
void csa2o_attn_decode_batch(const float* q, int B, int H, const uint8_t* codes,
                             const uint8_t* scales, int64_t cap, const int32_t* idx, int topk,
                             const uint8_t* swa_k, const uint8_t* swa_v, const float* swa_ks,
                             const float* swa_vs, const int32_t* swa_len, float sm_scale,
                             float* out, float* lse);
/* batched chunk: q [B][Q][H][128], idx [B][Q][topk], chunk SWA [B][Q][128];
 * query i sees chunk SWA tokens [max(0, i - 127), i]. */
void csa2o_attn_chunk_batch(const float* q, int B, int Q, int H, const uint8_t* codes,
                            const uint8_t* scales, int64_t cap, const int32_t* idx, int topk,
                            const uint8_t* swa_k, const uint8_t* swa_v, const float* swa_ks,
                            const float* swa_vs, float sm_scale, float* out, float* lse);

/* ---- FP4 indexer key (36 B per position: codes [n][32], scales [n][4]) ---- */
void  csa2o_idx4_quant_rows(const float* x, int64_t n, uint8_t* codes, uint8_t* scales);
float csa2o_score4(const uint8_t* qc, const float* wq, const uint8_t* kc, const uint8_t* ks);
int csa2o_index_full4(const uint8_t* kc4, const uint8_t* ks4, int64_t n_vis, const float* iq,
                      const float* iw, int topk, int pool_blocks, int32_t* topk_idx,
                      int32_t* pool_idx, float* scores);
int csa2o_index_reindex4(const uint8_t* kc4, const uint8_t* ks4, int64_t n_vis, const float* iq,
                         const float* iw, const int32_t* pool_idx, int pool_blocks, int topk,
                         int32_t* topk_idx);
int csa2o_index_full4_batch(const uint8_t* kc4, const uint8_t* ks4, int64_t cap, int B, int Q,
                            const float* iq, const float* iw, const int32_t* n_vis, int topk,
                            int pool_blocks, int32_t* topk_idx, int32_t* pool_idx);
int csa2o_index_reindex4_batch(const uint8_t* kc4, const uint8_t* ks4, int64_t cap, int B, int Q,
                               const float* iq, const float* iw, const int32_t* n_vis,
                               const int32_t* pool_idx, int pool_blocks, int topk,
                               int32_t* topk_idx);

int csa2o_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
