/*
 * csa2_oracle.c -- plain, slow CPU oracle for the CSA2 decode path.
 *
 * TEST INFRASTRUCTURE ONLY (see csa2_oracle.h).  Built with gcc, -O2,
 * -ffp-contract=off, no fast-math: every float expression below is the IEEE
 * single-precision operation it reads as, in the order it is written.
 *
 * Page references use the two technical pages:
 *   [notes]  "DeepSeek V4.1 Flash: architecture study notes", sections 1-4;
 *   [digest] "DeepSeek V4.1 Flash is live", sections "CSA2 attention" and
 *            "cache precision and persistence tiers".
 */
#include "csa2_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX_HEADS 4
#define IDX_DIM 64
#define HEAD_DIM 128
#define WINDOW 128
#define BLOCK 8

int csa2o_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Number formats.  [notes] section 4 / [digest] "cache precision": main KV
 * values are E2M1 with one E4M3 scale per 16 channels; SWA KV stays FP8.
 * E4M3 here is the OCP 8-bit format: 1 sign, 4 exponent bits (bias 7),
 * 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448.
 * ---------------------------------------------------------------------- */
double csa2o_e4m3_decode(uint8_t code) {
    int sign = code >> 7;
    int exp_field = (code >> 3) & 0xF;
    int mant = code & 0x7;
    double mag;
    if (exp_field == 0xF && mant == 0x7) return NAN;
    if (exp_field == 0)
        mag = ldexp((double)mant / 8.0, 1 - 7);          /* subnormal */
    else
        mag = ldexp(1.0 + (double)mant / 8.0, exp_field - 7);
    return sign ? -mag : mag;
}

/* Round to the nearest finite E4M3 value; on an exact tie take the code
 * whose last mantissa bit is 0; anything beyond 448 saturates to 448.
 * Codes 0x00..0x7E list the non-negative finite values in increasing order,
 * so the nearest one is found by a binary search over those 127 codes. */
uint8_t csa2o_e4m3_encode(float x) {
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    int lo = 0, hi = 0x7E;
    if (a >= csa2o_e4m3_decode(0x7E)) return sign | 0x7E;
    /* invariant: value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (csa2o_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    double d_lo = a - csa2o_e4m3_decode((uint8_t)lo);
    double d_hi = csa2o_e4m3_decode((uint8_t)hi) - a;
    int code;
    if (d_lo < d_hi) code = lo;
    else if (d_hi < d_lo) code = hi;
    else code = (lo % 2 == 0) ? lo : hi;
    return sign | (uint8_t)code;
}

/* OCP MX E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit.
 * Magnitudes by code 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double csa2o_e2m1_decode(uint8_t code) {
    int sign = (code >> 3) & 1;
    int exp_field = (code >> 1) & 0x3;
    int mant = code & 1;
    double mag;
    if (exp_field == 0)
        mag = 0.5 * mant;                                  /* subnormal: m * 2^(1-1) / 2 */
    else
        mag = ldexp(1.0 + 0.5 * mant, exp_field - 1);
    return sign ? -mag : mag;
}

/* Nearest of the 8 magnitudes, ties to the even code, saturating at 6. */
uint8_t csa2o_e2m1_encode(float t) {
    uint8_t sign = signbit(t) ? 0x8 : 0x0;
    double a = fabs((double)t);
    if (a >= 6.0) return sign | 7;                         /* saturate (also +-inf) */
    int best = 0;
    double best_d = a;                                     /* distance to code 0 (value 0) */
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - csa2o_e2m1_decode((uint8_t)c));
        if (d < best_d || (d == best_d && c % 2 == 0 && best % 2 != 0)) {
            best = c;
            best_d = d;
        }
    }
    return sign | (uint8_t)best;
}

/* ------------------------------------------------------------------------
 * Write path.
 * ---------------------------------------------------------------------- */

/* [notes] section 3: encoder groups merge 2 tokens into 1 entry; [digest]
 * "CSA2 attention": adjacent compressed entries do not overlap.  Reading:
 * the entry is the plain mean of a disjoint pair, fl(fl(a+b)*0.5). */
void csa2o_average_pair(const float* a, const float* b, int n, float* out) {
    for (int c = 0; c < n; ++c) {
        float s = a[c] + b[c];
        out[c] = s * 0.5f;
    }
}

/* [digest] "cache precision": the quantisation point is after RoPE.  Reading:
 * RoPE on channels 0..63 of K, interleaved pairs, base 10000, angles in fp64,
 * rounded to fp32 once. */
void csa2o_rope_table(const int64_t* pos, int64_t n, double base, float* cs) {
    for (int64_t i = 0; i < n; ++i) {
        for (int j = 0; j < 32; ++j) {
            double theta = pow(base, -(double)j / 32.0);
            double ang = (double)pos[i] * theta;
            cs[(i * 32 + j) * 2 + 0] = (float)cos(ang);
            cs[(i * 32 + j) * 2 + 1] = (float)sin(ang);
        }
    }
}

void csa2o_rope_apply(float* x, const float* cs_row) {
    for (int j = 0; j < 32; ++j) {
        float c = cs_row[2 * j + 0];
        float s = cs_row[2 * j + 1];
        float x0 = x[2 * j];
        float x1 = x[2 * j + 1];
        float a = x0 * c;
        float b = x1 * s;
        float d = x0 * s;
        float e = x1 * c;
        x[2 * j] = a - b;
        x[2 * j + 1] = d + e;
    }
}

/* [notes] section 4: E2M1 values, one 8-bit (E4M3) scale per 16 channels,
 * 4 + 8/16 = 4.5 bits per value; [digest] "cache precision": no second-level
 * global scale.  Reading: scale = RNE_E4M3(amax/6); a zero scale gives
 * signed-zero codes; code = RNE_E2M1(x/scale). */
void csa2o_fp4_quant_vec(const float* x, uint8_t* codes, uint8_t* scales) {
    csa2o_fp4_quant_groups(x, HEAD_DIM / 16, codes, scales);
}

void csa2o_fp4_quant_groups(const float* x, int n_groups, uint8_t* codes, uint8_t* scales) {
    for (int g = 0; g < n_groups; ++g) {
        const float* xg = x + 16 * g;
        float amax = 0.0f;
        for (int i = 0; i < 16; ++i) {
            float a = fabsf(xg[i]);
            if (a > amax) amax = a;
        }
        float s32 = amax / 6.0f;
        uint8_t sc = csa2o_e4m3_encode(s32);
        float sd = (float)csa2o_e4m3_decode(sc);
        scales[g] = sc;
        for (int i = 0; i < 16; ++i) {
            uint8_t code;
            if (sd == 0.0f) {
                code = signbit(xg[i]) ? 0x8 : 0x0;
            } else {
                float t = xg[i] / sd;
                code = csa2o_e2m1_encode(t);
            }
            int ch = 16 * g + i;
            if (ch % 2 == 0)
                codes[ch / 2] = (uint8_t)((codes[ch / 2] & 0xF0) | code);
            else
                codes[ch / 2] = (uint8_t)((codes[ch / 2] & 0x0F) | (code << 4));
        }
    }
}

int csa2o_quant_fp4(const float* k, const float* v, int64_t n_tok, int ratio,
                    const float* rope_cs, uint8_t* codes, uint8_t* scales) {
    if (ratio != 1 && ratio != 2) return -1;
    if (n_tok % ratio != 0) return -1;
    if (ratio == 2 && rope_cs != NULL) return -1;
    int64_t n_ent = n_tok / ratio;
    for (int64_t e = 0; e < n_ent; ++e) {
        float kx[HEAD_DIM], vx[HEAD_DIM];
        if (ratio == 2) {
            csa2o_average_pair(k + (2 * e) * HEAD_DIM, k + (2 * e + 1) * HEAD_DIM, HEAD_DIM, kx);
            csa2o_average_pair(v + (2 * e) * HEAD_DIM, v + (2 * e + 1) * HEAD_DIM, HEAD_DIM, vx);
        } else {
            memcpy(kx, k + e * HEAD_DIM, sizeof kx);
            memcpy(vx, v + e * HEAD_DIM, sizeof vx);
        }
        if (rope_cs != NULL) csa2o_rope_apply(kx, rope_cs + e * 64);
        uint8_t* c = codes + e * 128;
        uint8_t* s = scales + e * 16;
        memset(c, 0, 128);
        csa2o_fp4_quant_vec(kx, c, s);
        csa2o_fp4_quant_vec(vx, c + 64, s + 8);
    }
    return 0;
}

int csa2o_entry_k(const float* k, int64_t n_tok, int ratio, const float* rope_cs, float* out) {
    if (ratio != 1 && ratio != 2) return -1;
    if (n_tok % ratio != 0) return -1;
    if (ratio == 2 && rope_cs != NULL) return -1;
    for (int64_t e = 0; e < n_tok / ratio; ++e) {
        float* x = out + e * HEAD_DIM;
        if (ratio == 2)
            csa2o_average_pair(k + (2 * e) * HEAD_DIM, k + (2 * e + 1) * HEAD_DIM, HEAD_DIM, x);
        else
            memcpy(x, k + e * HEAD_DIM, HEAD_DIM * sizeof(float));
        if (rope_cs != NULL) csa2o_rope_apply(x, rope_cs + e * 64);
    }
    return 0;
}

/* [digest] "CSA2 attention": the indexer key is projected from the main-KV
 * entry, not compressed from hidden states separately.  Reading: a 128 -> 64
 * linear map of the entry's fp32 K (after the pair mean / RoPE, before FP4
 * quantisation), each output one fp32 accumulation over the input channels in
 * ascending order, every step a fused multiply-add (C99 fmaf: one rounding),
 * starting from +0. */
void csa2o_project_idx(const float* x, const float* W, float* key) {
    for (int j = 0; j < IDX_DIM; ++j) {
        float acc = 0.0f;
        for (int c = 0; c < HEAD_DIM; ++c) acc = fmaf(W[j * HEAD_DIM + c], x[c], acc);
        key[j] = acc;
    }
}

void csa2o_project_idx_rows(const float* x, int64_t n, const float* W, float* keys) {
    for (int64_t i = 0; i < n; ++i) csa2o_project_idx(x + i * HEAD_DIM, W, keys + i * IDX_DIM);
}

/* SWA K/V and indexer K are FP8 ([notes] section 4, [digest] "cache
 * precision").  Reading: one fp32 scale per row, sigma = amax/448. */
void csa2o_fp8_quant_row(const float* x, int dim, uint8_t* codes, float* sigma) {
    float amax = 0.0f;
    for (int i = 0; i < dim; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float s = amax / 448.0f;
    *sigma = s;
    for (int i = 0; i < dim; ++i) {
        if (s == 0.0f)
            codes[i] = signbit(x[i]) ? 0x80 : 0x00;
        else
            codes[i] = csa2o_e4m3_encode(x[i] / s);
    }
}

void csa2o_quant_fp8_rows(const float* x, int64_t n_rows, int dim, uint8_t* codes, float* sigma) {
    for (int64_t r = 0; r < n_rows; ++r)
        csa2o_fp8_quant_row(x + r * dim, dim, codes + r * dim, sigma + r);
}

/* ------------------------------------------------------------------------
 * Indexer.  [notes] section 2: Full builds the global KV and picks this
 * step's positions; Reindex rescores with its own indexer query; Reuse keeps
 * the latest top-K; at most 512 global records per query; the decoder's
 * first Full layer scans every causally visible position and builds a pool
 * of at most 2048 blocks x 8 positions (Figure 5), Reindex layers pick
 * their own top-512 inside it.
 * ---------------------------------------------------------------------- */

/* Indexer query in E4M3 with a per-head fp32 scale folded into the head
 * weight: sq = amax/448, code = RNE_E4M3(q/sq), w' = w*sq. */
void csa2o_quant_iq(const float* iq, const float* iw, uint8_t* qc, float* wq) {
    for (int h = 0; h < IDX_HEADS; ++h) {
        float sq;
        csa2o_fp8_quant_row(iq + h * IDX_DIM, IDX_DIM, qc + h * IDX_DIM, &sq);
        wq[h] = iw[h] * sq;
    }
}

/* score = sigma * sum_h w'_h * ReLU(q_h . k), all in fp32:
 *   dot_h: channels 0..63 in order, starting from +0 (each E4M3 x E4M3
 *          product is exact in fp32, so only the order of the sums matters);
 *   r_h  = dot_h if dot_h > 0 else +0;
 *   t    = w'_0 r_0, then t += w'_h r_h for h = 1..3 (rounded mul, then add);
 *   score = sigma * t. */
float csa2o_score(const uint8_t* qc, const float* wq, const uint8_t* kc, float sigma) {
    float t = 0.0f;
    for (int h = 0; h < IDX_HEADS; ++h) {
        float dot = 0.0f;
        for (int c = 0; c < IDX_DIM; ++c) {
            float a = (float)csa2o_e4m3_decode(qc[h * IDX_DIM + c]);
            float b = (float)csa2o_e4m3_decode(kc[c]);
            float p = a * b;
            dot = dot + p;
        }
        float r = dot > 0.0f ? dot : 0.0f;
        float wr = wq[h] * r;
        t = (h == 0) ? wr : t + wr;
    }
    return sigma * t;
}

typedef struct {
    float key;
    int64_t index;
} ranked_t;

/* larger key first; equal keys: lower index first (floats compare, so -0 == +0) */
static int cmp_rank(const void* pa, const void* pb) {
    const ranked_t* a = (const ranked_t*)pa;
    const ranked_t* b = (const ranked_t*)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    if (a->index < b->index) return -1;
    if (a->index > b->index) return 1;
    return 0;
}

static int cmp_i32(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

/* Take the first `keep` entries of `r[0..n)` in rank order, write their
 * indices ascending into out[0..cap), pad with -1. */
static void take_top(ranked_t* r, int64_t n, int cap, int32_t* out) {
    qsort(r, (size_t)n, sizeof(ranked_t), cmp_rank);
    int64_t keep = n < cap ? n : cap;
    for (int64_t i = 0; i < keep; ++i) out[i] = (int32_t)r[i].index;
    qsort(out, (size_t)keep, sizeof(int32_t), cmp_i32);
    for (int64_t i = keep; i < cap; ++i) out[i] = -1;
}

/* score of visible position s of one sequence's indexer keys */
typedef float (*row_score_fn)(const uint8_t* qc, const float* wq, const void* kc, const void* ks,
                              int64_t s);

static float score_fp8_row(const uint8_t* qc, const float* wq, const void* kc, const void* ks,
                           int64_t s) {
    return csa2o_score(qc, wq, (const uint8_t*)kc + s * IDX_DIM, ((const float*)ks)[s]);
}

static float score_fp4_row(const uint8_t* qc, const float* wq, const void* kc, const void* ks,
                           int64_t s) {
    return csa2o_score4(qc, wq, (const uint8_t*)kc + s * (IDX_DIM / 2),
                        (const uint8_t*)ks + s * (IDX_DIM / 16));
}

static int index_full_any(row_score_fn fn, const void* kc, const void* ks, int64_t n_vis,
                          const float* iq, const float* iw, int topk, int pool_blocks,
                          int32_t* topk_idx, int32_t* pool_idx, float* scores) {
    if (n_vis < 0 || topk < 0 || pool_blocks < 0) return -1;
    uint8_t qc[IDX_HEADS * IDX_DIM];
    float wq[IDX_HEADS];
    csa2o_quant_iq(iq, iw, qc, wq);

    float* sc = (float*)malloc(sizeof(float) * (size_t)(n_vis > 0 ? n_vis : 1));
    for (int64_t s = 0; s < n_vis; ++s) sc[s] = fn(qc, wq, kc, ks, s);
    if (scores) memcpy(scores, sc, sizeof(float) * (size_t)n_vis);

    /* own top-K over every visible position */
    ranked_t* r = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)(n_vis > 0 ? n_vis : 1));
    for (int64_t s = 0; s < n_vis; ++s) { r[s].key = sc[s]; r[s].index = s; }
    take_top(r, n_vis, topk, topk_idx);

    /* block pool: block b covers positions [8b, 8b+8) that are visible;
     * its score is the max over those positions */
    if (pool_blocks > 0) {
        int64_t n_blocks = (n_vis + BLOCK - 1) / BLOCK;
        for (int64_t b = 0; b < n_blocks; ++b) {
            float m = sc[b * BLOCK];
            for (int64_t s = b * BLOCK + 1; s < b * BLOCK + BLOCK && s < n_vis; ++s)
                if (sc[s] > m) m = sc[s];
            r[b].key = m;
            r[b].index = b;
        }
        take_top(r, n_blocks, pool_blocks, pool_idx);
    }
    free(r);
    free(sc);
    return 0;
}

static int index_reindex_any(row_score_fn fn, const void* kc, const void* ks, int64_t n_vis,
                             const float* iq, const float* iw, const int32_t* pool_idx,
                             int pool_blocks, int topk, int32_t* topk_idx) {
    if (n_vis < 0 || topk < 0 || pool_blocks < 0) return -1;
    uint8_t qc[IDX_HEADS * IDX_DIM];
    float wq[IDX_HEADS];
    csa2o_quant_iq(iq, iw, qc, wq);
    ranked_t* r = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)pool_blocks * BLOCK + 1);
    int64_t n = 0;
    for (int j = 0; j < pool_blocks; ++j) {
        int32_t b = pool_idx[j];
        if (b < 0) continue;
        for (int64_t s = (int64_t)b * BLOCK; s < (int64_t)b * BLOCK + BLOCK; ++s) {
            if (s >= n_vis) break;
            r[n].key = fn(qc, wq, kc, ks, s);
            r[n].index = s;
            ++n;
        }
    }
    take_top(r, n, topk, topk_idx);
    free(r);
    return 0;
}

int csa2o_index_full(const uint8_t* ikc, const float* iks, int64_t n_vis,
                     const float* iq, const float* iw, int topk, int pool_blocks,
                     int32_t* topk_idx, int32_t* pool_idx, float* scores) {
    return index_full_any(score_fp8_row, ikc, iks, n_vis, iq, iw, topk, pool_blocks, topk_idx,
                          pool_idx, scores);
}

int csa2o_index_reindex(const uint8_t* ikc, const float* iks, int64_t n_vis,
                        const float* iq, const float* iw, const int32_t* pool_idx,
                        int pool_blocks, int topk, int32_t* topk_idx) {
    return index_reindex_any(score_fp8_row, ikc, iks, n_vis, iq, iw, pool_idx, pool_blocks, topk,
                             topk_idx);
}

/* ------------------------------------------------------------------------
 * FP4 indexer key.  [notes] section 4: the FP4 main KV builds on the previous
 * generation's FP4 indexer key.  Reading: the indexer key in the main KV's
 * FP4 format -- E2M1 codes (low nibble = even channel) with one E4M3 scale
 * per 16 channels, no per-position scale: 32 + 4 = 36 bytes per position.
 * Score: the block-scaled dot product (the form the OCP Microscaling
 * specification gives for the dot product of block-scaled vectors: each
 * block's element products summed, then scaled by the block scale):
 *   inner_hg = fp32 sum over the 16 channels c of group g in ascending order
 *              of E4M3(q_hc) * E2M1(k_c) (each product exact), from +0;
 *   dot_h    = fused multiply-add chain over g = 0..3 of scale_g * inner_hg,
 *              from +0;
 *   r_h, t as for the FP8 key; score = t (no per-position scale).
 * ---------------------------------------------------------------------- */
void csa2o_idx4_quant_rows(const float* x, int64_t n, uint8_t* codes, uint8_t* scales) {
    for (int64_t i = 0; i < n; ++i)
        csa2o_fp4_quant_groups(x + i * IDX_DIM, IDX_DIM / 16, codes + i * (IDX_DIM / 2),
                               scales + i * (IDX_DIM / 16));
}

float csa2o_score4(const uint8_t* qc, const float* wq, const uint8_t* kc, const uint8_t* ks) {
    float t = 0.0f;
    for (int h = 0; h < IDX_HEADS; ++h) {
        float dot = 0.0f;
        for (int g = 0; g < IDX_DIM / 16; ++g) {
            float inner = 0.0f;
            for (int c = 16 * g; c < 16 * g + 16; ++c) {
                uint8_t nib = (c % 2 == 0) ? (kc[c / 2] & 0x0F) : (kc[c / 2] >> 4);
                float a = (float)csa2o_e4m3_decode(qc[h * IDX_DIM + c]);
                float b = (float)csa2o_e2m1_decode(nib);
                float p = a * b;
                inner = inner + p;
            }
            dot = fmaf((float)csa2o_e4m3_decode(ks[g]), inner, dot);
        }
        float r = dot > 0.0f ? dot : 0.0f;
        float wr = wq[h] * r;
        t = (h == 0) ? wr : t + wr;
    }
    return t;
}

int csa2o_index_full4(const uint8_t* kc4, const uint8_t* ks4, int64_t n_vis, const float* iq,
                      const float* iw, int topk, int pool_blocks, int32_t* topk_idx,
                      int32_t* pool_idx, float* scores) {
    return index_full_any(score_fp4_row, kc4, ks4, n_vis, iq, iw, topk, pool_blocks, topk_idx,
                          pool_idx, scores);
}

int csa2o_index_reindex4(const uint8_t* kc4, const uint8_t* ks4, int64_t n_vis, const float* iq,
                         const float* iw, const int32_t* pool_idx, int pool_blocks, int topk,
                         int32_t* topk_idx) {
    return index_reindex_any(score_fp4_row, kc4, ks4, n_vis, iq, iw, pool_idx, pool_blocks, topk,
                             topk_idx);
}

int csa2o_index_full4_batch(const uint8_t* kc4, const uint8_t* ks4, int64_t cap, int B, int Q,
                            const float* iq, const float* iw, const int32_t* n_vis, int topk,
                            int pool_blocks, int32_t* topk_idx, int32_t* pool_idx) {
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t bq = 0; bq < (int64_t)B * Q; ++bq) {
        int64_t b = bq / Q;
        int rc = csa2o_index_full4(kc4 + b * cap * (IDX_DIM / 2), ks4 + b * cap * (IDX_DIM / 16),
                                   n_vis[bq], iq + bq * IDX_HEADS * IDX_DIM, iw + bq * IDX_HEADS,
                                   topk, pool_blocks, topk_idx + bq * topk,
                                   pool_blocks > 0 ? pool_idx + bq * pool_blocks : NULL, NULL);
        bad |= (rc != 0);
    }
    return bad ? -1 : 0;
}

int csa2o_index_reindex4_batch(const uint8_t* kc4, const uint8_t* ks4, int64_t cap, int B, int Q,
                               const float* iq, const float* iw, const int32_t* n_vis,
                               const int32_t* pool_idx, int pool_blocks, int topk,
                               int32_t* topk_idx) {
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t bq = 0; bq < (int64_t)B * Q; ++bq) {
        int64_t b = bq / Q;
        int rc = csa2o_index_reindex4(kc4 + b * cap * (IDX_DIM / 2),
                                      ks4 + b * cap * (IDX_DIM / 16), n_vis[bq],
                                      iq + bq * IDX_HEADS * IDX_DIM, iw + bq * IDX_HEADS,
                                      pool_idx + bq * pool_blocks, pool_blocks, topk,
                                      topk_idx + bq * topk);
        bad |= (rc != 0);
    }
    return bad ? -1 : 0;
}

int csa2o_index_full_batch(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                           const float* iq, const float* iw, const int32_t* n_vis,
                           int topk, int pool_blocks, int32_t* topk_idx, int32_t* pool_idx) {
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t bq = 0; bq < (int64_t)B * Q; ++bq) {
        int64_t b = bq / Q;
        int rc = csa2o_index_full(ikc + b * cap * IDX_DIM, iks + b * cap, n_vis[bq],
                                  iq + bq * IDX_HEADS * IDX_DIM, iw + bq * IDX_HEADS, topk,
                                  pool_blocks, topk_idx + bq * topk,
                                  pool_blocks > 0 ? pool_idx + bq * pool_blocks : NULL, NULL);
        bad |= (rc != 0);
    }
    return bad ? -1 : 0;
}

int csa2o_index_reindex_batch(const uint8_t* ikc, const float* iks, int64_t cap, int B, int Q,
                              const float* iq, const float* iw, const int32_t* n_vis,
                              const int32_t* pool_idx, int pool_blocks, int topk,
                              int32_t* topk_idx) {
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t bq = 0; bq < (int64_t)B * Q; ++bq) {
        int64_t b = bq / Q;
        int rc = csa2o_index_reindex(ikc + b * cap * IDX_DIM, iks + b * cap, n_vis[bq],
                                     iq + bq * IDX_HEADS * IDX_DIM, iw + bq * IDX_HEADS,
                                     pool_idx + bq * pool_blocks, pool_blocks, topk,
                                     topk_idx + bq * topk);
        bad |= (rc != 0);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------
 * Sparse attention.  [notes] section 2: each query attends to at most 512
 * selected global records together with the local window; [notes] section 1:
 * the local SWA window is 128 tokens; [notes] section 4: values are
 * dequantised on read and then fed to ordinary attention.  Reading: one
 * softmax over (selected entries) u (SWA tokens), logits scaled by sm_scale,
 * evaluated here in fp64 from the exact dequantised values.
 * ---------------------------------------------------------------------- */
static double fp4_value(const uint8_t* codes, const uint8_t* scales, int ch) {
    uint8_t byte = codes[ch / 2];
    uint8_t code = (ch % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    return csa2o_e2m1_decode(code) * csa2o_e4m3_decode(scales[ch / 16]);
}

void csa2o_attn(const float* q, int H, const uint8_t* codes, const uint8_t* scales,
                const int32_t* idx, int topk, const uint8_t* swa_k, const uint8_t* swa_v,
                const float* swa_ks, const float* swa_vs, int swa_len, float sm_scale,
                float* out, float* lse) {
    int n_keys = 0;
    for (int j = 0; j < topk; ++j) n_keys += idx[j] >= 0;
    n_keys += swa_len;
    double* kmat = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1) * HEAD_DIM);
    double* vmat = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1) * HEAD_DIM);
    int n = 0;
    for (int j = 0; j < topk; ++j) {
        if (idx[j] < 0) continue;
        const uint8_t* c = codes + (int64_t)idx[j] * 128;
        const uint8_t* s = scales + (int64_t)idx[j] * 16;
        for (int ch = 0; ch < HEAD_DIM; ++ch) {
            kmat[n * HEAD_DIM + ch] = fp4_value(c, s, ch);
            vmat[n * HEAD_DIM + ch] = fp4_value(c + 64, s + 8, ch);
        }
        ++n;
    }
    for (int t = 0; t < swa_len; ++t) {
        for (int ch = 0; ch < HEAD_DIM; ++ch) {
            kmat[n * HEAD_DIM + ch] = csa2o_e4m3_decode(swa_k[t * HEAD_DIM + ch]) * (double)swa_ks[t];
            vmat[n * HEAD_DIM + ch] = csa2o_e4m3_decode(swa_v[t * HEAD_DIM + ch]) * (double)swa_vs[t];
        }
        ++n;
    }
    double* logit = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int h = 0; h < H; ++h) {
        const float* qh = q + (int64_t)h * HEAD_DIM;
        if (n == 0) {
            for (int ch = 0; ch < HEAD_DIM; ++ch) out[(int64_t)h * HEAD_DIM + ch] = 0.0f;
            lse[h] = -INFINITY;
            continue;
        }
        double m = -INFINITY;
        for (int j = 0; j < n; ++j) {
            double dot = 0.0;
            for (int ch = 0; ch < HEAD_DIM; ++ch) dot += (double)qh[ch] * kmat[j * HEAD_DIM + ch];
            logit[j] = dot * (double)sm_scale;
            if (logit[j] > m) m = logit[j];
        }
        double denom = 0.0;
        for (int j = 0; j < n; ++j) {
            logit[j] = exp(logit[j] - m);
            denom += logit[j];
        }
        for (int ch = 0; ch < HEAD_DIM; ++ch) {
            double acc = 0.0;
            for (int j = 0; j < n; ++j) acc += logit[j] * vmat[j * HEAD_DIM + ch];
            out[(int64_t)h * HEAD_DIM + ch] = (float)(acc / denom);
        }
        lse[h] = (float)(m + log(denom));
    }
    free(logit);
    free(kmat);
    free(vmat);
}

void csa2o_attn_decode_batch(const float* q, int B, int H, const uint8_t* codes,
                             const uint8_t* scales, int64_t cap, const int32_t* idx, int topk,
                             const uint8_t* swa_k, const uint8_t* swa_v, const float* swa_ks,
                             const float* swa_vs, const int32_t* swa_len, float sm_scale,
                             float* out, float* lse) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        csa2o_attn(q + (int64_t)b * H * HEAD_DIM, H, codes + (int64_t)b * cap * 128,
                   scales + (int64_t)b * cap * 16, idx + (int64_t)b * topk, topk,
                   swa_k + (int64_t)b * 128 * HEAD_DIM, swa_v + (int64_t)b * 128 * HEAD_DIM,
                   swa_ks + (int64_t)b * 128, swa_vs + (int64_t)b * 128, swa_len[b], sm_scale,
                   out + (int64_t)b * H * HEAD_DIM, lse + (int64_t)b * H);
    }
}

void csa2o_attn_chunk_batch(const float* q, int B, int Q, int H, const uint8_t* codes,
                            const uint8_t* scales, int64_t cap, const int32_t* idx, int topk,
                            const uint8_t* swa_k, const uint8_t* swa_v, const float* swa_ks,
                            const float* swa_vs, float sm_scale, float* out, float* lse) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bq = 0; bq < (int64_t)B * Q; ++bq) {
        int64_t b = bq / Q;
        int i = (int)(bq % Q);
        /* the window of chunk token i: the last 128 chunk tokens up to and
         * including it ([notes] section 1: a 128-token window per layer) */
        int start = i + 1 > WINDOW ? i + 1 - WINDOW : 0;
        int64_t w0 = b * Q + start;
        csa2o_attn(q + bq * H * HEAD_DIM, H, codes + b * cap * 128, scales + b * cap * 16,
                   idx + bq * topk, topk, swa_k + w0 * HEAD_DIM, swa_v + w0 * HEAD_DIM,
                   swa_ks + w0, swa_vs + w0, i + 1 - start, sm_scale, out + bq * H * HEAD_DIM,
                   lse + bq * H);
    }
}
