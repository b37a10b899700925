/* Drives every oracle function on small seeded inputs (ragged, empty and
 * over-long cases included) so that an AddressSanitizer / UndefinedBehavior-
 * Sanitizer build of the oracle can check its memory accesses.  Test
 * infrastructure: built and run by tests/test_oracle_sanitize.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "csa2_oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static float unit_normal(void) {  /* sum of 12 uniforms - 6 (a rough normal) */
    float s = 0.0f;
    for (int i = 0; i < 12; ++i) {
        state = state * 6364136223846793005ull + 1442695040888963407ull;
        s += (float)(state >> 40) / (float)(1ull << 24);
    }
    return s - 6.0f;
}
static void fill(float* x, int64_t n) { for (int64_t i = 0; i < n; ++i) x[i] = unit_normal(); }
static void* xmalloc(size_t n) { void* p = malloc(n ? n : 1); if (!p) abort(); return p; }

int main(void) {
    enum { N = 300, H = 16, Q = 140 };
    float* k = xmalloc(sizeof(float) * 2 * N * 128);
    float* v = xmalloc(sizeof(float) * 2 * N * 128);
    fill(k, 2 * N * 128);
    fill(v, 2 * N * 128);
    int64_t pos[N];
    for (int i = 0; i < N; ++i) pos[i] = 1000 + i;
    float* cs = xmalloc(sizeof(float) * N * 64);
    csa2o_rope_table(pos, N, 10000.0, cs);
    uint8_t* codes = xmalloc(N * 128);
    uint8_t* scales = xmalloc(N * 16);
    if (csa2o_quant_fp4(k, v, N, 1, cs, codes, scales)) return 1;
    if (csa2o_quant_fp4(k, v, 2 * N, 2, NULL, codes, scales)) return 1;  /* N entries */
    if (csa2o_quant_fp4(k, v, 7, 2, NULL, codes, scales) != -1) return 1;

    /* indexer keys: projected, FP8 and FP4 */
    float* W = xmalloc(sizeof(float) * 64 * 128);
    fill(W, 64 * 128);
    float* ek = xmalloc(sizeof(float) * N * 128);
    float* key = xmalloc(sizeof(float) * N * 64);
    if (csa2o_entry_k(k, N, 1, cs, ek)) return 1;
    csa2o_project_idx_rows(ek, N, W, key);
    uint8_t* ikc = xmalloc(N * 64);
    float* iks = xmalloc(sizeof(float) * N);
    csa2o_quant_fp8_rows(key, N, 64, ikc, iks);
    uint8_t* kc4 = xmalloc(N * 32);
    uint8_t* ks4 = xmalloc(N * 4);
    csa2o_idx4_quant_rows(key, N, kc4, ks4);

    float iq[Q * 256], iw[Q * 4];
    fill(iq, Q * 256);
    for (int i = 0; i < Q * 4; ++i) iw[i] = fabsf(unit_normal());
    int32_t nvis[Q];
    for (int i = 0; i < Q; ++i) nvis[i] = (i * 37) % (N + 1);  /* 0 .. N, ragged */
    int32_t* tk = xmalloc(sizeof(int32_t) * Q * 64);
    int32_t* pl = xmalloc(sizeof(int32_t) * Q * 16);
    int32_t* rk = xmalloc(sizeof(int32_t) * Q * 24);
    float* sc = xmalloc(sizeof(float) * N);
    for (int fmt = 0; fmt < 2; ++fmt) {
        if (fmt == 0) {
            if (csa2o_index_full_batch(ikc, iks, N, 1, Q, iq, iw, nvis, 64, 16, tk, pl)) return 1;
            if (csa2o_index_reindex_batch(ikc, iks, N, 1, Q, iq, iw, nvis, pl, 16, 24, rk)) return 1;
            if (csa2o_index_full(ikc, iks, N, iq, iw, 500, 0, tk, NULL, sc)) return 1;
        } else {
            if (csa2o_index_full4_batch(kc4, ks4, N, 1, Q, iq, iw, nvis, 64, 16, tk, pl)) return 1;
            if (csa2o_index_reindex4_batch(kc4, ks4, N, 1, Q, iq, iw, nvis, pl, 16, 24, rk)) return 1;
            if (csa2o_index_full4(kc4, ks4, N, iq, iw, 500, 0, tk, NULL, sc)) return 1;
        }
    }

    /* attention: decode (window lengths 0 .. 128) and a chunk past 128 tokens */
    float* q = xmalloc(sizeof(float) * Q * H * 128);
    fill(q, Q * H * 128);
    float* wx = xmalloc(sizeof(float) * Q * 128);
    fill(wx, Q * 128);
    uint8_t* swk = xmalloc(Q * 128);
    uint8_t* swv = xmalloc(Q * 128);
    float* sks = xmalloc(sizeof(float) * Q);
    float* svs = xmalloc(sizeof(float) * Q);
    csa2o_quant_fp8_rows(wx, Q, 128, swk, sks);
    fill(wx, Q * 128);
    csa2o_quant_fp8_rows(wx, Q, 128, swv, svs);
    int32_t idx[Q * 64];
    for (int i = 0; i < Q * 64; ++i) idx[i] = (i % 7 == 0) ? -1 : (int32_t)((i * 13) % N);
    float* out = xmalloc(sizeof(float) * Q * H * 128);
    float* lse = xmalloc(sizeof(float) * Q * H);
    int32_t swa_len[1];
    for (int len = 0; len <= 128; len += 64) {
        swa_len[0] = len;
        csa2o_attn_decode_batch(q, 1, H, codes, scales, N, idx, 64, swk, swv, sks, svs, swa_len,
                                0.088f, out, lse);
    }
    csa2o_attn_chunk_batch(q, 1, Q, H, codes, scales, N, idx, 64, swk, swv, sks, svs, 0.088f,
                           out, lse);
    double check = 0.0;
    for (int i = 0; i < Q * H * 128; ++i) check += out[i];
    printf("oracle sanitize run ok (%g)\n", check);
    free(k); free(v); free(cs); free(codes); free(scales); free(W); free(ek); free(key);
    free(ikc); free(iks); free(kc4); free(ks4); free(tk); free(pl); free(rk); free(sc);
    free(q); free(wx); free(swk); free(swv); free(sks); free(svs); free(out); free(lse);
    return 0;
}
