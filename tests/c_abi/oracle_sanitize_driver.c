/*
 * The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
 * code only): random small cases -- ids in [-1, E] (invalid ones included),
 * every row element size, both useWeights, 0..70 forwarded scales, bf16 and
 * fp32 combine rows into bf16 and fp32 output --
 * through oracle_dispatch, oracle_combine, oracle_combine_push and
 * oracle_combine_reduce, every buffer malloc'd at exactly its documented
 * size so that any access past an end is reported.  Exit 0 = clean.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_dispatch(int32_t W, int32_t H, int32_t M, int32_t Epr, int32_t K, int32_t useWeights, int32_t T,
                    int32_t elemBytes, int32_t S, const void *x, const int32_t *expertIds, const float *weights,
                    const float *scales, void *recvX, int32_t *recvTokIdx, int32_t *recvExpertIds,
                    float *recvWeights, float *recvScales, int32_t *recvCount, int32_t *sendMap);
int oracle_combine(int32_t W, int32_t H, int32_t M, int32_t Epr, int32_t K, int32_t useWeights, int32_t T,
                   int32_t inFp32, int32_t outFp32, const void *y, const int32_t *expertIds, const float *weights,
                   const int32_t *sendMap, const int32_t *tokens, int32_t nList, float *acc, void *out);
int oracle_combine_push(int32_t W, int32_t H, int32_t M, int32_t Epr, int32_t K, int32_t useWeights, int32_t T,
                        int32_t fp32, const void *y, const int32_t *recvExpertIds, const float *recvWeights,
                        const int32_t *recvCount, void *landing, float *landScale);
int oracle_combine_reduce(int32_t W, int32_t H, int32_t M, int32_t Epr, int32_t K, int32_t useWeights, int32_t T,
                          int32_t inFp32, int32_t outFp32, const void *landing, const float *landScale,
                          const int32_t *recvCount, const int32_t *sendMap, const int32_t *tokens, int32_t nList,
                          float *acc, void *out);

static uint64_t s = 88172645463325252ull;
static uint32_t rnd(void) {
    s ^= s << 13;
    s ^= s >> 7;
    s ^= s << 17;
    return (uint32_t)s;
}
static int32_t range(int32_t lo, int32_t hi) { return lo + (int32_t)(rnd() % (uint32_t)(hi - lo + 1)); }

int main(void) {
    for (int c = 0; c < 400; ++c) {
        const int32_t W = range(1, 9), Epr = range(1, 4), E = W * Epr;
        const int32_t K = range(1, E < 9 ? E : 9), T = range(0, 40), M = T + range(0, 3) + (T == 0);
        const int32_t H = range(1, 24), eb = (int32_t[]){1, 2, 4}[c % 3], useW = (c / 3) % 2;
        const int32_t fp32 = (c / 6) % 2, yb = fp32 ? 4 : 2, land = T * (W < K ? W : K);
        const int32_t ofp32 = (c / 12) % 2, ob = ofp32 ? 4 : 2, S = (c % 5 == 0) ? 0 : range(1, 70);
        unsigned char *x = malloc((size_t)T * H * eb + 1), *recvX = malloc((size_t)W * M * H * eb);
        int32_t *ids = malloc(sizeof(int32_t) * T * K + 1), *tok = malloc(sizeof(int32_t) * W * M);
        int32_t *rids = malloc(sizeof(int32_t) * W * M * K), *cnt = malloc(sizeof(int32_t) * W);
        int32_t *map = malloc(sizeof(int32_t) * T * K + 1);
        float *w = malloc(sizeof(float) * T * K + 1), *rw = malloc(sizeof(float) * W * M * K);
        unsigned char *y = malloc((size_t)W * M * H * yb), *out = malloc((size_t)T * H * ob + 1);
        unsigned char *out2 = malloc((size_t)T * H * ob + 1), *landing = malloc((size_t)land * H * yb + 1);
        float *scl = malloc(sizeof(float) * T * S + 1), *rscl = malloc(sizeof(float) * W * M * S + 1);
        for (int32_t i = 0; i < T * S; ++i) scl[i] = (float)range(-100, 100) / 64.0f;
        float *scale = malloc(sizeof(float) * land + 1), *acc = malloc(sizeof(float) * H);
        for (int32_t i = 0; i < T * H * eb; ++i) x[i] = (unsigned char)rnd();
        for (int32_t i = 0; i < T * K; ++i) {
            ids[i] = range(-1, E);
            w[i] = (float)range(-1000, 1000) / 500.0f;
        }
        for (int32_t i = 0; i < W * M * H; ++i) {
            if (fp32) ((float *)y)[i] = (float)range(-4000, 4000) / 1000.0f;
            else ((uint16_t *)y)[i] = (uint16_t)(((rnd() & 1u) << 15) | ((120u + rnd() % 14u) << 7) | (rnd() & 0x7fu));
        }
        memset(recvX, 0, (size_t)W * M * H * eb);
        memset(tok, 0, sizeof(int32_t) * W * M);
        memset(rids, 0, sizeof(int32_t) * W * M * K);
        memset(rw, 0, sizeof(float) * W * M * K);
        int rc = oracle_dispatch(W, H, M, Epr, K, useW, T, eb, S, x, ids, useW ? w : NULL, S ? scl : NULL, recvX,
                                 tok, rids, useW ? rw : NULL, S ? rscl : NULL, cnt, map);
        rc |= oracle_combine(W, H, M, Epr, K, useW, T, fp32, ofp32, y, ids, useW ? w : NULL, map, NULL, T, acc,
                             out);
        rc |= oracle_combine_push(W, H, M, Epr, K, useW, T, fp32, y, rids, useW ? rw : NULL, cnt, landing,
                                  useW ? scale : NULL);
        rc |= oracle_combine_reduce(W, H, M, Epr, K, useW, T, fp32, ofp32, landing, useW ? scale : NULL, cnt, map,
                                    NULL, T, acc, out2);
        if (rc) {
            fprintf(stderr, "case %d rejected (W %d K %d T %d)\n", c, W, K, T);
            return 1;
        }
        if (T && memcmp(out, out2, (size_t)T * H * ob) != 0) {
            fprintf(stderr, "case %d: push + reduce differs from the gather\n", c);
            return 1;
        }
        free(x); free(recvX); free(ids); free(tok); free(rids); free(cnt); free(map); free(w); free(rw);
        free(y); free(out); free(out2); free(landing); free(scale); free(acc); free(scl); free(rscl);
    }
    printf("oracle sanitized ok\n");
    return 0;
}
