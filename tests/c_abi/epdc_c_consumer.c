/*
 * A plain C consumer of libepdc.so: the HIP runtime for device memory and the
 * stream, include/epdc.h for the calls, no PyTorch and no Python.  One small
 * problem (worldSize 4, 3 experts per rank, topk 5, 150 tokens, bf16 rows of
 * 1040 bytes -- not a whole number of 1 KiB chunks -- with some invalid
 * expert ids and 5 forwarded scales per token) goes through dispatch, the
 * gather combine into bf16 and into fp32 output, push and reduce; every
 * output is compared bit for bit with the CPU oracle (liboracle.so).
 *
 * Test infrastructure: it links the oracle.  Exit status 0 = all equal,
 * 1 = a mismatch or a failing call, 77 = no GPU on this host.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/epdc.h"

/* The oracle's entry points (oracle/epdc_oracle.c). */
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

enum { W = 4, EPR = 3, K = 5, M = 200, T = 150, H = 520, S = 5 };

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
/* A finite bf16 pattern of magnitude in [2^-7, 2^8). */
static uint16_t rand_bf16(void) {
    uint32_t r = next_u32();
    return (uint16_t)(((r & 1u) << 15) | ((120u + (r >> 1) % 15u) << 7) | ((r >> 8) & 0x7fu));
}

#define CHECK_HIP(call)                                                                   \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));             \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)
#define CHECK_EPDC(call)                                                                  \
    do {                                                                                  \
        int rc_ = (call);                                                                 \
        if (rc_ != EPDC_OK) {                                                             \
            fprintf(stderr, "%s returned %d: %s\n", #call, rc_, epdc_last_error());       \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

static int same(const char *what, const void *a, const void *b, size_t n) {
    if (memcmp(a, b, n) == 0) return 1;
    const unsigned char *x = (const unsigned char *)a, *y = (const unsigned char *)b;
    size_t i = 0;
    while (x[i] == y[i]) ++i;
    fprintf(stderr, "%s differs first at byte %zu (%02x vs oracle %02x)\n", what, i, x[i], y[i]);
    return 0;
}

int main(void) {
    int nDev = 0;
    if (hipGetDeviceCount(&nDev) != hipSuccess || nDev < 1) {
        printf("no GPU\n");
        return 77;
    }
    CHECK_HIP(hipSetDevice(0));
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));

    const epdc_cfg cfg = {W, H, M, EPR, K, EPDC_BF16, 1, S};
    const size_t rowB = (size_t)H * 2, nWin = (size_t)W * M;
    const int32_t landRows = epdc_landing_rows(&cfg, T);
    const size_t scratchB = epdc_dispatch_scratch_bytes(&cfg);
    if (landRows != T * K - (K - W) * T || scratchB == 0) {  /* T * min(W, K) with K > W */
        fprintf(stderr, "landing rows %d / scratch %zu unexpected\n", landRows, scratchB);
        return 1;
    }

    /* host inputs */
    uint16_t *x = malloc(T * rowB), *y = malloc(nWin * rowB);
    int32_t *ids = malloc(sizeof(int32_t) * T * K);
    float *wts = malloc(sizeof(float) * T * K), *scl = malloc(sizeof(float) * T * S);
    for (int i = 0; i < T * S; ++i) scl[i] = (float)(next_u32() % 4096) / 256.0f;
    for (size_t i = 0; i < (size_t)T * H; ++i) x[i] = rand_bf16();
    for (size_t i = 0; i < nWin * H; ++i) y[i] = rand_bf16();
    for (int i = 0; i < T * K; ++i) {
        ids[i] = (int32_t)(next_u32() % (W * EPR + 2)) - 1; /* [-1, E]: the ends are dropped slots */
        wts[i] = (float)(next_u32() % 2001) / 1000.0f - 1.0f;
    }

    /* device buffers, outputs pre-filled with sentinels */
    void *dx, *dy, *drecvX, *dout, *dout2, *dout32, *dland, *dscratch;
    int32_t *dids, *dtok, *drids, *dcnt, *dmap;
    float *dw, *drw, *dscale, *dscl, *drscl;
    CHECK_HIP(hipMalloc((void **)&dscl, sizeof(float) * T * S));
    CHECK_HIP(hipMalloc((void **)&drscl, sizeof(float) * nWin * S));
    CHECK_HIP(hipMalloc(&dout32, (size_t)T * H * 4));
    CHECK_HIP(hipMemcpy(dscl, scl, sizeof(float) * T * S, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(drscl, 0x55, sizeof(float) * nWin * S));
    CHECK_HIP(hipMalloc(&dx, T * rowB));
    CHECK_HIP(hipMalloc(&dy, nWin * rowB));
    CHECK_HIP(hipMalloc((void **)&dids, sizeof(int32_t) * T * K));
    CHECK_HIP(hipMalloc((void **)&dw, sizeof(float) * T * K));
    CHECK_HIP(hipMalloc(&drecvX, nWin * rowB));
    CHECK_HIP(hipMalloc((void **)&dtok, sizeof(int32_t) * nWin));
    CHECK_HIP(hipMalloc((void **)&drids, sizeof(int32_t) * nWin * K));
    CHECK_HIP(hipMalloc((void **)&drw, sizeof(float) * nWin * K));
    CHECK_HIP(hipMalloc((void **)&dcnt, sizeof(int32_t) * W));
    CHECK_HIP(hipMalloc((void **)&dmap, sizeof(int32_t) * T * K));
    CHECK_HIP(hipMalloc(&dscratch, scratchB));
    CHECK_HIP(hipMalloc(&dout, T * rowB));
    CHECK_HIP(hipMalloc(&dout2, T * rowB));
    CHECK_HIP(hipMalloc(&dland, (size_t)landRows * rowB));
    CHECK_HIP(hipMalloc((void **)&dscale, sizeof(float) * landRows));
    CHECK_HIP(hipMemcpy(dx, x, T * rowB, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dy, y, nWin * rowB, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dids, ids, sizeof(int32_t) * T * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dw, wts, sizeof(float) * T * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(drecvX, 0xAD, nWin * rowB));
    CHECK_HIP(hipMemset(dtok, 0x11, sizeof(int32_t) * nWin));
    CHECK_HIP(hipMemset(drids, 0x22, sizeof(int32_t) * nWin * K));
    CHECK_HIP(hipMemset(drw, 0x33, sizeof(float) * nWin * K));
    CHECK_HIP(hipMemset(dscratch, 0, scratchB));
    CHECK_HIP(hipMemset(dland, 0xA5, (size_t)landRows * rowB));
    CHECK_HIP(hipMemset(dscale, 0x44, sizeof(float) * landRows));

    CHECK_EPDC(epdc_dispatch(&cfg, T, dx, dids, dw, dscl, drecvX, dtok, drids, drw, drscl, dcnt, dmap, dscratch,
                             scratchB, stream));
    CHECK_EPDC(epdc_combine(&cfg, T, dy, dids, dw, dmap, dout, EPDC_BF16, stream));
    CHECK_EPDC(epdc_combine(&cfg, T, dy, dids, dw, dmap, dout32, EPDC_FP32, stream));
    CHECK_EPDC(epdc_combine_push(&cfg, T, dy, drids, drw, dcnt, dland, dscale, stream));
    CHECK_EPDC(epdc_combine_reduce(&cfg, T, dland, dscale, dcnt, dmap, dout2, EPDC_BF16, stream));
    CHECK_HIP(hipStreamSynchronize(stream));

    /* the same on the oracle, outputs pre-filled with the same sentinels */
    uint16_t *orecvX = malloc(nWin * rowB), *oout = malloc(T * rowB), *oout2 = malloc(T * rowB);
    uint16_t *oland = malloc((size_t)landRows * rowB);
    int32_t *otok = malloc(sizeof(int32_t) * nWin), *orids = malloc(sizeof(int32_t) * nWin * K);
    int32_t *ocnt = malloc(sizeof(int32_t) * W), *omap = malloc(sizeof(int32_t) * T * K);
    float *orw = malloc(sizeof(float) * nWin * K), *oscale = malloc(sizeof(float) * landRows);
    float *acc = malloc(sizeof(float) * H), *orscl = malloc(sizeof(float) * nWin * S);
    float *oout32 = malloc(sizeof(float) * T * H);
    memset(orscl, 0x55, sizeof(float) * nWin * S);
    memset(orecvX, 0xAD, nWin * rowB);
    memset(otok, 0x11, sizeof(int32_t) * nWin);
    memset(orids, 0x22, sizeof(int32_t) * nWin * K);
    memset(orw, 0x33, sizeof(float) * nWin * K);
    memset(oland, 0xA5, (size_t)landRows * rowB);
    memset(oscale, 0x44, sizeof(float) * landRows);
    if (oracle_dispatch(W, H, M, EPR, K, 1, T, 2, S, x, ids, wts, scl, orecvX, otok, orids, orw, orscl, ocnt,
                        omap) ||
        oracle_combine(W, H, M, EPR, K, 1, T, 0, 0, y, ids, wts, omap, NULL, T, acc, oout) ||
        oracle_combine(W, H, M, EPR, K, 1, T, 0, 1, y, ids, wts, omap, NULL, T, acc, oout32) ||
        oracle_combine_push(W, H, M, EPR, K, 1, T, 0, y, orids, orw, ocnt, oland, oscale) ||
        oracle_combine_reduce(W, H, M, EPR, K, 1, T, 0, 0, oland, oscale, ocnt, omap, NULL, T, acc, oout2)) {
        fprintf(stderr, "the oracle rejected the problem\n");
        return 1;
    }

    /* compare every output buffer */
    size_t gB = nWin * rowB > (size_t)landRows * rowB ? nWin * rowB : (size_t)landRows * rowB;
    if (gB < (size_t)T * H * 4) gB = (size_t)T * H * 4;
    void *g = malloc(gB);
    int ok = 1;
#define CMP(dev, host, bytes, name)                                      \
    CHECK_HIP(hipMemcpy(g, dev, bytes, hipMemcpyDeviceToHost));          \
    ok &= same(name, g, host, bytes);
    CMP(dcnt, ocnt, sizeof(int32_t) * W, "recvCount")
    CMP(dmap, omap, sizeof(int32_t) * T * K, "sendMap")
    CMP(drecvX, orecvX, nWin * rowB, "recvX")
    CMP(dtok, otok, sizeof(int32_t) * nWin, "recvTokIdx")
    CMP(drids, orids, sizeof(int32_t) * nWin * K, "recvExpertIds")
    CMP(drw, orw, sizeof(float) * nWin * K, "recvWeights")
    CMP(drscl, orscl, sizeof(float) * nWin * S, "recvScales")
    CMP(dout, oout, T * rowB, "combine out")
    CMP(dout32, oout32, sizeof(float) * T * H, "combine fp32 out")
    CMP(dland, oland, (size_t)landRows * rowB, "landing")
    CMP(dscale, oscale, sizeof(float) * landRows, "landScale")
    CMP(dout2, oout2, T * rowB, "reduce out")
    if (!ok) return 1;
    int32_t U = 0;
    for (int p = 0; p < W; ++p) U += ocnt[p];
    printf("c abi ok: T=%d U=%d landing rows %d\n", T, U, landRows);
    return 0;
}
