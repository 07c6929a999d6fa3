/*
 * CPU oracle for one source rank's share of MoE expert-parallel dispatch and
 * combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
 * link or execute this file or the library built from it: only tests/,
 * __graft_entry__.smoke() and bench.py's cpu_baseline leg do.  It shares no
 * code, header, table or helper with the HIP library; the two meet only in
 * the seeded input generator (tests/workloads.py).
 *
 * Plain, sequential, single-threaded C.  Build with -O2 -ffp-contract=off so
 * that the only fused multiply-add is the explicit fmaf() below.
 *
 * Notation (names as in the pages' EpCfg, MORI JIT v2 design doc, §3.2):
 *   W  = worldSize           Epr = numExpertPerRank    E = W*Epr
 *   K  = numExpertPerToken   H   = hiddenDim (elements per row)
 *   M  = maxTokPerRank       T   = numTokens (0 <= T <= M)
 * Row element types (the pages' EpDType, MORI JIT v2 design doc, §3.7):
 * dispatch moves rows of H elements of 2 (bf16), 4 (fp32) or 1 byte (fp8,
 * and fp4x2 where H counts bytes); combine reduces bf16 or fp32 rows and
 * writes bf16 or fp32 rows (§5: the combine's output is bf16 or fp32).
 * bf16 values travel as their 16-bit patterns (uint16_t).
 *   S  = scaleDim: fp32 quantisation scales per token that the dispatch
 *        forwards with the token (0 = none; MORI JIT v2 §4 and §5, the
 *        dispatch's `scales` argument and the `out_scales` region that exists
 *        only when scale_dim > 0).
 *
 * The scatter (push) combine at the end of this file is a second form of
 * combine: the rows go to packed landing rows first, then a reduction.
 *
 * Parity pins (see tests/test_oracle_pins.py): brute force on tiny inputs,
 * the closed-form expected count of unique (token, PE) pairs, the two
 * statistics the pages print (about 1374 dropped-slot null entries at
 * ct=512/topk=6/EP4; a 311 MB combine staging copy at EP8/4096 tokens/h7168),
 * structural invariants, identity-expert special cases and an fp64
 * recomputation within the fp32 summation error bound.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 -> fp32 is exact: the bf16 pattern is the upper half of the fp32. */
static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even (the IEEE default rounding
 * applied at bf16 precision).  NaN stays a quiet NaN of the same sign. */
static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* Destination PE of one expert id, or -1 for an id outside [0, E).
 * Experts are laid out in contiguous blocks of numExpertPerRank per PE; the
 * kernels on the MORI JIT v2 page (§8) divide by numExpertPerRank for this. */
static int32_t dest_pe(int32_t e, int32_t W, int32_t Epr) {
    if (e < 0 || (int64_t)e >= (int64_t)W * Epr) return -1;
    return e / Epr;
}

/*
 * DISPATCH: COUNT + SCAN + FINALIZE, done as one sequential pass.
 *
 * mori PR #599 "Perf/ep disp 1250 ship" (items "ballot dedup" and "cached
 * destPe/keep + deferred null write") describes the dispatch in two phases:
 * COUNT finds each slot's destination PE and drops the slots of a token that
 * hit a PE already taken by that token, so a token goes to each PE once; the
 * dropped slots each receive a 4-byte "null" entry, written in FINALIZE
 * together with the payload rows and the per-token metadata (three fields,
 * the "perTokM" tokCap note of the same PR).  Dispatch only moves bytes
 * (MORI JIT v2 §3.7), so rows and metadata are bitwise copies.
 *
 * Readings of what the pages leave open:
 *   - the lowest slot index of a token keeps a PE, later slots drop;
 *   - rows of each destination window are in ascending token order;
 *   - window stride maxTokPerRank rows, flat index p*M + r, null = -1;
 *   - per received row: source token index, the token's K expert ids and
 *     its K weights (weights only when useWeights);
 *   - with S > 0, also the token's S scales: a fourth metadata field that
 *     travels with the row (the mori PR #599 page, in the merge notes of the
 *     branch that transports scales, keeps a per-token scale row beside the
 *     other metadata fields; MORI JIT v2 §9 names forwarding of per-token
 *     scales as a FlyDSL-backend feature).  Like the others it is copied
 *     bitwise;
 *   - ids outside [0, E) are dropped slots (null entry, no row);
 *   - recvCount is stored, not accumulated (mori PR #599 follow-up commits:
 *     the dispatch stores the received count so callers need no reset).
 *
 * Rows r >= recvCount[p] of every window are left untouched.  Rows are
 * elemBytes * H bytes (the element type does not matter to a copy).
 * Returns 0, or -1 on a bad size.
 */
int oracle_dispatch(int32_t W, int32_t H, int32_t M, int32_t Epr, int32_t K,
                    int32_t useWeights, int32_t T, int32_t elemBytes, int32_t S,
                    const void *x, const int32_t *expertIds, const float *weights,
                    const float *scales, void *recvX, int32_t *recvTokIdx,
                    int32_t *recvExpertIds, float *recvWeights, float *recvScales,
                    int32_t *recvCount, int32_t *sendMap) {
    if (W <= 0 || H <= 0 || M <= 0 || Epr <= 0 || K <= 0 || T < 0 || T > M || S < 0) return -1;
    if (elemBytes != 1 && elemBytes != 2 && elemBytes != 4) return -1;
    const int64_t rowBytes = (int64_t)H * elemBytes;
    const unsigned char *xb = (const unsigned char *)x;
    unsigned char *rb = (unsigned char *)recvX;
    for (int32_t p = 0; p < W; ++p) recvCount[p] = 0;

    for (int32_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int32_t e = expertIds[(int64_t)t * K + k];
            int32_t p = dest_pe(e, W, Epr);
            int keep = (p >= 0);
            /* dedup: a PE already reached by an earlier slot of t drops k */
            for (int32_t j = 0; keep && j < k; ++j)
                if (dest_pe(expertIds[(int64_t)t * K + j], W, Epr) == p) keep = 0;
            if (!keep) {
                sendMap[(int64_t)t * K + k] = -1; /* the null entry */
                continue;
            }
            int32_t r = recvCount[p]++;
            int64_t row = (int64_t)p * M + r;
            memcpy(rb + row * rowBytes, xb + (int64_t)t * rowBytes, (size_t)rowBytes);
            recvTokIdx[row] = t;
            memcpy(recvExpertIds + row * K, expertIds + (int64_t)t * K, (size_t)K * sizeof(int32_t));
            if (useWeights)
                memcpy(recvWeights + row * K, weights + (int64_t)t * K, (size_t)K * sizeof(float));
            if (S > 0)
                memcpy(recvScales + row * S, scales + (int64_t)t * S, (size_t)S * sizeof(float));
            sendMap[(int64_t)t * K + k] = (int32_t)row;
        }
    }
    return 0;
}

/*
 * COMBINE for one token: gather the rows this token's PEs returned and
 * reduce them (MORI JIT v2 §5 and §9: the HIP backend's combine is a gather,
 * PULL/QUAD, that reduces in place of a scatter; §3.7: combine sums, so it
 * needs an arithmetic type).
 *
 * Readings:
 *   - the PEs are visited in first-appearance slot order (the kept slots of
 *     sendMap in ascending k);
 *   - the scale of PE p is the fp32 sum, in slot order starting from +0, of
 *     the weights of every slot of t whose expert lives on p (valid ids
 *     only); with useWeights == 0 it is 1;
 *   - accumulation in fp32 from +0 with one fused multiply-add per PE;
 *   - the returned rows are bf16 or fp32 (inFp32), and so is the output
 *     (outFp32), chosen independently (MORI JIT v2 §5: the combine reduces
 *     bf16 or fp32 rows and outputs bf16 or fp32; byte types cannot be
 *     summed, §3.7): a bf16 output is the accumulator rounded to bf16,
 *     nearest-even, an fp32 output is the accumulator itself;
 *   - a token with no kept slot gives a +0 row.
 */
/* acc[h] = fmaf(s, row[h], acc[h]) over one returned row (bf16 bits or fp32). */
static void fma_row(float *acc, float s, const void *row, int32_t H, int32_t fp32) {
    if (fp32) {
        const float *src = (const float *)row;
        for (int32_t h = 0; h < H; ++h) acc[h] = fmaf(s, src[h], acc[h]);
    } else {
        const uint16_t *src = (const uint16_t *)row;
        for (int32_t h = 0; h < H; ++h) acc[h] = fmaf(s, bf16_to_f32(src[h]), acc[h]);
    }
}

/* The output row: bf16 nearest-even, or the fp32 accumulator itself. */
static void store_row(void *outRow, const float *acc, int32_t H, int32_t fp32) {
    if (fp32) {
        memcpy(outRow, acc, (size_t)H * sizeof(float));
    } else {
        uint16_t *o = (uint16_t *)outRow;
        for (int32_t h = 0; h < H; ++h) o[h] = f32_to_bf16_rne(acc[h]);
    }
}

static void combine_token(int32_t W, int32_t H, int32_t M, int32_t Epr, int32_t K,
                          int32_t useWeights, int32_t inFp32, int32_t outFp32, int32_t t,
                          const void *y, const int32_t *expertIds, const float *weights,
                          const int32_t *sendMap, float *acc, void *outRow) {
    for (int32_t h = 0; h < H; ++h) acc[h] = 0.0f;
    for (int32_t k0 = 0; k0 < K; ++k0) {
        int32_t flat = sendMap[(int64_t)t * K + k0];
        if (flat < 0) continue;
        int32_t p = flat / M;
        int32_t r = flat % M;
        float s = 1.0f;
        if (useWeights) {
            s = 0.0f;
            for (int32_t k = k0; k < K; ++k)
                if (dest_pe(expertIds[(int64_t)t * K + k], W, Epr) == p)
                    s = s + weights[(int64_t)t * K + k];
        }
        const int64_t row = (int64_t)p * M + r;
        fma_row(acc, s, (const unsigned char *)y + row * H * (inFp32 ? 4 : 2), H, inFp32);
    }
    store_row(outRow, acc, H, outFp32);
}

/*
 * COMBINE over tokens, of bf16 rows (inFp32 == 0) or fp32 rows (inFp32 ==
 * 1) into bf16 (outFp32 == 0) or fp32 (outFp32 == 1) output rows.
 * With tokens == NULL every token t in [0, T) is combined into out[t][:].  Otherwise out[i][:] receives token tokens[i]
 * for i in [0, nList): the per-token form used to check sampled outputs of
 * large runs.  acc is caller scratch of H floats.
 * Returns 0, or -1 on a bad size or token index.
 */
int oracle_combine(int32_t W, int32_t H, int32_t M, int32_t Epr, int32_t K,
                   int32_t useWeights, int32_t T, int32_t inFp32, int32_t outFp32,
                   const void *y, const int32_t *expertIds, const float *weights,
                   const int32_t *sendMap, const int32_t *tokens, int32_t nList,
                   float *acc, void *out) {
    if (W <= 0 || H <= 0 || M <= 0 || Epr <= 0 || K <= 0 || T < 0 || T > M) return -1;
    if ((inFp32 != 0 && inFp32 != 1) || (outFp32 != 0 && outFp32 != 1)) return -1;
    const int64_t outRowBytes = (int64_t)H * (outFp32 ? 4 : 2);
    int32_t n = tokens ? nList : T;
    for (int32_t i = 0; i < n; ++i) {
        int32_t t = tokens ? tokens[i] : i;
        if (t < 0 || t >= T) return -1;
        combine_token(W, H, M, Epr, K, useWeights, inFp32, outFp32, t, y, expertIds, weights, sendMap,
                      acc, (unsigned char *)out + (int64_t)i * outRowBytes);
    }
    return 0;
}

/*
 * SCATTER (PUSH) COMBINE: the same reduction as oracle_combine, in two halves.
 *
 * MORI JIT v2 design doc, §5 and §9: the FlyDSL backend also has a scatter
 * combine, which the HIP backend refuses.  The aiter MegaMoE commits on the
 * mori PR #599 page (Oct 27, 2026) size it: the dispatch hands the push
 * combine a landing offset per destination, and the landing buffer holds
 * one row per (token, destination PE), max_tokens * min(world_size, topk)
 * rows.  A later page (mori PR #817) says the scatter combine's last stage
 * loads its rows with the non-temporal hint, i.e. streams the landing rows.
 *
 * Readings:
 *   - PUSH is what each destination PE p does with the rows it returns to
 *     this source: row r of window p (r < recvCount[p]) lands at landing row
 *     landOff[p] + r, landOff being the exclusive prefix sum of recvCount in
 *     PE order (the per-destination offsets the dispatch hands over).  The
 *     landing rows are packed: U = sum of recvCount rows, at most
 *     T * min(W, K) since a token reaches at most min(W, K) PEs;
 *   - with useWeights, the destination forwards one fp32 scale per landed
 *     row, computed from the metadata the dispatch delivered with that row
 *     (recvExpertIds, recvWeights): the sum, in slot order from +0, of the
 *     token's weights whose valid expert lives on p -- the gather combine's
 *     scale for that PE;
 *   - REDUCE is what the source does: for token t, its kept slots (sendMap
 *     >= 0) in ascending order give (p, r) and so the landing row; from +0,
 *     acc = fmaf(scale, row, acc) in fp32 (scale 1 without useWeights),
 *     then a bf16 (nearest-even) or fp32 output row, as in oracle_combine.
 *   So push then reduce gives oracle_combine's bits.
 */

/* Rows r >= recvCount[p] are not pushed; landing rows >= U and their scales
 * are left untouched, and landScale is not written without useWeights.
 * Returns 0, or -1 on a bad size, a count outside [0, M] or more landed rows
 * than T * min(W, K). */
int oracle_combine_push(int32_t W, int32_t H, int32_t M, int32_t Epr, int32_t K,
                        int32_t useWeights, int32_t T, int32_t fp32,
                        const void *y, const int32_t *recvExpertIds, const float *recvWeights,
                        const int32_t *recvCount, void *landing, float *landScale) {
    if (W <= 0 || H <= 0 || M <= 0 || Epr <= 0 || K <= 0 || T < 0 || T > M) return -1;
    if (fp32 != 0 && fp32 != 1) return -1;
    const int64_t rowBytes = (int64_t)H * (fp32 ? 4 : 2);
    const int64_t capacity = (int64_t)T * (W < K ? W : K);
    const unsigned char *yb = (const unsigned char *)y;
    unsigned char *lb = (unsigned char *)landing;
    int64_t landOff = 0; /* rows landed by PEs 0..p-1 */
    for (int32_t p = 0; p < W; ++p) {
        const int32_t n = recvCount[p];
        if (n < 0 || n > M) return -1;
        for (int32_t r = 0; r < n; ++r) {
            const int64_t src = (int64_t)p * M + r; /* window row, as in recvX */
            const int64_t L = landOff + r;
            if (L >= capacity) return -1;
            memcpy(lb + L * rowBytes, yb + src * rowBytes, (size_t)rowBytes);
            if (useWeights) {
                float s = 0.0f;
                for (int32_t k = 0; k < K; ++k)
                    if (dest_pe(recvExpertIds[src * K + k], W, Epr) == p)
                        s = s + recvWeights[src * K + k];
                landScale[L] = s;
            }
        }
        landOff += n;
    }
    return 0;
}

/* REDUCE over tokens; tokens / nList / acc / out as in oracle_combine.
 * Returns 0, or -1 on a bad size, count or token index, or a kept slot whose
 * landing row is outside [0, U). */
int oracle_combine_reduce(int32_t W, int32_t H, int32_t M, int32_t Epr, int32_t K,
                          int32_t useWeights, int32_t T, int32_t inFp32, int32_t outFp32,
                          const void *landing, const float *landScale, const int32_t *recvCount,
                          const int32_t *sendMap, const int32_t *tokens, int32_t nList,
                          float *acc, void *out) {
    if (W <= 0 || H <= 0 || M <= 0 || Epr <= 0 || K <= 0 || T < 0 || T > M) return -1;
    if ((inFp32 != 0 && inFp32 != 1) || (outFp32 != 0 && outFp32 != 1)) return -1;
    (void)Epr;
    const int64_t rowBytes = (int64_t)H * (inFp32 ? 4 : 2);
    const int64_t outRowBytes = (int64_t)H * (outFp32 ? 4 : 2);
    int64_t *landOff = (int64_t *)malloc(sizeof(int64_t) * (size_t)(W + 1));
    if (!landOff) return -1;
    landOff[0] = 0;
    for (int32_t p = 0; p < W; ++p) {
        if (recvCount[p] < 0 || recvCount[p] > M) { free(landOff); return -1; }
        landOff[p + 1] = landOff[p] + recvCount[p];
    }
    const unsigned char *lb = (const unsigned char *)landing;
    int32_t n = tokens ? nList : T;
    int rc = 0;
    for (int32_t i = 0; i < n && rc == 0; ++i) {
        int32_t t = tokens ? tokens[i] : i;
        if (t < 0 || t >= T) { rc = -1; break; }
        memset(acc, 0, (size_t)H * sizeof(float)); /* +0.0f */
        for (int32_t k0 = 0; k0 < K; ++k0) {
            int32_t flat = sendMap[(int64_t)t * K + k0];
            if (flat < 0) continue;
            int32_t p = flat / M;
            int32_t r = flat % M;
            if (p >= W || landOff[p] + r >= landOff[W]) { rc = -1; break; }
            int64_t L = landOff[p] + r;
            float s = useWeights ? landScale[L] : 1.0f;
            fma_row(acc, s, lb + L * rowBytes, H, inFp32);
        }
        store_row((unsigned char *)out + (int64_t)i * outRowBytes, acc, H, outFp32);
    }
    free(landOff);
    return rc;
}
