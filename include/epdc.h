/*
 * epdc.h -- C ABI of libepdc.so: one source rank's share of MoE
 * expert-parallel token dispatch and combine on one MI355X (gfx950).
 *
 * Operations (definitions from the pages):
 *   dispatch  COUNT -> SCAN -> FINALIZE.  mori PR #599 "Perf/ep disp 1250
 *             ship", items "ballot dedup" and "cached destPe/keep + deferred
 *             null write": each (token, top-k slot) maps to a destination PE;
 *             a token reaches each PE at most once; the rows and per-token
 *             metadata are written into per-PE receive windows and every
 *             dropped slot gets a 4-byte null entry.  Dispatch only moves bytes
 *             (MORI JIT v2 design doc, §3.7).
 *   combine   MORI JIT v2 design doc, §5 and §9: a gather combine -- each token
 *             pulls the rows its PEs returned and reduces them.
 *   scatter combine (push + reduce)  MORI JIT v2 design doc, §5 and §9 (the
 *             FlyDSL backend's scatter combine) with the landing rows sized
 *             in the aiter MegaMoE commits on the mori PR #599 page: each
 *             destination pushes its returned rows into per-(token, PE)
 *             landing rows at offsets the dispatch hands over, then the
 *             source reduces them.  Same result as the gather combine.
 *
 * Argument names follow EpCfg (MORI JIT v2 design doc, §3.2).  The geometry
 * fields of EpCfg (blockNum, warpPerBlock, waveSize) are not part of the ABI:
 * the library picks launch geometry itself.
 *
 * Conventions for every entry point:
 *   - Every pointer named "device" is device memory owned by the caller; the
 *     library allocates nothing, copies nothing to the host and never
 *     synchronises.  Calls are asynchronous on `stream`, so they can be
 *     captured into a HIP graph.  `stream` is a hipStream_t passed as void *
 *     (NULL is the default stream): the header then compiles without the HIP
 *     headers, and a hipStream_t converts to it implicitly.
 *   - All checks run on the host before any launch.  On failure a negative
 *     EPDC_ERR_* code is returned, nothing is launched, and epdc_last_error()
 *     describes the failure.  No entry point throws (MORI JIT v2 design doc,
 *     §6: every C entry point is noexcept and reports through a last-error
 *     string).
 *   - Index layout: T = numTokens, K = numExpertPerToken, W = worldSize,
 *     M = maxTokPerRank, H = hiddenDim, Epr = numExpertPerRank, E = W*Epr.
 *     All arrays are dense row-major with exactly these extents.
 */
#ifndef EPDC_H
#define EPDC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Row element types, numbered as the pages' EpDType (MORI JIT v2 design doc,
 * §3.7 and §7: the enum values must match the binding's table).  Dispatch
 * only moves rows, so it takes all four: bf16 (2 bytes per element), fp32 (4)
 * and the one-byte fp8 and fp4x2 (for fp4x2 one element is a byte holding
 * two e2m1 values, so hiddenDim counts bytes).  Combine sums rows, so it
 * takes only EPDC_BF16 and EPDC_FP32, for its returned rows and, chosen
 * apart, for its output (§5: the combine outputs bf16 or fp32).  A
 * narrow-wire pair (fp8 or fp4x2 dispatch, bf16 combine) is two calls with
 * two cfgs.  The quantisation scales of a narrow-wire row travel beside it as
 * per-token metadata (scaleDim, below). */
typedef enum {
    EPDC_BF16 = 0,
    EPDC_FP32 = 1,
    EPDC_FP8 = 2,
    EPDC_FP4X2 = 3
} epdc_dtype;

enum {
    EPDC_OK = 0,
    EPDC_ERR_INVALID_ARG = -1, /* a cfg field out of range, numTokens < 0, K > E, W*M too large */
    EPDC_ERR_UNSUPPORTED = -2, /* dtype not allowed on this call (see above), useWeights not 0/1 */
    EPDC_ERR_CAPACITY = -3,    /* numTokens > maxTokPerRank                                    */
    EPDC_ERR_ALIGN = -4,       /* row bytes not a multiple of 16, or a misaligned pointer      */
    EPDC_ERR_NULLPTR = -5,     /* a required pointer (or cfg) is NULL                          */
    EPDC_ERR_SCRATCH = -6,     /* scratchBytes below epdc_dispatch_scratch_bytes(cfg)          */
    EPDC_ERR_HIP = -7          /* the HIP runtime reported an error (no device, launch failed) */
};

/* Shape and options of one dispatch/combine pair (EpCfg field names).
 *   worldSize          W, 1..64 (one bit per PE in a 64-lane wavefront)
 *   hiddenDim          H elements per token row; the row, H times the element
 *                      size of dtype, must be a multiple of 16 bytes
 *   maxTokPerRank      M >= 1: capacity of x and of each receive window, in rows;
 *                      W*M must not exceed 2^31-1 (flat indices are int32)
 *   numExpertPerRank   Epr >= 1; expert e lives on PE e / Epr
 *   numExpertPerToken  K, 1..64, K <= E
 *   dtype              row element type (epdc_dtype; see above for each call)
 *   useWeights         1: dispatch copies the weights, combine applies them; 0: ignored
 *   scaleDim           S, 0..EPDC_MAX_SCALE_DIM: fp32 scales per token that the
 *                      dispatch forwards with each of the token's rows (0: none).
 *                      MORI JIT v2 design doc, §4 (the dispatch takes a `scales`
 *                      argument) and §5 (an `out_scales` region exists only when
 *                      scale_dim > 0); the mori PR #599 page's merge notes carry
 *                      the per-token scale row as a fourth metadata field beside
 *                      token index, expert ids and weights.  Combine, push and
 *                      reduce ignore it. */
typedef struct epdc_cfg {
    int32_t worldSize;
    int32_t hiddenDim;
    int32_t maxTokPerRank;
    int32_t numExpertPerRank;
    int32_t numExpertPerToken;
    int32_t dtype;
    int32_t useWeights;
    int32_t scaleDim;
} epdc_cfg;

/* Largest scaleDim: one fp32 scale per 16 elements of a 16384-wide row. */
#define EPDC_MAX_SCALE_DIM 1024

/* Bytes of device scratch epdc_dispatch needs for this cfg: a 4224-byte header
 * (completion counters and a status word) plus two 32-bit words per (64-token
 * tile, PE) of maxTokPerRank tokens -- a few KB.  Returns 0 if cfg is invalid.
 *
 * The pages' dispatch reserves rows with a cross-device fetch_add; this one
 * instead computes every row in ascending token order (so windows are stable
 * and the result deterministic) from per-tile counts that the kernel's blocks
 * exchange through this buffer: one block per 64-token tile publishes the
 * tile's count per PE and the blocks of later tiles sum them.
 *
 * The scratch must be zero-filled once before its first use (e.g. one
 * hipMemset at allocation).  Every dispatch leaves it zeroed again, so it
 * needs no reset between calls or graph replays -- except the status word.
 * One scratch buffer serves one dispatch at a time: calls that may run
 * concurrently need separate buffers. */
size_t epdc_dispatch_scratch_bytes(const epdc_cfg *cfg);

/* Status word of a dispatch scratch buffer: the 32-bit word at byte offset
 * 4 * EPDC_STATUS_WORD.  A dispatch sets it nonzero -- and never clears it --
 * when that call's outputs are invalid:
 *   EPDC_STATUS_WAIT_TIMEOUT   one of its bounded in-kernel waits gave up
 *                              (instead of hanging the GPU);
 *   EPDC_STATUS_ROW_OUTSIDE    a computed row fell outside its window (only
 *                              possible when the scratch was not zero at
 *                              launch; such rows are skipped and nothing is
 *                              written outside the windows).
 * It stays zero in correct operation.  Read it after the caller's own
 * synchronisation with the stream (one 4-byte device-to-host copy); a caller
 * that sees it nonzero discards the outputs and zeroes the scratch again. */
#define EPDC_STATUS_WORD 2
#define EPDC_STATUS_WAIT_TIMEOUT 1
#define EPDC_STATUS_ROW_OUTSIDE 2

/*
 * Dispatch numTokens tokens (0 <= numTokens <= maxTokPerRank).
 *
 * Inputs (device, read only):
 *   x            [T][H] token rows of cfg->dtype, 16-byte aligned
 *   expertIds    [T][K] int32 top-k expert ids; an id outside [0, E) marks a
 *                dropped slot (ids are not range-checked on the host)
 *   weights      [T][K] fp32; may be NULL iff useWeights == 0
 *   scales       [T][S] fp32 per-token scales (S = scaleDim); may be NULL iff S == 0
 * Outputs (device, written):
 *   recvX          [W][M][H] of cfg->dtype, 16-byte aligned: recvX[p][r] is a bitwise copy
 *                  of the r-th token (ascending token order) that reaches PE p
 *   recvTokIdx     [W][M] int32: that token's index
 *   recvExpertIds  [W][M][K] int32: that token's K expert ids
 *   recvWeights    [W][M][K] fp32: that token's K weights; NULL iff useWeights == 0
 *   recvScales     [W][M][S] fp32: that token's S scales, bitwise; NULL iff S == 0
 *   recvCount      [W] int32: rows written per PE -- stored, not accumulated
 *                  (mori PR #599 follow-up commits: the dispatch stores the
 *                  received count, so callers need no reset kernel)
 *   sendMap        [T][K] int32: for the lowest slot k of token t on PE p,
 *                  p*M + r; for every other slot (duplicate PE or invalid
 *                  id) -1, the null entry
 *   Rows r >= recvCount[p] of every window are left untouched.
 * Scratch (device): at least epdc_dispatch_scratch_bytes(cfg) bytes, 16-byte
 *   aligned, zero-filled before its first use (see above).
 * With numTokens == 0 only recvCount is written (zeros); the token-sized
 * pointers may then be NULL.
 */
int epdc_dispatch(const epdc_cfg *cfg, int32_t numTokens,
                  const void *x, const int32_t *expertIds, const float *weights, const float *scales,
                  void *recvX, int32_t *recvTokIdx, int32_t *recvExpertIds,
                  float *recvWeights, float *recvScales, int32_t *recvCount, int32_t *sendMap,
                  void *scratch, size_t scratchBytes, void *stream);

/*
 * epdc_dispatch without a caller scratch buffer, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus scratch and
 * scratchBytes), same kernels and bit-identical outputs.  The scratch is the
 * library's own: a 1 MiB device array per GPU, held until the process ends,
 * zeroed by a small kernel on `stream` at the first call on that device and
 * left zeroed by every call.  It allocates nothing (no hipMalloc, no library
 * allocator) on any call.
 *
 * Limit: the scratch must hold 4224 + 8 * ceil(numTokens / 64) * W' bytes (W'
 * = worldSize rounded up to a power of two), i.e. up to 130,496 tokens at 64
 * PEs, 1,044,352 at 8; beyond that the call fails with EPDC_ERR_SCRATCH and
 * launches nothing.  Calls on one GPU share its array: calls that may run at
 * the same time on that GPU (on different streams, or from several threads)
 * race and give invalid outputs -- serialise them, or use epdc_dispatch with
 * a buffer per stream.  The array's status word is not exposed.
 */
int epdc_dispatch_noalloc(const epdc_cfg *cfg, int32_t numTokens,
                          const void *x, const int32_t *expertIds, const float *weights, const float *scales,
                          void *recvX, int32_t *recvTokIdx, int32_t *recvExpertIds,
                          float *recvWeights, float *recvScales, int32_t *recvCount, int32_t *sendMap,
                          void *stream);

/*
 * Combine numTokens tokens from the rows their PEs returned.
 *
 * cfg->dtype is EPDC_BF16 or EPDC_FP32: the type of y.  outDtype is
 * EPDC_BF16 or EPDC_FP32: the type of out (either with either).
 * Inputs (device, read only):
 *   y          [W][M][H] of cfg->dtype, 16-byte aligned: returned rows, indexed like recvX
 *   expertIds  [T][K] int32, the ids given to the matching dispatch; read only
 *              when useWeights == 1 (else may be NULL)
 *   weights    [T][K] fp32 or NULL iff useWeights == 0
 *   sendMap    [T][K] int32 as written by the matching dispatch
 * Output (device): out [T][H] of outDtype, 16-byte aligned.
 *
 * For token t, the PEs of its kept slots (sendMap >= 0) are visited in
 * ascending slot order.  PE p's scale is the fp32 sum, in slot order from +0,
 * of the weights of t's slots whose valid expert lives on p (1 when
 * useWeights == 0).  acc = fmaf(scale_p, y[p][r_p][h], acc) over those PEs
 * from acc = +0 in fp32; out[t][h] = bf16_rne(acc) for a bf16 output
 * (nearest, ties to even) and acc itself for an fp32 output.  A token with no
 * kept slot yields +0.  A sendMap entry outside [0, W*M) counts as a dropped
 * slot.  Results are deterministic and bit-identical run to run.
 */
int epdc_combine(const epdc_cfg *cfg, int32_t numTokens,
                 const void *y, const int32_t *expertIds, const float *weights,
                 const int32_t *sendMap, void *out, int32_t outDtype, void *stream);

/* Landing rows of the scatter combine for numTokens tokens: numTokens *
 * min(W, K), one per (token, PE) a token can reach.  -1 if cfg (with a
 * combine dtype) or numTokens is invalid. */
int32_t epdc_landing_rows(const epdc_cfg *cfg, int32_t numTokens);

/*
 * Scatter combine, push half: what the destination PEs do.  Every window's
 * returned rows move into packed landing rows, each with a forwarded scale.
 *
 * cfg->dtype is EPDC_BF16 or EPDC_FP32: the type of y and landing.
 * numTokens is the source's token count of the matching dispatch; it sizes
 * the landing buffer (R = epdc_landing_rows(cfg, numTokens) rows).
 * Inputs (device, read only):
 *   y              [W][M][H] returned rows, indexed like recvX, 16-byte aligned
 *   recvExpertIds  [W][M][K] int32 and
 *   recvWeights    [W][M][K] fp32, as the matching dispatch wrote them; both
 *                  are read only when useWeights == 1 (else may be NULL)
 *   recvCount      [W] int32 as the matching dispatch wrote it
 * Outputs (device):
 *   landing    [R][H] of cfg->dtype, 16-byte aligned: row r < recvCount[p] of
 *              window p lands at row landOff[p] + r, landOff[p] being the sum
 *              of recvCount[q] over q < p (each count taken in [0, M]);
 *              rows from the total count on, and rows that would fall at or
 *              past R, are not written
 *   landScale  [R] fp32, written only when useWeights == 1 (else may be
 *              NULL): for each landed row, the fp32 sum, in slot order from
 *              +0, of its token's weights (recvWeights) whose valid expert
 *              (recvExpertIds) lives on p -- the scale the gather combine
 *              gives PE p for that token
 * A recvCount from the matching dispatch never exceeds R rows in total.
 */
int epdc_combine_push(const epdc_cfg *cfg, int32_t numTokens,
                      const void *y, const int32_t *recvExpertIds, const float *recvWeights,
                      const int32_t *recvCount, void *landing, float *landScale, void *stream);

/*
 * Scatter combine, reduce half: what the source does with its landing rows.
 *
 * cfg->dtype is EPDC_BF16 or EPDC_FP32: the type of landing; outDtype
 * (EPDC_BF16 or EPDC_FP32) the type of out.
 * Inputs (device, read only):
 *   landing    [R][H], landScale [R] (NULL iff useWeights == 0): as written by
 *              epdc_combine_push with the same cfg, numTokens and recvCount
 *   recvCount  [W] int32 and sendMap [T][K] int32 from the matching dispatch
 * Output (device): out [T][H] of outDtype, 16-byte aligned.
 *
 * For token t, the kept slots (sendMap >= 0) in ascending order give (p, r)
 * = (sendMap / M, sendMap % M) and so landing row landOff[p] + r;
 * acc = fmaf(scale, landing[row][h], acc) from +0 in fp32, scale = landScale
 * of that row (1 when useWeights == 0); out as in epdc_combine.  This is the
 * gather combine's order and arithmetic, so out is bit-identical to
 * epdc_combine's on the same rows.  A slot whose row lies outside the landed
 * rows (or outside [0, W*M)) counts as dropped.
 */
int epdc_combine_reduce(const epdc_cfg *cfg, int32_t numTokens,
                        const void *landing, const float *landScale, const int32_t *recvCount,
                        const int32_t *sendMap, void *out, int32_t outDtype, void *stream);

/* Message for the last failing call on this thread ("" if none).  The
 * pointer stays valid until the next epdc_* call on the same thread.  MORI
 * JIT v2 design doc, §6: the C entry points report failures through a
 * thread's last-error string rather than exceptions. */
const char *epdc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EPDC_H */
