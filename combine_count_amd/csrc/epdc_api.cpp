// Host side of the C ABI declared in include/epdc.h: argument checks, error
// reporting and the launch.  Every check runs before anything is enqueued;
// no entry point lets an exception escape (MORI JIT v2 design doc, §6: all
// C entry points are noexcept and report through a last-error string).
#include "../../include/epdc.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "epdc_internal.h"

static_assert(EPDC_STATUS_WORD == epdc::kScratchError, "status word offset");
static_assert(EPDC_STATUS_WAIT_TIMEOUT == epdc::kStatusWaitTimeout, "status value");
static_assert(EPDC_STATUS_ROW_OUTSIDE == epdc::kStatusRowOutside, "status value");

namespace {

thread_local std::string g_lastError;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_lastError = buf;
    return code;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int32_t pow2_ceil(int32_t v) {
    int32_t r = 1;
    while (r < v) r <<= 1;
    return r;
}

int32_t log2_exact(int32_t v) {
    if (v <= 0 || (v & (v - 1))) return -1;
    int32_t s = 0;
    while ((1 << s) < v) ++s;
    return s;
}

// Bytes per element of a row.  Dispatch moves any EpDType (fp8 and fp4x2 are
// one byte each; for fp4x2 hiddenDim counts bytes); combine sums, so only
// the arithmetic types bf16 and fp32 (MORI JIT v2 design doc, §3.7 and §5).
// -1 if the dtype is not allowed on that leg.
int32_t elem_bytes(int32_t dtype, bool combine) {
    switch (dtype) {
        case EPDC_BF16: return 2;
        case EPDC_FP32: return 4;
        case EPDC_FP8:
        case EPDC_FP4X2: return combine ? -1 : 1;
        default: return -1;
    }
}

// Checks shared by both entry points (EpCfg validity: MORI JIT v2 design doc,
// §3.5 -- 16-byte token rows, topk and worldSize within one wavefront,
// receive capacity covering the worst case).
int check_cfg(const epdc_cfg *c, int32_t numTokens, bool combine) {
    if (!c) return fail(EPDC_ERR_NULLPTR, "cfg is NULL");
    if (c->worldSize < 1 || c->worldSize > 64)
        return fail(EPDC_ERR_INVALID_ARG, "worldSize %d outside [1, 64]", c->worldSize);
    if (c->numExpertPerToken < 1 || c->numExpertPerToken > 64)
        return fail(EPDC_ERR_INVALID_ARG, "numExpertPerToken %d outside [1, 64]", c->numExpertPerToken);
    if (c->numExpertPerRank < 1)
        return fail(EPDC_ERR_INVALID_ARG, "numExpertPerRank %d < 1", c->numExpertPerRank);
    const int64_t E = (int64_t)c->worldSize * c->numExpertPerRank;
    if (E > INT32_MAX) return fail(EPDC_ERR_INVALID_ARG, "worldSize*numExpertPerRank overflows int32");
    if (c->numExpertPerToken > E)
        return fail(EPDC_ERR_INVALID_ARG, "numExpertPerToken %d > number of experts %lld",
                    c->numExpertPerToken, (long long)E);
    if (c->hiddenDim < 1) return fail(EPDC_ERR_INVALID_ARG, "hiddenDim %d < 1", c->hiddenDim);
    if (c->maxTokPerRank < 1) return fail(EPDC_ERR_INVALID_ARG, "maxTokPerRank %d < 1", c->maxTokPerRank);
    if ((int64_t)c->worldSize * c->maxTokPerRank > INT32_MAX)
        return fail(EPDC_ERR_INVALID_ARG, "worldSize*maxTokPerRank overflows the int32 flat index");
    const int32_t eb = elem_bytes(c->dtype, combine);
    if (eb < 0)
        return combine ? fail(EPDC_ERR_UNSUPPORTED, "combine sums its rows: dtype %d is not EPDC_BF16 or EPDC_FP32",
                              c->dtype)
                       : fail(EPDC_ERR_UNSUPPORTED, "dtype %d is not an EPDC dtype (0..3)", c->dtype);
    if (c->useWeights != 0 && c->useWeights != 1)
        return fail(EPDC_ERR_UNSUPPORTED, "useWeights must be 0 or 1, got %d", c->useWeights);
    if (c->scaleDim < 0 || c->scaleDim > EPDC_MAX_SCALE_DIM)
        return fail(EPDC_ERR_INVALID_ARG, "scaleDim %d outside [0, %d]", c->scaleDim, EPDC_MAX_SCALE_DIM);
    if (((int64_t)c->hiddenDim * eb) % 16 != 0)
        return fail(EPDC_ERR_ALIGN, "row of hiddenDim*%d = %lld bytes is not a multiple of 16", eb,
                    (long long)c->hiddenDim * eb);
    if ((int64_t)c->hiddenDim * eb > INT32_MAX)
        return fail(EPDC_ERR_INVALID_ARG, "row of %lld bytes is too long", (long long)c->hiddenDim * eb);
    if (numTokens < 0) return fail(EPDC_ERR_INVALID_ARG, "numTokens %d < 0", numTokens);
    if (numTokens > c->maxTokPerRank)
        return fail(EPDC_ERR_CAPACITY, "numTokens %d > maxTokPerRank %d", numTokens, c->maxTokPerRank);
    return EPDC_OK;
}

size_t scratch_bytes(const epdc_cfg *c) {
    const int64_t nTiles = ((int64_t)c->maxTokPerRank + epdc::kTile - 1) / epdc::kTile;
    return (size_t)((epdc::kScratchHeaderWords + 2 * nTiles * pow2_ceil(c->worldSize)) * sizeof(uint32_t));
}

// Landing rows of the scatter combine: one per (token, PE), at most
// min(W, K) PEs per token.  numTokens <= M and W*M fits int32, so this does.
int32_t landing_rows(const epdc_cfg *c, int32_t numTokens) {
    const int32_t perToken = c->worldSize < c->numExpertPerToken ? c->worldSize : c->numExpertPerToken;
    return numTokens * perToken;
}

// Output type of a combine or reduce: bf16 or fp32 (MORI JIT v2 design doc,
// §5), independent of the rows' type.  -1 if it is neither.
int32_t out_elem_bytes(int32_t outDtype) {
    return outDtype == EPDC_BF16 ? 2 : outDtype == EPDC_FP32 ? 4 : -1;
}

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return EPDC_OK;
    return fail(EPDC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Checks of every dispatch argument but the scratch, and the kernel
// parameters (the scratch pointer left for the caller to set).
int dispatch_params(const epdc_cfg *cfg, int32_t numTokens, const void *x, const int32_t *expertIds,
                    const float *weights, const float *scales, void *recvX, int32_t *recvTokIdx,
                    int32_t *recvExpertIds, float *recvWeights, float *recvScales, int32_t *recvCount,
                    int32_t *sendMap, epdc::DispatchParams &P) {
    int rc = check_cfg(cfg, numTokens, false);
    if (rc != EPDC_OK) return rc;
    if (!recvCount) return fail(EPDC_ERR_NULLPTR, "recvCount is NULL");
    if (!aligned(recvCount, 4)) return fail(EPDC_ERR_ALIGN, "recvCount not 4-byte aligned");
    if (numTokens > 0) {
        if (!x || !expertIds || !recvX || !recvTokIdx || !recvExpertIds || !sendMap)
            return fail(EPDC_ERR_NULLPTR, "a required dispatch pointer is NULL");
        if (cfg->useWeights && (!weights || !recvWeights))
            return fail(EPDC_ERR_NULLPTR, "useWeights=1 needs weights and recvWeights");
        if (cfg->scaleDim > 0 && (!scales || !recvScales))
            return fail(EPDC_ERR_NULLPTR, "scaleDim > 0 needs scales and recvScales");
        if (cfg->scaleDim > 0 && (!aligned(scales, 4) || !aligned(recvScales, 4)))
            return fail(EPDC_ERR_ALIGN, "scales and recvScales must be 4-byte aligned");
        if (!aligned(x, 16) || !aligned(recvX, 16)) return fail(EPDC_ERR_ALIGN, "x and recvX must be 16-byte aligned");
        if (!aligned(expertIds, 4) || !aligned(recvTokIdx, 4) || !aligned(recvExpertIds, 4) ||
            !aligned(sendMap, 4) || (cfg->useWeights && (!aligned(weights, 4) || !aligned(recvWeights, 4))))
            return fail(EPDC_ERR_ALIGN, "int32/fp32 arrays must be 4-byte aligned");
    }
    P.W = cfg->worldSize;
    P.H = cfg->hiddenDim;
    P.M = cfg->maxTokPerRank;
    P.Epr = cfg->numExpertPerRank;
    P.K = cfg->numExpertPerToken;
    P.T = numTokens;
    P.useWeights = cfg->useWeights;
    P.S = cfg->scaleDim;
    P.Wp = pow2_ceil(cfg->worldSize);
    const epdc::DivMagic dm = epdc::div_magic((uint32_t)cfg->numExpertPerRank);
    P.eprMagic = dm.magic;
    P.eprSh1 = dm.sh1;
    P.eprSh2 = dm.sh2;
    P.rowBytes = cfg->hiddenDim * elem_bytes(cfg->dtype, false);
    P.nChunks = epdc::ceil_div(P.rowBytes, epdc::kChunkBytes);
    P.x = static_cast<const uint8_t *>(x);
    P.expertIds = expertIds;
    P.weights = cfg->useWeights ? weights : nullptr;
    P.scales = cfg->scaleDim > 0 ? scales : nullptr;
    P.recvX = static_cast<uint8_t *>(recvX);
    P.recvTokIdx = recvTokIdx;
    P.recvExpertIds = recvExpertIds;
    P.recvWeights = cfg->useWeights ? recvWeights : nullptr;
    P.recvScales = cfg->scaleDim > 0 ? recvScales : nullptr;
    P.recvCount = recvCount;
    P.sendMap = sendMap;
    return EPDC_OK;
}

}  // namespace

extern "C" {

size_t epdc_dispatch_scratch_bytes(const epdc_cfg *cfg) {
    try {
        if (check_cfg(cfg, 0, false) != EPDC_OK) return 0;
        return scratch_bytes(cfg);
    } catch (...) {
        return 0;
    }
}

int epdc_dispatch(const epdc_cfg *cfg, int32_t numTokens, const void *x, const int32_t *expertIds,
                  const float *weights, const float *scales, void *recvX, int32_t *recvTokIdx,
                  int32_t *recvExpertIds, float *recvWeights, float *recvScales, int32_t *recvCount,
                  int32_t *sendMap, void *scratch, size_t scratchBytes, void *stream) {
    try {
        g_lastError.clear();
        epdc::DispatchParams P{};
        int rc = dispatch_params(cfg, numTokens, x, expertIds, weights, scales, recvX, recvTokIdx, recvExpertIds,
                                 recvWeights, recvScales, recvCount, sendMap, P);
        if (rc != EPDC_OK) return rc;
        if (numTokens > 0) {
            if (!scratch) return fail(EPDC_ERR_NULLPTR, "scratch is NULL");
            if (!aligned(scratch, 16)) return fail(EPDC_ERR_ALIGN, "scratch must be 16-byte aligned");
            if (scratchBytes < scratch_bytes(cfg))
                return fail(EPDC_ERR_SCRATCH, "scratchBytes %zu < %zu required", scratchBytes,
                            scratch_bytes(cfg));
        }
        P.scratch = static_cast<uint32_t *>(scratch);
        return hip_status(epdc::launch_dispatch(P, static_cast<hipStream_t>(stream)), "dispatch launch");
    } catch (...) {
        return fail(EPDC_ERR_HIP, "unexpected C++ exception in epdc_dispatch");
    }
}

int epdc_dispatch_noalloc(const epdc_cfg *cfg, int32_t numTokens, const void *x, const int32_t *expertIds,
                          const float *weights, const float *scales, void *recvX, int32_t *recvTokIdx,
                          int32_t *recvExpertIds, float *recvWeights, float *recvScales, int32_t *recvCount,
                          int32_t *sendMap, void *stream) {
    try {
        g_lastError.clear();
        epdc::DispatchParams P{};
        int rc = dispatch_params(cfg, numTokens, x, expertIds, weights, scales, recvX, recvTokIdx, recvExpertIds,
                                 recvWeights, recvScales, recvCount, sendMap, P);
        if (rc != EPDC_OK) return rc;
        const int64_t words = epdc::dispatch_scratch_words(numTokens, cfg->worldSize);
        if (words > epdc::kStaticScratchWords)
            return fail(EPDC_ERR_SCRATCH,
                        "%d tokens to %d PEs need %lld bytes of scratch; the library's own holds %d "
                        "(use epdc_dispatch with a caller scratch buffer)",
                        numTokens, cfg->worldSize, (long long)words * 4, epdc::kStaticScratchWords * 4);
        uint32_t *dev = nullptr;
        rc = hip_status(epdc::static_scratch(&dev, static_cast<hipStream_t>(stream)), "library scratch");
        if (rc != EPDC_OK) return rc;
        P.scratch = dev;
        return hip_status(epdc::launch_dispatch(P, static_cast<hipStream_t>(stream)), "dispatch launch");
    } catch (...) {
        return fail(EPDC_ERR_HIP, "unexpected C++ exception in epdc_dispatch_noalloc");
    }
}

int epdc_combine(const epdc_cfg *cfg, int32_t numTokens, const void *y, const int32_t *expertIds,
                 const float *weights, const int32_t *sendMap, void *out, int32_t outDtype, void *stream) {
    try {
        g_lastError.clear();
        int rc = check_cfg(cfg, numTokens, true);
        if (rc != EPDC_OK) return rc;
        if (out_elem_bytes(outDtype) < 0)
            return fail(EPDC_ERR_UNSUPPORTED, "outDtype %d is not EPDC_BF16 or EPDC_FP32", outDtype);
        if (numTokens == 0) return EPDC_OK;
        if (!y || !sendMap || !out) return fail(EPDC_ERR_NULLPTR, "a required combine pointer is NULL");
        if (cfg->useWeights && (!weights || !expertIds))
            return fail(EPDC_ERR_NULLPTR, "useWeights=1 needs expertIds and weights");
        if (!aligned(y, 16) || !aligned(out, 16))
            return fail(EPDC_ERR_ALIGN, "y and out must be 16-byte aligned");
        if (!aligned(sendMap, 4) || (cfg->useWeights && (!aligned(weights, 4) || !aligned(expertIds, 4))))
            return fail(EPDC_ERR_ALIGN, "int32/fp32 arrays must be 4-byte aligned");
        epdc::CombineParams P{};
        P.W = cfg->worldSize;
        P.H = cfg->hiddenDim;
        P.M = cfg->maxTokPerRank;
        P.Epr = cfg->numExpertPerRank;
        P.K = cfg->numExpertPerToken;
        P.T = numTokens;
        P.useWeights = cfg->useWeights;
        P.eprShift = log2_exact(cfg->numExpertPerRank);
        P.rowBytes = cfg->hiddenDim * elem_bytes(cfg->dtype, true);
        P.outRowBytes = cfg->hiddenDim * out_elem_bytes(outDtype);
        P.nChunks = epdc::ceil_div(P.rowBytes, epdc::kChunkBytes);
        P.y = static_cast<const uint8_t *>(y);
        P.expertIds = cfg->useWeights ? expertIds : nullptr;
        P.weights = cfg->useWeights ? weights : nullptr;
        P.sendMap = sendMap;
        P.out = static_cast<uint8_t *>(out);
        return hip_status(epdc::launch_combine(P, cfg->dtype == EPDC_FP32, outDtype == EPDC_FP32, false,
                                               static_cast<hipStream_t>(stream)),
                          "combine launch");
    } catch (...) {
        return fail(EPDC_ERR_HIP, "unexpected C++ exception in epdc_combine");
    }
}

int32_t epdc_landing_rows(const epdc_cfg *cfg, int32_t numTokens) {
    try {
        if (check_cfg(cfg, numTokens, true) != EPDC_OK) return -1;
        return landing_rows(cfg, numTokens);
    } catch (...) {
        return -1;
    }
}

int epdc_combine_push(const epdc_cfg *cfg, int32_t numTokens, const void *y, const int32_t *recvExpertIds,
                      const float *recvWeights, const int32_t *recvCount, void *landing, float *landScale,
                      void *stream) {
    try {
        g_lastError.clear();
        int rc = check_cfg(cfg, numTokens, true);
        if (rc != EPDC_OK) return rc;
        if (numTokens == 0) return EPDC_OK;
        if (!y || !recvCount || !landing) return fail(EPDC_ERR_NULLPTR, "a required push pointer is NULL");
        if (cfg->useWeights && (!recvExpertIds || !recvWeights || !landScale))
            return fail(EPDC_ERR_NULLPTR, "useWeights=1 needs recvExpertIds, recvWeights and landScale");
        if (!aligned(y, 16) || !aligned(landing, 16))
            return fail(EPDC_ERR_ALIGN, "y and landing must be 16-byte aligned");
        if (!aligned(recvCount, 4) ||
            (cfg->useWeights && (!aligned(recvExpertIds, 4) || !aligned(recvWeights, 4) || !aligned(landScale, 4))))
            return fail(EPDC_ERR_ALIGN, "int32/fp32 arrays must be 4-byte aligned");
        epdc::PushParams P{};
        P.W = cfg->worldSize;
        P.M = cfg->maxTokPerRank;
        P.Epr = cfg->numExpertPerRank;
        P.K = cfg->numExpertPerToken;
        P.useWeights = cfg->useWeights;
        P.rowBytes = cfg->hiddenDim * elem_bytes(cfg->dtype, true);
        P.eprShift = log2_exact(cfg->numExpertPerRank);
        P.nChunks = epdc::ceil_div(P.rowBytes, epdc::kChunkBytes);
        P.landRows = landing_rows(cfg, numTokens);
        P.y = static_cast<const uint8_t *>(y);
        P.recvExpertIds = cfg->useWeights ? recvExpertIds : nullptr;
        P.recvWeights = cfg->useWeights ? recvWeights : nullptr;
        P.recvCount = recvCount;
        P.landing = static_cast<uint8_t *>(landing);
        P.landScale = cfg->useWeights ? landScale : nullptr;
        return hip_status(epdc::launch_combine_push(P, static_cast<hipStream_t>(stream)), "push launch");
    } catch (...) {
        return fail(EPDC_ERR_HIP, "unexpected C++ exception in epdc_combine_push");
    }
}

int epdc_combine_reduce(const epdc_cfg *cfg, int32_t numTokens, const void *landing, const float *landScale,
                        const int32_t *recvCount, const int32_t *sendMap, void *out, int32_t outDtype,
                        void *stream) {
    try {
        g_lastError.clear();
        int rc = check_cfg(cfg, numTokens, true);
        if (rc != EPDC_OK) return rc;
        if (out_elem_bytes(outDtype) < 0)
            return fail(EPDC_ERR_UNSUPPORTED, "outDtype %d is not EPDC_BF16 or EPDC_FP32", outDtype);
        if (numTokens == 0) return EPDC_OK;
        if (!landing || !recvCount || !sendMap || !out)
            return fail(EPDC_ERR_NULLPTR, "a required reduce pointer is NULL");
        if (cfg->useWeights && !landScale) return fail(EPDC_ERR_NULLPTR, "useWeights=1 needs landScale");
        if (!aligned(landing, 16) || !aligned(out, 16))
            return fail(EPDC_ERR_ALIGN, "landing and out must be 16-byte aligned");
        if (!aligned(recvCount, 4) || !aligned(sendMap, 4) || (cfg->useWeights && !aligned(landScale, 4)))
            return fail(EPDC_ERR_ALIGN, "int32/fp32 arrays must be 4-byte aligned");
        epdc::CombineParams P{};
        P.W = cfg->worldSize;
        P.H = cfg->hiddenDim;
        P.M = cfg->maxTokPerRank;
        P.Epr = cfg->numExpertPerRank;
        P.K = cfg->numExpertPerToken;
        P.T = numTokens;
        P.useWeights = cfg->useWeights;
        P.eprShift = log2_exact(cfg->numExpertPerRank);
        P.rowBytes = cfg->hiddenDim * elem_bytes(cfg->dtype, true);
        P.outRowBytes = cfg->hiddenDim * out_elem_bytes(outDtype);
        P.nChunks = epdc::ceil_div(P.rowBytes, epdc::kChunkBytes);
        P.y = static_cast<const uint8_t *>(landing);
        P.sendMap = sendMap;
        P.out = static_cast<uint8_t *>(out);
        P.landScale = cfg->useWeights ? landScale : nullptr;
        P.recvCount = recvCount;
        P.landRows = landing_rows(cfg, numTokens);
        return hip_status(epdc::launch_combine(P, cfg->dtype == EPDC_FP32, outDtype == EPDC_FP32, true,
                                               static_cast<hipStream_t>(stream)),
                          "reduce launch");
    } catch (...) {
        return fail(EPDC_ERR_HIP, "unexpected C++ exception in epdc_combine_reduce");
    }
}

const char *epdc_last_error(void) { return g_lastError.c_str(); }

}  // extern "C"
