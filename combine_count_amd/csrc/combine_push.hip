// Push half of the scatter combine for gfx950: the rows every destination PE
// returns to this source move into packed landing rows, each with a
// forwarded fp32 scale.  The reduce half is combine_kernel over the landing
// rows (combine.hip).
//
// MORI JIT v2 design doc, §5 and §9: besides the gather combine there is a
// scatter combine (on the FlyDSL backend there), in which each destination
// pushes the rows it returns into the source's landing buffer and the source
// then reduces them.  The aiter MegaMoE commits on the mori PR #599 page size
// that buffer: one landing row per (token, destination PE), at most
// T * min(W, K) rows, at per-destination landing offsets that the dispatch
// hands over.
//
// Landing row of window row (p, r): landOff[p] + r, where landOff is the
// exclusive prefix sum, in PE order, of recvCount (each count clamped to
// [0, M]).  No row at or past T * min(W, K) is written.
//
// One wave64 per (landing row, slab of CPW 1 KiB chunks):
//   * lanes < W load recvCount; a wave scan gives every PE's landing offset
//     and the number of landed rows U; waves past U exit;
//   * a ballot over the offsets names the window the row comes from;
//   * the slab is requested, 16 bytes per lane per chunk, then (slab-0 waves
//     of a weighted call) the row's K expert ids and weights, the metadata
//     the dispatch delivered with it; the slab is stored;
//   * those waves forward the scale: the fp32 sum, in slot order from +0, of
//     the weights whose expert lives on this PE -- the gather combine's scale
//     for that PE.
#include "epdc_internal.h"

namespace epdc {
namespace {

template <int CPW, bool FULL>
__global__ __launch_bounds__(256) void push_kernel(PushParams P, int nSlabs) {
    const int lane = threadIdx.x & 63;
    const int32_t item = uniform((int32_t)blockIdx.x * 4 + (int32_t)(threadIdx.x >> 6));
    const int32_t L = item / nSlabs;
    const int32_t slab = item - L * nSlabs;
    if (L >= P.landRows) return;  // whole wave

    // Landing offsets of the windows, and the number of landed rows.
    int32_t c = 0;
    if (lane < P.W) {
        c = P.recvCount[lane];
        c = c < 0 ? 0 : (c > P.M ? P.M : c);
    }
    const int32_t incl = wave_incl_scan(c);
    const int32_t U = uniform(__shfl(incl, 63));
    if (L >= U) return;
    // Window p: the PEs whose rows all land before L are exactly the lanes
    // with incl <= L; L < U keeps p below W, and 0 <= r < count[p].
    const int32_t p = __popcll(__ballot(lane < P.W && incl <= L));
    const int32_t r = L - uniform(__shfl(incl - c, p));
    const int64_t src = (int64_t)p * P.M + r;

    const uint8_t *srow = P.y + src * P.rowBytes;
    uint8_t *drow = P.landing + (int64_t)L * P.rowBytes;
    // Every lane loads (a lane past the row's end reads the row's first 16
    // bytes instead, in bounds) and only in-row lanes store: unconditional
    // loads are issued back to back with no branch or wait between them.
    u32x4 v[CPW];
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
        const int gc = slab * CPW + k;
        const int e = gc * kChunkBytes + lane * 16;
        v[k] = load16<kPushNtLoad>(srow + ((FULL || (gc < P.nChunks && e < P.rowBytes)) ? e : 0));
    }
    // The row's metadata goes out behind its slab, so nothing waits for it
    // before the slab is requested.
    const bool doScale = P.useWeights && slab == 0;
    int32_t e = -1;
    float w = 0.0f;
    if (doScale && lane < P.K) {
        const int64_t o = src * P.K + lane;
        e = P.recvExpertIds[o];
        w = P.recvWeights[o];
    }
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
        const int gc = slab * CPW + k;
        const int eb = gc * kChunkBytes + lane * 16;
        if (FULL || (gc < P.nChunks && eb < P.rowBytes)) store16<kPushNtStore>(drow + eb, v[k]);
    }

    if (doScale) {
        int32_t pe = -1;
        if (e >= 0 && e < P.W * P.Epr) pe = P.eprShift >= 0 ? (e >> P.eprShift) : (e / P.Epr);
        float s = 0.0f;
        for (int k = 0; k < P.K; ++k) {
            const int32_t pk = __shfl(pe, k);
            const float wk = __shfl(w, k);
            if (pk == p) s = s + wk;
        }
        if (lane == 0) P.landScale[L] = s;
    }
}

// Runs a plan (plan_push in epdc_internal.h) with its compiled variant.
template <int CPW>
hipError_t launch_cpw(const PushParams &P, const RowPlan &pl, hipStream_t stream) {
    if (pl.waves > INT32_MAX - 3) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)pl.nBlocks);
    if (pl.full)
        hipLaunchKernelGGL((push_kernel<CPW, true>), grid, dim3(256), 0, stream, P, pl.nSlabs);
    else
        hipLaunchKernelGGL((push_kernel<CPW, false>), grid, dim3(256), 0, stream, P, pl.nSlabs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_push(const PushParams &P, hipStream_t stream) {
    if (P.landRows == 0) return hipSuccess;
    const RowPlan pl = plan_push(P.landRows, P.rowBytes);
    switch (pl.cpw) {
        case 1: return launch_cpw<1>(P, pl, stream);
        case 2: return launch_cpw<2>(P, pl, stream);
        case 4: return launch_cpw<4>(P, pl, stream);
        case 7: return launch_cpw<7>(P, pl, stream);
        case 8: return launch_cpw<8>(P, pl, stream);
        default: return hipErrorInvalidConfiguration;
    }
}

}  // namespace epdc
