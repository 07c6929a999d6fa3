// EP dispatch for gfx950: COUNT -> SCAN -> FINALIZE.
//
// The phases are those of mori PR #599 "Perf/ep disp 1250 ship": COUNT maps
// each (token, top-k slot) to its destination PE and deduplicates so a token
// reaches each PE once (items "ballot dedup" and "cached destPe/keep");
// FINALIZE writes the payload rows, the per-token metadata and one null entry
// per dropped slot.  Where that PR reserves rows with a cross-card fetch_add
// (whose order is not deterministic), this path computes each row with an
// exclusive scan in ascending token order, so windows are stable.
//
// Wave64 design:
//   * one lane per token: the token's destination set is a 64-bit PE mask
//     built in registers from its K ids (dedup is a bit test, lowest slot
//     keeps);
//   * W ballots over the mask bits give, per PE, the tile's histogram
//     (popcount) and every token's rank inside the tile (popcount of the
//     lanes below it) -- no per-slot shuffles;
//   * the payload loop walks the set bits of a token's PE mask (only live
//     destinations), moving 16 bytes per lane per access, each source chunk
//     loaded once and stored to every destination.
#include "epdc_internal.h"

namespace epdc {
namespace {

__device__ __forceinline__ int32_t dest_pe(int32_t e, int32_t E, int32_t Epr, int32_t eprShift) {
    if (e < 0 || e >= E) return -1;
    return eprShift >= 0 ? (e >> eprShift) : (e / Epr);
}

// Destination-PE set of token t (bit p set iff some valid slot of t is on p).
__device__ __forceinline__ uint64_t token_pe_mask(const DispatchParams &P, int32_t t) {
    const int32_t E = P.W * P.Epr;
    const int32_t *ids = P.expertIds + (int64_t)t * P.K;
    uint64_t m = 0;
    for (int k = 0; k < P.K; ++k) {
        int32_t p = dest_pe(ids[k], E, P.Epr, P.eprShift);
        if (p >= 0) m |= 1ull << p;
    }
    return m;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// ---------------------------------------------------------------- COUNT
// One wave per 64-token tile: tileCount[tile][p] = tokens of the tile on p.
__global__ __launch_bounds__(64) void count_kernel(DispatchParams P) {
    const int lane = threadIdx.x;
    const int tile = blockIdx.x;
    const int32_t t = tile * kTile + lane;
    const uint64_t m = (t < P.T) ? token_pe_mask(P, t) : 0ull;
    int cnt = 0;
    for (int p = 0; p < P.W; ++p) {
        const uint64_t b = __ballot((m >> p) & 1ull);
        if (lane == p) cnt = __popcll(b);
    }
    if (lane < P.Wp) P.tileCount[(int64_t)tile * P.Wp + lane] = cnt;
}

__global__ __launch_bounds__(64) void zero_count_kernel(int32_t *recvCount, int32_t W) {
    if ((int)threadIdx.x < W) recvCount[threadIdx.x] = 0;
}

// Chunks [slab*CPW, slab*CPW + CPW) of one row, 16 bytes per lane.  With
// FULL every chunk is known to lie inside the row (H a multiple of 512 and
// the chunk count a multiple of CPW), so there is no per-lane bound check.
template <int CPW, bool FULL>
__device__ __forceinline__ void load_slab(u32x4 (&v)[CPW], const uint16_t *row, int slab, int nChunks,
                                          int H, int lane) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int gc = slab * CPW + c;
        const int e = gc * kChunkElems + lane * 8;
        if (FULL || (gc < nChunks && e < H)) v[c] = *reinterpret_cast<const u32x4 *>(row + e);
    }
}

template <int CPW, bool FULL>
__device__ __forceinline__ void store_slab(const u32x4 (&v)[CPW], uint16_t *row, int slab, int nChunks,
                                           int H, int lane) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int gc = slab * CPW + c;
        const int e = gc * kChunkElems + lane * 8;
        if (FULL || (gc < nChunks && e < H)) *reinterpret_cast<u32x4 *>(row + e) = v[c];
    }
}

// Stores one token's slab to every destination PE in its mask (the "ballot
// walk": only live destinations are visited).  Straight-line for up to 8
// destinations, so the stores sit in no loop and the only wait is the one
// for this token's own loads.
template <int CPW, bool FULL>
__device__ __forceinline__ void store_dest(const DispatchParams &P, const u32x4 (&v)[CPW],
                                           const uint64_t *sBal, const int32_t *sPre, uint64_t lt,
                                           int p, int slab, int lane) {
    const int32_t r = uniform(sPre[p] + __popcll(sBal[p] & lt));
    store_slab<CPW, FULL>(v, P.recvX + ((int64_t)p * P.M + r) * P.H, slab, P.nChunks, P.H, lane);
}

template <int CPW, bool FULL>
__device__ __forceinline__ void store_token(const DispatchParams &P, const u32x4 (&v)[CPW],
                                            const uint64_t *sMask, const uint64_t *sBal,
                                            const int32_t *sPre, int i, int slab, int lane) {
    uint64_t m = uniform64(sMask[i]);
    const uint64_t lt = lanemask_lt(i);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (m) {
            const int p = __builtin_ctzll(m);
            m &= m - 1;
            store_dest<CPW, FULL>(P, v, sBal, sPre, lt, p, slab, lane);
        }
    }
    while (m) {  // more than 8 destinations (worldSize and topk both above 8)
        const int p = __builtin_ctzll(m);
        m &= m - 1;
        store_dest<CPW, FULL>(P, v, sBal, sPre, lt, p, slab, lane);
    }
}

// ------------------------------------------------------ SCAN + FINALIZE
// Block = 4 waves on one (64-token tile, token subset, column slab).
// blockIdx.x = (tile * nSubs + sub) * nSlabs + slab; the block copies tokens
// [sub*tpb, (sub+1)*tpb) of the tile, tpb = 64 / nSubs, over chunks
// [slab*CPW, (slab+1)*CPW).
//   SCAN: the tile's base row on each PE is the sum of the counts of all
//   earlier tiles (every thread sums a strided share; LDS adds combine them).
//   The tile's routing is recomputed by wave 0 (ids are tiny and L2-hot).
//   FINALIZE: each wave copies the slab of every 4th token of the subset to
//   each of its destinations; the (sub 0, slab 0) block of a tile also writes
//   the metadata, the sendMap entries (row or null) and, for the last tile,
//   recvCount.
template <int CPW, bool FULL>
__global__ __launch_bounds__(256) void finalize_kernel(DispatchParams P, int nSlabs, int nSubs) {
    __shared__ uint64_t sMask[kTile];  // destination-PE set of each token of the tile
    __shared__ uint64_t sBal[64];      // per PE: which tokens of the tile go there
    __shared__ int32_t sPre[64];       // per PE: rows taken by earlier tiles

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int slab = blockIdx.x % nSlabs;
    const int ts = blockIdx.x / nSlabs;
    const int sub = ts % nSubs;
    const int tile = ts / nSubs;
    const int32_t tok0 = tile * kTile;
    const int nTok = min(kTile, P.T - tok0);
    const int tpb = kTile / nSubs;
    const int iEnd = min(nTok, (sub + 1) * tpb);
    const int iBeg = sub * tpb + wave;

    // Start this wave's first row load before the scan.
    u32x4 bufA[CPW], bufB[CPW];
    const uint16_t *xTile = P.x + (int64_t)tok0 * P.H;
    if (iBeg < iEnd) load_slab<CPW, FULL>(bufA, xTile + (int64_t)iBeg * P.H, slab, P.nChunks, P.H, lane);

    if (tid < 64) sPre[tid] = 0;
    __syncthreads();

    // SCAN: exclusive base of this tile on each PE.  The row stride Wp is a
    // power of two dividing 256, so thread tid only ever sums PE tid % Wp.
    {
        const int n = tile * P.Wp;
        int acc = 0;
        int idx = tid;
        for (; idx + 3 * 256 < n; idx += 4 * 256) {
            const int a = P.tileCount[idx], b = P.tileCount[idx + 256];
            const int c = P.tileCount[idx + 512], d = P.tileCount[idx + 768];
            acc += a + b + c + d;
        }
        for (; idx < n; idx += 256) acc += P.tileCount[idx];
        if (acc) atomicAdd(&sPre[tid & (P.Wp - 1)], acc);
    }

    // COUNT again for this tile (wave 0): PE masks and per-PE ballots.
    if (wave == 0) {
        const int32_t t = tok0 + lane;
        const uint64_t m = (lane < nTok) ? token_pe_mask(P, t) : 0ull;
        sMask[lane] = m;
        for (int p = 0; p < P.W; ++p) {
            const uint64_t b = __ballot((m >> p) & 1ull);
            if (lane == 0) sBal[p] = b;
        }
    }
    __syncthreads();

    if (slab == 0 && sub == 0 && wave == 0) {
        if (lane < nTok) {
            const int32_t t = tok0 + lane;
            const int32_t E = P.W * P.Epr;
            const int32_t *ids = P.expertIds + (int64_t)t * P.K;
            const float *wts = P.weights + (int64_t)t * P.K;
            uint64_t seen = 0;
            for (int k = 0; k < P.K; ++k) {
                const int32_t p = dest_pe(ids[k], E, P.Epr, P.eprShift);
                int32_t flat = -1;  // the null entry of a dropped slot
                if (p >= 0 && !((seen >> p) & 1ull)) {
                    seen |= 1ull << p;
                    const int32_t r = sPre[p] + __popcll(sBal[p] & lanemask_lt(lane));
                    flat = p * P.M + r;
                    P.recvTokIdx[flat] = t;
                    int32_t *dIds = P.recvExpertIds + (int64_t)flat * P.K;
                    for (int j = 0; j < P.K; ++j) dIds[j] = ids[j];
                    if (P.useWeights) {
                        float *dW = P.recvWeights + (int64_t)flat * P.K;
                        for (int j = 0; j < P.K; ++j) dW[j] = wts[j];
                    }
                }
                P.sendMap[(int64_t)t * P.K + k] = flat;
            }
        }
        if (tok0 + kTile >= P.T && lane < P.W)
            P.recvCount[lane] = sPre[lane] + __popcll(sBal[lane]);
    }

    // FINALIZE payload, software-pipelined over this wave's tokens: the next
    // token's slab is requested before the current one is stored, so a wait
    // for a load never has to wait for earlier stores (one in-order vmcnt).
    // The prefetch is unconditional -- the last token re-reads its own row --
    // to keep every wait count exact.
    // One explicit wait per token -- "all but the CPW loads just issued" --
    // marks the current buffer complete before the destination branches,
    // which would otherwise each get a conservative wait that also drains
    // the previous destination's stores.
    int i = iBeg;
    while (i < iEnd) {
        load_slab<CPW, FULL>(bufB, xTile + (int64_t)(i + 4 < iEnd ? i + 4 : i) * P.H, slab, P.nChunks,
                             P.H, lane);
        if (FULL) wait_vmcnt<CPW>(); else wait_vmcnt<0>();
        store_token<CPW, FULL>(P, bufA, sMask, sBal, sPre, i, slab, lane);
        i += 4;
        if (i >= iEnd) break;
        load_slab<CPW, FULL>(bufA, xTile + (int64_t)(i + 4 < iEnd ? i + 4 : i) * P.H, slab, P.nChunks,
                             P.H, lane);
        if (FULL) wait_vmcnt<CPW>(); else wait_vmcnt<0>();
        store_token<CPW, FULL>(P, bufB, sMask, sBal, sPre, i, slab, lane);
        i += 4;
    }
}

template <int CPW>
hipError_t launch_finalize(const DispatchParams &P, int nTiles, int nSubs, hipStream_t stream) {
    const int nSlabs = ceil_div(P.nChunks, CPW);
    const dim3 grid(nTiles * nSubs * nSlabs);
    if (P.H % kChunkElems == 0 && P.nChunks % CPW == 0)
        hipLaunchKernelGGL((finalize_kernel<CPW, true>), grid, dim3(256), 0, stream, P, nSlabs, nSubs);
    else
        hipLaunchKernelGGL((finalize_kernel<CPW, false>), grid, dim3(256), 0, stream, P, nSlabs, nSubs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const DispatchParams &P, hipStream_t stream) {
    if (P.T == 0) {
        hipLaunchKernelGGL(zero_count_kernel, dim3(1), dim3(64), 0, stream, P.recvCount, P.W);
        return hipGetLastError();
    }
    const int nTiles = ceil_div(P.T, kTile);
    hipLaunchKernelGGL(count_kernel, dim3(nTiles), dim3(64), 0, stream, P);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // Geometry: the largest work per block that still gives about 1536
    // blocks (6 per CU), preferring 2-chunk slabs, then 1-chunk slabs with
    // the tile's tokens split over 1..16 blocks.
    constexpr int kTargetBlocks = 1536;
    if (P.nChunks >= 2 && (int64_t)nTiles * ceil_div(P.nChunks, 2) >= kTargetBlocks)
        return launch_finalize<2>(P, nTiles, 1, stream);
    int nSubs = 1;
    while (nSubs < 16 && (int64_t)nTiles * nSubs * P.nChunks < kTargetBlocks) nSubs *= 2;
    return launch_finalize<1>(P, nTiles, nSubs, stream);
}

}  // namespace epdc
