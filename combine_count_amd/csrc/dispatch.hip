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

#include <mutex>

namespace epdc {
namespace {

constexpr bool kNtLoad = kDispatchNtLoad;
constexpr bool kNtStore = kDispatchNtStore;

// PE of expert e (-1 if e is not an expert id): e / Epr by multiply-high
// (div_magic), a few instructions for any Epr.
__device__ __forceinline__ int32_t dest_pe(const DispatchParams &P, int32_t e, int32_t E) {
    if ((uint32_t)e >= (uint32_t)E) return -1;
    const uint32_t t = __umulhi((uint32_t)e, P.eprMagic);
    return (int32_t)((t + (((uint32_t)e - t) >> P.eprSh1)) >> P.eprSh2);
}

// Expert ids of token t in slots 0..7, requested together (slots past K
// repeat slot K-1, which leaves the token's PE set unchanged): a tile's ids
// then cost one memory round trip instead of one per slot.
__device__ __forceinline__ void load_ids(const DispatchParams &P, int32_t t, int32_t (&v)[8]) {
    const int32_t *ids = P.expertIds + (int64_t)t * P.K;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = ids[min(k, P.K - 1)];
}

// Destination-PE set of token t (bit p set iff some valid slot of t is on p)
// from its ids as load_ids requested them; slots 8.. (topk above 8) are read
// here.
__device__ __forceinline__ uint64_t pe_mask(const DispatchParams &P, const int32_t (&v)[8], int32_t t) {
    const int32_t E = P.W * P.Epr;
    uint64_t m = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int32_t p = dest_pe(P, v[k], E);
        if (p >= 0) m |= 1ull << p;
    }
    const int32_t *ids = P.expertIds + (int64_t)t * P.K;
    for (int k = 8; k < P.K; ++k) {
        const int32_t p = dest_pe(P, ids[k], E);
        if (p >= 0) m |= 1ull << p;
    }
    return m;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Published count of tile j on PE p, waited for with a bound.  Forward
// progress: workgroups are dispatched in increasing blockIdx order (per XCD),
// so every block of an earlier tile was dispatched before any block that
// waits on it, and a block publishes before it waits on anything.  The bound
// only matters if that ever fails with every slot held by waiting blocks: the
// wait then gives up and flags the scratch error word (outputs invalid)
// instead of hanging the GPU.
constexpr int kMaxSpins = 1 << 18;

__device__ __forceinline__ uint32_t load_published(uint32_t *slot) {
    return __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __noinline__ uint32_t wait_published(uint32_t *slot, uint32_t *errWord) {
    uint32_t v = load_published(slot);
    for (int spins = 0; v == 0; ++spins) {
        if (spins >= kMaxSpins) {
            __hip_atomic_store(errWord, kStatusWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return 1u;
        }
        __builtin_amdgcn_s_sleep(2);
        v = load_published(slot);
    }
    return v;
}

__global__ __launch_bounds__(64) void zero_count_kernel(int32_t *recvCount, int32_t W) {
    if ((int)threadIdx.x < W) recvCount[threadIdx.x] = 0;
}

// Chunks [slab*CPW, slab*CPW + CPW) of one row, 16 bytes per lane.  With
// FULL every chunk is known to lie inside the row (the row a whole number of
// 1 KiB chunks and the chunk count a multiple of CPW), so there is no
// per-lane bound check.  Rows are bytes: the wire dtype does not matter.
template <int CPW, bool FULL>
__device__ __forceinline__ void load_slab(u32x4 (&v)[CPW], const uint8_t *row, int slab, int nChunks,
                                          int rowBytes, int lane) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int gc = slab * CPW + c;
        const int e = gc * kChunkBytes + lane * 16;
        // A lane past the row's end loads the row's first 16 bytes (in
        // bounds, never stored): unconditional loads need no branch or wait.
        v[c] = load16<kNtLoad>(row + ((FULL || (gc < nChunks && e < rowBytes)) ? e : 0));
    }
}

// Row stores: non-temporal and device-scope (nt sc1).  Against nt alone,
// one library per process, 2 rounds, dispatch + combine step: EpCfg defaults
// 12.45 -> 12.07 us, 16384 tokens 529 -> 524, 4096 tokens x h7168 82.2 ->
// 82.0, the others even; sc1 without nt was 19% slower at 4096 tokens.
template <int CPW, bool FULL>
__device__ __forceinline__ void store_slab(const u32x4 (&v)[CPW], uint8_t *row, int slab, int nChunks,
                                           int rowBytes, int lane) {
    static_assert(kNtStore, "row stores are non-temporal");
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int gc = slab * CPW + c;
        const int e = gc * kChunkBytes + lane * 16;
        if (FULL || (gc < nChunks && e < rowBytes)) store16_nt_dev(row, e, v[c]);
    }
}

// Stores one token's slab to every destination PE in its mask (the "ballot
// walk": only live destinations are visited), all uniform scalar control.
// A row outside [0, maxTokPerRank) can only come from a scratch that was not
// zero at launch (its counts then sum to anything, negative included); it is
// flagged and skipped rather than written.
__device__ __forceinline__ bool row_ok(const DispatchParams &P, int32_t r) {
    if ((uint32_t)r < (uint32_t)P.M) return true;
    __hip_atomic_store(P.scratch + kScratchError, kStatusRowOutside, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
}

template <int CPW, bool FULL>
__device__ __forceinline__ void store_dest(const DispatchParams &P, const u32x4 (&v)[CPW],
                                           const uint64_t *sBal, const int32_t *sPre, uint64_t lt,
                                           int p, int slab, int lane) {
    const int32_t r = uniform((int32_t)((uint32_t)sPre[p] + (uint32_t)__popcll(sBal[p] & lt)));
    if (row_ok(P, r))
        store_slab<CPW, FULL>(v, P.recvX + ((int64_t)p * P.M + r) * P.rowBytes, slab, P.nChunks, P.rowBytes, lane);
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

// Scales 64.. of token t to each of its destination rows (its PE mask m):
// scale rows longer than a wave, loaded here 64 at a time (the first 64
// travel in registers from the metadata loads).  Runs after the wave's other
// stores, so the loads' wait also covers those stores; such rows are rare.
__device__ __forceinline__ void copy_scale_tail(const DispatchParams &P, int32_t t, uint64_t m, uint64_t lt,
                                             const uint64_t *sBal, const int32_t *sPre, int lane) {
    for (int s0 = 64; s0 < P.S; s0 += 64) {
        const bool in = s0 + lane < P.S;
        const float v = in ? P.scales[(int64_t)t * P.S + s0 + lane] : 0.0f;
        uint64_t rest = m;
        while (rest) {
            const int p = __builtin_ctzll(rest);
            rest &= rest - 1;
            const int32_t r = uniform((int32_t)((uint32_t)sPre[p] + (uint32_t)__popcll(sBal[p] & lt)));
            if ((uint32_t)r >= (uint32_t)P.M) continue;  // flagged by the metadata loop
            if (in) P.recvScales[((int64_t)p * P.M + r) * P.S + s0 + lane] = v;
        }
    }
}

// ------------------------------------------- COUNT + SCAN + FINALIZE
// One kernel.  A block has 4 waves and copies the 4*NTW tokens
// [sub*4*NTW, (sub+1)*4*NTW) of a 64-token tile -- NTW consecutive tokens per
// wave -- over chunks [slab*CPW, (slab+1)*CPW).  Block b = blockIdx.x is
// (tile * nSubs + sub) * nSlabs + slab, except where every block sums the
// SCAN (SCAN self), where the tile leaders (sub 0, slab 0) come first:
// blocks 0..nTiles-1, then every tile's other blocks in the same order.  The
// leaders' COUNT then starts in the first blocks of the grid, before the
// rest of it floods the memory with row loads (4096 tokens: fp4x2 rows 16.1
// -> 15.4 us, h2048 17.2 -> 16.6; larger launches, whose blocks wait on
// their leader, lose 2-5% with it).
//   0. Loads.  A local scan (launches of at most kLocalScanTiles tiles)
//      requests every load up front: the ids it counts, then the x slabs and
//      the metadata rows.  The other forms request the wave's x slabs before
//      COUNT (with x cold in HBM, the sooner they are in flight the better),
//      with COUNT's ids ahead of them when every block sums the SCAN and
//      behind them when the tile leaders publish (plan_dispatch in
//      epdc_internal.h has the measurements).
//   1. COUNT (wave 0): the tile's PE masks (each lane's ids requested
//      together) and per-PE ballots; the tile's leader (its first block:
//      sub 0, slab 0) publishes the per-PE counts as count+1.
//   2. SCAN: the leader sums the published counts of all earlier tiles into
//      the tile's base row on each PE and publishes it as base+1; the
//      tile's other blocks wait for that single line (so polling traffic
//      does not grow with the number of blocks per tile).  With SCAN self
//      every block sums the counts itself, which takes the
//      publish-and-poll round trip off the path.
//   3. The slab-0 waves' metadata rows (ids, weights and scales) are
//      requested once the SCAN is done.
//   4. FINALIZE: one wait for the wave's loads, then every store of its NTW
//      tokens to every destination, with no further wait (vmcnt is one
//      in-order counter for loads and stores on this ISA, so waiting on a
//      load issued after a store would also wait for the store).  Then the
//      waves of slab-0 blocks write their tokens' metadata and sendMap
//      entries (row or null), and the last tile's leader recvCount.
//   5. The last block to finish clears the published counts; the done
//      counters wrap to zero by themselves, so the scratch is zero again for
//      the next call (and for every replay of a captured graph).
// The SCAN form (and with it the load order) is a compile-time choice: with
// the order a runtime flag, the compiler's waits had to cover every order at
// once (measured: the 4096-token h7168 launch 1.4% slower).
template <int CPW, int NTW, bool FULL, int SCAN>
__global__ __launch_bounds__(256) void dispatch_kernel(DispatchParams P, int nSlabs, int nSubs, int nBlocks) {
    constexpr bool localScan = SCAN == kScanLocal;
    constexpr bool selfScan = SCAN == kScanSelf;
    __shared__ uint64_t sMask[kTile];  // destination-PE set of each token of the tile
    __shared__ uint64_t sBal[64];      // per PE: which tokens of the tile go there
    __shared__ int32_t sPre[64];       // per PE: rows taken by earlier tiles
    __shared__ uint32_t sLast;  // 1 in the block that finishes last

    uint32_t *const hdr = P.scratch;
    const int nTilesAll = ceil_div(P.T, kTile);
    uint32_t *const published = P.scratch + kScratchHeaderWords;   // [tile][Wp]: count + 1
    uint32_t *const prefixes = published + (int64_t)nTilesAll * P.Wp;  // [tile][Wp]: base + 1
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);

    if (tid < 64) sPre[tid] = 0;
    __syncthreads();
    const int b = blockIdx.x;
    int slab, sub, tile;
    if constexpr (selfScan) {  // leaders first
        if (b < nTilesAll) {
            tile = b;
            sub = 0;
            slab = 0;
        } else {
            const int per = nSubs * nSlabs - 1;  // >= 3: nSubs >= 4
            const int bb = b - nTilesAll;
            tile = bb / per;
            const int r = bb - tile * per + 1;
            sub = r / nSlabs;
            slab = r - sub * nSlabs;
        }
    } else {
        slab = b % nSlabs;
        const int ts = b / nSlabs;
        sub = ts % nSubs;
        tile = ts / nSubs;
    }
    const int32_t tok0 = tile * kTile;
    const int nTok = min(kTile, P.T - tok0);
    const int iBeg = (sub * 4 + wave) * NTW;  // this wave's tokens: [iBeg, iBeg + NTW) of the tile
    const uint8_t *xTile = P.x + (int64_t)tok0 * P.rowBytes;
    // SCAN local (launches of at most kLocalScanTiles tiles): every block
    // counts the earlier tiles' tokens itself (their ids are a few KB, read
    // from L2), so there is no publishing, no cross-block wait and no
    // scratch, and every load can be issued up front -- small launches are
    // bound by round trips, not bytes.  (One tile: its base rows are 0.)  A
    // separate instantiation, so the scratch path compiles as if alone.  A
    // block whose token group lies past the last token only counts itself
    // done.
    const bool active = sub * 4 * NTW < nTok;
    if (active) {

    // Every x slab of this wave (a token past the end of the tile re-reads
    // the last one; it is not stored), and the slab-0 waves' metadata rows
    // (lanes are slots; with scales, lanes are also the first 64 scales).
    u32x4 buf[NTW][CPW];
    auto load_x = [&]() {
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int i = min(iBeg + j, nTok - 1);
            load_slab<CPW, FULL>(buf[j], xTile + (int64_t)i * P.rowBytes, slab, P.nChunks, P.rowBytes, lane);
        }
    };
    int32_t mid[NTW];
    float mwt[NTW], msc[NTW];
    auto load_meta = [&]() {
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            mid[j] = -1;
            mwt[j] = 0.0f;
            msc[j] = 0.0f;
            const int i = iBeg + j;
            if (slab == 0 && i < nTok && lane < P.K) {
                const int64_t o = (int64_t)(tok0 + i) * P.K + lane;
                mid[j] = P.expertIds[o];
                if (P.useWeights) mwt[j] = P.weights[o];
            }
            if (slab == 0 && i < nTok && lane < P.S) msc[j] = P.scales[(int64_t)(tok0 + i) * P.S + lane];
        }
    };
    // 0. Loads.  The ids COUNT reads (wave 0: a token of the tile per lane)
    // and, for a local scan, those of the earlier tiles this wave counts
    // (tiles wave, wave + 4, ...; all full) go out before the local scan's
    // x slabs, so counting waits for them alone (one round trip where a scan
    // is a chain of them); so do they when every block sums the SCAN.  When
    // the tile leaders publish, the x slabs go out first: there the blocks
    // that count sooner only reach the wait for the leader's line sooner.
    constexpr int kScanPerWave = (kLocalScanTiles + 2) / 4 > 0 ? (kLocalScanTiles + 2) / 4 : 1;
    int32_t idOwn[8];
    int32_t idScan[kScanPerWave][8];
    if constexpr (SCAN == kScanLeader) load_x();
    if (wave == 0) load_ids(P, tok0 + min(lane, nTok - 1), idOwn);
    if constexpr (selfScan) load_x();
    if constexpr (localScan) {
#pragma unroll
        for (int i = 0; i < kScanPerWave; ++i)
            if (wave + 4 * i < tile) load_ids(P, (wave + 4 * i) * kTile + lane, idScan[i]);
        load_x();
        load_meta();
    }

    // 1. COUNT for this tile (wave 0); the tile's leader block (sub 0,
    // slab 0: the first block of the tile) publishes the per-PE counts.
    const bool leader = (sub == 0 && slab == 0);
    if (wave == 0) {
        const int32_t t = tok0 + lane;
        const uint64_t m = (lane < nTok) ? pe_mask(P, idOwn, t) : 0ull;
        sMask[lane] = m;
        int cnt = 0;
        for (int p = 0; p < P.W; ++p) {
            const uint64_t bal = __ballot((m >> p) & 1ull);
            if (lane == 0) sBal[p] = bal;
            if (lane == p) cnt = __popcll(bal);
        }
        if (!localScan && leader && lane < P.Wp)
            __hip_atomic_store(published + (int64_t)tile * P.Wp + lane, (uint32_t)cnt + 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }

    // 2. SCAN: exclusive base of this tile on each PE.  The leader sums the
    // published counts of all earlier tiles (the row stride Wp is a power of
    // two dividing 256, so thread tid only ever sums PE tid % Wp) and
    // publishes the result; the tile's other blocks wait for that one line.
    // With SCAN self every block sums for itself and nothing is published:
    // a block still waits only for the counts of earlier tiles, whose
    // leaders were dispatched before it.
    // Tile 0's base rows are 0: nothing to sum, publish or wait for.  A
    // local scan counts the earlier tiles (all full) in this block instead,
    // the 4 waves taking tiles wave, wave + 4, ...
    if constexpr (localScan) {
        static_assert(4 * kScanPerWave >= kLocalScanTiles - 1, "every earlier tile has a wave");
#pragma unroll
        for (int i = 0; i < kScanPerWave; ++i) {
            const int j = wave + 4 * i;
            if (j >= tile) break;
            const uint64_t m = pe_mask(P, idScan[i], j * kTile + lane);
            for (int p = 0; p < P.W; ++p) {
                const uint64_t bal = __ballot((m >> p) & 1ull);
                if (lane == p && bal) atomicAdd(&sPre[p], (int32_t)__popcll(bal));
            }
        }
    } else if (tile > 0 && (leader || selfScan)) {
        const int n = tile * P.Wp;
        uint32_t acc = 0;
        int idx = tid;
        for (; idx + 3 * 256 < n; idx += 4 * 256) {
            uint32_t v0 = load_published(published + idx), v1 = load_published(published + idx + 256);
            uint32_t v2 = load_published(published + idx + 512), v3 = load_published(published + idx + 768);
            if (v0 == 0) v0 = wait_published(published + idx, hdr + kScratchError);
            if (v1 == 0) v1 = wait_published(published + idx + 256, hdr + kScratchError);
            if (v2 == 0) v2 = wait_published(published + idx + 512, hdr + kScratchError);
            if (v3 == 0) v3 = wait_published(published + idx + 768, hdr + kScratchError);
            acc += v0 + v1 + v2 + v3 - 4u;
        }
        for (; idx < n; idx += 256) {
            uint32_t v = load_published(published + idx);
            if (v == 0) v = wait_published(published + idx, hdr + kScratchError);
            acc += v - 1u;
        }
        if (acc) atomicAdd(&sPre[tid & (P.Wp - 1)], (int32_t)acc);
        if constexpr (!selfScan) {
            __syncthreads();
            if (tid < P.Wp)
                __hip_atomic_store(prefixes + (int64_t)tile * P.Wp + tid, (uint32_t)sPre[tid] + 1u,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else if (tile > 0 && tid < P.Wp) {
        uint32_t v = load_published(prefixes + (int64_t)tile * P.Wp + tid);
        if (v == 0) v = wait_published(prefixes + (int64_t)tile * P.Wp + tid, hdr + kScratchError);
        sPre[tid] = (int32_t)(v - 1u);
    }
    __syncthreads();

    // 3. Scanning through the scratch, the metadata rows are requested only
    // now (the slab-0 waves' ids, weights and scales).  No wait below
    // follows a store.
    const int32_t E = P.W * P.Epr;
    if constexpr (!localScan) load_meta();

    // 4. FINALIZE payload: one wait for every load above, then only stores.
    wait_vmcnt<0>();
#pragma unroll
    for (int j = 0; j < NTW; ++j)
        if (iBeg + j < nTok) store_token<CPW, FULL>(P, buf[j], sMask, sBal, sPre, iBeg + j, slab, lane);

    // 4. FINALIZE metadata (slab-0 blocks, each wave for its own tokens).
    // Each destination's id / weight copies and the token's sendMap row are
    // one coalesced store each.  The kept slot of PE p is the lowest lane
    // whose expert lives on p; every other slot gets the null entry -1.
    if (slab == 0) {
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int i = iBeg + j;
            if (i < nTok) {
                const int32_t t = tok0 + i;
                const int32_t pe = dest_pe(P, mid[j], E);
                int32_t flat = -1;
                uint64_t m = uniform64(sMask[i]);
                const uint64_t lt = lanemask_lt(i);
                while (m) {
                    const int p = __builtin_ctzll(m);
                    m &= m - 1;
                    const int32_t r = uniform((int32_t)((uint32_t)sPre[p] + (uint32_t)__popcll(sBal[p] & lt)));
                    if (!row_ok(P, r)) continue;
                    const int32_t f = p * P.M + r;
                    const uint64_t onP = __ballot(lane < P.K && pe == p);
                    if (lane == __builtin_ctzll(onP)) flat = f;
                    if (lane < P.K) {
                        P.recvExpertIds[(int64_t)f * P.K + lane] = mid[j];
                        if (P.useWeights) P.recvWeights[(int64_t)f * P.K + lane] = mwt[j];
                    }
                    if (lane < P.S) P.recvScales[(int64_t)f * P.S + lane] = msc[j];
                    if (lane == 0) P.recvTokIdx[f] = t;
                }
                if (lane < P.K) P.sendMap[(int64_t)t * P.K + lane] = flat;
                if (P.S > 64) copy_scale_tail(P, t, uniform64(sMask[i]), lt, sBal, sPre, lane);
            }
        }
        if (sub == 0 && wave == 0 && tok0 + kTile >= P.T && lane < P.W)
            P.recvCount[lane] = (int32_t)((uint32_t)sPre[lane] + (uint32_t)__popcll(sBal[lane]));
    }

    }  // active

    // 5. Completion.  Every block has read all the counts it needs (their
    // values were consumed before the barrier above) before it counts itself
    // done, so the last one may clear them.
    // Two-level count so that no counter takes more than ~nBlocks/32 atomics:
    // the last block of each group (b % 32) counts its group done.
    if constexpr (localScan) return;
    __syncthreads();
    if (tid == 0) {
        // Every publish of this block (counts and base rows) was made by
        // wave 0 with agent-scope stores; they have retired before its done
        // count, so the last block's clearing stores come after all of them.
        wait_vmcnt<0>();
        const int g = b % kDoneGroups;
        const int nGroups = min(nBlocks, kDoneGroups);
        const uint32_t inGroup = (uint32_t)((nBlocks - 1 - g) / kDoneGroups + 1);
        uint32_t last = 0;
        if (atomicInc(hdr + kScratchGroupBase + g * kDoneStride, inGroup - 1) == inGroup - 1)
            last = atomicInc(hdr + kScratchDone, (uint32_t)(nGroups - 1)) == (uint32_t)(nGroups - 1);
        sLast = last;
    }
    __syncthreads();
    if (sLast) {
        for (int i = tid; i < 2 * nTilesAll * P.Wp; i += 256)
            __hip_atomic_store(published + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Runs a plan (plan_dispatch in epdc_internal.h) with its compiled variant.
template <int CPW, int NTW, bool FULL, int SCAN>
hipError_t launch_variant(const DispatchParams &P, const DispatchPlan &pl, hipStream_t stream) {
    hipLaunchKernelGGL((dispatch_kernel<CPW, NTW, FULL, SCAN>), dim3((uint32_t)pl.nBlocks), dim3(256), 0, stream, P,
                       pl.nSlabs, pl.nSubs, (int)pl.nBlocks);
    return hipGetLastError();
}

template <int CPW, int NTW, int SCAN>
hipError_t launch_full(const DispatchParams &P, const DispatchPlan &pl, hipStream_t stream) {
    return pl.full ? launch_variant<CPW, NTW, true, SCAN>(P, pl, stream)
                   : launch_variant<CPW, NTW, false, SCAN>(P, pl, stream);
}

template <int CPW, int NTW>
hipError_t launch_fused(const DispatchParams &P, const DispatchPlan &pl, hipStream_t stream) {
    static_assert(kTile % (4 * NTW) == 0, "a block's tokens must tile the 64-token tile");
    if (pl.nBlocks > INT32_MAX) return hipErrorInvalidConfiguration;
    if constexpr (NTW == 1) {
        if (pl.scan == kScanLocal) return launch_full<CPW, NTW, kScanLocal>(P, pl, stream);
        if (pl.scan == kScanSelf) return launch_full<CPW, NTW, kScanSelf>(P, pl, stream);
    }
    // Several tokens per wave only come with launches of over 8192 blocks,
    // whose tile leaders always publish (plan_dispatch).
    if (pl.scan != kScanLeader) return hipErrorInvalidConfiguration;
    return launch_full<CPW, NTW, kScanLeader>(P, pl, stream);
}

template <int CPW>
hipError_t launch_cpw(const DispatchParams &P, const DispatchPlan &pl, hipStream_t stream) {
    switch (pl.ntw) {
        case 1: return launch_fused<CPW, 1>(P, pl, stream);
        case 2: return launch_fused<CPW, 2>(P, pl, stream);
        case 4: return launch_fused<CPW, 4>(P, pl, stream);
        default: return hipErrorInvalidConfiguration;
    }
}

}  // namespace

hipError_t launch_dispatch(const DispatchParams &P, hipStream_t stream) {
    if (P.T == 0) {
        hipLaunchKernelGGL(zero_count_kernel, dim3(1), dim3(64), 0, stream, P.recvCount, P.W);
        return hipGetLastError();
    }
    const DispatchPlan pl = plan_dispatch(P.T, P.rowBytes, P.W);
    switch (pl.cpw) {
        case 1: return launch_cpw<1>(P, pl, stream);
        case 2: return launch_cpw<2>(P, pl, stream);
        case 4: return launch_cpw<4>(P, pl, stream);
        case 7: return launch_cpw<7>(P, pl, stream);
        case 8: return launch_cpw<8>(P, pl, stream);
        default: return hipErrorInvalidConfiguration;
    }
}

// ------------------------------------------- allocation-free dispatch
// The scratch of epdc_dispatch_noalloc: a device array of this library's
// code object, one copy per GPU, held until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: its device address
// comes from hipGetSymbolAddress, once per device, and only that address is
// used (as the kernels' scratch argument and for the clearing kernel).
namespace {

static __device__ __align__(256) uint32_t scratch[kStaticScratchWords];

constexpr int kMaxDevices = 64;
std::mutex g_staticMutex;
uint32_t *g_staticScratch[kMaxDevices] = {};  // device address per device, once resolved

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *words, int32_t n) {
    for (int32_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) words[i] = 0u;
}

}  // namespace

int64_t dispatch_scratch_words(int32_t numTokens, int32_t W) {
    int32_t wp = 1;
    while (wp < W) wp <<= 1;
    return kScratchHeaderWords + 2 * (int64_t)ceil_div(numTokens, kTile) * wp;
}

hipError_t static_scratch(uint32_t **out, hipStream_t stream) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_staticMutex);
    if (!g_staticScratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        // Zero it once, on the caller's stream, before its first use (a
        // kernel, not a memset, so that it is also right inside a captured
        // graph); every dispatch leaves it zeroed again.
        hipLaunchKernelGGL(clear_words_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint32_t *>(p),
                           kStaticScratchWords);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_staticScratch[dev] = static_cast<uint32_t *>(p);
    }
    *out = g_staticScratch[dev];
    return hipSuccess;
}

}  // namespace epdc
