// Internal interface between the host entry points (epdc_api.cpp) and the
// kernel launchers (dispatch.hip, combine.hip, combine_push.hip).  Not part
// of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace epdc {

// Native clang vector (not HIP's uint4 class, whose copies lower to memcpy
// through a private alloca): 16 bytes, one dwordx4 access per lane.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Wave-uniform copies of a value (forces scalar registers and scalar
// branches; the compiler cannot prove uniformity of values read from LDS or
// derived from threadIdx.x / 64).
__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum over the lanes of a wave64: lane i gets v_0 + ... + v_i.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t o = __shfl_up(v, d);
        if (lane >= d) v += o;
    }
    return v;
}

// s_waitcnt vmcnt(N) with no lgkm/exp wait (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).  vmcnt counts loads and
// stores in issue order, so this waits until at most N of the wave's vector
// memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Measured choices (each was timed against its alternatives; the reasons
// are with the code that uses them).
constexpr bool kDispatchNtLoad = false;     // x rows: plain loads
constexpr bool kDispatchNtStore = true;     // recvX rows: non-temporal, device-scope stores (store16_nt_dev)
constexpr bool kCombineNtLoad = true;       // returned rows: non-temporal loads
constexpr bool kCombineNtStore = true;      // out rows: non-temporal stores
constexpr bool kPushNtLoad = true;          // rows the push moves: non-temporal loads
constexpr bool kPushNtStore = true;         // landing rows: non-temporal stores
constexpr int kXEarlyBlocks = 2560;         // launches of more blocks (not self-summing) request x before COUNT
constexpr int kSelfScanBlocks = 1024;       // launches of up to this many blocks sum the tile counts in every block
                                            // (and, within kSelfScanWords, any launch of slabs of <= 4 chunks)
constexpr int kXMidSelfCpw = 4;             // self-summing launches with slabs of at most this many chunks request
                                            // x between COUNT and the SCAN's wait
constexpr int kSelfScanWords = 8192;        // ... and sum up to this many published words per block at any size
constexpr int kNarrowTiles = 4;             // launches of up to this many tiles use 1- or 2-chunk slabs
constexpr int kLocalScanTiles = 8;          // launches of up to this many 64-token tiles scan in every block
constexpr int kCombineGroup = 8;            // returned rows requested together per wave (gather combine)

// 16-byte access, optionally with the non-temporal (streaming) hint.
template <bool NT>
__device__ __forceinline__ u32x4 load16(const uint8_t *p) {
    if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return *reinterpret_cast<const u32x4 *>(p);
}

template <bool NT>
__device__ __forceinline__ void store16(uint8_t *p, u32x4 v) {
    if (NT)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
    else
        *reinterpret_cast<u32x4 *>(p) = v;
}

// 16-byte store with the non-temporal hint and device scope (nt sc1: the
// line streams through the caches towards memory instead of staying dirty in
// this XCD's L2).  `row` is wave-uniform (it becomes a buffer descriptor in
// scalar registers); off is the lane's byte offset in it, below 2^31.
__device__ __forceinline__ void store16_nt_dev(uint8_t *row, int off, u32x4 v) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(row, 0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, /*nt*/ 2 | /*sc1*/ 16);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 8-byte load (four bf16 values), optionally non-temporal.
template <bool NT>
__device__ __forceinline__ u32x2 load8(const uint8_t *p) {
    if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    return *reinterpret_cast<const u32x2 *>(p);
}

// 8-byte store (four bf16 values), optionally non-temporal.
template <bool NT>
__device__ __forceinline__ void store8(uint8_t *p, u32x2 v) {
    if (NT)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
    else
        *reinterpret_cast<u32x2 *>(p) = v;
}

// Routing tile: 64 tokens, one per lane of a wave64.
constexpr int kTile = 64;
// One 16-byte access per lane of a wave64 moves a 1 KiB chunk of a row
// (512 bf16, 256 fp32 or 1024 one-byte elements).
constexpr int kChunkBytes = 1024;

struct DispatchParams {
    int32_t W, H, M, Epr, K, T, useWeights;
    int32_t S;         // scaleDim: fp32 scales per token (0: none)
    int32_t rowBytes;  // H * element size of the wire dtype (a multiple of 16)
    int32_t Wp;        // W rounded up to a power of two (tile-count row stride)
    // e / Epr for any 32-bit e without a divide (div_magic): magic, shifts
    uint32_t eprMagic;
    int32_t eprSh1, eprSh2;
    int32_t nChunks;   // ceil(rowBytes / kChunkBytes)
    const uint8_t *x;
    const int32_t *expertIds;
    const float *weights;
    const float *scales;   // [T][S], NULL when S == 0
    uint8_t *recvX;
    int32_t *recvTokIdx;
    int32_t *recvExpertIds;
    float *recvWeights;
    float *recvScales;     // [W][M][S], NULL when S == 0
    int32_t *recvCount;
    int32_t *sendMap;
    uint32_t *scratch;  // scratch: header words, then tile counts [nTilesMax][Wp]
};

// Dispatch scratch layout (32-bit words).  Zero-filled by the caller before
// first use; every dispatch leaves it zeroed again (the error word aside).
constexpr int kScratchDone = 0;    // groups finished (wraps to 0 after the last)
constexpr int kScratchError = 2;   // status word: nonzero if this buffer's outputs are invalid
constexpr uint32_t kStatusWaitTimeout = 1;  // a bounded wait gave up
constexpr uint32_t kStatusRowOutside = 2;   // a computed row fell outside its window
constexpr int kDoneGroups = 32;    // blocks finished, per group b % 32, one 128-byte line each
constexpr int kDoneStride = 32;    // words between group counters
constexpr int kScratchGroupBase = 32;
constexpr int kScratchHeaderWords = kScratchGroupBase + kDoneGroups * kDoneStride;  // 4224 bytes
// Published tile count: count + 1 (0 = not yet published by this call).

struct CombineParams {
    int32_t W, H, M, Epr, K, T, useWeights;
    int32_t rowBytes;  // returned rows: H * 2 (bf16) or H * 4 (fp32)
    int32_t outRowBytes;  // output rows: H * 2 (bf16) or H * 4 (fp32)
    int32_t eprShift;
    int32_t nChunks;   // ceil(rowBytes / kChunkBytes)
    const uint8_t *y;  // returned rows [W][M] (gather) or landing rows [landRows] (reduce)
    const int32_t *expertIds;  // gather with useWeights only
    const float *weights;      // gather with useWeights only
    const int32_t *sendMap;
    uint8_t *out;
    // reduce over landing rows (scatter combine) only
    const float *landScale;    // [landRows], NULL without useWeights
    const int32_t *recvCount;  // [W]: landing offsets are its exclusive prefix sums
    int32_t landRows;          // T * min(W, K)
};

// Push half of the scatter combine: window rows -> packed landing rows.
struct PushParams {
    int32_t W, M, Epr, K, useWeights;
    int32_t rowBytes;  // H * 2 (bf16) or H * 4 (fp32)
    int32_t eprShift;
    int32_t nChunks;
    int32_t landRows;  // T * min(W, K)
    const uint8_t *y;  // [W][M] returned rows
    const int32_t *recvExpertIds;  // [W][M][K]
    const float *recvWeights;      // [W][M][K], NULL without useWeights
    const int32_t *recvCount;      // [W]
    uint8_t *landing;              // [landRows] rows
    float *landScale;              // [landRows], NULL without useWeights
};

__host__ __device__ inline int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

// Unsigned division by an invariant d >= 1 with one multiply-high (Granlund
// and Montgomery, "Division by invariant integers using multiplication",
// PLDI 1994, the unsigned case for N = 32): with l = ceil(log2 d),
// magic = floor(2^32 (2^l - d) / d) + 1 (it fits 32 bits), sh1 = min(l, 1)
// and sh2 = max(l - 1, 0), every 32-bit n has
// n / d = (t + ((n - t) >> sh1)) >> sh2 where t = umulhi(n, magic).
struct DivMagic {
    uint32_t magic;
    int32_t sh1, sh2;
};
inline DivMagic div_magic(uint32_t d) {
    int l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1;
    return DivMagic{(uint32_t)m, l < 1 ? l : 1, l > 1 ? l - 1 : 0};
}

// Launch geometry of one dispatch, chosen from the token count and the row
// size alone (host code; the launcher runs exactly this plan, and a host test
// pins it for the documented shapes).
// When a dispatch wave requests its x slabs (a compile-time choice of the
// kernel): after the SCAN, before COUNT, or between COUNT and the SCAN's wait
// (once the SCAN's own reads are out).
constexpr int kXOrderLate = 0;
constexpr int kXOrderEarly = 1;
constexpr int kXOrderMid = 2;

struct DispatchPlan {
    int32_t cpw;      // 1 KiB chunks per slab: 1, 2, 4, 7 or 8
    int32_t ntw;      // tokens per wave: 1, 2 or 4
    int32_t nSlabs;   // slabs per row
    int32_t nSubs;    // blocks per tile and slab (64 / (4 * ntw))
    int64_t nBlocks;  // grid size (0: no tokens, only recvCount is written)
    bool full;        // every slab lies inside the row: no per-lane bound checks
    bool local;       // local scan: every block counts the earlier tiles' ids
    bool selfScan;    // every block sums the published tile counts
    int32_t xOrder;   // when the x slabs are requested: kXOrderLate / kXOrderEarly / kXOrderMid
};

inline DispatchPlan plan_dispatch(int32_t T, int32_t rowBytes, int32_t W) {
    DispatchPlan pl{};
    if (T <= 0) return pl;
    const int32_t nTiles = ceil_div(T, kTile);
    const int32_t nChunks = ceil_div(rowBytes, kChunkBytes);
    const bool whole = rowBytes % kChunkBytes == 0;
    // Slab width.  Launches of at most kNarrowTiles tiles are
    // bound by round trips, not bytes: 2-chunk slabs (1 for an odd chunk
    // count) spread a token's stores over more waves (64 tokens x h7168:
    // 4.9 -> 4.2 us).  Otherwise the widest of 8/7/4/2 chunks that divides
    // the row (a wave then moves up to 8 KiB of a token with no bound
    // checks); other rows (not a whole number of 1 KiB chunks, e.g. 3.5 KiB
    // fp4x2 rows at hidden 7168) take the narrowest of 1/2/4/7/8 chunks that
    // covers the row (8 beyond that) with bound checks on the tail.  Rows of
    // exactly 7 chunks (fp8 rows at h7168, bf16 at h3584) take two
    // bound-checked 4-chunk slabs (4 + 3), which puts them under the
    // self-summing SCAN with x mid below (4096 tokens: fp8 rows 24.33 ->
    // 23.97 us, h3584 24.24 -> 23.91; 8192 fp8 tokens 44.2 -> 41.7).
    if (nTiles <= kNarrowTiles)
        pl.cpw = nChunks <= 1 ? 1 : (!whole || nChunks % 2 == 0) ? 2 : 1;
    else if (whole && nChunks == 7)
        pl.cpw = 4;
    else if (whole)
        pl.cpw = nChunks % 8 == 0 ? 8 : nChunks % 7 == 0 ? 7 : nChunks % 4 == 0 ? 4 : nChunks % 2 == 0 ? 2 : 1;
    else
        pl.cpw = nChunks <= 1 ? 1 : nChunks <= 2 ? 2 : nChunks <= 4 ? 4 : nChunks <= 7 ? 7 : 8;
    // Tokens per wave: one (most blocks, measured fastest at 4096 and 16384
    // tokens) unless that would exceed 16384 blocks.
    const int64_t perTokenWave = (int64_t)nTiles * (kTile / 4) * ceil_div(nChunks, pl.cpw);
    pl.ntw = perTokenWave <= 16384 ? 1 : perTokenWave <= 2 * 16384 ? 2 : 4;
    pl.nSubs = kTile / (4 * pl.ntw);
    pl.nSlabs = ceil_div(nChunks, pl.cpw);
    pl.nBlocks = (int64_t)nTiles * pl.nSubs * pl.nSlabs;
    pl.full = whole && nChunks % pl.cpw == 0;
    // The local scan is built for one token per wave only: more tokens per
    // wave within 8 tiles takes over 128 slabs per row (rows of 128 KiB and
    // up), and its id registers would then cost occupancy; such launches scan
    // through the scratch.
    pl.local = pl.ntw == 1 && nTiles <= kLocalScanTiles;
    // Every block sums the earlier tiles' counts itself in launches of up to
    // 4 blocks per CU, where it saves a round trip (measured at 4096 tokens:
    // fp4x2 rows 2.6%, h2048 2.3%; 640 / 1024 tokens at h7168 5.3% / 3.6%).
    // In larger launches of 7- and 8-chunk slabs the tile leader's one
    // published line is faster (1.5% at 2048 blocks, 1.6% for fp8 rows at
    // 1536; every block summing with x mid: 16384 tokens 5% slower).  One-
    // token-per-wave launches of slabs of at most 4 chunks sum in every
    // block at any size, with x mid, while a block's sum stays within
    // kSelfScanWords published words (one library per process, 3 rounds,
    // against the leader's line with x before COUNT: fp4x2 rows at 8192 /
    // 16384 / 65536 tokens 28.6 -> 24.3, 49.4 -> 43.0, 236.4 -> 188.0 us;
    // h2048 at 16384 tokens 53.3 -> 48.0; h1024 at 16384 / 65536 tokens
    // 37.6 -> 29.5, 173.3 -> 131.8).
    int32_t wp = 1;
    while (wp < W) wp <<= 1;
    pl.selfScan = !pl.local && (pl.nBlocks <= kSelfScanBlocks ||
                                (pl.cpw <= kXMidSelfCpw && pl.ntw == 1 && (int64_t)nTiles * wp <= kSelfScanWords));
    // x before COUNT in launches of well over one round of resident blocks
    // (about 7 per CU, 1792 on the chip): blocks that start once HBM is
    // saturated would otherwise idle through the SCAN's round trips, each
    // queued behind streaming traffic.  In smaller launches the early x flood
    // delays the SCAN instead.  Measured crossover: between 2048 blocks (after
    // the SCAN 1-3% faster) and 3072 (before COUNT 4% faster; 8-10% at 4096).
    // Self-summing launches whose slabs are at most 4 chunks request x once
    // COUNT is done and the SCAN's reads are out, before waiting for them:
    // the ids' round trip then runs without the x flood and the x loads
    // overlap the SCAN's (4096 tokens, one library per process, 3 rounds,
    // against x before COUNT: fp4x2 rows 16.06 -> 15.62 us, h2048 17.27 ->
    // 16.67, h1024 12.04 -> 11.59, fp8 rows at h4096 17.25 -> 16.62; x after
    // the SCAN was slower than both).  With 7- or 8-chunk slabs the order
    // between COUNT and the SCAN's wait was mixed (fp8 rows at h7168 1.7%
    // slower, 2000 tokens at h7168 1.5% faster), so they keep x after the
    // SCAN.  (A local scan requests every load up front anyway.)
    if (pl.local)
        pl.xOrder = kXOrderLate;
    else if (pl.selfScan && pl.cpw <= kXMidSelfCpw)
        pl.xOrder = kXOrderMid;
    else if (pl.nBlocks > kXEarlyBlocks)
        pl.xOrder = kXOrderEarly;
    else
        pl.xOrder = kXOrderLate;
    return pl;
}

// Launch geometry of a combine (gather or reduce, one row per token) or a
// push (one row per landing row): one wave per (row, slab of cpw 1 KiB
// chunks), 4 waves per block.
struct RowPlan {
    int32_t cpw;      // 1 KiB chunks per slab
    int32_t nSlabs;   // slabs per row
    int64_t waves;    // rows * nSlabs
    int64_t nBlocks;  // ceil(waves / 4)
    bool full;        // every slab lies inside the row: no per-lane bound checks
};

inline RowPlan row_plan(int64_t rows, int32_t rowBytes, int32_t cpw) {
    RowPlan pl{};
    const int32_t nChunks = ceil_div(rowBytes, kChunkBytes);
    pl.cpw = cpw;
    pl.nSlabs = ceil_div(nChunks, cpw);
    pl.waves = rows * pl.nSlabs;
    pl.nBlocks = (pl.waves + 3) / 4;
    pl.full = rowBytes % kChunkBytes == 0 && nChunks % cpw == 0;
    return pl;
}

inline RowPlan plan_combine(int32_t T, int32_t rowBytes) {
    // 2-chunk slabs when the row splits into them evenly and that still
    // leaves at least 8192 waves; 1-chunk slabs otherwise.
    const int32_t nChunks = ceil_div(rowBytes, kChunkBytes);
    const int32_t cpw = nChunks % 2 == 0 && (int64_t)T * (nChunks / 2) >= 8192 ? 2 : 1;
    return row_plan(T, rowBytes, cpw);
}

inline RowPlan plan_push(int32_t landRows, int32_t rowBytes) {
    // Slab width as in the dispatch: the widest of 8/7/4/2 chunks dividing a
    // whole-chunk row, else the narrowest width covering the row (8 beyond).
    const int32_t nChunks = ceil_div(rowBytes, kChunkBytes);
    int32_t cpw;
    if (rowBytes % kChunkBytes == 0)
        cpw = nChunks % 8 == 0 ? 8 : nChunks % 7 == 0 ? 7 : nChunks % 4 == 0 ? 4 : nChunks % 2 == 0 ? 2 : 1;
    else
        cpw = nChunks <= 1 ? 1 : nChunks <= 2 ? 2 : nChunks <= 4 ? 4 : nChunks <= 7 ? 7 : 8;
    return row_plan(landRows, rowBytes, cpw);
}

// Launchers: enqueue on `stream`, return the hipGetLastError() after launch.
hipError_t launch_dispatch(const DispatchParams &p, hipStream_t stream);

// Allocation-free dispatch: the library's own scratch, a 1 MiB device array
// per GPU (dispatch.hip).  dispatch_scratch_words gives the 32-bit words a
// dispatch of numTokens tokens to W PEs uses; static_scratch resolves (once
// per device, clearing it on `stream` that first time) the current device's
// copy.
constexpr int32_t kStaticScratchWords = 1 << 18;
int64_t dispatch_scratch_words(int32_t numTokens, int32_t W);
hipError_t static_scratch(uint32_t **out, hipStream_t stream);
hipError_t launch_combine(const CombineParams &p, bool fp32, bool out32, bool landing, hipStream_t stream);
hipError_t launch_combine_push(const PushParams &p, hipStream_t stream);

}  // namespace epdc
