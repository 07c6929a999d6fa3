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
constexpr bool kDispatchNtLoad = true;      // x rows: non-temporal loads
constexpr bool kDispatchNtStore = true;     // recvX rows: non-temporal, device-scope stores (store16_nt_dev)
constexpr bool kCombineNtLoad = true;       // returned rows: non-temporal loads
constexpr bool kCombineNtStore = true;      // out rows: non-temporal stores
constexpr bool kPushNtLoad = true;          // rows the push moves: non-temporal loads
constexpr bool kPushNtStore = true;         // landing rows: non-temporal stores
constexpr int kSelfScanBlocks = 1024;       // launches of up to this many blocks sum the tile counts in every block
constexpr int kSelfScanAnyCpw = 4;          // ... and launches of slabs of at most this many chunks, at any size
constexpr int kSelfScanWords = 8192;        //     while a block sums at most this many published words
constexpr int kWideFillBlocks = 7 * 256;   // wide-slab grids of this many blocks fill the GPU: 2-chunk slabs instead
constexpr int kOneTokenWaveBlocks = 16384; // launches of up to this many blocks move one token per wave
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

// Launch geometry of one dispatch, chosen from the token count, the row size
// and the world size (host code; the launcher runs exactly this plan, and a
// host test pins it for the documented shapes).
// The SCAN's form, a compile-time choice of the kernel (dispatch.hip, step
// 3): every block counts the earlier tiles' ids itself (local); every block
// sums the counts the tile leaders publish (self); or the tile leader sums
// them and publishes the tile's base rows, which its other blocks read
// (leader).
constexpr int kScanLocal = 0;
constexpr int kScanSelf = 1;
constexpr int kScanLeader = 2;

struct DispatchPlan {
    int32_t cpw;      // 1 KiB chunks per slab: 1, 2, 4, 7 or 8
    int32_t ntw;      // tokens per wave: 1, 2 or 4
    int32_t nSlabs;   // slabs per row
    int32_t nSubs;    // blocks per tile and slab (64 / (4 * ntw))
    int64_t nBlocks;  // grid size (0: no tokens, only recvCount is written)
    bool full;        // every slab lies inside the row: no per-lane bound checks
    int32_t scan;     // kScanLocal / kScanSelf / kScanLeader
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
    // exactly 7 chunks (fp8 rows at h7168, bf16 at h3584) in launches whose
    // 7-chunk slabs would pass kSelfScanBlocks take two bound-checked 4-chunk
    // slabs (4 + 3) instead, which keeps them under the self-summing SCAN
    // below (8192 fp8 tokens 52.1 -> 49.8 us; at 4096 tokens one 7-chunk
    // slab, already self-summing, is faster: 25.6 against 30.2).
    // Wide slabs (7 or 8 chunks) of a whole row of at least 8 chunks, an even
    // number, become 2-chunk slabs where the wide grid would fill every
    // block slot of the GPU at once (kWideFillBlocks: 256 CUs x 7 blocks, the
    // wide kernels' occupancy) and the 2-chunk grid still moves one token per
    // wave; such launches then sum the SCAN in every block (below) instead of
    // waiting on the tile leaders' line, and the later blocks of the longer
    // grid find the counts published when they start.  Cold x, one library
    // per process, 2 rounds, dispatch us: h7168 at 3584 / 4096 / 6144 / 8192
    // tokens 44.8 -> 41.1, 50.7 -> 45.8, 73.6 -> 66.7, 98.6 -> 87.0; fp32
    // rows (28 chunks) at 2048 / 4096 tokens 48.3 -> 44.7, 94.1 -> 85.0; h4096
    // at 8192 tokens 58.3 -> 53.0.  Below the fill point they lose (h7168 at
    // 2560 / 3072 tokens, 1280 / 1536 wide blocks: 29.2 -> 30.8, 34.8 -> 36.0;
    // fp32 rows at 1536 tokens 33.8 -> 34.9), and so do 1-chunk slabs (63.3
    // at 4096 tokens) and 2-chunk slabs with the leaders' line (63.3); at
    // 16384 tokens (28,672 2-chunk blocks) they were even (276.8 against
    // 276.1).
    int32_t wp = 1;
    while (wp < W) wp <<= 1;
    if (nTiles <= kNarrowTiles) {
        pl.cpw = nChunks <= 1 ? 1 : (!whole || nChunks % 2 == 0) ? 2 : 1;
    } else if (whole && nChunks == 7 && (int64_t)nTiles * (kTile / 4) > kSelfScanBlocks) {
        pl.cpw = 4;
    } else if (whole) {
        pl.cpw = nChunks % 8 == 0 ? 8 : nChunks % 7 == 0 ? 7 : nChunks % 4 == 0 ? 4 : nChunks % 2 == 0 ? 2 : 1;
        const int64_t perTile = kTile / 4;  // one-token-per-wave blocks per tile and slab
        if (pl.cpw > kSelfScanAnyCpw && nChunks >= 8 && nChunks % 2 == 0 &&
            (int64_t)nTiles * perTile * (nChunks / pl.cpw) >= kWideFillBlocks &&
            (int64_t)nTiles * perTile * (nChunks / 2) <= kOneTokenWaveBlocks && (int64_t)nTiles * wp <= kSelfScanWords)
            pl.cpw = 2;
    } else {
        pl.cpw = nChunks <= 1 ? 1 : nChunks <= 2 ? 2 : nChunks <= 4 ? 4 : nChunks <= 7 ? 7 : 8;
    }
    // Tokens per wave: one (most blocks, measured fastest at 4096 and 16384
    // tokens) unless that would exceed kOneTokenWaveBlocks blocks.
    const int64_t perTokenWave = (int64_t)nTiles * (kTile / 4) * ceil_div(nChunks, pl.cpw);
    pl.ntw = perTokenWave <= kOneTokenWaveBlocks ? 1 : perTokenWave <= 2 * kOneTokenWaveBlocks ? 2 : 4;
    pl.nSubs = kTile / (4 * pl.ntw);
    pl.nSlabs = ceil_div(nChunks, pl.cpw);
    pl.nBlocks = (int64_t)nTiles * pl.nSubs * pl.nSlabs;
    pl.full = whole && nChunks % pl.cpw == 0;
    // The local scan is built for one token per wave only: more tokens per
    // wave within 8 tiles takes over 128 slabs per row (rows of 128 KiB and
    // up), and its id registers would then cost occupancy; such launches scan
    // through the scratch.
    // Every block sums the earlier tiles' counts itself in launches of up to
    // 4 blocks per CU, where it saves a round trip (measured at 4096 tokens:
    // fp4x2 rows 2.6%, h2048 2.3%; 640 / 1024 tokens at h7168 5.3% / 3.6%).
    // In larger launches of 7- and 8-chunk slabs the tile leader's one
    // published line is faster (1.5% at 2048 blocks, 1.6% for fp8 rows at
    // 1536; every block summing at 16384 tokens: 7.5% slower).  One-token-
    // per-wave launches of slabs of at most 4 chunks sum in every block at
    // any size, while a block sums at most kSelfScanWords published words
    // (cold x, one library per process, 3 rounds, against the leader's line:
    // fp4x2 rows at 16384 tokens 57.4 -> 50.1 us, h2048 at 16384 tokens 63.2
    // -> 56.3, fp8 rows at 8192 tokens 60.3 -> 50.1).
    if (pl.ntw == 1 && nTiles <= kLocalScanTiles)
        pl.scan = kScanLocal;
    else if (pl.nBlocks <= kSelfScanBlocks ||
             (pl.cpw <= kSelfScanAnyCpw && pl.ntw == 1 && (int64_t)nTiles * wp <= kSelfScanWords))
        pl.scan = kScanSelf;
    else
        pl.scan = kScanLeader;
    // The x order goes with the SCAN form (dispatch.hip): a local scan
    // requests every load up front, the ids first; the other forms request
    // the x slabs before COUNT, with the ids ahead of them when every block
    // sums (a block counts sooner and its first poll finds the leaders'
    // counts; 4096 tokens, cold x: fp4x2 rows 16.16 -> 15.70 us, h2048
    // 17.55 -> 17.16) and behind them when the leaders publish (there
    // counting sooner only lengthens the wait for the leader's line: 4096
    // tokens x h7168 in 7-chunk slabs 50.84 against 51.63).  With x cold in
    // HBM every launch gains from requesting x before COUNT (the same launch
    // 55.4 -> 50.8 us; x after the SCAN, and x between COUNT and the SCAN's wait, were
    // tuned with x left in the memory-side cache by the previous call, where
    // they won).
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
