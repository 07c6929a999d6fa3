// EP combine for gfx950: gather + weighted reduction, fp32 accumulate; a
// bf16 output rounded to nearest even, or the fp32 accumulator itself.
//
// MORI JIT v2 design doc, §5 and §9: the HIP backend's combine is a gather
// (each token pulls the rows its PEs returned); §3.7: combine sums, so it
// needs an arithmetic dtype (bf16 or fp32 rows here; §5: the HIP backend's
// combine outputs bf16 or fp32 -- chosen apart from the rows' type).  mori PR
// #599 "Perf/ep disp 1250 ship", item "meta prefetch": the gather's per-token
// metadata (token indices, weights) is loaded once, up front.
//
// One wave64 per (token, column slab of CPW 1 KiB chunks):
//   * lanes k < K load the token's K sendMap entries (and, weighted, its
//     expert ids and weights) once; a ballot over "sendMap >= 0" gives the
//     kept slots, i.e. the token's PEs in first-appearance order;
//   * lane k0 of a kept slot sums, in slot order from +0, the weights of the
//     slots on its PE (read from the other lanes by shuffles) -- once the
//     first group's rows are requested, so that the wait for the ids and
//     weights and this sum overlap those rows in flight (cold, against a
//     form whose ids and weights were waited for before the ballot: 4096
//     tokens x h7168 41.3 -> 40.2 us, h2048 14.93 -> 14.34; 16384 tokens
//     with uniform routing, ~5.3 rows a token, 237.9 -> 245.2, where fewer
//     rows in flight per CU are faster);
//   * the PE loop walks the kept slots in ascending order, a group of up to
//     kCombineGroup rows at a time: all of a group's row loads are issued
//     before its first FMA; every lane owns 16 contiguous bytes per chunk
//     (8 bf16 or 4 fp32 elements), one 16-byte access;
//   * the lane's elements go out as 16 bytes (bf16 rows to bf16 output, fp32
//     to fp32), 8 bytes (fp32 rows to bf16 output) or, for bf16 rows to an
//     fp32 output, two 16-byte stores, each instruction one contiguous 1 KiB:
//     there a lane loads two 8-byte pieces of the chunk, one from each half
//     (two 16-byte stores 32 bytes apart wrote partial lines: 7.7% more
//     write traffic than the output's size).
// The same kernel (LAND = true) is the reduce half of the scatter combine:
// the rows come from the packed landing rows the push wrote and each row's
// scale from the push's forwarded scales (combine_push.hip).
#include "epdc_internal.h"

namespace epdc {
namespace {

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ void fma8(float (&a)[8], float s, u32x4 v) {
    a[0] = __builtin_fmaf(s, bf16lo(v.x), a[0]);
    a[1] = __builtin_fmaf(s, bf16hi(v.x), a[1]);
    a[2] = __builtin_fmaf(s, bf16lo(v.y), a[2]);
    a[3] = __builtin_fmaf(s, bf16hi(v.y), a[3]);
    a[4] = __builtin_fmaf(s, bf16lo(v.z), a[4]);
    a[5] = __builtin_fmaf(s, bf16hi(v.z), a[5]);
    a[6] = __builtin_fmaf(s, bf16lo(v.w), a[6]);
    a[7] = __builtin_fmaf(s, bf16hi(v.w), a[7]);
}

// Loads chunks [slab*CPW, slab*CPW + CPW) of a row, 16 bytes per lane; with
// FULL every chunk is known to be inside the row (the row a whole number of
// 1 KiB chunks, the chunk count a multiple of CPW).
// SPLIT (bf16 rows, fp32 output): the lane's 16 bytes are instead bytes
// [8 lane, 8 lane + 8) of each half of the chunk, so that its 8 results are
// output elements 4 lane.. and 256 + 4 lane.. of the chunk: each of the two
// output stores is then one contiguous 1 KiB.
template <int CPW, bool FULL, bool SPLIT>
__device__ __forceinline__ void load_slab(u32x4 (&v)[CPW], const uint8_t *row, int slab, int nChunks,
                                          int rowBytes, int lane) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int gc = slab * CPW + c;
        if constexpr (SPLIT) {
            // Rows are whole 16-byte units, so a piece that starts inside
            // the row ends inside it.
            const int e0 = gc * kChunkBytes + lane * 8, e1 = e0 + kChunkBytes / 2;
            const u32x2 a = load8<kCombineNtLoad>(row + ((FULL || (gc < nChunks && e0 < rowBytes)) ? e0 : 0));
            const u32x2 b = load8<kCombineNtLoad>(row + ((FULL || (gc < nChunks && e1 < rowBytes)) ? e1 : 0));
            v[c] = u32x4{a.x, a.y, b.x, b.y};
        } else {
            const int e = gc * kChunkBytes + lane * 16;
            // A lane past the row's end loads the row's first 16 bytes (in
            // bounds; its sums are never stored): no branch or wait per load.
            v[c] = load16<kCombineNtLoad>(row + ((FULL || (gc < nChunks && e < rowBytes)) ? e : 0));
        }
    }
}

// acc += s * row for one lane's 16 bytes: 8 bf16 or 4 fp32 elements.
template <bool FP32>
__device__ __forceinline__ void fma_chunk(float (&a)[8], float s, u32x4 v) {
    if (FP32) {
        a[0] = __builtin_fmaf(s, __uint_as_float(v.x), a[0]);
        a[1] = __builtin_fmaf(s, __uint_as_float(v.y), a[1]);
        a[2] = __builtin_fmaf(s, __uint_as_float(v.z), a[2]);
        a[3] = __builtin_fmaf(s, __uint_as_float(v.w), a[3]);
    } else {
        fma8(a, s, v);
    }
}

// acc += sc[j] * row j for j = 0..N-1, in that order; all N rows' chunks are
// loaded first.  A scheduling barrier after each row's FMAs keeps the bf16
// unpacking of a row next to its use: left free, the scheduler unpacks
// several rows ahead and the extra registers cost occupancy (92 against 73
// VGPRs at 4 rows, 107 against 89 at 6).
// mid(sc) runs between the loads and the first FMA: it fills the group's
// scales (computing them first for the token's first group).
template <int N, int CPW, bool FULL, bool FP32, bool SPLIT, class Mid>
__device__ __forceinline__ void gather_reduce(float (&acc)[CPW][8], const CombineParams &P,
                                              const int32_t (&fl)[8], float (&sc)[8], int slab,
                                              int lane, Mid &mid) {
    u32x4 v[N][CPW];
#pragma unroll
    for (int j = 0; j < N; ++j)
        load_slab<CPW, FULL, SPLIT>(v[j], P.y + (int64_t)fl[j] * P.rowBytes, slab, P.nChunks, P.rowBytes, lane);
    mid(sc);
#pragma unroll
    for (int j = 0; j < N; ++j) {
#pragma unroll
        for (int c = 0; c < CPW; ++c) fma_chunk<FP32>(acc[c], sc[j], v[j][c]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// LAND = false: the gather combine over the returned rows y[W][M].
// LAND = true: the reduce half of the scatter combine over the landing rows
// (combine_push.hip), with the scale each landed row carries; same order,
// same arithmetic, so the same bits.
// FP32: fp32 returned rows (else bf16); OUT32: fp32 output (else bf16).
template <int CPW, bool FULL, bool FP32, bool OUT32, bool LAND>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams P, int nSlabs) {
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int32_t t = item / nSlabs;
    const int slab = item - t * nSlabs;
    if (t >= P.T) return;  // whole wave

    // Per-token metadata, one slot per lane; `flat` becomes the row index
    // into P.y of each kept slot and `s` its PE's scale.
    int32_t flat = -1;
    uint64_t kept;
    float s = 1.0f;
    int32_t eid = -1;  // the slot's expert id (its PE is derived once the rows are requested)
    float ew = 0.0f;
    bool scalesDue = !LAND && P.useWeights;
    if constexpr (LAND) {
        // Landing offsets: exclusive prefix sums of the counts (each clamped
        // to [0, M]) in PE order; rows at or past the landed total (or the
        // landing capacity) were never written and count as dropped.
        int32_t c = 0;
        if (lane < P.W) {
            c = P.recvCount[lane];
            c = c < 0 ? 0 : (c > P.M ? P.M : c);
        }
        const int32_t incl = wave_incl_scan(c);
        const int32_t landed = min(uniform(__shfl(incl, 63)), P.landRows);
        int32_t f = -1;
        if (lane < P.K) f = P.sendMap[(int64_t)t * P.K + lane];
        bool ok = lane < P.K && f >= 0 && f < P.W * P.M;
        const int32_t p = ok ? f / P.M : 0;
        const int32_t L = __shfl(incl - c, p) + (f - p * P.M);
        ok = ok && L < landed;
        kept = __ballot(ok);
        flat = L;
        if (P.useWeights && ok) s = P.landScale[L];
    } else {
        // The three loads go out back to back, unconditionally (an
        // unweighted call, whose ids and weights may be NULL, re-reads its
        // sendMap entry in their place), so that the ballot waits for
        // sendMap alone; the expert id stays raw until the scale step, which
        // runs once the first rows are requested.  (Deriving the PE here made
        // the compiled code wait for the ids and only then request the
        // weights: two round trips before the first row load.)
        if (lane < P.K) {
            const int64_t o = (int64_t)t * P.K + lane;
            const int32_t *ids = P.useWeights ? P.expertIds : P.sendMap;
            const float *wts = P.useWeights ? P.weights : reinterpret_cast<const float *>(P.sendMap);
            flat = P.sendMap[o];
            eid = ids[o];
            ew = wts[o];
        }
        // Kept slots; an entry outside [0, W*M) (not written by a dispatch
        // of this cfg) counts as dropped rather than being read out of bounds.
        kept = __ballot(lane < P.K && flat >= 0 && flat < P.W * P.M);
        // Scale of each kept slot's PE: sum of the token's weights on that
        // PE, in slot order starting from +0 (computed once the first
        // group's rows are requested).
    }

    constexpr bool kSplit = OUT32 && !FP32;
    float acc[CPW][8];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[c][j] = 0.0f;

    // PE loop over the kept slots in ascending order, in groups of up to
    // kGroup: every row of a group is requested before the first is reduced,
    // and the group is straight-line code, so each wait is for exactly one
    // row.  kGroup bounds the registers held by in-flight rows (and so sets
    // the occupancy).
    // The reduce over landing rows keeps groups of 4 (occupancy 6): on Zipf
    // routing (~3 PEs per token) it is 5% faster than with 8, though 6%
    // slower when tokens reach ~5 PEs (uniform routing); the gather is even
    // on the former and gains on the latter with 8.
    constexpr int kGroup = LAND ? 4 : kCombineGroup;
    uint64_t rem = kept;
    while (rem) {
        int32_t fl[8], ks[8];
        float sc[8];
        int n = 0;
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            const int k = rem ? __builtin_ctzll(rem) : 0;
            fl[j] = __builtin_amdgcn_readlane(flat, k);
            ks[j] = k;
            n += rem ? 1 : 0;
            rem &= rem - 1;
        }
        auto mid = [&](float (&scl)[8]) {
            if (scalesDue) {
                const int32_t E = P.W * P.Epr;
                int32_t epe = -1;
                // Keeps the id's first use (and so the wait for it) here,
                // behind the row loads, rather than hoisted above them.
                asm volatile("" : "+v"(eid));
                if (eid >= 0 && eid < E) epe = P.eprShift >= 0 ? (eid >> P.eprShift) : (eid / P.Epr);
                s = 0.0f;
                for (int k = 0; k < P.K; ++k) {
                    const int32_t pk = __shfl(epe, k);
                    const float wk = __shfl(ew, k);
                    if (k >= lane && epe >= 0 && pk == epe) s = s + wk;
                }
                scalesDue = false;
            }
#pragma unroll
            for (int j = 0; j < kGroup; ++j) scl[j] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(s), ks[j]));
        };
        switch (n) {
            case 1: gather_reduce<1, CPW, FULL, FP32, kSplit>(acc, P, fl, sc, slab, lane, mid); break;
            case 2: if constexpr (kGroup >= 2) gather_reduce<2, CPW, FULL, FP32, kSplit>(acc, P, fl, sc, slab, lane, mid); break;
            case 3: if constexpr (kGroup >= 3) gather_reduce<3, CPW, FULL, FP32, kSplit>(acc, P, fl, sc, slab, lane, mid); break;
            case 4: if constexpr (kGroup >= 4) gather_reduce<4, CPW, FULL, FP32, kSplit>(acc, P, fl, sc, slab, lane, mid); break;
            case 5: if constexpr (kGroup >= 5) gather_reduce<5, CPW, FULL, FP32, kSplit>(acc, P, fl, sc, slab, lane, mid); break;
            case 6: if constexpr (kGroup >= 6) gather_reduce<6, CPW, FULL, FP32, kSplit>(acc, P, fl, sc, slab, lane, mid); break;
            case 7: if constexpr (kGroup >= 7) gather_reduce<7, CPW, FULL, FP32, kSplit>(acc, P, fl, sc, slab, lane, mid); break;
            default: if constexpr (kGroup >= 8) gather_reduce<8, CPW, FULL, FP32, kSplit>(acc, P, fl, sc, slab, lane, mid); break;
        }
    }

    // The lane's elements start at element e / (bytes per row element) of
    // the row, so at byte e * (output element size / row element size) of
    // the output row.
    uint8_t *orow = P.out + (int64_t)t * P.outRowBytes;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int gc = slab * CPW + c;
        if constexpr (kSplit) {  // row bytes e0 / e1 -> output bytes 2 e0 / 2 e1
            const int e0 = gc * kChunkBytes + lane * 8, e1 = e0 + kChunkBytes / 2;
            if (FULL || (gc < P.nChunks && e0 < P.rowBytes))
                store16<kCombineNtStore>(orow + 2 * e0, u32x4{__float_as_uint(acc[c][0]), __float_as_uint(acc[c][1]),
                                                              __float_as_uint(acc[c][2]), __float_as_uint(acc[c][3])});
            if (FULL || (gc < P.nChunks && e1 < P.rowBytes))
                store16<kCombineNtStore>(orow + 2 * e1, u32x4{__float_as_uint(acc[c][4]), __float_as_uint(acc[c][5]),
                                                              __float_as_uint(acc[c][6]), __float_as_uint(acc[c][7])});
            continue;
        }
        const int e = gc * kChunkBytes + lane * 16;
        if (FULL || (gc < P.nChunks && e < P.rowBytes)) {
            if (FP32 && OUT32) {
                store16<kCombineNtStore>(orow + e, u32x4{__float_as_uint(acc[c][0]), __float_as_uint(acc[c][1]),
                                                         __float_as_uint(acc[c][2]), __float_as_uint(acc[c][3])});
            } else if (FP32) {  // 4 fp32 elements -> 8 bytes of bf16
                store8<kCombineNtStore>(orow + e / 2, u32x2{f32_to_bf16(acc[c][0]) | (f32_to_bf16(acc[c][1]) << 16),
                                                            f32_to_bf16(acc[c][2]) | (f32_to_bf16(acc[c][3]) << 16)});
            } else {
                store16<kCombineNtStore>(orow + e, u32x4{f32_to_bf16(acc[c][0]) | (f32_to_bf16(acc[c][1]) << 16),
                                                         f32_to_bf16(acc[c][2]) | (f32_to_bf16(acc[c][3]) << 16),
                                                         f32_to_bf16(acc[c][4]) | (f32_to_bf16(acc[c][5]) << 16),
                                                         f32_to_bf16(acc[c][6]) | (f32_to_bf16(acc[c][7]) << 16)});
            }
        }
    }
}

// Runs a plan (plan_combine in epdc_internal.h) with its compiled variant.
template <int CPW, bool FP32, bool OUT32, bool LAND>
hipError_t launch(const CombineParams &P, const RowPlan &pl, hipStream_t stream) {
    if (pl.waves > INT32_MAX - 3) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)pl.nBlocks);
    if (pl.full)
        hipLaunchKernelGGL((combine_kernel<CPW, true, FP32, OUT32, LAND>), grid, dim3(256), 0, stream, P, pl.nSlabs);
    else
        hipLaunchKernelGGL((combine_kernel<CPW, false, FP32, OUT32, LAND>), grid, dim3(256), 0, stream, P, pl.nSlabs);
    return hipGetLastError();
}

template <bool FP32, bool OUT32, bool LAND>
hipError_t launch_dtype(const CombineParams &P, hipStream_t stream) {
    const RowPlan pl = plan_combine(P.T, P.rowBytes);
    return pl.cpw == 2 ? launch<2, FP32, OUT32, LAND>(P, pl, stream) : launch<1, FP32, OUT32, LAND>(P, pl, stream);
}

template <bool LAND>
hipError_t launch_types(const CombineParams &P, bool fp32, bool out32, hipStream_t stream) {
    if (fp32)
        return out32 ? launch_dtype<true, true, LAND>(P, stream) : launch_dtype<true, false, LAND>(P, stream);
    return out32 ? launch_dtype<false, true, LAND>(P, stream) : launch_dtype<false, false, LAND>(P, stream);
}

}  // namespace

hipError_t launch_combine(const CombineParams &P, bool fp32, bool out32, bool landing, hipStream_t stream) {
    if (P.T == 0) return hipSuccess;
    return landing ? launch_types<true>(P, fp32, out32, stream) : launch_types<false>(P, fp32, out32, stream);
}

}  // namespace epdc
