// Internal interface between the host entry points (epdc_api.cpp) and the
// kernel launchers (dispatch.hip, combine.hip).  Not part of the C ABI.
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

// s_waitcnt vmcnt(N) with no lgkm/exp wait (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).  vmcnt counts loads and
// stores in issue order, so this waits until at most N of the wave's vector
// memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Routing tile: 64 tokens, one per lane of a wave64.
constexpr int kTile = 64;
// One 16-byte access per lane of a wave64 moves 512 bf16 elements (1 KiB).
constexpr int kChunkElems = 512;

struct DispatchParams {
    int32_t W, H, M, Epr, K, T, useWeights;
    int32_t Wp;        // W rounded up to a power of two (tile-count row stride)
    int32_t eprShift;  // log2(Epr) when Epr is a power of two, else -1
    int32_t nChunks;   // ceil(H / kChunkElems)
    const uint16_t *x;
    const int32_t *expertIds;
    const float *weights;
    uint16_t *recvX;
    int32_t *recvTokIdx;
    int32_t *recvExpertIds;
    float *recvWeights;
    int32_t *recvCount;
    int32_t *sendMap;
    int32_t *tileCount;  // scratch: [nTiles][Wp]
};

struct CombineParams {
    int32_t W, H, M, Epr, K, T, useWeights;
    int32_t eprShift;
    int32_t nChunks;
    const uint16_t *y;
    const int32_t *expertIds;
    const float *weights;
    const int32_t *sendMap;
    uint16_t *out;
};

inline int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

// Launchers: enqueue on `stream`, return the hipGetLastError() after launch.
hipError_t launch_dispatch(const DispatchParams &p, hipStream_t stream);
hipError_t launch_combine(const CombineParams &p, hipStream_t stream);

}  // namespace epdc
