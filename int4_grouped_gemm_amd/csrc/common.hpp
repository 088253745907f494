// Internal helpers shared by the HIP sources of the MoE layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lily_moe.h"

namespace lily {

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kGroup = 64;     // weights per (scale, bias) group
constexpr int kMaxExperts = 512;
constexpr int kMaxTopk = 64;
// The routing's sched array: kQueueInts words for the fused decode kernel's
// barrier, then the split-K tile counters of each GEMM (kTileCounters per
// GEMM), then each GEMM's queue counters and finished-workgroup counter
// (kQueueCtrs, one per 128-byte line: counters that share a line serialise
// their atomics; kCounterInts ints up to here), then the route's per-part
// expert histograms: kMaxParts rows of kMaxExperts counts and one arrival
// counter.
constexpr int kSchedInts = LILY_SCHED_INTS;
constexpr int kQueueInts = 32;
constexpr int kTileCounters = 512;
constexpr int kQueueLine = 32;  // ints per 128-byte cache line
constexpr int kQueueCtrs = 9;   // 8 XCD queues and the finished-workgroup count
constexpr int kQueueBase = kQueueInts + 2 * kTileCounters;
constexpr int kCounterInts = kQueueBase + 2 * kQueueCtrs * kQueueLine;
constexpr int kMaxParts = 64;
constexpr int kPartBase = kCounterInts;
static_assert(kPartBase + kMaxParts * kMaxExperts + 1 == kSchedInts, "sched layout");
// sched[28], sched[29]: the fused decode kernel's device-wide barrier
// (arrivals, exits); sched[30]: set if one of its barrier waits gave up.
constexpr int kDecodeBarrier = 28;
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor: raw, 32-bit data format
constexpr int kCoherentLoad = 16;       // buffer load/store cache policy: sc1 (device-coherent)
// sched[30], the give-up flag of every bounded device-wide wait (the decode
// kernels' barriers and exchanges, the one-launch FFN's block tallies):
// sticky, cleared by no launch, only by the caller.
constexpr int kGiveUpFlag = kDecodeBarrier + 2;

// Device buffers of the forward workspace.
struct ForwardWorkspace {
    uint16_t* h;  // bf16 [P + T, F]
    float* y;     // fp32 [P + T, H]
    float* part;  // split-K partial sums
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
    return __uint_as_float(h << 16);
}

// Two floats -> packed bf16x2 bits, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

// A wave-uniform pointer, made explicit so that it lives in SGPRs.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Host-side launch bookkeeping shared by the sources.
struct LaunchError {
    int code;
    const char* what;
};

size_t decode_workspace_bytes(const lily_moe_dims& d);  // 0 when T is too large

int trace_ffn_items(unsigned long long* dst, int max_wgs, hipStream_t stream);
int trace_decode_stack(unsigned long long* dst, int max_wgs, hipStream_t stream);

// Records the thread's last error text; returns code.
int set_error(int code, const char* fmt, ...);
int check_launch(const char* what);

}  // namespace lily
