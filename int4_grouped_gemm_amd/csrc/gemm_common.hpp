// Pieces shared by the two grouped-GEMM kernels (gfx950): the kernel
// arguments, the schedule of work items over the XCD queues, the LDS swizzle,
// hand-counted memory waits and the global -> LDS DMA instructions.
#pragma once

#include "common.hpp"
#include "w4.hpp"

namespace lily {

struct GemmArgs {
    const uint16_t* a;              // A rows: gate/up -> x [T, K]; down -> h [P + T, K]
    const int32_t* sorted_pairs;    // gate/up: routed row r reads x[sorted_pairs[r] / topk]
    int topk;
    const char* w[2];               // packed routed stacks: gate/up -> gate, up; down -> W_down twice
    const char* sw[2];              // packed shared-expert stacks, same roles
    int N, K;
    const int4* block_info;         // per schedule position: expert, first row, rows, block
    const int32_t* num_blocks;
    int shared_blocks;  // ceil(T / BM)
    int P, T;
    int32_t* sched;     // queue_ctr(sched, q): the kXcds queue counters and (q = kXcds) finished workgroups
    uint16_t* h_out;    // gate/up: h [P + T, N] bf16
    float* y_out;       // down: y [P + T, N] fp32
    // Split K (small block maps): each tile's K runs as kc items of K / kc;
    // their fp32 partial sums go to part [kc][P + T][NP] (NP = 2N for
    // gate/up: g then u; N for down) and the item that finishes a tile, as
    // counted in tile_ctr [tiles], sums them in chunk order.
    int kc;
    float* part;
    int32_t* tile_ctr;
    // Gate/up and down in one launch: per schedule block, the gate/up tiles
    // that have stored their h rows; a down item of the block starts once
    // all of them have (blk_need tiles). NULL in the separate launches.
    int32_t* blk_done;
    int blk_need;
    int32_t* sched_flag;  // set if such a wait gave up
};

constexpr int kXcds = 8;        // MI355X: 8 XCDs of 32 CUs, each with its own L2
static_assert(kQueueCtrs == kXcds + 1, "a counter per queue and the finished count");
constexpr int kQueueChunk = 4;  // consecutive schedule blocks per queue turn

// Counter q (< kXcds: a queue; kXcds: the finished workgroups) of a GEMM's
// queue counters, each alone on its 128-byte line: every workgroup of a
// launch takes its items with atomics on them, and atomics on one line
// serialise (eight counters on one line cost a launch tens of microseconds).
__device__ __forceinline__ int32_t* queue_ctr(int32_t* sched, int q) { return sched + q * kQueueLine; }

// Output columns of one work item: the gate/up GEMM takes 128 features
// (128 gate and the same 128 up weight rows, so that SwiGLU is local to a
// lane), the down GEMM 256 rows of W_down. Either way two packed slabs.
template <bool GATED>
struct GemmShape {
    static constexpr int BN = GATED ? 128 : 256;
};

// The schedule (the shared expert's blocks, then the routed blocks in
// block_order) is dealt to kXcds queues in rounds of kXcds * kQueueChunk
// blocks. In each full round queue q takes kQueueChunk consecutive blocks
// (q*c .. q*c + c-1 of the round, c = kQueueChunk), so that most blocks of a
// hot expert meet its weight slabs in one XCD's L2. The blocks after the
// last full round (the smallest: block_order ends with the partial blocks)
// go one at a time, q, q + 8, ..., so that the queues' block counts differ
// by at most one (dealt in turns of c they differ by up to c, an eighth of
// a launch's items at T = 2048). Each block contributes n_tiles * kc
// consecutive items.
__device__ __forceinline__ int queue_items(int nb_total, int q, int per_block) {
    constexpr int round = kXcds * kQueueChunk;
    const int full = nb_total / round, rem = nb_total - full * round;
    return (full * kQueueChunk + (rem > q ? (rem - q + kXcds - 1) / kXcds : 0)) * per_block;
}
// Schedule position of the qi-th block of queue q.
__device__ __forceinline__ int queue_block(int nb_total, int q, int qi) {
    constexpr int round = kXcds * kQueueChunk;
    const int full = nb_total / round;
    if (qi < full * kQueueChunk) return ((qi / kQueueChunk) * kXcds + q) * kQueueChunk + qi % kQueueChunk;
    return full * round + (qi - full * kQueueChunk) * kXcds + q;
}

// LDS tiles of 64 bf16 per row ([rows][64]) store the 16-byte chunks of a
// row XOR-swizzled by ((row >> 1) & 7). The LDS has 64 four-byte banks, so a
// 16-lane phase of a 16-byte access covers 256 bytes: rows r and r + 1 of
// one chunk column already fall in different halves of the banks, and the
// swizzle spreads each half's eight rows over its eight chunk slots.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// s_waitcnt with only a vmcnt limit (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}
// Workgroup barrier without the memory fences of __syncthreads (which would
// drain every load in flight); the empty asm statements keep the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void barrier_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Global -> LDS load (gfx950 LDS DMA) with a wave-uniform 64-bit base in
// SGPRs and a 32-bit per-lane byte offset; lane l lands at LDS address
// m0 + l * size. The loads count in vmcnt like any vector memory load, but
// the compiler does not see them: their waits are counted by hand.
__device__ __forceinline__ void dma16(const void* base, uint32_t lane_off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane((int)lds_addr)), "v"(lane_off),
                    "s"(uniform_ptr(base)) : "memory");
}
// The same load, device-coherent (sc1): it reads data that another
// workgroup of the same launch wrote with device-coherent stores.
__device__ __forceinline__ void dma16_coh(const void* base, uint32_t lane_off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 sc1"
                 :: "s"(__builtin_amdgcn_readfirstlane((int)lds_addr)), "v"(lane_off),
                    "s"(uniform_ptr(base)) : "memory");
}
// A 16-byte store through to the device-coherent level (sc1), as the
// device-scope atomic stores are, at byte offset `off` of a buffer of
// `bytes` bytes. A buffer-store builtin rather than inline asm: the compiler
// then knows the store's data registers and keeps them intact until the
// store has read them (it cannot see into an asm statement).
__device__ __forceinline__ void store16_coherent(const void* base, uint32_t bytes, uint32_t off, u32x4 v) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(base)), 0, (int)bytes, kRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)off, 0, kCoherentLoad);
}
__device__ __forceinline__ void dma4(const void* base, uint32_t lane_off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane((int)lds_addr)), "v"(lane_off),
                    "s"(uniform_ptr(base)) : "memory");
}

}  // namespace lily
