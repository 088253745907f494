// Grouped expert GEMMs with the int4 -> bf16 dequantisation fused into the
// tile loads, SwiGLU, and the weighted gather-combine (gfx950).
//
// The Lily articles rebuild the 4-bit weights as bf16 tile by tile inside
// the grouped GEMM, keep them in on-chip memory and accumulate in FP32, so
// the expanded weights never reach main memory (news.ainew.jp Lily article,
// section "Prefill"). Here the on-chip memory is the LDS of a CDNA4 compute
// unit and the products run on bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// A tile is one (block, n-tile) pair of one expert:
//   rows  = a block of the block map (or of the shared expert's T rows);
//   cols  = BN outputs of the expert's weight matrix (for the gate/up GEMM,
//           BN columns of both gate and up, so that SwiGLU can be applied
//           in the epilogue).
// K runs in steps of 64 = one quantisation group per weight row, so each
// step needs one scale and one bias per row. Operands move global -> LDS by
// DMA a few steps ahead of use; each wavefront dequantises its own weights
// from LDS straight into MFMA operand registers. The weights are read in
// the packed layout of lily_w4_pack: the 128 rows x 64 k of a slab and
// group, with their scales and biases, are one contiguous 4608-byte block.
//
// The grid is persistent (as many workgroups as fit on the device) and
// takes tiles from eight work queues, one per XCD. The schedule (the shared
// expert's blocks, then the routed blocks in block_order, largest first,
// read resolved from block_info) is dealt to the queues mostly in turns of
// kQueueChunk consecutive blocks, so that most blocks of a hot expert meet
// its weight slabs in one XCD's L2; a block's n-tiles are consecutive, so
// that they meet the same A rows there too.
//
// LDS A tiles are [rows][64] bf16 with the chunk swizzle of gemm_common.hpp.
#include <algorithm>

#include "gemm_common.hpp"

namespace lily {

#ifdef LILY_TRACE_ITEMS
// Item trace of moe_w4_ffn, compiled into the tracing build of the library
// only (liblily_moe_trace.so). Per workgroup and item, in the order taken:
// the wall clock (s_memrealtime, 100 MHz) at its start and at its end (after
// its stores), what it was, and the ticks it waited for its block's gate/up
// tiles; slot kTraceSlots: the launch entry and exit, the items run and the
// grid size. Thread 0 of each workgroup writes its own rows.
constexpr int kTraceWgs = 1024, kTraceSlots = 32;
__device__ unsigned long long g_ffn_trace[kTraceWgs][kTraceSlots + 1][4];
__device__ unsigned long long g_ffn_wait[kTraceWgs];
#endif

// Tile geometry. A workgroup has 4 wavefronts that split the output columns;
// every wavefront covers all BM rows of the block. The workgroup owns 256
// weight rows, two packed slabs: for the gate/up GEMM slab n-tile of the
// gate matrix and the same slab of the up matrix (so SwiGLU is local to a
// lane), for the down GEMM slabs 2 n-tile and 2 n-tile + 1 of W_down.
// Wavefront w takes two groups of 32 weight rows: gate/up -> gate rows
// 32w.. and up rows 128+32w..; down -> rows 64w.. and 64w+32...
//
// Every operand travels global -> LDS with global_load_lds (no registers,
// no compiler-managed waits), NS k-steps in flight:
//   A stage  [BM rows][64 bf16], 16-byte chunks XOR-swizzled (swz);
//   Q stage  [2 halves][256 rows][16 B] of int4 weights;
//   SB stage the 256 scales, then the 256 biases of the step's group.
// Each lane then dequantises its own 32 weights of a k-step from LDS into
// MFMA operand registers (no weight is dequantised twice in a workgroup).
//
// K mapping inside a 64-wide k-step: lanes 0-31 (h = 0) hold k 0..31 and
// lanes 32-63 (h = 1) hold k 32..63; MFMA step s (16 k) pairs elements
// 8s..8s+7 of each half, for A and B alike. So a lane's A operand for step s
// is the 16-byte chunk 4h + s of its row.
constexpr int kGemmThreads = 256;

// Per tile height: k-steps in flight through LDS and wavefronts per SIMD.
// A single wavefront issues a VALU instruction only every few cycles, so the
// dequantisation throughput of a SIMD grows with the number of wavefronts it
// holds; 128-row tiles need ~250 VGPRs and hold 2.
template <int BM>
struct Occ {
    static constexpr int NS = BM >= 128 ? 3 : 2;
    static constexpr int WAVES_PER_SIMD = BM >= 128 ? 2 : (BM == 64 ? 3 : 4);
};

// LDS layout of a workgroup, per stage: the weights (Q: [2 halves][256
// rows][16 B]), the scales and biases (SB: [256] bf16 then [256] bf16) and
// the A tile ([BM rows][64 bf16]). All stage bases stay below 64 KB so they
// fit the immediate offset of ds_read.
//
// W4 = false is the unfused twin: the weights arrive as bf16 rows ([256
// rows][64 bf16], 16-byte chunks swizzled like A) and nothing is
// dequantised. Its stages are four times larger, so it keeps two stages
// and BM <= 64 (two workgroups per compute unit).
template <int BM, bool W4 = true>
struct Lds {
    static constexpr int NS = W4 ? Occ<BM>::NS : 2;
    static constexpr int Q = W4 ? 256 * 32 : 256 * 128;
    static constexpr int SB = W4 ? 256 * 2 * 2 : 0;
    static constexpr int A = BM * 128;
    static constexpr int Q_OFF = W4 ? 0 : NS * A;
    static constexpr int SB_OFF = Q_OFF + NS * Q;
    static constexpr int A_OFF = W4 ? SB_OFF + NS * SB : 0;
    static constexpr int TOTAL = NS * (A + Q + SB);
    static_assert(A_OFF + (NS - 1) * A < 65536 && Q_OFF + (NS - 1) * Q < 65536,
                  "stage bases must fit ds_read offsets");
};

// Next item of a work queue, the same value in every thread of the
// workgroup. Consecutive calls alternate between two LDS slots, so a slot is
// rewritten only after the barrier of the following call, which every
// wavefront reaches after reading it. Only LDS is waited for: DMA loads in
// flight stay in flight. (Taking the ticket one item ahead, to hide the
// atomic's latency, was slower: at the end of a launch the reserved items
// wait on busy workgroups while others idle.)
__device__ __forceinline__ int grab(int32_t* ctr, int* s_slot, int& toggle) {
    int* slot = s_slot + toggle;
    toggle ^= 1;
    if (threadIdx.x == 0) *slot = atomicAdd(ctr, 1);
    wait_lgkmcnt0();
    barrier_only();
    return __builtin_amdgcn_readfirstlane(*slot);
}

// One work item (a (block, n-tile) tile) and the load plan of one
// wavefront for it: the A row offsets of its DMA loads and the packed block
// of its weight slab at k-step 0 (+ kt * kPackBlock).
template <int MI, bool W4 = true>
struct Item {
    bool valid;
    bool prefetched;         // its first NS - 1 stages are already in flight
    int r0, rows, n0;
    int mia;                 // 32-row sub-tiles that hold rows: min(MI, ceil(rows / 32))
    int chunk, tile;         // K chunk of the item (split K) and its tile's counter index
    int vb;                  // schedule block
    bool down;               // a down item (the one-launch FFN only)
    const char* a_base;      // A rows: + kt * 128
    uint32_t a_off[MI];      // row byte offset + swizzled chunk
    const char* w_base;      // packed weights (W4), or the wavefront's bf16 matrix: + kt * 128
    uint32_t b_off[W4 ? 1 : 8];  // bf16 weights: row byte offset + swizzled chunk
};

// DMA of one k-step stage of an item by one wavefront: its n_a A loads
// (8 rows each, n_a <= MI), then half wh of weight slab wb (rows 0-63 and
// 64-127, 1 KB each) and the slab's 128 scales (wh = 0) or biases (wh = 1).
// N_DMA = n_a + 3 loads in all.
// The unfused twin (W4 = false) loads the wavefront's 64 bf16 weight rows
// instead: 8 loads of 8 rows. N_DMA = n_a + 8.
template <int BM, bool W4 = true, bool COH = false>
__device__ __forceinline__ void issue_stage(const Item<BM / 32, W4>& it, int n_a, int kt, int buf,
                                            uint32_t smem, uint32_t wave, int lane) {
    using Ld = Lds<BM, W4>;
#pragma unroll
    for (int j = 0; j < BM / 32; ++j)
        if (j < n_a) {
            const uint32_t dst = smem + Ld::A_OFF + buf * Ld::A + (32 * j + 8 * wave) * 128;
            if constexpr (COH) dma16_coh(it.a_base + kt * 128, it.a_off[j], dst);
            else dma16(it.a_base + kt * 128, it.a_off[j], dst);
        }
    if constexpr (!W4) {
        const uint32_t b_lds = smem + Ld::Q_OFF + buf * Ld::Q + 64u * wave * 128u;
#pragma unroll
        for (int j = 0; j < 8; ++j) dma16(it.w_base + kt * 128, it.b_off[j], b_lds + j * 8 * 128);
        return;
    }
    const uint32_t wh = wave & 1u, wb = wave >> 1;
    const uint32_t q_off = (wh * 128u + (uint32_t)lane) * 16u;
    const uint32_t sb_off = (uint32_t)kPackQ + wh * 256u + (uint32_t)lane * 4u;
    const uint32_t q_lds = smem + Ld::Q_OFF + buf * Ld::Q + (wh * 256u + wb * 128u) * 16u;
    const uint32_t sb_lds = smem + Ld::SB_OFF + buf * Ld::SB + wh * 512u + wb * 256u;
    const char* blk = it.w_base + (size_t)kt * kPackBlock;
    dma16(blk, q_off, q_lds);
    dma16(blk, q_off + 64 * 16, q_lds + 64 * 16);
    dma4(blk, sb_off, sb_lds);
}

// Waits (bounded) until the gate/up tiles of block vb have all stored
// their h rows; a wait that gives up sets sched[30].
__device__ __forceinline__ void wait_block_done(const GemmArgs& args, int vb) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(args.blk_done + vb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
           args.blk_need) {
        __builtin_amdgcn_s_sleep(2);
        if (__builtin_amdgcn_s_memrealtime() - t0 > 50000000ull) {  // 0.5 s at 100 MHz
            __hip_atomic_store(args.sched_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
#ifdef LILY_TRACE_ITEMS
    if (threadIdx.x == 0 && blockIdx.x < kTraceWgs)
        g_ffn_wait[blockIdx.x] += __builtin_amdgcn_s_memrealtime() - t0;
#endif
}

// Loads, multiplies and stores one tile. `prep_next` runs between the
// k-loop and the stores: it takes and resolves the workgroup's next item, so
// that the latency of its metadata loads overlaps the stores.
// FUSED (the one-launch FFN): a gate/up tile stores h device-coherently and
// then counts itself in blk_done; a down tile waits for that count before
// its first loads and reads h device-coherently.
template <int BM, bool GATED, int MIA, bool W4, bool FUSED, typename PrepNext>
__device__ __forceinline__ void gemm_main(const GemmArgs& args, char* smem_p,
                                          const Item<BM / 32, W4>& lp, uint32_t wave, int* s_flag,
                                          PrepNext&& prep_next) {
    using Ld = Lds<BM, W4>;
    constexpr int NS = Ld::NS;
    constexpr int NI = 2;
    constexpr int N_A = MIA;  // A loads per wavefront per k-step (8 rows each)
    constexpr int N_DMA = N_A + (W4 ? 3 : 8);
    static_assert(NS == 2 || NS == 3, "stage count");
    const uint32_t smem = (uint32_t)(size_t)smem_p;  // LDS byte address
    const int lane = threadIdx.x % kWave;
    const int h = lane / 32;
    const int nk = args.K / 64 / args.kc;  // k-steps of this item (a_base, w_base start at its chunk)
    const int r0 = lp.r0, rows = lp.rows;
    int brow[2], col0[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        brow[g] = GATED ? 128 * g + 32 * (int)wave + lane % 32 : 64 * (int)wave + 32 * g + lane % 32;
        col0[g] = GATED ? lp.n0 + 32 * (int)wave : lp.n0 + 64 * (int)wave + 32 * g;
    }

    auto issue = [&](int kt, int buf) {
        issue_stage<BM, W4, FUSED && !GATED>(lp, MIA, kt, buf, smem, wave, lane);
    };

    f32x16 acc[MIA][NI];
#pragma unroll
    for (int i = 0; i < MIA; ++i)
#pragma unroll
        for (int g = 0; g < NI; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][g][r] = 0.0f;

    // Per-lane LDS read offsets inside a stage. The swizzle depends on row
    // bits 1-3 only, so the 32-row sub-tiles i differ by a constant i * 4096.
    uint32_t a_rd[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int row = lane % 32;
        a_rd[s] = row * 128 + swz(row, 4 * h + s) * 16;
    }
    uint32_t q_rd[NI], sb_rd[NI], b_rd[NI][4];
#pragma unroll
    for (int g = 0; g < NI; ++g) {
        q_rd[g] = (h * 256 + brow[g]) * 16;
        sb_rd[g] = brow[g] * 2;
#pragma unroll
        for (int s = 0; s < 4; ++s) b_rd[g][s] = brow[g] * 128 + swz(brow[g], 4 * h + s) * 16;
    }

    // One k-step on stage buffer `buf` (a compile-time constant after the
    // loop below is unrolled by NS).
    auto step = [&](int kt, int buf) {
        if (NS == 2 || kt + 1 >= nk) wait_vmcnt<0>();
        else wait_vmcnt<N_DMA>();
        barrier_only();
        if (kt + NS - 1 < nk) issue(kt + NS - 1, (buf + NS - 1) % NS);

        const char* Ab = smem_p + Ld::A_OFF + buf * Ld::A;
        const char* Qb = smem_p + Ld::Q_OFF + buf * Ld::Q;
        const char* Sb = smem_p + Ld::SB_OFF + buf * Ld::SB;
        if constexpr (!W4) {
            // Unfused twin: the bf16 weight fragments are read from LDS like
            // the A fragments; nothing is dequantised.
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 af[MIA], bfr[NI];
#pragma unroll
                for (int i = 0; i < MIA; ++i)
                    af[i] = *reinterpret_cast<const bf16x8*>(Ab + i * 4096 + a_rd[s]);
#pragma unroll
                for (int g = 0; g < NI; ++g) bfr[g] = *reinterpret_cast<const bf16x8*>(Qb + b_rd[g][s]);
#pragma unroll
                for (int i = 0; i < MIA; ++i)
#pragma unroll
                    for (int g = 0; g < NI; ++g)
                        acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[g], af[i], acc[i][g], 0, 0, 0);
            }
            wait_lgkmcnt0();
            return;
        }
        if constexpr (MIA <= 2) {
            // Few rows: the step is bound by the dequantisation, so all
            // 4 x NI words of the step are rebuilt first, as independent
            // chains that the VALU can issue back to back, then the MFMAs
            // run on A fragments read meanwhile.
            u32x4 q[NI];
            float s512[NI], bias[NI];
#pragma unroll
            for (int g = 0; g < NI; ++g) {
                q[g] = *reinterpret_cast<const u32x4*>(Qb + q_rd[g]);
                s512[g] = bf16_bits_to_float(*reinterpret_cast<const uint16_t*>(Sb + sb_rd[g])) * 512.0f;
                bias[g] = bf16_bits_to_float(*reinterpret_cast<const uint16_t*>(Sb + 512 + sb_rd[g]));
            }
            bf16x8 af[4][MIA];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                for (int i = 0; i < MIA; ++i)
                    af[s4][i] = *reinterpret_cast<const bf16x8*>(Ab + i * 4096 + a_rd[s4]);
            bf16x8 bfr[4][NI];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                for (int g = 0; g < NI; ++g) {
                    uint32_t w[4];
                    dequant8(q[g][s4], s512[g], bias[g], w);
                    bfr[s4][g] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
                }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                for (int i = 0; i < MIA; ++i)
#pragma unroll
                    for (int g = 0; g < NI; ++g)
                        acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[s4][g], af[s4][i],
                                                                            acc[i][g], 0, 0, 0);
            wait_lgkmcnt0();
            return;
        }
        // Full tiles: the weights' LDS reads are issued first and each
        // sub-step's A fragments one sub-step ahead; the MFMAs of sub-step s
        // run while the weights of sub-step s + 1 are dequantised.
        u32x4 q[NI];
        uint16_t sbits[NI], bbits[NI];
#pragma unroll
        for (int g = 0; g < NI; ++g) {
            q[g] = *reinterpret_cast<const u32x4*>(Qb + q_rd[g]);
            sbits[g] = *reinterpret_cast<const uint16_t*>(Sb + sb_rd[g]);
            bbits[g] = *reinterpret_cast<const uint16_t*>(Sb + 512 + sb_rd[g]);
        }
        bf16x8 af[2][MIA];
#pragma unroll
        for (int i = 0; i < MIA; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(Ab + i * 4096 + a_rd[0]);
        float s512[NI], bias[NI];
#pragma unroll
        for (int g = 0; g < NI; ++g) {
            s512[g] = bf16_bits_to_float(sbits[g]) * 512.0f;
            bias[g] = bf16_bits_to_float(bbits[g]);
        }
        bf16x8 bfr[2][NI];
        auto dq = [&](int s, bf16x8* dst) {
#pragma unroll
            for (int g = 0; g < NI; ++g) {
                uint32_t w[4];
                dequant8(q[g][s], s512[g], bias[g], w);
                dst[g] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
            }
        };
        dq(0, bfr[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) {
#pragma unroll
                for (int i = 0; i < MIA; ++i)
                    af[(s + 1) & 1][i] = *reinterpret_cast<const bf16x8*>(Ab + i * 4096 + a_rd[s + 1]);
                dq(s + 1, bfr[(s + 1) & 1]);
            }
#pragma unroll
            for (int i = 0; i < MIA; ++i)
#pragma unroll
                for (int g = 0; g < NI; ++g)
                    acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[s & 1][g], af[s & 1][i], acc[i][g], 0, 0, 0);
        }
        // Issue order for the scheduler: the weights' reads and sub-step 0's
        // A reads, the scale/bias conversion and sub-step 0's dequantisation;
        // then per sub-step the next A reads and each MFMA followed by a
        // share of the next sub-step's dequantisation.
        constexpr int kMfmaPerSub = MIA * NI;
        constexpr int kDqValu = 19 * NI;
        constexpr int kValuPerMfma = (kDqValu + kMfmaPerSub - 1) / kMfmaPerSub;
        __builtin_amdgcn_sched_group_barrier(0x100, 3 * NI + MIA, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4 * NI + kDqValu, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) __builtin_amdgcn_sched_group_barrier(0x100, MIA, 0);
#pragma unroll
            for (int m = 0; m < kMfmaPerSub; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (s < 3) __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
            }
        }
        wait_lgkmcnt0();  // this wavefront's LDS reads of the stage are done
    };

    if (!lp.prefetched) {
        if constexpr (FUSED && !GATED) wait_block_done(args, lp.vb);
        issue(0, 0);
        if (NS == 3 && nk > 1) issue(1, 1);
    }
    // Whole rounds of NS steps, then the remaining steps (buffers 0, 1, ..):
    // no step of the main loop is conditional, so the accumulators keep
    // their registers across the back edge.
    int kt = 0;
    for (; kt + NS <= nk; kt += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) step(kt + u, u);
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
        if (kt + u < nk) step(kt + u, u);

    prep_next();

    // The MFMAs take the weights as their first operand and the A rows as the
    // second, so lane l, register r of tile (i, g) holds output row
    // 32 i + l % 32 and column col0[g] + 8 (r / 4) + 4 (l / 32) + r % 4: four
    // consecutive columns per group of four registers, stored together.
    const int x = lane % 32;
    if (args.kc > 1) {
        // Split K: publish this chunk's partial sums; the item that
        // completes the tile (the kc-th to arrive at its counter) adds all
        // chunks in chunk order, so the result does not depend on which
        // workgroup finishes last.
        const int np = GATED ? 2 * args.N : args.N;
        const size_t chunk_stride = (size_t)(args.P + args.T) * np;
#pragma unroll
        for (int i = 0; i < MIA; ++i) {
            const int row = 32 * i + x;
            if (row >= rows) continue;
            float* prow = args.part + lp.chunk * chunk_stride + (size_t)(r0 + row) * np;
#pragma unroll
            for (int g = 0; g < NI; ++g)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    __hip_atomic_store(prow + (GATED ? g * args.N + col0[0] : col0[g]) + 8 * (r / 4) + 4 * h + r % 4,
                                       acc[i][g][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // The partials are device-coherent stores (they write through the
        // XCD's L2). Every wavefront waits for its own stores to complete
        // before the barrier (a workgroup barrier alone does not wait for
        // global stores), so all of them are complete before the chunk
        // counts in; they are read back with device-coherent loads. No
        // fence, which on this GPU would write back the whole L2.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0)
            *s_flag = __hip_atomic_fetch_add(args.tile_ctr + lp.tile, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(*s_flag) != args.kc - 1) return;
#pragma unroll
        for (int i = 0; i < MIA; ++i) {
            const int row = 32 * i + x;
            if (row >= rows) continue;
            const float* prow = args.part + (size_t)(r0 + row) * np;
#pragma unroll
            for (int g = 0; g < NI; ++g)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int col = (GATED ? g * args.N + col0[0] : col0[g]) + 8 * (r / 4) + 4 * h + r % 4;
                    float sum = 0.0f;
                    for (int c = 0; c < args.kc; ++c)
                        sum += __hip_atomic_load(prow + c * chunk_stride + col, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                    acc[i][g][r] = sum;
                }
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(args.tile_ctr + lp.tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    if constexpr (!GATED && NS == 3) {
        // y through LDS, so that every store writes whole 128-byte lines: in
        // the MFMA layout a 16-byte store covers 32 rows with 32 bytes each,
        // and y's partial-line writes cost the launch ~5% (T = 2048) to 7%
        // (T = 8192). Each wavefront turns its own 64 columns around in a
        // private 4 KB of the third stage buffer (free: the next item's
        // prefetch fills the first two, and its first step's barrier comes
        // before that buffer is loaded again), 16 rows at a time: the lanes
        // write their 16-byte chunks (chunk index XOR-swizzled by the row
        // against bank conflicts), then each lane reads one chunk of four
        // rows and one store covers 4 rows x 256 bytes. A wavefront's LDS
        // accesses run in order, so no barrier and no wait is needed between
        // its writes and reads.
        char* const tb = smem_p + Ld::A_OFF + 2 * Ld::A + (int)wave * 4096;
        const int c = lane % 16, rq = lane / 16;
        const int y16 = lane % 16, q0 = (lane / 16) % 2;
        float* const ybase = args.y_out + lp.n0 + 64 * (int)wave + 4 * c;
#pragma unroll
        for (int i = 0; i < MIA; ++i) {
            // One v_permlane16_swap per register pairs column groups 2 q1 and
            // 2 q1 + 1: then set 0 holds rows 0-15 of the sub-tile and set 1
            // rows 16-31, lane l holding row l % 16 at column group 4 q1 +
            // 2 q0 + h (q0 = l / 16 % 2), so that all 64 lanes write each band.
            // (__float_as_uint, not __builtin_bit_cast: a bit_cast of a
            // vector element compiles to a read of element 0 here.)
            f32x4 band[2][NI][2];
#pragma unroll
            for (int g = 0; g < NI; ++g)
#pragma unroll
                for (int q1 = 0; q1 < 2; ++q1)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const auto sw = __builtin_amdgcn_permlane16_swap(
                            __float_as_uint(acc[i][g][8 * q1 + e]), __float_as_uint(acc[i][g][8 * q1 + 4 + e]),
                            false, false);
                        band[0][g][q1][e] = __uint_as_float((uint32_t)sw[0]);
                        band[1][g][q1][e] = __uint_as_float((uint32_t)sw[1]);
                    }
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int g = 0; g < NI; ++g)
#pragma unroll
                    for (int q1 = 0; q1 < 2; ++q1)
                        *reinterpret_cast<f32x4*>(tb + y16 * 256 + ((8 * g + 4 * q1 + 2 * q0 + h) ^ y16) * 16) =
                            band[hf][g][q1];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int rr = 4 * k + rq, row = 32 * i + 16 * hf + rr;
                    const f32x4 v = *reinterpret_cast<const f32x4*>(tb + rr * 256 + (c ^ rr) * 16);
                    if (row < rows) *reinterpret_cast<f32x4*>(ybase + (size_t)(r0 + row) * args.N) = v;
                }
            }
        }
        return;
    }
    if constexpr (!GATED) {
        // y of the shorter tiles (two stages: no free stage buffer to turn
        // it around in), in half lines: one v_permlane16_swap per register
        // pairs column groups 2 q1 and 2 q1 + 1, after which the first set
        // holds rows 0-15 of the sub-tile and the second rows 16-31, each row
        // in four lanes (l / 16 = 2 h + q0) with 64 contiguous bytes.
        const int y16 = lane % 16, q0 = (lane / 16) % 2;
#pragma unroll
        for (int i = 0; i < MIA; ++i)
#pragma unroll
            for (int g = 0; g < NI; ++g)
#pragma unroll
                for (int q1 = 0; q1 < 2; ++q1) {
                    f32x4 lo, hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // (__float_as_uint, not __builtin_bit_cast: a bit_cast of
                        // a vector element compiles to a read of element 0 here)
                        const auto sw = __builtin_amdgcn_permlane16_swap(
                            __float_as_uint(acc[i][g][8 * q1 + e]), __float_as_uint(acc[i][g][8 * q1 + 4 + e]),
                            false, false);
                        lo[e] = __uint_as_float((uint32_t)sw[0]);
                        hi[e] = __uint_as_float((uint32_t)sw[1]);
                    }
                    const int col = col0[g] + 16 * q1 + 8 * q0 + 4 * h;
                    const int row_lo = 32 * i + y16, row_hi = row_lo + 16;
                    if (row_lo < rows)
                        *reinterpret_cast<f32x4*>(args.y_out + (size_t)(r0 + row_lo) * args.N + col) = lo;
                    if (row_hi < rows)
                        *reinterpret_cast<f32x4*>(args.y_out + (size_t)(r0 + row_hi) * args.N + col) = hi;
                }
        return;
    }
    // Epilogue: h, 16 bytes per store. In the MFMA layout lanes x and x + 32
    // hold row x, four features each per column group q; one
    // v_permlane32_swap per pair of registers gathers features 8 q .. 8 q + 7
    // of groups q = 2 q1 (lane x) and 2 q1 + 1 (lane x + 32) in one lane
    // each, so that a store writes 32 rows x 32 contiguous bytes instead of
    // 32 rows x 16 bytes.
    const uint32_t h_bytes = (uint32_t)((size_t)(args.P + args.T) * args.N * 2);
#pragma unroll
    for (int i = 0; i < MIA; ++i) {
        const int row = 32 * i + x;
        const uint32_t hoff = (uint32_t)(((size_t)(r0 + row) * args.N + col0[0] + 8 * h) * 2);
        uint16_t* const hrow = args.h_out + (size_t)(r0 + row) * args.N + col0[0] + 8 * h;
#pragma unroll
        for (int q1 = 0; q1 < 2; ++q1) {
            uint32_t w[2][2];  // [q - 2 q1][features 0-1, 2-3]
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int q = 2 * q1 + k;
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = silu(acc[i][0][4 * q + j]) * acc[i][1][4 * q + j];
                w[k][0] = pack_bf16x2(v[0], v[1]);
                w[k][1] = pack_bf16x2(v[2], v[3]);
            }
            const auto s0 = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
            const u32x4 out = {(uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]};
            if (row < rows) {
                if constexpr (FUSED) store16_coherent(args.h_out, h_bytes, hoff + 32 * q1, out);
                else *reinterpret_cast<u32x4*>(hrow + 16 * q1) = out;
            }
        }
    }
    if constexpr (FUSED && GATED) {
        // Every wavefront's h stores have reached the device-coherent level
        // before the tile counts itself in its block's tally.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier_only();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(args.blk_done + lp.vb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Resolves the rows, expert and load plan of tile (vb, nt), K chunk `chunk`,
// of one GEMM for this wavefront (one load of block_info).
template <int BM, bool GATED, bool W4>
__device__ __forceinline__ void resolve_item(const GemmArgs& args, int vb, int nt, int chunk,
                                             uint32_t wave, int lane, Item<BM / 32, W4>& it) {
    constexpr int BN = GemmShape<GATED>::BN;
    constexpr int MI = BM / 32;
    const int n_tiles = args.N / BN;
    const int n_slabs = args.N / kPackRows;
    const size_t slab_bytes = (size_t)(args.K / 64) * kPackBlock;
    it.chunk = chunk;
    it.vb = vb;
    it.tile = vb * n_tiles + nt;
    int e = 0;
    bool shared;
    if (vb < args.shared_blocks) {
        it.r0 = args.P + vb * BM;
        it.rows = min(BM, args.P + args.T - it.r0);
        shared = true;
    } else {
        const int4 info = args.block_info[vb - args.shared_blocks];
        e = info.x;
        it.r0 = info.y;
        it.rows = info.z;
        shared = false;
    }
    it.mia = min(MI, (it.rows + 31) / 32);
    it.prefetched = false;
    it.n0 = nt * BN;
    // A loads: load j of wavefront w fills LDS rows 32j + 8w + lane/8,
    // physical chunk lane%8, which holds logical chunk swz(row, lane%8).
    // Rows past the block read the block's first row: their products land
    // in output rows that are never stored.
    const int kt0 = chunk * (args.K / 64 / args.kc);  // first k-step of the chunk
    it.a_base = reinterpret_cast<const char*>(args.a) + kt0 * 128;
#pragma unroll
    for (int j = 0; j < MI; ++j) {
        const int row = 32 * j + 8 * (int)wave + lane / 8;
        const int r = it.r0 + (row < it.rows ? row : 0);
        int src_row = r;
        if (GATED) src_row = (r < args.P) ? args.sorted_pairs[r] / args.topk : r - args.P;
        it.a_off[j] = (uint32_t)src_row * (uint32_t)(args.K * 2) + (uint32_t)(swz(row, lane % 8) * 16);
    }
    // Weight slab wb = wave / 2 of the workgroup: gate/up -> slab nt of the
    // gate (wb = 0) or up (wb = 1) stack; down -> slab 2 nt + wb.
    const int wb = (int)(wave >> 1);
    const char* stack = shared ? args.sw[GATED ? wb : 0] : args.w[GATED ? wb : 0];
    if constexpr (W4) {
        const int slab = GATED ? nt : 2 * nt + wb;
        it.w_base = stack + ((size_t)e * n_slabs + slab) * slab_bytes + (size_t)kt0 * kPackBlock;
    } else {
        // bf16 [n][N][K] stacks: the wavefront loads the workgroup's weight
        // rows 64 w .. 64 w + 63 (LDS rows, swizzled like A): gate/up -> row
        // n0 + (64 w + i) % 128 of the gate or up matrix; down -> row
        // n0 + 64 w + i.
        it.w_base = stack + (size_t)e * args.N * args.K * 2 + (size_t)kt0 * 128;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int lrow = 64 * (int)wave + 8 * j + lane / 8;
            const int n = it.n0 + (GATED ? lrow % 128 : lrow);
            it.b_off[j] = (uint32_t)n * (uint32_t)(args.K * 2) + (uint32_t)(swz(lrow, lane % 8) * 16);
        }
    }
    it.down = !GATED;
    it.valid = true;
}

template <int BM, bool GATED, bool W4 = true>
__global__ void __launch_bounds__(kGemmThreads, W4 ? Occ<BM>::WAVES_PER_SIMD : 2)
    moe_w4_gemm(GemmArgs args) {
    constexpr int BN = GemmShape<GATED>::BN;
    constexpr int MI = BM / 32;
    __shared__ __attribute__((aligned(16))) char smem[Lds<BM, W4>::TOTAL];
    __shared__ int s_slot[3];  // two alternating queue slots, the split-K arrival count

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);

    // Work queue x = blockIdx.x % 8: with round-robin dispatch of workgroups
    // over the XCDs all of a queue's workgroups share one L2. A workgroup
    // drains its own queue; each item is taken exactly once through the
    // queue's counter. Correctness does not depend on the XCD mapping.
    // (Taking items from other queues once the own queue is empty costs
    // more than the imbalance it removes: the idle workgroups all contend
    // for the last counters.)
    const int n_tiles = args.N / BN;
    const int nb_total = args.shared_blocks + args.num_blocks[0];
    const int cq = blockIdx.x % kXcds;
    int toggle = 0;

    // Items of queue q: its blocks times the n-tiles times the K chunks (the
    // chunks of a tile consecutive), dealt as queue_items describes.
    auto items_of = [&](int q) { return queue_items(nb_total, q, n_tiles * args.kc); };
    // Takes the next item of queue cq (one atomic) and resolves its rows,
    // expert and load plan (one load of block_info); it.valid = false if the
    // queue is empty.
    auto take = [&](Item<MI, W4>& it) {
        it.valid = false;
        const int c = grab(queue_ctr(args.sched, cq), s_slot, toggle);
        if (c >= items_of(cq)) return;
        const int ct = c / args.kc;  // tile of the queue
        resolve_item<BM, GATED, W4>(args, queue_block(nb_total, cq, ct / n_tiles), ct % n_tiles, c - ct * args.kc,
                                    wave, lane, it);
    };
    // Every decision follows a value that grab() sent through LDS, so all
    // wavefronts take the same path and meet at the same barriers.
    const uint32_t smem_addr = (uint32_t)(size_t)smem;
    Item<MI, W4> cur;
    take(cur);
    while (cur.valid) {
        Item<MI, W4> nxt;
        // After the k-loop (every wavefront is done with the LDS stages):
        // take the next item and start its first stages, so that their
        // latency overlaps this tile's stores.
        auto prep = [&]() {
            take(nxt);
            if (nxt.valid) {
#pragma unroll
                for (int u = 0; u < Lds<BM, W4>::NS - 1; ++u)
                    if (u < args.K / 64 / args.kc) issue_stage<BM, W4>(nxt, nxt.mia, u, u, smem_addr, wave, lane);
                nxt.prefetched = true;
            }
        };
        // Only the 32-row sub-tiles that hold rows of the block are loaded
        // and multiplied.
        const int mia = cur.mia;
        if (mia >= MI) gemm_main<BM, GATED, MI, W4, false>(args, smem, cur, wave, s_slot + 2, prep);
        else if (mia == 1) gemm_main<BM, GATED, 1, W4, false>(args, smem, cur, wave, s_slot + 2, prep);
        else if (mia == 2)
            gemm_main<BM, GATED, (MI > 2 ? 2 : 1), W4, false>(args, smem, cur, wave, s_slot + 2, prep);
        else gemm_main<BM, GATED, (MI > 3 ? 3 : 1), W4, false>(args, smem, cur, wave, s_slot + 2, prep);
        cur = nxt;
    }

    // A workgroup gets here once every queue has run out, so when the last
    // one arrives every item has been taken; it clears the counters for the
    // next launch.
    if (tid == 0 && atomicAdd(queue_ctr(args.sched, kXcds), 1) == (int)gridDim.x - 1) {
        for (int i = 0; i <= kXcds; ++i) atomicExch(queue_ctr(args.sched, i), 0);
    }
}

// Gate/up and down in one launch (no split K). Queue q takes its gate/up
// items, then its down items (the same blocks, dealt the same way), from
// one counter, so a workgroup whose gate/up work has run out starts on down
// tiles while the last gate/up tiles finish elsewhere, instead of idling
// until a second launch. A down item waits until its block's gate/up tiles
// have counted in; they were all taken before it from the same counter, by
// workgroups that are running and wait on nothing, so the wait ends. Those
// h rows are stored and read device-coherently, because producer and
// consumer may sit on different XCDs (each with its own L2).
template <int BM>
__global__ void __launch_bounds__(kGemmThreads, Occ<BM>::WAVES_PER_SIMD)
    moe_w4_ffn(GemmArgs gu, GemmArgs dn) {
    constexpr int MI = BM / 32;
    constexpr int NS = Lds<BM, true>::NS;
    __shared__ __attribute__((aligned(16))) char smem[Lds<BM, true>::TOTAL];
    __shared__ int s_slot[3];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nb_total = gu.shared_blocks + gu.num_blocks[0];
    const int nt_gu = gu.N / GemmShape<true>::BN, nt_dn = dn.N / GemmShape<false>::BN;
    const int cq = blockIdx.x % kXcds;
    const int n_gu = queue_items(nb_total, cq, nt_gu);
    const int n_dn = queue_items(nb_total, cq, nt_dn);
    int toggle = 0;
    auto take = [&](Item<MI, true>& it) {
        it.valid = false;
        int c = grab(queue_ctr(gu.sched, cq), s_slot, toggle);
        if (c < n_gu) {
            resolve_item<BM, true, true>(gu, queue_block(nb_total, cq, c / nt_gu), c % nt_gu, 0, wave, lane, it);
        } else if ((c -= n_gu) < n_dn) {
            resolve_item<BM, false, true>(dn, queue_block(nb_total, cq, c / nt_dn), c % nt_dn, 0, wave, lane, it);
        }
    };
    const uint32_t smem_addr = (uint32_t)(size_t)smem;
#ifdef LILY_TRACE_ITEMS
    const unsigned long long t_entry = __builtin_amdgcn_s_memrealtime();
    const bool traced = tid == 0 && blockIdx.x < kTraceWgs;
    unsigned long long(*trace)[4] = g_ffn_trace[blockIdx.x < kTraceWgs ? blockIdx.x : 0];
    int n_run = 0;
    if (traced) g_ffn_wait[blockIdx.x] = 0;
#endif
    Item<MI, true> cur;
    take(cur);
    while (cur.valid) {
#ifdef LILY_TRACE_ITEMS
        if (traced && n_run < kTraceSlots) {
            trace[n_run][0] = __builtin_amdgcn_s_memrealtime();
            trace[n_run][2] = (unsigned long long)cur.mia | ((unsigned long long)cur.down << 8) |
                              ((unsigned long long)cur.n0 << 16) |
                              ((unsigned long long)cur.vb << 32);
            trace[n_run][3] = g_ffn_wait[blockIdx.x];
        }
#endif
        Item<MI, true> nxt;
        // As in the separate launches; a down item's first stages are
        // prefetched only if its block is already complete.
        auto prep = [&]() {
            take(nxt);
            if (nxt.valid &&
                (!nxt.down || __hip_atomic_load(dn.blk_done + nxt.vb, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) >= dn.blk_need)) {
#pragma unroll
                for (int u = 0; u < NS - 1; ++u) {
                    if (u >= gu.K / 64 && !nxt.down) continue;
                    if (u >= dn.K / 64 && nxt.down) continue;
                    if (nxt.down) issue_stage<BM, true, true>(nxt, nxt.mia, u, u, smem_addr, wave, lane);
                    else issue_stage<BM, true, false>(nxt, nxt.mia, u, u, smem_addr, wave, lane);
                }
                nxt.prefetched = true;
            }
        };
        const int mia = cur.mia;
        if (!cur.down) {
            if (mia >= MI) gemm_main<BM, true, MI, true, true>(gu, smem, cur, wave, s_slot + 2, prep);
            else if (mia == 1) gemm_main<BM, true, 1, true, true>(gu, smem, cur, wave, s_slot + 2, prep);
            else if (mia == 2)
                gemm_main<BM, true, (MI > 2 ? 2 : 1), true, true>(gu, smem, cur, wave, s_slot + 2, prep);
            else gemm_main<BM, true, (MI > 3 ? 3 : 1), true, true>(gu, smem, cur, wave, s_slot + 2, prep);
        } else {
            if (mia >= MI) gemm_main<BM, false, MI, true, true>(dn, smem, cur, wave, s_slot + 2, prep);
            else if (mia == 1) gemm_main<BM, false, 1, true, true>(dn, smem, cur, wave, s_slot + 2, prep);
            else if (mia == 2)
                gemm_main<BM, false, (MI > 2 ? 2 : 1), true, true>(dn, smem, cur, wave, s_slot + 2, prep);
            else gemm_main<BM, false, (MI > 3 ? 3 : 1), true, true>(dn, smem, cur, wave, s_slot + 2, prep);
        }
#ifdef LILY_TRACE_ITEMS
        if (traced && n_run < kTraceSlots) {
            trace[n_run][1] = __builtin_amdgcn_s_memrealtime();
            trace[n_run][3] = g_ffn_wait[blockIdx.x] - trace[n_run][3];
        }
        ++n_run;
#endif
        cur = nxt;
    }
#ifdef LILY_TRACE_ITEMS
    if (traced) {
        trace[kTraceSlots][0] = t_entry;
        trace[kTraceSlots][1] = __builtin_amdgcn_s_memrealtime();
        trace[kTraceSlots][2] = (unsigned long long)n_run;
        trace[kTraceSlots][3] = gridDim.x;
    }
#endif

    // The last workgroup to get here (every item taken and finished) clears
    // the queue counters and the block tallies for the next launch.
    if (tid == 0) s_slot[2] = atomicAdd(queue_ctr(gu.sched, kXcds), 1) == (int)gridDim.x - 1;
    __syncthreads();
    if (s_slot[2]) {
        for (int i = tid; i < nb_total; i += kGemmThreads)
            __hip_atomic_store(gu.blk_done + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid <= kXcds) atomicExch(queue_ctr(gu.sched, tid), 0);
    }
}

// 16-row tiles (tile_m 16): the tile height the Lily articles start from
// (news.ainew.jp Lily article, section "Prefill", 16 against 32 rows per
// threadgroup tile). A block of <= 16 rows against the same 256 weight rows
// of two packed slabs as the taller tiles, on v_mfma_f32_16x16x32_bf16:
// the weights are the first operand (16 rows x 32 k), the block's rows the
// second. A wavefront holds 16 accumulators (4 groups of 16 weight rows x
// 16 tokens), so four wavefronts fit per SIMD, which is what the
// dequant-bound small blocks want; the dequantisation per k-step and
// workgroup is the same 256 x 64 weights as in the taller tiles.
//
// K mapping inside a 64-wide k-step: MFMA m (0, 1) of lane quarter q =
// lane / 16 takes k 16q + 8m .. 16q + 8m + 7, for both operands. So a lane
// reads 8 bytes of int4 per weight row (k 16q .. 16q + 15, one ds_read_b64
// from half q / 2 of the packed row) and 16-byte A chunks 2q and 2q + 1.
// Weight groups of wavefront w: gate/up -> gate rows 32w, 32w + 16 and the
// same up rows (SwiGLU local to a lane); down -> rows 64w + 16g.
struct Lds16 {
    static constexpr int NS = 3;
    static constexpr int Q = 256 * 32;
    static constexpr int SB = 256 * 2 * 2;
    static constexpr int A = 16 * 128;
    static constexpr int Q_OFF = 0;
    static constexpr int SB_OFF = Q_OFF + NS * Q;
    static constexpr int A_OFF = SB_OFF + NS * SB;
    static constexpr int TOTAL = NS * (A + Q + SB);
};

struct Item16 {
    bool valid;
    bool prefetched;
    int r0, rows, n0;
    const char* a_base;  // + kt * 128
    uint32_t a_off;      // this lane's A row byte offset + swizzled chunk (lanes 0-31)
    const char* w_base;  // + kt * kPackBlock
};

// One k-step stage by one wavefront: A rows 4w .. 4w + 3 (lanes 0-31), then
// its share of the weight slabs and scales as in issue_stage. 4 loads.
__device__ __forceinline__ void issue_stage16(const Item16& it, int kt, int buf, uint32_t smem,
                                              uint32_t wave, int lane) {
    if (lane < 32)
        dma16(it.a_base + kt * 128, it.a_off, smem + Lds16::A_OFF + buf * Lds16::A + 4 * wave * 128);
    const uint32_t wh = wave & 1u, wb = wave >> 1;
    const uint32_t q_off = (wh * 128u + (uint32_t)lane) * 16u;
    const uint32_t sb_off = (uint32_t)kPackQ + wh * 256u + (uint32_t)lane * 4u;
    const uint32_t q_lds = smem + Lds16::Q_OFF + buf * Lds16::Q + (wh * 256u + wb * 128u) * 16u;
    const uint32_t sb_lds = smem + Lds16::SB_OFF + buf * Lds16::SB + wh * 512u + wb * 256u;
    const char* blk = it.w_base + (size_t)kt * kPackBlock;
    dma16(blk, q_off, q_lds);
    dma16(blk, q_off + 64 * 16, q_lds + 64 * 16);
    dma4(blk, sb_off, sb_lds);
}

template <bool GATED>
__global__ void __launch_bounds__(kGemmThreads, 4) moe_w4_gemm16(GemmArgs args) {
    constexpr int BN = GemmShape<GATED>::BN;
    constexpr int NS = Lds16::NS;
    constexpr int N_DMA = 4;
    __shared__ __attribute__((aligned(16))) char smem[Lds16::TOTAL];
    __shared__ int s_slot[2];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int q = lane / 16, x = lane % 16;
    const int n_tiles = args.N / BN;
    const int n_slabs = args.N / kPackRows;
    const size_t slab_bytes = (size_t)(args.K / 64) * kPackBlock;
    const int nb_total = args.shared_blocks + args.num_blocks[0];
    const int nk = args.K / 64;
    const int cq = blockIdx.x % kXcds;
    const int n_items = queue_items(nb_total, cq, n_tiles);
    int toggle = 0;

    auto take = [&](Item16& it) {
        it.valid = false;
        const int c = grab(queue_ctr(args.sched, cq), s_slot, toggle);
        if (c >= n_items) return;
        const int vb = queue_block(nb_total, cq, c / n_tiles), nt = c % n_tiles;
        int e = 0;
        bool shared;
        if (vb < args.shared_blocks) {
            it.r0 = args.P + vb * 16;
            it.rows = min(16, args.P + args.T - it.r0);
            shared = true;
        } else {
            const int4 info = args.block_info[vb - args.shared_blocks];
            e = info.x;
            it.r0 = info.y;
            it.rows = info.z;
            shared = false;
        }
        it.n0 = nt * BN;
        it.prefetched = false;
        it.a_base = reinterpret_cast<const char*>(args.a);
        // lanes 0-31 load LDS rows 4w + lane / 8, physical chunk lane % 8
        // (logical chunk swz(row, lane % 8)); rows past the block read its
        // first row, whose products land in outputs that are never stored
        const int row = 4 * (int)wave + (lane % 32) / 8;
        const int r = it.r0 + (row < it.rows ? row : 0);
        const int src_row = GATED ? ((r < args.P) ? args.sorted_pairs[r] / args.topk : r - args.P) : r;
        it.a_off = (uint32_t)src_row * (uint32_t)(args.K * 2) + (uint32_t)(swz(row, lane % 8) * 16);
        const int wb = (int)(wave >> 1);
        const char* stack = shared ? args.sw[GATED ? wb : 0] : args.w[GATED ? wb : 0];
        const int slab = GATED ? nt : 2 * nt + wb;
        it.w_base = stack + ((size_t)e * n_slabs + slab) * slab_bytes;
        it.valid = true;
    };

    // Per-lane LDS read offsets inside a stage.
    uint32_t a_rd[2], q_rd[4], sb_rd[4];
#pragma unroll
    for (int m = 0; m < 2; ++m) a_rd[m] = x * 128 + swz(x, 2 * q + m) * 16;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int qrow = GATED ? (g < 2 ? 32 * (int)wave + 16 * g : 128 + 32 * (int)wave + 16 * (g - 2)) + x
                               : 64 * (int)wave + 16 * g + x;
        q_rd[g] = ((q / 2) * 256 + qrow) * 16 + (q % 2) * 8;
        sb_rd[g] = qrow * 2;
    }

    const uint32_t smem_addr = (uint32_t)(size_t)smem;
    Item16 cur;
    take(cur);
    while (cur.valid) {
        f32x4 acc[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (!cur.prefetched) {
#pragma unroll
            for (int u = 0; u < NS - 1; ++u)
                if (u < nk) issue_stage16(cur, u, u, smem_addr, wave, lane);
        }
        auto step = [&](int kt, int buf) {
            if (kt + 1 >= nk) wait_vmcnt<0>();
            else wait_vmcnt<N_DMA>();
            barrier_only();
            if (kt + NS - 1 < nk) issue_stage16(cur, kt + NS - 1, (buf + NS - 1) % NS, smem_addr, wave, lane);
            const char* Ab = smem + Lds16::A_OFF + buf * Lds16::A;
            const char* Qb = smem + Lds16::Q_OFF + buf * Lds16::Q;
            const char* Sb = smem + Lds16::SB_OFF + buf * Lds16::SB;
            u32x2 qw[4];
            float s512[4], bias[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                qw[g] = *reinterpret_cast<const u32x2*>(Qb + q_rd[g]);
                s512[g] = bf16_bits_to_float(*reinterpret_cast<const uint16_t*>(Sb + sb_rd[g])) * 512.0f;
                bias[g] = bf16_bits_to_float(*reinterpret_cast<const uint16_t*>(Sb + 512 + sb_rd[g]));
            }
            bf16x8 af[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) af[m] = *reinterpret_cast<const bf16x8*>(Ab + a_rd[m]);
            bf16x8 bw[4][2];
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    uint32_t w[4];
                    dequant8(qw[g][m], s512[g], bias[g], w);
                    bw[g][m] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
                }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[g][m], af[m], acc[g], 0, 0, 0);
            wait_lgkmcnt0();
        };
        int kt = 0;
        for (; kt + NS <= nk; kt += NS) {
#pragma unroll
            for (int u = 0; u < NS; ++u) step(kt + u, u);
        }
#pragma unroll
        for (int u = 0; u < NS - 1; ++u)
            if (kt + u < nk) step(kt + u, u);

        // next item and its first stages, overlapping the stores below
        Item16 nxt;
        take(nxt);
        if (nxt.valid) {
#pragma unroll
            for (int u = 0; u < NS - 1; ++u)
                if (u < nk) issue_stage16(nxt, u, u, smem_addr, wave, lane);
            nxt.prefetched = true;
        }
        // Lane l, register r of group g holds weight row 4 (l / 16) + r of
        // the group for token l % 16: four consecutive output columns.
        if (x < cur.rows) {
            const size_t orow = (size_t)(cur.r0 + x) * args.N;
            if (GATED) {
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    float v[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = silu(acc[g][j]) * acc[g + 2][j];
                    *reinterpret_cast<u32x2*>(args.h_out + orow + cur.n0 + 32 * (int)wave + 16 * g + 4 * q) =
                        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                }
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<f32x4*>(args.y_out + orow + cur.n0 + 64 * (int)wave + 16 * g + 4 * q) =
                        acc[g];
            }
        }
        cur = nxt;
    }
    if (tid == 0 && atomicAdd(queue_ctr(args.sched, kXcds), 1) == (int)gridDim.x - 1) {
        for (int i = 0; i <= kXcds; ++i) atomicExch(queue_ctr(args.sched, i), 0);
    }
}

// One thread per (expert, row, group): the row's 32 q bytes of the group go
// to the two halves of its packed block, the scale and bias behind them.
__global__ void __launch_bounds__(256) pack_w4_kernel(const uint8_t* __restrict__ q,
                                                      const uint16_t* __restrict__ scale,
                                                      const uint16_t* __restrict__ bias, int n,
                                                      int N, int K, char* __restrict__ out) {
    const int groups = K / 64;
    const long total = (long)n * N * groups;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const long er = idx / groups;  // e * N + row
    const int g = (int)(idx - er * groups);
    const int row = (int)(er % N);
    const long e = er / N;
    char* blk = out + ((e * (N / kPackRows) + row / kPackRows) * groups + g) * (long)kPackBlock;
    const int r = row % kPackRows;
    const u32x4* src = reinterpret_cast<const u32x4*>(q + er * (K / 2) + g * 32);
    *reinterpret_cast<u32x4*>(blk + r * 16) = src[0];
    *reinterpret_cast<u32x4*>(blk + (kPackRows + r) * 16) = src[1];
    *reinterpret_cast<uint16_t*>(blk + kPackQ + r * 2) = scale[idx];
    *reinterpret_cast<uint16_t*>(blk + kPackQ + 2 * kPackRows + r * 2) = bias[idx];
}

// Unfused twin: the packed int4 stack -> bf16 [n][N][K] in device memory,
// with the same dequantisation as the fused GEMMs (so the GEMMs that read
// it compute bit for bit what the fused ones do). One thread per (expert,
// row, group of 64); experts with counts[e] == 0 are skipped (counts may be
// NULL: all experts).
__global__ void __launch_bounds__(256) dequant_w4_kernel(const char* __restrict__ packed, int n,
                                                         int N, int K,
                                                         const int32_t* __restrict__ counts,
                                                         uint16_t* __restrict__ out) {
    const int groups = K / 64;
    const long total = (long)n * N * groups;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const long er = idx / groups;  // e * N + row
    const int g = (int)(idx - er * groups);
    const int row = (int)(er % N);
    const long e = er / N;
    if (counts && counts[e] == 0) return;
    const char* blk = packed + ((e * (N / kPackRows) + row / kPackRows) * groups + g) * (long)kPackBlock;
    const int r = row % kPackRows;
    const float s512 = bf16_bits_to_float(*reinterpret_cast<const uint16_t*>(blk + kPackQ + r * 2)) * 512.0f;
    const float b = bf16_bits_to_float(*reinterpret_cast<const uint16_t*>(blk + kPackQ + 2 * kPackRows + r * 2));
    u32x4* dst = reinterpret_cast<u32x4*>(out + er * K + g * 64);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(blk + (half * kPackRows + r) * 16);
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            uint32_t o[4];
            dequant8(q[wd], s512, b, o);
            dst[half * 4 + wd] = u32x4{o[0], o[1], o[2], o[3]};
        }
    }
}

int launch_dequant(const void* packed, int n, int N, int K, const int32_t* counts, void* out,
                   hipStream_t stream) {
    const long total = (long)n * N * (K / 64);
    const long grid = (total + 255) / 256;
    hipLaunchKernelGGL(dequant_w4_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const char*>(packed), n, N, K, counts,
                       static_cast<uint16_t*>(out));
    return check_launch("dequant_w4");
}

// out[t] = bf16(y[P + t] + sum_j w[t, j] * y[pair_rows[t * topk + j]]), fp32,
// in slot order. One workgroup per token, 4 columns per thread per pass.
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ pair_rows,
                                                      const float* __restrict__ topk_w, int P,
                                                      int H, int topk, uint16_t* __restrict__ out) {
    const int t = blockIdx.x;
    __shared__ int32_t rows_s[kMaxTopk];
    __shared__ float w_s[kMaxTopk];
    if (threadIdx.x < topk) {
        rows_s[threadIdx.x] = pair_rows[(size_t)t * topk + threadIdx.x];
        w_s[threadIdx.x] = topk_w[(size_t)t * topk + threadIdx.x];
    }
    __syncthreads();
    for (int n = threadIdx.x * 4; n < H; n += blockDim.x * 4) {
        f32x4 acc = *reinterpret_cast<const f32x4*>(y + (size_t)(P + t) * H + n);
        for (int j = 0; j < topk; ++j) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(y + (size_t)rows_s[j] * H + n);
            const float w = w_s[j];
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = __fadd_rn(acc[c], __fmul_rn(w, v[c]));
        }
        u32x2 o;
        o[0] = pack_bf16x2(acc[0], acc[1]);
        o[1] = pack_bf16x2(acc[2], acc[3]);
        *reinterpret_cast<u32x2*>(out + (size_t)t * H + n) = o;
    }
}

// Workspace layout: h bf16 [P + T, F], then y fp32 [P + T, H], then (when a
// GEMM splits K) the fp32 partial sums, each 256-byte aligned.
static size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Split K while the largest possible block map has few tiles: double the
// chunk count while the items stay within kSplitItems and each chunk keeps
// at least kSplitMinSteps k-steps. Depends on the sizes only, so that the
// workspace size is known on the host.
constexpr long kSplitItems = 1024;
constexpr int kSplitMinSteps = 4;
static_assert(kSplitItems / 2 <= kTileCounters, "split-K tile counters");

static int split_k(const lily_moe_dims& d, int max_blocks, bool gated) {
    if (d.tile_m == 16) return 1;  // the 16-row tiles do not split K
    const int BN = gated ? 128 : 256;
    const int N = gated ? d.F : d.H;
    const int nk = (gated ? d.H : d.F) / 64;
    const long tiles = (long)(max_blocks + (d.T + d.tile_m - 1) / d.tile_m) * (N / BN);
    int kc = 1;
    while (nk % (2 * kc) == 0 && nk / (2 * kc) >= kSplitMinSteps && tiles * 2 * kc <= kSplitItems)
        kc *= 2;
    return kc;
}

static size_t part_bytes(const lily_moe_dims& d, int max_blocks) {
    const size_t rows = (size_t)d.T * d.topk + d.T;
    const int kg = split_k(d, max_blocks, true), kd = split_k(d, max_blocks, false);
    size_t b = 0;
    if (kg > 1) b = (size_t)kg * rows * 2 * d.F * sizeof(float);
    if (kd > 1) b = std::max(b, (size_t)kd * rows * d.H * sizeof(float));
    return b;
}

size_t forward_workspace_bytes(const lily_moe_dims& d, int max_blocks) {
    const size_t rows = (size_t)d.T * d.topk + d.T;
    const size_t fwd = align_up(rows * d.F * sizeof(uint16_t)) + align_up(rows * d.H * sizeof(float)) +
                       align_up(part_bytes(d, max_blocks));
    return std::max(fwd, decode_workspace_bytes(d));  // lily_moe_decode uses the same workspace
}

ForwardWorkspace forward_workspace_split(const lily_moe_dims& d, void* ws) {
    const size_t rows = (size_t)d.T * d.topk + d.T;
    char* p = reinterpret_cast<char*>(ws);
    ForwardWorkspace w;
    w.h = reinterpret_cast<uint16_t*>(p);
    p += align_up(rows * d.F * sizeof(uint16_t));
    w.y = reinterpret_cast<float*>(p);
    p += align_up(rows * d.H * sizeof(float));
    w.part = reinterpret_cast<float*>(p);
    return w;
}

static GemmArgs routing_args(const lily_moe_dims& d, const lily_moe_routing& r) {
    GemmArgs g{};
    g.topk = d.topk;
    g.block_info = reinterpret_cast<const int4*>(r.block_info);
    g.num_blocks = r.num_blocks;
    g.P = d.T * d.topk;
    g.T = d.T;
    return g;
}

// Persistent grid: the workgroups that fit on the device at once (from the
// kernel's own occupancy), fewer if the largest possible block map has
// fewer items (tiles times K chunks), a multiple of the queue count.
template <int BM, bool GATED, bool W4>
static int gemm_grid(GemmArgs& g, int max_blocks) {
    constexpr int kMaxDevices = 64;
    static int resident[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    int slots = dev < kMaxDevices ? resident[dev] : 0;
    if (slots == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_w4_gemm<BM, GATED, W4>,
                                                         kGemmThreads, 0) != hipSuccess)
            per_cu = 0;
        slots = (cus > 0 ? cus : 256) * (per_cu > 0 ? per_cu : 1);
        if (dev < kMaxDevices) resident[dev] = slots;
    }
    g.shared_blocks = (g.T + BM - 1) / BM;
    const long items = (long)(max_blocks + g.shared_blocks) * (g.N / GemmShape<GATED>::BN) * g.kc;
    const long grid = items < slots ? items : slots;
    return (int)((grid + kXcds - 1) / kXcds * kXcds);
}

template <int BM, bool W4>
static int launch_gate_up_bm(GemmArgs g, int max_blocks, hipStream_t stream) {
    const dim3 grid(gemm_grid<BM, true, W4>(g, max_blocks));
    hipLaunchKernelGGL((moe_w4_gemm<BM, true, W4>), grid, dim3(kGemmThreads), 0, stream, g);
    return check_launch("gate_up_gemm");
}

template <int BM, bool W4>
static int launch_down_bm(GemmArgs g, int max_blocks, hipStream_t stream) {
    const dim3 grid(gemm_grid<BM, false, W4>(g, max_blocks));
    hipLaunchKernelGGL((moe_w4_gemm<BM, false, W4>), grid, dim3(kGemmThreads), 0, stream, g);
    return check_launch("down_gemm");
}

static GemmArgs gate_up_args(const lily_moe_dims& d, const lily_moe_weights& w, const uint16_t* x,
                             const lily_moe_routing& r, int max_blocks, const ForwardWorkspace& ws) {
    GemmArgs g = routing_args(d, r);
    g.a = x;
    g.sorted_pairs = r.sorted_pairs;
    g.w[0] = static_cast<const char*>(w.gate);
    g.w[1] = static_cast<const char*>(w.up);
    g.sw[0] = static_cast<const char*>(w.sh_gate);
    g.sw[1] = static_cast<const char*>(w.sh_up);
    g.N = d.F;
    g.K = d.H;
    g.sched = r.sched + kQueueBase;
    g.h_out = ws.h;
    g.kc = split_k(d, max_blocks, true);
    g.part = ws.part;
    g.tile_ctr = r.sched + kQueueInts;
    return g;
}

static GemmArgs down_args(const lily_moe_dims& d, const lily_moe_weights& w, const lily_moe_routing& r,
                          int max_blocks, const ForwardWorkspace& ws) {
    GemmArgs g = routing_args(d, r);
    g.a = ws.h;
    g.w[0] = g.w[1] = static_cast<const char*>(w.down);
    g.sw[0] = g.sw[1] = static_cast<const char*>(w.sh_down);
    g.N = d.H;
    g.K = d.F;
    g.sched = r.sched + kQueueBase + kQueueCtrs * kQueueLine;
    g.y_out = ws.y;
    g.kc = split_k(d, max_blocks, false);
    g.part = ws.part;
    g.tile_ctr = r.sched + kQueueInts + kTileCounters;
    return g;
}

template <bool GATED>
static int launch_gemm16(GemmArgs g, int max_blocks, hipStream_t stream) {
    constexpr int kMaxDevices = 64;
    static int resident[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    int slots = dev < kMaxDevices ? resident[dev] : 0;
    if (slots == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_w4_gemm16<GATED>, kGemmThreads,
                                                         0) != hipSuccess)
            per_cu = 0;
        slots = (cus > 0 ? cus : 256) * (per_cu > 0 ? per_cu : 1);
        if (dev < kMaxDevices) resident[dev] = slots;
    }
    g.shared_blocks = (g.T + 15) / 16;
    const long items = (long)(max_blocks + g.shared_blocks) * (g.N / GemmShape<GATED>::BN);
    const long grid = items < slots ? items : slots;
    hipLaunchKernelGGL(moe_w4_gemm16<GATED>, dim3((unsigned)((grid + kXcds - 1) / kXcds * kXcds)),
                       dim3(kGemmThreads), 0, stream, g);
    return check_launch(GATED ? "gate_up_gemm16" : "down_gemm16");
}

// G1 + G2 (and the shared expert's rows): h = bf16(silu(x Wg^T) * (x Wu^T)).
// w4 = false: the unfused twin, whose weights are bf16 [n][N][K] stacks.
int launch_gate_up(const lily_moe_dims& d, const lily_moe_weights& w, const uint16_t* x,
                   const lily_moe_routing& r, int max_blocks, const ForwardWorkspace& ws,
                   hipStream_t stream, bool w4) {
    GemmArgs g = gate_up_args(d, w, x, r, max_blocks, ws);
    if (!w4) {
        if (d.tile_m == 32) return launch_gate_up_bm<32, false>(g, max_blocks, stream);
        if (d.tile_m == 64) return launch_gate_up_bm<64, false>(g, max_blocks, stream);
        return set_error(LILY_ERR_UNSUPPORTED, "tile_m %d; the bf16 GEMMs take 32 or 64", d.tile_m);
    }
    switch (d.tile_m) {
        case 16: return launch_gemm16<true>(g, max_blocks, stream);
        case 32: return launch_gate_up_bm<32, true>(g, max_blocks, stream);
        case 64: return launch_gate_up_bm<64, true>(g, max_blocks, stream);
        case 128: return launch_gate_up_bm<128, true>(g, max_blocks, stream);
    }
    return set_error(LILY_ERR_UNSUPPORTED, "tile_m %d not supported", d.tile_m);
}

// G3 (and the shared expert's rows): y = h Wd^T in fp32.
int launch_down(const lily_moe_dims& d, const lily_moe_weights& w, const lily_moe_routing& r,
                int max_blocks, const ForwardWorkspace& ws, hipStream_t stream, bool w4) {
    GemmArgs g = down_args(d, w, r, max_blocks, ws);
    if (!w4) {
        if (d.tile_m == 32) return launch_down_bm<32, false>(g, max_blocks, stream);
        if (d.tile_m == 64) return launch_down_bm<64, false>(g, max_blocks, stream);
        return set_error(LILY_ERR_UNSUPPORTED, "tile_m %d; the bf16 GEMMs take 32 or 64", d.tile_m);
    }
    switch (d.tile_m) {
        case 16: return launch_gemm16<false>(g, max_blocks, stream);
        case 32: return launch_down_bm<32, true>(g, max_blocks, stream);
        case 64: return launch_down_bm<64, true>(g, max_blocks, stream);
        case 128: return launch_down_bm<128, true>(g, max_blocks, stream);
    }
    return set_error(LILY_ERR_UNSUPPORTED, "tile_m %d not supported", d.tile_m);
}

template <int BM>
static int launch_ffn_bm(GemmArgs gu, GemmArgs dn, int max_blocks, hipStream_t stream) {
    constexpr int kMaxDevices = 64;
    static int resident[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    int slots = dev < kMaxDevices ? resident[dev] : 0;
    if (slots == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_w4_ffn<BM>, kGemmThreads, 0) !=
            hipSuccess)
            per_cu = 0;
        slots = (cus > 0 ? cus : 256) * (per_cu > 0 ? per_cu : 1);
        if (dev < kMaxDevices) resident[dev] = slots;
    }
    const long items = (long)(max_blocks + gu.shared_blocks) *
                       (gu.N / GemmShape<true>::BN + dn.N / GemmShape<false>::BN);
    const long grid = items < slots ? items : slots;
    hipLaunchKernelGGL(moe_w4_ffn<BM>, dim3((unsigned)((grid + kXcds - 1) / kXcds * kXcds)),
                       dim3(kGemmThreads), 0, stream, gu, dn);
    return check_launch("ffn_gemms");
}

// G1-G3 in one launch (moe_w4_ffn) when neither GEMM splits K and the
// schedule's blocks fit the block tallies (which take the split-K tile
// counters of both GEMMs, unused then). Returns 1, having launched
// nothing, when it does not apply.
int launch_ffn(const lily_moe_dims& d, const lily_moe_weights& w, const uint16_t* x,
               const lily_moe_routing& r, int max_blocks, const ForwardWorkspace& ws,
               hipStream_t stream) {
    GemmArgs gu = gate_up_args(d, w, x, r, max_blocks, ws);
    GemmArgs dn = down_args(d, w, r, max_blocks, ws);
    const int shared_blocks = (d.T + d.tile_m - 1) / d.tile_m;
    if (gu.kc != 1 || dn.kc != 1 || (long)max_blocks + shared_blocks > 2L * kTileCounters ||
        d.F % GemmShape<true>::BN != 0)
        return 1;
    gu.shared_blocks = dn.shared_blocks = shared_blocks;
    gu.blk_done = dn.blk_done = r.sched + kQueueInts;
    gu.blk_need = dn.blk_need = d.F / GemmShape<true>::BN;
    gu.sched_flag = dn.sched_flag = r.sched + kGiveUpFlag;
    dn.sched = gu.sched;
    switch (d.tile_m) {
        case 32: return launch_ffn_bm<32>(gu, dn, max_blocks, stream);
        case 64: return launch_ffn_bm<64>(gu, dn, max_blocks, stream);
        case 128: return launch_ffn_bm<128>(gu, dn, max_blocks, stream);
    }
    return 1;
}

size_t packed_w4_bytes(int n, int N, int K) {
    return (size_t)n * N * K / 64 * (kPackBlock / kPackRows);
}

int launch_pack(const lily_w4& w, int n, int N, int K, void* packed, hipStream_t stream) {
    const long total = (long)n * N * (K / 64);
    const long grid = (total + 255) / 256;
    hipLaunchKernelGGL(pack_w4_kernel, dim3((unsigned)grid), dim3(256), 0, stream, w.q, w.scale,
                       w.bias, n, N, K, static_cast<char*>(packed));
    return check_launch("pack_w4");
}

// G5: weighted gather-combine.
int launch_combine(const lily_moe_dims& d, const ForwardWorkspace& ws, const lily_moe_routing& r,
                   uint16_t* out, hipStream_t stream) {
    const float* y = ws.y;
    hipLaunchKernelGGL(combine_kernel, dim3(d.T), dim3(256), 0, stream, y, r.pair_rows, r.topk_w,
                       d.T * d.topk, d.H, d.topk, out);
    return check_launch("combine");
}


// Copies the item trace of the last moe_w4_ffn launch (tracing build only).
int trace_ffn_items(unsigned long long* dst, int max_wgs, hipStream_t stream) {
#ifdef LILY_TRACE_ITEMS
    if (!dst || max_wgs < 1)
        return set_error(LILY_ERR_INVALID_ARG, "trace_ffn_items: dst non-NULL, max_wgs >= 1");
    const int n = max_wgs < kTraceWgs ? max_wgs : kTraceWgs;
    const size_t row = sizeof(g_ffn_trace[0]);
    if (hipStreamSynchronize(stream) != hipSuccess ||
        hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_ffn_trace), row * n, 0, hipMemcpyDeviceToHost) !=
            hipSuccess)
        return set_error(LILY_ERR_HIP, "trace_ffn_items: copy failed");
    return n;
#else
    (void)dst;
    (void)max_wgs;
    (void)stream;
    return set_error(LILY_ERR_UNSUPPORTED,
                     "trace_ffn_items: this library was built without the item trace "
                     "(liblily_moe_trace.so has it)");
#endif
}

}  // namespace lily
