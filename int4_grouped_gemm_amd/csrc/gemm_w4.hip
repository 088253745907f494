// Grouped expert GEMMs with the int4 -> bf16 dequantisation fused into the
// tile loads, SwiGLU, and the weighted gather-combine (gfx950).
//
// The Lily articles rebuild the 4-bit weights as bf16 tile by tile inside
// the grouped GEMM, keep them in on-chip memory and accumulate in FP32, so
// the expanded weights never reach main memory (news.ainew.jp Lily article,
// section "Prefill"). Here the on-chip memory is the LDS of a CDNA4 compute
// unit and the products run on bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// One workgroup computes one (block, n-tile) of one expert:
//   rows  = a block of the block map (or of the shared expert's T rows);
//   cols  = BN outputs of the expert's weight matrix (for the gate/up GEMM,
//           BN columns of both gate and up, so that SwiGLU can be applied
//           in the epilogue).
// K runs in steps of 64 = one quantisation group per weight row, so each
// step needs one scale and one bias per row. Global loads of step s+1 are
// issued before the MFMAs of step s (register prefetch); dequantisation
// happens when the prefetched nibbles are written to LDS.
//
// LDS tiles are [rows][64] bf16 with the 16-byte chunks of each row
// XOR-swizzled by (row & 7), so that 32 lanes reading one chunk column of
// 32 consecutive rows hit distinct banks.
#include "common.hpp"

namespace lily {

struct GemmArgs {
    const uint16_t* a;              // A rows: gate/up -> x [T, K]; down -> h [P + T, K]
    const int32_t* sorted_pairs;    // gate/up: routed row r reads x[sorted_pairs[r] / topk]
    int topk;
    const uint8_t* q[2];            // routed weights [E, N, K/2] (gate/up: [0]=gate, [1]=up)
    const uint16_t* sc[2];          // [E, N, K/64]
    const uint16_t* bi[2];
    const uint8_t* sq[2];           // shared expert weights [1, N, K/2]
    const uint16_t* ssc[2];
    const uint16_t* sbi[2];
    int N, K;
    const int32_t* block_expert;
    const int32_t* block_row0;
    const int32_t* num_blocks;
    const int32_t* offsets;
    int max_blocks;
    int shared_blocks;  // ceil(T / BM)
    int P, T;
    uint16_t* h_out;  // gate/up: h [P + T, N] bf16
    float* y_out;     // down: y [P + T, N] fp32
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

// silu(z) = z / (1 + e^-z) with the hardware exp2 and reciprocal (a few ulp
// of fp32, far below the bf16 rounding of h that follows).
__device__ __forceinline__ float silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// Eight int4 weights (one 32-bit word: element 2i in the low nibble of byte
// i) -> four bf16x2 words of w = bf16(scale * q + bias), elements in order.
// A byte 0x00..0x0F read as an OCP e4m3 value is exactly q * 2^-9 (exponent
// field 0 or 1), so one v_cvt_pk_f32_fp8 widens two nibbles, and with
// s512 = scale * 2^9 (exact) fma(s512, q * 2^-9, bias) is the same single
// rounding of scale * q + bias as fma(scale, q, bias).
__device__ __forceinline__ void dequant8(uint32_t v, float s512, float b, uint32_t out[4]) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const uint32_t lo = v & 0x0F0F0F0Fu;         // elements 0, 2, 4, 6
    const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;  // elements 1, 3, 5, 7
    const f2 e02 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
    const f2 e46 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
    const f2 e13 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    const f2 e57 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    out[0] = pack_bf16x2(fmaf(s512, e02[0], b), fmaf(s512, e13[0], b));
    out[1] = pack_bf16x2(fmaf(s512, e02[1], b), fmaf(s512, e13[1], b));
    out[2] = pack_bf16x2(fmaf(s512, e46[0], b), fmaf(s512, e57[0], b));
    out[3] = pack_bf16x2(fmaf(s512, e46[1], b), fmaf(s512, e57[1], b));
}

// Tile geometry. A workgroup has 4 wavefronts that split the output columns;
// every wavefront covers all BM rows of the block. The workgroup owns 256
// weight rows: for the gate/up GEMM 128 gate rows and the same 128 up rows
// (so SwiGLU is local to a lane), for the down GEMM 256 rows of W_down.
// Wavefront w takes two groups of 32 weight rows: gate/up -> gate rows
// 32w.. and up rows 128+32w..; down -> rows 64w.. and 64w+32...
//
// Every operand travels global -> LDS with global_load_lds (no registers,
// no compiler-managed waits), kNS k-steps in flight:
//   A stage  [BM rows][64 bf16], 16-byte chunks XOR-swizzled by (row & 7);
//   Q stage  [2 halves][256 rows][16 bytes] of int4 weights;
//   SB ring  scales then biases of the 256 rows for two k-steps (4 bytes a
//            row), refreshed every other k-step.
// Each lane then dequantises its own 32 weights of a k-step from LDS into
// MFMA operand registers (no weight is dequantised twice in a workgroup).
//
// K mapping inside a 64-wide k-step: lanes 0-31 (h = 0) hold k 0..31 and
// lanes 32-63 (h = 1) hold k 32..63; MFMA step s (16 k) pairs elements
// 8s..8s+7 of each half, for A and B alike. So a lane's A operand for step s
// is the 16-byte chunk 4h + s of its row.
constexpr int kGemmThreads = 256;
constexpr int kGemmWaves = kGemmThreads / kWave;
constexpr int kXcds = 8;  // MI355X: 8 XCDs of 32 CUs, each with its own L2

template <bool GATED>
struct GemmShape {
    static constexpr int BN = GATED ? 128 : 256;  // output columns per workgroup
};

// Per tile height: k-steps in flight through LDS and workgroups per CU.
// A single wavefront issues a VALU instruction only every few cycles, so the
// dequantisation throughput of a SIMD grows with the number of wavefronts it
// holds: tiles of up to 64 rows keep 4 wavefronts per SIMD (<= 128 VGPRs,
// <= 40 KB of LDS per workgroup) and double-buffer; 128-row tiles hold 2.
template <int BM>
struct Occ {
    static constexpr int NS = BM >= 128 ? 3 : 2;
    static constexpr int WAVES_PER_SIMD = BM >= 128 ? 2 : 4;
};

// LDS layout of a workgroup: per stage, the weights (Q: [2 halves][256
// rows][16 B]), the scale/bias words (SB: [256 rows] scales then [256 rows]
// biases, 4 bytes = the aligned pair of groups holding this k-step's) and
// the A tile ([BM rows][64 bf16]). All stage bases stay below 64 KB so they
// fit the immediate offset of ds_read.
template <int BM>
struct Lds {
    static constexpr int NS = Occ<BM>::NS;
    static constexpr int Q = 256 * 32;
    static constexpr int SB = 256 * 4 * 2;
    static constexpr int A = BM * 128;
    static constexpr int Q_OFF = 0;
    static constexpr int SB_OFF = Q_OFF + NS * Q;
    static constexpr int A_OFF = SB_OFF + NS * SB;
    static constexpr int TOTAL = A_OFF + NS * A;
    static_assert(A_OFF + (NS - 1) * A < 65536, "stage bases must fit ds_read offsets");
};

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
// m0 + l * size. The kernel's own code uses M0 for nothing else.
__device__ __forceinline__ void dma16(const void* base, uint32_t lane_off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds_addr), "v"(lane_off), "s"(base) : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t lane_off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(lds_addr), "v"(lane_off), "s"(base) : "memory");
}

// Per-workgroup load plan: for each DMA instruction of this wavefront, a
// uniform base (advanced per k-step by a fixed stride) and a lane offset.
template <int MI>
struct LoadPlan {
    const char* a_base;      // A rows: + kt * 128
    uint32_t a_off[MI];      // row byte offset + swizzled chunk
    const char* q_base[2];   // weight halves: + kt * 32
    uint32_t q_off[2];
    const char* sb_base[2];  // scale/bias pairs: + (kt & ~1) * 2
    uint32_t sb_off[2];
};

template <int BM, bool GATED, int MIA>
__device__ __forceinline__ void gemm_main(const GemmArgs& args, char* smem_p,
                                          const LoadPlan<BM / 32>& lp, uint32_t wave, int r0,
                                          int rows, const int* brow, const int* col0) {
    using Ld = Lds<BM>;
    constexpr int NS = Ld::NS;
    constexpr int NI = 2;
    constexpr int N_A = MIA;  // A loads per wavefront per k-step (8 rows each)
    constexpr int N_DMA = N_A + 2 + 2;
    static_assert(NS == 2 || NS == 3, "stage count");
    const uint32_t smem = (uint32_t)(size_t)smem_p;  // LDS byte address
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int h = lane / 32;
    const int nk = args.K / 64;

    auto issue = [&](int kt, int buf) {
#pragma unroll
        for (int j = 0; j < N_A; ++j)
            dma16(lp.a_base + kt * 128, lp.a_off[j],
                  smem + Ld::A_OFF + buf * Ld::A + (32 * j + 8 * wave) * 128);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            dma16(lp.q_base[j] + kt * 32, lp.q_off[j],
                  smem + Ld::Q_OFF + buf * Ld::Q + 64 * (2 * wave + j) * 16);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            dma4(lp.sb_base[j] + (kt & ~1) * 2, lp.sb_off[j],
                 smem + Ld::SB_OFF + buf * Ld::SB + 64 * (2 * wave + j) * 4);
    };

    f32x16 acc[MIA][NI];
#pragma unroll
    for (int i = 0; i < MIA; ++i)
#pragma unroll
        for (int g = 0; g < NI; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][g][r] = 0.0f;

    // Per-lane LDS read offsets inside a stage.
    uint32_t a_rd[MIA][4];
#pragma unroll
    for (int i = 0; i < MIA; ++i)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int row = 32 * i + lane % 32;
            a_rd[i][s] = row * 128 + swz(row, 4 * h + s) * 16;
        }
    uint32_t q_rd[NI], sb_rd[NI];
#pragma unroll
    for (int g = 0; g < NI; ++g) {
        q_rd[g] = (h * 256 + brow[g]) * 16;
        sb_rd[g] = brow[g] * 4;
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
        const char* Sb = smem_p + Ld::SB_OFF + buf * Ld::SB + (kt & 1) * 2;
        u32x4 q[NI];
        uint16_t sbits[NI], bbits[NI];
#pragma unroll
        for (int g = 0; g < NI; ++g) {
            q[g] = *reinterpret_cast<const u32x4*>(Qb + q_rd[g]);
            sbits[g] = *reinterpret_cast<const uint16_t*>(Sb + sb_rd[g]);
            bbits[g] = *reinterpret_cast<const uint16_t*>(Sb + 1024 + sb_rd[g]);
        }
        bf16x8 af_cur[MIA], af_nxt[MIA];
#pragma unroll
        for (int i = 0; i < MIA; ++i) af_cur[i] = *reinterpret_cast<const bf16x8*>(Ab + a_rd[i][0]);
        float s512[NI], bias[NI];
#pragma unroll
        for (int g = 0; g < NI; ++g) {
            s512[g] = bf16_bits_to_float(sbits[g]) * 512.0f;
            bias[g] = bf16_bits_to_float(bbits[g]);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) {
#pragma unroll
                for (int i = 0; i < MIA; ++i)
                    af_nxt[i] = *reinterpret_cast<const bf16x8*>(Ab + a_rd[i][s + 1]);
            }
            bf16x8 bfr[NI];
#pragma unroll
            for (int g = 0; g < NI; ++g) {
                uint32_t w[4];
                dequant8(q[g][s], s512[g], bias[g], w);
                bfr[g] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
            }
#pragma unroll
            for (int i = 0; i < MIA; ++i)
#pragma unroll
                for (int g = 0; g < NI; ++g)
                    acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af_cur[i], bfr[g], acc[i][g], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < MIA; ++i) af_cur[i] = af_nxt[i];
        }
        wait_lgkmcnt0();  // this wavefront's LDS reads of the stage are done
    };

    issue(0, 0);
    if (NS == 3 && nk > 1) issue(1, 1);
    for (int kt = 0; kt < nk; kt += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u)
            if (kt + u < nk) step(kt + u, u);
    }

    // Epilogue. C layout of a 32x32 tile: lane l, register r holds row
    // 8*(r/4) + 4*(l/32) + r%4 and column l%32.
#pragma unroll
    for (int i = 0; i < MIA; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
            if (row < rows) {
                const size_t orow = (size_t)(r0 + row) * args.N;
                if (GATED) {
                    const float g = acc[i][0][r];
                    const float u = acc[i][1][r];
                    args.h_out[orow + col0[0] + lane % 32] = float_to_bf16_bits(silu(g) * u);
                } else {
#pragma unroll
                    for (int g = 0; g < NI; ++g) args.y_out[orow + col0[g] + lane % 32] = acc[i][g][r];
                }
            }
        }
    }
}

template <int BM, bool GATED>
__global__ void __launch_bounds__(kGemmThreads, Occ<BM>::WAVES_PER_SIMD) moe_w4_gemm(GemmArgs args) {
    constexpr int BN = GemmShape<GATED>::BN;
    constexpr int MI = BM / 32;
    __shared__ __attribute__((aligned(16))) char smem[Lds<BM>::TOTAL];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);

    // Tiles are (block, n-tile) pairs: the routed blocks of the block map,
    // then the shared expert's blocks; n-tiles vary fastest. Workgroups are
    // dispatched to the 8 XCDs round-robin, so workgroup L runs on XCD L % 8;
    // each XCD takes a contiguous range of the live tiles, so that the
    // n-tiles of a block (same A rows) and consecutive blocks of an expert
    // (same weights) meet in one L2.
    const int n_tiles = args.N / BN;
    const int live = (args.num_blocks[0] + args.shared_blocks) * n_tiles;
    const int per_xcd = (live + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    const int tile = (blockIdx.x % kXcds) * per_xcd + slot;
    if (slot >= per_xcd || tile >= live) return;
    const int blk = tile / n_tiles;
    const int n0 = (tile % n_tiles) * BN;

    // Which rows, which expert.
    int r0, r_end;
    bool shared;
    int e = 0;
    if (blk < args.num_blocks[0]) {
        e = args.block_expert[blk];
        r0 = args.block_row0[blk];
        r_end = args.offsets[e + 1];
        shared = false;
    } else {
        r0 = args.P + (blk - args.num_blocks[0]) * BM;
        r_end = args.P + args.T;
        shared = true;
    }
    const int rows = min(BM, r_end - r0);
    const int K = args.K;

    LoadPlan<MI> lp;
    // A loads: load j of wavefront w fills LDS rows 32j + 8w + lane/8,
    // physical chunk lane%8, which holds logical chunk (lane%8) ^ (row & 7).
    // Rows past the block read the block's first row: their products land in
    // output rows that are never stored.
    lp.a_base = reinterpret_cast<const char*>(args.a);
#pragma unroll
    for (int j = 0; j < MI; ++j) {
        const int row = 32 * j + 8 * (int)wave + lane / 8;
        const int r = r0 + (row < rows ? row : 0);
        int src_row = r;
        if (GATED) src_row = (r < args.P) ? args.sorted_pairs[r] / args.topk : r - args.P;
        lp.a_off[j] = (uint32_t)src_row * (uint32_t)(K * 2) + (uint32_t)(((lane % 8) ^ (row & 7)) * 16);
    }
    // Weight loads. The workgroup's 256 weight rows: gate/up -> rows n0.. of
    // the gate matrix then the same rows of the up matrix; down -> rows n0..
    // of W_down. Load j of wavefront w covers 64 consecutive slots
    // c = 64 (2w + j) + lane: for weights slot (half, row) = (c / 256, c % 256),
    // for scales c < 256 and biases c >= 256, row c % 256. Each load stays in
    // one matrix, so its base is uniform.
    const size_t mat = shared ? 0 : (size_t)e * args.N;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c0 = 64 * (2 * (int)wave + j);        // uniform
        const int r_loc = (c0 % 256) + lane;
        const int m = GATED ? (c0 % 256) / 128 : 0;      // uniform
        const int n_in = GATED ? r_loc % 128 : r_loc;    // row inside the workgroup's span
        const uint8_t* qm = shared ? args.sq[m] : args.q[m];
        lp.q_base[j] = reinterpret_cast<const char*>(qm + (mat + n0) * (K / 2)) + (c0 / 256) * 16;
        lp.q_off[j] = (uint32_t)n_in * (uint32_t)(K / 2);
        const bool is_bias = c0 >= 256;
        const uint16_t* sm = is_bias ? (shared ? args.sbi[m] : args.bi[m])
                                     : (shared ? args.ssc[m] : args.sc[m]);
        lp.sb_base[j] = reinterpret_cast<const char*>(sm + (mat + n0) * (K / 64));
        lp.sb_off[j] = (uint32_t)n_in * (uint32_t)(K / 64) * 2u;
    }
    int brow[2], col0[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        brow[g] = GATED ? 128 * g + 32 * (int)wave + lane % 32 : 64 * (int)wave + 32 * g + lane % 32;
        col0[g] = GATED ? n0 + 32 * (int)wave : n0 + 64 * (int)wave + 32 * g;
    }

    // Only the 32-row sub-tiles that hold rows of the block are loaded and
    // multiplied.
    const int mia = (rows + 31) / 32;
    if (mia >= MI) gemm_main<BM, GATED, MI>(args, smem, lp, wave, r0, rows, brow, col0);
    else if (mia == 1) gemm_main<BM, GATED, 1>(args, smem, lp, wave, r0, rows, brow, col0);
    else if (mia == 2) gemm_main<BM, GATED, (MI > 2 ? 2 : 1)>(args, smem, lp, wave, r0, rows, brow, col0);
    else gemm_main<BM, GATED, (MI > 3 ? 3 : 1)>(args, smem, lp, wave, r0, rows, brow, col0);
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

// Workspace layout: h bf16 [P + T, F] then y fp32 [P + T, H], 256-byte aligned.
static size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

size_t forward_workspace_bytes(const lily_moe_dims& d) {
    const size_t rows = (size_t)d.T * d.topk + d.T;
    return align_up(rows * d.F * sizeof(uint16_t)) + align_up(rows * d.H * sizeof(float));
}

static GemmArgs routing_args(const lily_moe_dims& d, const lily_moe_routing& r, int max_blocks) {
    GemmArgs g{};
    g.topk = d.topk;
    g.block_expert = r.block_expert;
    g.block_row0 = r.block_row0;
    g.num_blocks = r.num_blocks;
    g.offsets = r.offsets;
    g.max_blocks = max_blocks;
    g.P = d.T * d.topk;
    g.T = d.T;
    return g;
}

// Grid: enough workgroups for the largest possible block map (the live
// count is only known on the device), a multiple of the XCD count.
template <int BM, bool GATED>
static dim3 gemm_grid(GemmArgs& g) {
    g.shared_blocks = (g.T + BM - 1) / BM;
    const long tiles = (long)(g.max_blocks + g.shared_blocks) * (g.N / GemmShape<GATED>::BN);
    return dim3((unsigned)((tiles + kXcds - 1) / kXcds * kXcds));
}

template <int BM>
static int launch_gate_up_bm(const lily_moe_dims& d, GemmArgs g, hipStream_t stream) {
    const dim3 grid = gemm_grid<BM, true>(g);
    hipLaunchKernelGGL((moe_w4_gemm<BM, true>), grid, dim3(kGemmThreads), 0, stream, g);
    return check_launch("gate_up_gemm");
}

template <int BM>
static int launch_down_bm(const lily_moe_dims& d, GemmArgs g, hipStream_t stream) {
    const dim3 grid = gemm_grid<BM, false>(g);
    hipLaunchKernelGGL((moe_w4_gemm<BM, false>), grid, dim3(kGemmThreads), 0, stream, g);
    return check_launch("down_gemm");
}

// G1 + G2 (and the shared expert's rows): h = bf16(silu(x Wg^T) * (x Wu^T)).
int launch_gate_up(const lily_moe_dims& d, const lily_moe_weights& w, const uint16_t* x,
                   const lily_moe_routing& r, int max_blocks, uint16_t* h, hipStream_t stream) {
    GemmArgs g = routing_args(d, r, max_blocks);
    g.a = x;
    g.sorted_pairs = r.sorted_pairs;
    g.q[0] = w.gate.q; g.sc[0] = w.gate.scale; g.bi[0] = w.gate.bias;
    g.q[1] = w.up.q;   g.sc[1] = w.up.scale;   g.bi[1] = w.up.bias;
    g.sq[0] = w.sh_gate.q; g.ssc[0] = w.sh_gate.scale; g.sbi[0] = w.sh_gate.bias;
    g.sq[1] = w.sh_up.q;   g.ssc[1] = w.sh_up.scale;   g.sbi[1] = w.sh_up.bias;
    g.N = d.F;
    g.K = d.H;
    g.h_out = h;
    switch (d.tile_m) {
        case 32: return launch_gate_up_bm<32>(d, g, stream);
        case 64: return launch_gate_up_bm<64>(d, g, stream);
        case 128: return launch_gate_up_bm<128>(d, g, stream);
    }
    return set_error(LILY_ERR_UNSUPPORTED, "tile_m %d not supported", d.tile_m);
}

// G3 (and the shared expert's rows): y = h Wd^T in fp32.
int launch_down(const lily_moe_dims& d, const lily_moe_weights& w, const uint16_t* h,
                const lily_moe_routing& r, int max_blocks, float* y, hipStream_t stream) {
    GemmArgs g = routing_args(d, r, max_blocks);
    g.a = h;
    g.q[0] = w.down.q; g.sc[0] = w.down.scale; g.bi[0] = w.down.bias;
    g.sq[0] = w.sh_down.q; g.ssc[0] = w.sh_down.scale; g.sbi[0] = w.sh_down.bias;
    g.N = d.H;
    g.K = d.F;
    g.y_out = y;
    switch (d.tile_m) {
        case 32: return launch_down_bm<32>(d, g, stream);
        case 64: return launch_down_bm<64>(d, g, stream);
        case 128: return launch_down_bm<128>(d, g, stream);
    }
    return set_error(LILY_ERR_UNSUPPORTED, "tile_m %d not supported", d.tile_m);
}

// G5: weighted gather-combine.
int launch_combine(const lily_moe_dims& d, const float* y, const lily_moe_routing& r,
                   uint16_t* out, hipStream_t stream) {
    hipLaunchKernelGGL(combine_kernel, dim3(d.T), dim3(256), 0, stream, y, r.pair_rows, r.topk_w,
                       d.T * d.topk, d.H, d.topk, out);
    return check_launch("combine");
}

void forward_workspace_split(const lily_moe_dims& d, void* ws, uint16_t** h, float** y) {
    const size_t rows = (size_t)d.T * d.topk + d.T;
    *h = reinterpret_cast<uint16_t*>(ws);
    *y = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                  align_up(rows * d.F * sizeof(uint16_t)));
}

}  // namespace lily
