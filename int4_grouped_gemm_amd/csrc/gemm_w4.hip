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
    int P, T;
    uint16_t* h_out;  // gate/up: h [P + T, N] bf16
    float* y_out;     // down: y [P + T, N] fp32
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// 32 int4 weights (16 bytes, element 2i in the low nibble of byte i) ->
// 32 bf16 as four 16-byte chunks: w = bf16(scale * q + bias).
__device__ __forceinline__ void dequant32(const u32x4 qv, float s, float b, u32x4 out[4]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t v = qv[w];  // 8 nibbles: elements 8w .. 8w+7
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = fmaf(s, (float)((v >> (4 * i)) & 0xFu), b);
        out[w][0] = pack_bf16x2(f[0], f[1]);
        out[w][1] = pack_bf16x2(f[2], f[3]);
        out[w][2] = pack_bf16x2(f[4], f[5]);
        out[w][3] = pack_bf16x2(f[6], f[7]);
    }
}

template <int BM, int BN, int NWM, int NWN, bool GATED>
__global__ void __launch_bounds__(NWM * NWN * kWave) grouped_w4_gemm(GemmArgs args) {
    constexpr int NT = NWM * NWN * kWave;
    constexpr int NB = GATED ? 2 : 1;
    constexpr int WM = BM / NWM, WN = BN / NWN;
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int A_CHUNKS = BM * 8;          // 16-byte chunks of bf16 per A k-step
    constexpr int A_PER_T = A_CHUNKS / NT;
    constexpr int B_CHUNKS = NB * BN * 2;     // 16-byte chunks of int4 per B k-step
    constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
    static_assert(A_CHUNKS % NT == 0, "A tile must split evenly");
    static_assert(MI >= 1 && NI >= 1, "wave tile must be at least 32x32");

    __shared__ __attribute__((aligned(16))) uint16_t As[BM * 64];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[NB][BN * 64];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int wm0 = (wave / NWN) * WM;
    const int wn0 = (wave % NWN) * WN;
    const int n0 = blockIdx.x * BN;

    // Which rows, which expert.
    const int bid = blockIdx.y;
    int r0, r_end;
    bool shared;
    int e = 0;
    if (bid < args.max_blocks) {
        if (bid >= args.num_blocks[0]) return;
        e = args.block_expert[bid];
        r0 = args.block_row0[bid];
        r_end = args.offsets[e + 1];
        shared = false;
    } else {
        r0 = args.P + (bid - args.max_blocks) * BM;
        r_end = args.P + args.T;
        shared = true;
    }
    const int rows = min(BM, r_end - r0);
    const int K = args.K;
    const int nk = K / 64;

    // Per-thread A sources (row pointers are fixed over K).
    const uint16_t* a_src[A_PER_T];
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
        const int c = tid + i * NT;
        const int row = c / 8;
        a_src[i] = nullptr;
        if (row < rows) {
            const int r = r0 + row;
            int src_row = r;
            if (GATED) src_row = (r < args.P) ? args.sorted_pairs[r] / args.topk : r - args.P;
            a_src[i] = args.a + (size_t)src_row * K + (c % 8) * 8;
        }
    }
    // Per-thread B sources.
    const uint8_t* b_q[B_PER_T];
    const uint16_t* b_s[B_PER_T];
    const uint16_t* b_b[B_PER_T];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
        const int c = tid + i * NT;
        b_q[i] = nullptr;
        if (c < B_CHUNKS) {
            const int m = c / (BN * 2);
            const int rr = (c % (BN * 2)) / 2;
            const int half = c % 2;
            const int n = n0 + rr;
            const size_t mat = shared ? 0 : (size_t)e * args.N;
            const uint8_t* qb = shared ? args.sq[m] : args.q[m];
            const uint16_t* sb = shared ? args.ssc[m] : args.sc[m];
            const uint16_t* bb = shared ? args.sbi[m] : args.bi[m];
            b_q[i] = qb + (mat + n) * (K / 2) + half * 16;
            b_s[i] = sb + (mat + n) * (K / 64);
            b_b[i] = bb + (mat + n) * (K / 64);
        }
    }

    u32x4 a_reg[A_PER_T];
    u32x4 q_reg[B_PER_T];
    uint16_t s_reg[B_PER_T], bb_reg[B_PER_T];

    auto load_tile = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            if (a_src[i]) a_reg[i] = *reinterpret_cast<const u32x4*>(a_src[i] + kt * 64);
            else a_reg[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            if (b_q[i]) {
                q_reg[i] = *reinterpret_cast<const u32x4*>(b_q[i] + kt * 32);
                s_reg[i] = b_s[i][kt];
                bb_reg[i] = b_b[i][kt];
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int c = tid + i * NT;
            const int row = c / 8;
            *reinterpret_cast<u32x4*>(&As[row * 64 + swz(row, c % 8) * 8]) = a_reg[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int c = tid + i * NT;
            if (c < B_CHUNKS) {
                const int m = c / (BN * 2);
                const int rr = (c % (BN * 2)) / 2;
                const int half = c % 2;
                u32x4 w[4];
                dequant32(q_reg[i], bf16_bits_to_float(s_reg[i]), bf16_bits_to_float(bb_reg[i]), w);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<u32x4*>(&Bs[m][rr * 64 + swz(rr, half * 4 + j) * 8]) = w[j];
            }
        }
    };

    f32x16 acc[NB][MI][NI];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.0f;

    load_tile(0);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (kt + 1 < nk) load_tile(kt + 1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int chunk = 2 * s + lane / 32;
            bf16x8 af[MI];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int row = wm0 + 32 * i + lane % 32;
                af[i] = *reinterpret_cast<const bf16x8*>(&As[row * 64 + swz(row, chunk) * 8]);
            }
#pragma unroll
            for (int m = 0; m < NB; ++m) {
#pragma unroll
                for (int j = 0; j < NI; ++j) {
                    const int col = wn0 + 32 * j + lane % 32;
                    const bf16x8 bfr =
                        *reinterpret_cast<const bf16x8*>(&Bs[m][col * 64 + swz(col, chunk) * 8]);
#pragma unroll
                    for (int i = 0; i < MI; ++i)
                        acc[m][i][j] =
                            __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr, acc[m][i][j], 0, 0, 0);
                }
            }
        }
    }

    // Epilogue. C layout of a 32x32 tile: lane l, register r holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int col = n0 + wn0 + 32 * j + lane % 32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm0 + 32 * i + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                if (row < rows) {
                    const size_t o = (size_t)(r0 + row) * args.N + col;
                    if (GATED) {
                        const float g = acc[0][i][j][r];
                        const float u = acc[NB - 1][i][j][r];
                        args.h_out[o] = float_to_bf16_bits(silu(g) * u);
                    } else {
                        args.y_out[o] = acc[0][i][j][r];
                    }
                }
            }
        }
    }
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

template <int BM>
static int launch_gemms(const lily_moe_dims& d, const lily_moe_weights& w, const uint16_t* x,
                        const lily_moe_routing& r, int max_blocks, uint16_t* h, float* y,
                        hipStream_t stream) {
    const int P = d.T * d.topk;
    const int shared_blocks = (d.T + BM - 1) / BM;
    GemmArgs g{};
    g.sorted_pairs = r.sorted_pairs;
    g.topk = d.topk;
    g.block_expert = r.block_expert;
    g.block_row0 = r.block_row0;
    g.num_blocks = r.num_blocks;
    g.offsets = r.offsets;
    g.max_blocks = max_blocks;
    g.P = P;
    g.T = d.T;

    // gate/up + SwiGLU: N = F, K = H
    g.a = x;
    g.q[0] = w.gate.q; g.sc[0] = w.gate.scale; g.bi[0] = w.gate.bias;
    g.q[1] = w.up.q;   g.sc[1] = w.up.scale;   g.bi[1] = w.up.bias;
    g.sq[0] = w.sh_gate.q; g.ssc[0] = w.sh_gate.scale; g.sbi[0] = w.sh_gate.bias;
    g.sq[1] = w.sh_up.q;   g.ssc[1] = w.sh_up.scale;   g.sbi[1] = w.sh_up.bias;
    g.N = d.F;
    g.K = d.H;
    g.h_out = h;
    {
        constexpr int BN = 64;
        dim3 grid(d.F / BN, max_blocks + shared_blocks);
        hipLaunchKernelGGL((grouped_w4_gemm<BM, BN, (BM >= 64 ? 2 : 1), 2, true>), grid,
                           dim3((BM >= 64 ? 2 : 1) * 2 * kWave), 0, stream, g);
        int rc = check_launch("gate_up_gemm");
        if (rc) return rc;
    }

    // down: N = H, K = F
    g.a = h;
    g.sorted_pairs = nullptr;
    g.q[0] = w.down.q; g.sc[0] = w.down.scale; g.bi[0] = w.down.bias;
    g.q[1] = nullptr;  g.sc[1] = nullptr;      g.bi[1] = nullptr;
    g.sq[0] = w.sh_down.q; g.ssc[0] = w.sh_down.scale; g.sbi[0] = w.sh_down.bias;
    g.sq[1] = nullptr;     g.ssc[1] = nullptr;         g.sbi[1] = nullptr;
    g.N = d.H;
    g.K = d.F;
    g.h_out = nullptr;
    g.y_out = y;
    {
        constexpr int BN = 128;
        dim3 grid(d.H / BN, max_blocks + shared_blocks);
        hipLaunchKernelGGL((grouped_w4_gemm<BM, BN, (BM >= 64 ? 2 : 1), 2, false>), grid,
                           dim3((BM >= 64 ? 2 : 1) * 2 * kWave), 0, stream, g);
        int rc = check_launch("down_gemm");
        if (rc) return rc;
    }
    return LILY_OK;
}

int launch_forward(const lily_moe_dims& d, const lily_moe_weights& w, const uint16_t* x,
                   const lily_moe_routing& r, uint16_t* out, void* ws, int max_blocks,
                   hipStream_t stream) {
    const size_t rows = (size_t)d.T * d.topk + d.T;
    uint16_t* h = reinterpret_cast<uint16_t*>(ws);
    float* y = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                        align_up(rows * d.F * sizeof(uint16_t)));
    int rc;
    switch (d.tile_m) {
        case 32: rc = launch_gemms<32>(d, w, x, r, max_blocks, h, y, stream); break;
        case 64: rc = launch_gemms<64>(d, w, x, r, max_blocks, h, y, stream); break;
        case 128: rc = launch_gemms<128>(d, w, x, r, max_blocks, h, y, stream); break;
        default: return set_error(LILY_ERR_UNSUPPORTED, "tile_m %d not supported", d.tile_m);
    }
    if (rc) return rc;
    hipLaunchKernelGGL(combine_kernel, dim3(d.T), dim3(256), 0, stream, y, r.pair_rows, r.topk_w,
                       d.T * d.topk, d.H, d.topk, out);
    return check_launch("combine");
}

}  // namespace lily
