// Router projection: logits = x Wr^T (gfx950).
//
// The router scores every expert for each token before the top-k (Lily
// articles, section on the three workload shapes). With bf16 activations and
// bf16 router weights every product is exact in fp32, so the projection is a
// bf16 MFMA with fp32 accumulation; only the order of the fp32 sums differs
// from a sequential dot product.
//
// One workgroup: a 32-token x 32-expert tile; its four wavefronts split K in
// quarters, one v_mfma_f32_32x32x16_bf16 per 16 k, and add their partial
// tiles through LDS in wavefront order. A wavefront moves its operands in
// rounds of 64 k: each row's 128 bytes are loaded by two lanes with 16-byte
// loads (whole cache lines), written to its own LDS area (rows padded to
// 144 bytes, so the fragment reads are free of bank conflicts) and read back
// as MFMA fragments. Loads run kRouterDepth rounds ahead. No workgroup
// barrier until the final sum: each wavefront only reads what it wrote, and
// a wavefront's LDS accesses run in order.
#include "common.hpp"

namespace lily {

constexpr int kRouterThreads = 256;
constexpr int kRouterTile = 32;
constexpr int kRouterRoundK = 64;                        // k per round
constexpr int kRouterRowBytes = kRouterRoundK * 2 + 16;  // padded LDS row
constexpr int kRouterChunks = kRouterRoundK / 8 / 2;     // 16-byte chunks per lane per round
constexpr int kRouterDepth = 4;                          // rounds in flight
constexpr int kRouterWaves = kRouterThreads / kWave;

__global__ void __launch_bounds__(kRouterThreads) router_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w,
                                                                float* __restrict__ logits, int T,
                                                                int H, int E) {
    __shared__ __attribute__((aligned(16))) char s_tile[kRouterWaves][2][kRouterTile * kRouterRowBytes];
    __shared__ float s_part[kRouterWaves - 1][16][kWave];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    // Workgroup id -> (token tile, expert tile) so that the expert tiles of
    // one token tile share an id residue mod 8: dispatch deals ids round robin
    // over the 8 XCDs, so they meet the token rows in one L2.
    const int n_et = (E + kRouterTile - 1) / kRouterTile;
    const int id = blockIdx.x, xcd = id % 8, q = id / 8;
    const int tt = (q / n_et) * 8 + xcd, et = q % n_et;
    if (tt * kRouterTile >= T) return;  // the same in the whole workgroup
    const int t0 = tt * kRouterTile, e0 = et * kRouterTile;
    const int kq = H / 4;                    // this wavefront's K quarter (H % 64 == 0)
    const int rounds = kq / kRouterRoundK;
    // loads: lane (row l / 2, half l % 2) moves 64 bytes of the row per round
    const int lr = lane / 2, lh = lane % 2;
    const u32x4* xg = reinterpret_cast<const u32x4*>(x + (size_t)min(t0 + lr, T - 1) * H + wave * kq) + kRouterChunks * lh;
    const u32x4* wg = reinterpret_cast<const u32x4*>(w + (size_t)min(e0 + lr, E - 1) * H + wave * kq) + kRouterChunks * lh;
    char* tx = s_tile[wave][0];
    char* tw = s_tile[wave][1];
    // fragments: lane (r, kh) reads row r, 16-byte chunk 2 u + kh of step u
    const int r = lane % 32, kh = lane / 32;
    f32x16 acc = {};
    u32x4 gx[kRouterDepth][kRouterChunks], gw[kRouterDepth][kRouterChunks];
#pragma unroll
    for (int d = 0; d < kRouterDepth; ++d) {
        const int rr = min(d, rounds - 1);  // rounds past the end repeat the last
#pragma unroll
        for (int c = 0; c < kRouterChunks; ++c) {
            gx[d][c] = xg[rr * 2 * kRouterChunks + c];
            gw[d][c] = wg[rr * 2 * kRouterChunks + c];
        }
    }
    // Register set d holds round rd + d; after it is written to LDS it is
    // refilled with round rd + d + kRouterDepth, so the sets rotate without
    // moving registers that have loads in flight.
    for (int rd = 0; rd < rounds; rd += kRouterDepth) {
#pragma unroll
        for (int d = 0; d < kRouterDepth; ++d) {
            if (rd + d < rounds) {
#pragma unroll
                for (int c = 0; c < kRouterChunks; ++c) {
                    *reinterpret_cast<u32x4*>(tx + lr * kRouterRowBytes + (kRouterChunks * lh + c) * 16) = gx[d][c];
                    *reinterpret_cast<u32x4*>(tw + lr * kRouterRowBytes + (kRouterChunks * lh + c) * 16) = gw[d][c];
                }
                const int rr = min(rd + d + kRouterDepth, rounds - 1);
#pragma unroll
                for (int c = 0; c < kRouterChunks; ++c) {
                    gx[d][c] = xg[rr * 2 * kRouterChunks + c];
                    gw[d][c] = wg[rr * 2 * kRouterChunks + c];
                }
#pragma unroll
                for (int u = 0; u < kRouterRoundK / 16; ++u) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(tx + r * kRouterRowBytes + (2 * u + kh) * 16);
                    const u32x4 b = *reinterpret_cast<const u32x4*>(tw + r * kRouterRowBytes + (2 * u + kh) * 16);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                  __builtin_bit_cast(bf16x8, b), acc,
                                                                  0, 0, 0);
                }
            }
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s_part[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave > 0) return;
    // C layout: register i of lane l holds row 8 (i / 4) + 4 (l / 32) + i % 4,
    // column l % 32.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float v = acc[i];
#pragma unroll
        for (int q = 0; q < kRouterWaves - 1; ++q) v += s_part[q][i][lane];
        const int t = t0 + 8 * (i / 4) + 4 * kh + i % 4;
        const int e = e0 + r;
        if (t < T && e < E) logits[(size_t)t * E + e] = v;
    }
}

int launch_router(const lily_moe_dims& d, const uint16_t* w_router, const uint16_t* x,
                  float* logits, hipStream_t stream) {
    const int n_tt = (d.T + kRouterTile - 1) / kRouterTile, n_et = (d.E + kRouterTile - 1) / kRouterTile;
    const dim3 grid((unsigned)(((n_tt + 7) / 8) * 8 * n_et));
    hipLaunchKernelGGL(router_kernel, grid, dim3(kRouterThreads), 0, stream, x, w_router, logits,
                       d.T, d.H, d.E);
    return check_launch("router");
}

}  // namespace lily
