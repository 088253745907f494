// Calibration kernels: the achievable peaks of the device, against which the
// MoE kernels' rooflines are also reported (MFMA throughput on changing
// operands, streaming HBM reads, and the shader clock under that load).
#include "gemm_common.hpp"

namespace lily {

__device__ __forceinline__ uint32_t calib_hash(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// Every wavefront runs `iters` rounds of 8 independent
// v_mfma_f32_32x32x16_bf16 on 8 accumulators. The operands are per-lane
// random bf16 values in [1, 2) and [2^-7, 2^-6); rounds alternate between two
// operand sets, so the matrix core multiplies changing data (an all-constant
// operand draws less power and runs at a higher clock). Lane 0 records the
// wavefront's shader-clock cycles (s_memtime) and 100 MHz wall ticks
// (s_memrealtime) over the loop.
__global__ void __launch_bounds__(512) calib_mfma_kernel(int iters, float* sink,
                                                         unsigned long long* times) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    uint32_t seed = calib_hash(blockIdx.x * 4096u + threadIdx.x + 1u);
    bf16x8 a[2][4], b[2][2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 t;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                seed = calib_hash(seed);
                t[j] = 0x3F803F80u | (seed & 0x007F007Fu);
            }
            a[v][i] = __builtin_bit_cast(bf16x8, t);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            u32x4 t;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                seed = calib_hash(seed);
                t[j] = 0x3C003C00u | (seed & 0x007F007Fu);
            }
            b[v][i] = __builtin_bit_cast(bf16x8, t);
        }
    }
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[v][j & 3], b[v][j >> 2], acc[j], 0, 0, 0);
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (lane == 0) {
        unsigned long long* tt = times + ((size_t)blockIdx.x * (blockDim.x / kWave) + wave) * 2;
        tt[0] = t1 - t0;
        tt[1] = r1 - r0;
    }
}

// Streaming read of n16 16-byte words, grid-stride, XOR-reduced per thread
// into sink (so that no load is dead). dma = 1: the loads go to LDS by LDS
// DMA (global_load_lds_dwordx4, as the GEMMs load their operands), four
// 1 KB loads in flight per wavefront before each wait; dma = 0: plain
// global_load_dwordx4 into registers.
__global__ void __launch_bounds__(256) calib_read_kernel(const u32x4* __restrict__ src,
                                                         size_t n16, int dma,
                                                         uint32_t* __restrict__ sink) {
    __shared__ __attribute__((aligned(16))) char lds[4][4][kWave * 16];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint32_t x = 0;
    if (!dma) {
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += 4 * stride) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = i + u * stride < n16 ? src[i + u * stride] : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < 4; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        }
    } else {
        // Each wavefront moves whole 1 KB runs (64 lanes x 16 bytes); runs
        // are dealt round robin over all wavefronts of the grid, four at a
        // time. n16 is a multiple of 64 (checked on the host).
        const size_t runs = n16 / kWave;
        const size_t waves = stride / kWave;
        const size_t w0 = (size_t)blockIdx.x * (blockDim.x / kWave) + wave;
        const uint32_t base = (uint32_t)(size_t)&lds[wave][0][0];
        for (size_t r = w0; r < runs; r += 4 * waves) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const size_t rr = r + u * waves < runs ? r + u * waves : r;
                dma16(src + rr * kWave, (uint32_t)lane * 16u, base + u * kWave * 16);
            }
            wait_vmcnt<0>();
            const u32x4* l = reinterpret_cast<const u32x4*>(&lds[wave][0][0]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x4 v = l[u * kWave + lane];
                x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
            }
        }
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// The grouped GEMMs' weight rebuild (dequant8: 8 int4 weights -> 4 bf16x2
// words of bf16(scale * q + bias)) alone: every wavefront runs `iters`
// rounds over 8 independent words per lane. Per word and round: one add that
// changes the word (so that no round can be hoisted), dequant8, and two
// 3-input sums that keep all four results live; 8 weights per word. Lane 0
// records the wavefront's shader-clock cycles and wall ticks over the loop.
__global__ void __launch_bounds__(1024) calib_dequant_kernel(int iters, uint32_t* sink,
                                                             unsigned long long* times) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    uint32_t seed = calib_hash(blockIdx.x * 4096u + threadIdx.x + 1u);
    uint32_t w[8], acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        seed = calib_hash(seed);
        w[j] = seed;
        acc[j] = 0;
    }
    seed = calib_hash(seed);
    const float s512 = (1.0f + (seed & 0xFF) * (1.0f / 256)) * 0.01f * 512.0f;
    const float bias = ((int)((seed >> 8) & 0xFF) - 128) * (1.0f / 16384);
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            w[j] += 0x13579BDFu;
            uint32_t o[4];
            dequant8(w[j], s512, bias, o);
            acc[j] += o[0] + o[1];
            acc[j] += o[2] + o[3];
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) x ^= acc[j];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
    if (lane == 0) {
        unsigned long long* tt = times + ((size_t)blockIdx.x * (blockDim.x / kWave) + wave) * 2;
        tt[0] = t1 - t0;
        tt[1] = r1 - r0;
    }
}

}  // namespace lily

using namespace lily;

extern "C" {

int lily_calib_mfma(int32_t grid, int32_t waves_per_cu, int32_t iters, float* sink,
                    unsigned long long* times, void* stream) {
    if (grid < 1 || waves_per_cu < 1 || waves_per_cu > 8 || iters < 2 || iters % 2)
        return set_error(LILY_ERR_INVALID_ARG,
                         "calib_mfma: grid %d >= 1, waves %d in 1..8, iters %d even and >= 2",
                         grid, waves_per_cu, iters);
    if (!sink || !times) return set_error(LILY_ERR_INVALID_ARG, "calib_mfma: NULL buffer");
    hipLaunchKernelGGL(calib_mfma_kernel, dim3(grid), dim3(waves_per_cu * kWave), 0,
                       reinterpret_cast<hipStream_t>(stream), iters, sink, times);
    return check_launch("calib_mfma");
}

int lily_calib_dequant(int32_t grid, int32_t waves_per_cu, int32_t iters, uint32_t* sink,
                       unsigned long long* times, void* stream) {
    if (grid < 1 || waves_per_cu < 1 || waves_per_cu > 16 || iters < 1)
        return set_error(LILY_ERR_INVALID_ARG,
                         "calib_dequant: grid %d >= 1, waves %d in 1..16, iters %d >= 1", grid,
                         waves_per_cu, iters);
    if (!sink || !times) return set_error(LILY_ERR_INVALID_ARG, "calib_dequant: NULL buffer");
    hipLaunchKernelGGL(calib_dequant_kernel, dim3(grid), dim3(waves_per_cu * kWave), 0,
                       reinterpret_cast<hipStream_t>(stream), iters, sink, times);
    return check_launch("calib_dequant");
}

int lily_calib_read(const void* src, size_t bytes, int32_t grid, int32_t dma, uint32_t* sink,
                    void* stream) {
    if (!src || !sink || grid < 1 || bytes == 0 || bytes % 1024 || ((uintptr_t)src & 15))
        return set_error(LILY_ERR_INVALID_ARG,
                         "calib_read: src/sink non-NULL, src 16-byte aligned, bytes a positive "
                         "multiple of 1024, grid >= 1");
    hipLaunchKernelGGL(calib_read_kernel, dim3(grid), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       bytes / 16, dma ? 1 : 0, sink);
    return check_launch("calib_read");
}

}  // extern "C"
