// Residual stream between stacked MoE layers: r += out, then a unit-gain
// RMSNorm of r rounded to bf16 as the next layer's input. The Lily articles
// describe a 40-layer stack but not this glue; a pre-norm residual is the
// reading taken. One workgroup per token; the sum of squares is reduced in a
// fixed order, so the result is deterministic.
#include "common.hpp"

namespace lily {

constexpr int kNormThreads = 256;

__global__ void __launch_bounds__(kNormThreads) residual_norm_kernel(
    int H, float* __restrict__ r, const uint16_t* __restrict__ out, uint16_t* __restrict__ x_next,
    float eps) {
    const int t = blockIdx.x;
    float* rr = r + (size_t)t * H;
    float ss = 0.0f;
    for (int n = threadIdx.x * 4; n < H; n += kNormThreads * 4) {
        f32x4 v = *reinterpret_cast<const f32x4*>(rr + n);
        if (out) {
            const u32x2 o = *reinterpret_cast<const u32x2*>(out + (size_t)t * H + n);
            v[0] += bf16_bits_to_float(o[0] & 0xFFFFu);
            v[1] += bf16_bits_to_float(o[0] >> 16);
            v[2] += bf16_bits_to_float(o[1] & 0xFFFFu);
            v[3] += bf16_bits_to_float(o[1] >> 16);
            *reinterpret_cast<f32x4*>(rr + n) = v;
        }
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    __shared__ float part[kNormThreads / kWave];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kNormThreads / kWave; ++w) tot += part[w];
    const float inv = 1.0f / sqrtf(tot / (float)H + eps);
    for (int n = threadIdx.x * 4; n < H; n += kNormThreads * 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(rr + n);
        u32x2 o;
        o[0] = pack_bf16x2(v[0] * inv, v[1] * inv);
        o[1] = pack_bf16x2(v[2] * inv, v[3] * inv);
        *reinterpret_cast<u32x2*>(x_next + (size_t)t * H + n) = o;
    }
}

int launch_residual_norm(int T, int H, float* r, const uint16_t* out, uint16_t* x_next, float eps,
                         hipStream_t stream) {
    hipLaunchKernelGGL(residual_norm_kernel, dim3(T), dim3(kNormThreads), 0, stream, H, r, out,
                       x_next, eps);
    return check_launch("residual_norm");
}

}  // namespace lily
