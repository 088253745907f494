// The packed int4 weight layout and the dequantisation shared by the grouped
// GEMMs and the fused decode kernel (gfx950 only).
//
// The weights are groupwise-affine 4-bit: 64 weights of a row share one bf16
// scale and one bf16 bias, and are rebuilt as bf16 before the products
// (Lily articles, section "Prefill"); w = bf16(scale * q + bias).
#pragma once

#include "common.hpp"

namespace lily {

// Packed weight layout (lily_w4_pack): one block per (expert, 128-row slab,
// group of 64 k); q as [2 halves][128 rows][16 bytes], then the 128 scales,
// then the 128 biases.
constexpr int kPackRows = 128;
constexpr int kPackQ = 4096;
constexpr int kPackBlock = 4608;

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

}  // namespace lily
