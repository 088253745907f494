// Top-k and softmax of one token by one wavefront, shared by the route
// kernels and the fused decode kernel (gfx950 only).
//
// The router keeps the k largest of E logits per token (Lily articles,
// section on the three workload shapes); the readings: larger logit first,
// equal logits (-0.0 and +0.0 equal) to the lower expert index, weights a
// softmax over the k selected logits summed in slot order.
#pragma once

#include "common.hpp"

namespace lily {

constexpr int kMaxPerLane = kMaxExperts / kWave;

// Order-preserving map of a float to uint32; -0.0 is folded onto +0.0 so
// that the two tie.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

// Maximum of a uint32 over the 64 lanes, returned uniformly: DPP within each
// row of 16 lanes (quad swaps, then rotations by 4 and 8), then the four row
// results through readlane. No LDS traffic.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false)); // row_ror 4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false)); // row_ror 8
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

// The k largest of one token's logits and their softmax, by one wavefront,
// from lv: lane l holds the logits of experts l, l + 64, ... (NPER =
// ceil(E / 64) per lane; entries past E are ignored). They become
// order-preserving keys; a taken expert's key becomes 0, below every real
// key. Each round takes the wavefront maximum and, among the experts holding
// it, the lowest index (ballots in expert order). Lane j < k receives slot
// j: my_id and my_w.
template <int NPER>
__device__ __forceinline__ void topk_select(const float (&lv)[NPER], int E, int k, int& my_id,
                                            float& my_w) {
    const int lane = threadIdx.x % kWave;
    uint32_t key[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) key[i] = (lane + i * kWave < E) ? ordered_bits(lv[i]) : 0u;
    my_id = 0;
    float my_l = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint32_t best = key[0];
#pragma unroll
        for (int i = 1; i < NPER; ++i) best = max(best, key[i]);
        best = wave_max_u32(best);
        int e_sel = 0;
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
            const uint64_t hit = __ballot(key[i] == best);
            if (hit) {
                e_sel = i * kWave + (int)__ffsll((long long)hit) - 1;
                break;
            }
        }
        if (lane == e_sel % kWave) {
#pragma unroll
            for (int i = 0; i < NPER; ++i)
                if (i == e_sel / kWave) key[i] = 0u;
        }
        if (lane == j) {
            my_id = e_sel;
            my_l = from_ordered_bits(best);
        }
    }
    // softmax over the selected logits, summed in slot order
    const float l0 = __shfl(my_l, 0, kWave);
    const float ex = expf(my_l - l0);
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), j));
    my_w = ex / sum;
}

// Loads token t's logits for topk_select. Every lane issues all its loads
// before the first use (indexes clamped into the row, so none is
// conditional); a load per branch would wait for each one in turn.
template <int NPER>
__device__ __forceinline__ void topk_load(const float* __restrict__ logits, int t, int E,
                                          float (&lv)[NPER]) {
    const int lane = threadIdx.x % kWave;
    const float* row = logits + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int e = lane + i * kWave;
        lv[i] = row[e < E ? e : E - 1];
    }
}

// Top-k and softmax of one token by one wavefront (topk_load, topk_select),
// written to topk_ids / topk_w [t * k + slot]. hist, when not null, counts
// the chosen experts (integer atomics: the totals do not depend on their
// order).
template <int NPER>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int t, int E, int k,
                                           int32_t* __restrict__ topk_ids,
                                           float* __restrict__ topk_w, int32_t* hist) {
    const int lane = threadIdx.x % kWave;
    float lv[NPER];
    topk_load<NPER>(logits, t, E, lv);
    int my_id;
    float my_w;
    topk_select<NPER>(lv, E, k, my_id, my_w);
    if (lane < k) {
        topk_ids[(size_t)t * k + lane] = my_id;
        topk_w[(size_t)t * k + lane] = my_w;
        if (hist) atomicAdd(hist + my_id, 1);
    }
}

// Top-k and softmax of token t (E <= kMaxExperts) by one wavefront.
__device__ __forceinline__ void topk_one_token(const float* __restrict__ logits, int t, int E,
                                               int k, int32_t* __restrict__ topk_ids,
                                               float* __restrict__ topk_w,
                                               int32_t* hist = nullptr) {
    switch ((E + kWave - 1) / kWave) {
        case 1: topk_token<1>(logits, t, E, k, topk_ids, topk_w, hist); break;
        case 2: topk_token<2>(logits, t, E, k, topk_ids, topk_w, hist); break;
        case 3: topk_token<3>(logits, t, E, k, topk_ids, topk_w, hist); break;
        case 4: topk_token<4>(logits, t, E, k, topk_ids, topk_w, hist); break;
        case 5: topk_token<5>(logits, t, E, k, topk_ids, topk_w, hist); break;
        case 6: topk_token<6>(logits, t, E, k, topk_ids, topk_w, hist); break;
        case 7: topk_token<7>(logits, t, E, k, topk_ids, topk_w, hist); break;
        default: topk_token<kMaxPerLane>(logits, t, E, k, topk_ids, topk_w, hist); break;
    }
}

}  // namespace lily
