// GPU-resident routing of one MoE layer (gfx950).
//
// The Lily articles keep the routing histogram, the prefix scan, the scatter
// and the block map inside one GPU command stream so that no MoE layer waits
// for the CPU (news.ainew.jp Lily article, section "Prefill"); the router
// itself scores E experts and keeps k (section on the three workload shapes).
//
// Two kernels on one stream, no host synchronisation:
//   route_topk:   one wavefront per token. Each lane holds E/64 logits as
//                 64-bit keys (order-preserving float bits, then the inverted
//                 expert index so that equal logits prefer the lower index);
//                 k rounds of a wavefront arg-max pick the experts in
//                 descending order; the softmax over the k picked logits runs
//                 in slot order. Writes topk_ids and topk_w.
//   route_finish: one 1024-thread workgroup. 16 wavefronts split the T*k
//                 (token, slot) pairs into contiguous spans. Pass 1 builds a
//                 per-wavefront histogram in LDS; ranks inside a span are
//                 found 64 pairs at a time with ballots over the expert-id
//                 bits (lanes holding the same expert form one group). Then
//                 per-expert bases across wavefronts, the exclusive scans of
//                 rows and of blocks, the block map, and pass 2, which
//                 re-walks each span and writes every pair to
//                 offsets[e] + (rows of e in earlier spans) + (earlier pairs
//                 of e in this span). This is a stable counting sort: no
//                 atomics, so the result is deterministic and bit-exact.
// For small T the top-k runs inside route_finish and the route is one launch.
#include "common.hpp"

namespace lily {

constexpr int kFinishThreads = 1024;
constexpr int kFinishWaves = kFinishThreads / kWave;
constexpr int kTopkThreads = 256;
constexpr int kTopkTokensPerWave = 4;
constexpr int kTopkTokensPerBlock = (kTopkThreads / kWave) * kTopkTokensPerWave;
constexpr int kMaxPerLane = kMaxExperts / kWave;
// Up to this many tokens the whole route runs in the single workgroup.
constexpr int kFusedRouteMaxT = 64;

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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, off, kWave);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, kWave);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// Top-k and softmax of one token by one wavefront.
__device__ __forceinline__ void topk_one_token(const float* __restrict__ logits, int t, int E,
                                               int k, int32_t* __restrict__ topk_ids,
                                               float* __restrict__ topk_w) {
    const int lane = threadIdx.x % kWave;
    const float* row = logits + (size_t)t * E;
    uint64_t key[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        int e = lane + i * kWave;
        key[i] = 0;  // below every real key
        if (e < E) key[i] = ((uint64_t)ordered_bits(row[e]) << 32) | (uint32_t)(~(uint32_t)e);
    }
    int my_id = 0;
    float my_l = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
            if (key[i] == best) key[i] = 0;  // unique: the low word names the expert
        if (lane == j) {
            my_id = (int)(~(uint32_t)best);
            my_l = from_ordered_bits((uint32_t)(best >> 32));
        }
    }
    // softmax over the selected logits, summed in slot order
    const float l0 = __shfl(my_l, 0, kWave);
    const float ex = expf(my_l - l0);
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += __shfl(ex, j, kWave);
    if (lane < k) {
        topk_ids[(size_t)t * k + lane] = my_id;
        topk_w[(size_t)t * k + lane] = ex / sum;
    }
}

__global__ void __launch_bounds__(kTopkThreads) route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w) {
    const int wave = threadIdx.x / kWave;
    const int t0 = blockIdx.x * kTopkTokensPerBlock + wave * kTopkTokensPerWave;
    for (int i = 0; i < kTopkTokensPerWave; ++i) {
        const int t = t0 + i;
        if (t < T) topk_one_token(logits, t, E, k, topk_ids, topk_w);
    }
}

// Lanes of the wavefront holding the same expert id as this lane (ids are
// below 2^nbits; lanes with id < 0 match nobody).
__device__ __forceinline__ uint64_t match_same(int id, int nbits) {
    uint64_t m = __ballot(id >= 0);
    for (int b = 0; b < nbits; ++b) {
        uint64_t bit = __ballot(id >= 0 && ((id >> b) & 1));
        m &= ((id >> b) & 1) ? bit : ~bit;
    }
    return id >= 0 ? m : 0ull;
}

__global__ void __launch_bounds__(kFinishThreads) route_finish_kernel(
    const float* __restrict__ logits, int T, int E, int k, int M, int fused_topk,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_rows, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ block_row0, int32_t* __restrict__ num_blocks) {
    __shared__ int32_t hist[kFinishWaves][kMaxExperts];  // per-span rows, then bases
    __shared__ int32_t s_off[kMaxExperts + 1];            // row offsets
    __shared__ int32_t s_bst[kMaxExperts + 1];            // block starts
    __shared__ int32_t s_wsum[2][kFinishWaves];

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int P = T * k;
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;

    if (fused_topk) {
        for (int t = wave; t < T; t += kFinishWaves) topk_one_token(logits, t, E, k, topk_ids, topk_w);
        __threadfence_block();
    }
    for (int i = tid; i < kFinishWaves * kMaxExperts; i += kFinishThreads) (&hist[0][0])[i] = 0;
    __syncthreads();

    // Contiguous span of pairs per wavefront, a multiple of 64.
    const int span = ((P + kFinishWaves - 1) / kFinishWaves + kWave - 1) / kWave * kWave;
    const int p_begin = wave * span;
    const int p_end = min(P, p_begin + span);
    const uint64_t below = (1ull << lane) - 1ull;

    // Pass 1: rows per expert in each span.
    for (int c = p_begin; c < p_end; c += kWave) {
        const int p = c + lane;
        const int e = p < p_end ? topk_ids[p] : -1;
        const uint64_t same = match_same(e, nbits);
        if (e >= 0 && (same & below) == 0ull)  // lowest lane of its group
            hist[wave][e] += __popcll(same);
    }
    __syncthreads();

    // Per-expert totals, and each span's base inside its expert.
    for (int e = tid; e < E; e += kFinishThreads) {
        int run = 0;
        for (int w = 0; w < kFinishWaves; ++w) {
            const int c = hist[w][e];
            hist[w][e] = run;
            run += c;
        }
        counts[e] = run;
        s_off[e] = run;
        s_bst[e] = (run + M - 1) / M;
    }
    __syncthreads();

    // Exclusive scans of rows (s_off) and blocks (s_bst) over the experts:
    // each thread owns one expert (E <= 512 < 1024 threads).
    {
        const int e = tid;
        int v_rows = e < E ? s_off[e] : 0;
        int v_blks = e < E ? s_bst[e] : 0;
        int inc_r = v_rows, inc_b = v_blks;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int r = __shfl_up(inc_r, off, kWave);
            const int b = __shfl_up(inc_b, off, kWave);
            if (lane >= off) {
                inc_r += r;
                inc_b += b;
            }
        }
        if (lane == kWave - 1) {
            s_wsum[0][wave] = inc_r;
            s_wsum[1][wave] = inc_b;
        }
        __syncthreads();
        int base_r = 0, base_b = 0;
        for (int w = 0; w < wave; ++w) {
            base_r += s_wsum[0][w];
            base_b += s_wsum[1][w];
        }
        __syncthreads();
        if (e < E) {
            s_off[e] = base_r + inc_r - v_rows;
            s_bst[e] = base_b + inc_b - v_blks;
        }
        if (e == E - 1) {
            s_off[E] = base_r + inc_r;
            s_bst[E] = base_b + inc_b;
        }
    }
    __syncthreads();

    for (int e = tid; e <= E; e += kFinishThreads) offsets[e] = s_off[e];
    const int nb = s_bst[E];
    if (tid == 0) num_blocks[0] = nb;

    // Block map: block b belongs to the last expert whose block start is <= b.
    for (int b = tid; b < nb; b += kFinishThreads) {
        int lo = 0, hi = E;  // invariant: s_bst[lo] <= b < s_bst[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_bst[mid] <= b) lo = mid; else hi = mid;
        }
        block_expert[b] = lo;
        block_row0[b] = s_off[lo] + (b - s_bst[lo]) * M;
    }

    // Pass 2: stable positions.
    for (int c = p_begin; c < p_end; c += kWave) {
        const int p = c + lane;
        const int e = p < p_end ? topk_ids[p] : -1;
        const uint64_t same = match_same(e, nbits);
        if (e >= 0) {
            const int base = hist[wave][e];
            const int row = s_off[e] + base + __popcll(same & below);
            sorted_pairs[row] = p;
            pair_rows[p] = row;
            // the highest lane of the group advances the span's cursor
            if ((same >> lane) == 1ull) hist[wave][e] = base + __popcll(same);
        }
    }
}

int launch_route(const lily_moe_dims& d, const float* logits, const lily_moe_routing& r,
                 hipStream_t stream) {
    const int fused = d.T <= kFusedRouteMaxT;
    if (!fused) {
        const int grid = (d.T + kTopkTokensPerBlock - 1) / kTopkTokensPerBlock;
        hipLaunchKernelGGL(route_topk_kernel, dim3(grid), dim3(kTopkThreads), 0, stream, logits,
                           d.T, d.E, d.topk, r.topk_ids, r.topk_w);
        int rc = check_launch("route_topk");
        if (rc) return rc;
    }
    hipLaunchKernelGGL(route_finish_kernel, dim3(1), dim3(kFinishThreads), 0, stream, logits, d.T,
                       d.E, d.topk, d.tile_m, fused, r.topk_ids, r.topk_w, r.counts, r.offsets,
                       r.sorted_pairs, r.pair_rows, r.block_expert, r.block_row0, r.num_blocks);
    return check_launch("route_finish");
}

}  // namespace lily
