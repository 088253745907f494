// GPU-resident routing of one MoE layer (gfx950).
//
// The Lily articles keep the routing histogram, the prefix scan, the scatter
// and the block map inside one GPU command stream so that no MoE layer waits
// for the CPU (news.ainew.jp Lily article, section "Prefill"); the router
// itself scores E experts and keeps k (section on the three workload shapes).
//
// Two kernels on one stream, no host synchronisation:
//   route_topk:   one wavefront per token. Each lane holds E/64 logits as
//                 order-preserving 32-bit keys; each of k rounds takes the
//                 wavefront maximum (DPP inside rows of 16 lanes, readlane
//                 across rows) and, among the experts holding it, the lowest
//                 index (ballots in expert order). The softmax over the k
//                 picked logits runs in slot order. Writes topk_ids, topk_w.
//   route_topk also counts each part's experts (parts of >= 128
//                 consecutive tokens, at most 64) into histograms in sched.
//   route_finish: one 1024-thread workgroup per part. Each takes the rows
//                 of earlier parts from the histograms; workgroup 0 alone
//                 writes counts, offsets, the block map and the schedule.
//                 Inside a part, 16 wavefronts split the tokens into
//                 contiguous spans. Pass 1 counts rows per
//                 expert per span (integer LDS atomics). Then per-expert
//                 bases across spans, the exclusive scans of rows and of
//                 blocks, the block map, and pass 2, which re-walks each span
//                 in chunks of whole tokens and writes every pair to
//                 offsets[e] + (rows of e in earlier spans) + (earlier pairs
//                 of e in this span); inside a chunk the earlier pairs come
//                 from a per-expert token bitmask. This is a stable counting
//                 sort whose result does not depend on the order of any
//                 atomic: deterministic and bit-exact. It also writes the
//                 schedule of the grouped GEMMs (block_order: full blocks in
//                 block order, then each expert's last, partial block by
//                 descending size class, ties in expert order), the same
//                 schedule resolved to (expert, first row, rows, block) in
//                 block_info, and clears their work-queue counters.
// For small T the top-k runs inside route_finish and the route is one launch.
#include "common.hpp"
#include "topk.hpp"

namespace lily {

constexpr int kFinishThreads = 1024;
constexpr int kFinishWaves = kFinishThreads / kWave;
constexpr int kTopkThreads = 256;
constexpr int kTopkTokensPerWave = 1;
constexpr int kTopkTokensPerBlock = (kTopkThreads / kWave) * kTopkTokensPerWave;
// Up to this many tokens the whole route runs in the single workgroup.
constexpr int kFusedRouteMaxT = 64;
// Chunks of 64 ids a wavefront loads at once in route_finish.
constexpr int kBatch = 16;
// Above kFusedRouteMaxT tokens route_finish runs one workgroup per part of
// at least kMinPartTokens consecutive tokens (at most kMaxParts parts).
constexpr int kMinPartTokens = 128;

static int part_tokens_for(int T) {
    const int s = (T + kMaxParts - 1) / kMaxParts;
    return s < kMinPartTokens ? kMinPartTokens : s;
}

// part_counts (may be null): per-part expert histograms; row t / part_tokens
// counts token t's experts.
__global__ void __launch_bounds__(kTopkThreads) route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int32_t* part_counts, int part_tokens) {
    const int wave = threadIdx.x / kWave;
    const int t0 = blockIdx.x * kTopkTokensPerBlock + wave * kTopkTokensPerWave;
    for (int i = 0; i < kTopkTokensPerWave; ++i) {
        const int t = t0 + i;
        if (t < T)
            topk_one_token(logits, t, E, k, topk_ids, topk_w,
                           part_counts ? part_counts + (t / part_tokens) * E : nullptr);
    }
}

// Workgroup barrier that waits for this thread's LDS accesses only. Global
// stores stay in flight: nothing in route_finish reads back what another
// thread of it stored (__syncthreads would wait for every store to reach
// memory first, a round trip per barrier).
__device__ __forceinline__ void lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Inclusive prefix sum over the 64 lanes of a wavefront: DPP shifts inside
// each row of 16 lanes (out-of-row sources read 0), then the row totals
// from lanes 15, 31, 47 added to the later rows. No LDS traffic.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr 1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr 2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr 4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr 8
    const int row = (threadIdx.x % kWave) / 16;
    const int t0 = __builtin_amdgcn_readlane(x, 15);
    const int t1 = __builtin_amdgcn_readlane(x, 31);
    const int t2 = __builtin_amdgcn_readlane(x, 47);
    return x + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// Exclusive prefix sums of NV values per thread over the 1024-thread
// workgroup, in thread order; tot[i] receives the sum of value i over all
// threads. The 16 wavefront totals of each value are scanned by the lanes
// of every wavefront (one LDS read per value). Every thread of the
// workgroup must call it.
// Only the first nw wavefronts hold values (the others' threads pass zeros
// and get zeros back): the scan runs on those alone, so that idle
// wavefronts do not share the SIMDs' issue slots with it.
template <int NV>
__device__ __forceinline__ void block_exclusive_scan(const int (&v)[NV], int (&ex)[NV],
                                                     int (&tot)[NV], int32_t* s_wsum, int nw) {
    static_assert(kFinishWaves == 16, "one 16-lane row scans the wavefront totals");
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const bool active = wave < nw;
    int inc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        inc[i] = active ? wave_inclusive_scan(v[i]) : 0;
        ex[i] = tot[i] = 0;
    }
    if (active && lane == kWave - 1) {
#pragma unroll
        for (int i = 0; i < NV; ++i) s_wsum[i * kFinishWaves + wave] = inc[i];
    }
    lds_sync();
    if (active) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int ws = wave_inclusive_scan(lane < nw ? s_wsum[i * kFinishWaves + lane] : 0);
            const int base = wave > 0 ? __builtin_amdgcn_readlane(ws, wave - 1) : 0;
            tot[i] = __builtin_amdgcn_readlane(ws, kFinishWaves - 1);
            ex[i] = base + inc[i] - v[i];
        }
    }
    lds_sync();
}

__global__ void __launch_bounds__(kFinishThreads) route_finish_kernel(
    const float* __restrict__ logits, int T, int E, int k, int M, int fused_topk,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_rows, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ block_row0, int32_t* __restrict__ num_blocks,
    int32_t* __restrict__ block_order, int32_t* __restrict__ sched,
    int32_t* __restrict__ block_info, int32_t* __restrict__ part_counts, int part_tokens) {
    __shared__ int32_t hist[kFinishWaves][kMaxExperts];    // rows per span, then cursors
    __shared__ uint32_t cmask[kFinishWaves][kMaxExperts];  // tokens of a chunk, per expert
    __shared__ int32_t s_off[kMaxExperts + 1];             // row offsets
    __shared__ int32_t s_bst[kMaxExperts + 1];             // block starts
    __shared__ int32_t s_fst[kMaxExperts];                 // full blocks of earlier experts
    __shared__ int32_t s_wsum[7 * kFinishWaves];

    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    // With part_counts, workgroup q places the pairs of tokens [T0, T1) and
    // takes the rows of earlier parts from the histograms the top-k kernel
    // counted; workgroup 0 also writes the per-expert results, the block map
    // and the schedule. Without, one workgroup routes all T tokens.
    const int parts = gridDim.x, q = blockIdx.x;
    const bool lead = q == 0;
    const int T0 = part_counts ? q * part_tokens : 0;
    const int T1 = part_counts ? min(T, T0 + part_tokens) : T;

    if (fused_topk) {
        for (int t = wave; t < T; t += kFinishWaves) topk_one_token(logits, t, E, k, topk_ids, topk_w);
        __threadfence_block();
    }
    for (int i = tid; i < kFinishWaves * kMaxExperts; i += kFinishThreads) {
        (&hist[0][0])[i] = 0;
        (&cmask[0][0])[i] = 0u;
    }
    __syncthreads();

    // Chunks of tpc whole tokens (tpc * k <= 64 pairs, tpc <= 32); each
    // wavefront owns a contiguous span of chunks, spans in token order.
    const int tpc = min(32, kWave / k);
    const int cpairs = tpc * k;
    const int n_chunks = (T1 - T0 + tpc - 1) / tpc;
    const int chunks_per_wave = (n_chunks + kFinishWaves - 1) / kFinishWaves;
    const int t_begin = min(T1, T0 + wave * chunks_per_wave * tpc);
    const int t_end = min(T1, t_begin + chunks_per_wave * tpc);
    const int p_begin = t_begin * k;
    const int p_end = t_end * k;
    const bool lane_in_chunk = lane < cpairs;

    // Pass 1: rows per expert in each span (integer LDS atomics: the totals
    // do not depend on their order). When the span is one batch, its ids
    // stay in registers for pass 2.
    const bool one_batch = p_end - p_begin <= cpairs * kBatch;
    int ids0[kBatch];
    for (int c0 = p_begin; c0 < p_end; c0 += cpairs * kBatch) {
        int ids[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int p = c0 + b * cpairs + lane;
            ids[b] = (lane_in_chunk && p < p_end) ? topk_ids[p] : -1;
            ids0[b] = ids[b];
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
            if (ids[b] >= 0) atomicAdd(&hist[wave][ids[b]], 1);
    }
    lds_sync();

    // Per-expert totals, and each span's base inside its expert (after the
    // rows of earlier parts).
    for (int e = tid; e < E; e += kFinishThreads) {
        int run = 0, total = 0;
        if (part_counts) {
            // 16 loads in flight at a time (a plain loop waits for each)
            for (int p0 = 0; p0 < parts; p0 += 16) {
                int c[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) c[j] = p0 + j < parts ? part_counts[(p0 + j) * E + e] : 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    run += p0 + j < q ? c[j] : 0;
                    total += c[j];
                }
            }
        }
        for (int w = 0; w < kFinishWaves; ++w) {
            const int c = hist[w][e];
            hist[w][e] = run;
            run += c;
        }
        if (!part_counts) total = run;
        if (lead) counts[e] = total;
        s_off[e] = total;
        s_bst[e] = (total + M - 1) / M;
    }
    lds_sync();

    // Exclusive scans over the experts, one expert per thread (E <= 512 <
    // 1024 threads): rows (s_off), blocks (s_bst), full blocks (s_fst), and
    // for the schedule the experts whose partial block falls in each size
    // class.
    {
        const int e = tid;
        const int rows_e = e < E ? s_off[e] : 0;
        const int full_e = rows_e / M;
        const int rem_e = rows_e - full_e * M;
        const int cls_e = rem_e > 0 ? (4 * rem_e + M - 1) / M : 0;  // 1..4: quarter of a block
        // values: rows, blocks, full blocks, then one flag per size class 4..1
        int v[7] = {rows_e, e < E ? s_bst[e] : 0, full_e, cls_e == 4, cls_e == 3, cls_e == 2,
                    cls_e == 1};
        int ex[7], tot[7];
        block_exclusive_scan<7>(v, ex, tot, s_wsum, (E + kWave - 1) / kWave);
        const int ex_rows = ex[0], ex_blks = ex[1], ex_full = ex[2];
        const int tot_rows = tot[0], tot_blks = tot[1];
        int cls_rank = 0, cls_base = tot[2];
#pragma unroll
        for (int c = 4; c >= 1; --c) {
            if (cls_e == c) cls_rank = cls_base + ex[3 + 4 - c];
            cls_base += tot[3 + 4 - c];
        }
        if (e < E) {
            s_off[e] = ex_rows;
            s_bst[e] = ex_blks;
            s_fst[e] = ex_full;
            if (rem_e > 0 && lead) {
                block_order[cls_rank] = ex_blks + full_e;
                *reinterpret_cast<int4*>(block_info + 4 * cls_rank) =
                    make_int4(e, ex_rows + full_e * M, rem_e, ex_blks + full_e);
            }
        }
        if (e == 0) {
            s_off[E] = tot_rows;
            s_bst[E] = tot_blks;
        }
    }
    if (lead)  // the counters, but not the give-up flag, which stays until the caller clears it
        for (int i = tid; i < kCounterInts; i += kFinishThreads)
            if (i != kGiveUpFlag) sched[i] = 0;
    lds_sync();

    if (lead)
        for (int e = tid; e <= E; e += kFinishThreads) offsets[e] = s_off[e];
    const int nb = s_bst[E];
    if (tid == 0 && lead) num_blocks[0] = nb;

    // Block map: block b belongs to the last expert whose block start is <= b.
    for (int b = tid; lead && b < nb; b += kFinishThreads) {
        int lo = 0, hi = E;  // invariant: s_bst[lo] <= b < s_bst[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_bst[mid] <= b) lo = mid; else hi = mid;
        }
        block_expert[b] = lo;
        block_row0[b] = s_off[lo] + (b - s_bst[lo]) * M;
        const int j = b - s_bst[lo];
        if (j < (s_off[lo + 1] - s_off[lo]) / M) {
            block_order[s_fst[lo] + j] = b;
            *reinterpret_cast<int4*>(block_info + 4 * (s_fst[lo] + j)) =
                make_int4(lo, s_off[lo] + j * M, M, b);
        }
    }

    // Pass 2: stable positions. The k experts of a token are distinct, so
    // inside a chunk the pairs of one expert are ordered by token: a bit per
    // token (atomic OR into cmask) gives each pair the number of earlier
    // pairs of its expert in the chunk; the chunk's last such pair advances
    // the span's cursor and clears the mask. LDS operations of a wavefront
    // complete in program order.
    const int tl = lane / k;  // token of this lane inside its chunk (< tpc <= 32)
    for (int c0 = p_begin; c0 < p_end; c0 += cpairs * kBatch) {
        int ids[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int p = c0 + b * cpairs + lane;
            ids[b] = one_batch ? ids0[b] : (lane_in_chunk && p < p_end) ? topk_ids[p] : -1;
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            if (c0 + b * cpairs >= p_end) break;
            const int e = ids[b];
            if (e >= 0) atomicOr(&cmask[wave][e], 1u << tl);
            if (e >= 0) {
                const int p = c0 + b * cpairs + lane;
                const uint32_t m = cmask[wave][e];
                const int base = hist[wave][e];
                const int row = s_off[e] + base + __popc(m & ((1u << tl) - 1u));
                sorted_pairs[row] = p;
                pair_rows[p] = row;
                if ((m >> tl) == 1u) {
                    hist[wave][e] = base + __popc(m);
                    cmask[wave][e] = 0u;
                }
            }
        }
    }

    // The last workgroup to get here (every one has read the histograms by
    // then) clears them and their arrival counter for the next launch.
    if (part_counts) {
        int32_t* arrivals = part_counts + kMaxParts * kMaxExperts;
        if (tid == 0) s_last = atomicAdd(arrivals, 1) == parts - 1;
        lds_sync();
        if (s_last) {
            for (int i = tid; i < parts * E; i += kFinishThreads) part_counts[i] = 0;
            if (tid == 0) *arrivals = 0;
        }
    }
}

// Top-k and softmax of every token only (the host-synchronised route).
int launch_topk_only(const lily_moe_dims& d, const float* logits, const lily_moe_routing& r,
                     hipStream_t stream) {
    const int grid = (d.T + kTopkTokensPerBlock - 1) / kTopkTokensPerBlock;
    hipLaunchKernelGGL(route_topk_kernel, dim3(grid), dim3(kTopkThreads), 0, stream, logits, d.T,
                       d.E, d.topk, r.topk_ids, r.topk_w, nullptr, 1);
    return check_launch("route_topk");
}

int launch_route(const lily_moe_dims& d, const float* logits, const lily_moe_routing& r,
                 hipStream_t stream) {
    const int fused = d.T <= kFusedRouteMaxT;
    int parts = 1, part_tokens = d.T;
    int32_t* part_counts = nullptr;
    if (!fused) {
        part_tokens = part_tokens_for(d.T);
        parts = (d.T + part_tokens - 1) / part_tokens;  // <= kMaxParts
        part_counts = r.sched + kPartBase;
        const int grid = (d.T + kTopkTokensPerBlock - 1) / kTopkTokensPerBlock;
        hipLaunchKernelGGL(route_topk_kernel, dim3(grid), dim3(kTopkThreads), 0, stream, logits,
                           d.T, d.E, d.topk, r.topk_ids, r.topk_w, part_counts, part_tokens);
        int rc = check_launch("route_topk");
        if (rc) return rc;
    }
    hipLaunchKernelGGL(route_finish_kernel, dim3(parts), dim3(kFinishThreads), 0, stream, logits,
                       d.T, d.E, d.topk, d.tile_m, fused, r.topk_ids, r.topk_w, r.counts,
                       r.offsets, r.sorted_pairs, r.pair_rows, r.block_expert, r.block_row0,
                       r.num_blocks, r.block_order, r.sched, r.block_info, part_counts,
                       part_tokens);
    return check_launch("route_finish");
}

}  // namespace lily
