// Ablation twin of lily_moe_route: the same routing with its histogram,
// scan, scatter and block map computed on the host after a stream
// synchronisation.
//
// The Lily articles keep these steps on the GPU, inside one command stream,
// and credit that with a large part of their prefill speed-up over a
// CPU-synchronised version (news.ainew.jp Lily article, section "Prefill").
// This entry point is that CPU-synchronised version, rebuilt for measuring
// the difference here: the top-k still runs on the GPU (route_topk), then
// the ids come to the host, the host computes R3-R6 with the definitions
// of the GPU route (so the result is bit-identical) and uploads them, and
// the stream is synchronised again before returning.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "common.hpp"

namespace lily {

int launch_topk_only(const lily_moe_dims& d, const float* logits, const lily_moe_routing& r,
                     hipStream_t stream);

static int hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) return set_error(LILY_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return LILY_OK;
}

int launch_route_host(const lily_moe_dims& d, const float* logits, const lily_moe_routing& r,
                      hipStream_t stream) {
    const int T = d.T, E = d.E, k = d.topk, M = d.tile_m;
    const int P = T * k;
    int rc = launch_topk_only(d, logits, r, stream);
    if (rc) return rc;
    std::vector<int32_t> ids(P);
    if ((rc = hip_check(hipMemcpyAsync(ids.data(), r.topk_ids, sizeof(int32_t) * P,
                                       hipMemcpyDeviceToHost, stream), "topk_ids to host")) ||
        (rc = hip_check(hipStreamSynchronize(stream), "stream synchronise")))
        return rc;

    // R3 histogram, R4 exclusive scan.
    std::vector<int32_t> counts(E, 0), offsets(E + 1, 0);
    for (int p = 0; p < P; ++p) {
        if (ids[p] < 0 || ids[p] >= E) return set_error(LILY_ERR_HIP, "top-k id out of range");
        ++counts[ids[p]];
    }
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    // R5 stable scatter: pairs in ascending (token, slot) order.
    std::vector<int32_t> sorted_pairs(P), pair_rows(P), cursor(offsets.begin(), offsets.end() - 1);
    for (int p = 0; p < P; ++p) {
        const int row = cursor[ids[p]]++;
        sorted_pairs[row] = p;
        pair_rows[p] = row;
    }
    // R6 block map, experts ascending; then the GEMM schedule: full blocks
    // in block order, then each expert's partial block by descending size
    // class ceil(4 rows / M), ties in expert order; and the schedule
    // resolved to (expert, first row, rows, block).
    std::vector<int32_t> block_expert, block_row0, first_block(E);
    for (int e = 0; e < E; ++e) {
        first_block[e] = (int)block_expert.size();
        for (int r0 = offsets[e]; r0 < offsets[e + 1]; r0 += M) {
            block_expert.push_back(e);
            block_row0.push_back(r0);
        }
    }
    const int nb = (int)block_expert.size();
    std::vector<int32_t> order;
    order.reserve(nb);
    for (int b = 0; b < nb; ++b)
        if (offsets[block_expert[b] + 1] - block_row0[b] >= M) order.push_back(b);
    for (int c = 4; c >= 1; --c)
        for (int e = 0; e < E; ++e) {
            const int rem = counts[e] % M;
            if (rem > 0 && (4 * rem + M - 1) / M == c) order.push_back(first_block[e] + counts[e] / M);
        }
    std::vector<int32_t> info(4 * (size_t)nb);
    for (int i = 0; i < nb; ++i) {
        const int b = order[i], e = block_expert[b];
        info[4 * i] = e;
        info[4 * i + 1] = block_row0[b];
        info[4 * i + 2] = std::min(M, offsets[e + 1] - block_row0[b]);
        info[4 * i + 3] = b;
    }

    auto up = [&](void* dst, const int32_t* src, size_t n, const char* what) {
        return n ? hip_check(hipMemcpyAsync(dst, src, sizeof(int32_t) * n, hipMemcpyHostToDevice,
                                            stream), what)
                 : LILY_OK;
    };
    if ((rc = up(r.counts, counts.data(), E, "counts")) ||
        (rc = up(r.offsets, offsets.data(), E + 1, "offsets")) ||
        (rc = up(r.sorted_pairs, sorted_pairs.data(), P, "sorted_pairs")) ||
        (rc = up(r.pair_rows, pair_rows.data(), P, "pair_rows")) ||
        (rc = up(r.block_expert, block_expert.data(), nb, "block_expert")) ||
        (rc = up(r.block_row0, block_row0.data(), nb, "block_row0")) ||
        (rc = up(r.num_blocks, &nb, 1, "num_blocks")) ||
        (rc = up(r.block_order, order.data(), nb, "block_order")) ||
        (rc = up(r.block_info, info.data(), 4 * (size_t)nb, "block_info")) ||
        (rc = hip_check(hipMemsetAsync(r.sched, 0, sizeof(int32_t) * kGiveUpFlag, stream), "sched")) ||
        (rc = hip_check(hipMemsetAsync(r.sched + kGiveUpFlag + 1, 0,
                                       sizeof(int32_t) * (kSchedInts - kGiveUpFlag - 1), stream),
                        "sched")))
        return rc;
    // The host buffers must outlive the copies.
    return hip_check(hipStreamSynchronize(stream), "stream synchronise");
}

}  // namespace lily
