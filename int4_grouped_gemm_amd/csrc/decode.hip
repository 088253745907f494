// Fused decode: routing and the whole MoE layer for a few tokens in one
// launch (gfx950).
//
// At one or a few tokens the layer is a stream of weights: each of the k
// routed experts and the shared expert is used by one row, so every weight
// is read once and multiplied once (Lily articles, section "Decode": the
// cost per token is the bytes moved). The grouped GEMM's tiles would put a
// 32-row MFMA and a long K loop on a handful of workgroups; here the weights
// are spread evenly over one workgroup per compute unit as matrix-vector
// products on the VALU (bf16 dot2 instructions on the dequantised weights):
//   phase 0  top-k and softmax of every token (each workgroup, redundantly);
//   phase A  gate/up: the packed blocks of all rows, in (row, gate/up, slab,
//            group) order, cut into equal contiguous ranges, one per
//            workgroup; a range's dot products are summed per 128-row
//            segment into fp32 partial sums, and the last workgroup to count
//            in for a (row, slab) adds that slab's partials in workgroup
//            order into h = bf16(silu(gate) * up);
//   one device-wide barrier;
//   phase B  down and combine: unit = (token, 8 output rows); the unit's
//            W_down slices of the k + 1 rows times their h, weighted by the
//            routing weights (1 for the shared expert), summed in fp32 and
//            written as bf16.
// The loads of a workgroup's first phase B unit are issued together with
// its phase A loads, so they arrive while phase A computes.
// Row r of the layer is token r / (k + 1), slot r % (k + 1): slots 0..k-1
// are the routed experts in top-k order, slot k the shared expert.
#include "common.hpp"
#include "topk.hpp"
#include "w4.hpp"

namespace lily {

constexpr int kDecThreads = 256;
constexpr int kDecodeMaxT = 4;       // lily_moe_decode serves T <= this
constexpr int kDecMaxGrid = 512;     // workgroups: at most one per compute unit and this
constexpr int kDecBatch = 12;        // phase A blocks loaded per round
constexpr int kDecBRounds = 6;       // phase B rounds per wavefront loaded at once
constexpr int kDecPieces = 4;        // segments one phase A range may touch
constexpr int kDecContrib = 8;       // phase A ranges one segment may span
constexpr int kDecLdsWords = 8192;   // LDS: x rows (phase A) or h rows (phase B), bf16 pairs
constexpr int kDecXWords = 16;       // x words staged per thread: 2 tokens of H <= 4096
constexpr int kDecHWords = kDecLdsWords / kDecThreads;  // h words staged per thread
constexpr int kDecPiece = 8;         // output rows per phase B unit
constexpr long kSpinTicks = 50000000;  // device-wide barrier wait limit: 0.5 s at 100 MHz
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor: raw, 32-bit data format

struct DecodeArgs {
    const float* logits;  // [T, E]
    const uint16_t* x;    // [T, H] bf16
    int T, H, F, E, k;
    const char* gate;     // packed stacks
    const char* up;
    const char* down;
    const char* sh_gate;
    const char* sh_up;
    const char* sh_down;
    int32_t* topk_ids;    // [T, k], written by workgroup 0
    float* topk_w;
    float* pa;            // [grid][kDecPieces][128] phase A partial sums
    uint16_t* h;          // [R][F] bf16
    uint16_t* out;        // [T, H]
    int32_t* ctr;         // [R][F / 128] arrivals per (row, slab): zero on entry, left zero
    int32_t* bar;         // [2] barrier arrivals, exits: zero on entry, left zero
    int32_t* err;         // set to 1 if the barrier wait gave up
};

// The weights are read with buffer loads: a wave-uniform descriptor (base,
// size) in SGPRs, a per-lane offset that stays the same from load to load,
// and a uniform offset; loads past the size return 0.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(base)), 0, bytes,
                                             kRsrcWord3);
}

// One 16-byte slice of a packed block: 32 weights of one row (one half of
// the group), with the row's scale and bias (bf16 bits).
struct Slice {
    u32x4 q;
    uint16_t sc, bi;
};

// q at voff_q, the scale at voff_s and the bias 256 bytes on, all + soff.
__device__ __forceinline__ Slice load_slice(Rsrc r, int voff_q, int voff_s, int soff) {
    Slice s;
    s.q = __builtin_amdgcn_raw_buffer_load_b128(r, voff_q, soff, 0);
    s.sc = __builtin_amdgcn_raw_buffer_load_b16(r, voff_s, soff, 0);
    s.bi = __builtin_amdgcn_raw_buffer_load_b16(r, voff_s + 2 * kPackRows, soff, 0);
    return s;
}

// Dot product of a slice's 32 weights, rebuilt as bf16 exactly as in the
// GEMMs, with 16 bf16 pairs of LDS (the matching k, in order).
__device__ __forceinline__ float dot_slice(const Slice& s, const uint32_t* v) {
    const float s512 = bf16_bits_to_float(s.sc) * 512.0f;
    const float bias = bf16_bits_to_float(s.bi);
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t wt[4];
        dequant8(s.q[w], s512, bias, wt);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wt[e]),
                                                  __builtin_bit_cast(bf16x2, v[4 * w + e]), acc,
                                                  false);
    }
    return acc;
}

// Workgroup barrier that waits for this thread's LDS accesses only: global
// loads in flight stay in flight (__syncthreads would drain them).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Device-wide barrier: count this workgroup, wait for `target` arrivals.
// Every global store of the workgroup is complete before it counts. The
// wait is bounded in time: on a timeout it flags the error and goes on, so
// no wave can wait forever.
__device__ __forceinline__ void device_barrier(int32_t* bar, int target, int32_t* err) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(bar, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(2);
            if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > kSpinTicks) {
                __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// Phase A ranges: workgroup w of G takes blocks [w NB / G, (w + 1) NB / G)
// (NB * G < 2^31 on the host's checks).
__device__ __forceinline__ int range_begin(int w, int nb, int g) { return (unsigned)(w * nb) / (unsigned)g; }
// The workgroup whose range holds block b (NB >= G, so no range is empty).
__device__ __forceinline__ int range_owner(int b, int nb, int g) {
    return (unsigned)((b + 1) * g - 1) / (unsigned)nb;
}

__global__ void __launch_bounds__(kDecThreads) moe_decode_kernel(DecodeArgs a) {
    __shared__ int32_t s_ids[kDecodeMaxT * kMaxTopk];
    __shared__ float s_w[kDecodeMaxT * kMaxTopk];
    __shared__ __attribute__((aligned(16))) uint32_t s_buf[kDecLdsWords];
    __shared__ float s_red[kDecPieces][kPackRows];
    __shared__ float s_bred[kDecThreads / kWave][kDecPiece];
    __shared__ int s_last[kDecPieces];

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int G = gridDim.x;
    const int wg = blockIdx.x;
    const int k = a.k;
    const int R = a.T * (k + 1);
    const int H = a.H, F = a.F;
    const int nkg = H / kGroup;        // groups along K of gate/up
    const int nsf = F / kPackRows;     // 128-row slabs of gate/up
    const int nkgF = F / kGroup;       // groups along K of down
    const int nsH = H / kPackRows;     // 128-row slabs of down

    // Phase A range, and the x rows it reads: t_lo and t_lo + 1 (a range
    // spans at most two tokens). Segment sg = (r * 2 + m) * nsf + slab holds
    // nkg consecutive blocks (its groups). x is loaded first, to arrive
    // together with the router logits.
    const int NB = R * 2 * nsf * nkg;
    const int b0 = range_begin(wg, NB, G), b1 = range_begin(wg + 1, NB, G);
    const int seg0 = b0 / nkg;
    const int t_lo = b0 / ((k + 1) * 2 * nsf * nkg);
    const int i = tid % kPackRows, hh = tid / kPackRows;
    const int x_words = (t_lo + 1 < a.T ? 2 : 1) * (H / 2);
    const Rsrc x_rs = make_rsrc(a.x + (size_t)t_lo * H, x_words * 4);
    uint32_t xr[kDecXWords];
#pragma unroll
    for (int n = 0; n < kDecXWords; ++n)  // x_words is a multiple of 256
        if (n * kDecThreads < x_words)
            xr[n] = __builtin_amdgcn_raw_buffer_load_b32(x_rs, tid * 4, n * kDecThreads * 4, 0);

    // Phase 0: every workgroup routes every token (wave t takes token t).
    if (wave < a.T) topk_one_token(a.logits, wave, a.E, k, s_ids, s_w);
#pragma unroll
    for (int n = 0; n < kDecXWords; ++n)
        if (n * kDecThreads < x_words) s_buf[tid + n * kDecThreads] = xr[n];
    __syncthreads();
    if (wg == 0 && tid < a.T * k) {
        a.topk_ids[tid] = s_ids[tid];
        a.topk_w[tid] = s_w[tid];
    }
    // Descriptor over segment sg's blocks, and its token.
    auto seg_rsrc = [&](int sg, int& t) -> Rsrc {
        const int s = sg % nsf;
        const int m = (sg / nsf) % 2;
        const int r = sg / (2 * nsf);
        t = r / (k + 1);
        const int j = r - t * (k + 1);
        const bool sh = (j == k);
        const int e = sh ? 0 : s_ids[t * k + j];
        const char* stack = sh ? (m ? a.sh_up : a.sh_gate) : (m ? a.up : a.gate);
        return make_rsrc(stack + ((size_t)e * nsf + s) * nkg * kPackBlock, nkg * kPackBlock);
    };
    const int a_voff_q = (hh * kPackRows + i) * 16, a_voff_s = kPackQ + i * 2;

    // Phase B units of this workgroup: wavefront v takes rounds v, v + 4, ...
    // of each. Round rho of a unit: slot j = rho / nq, groups 4 gq .. 4 gq + 3
    // with gq = rho % nq; lane l: group 4 gq + l / 16, half (l / 8) % 2,
    // output row l % 8.
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int pieces_per_tok = H / kDecPiece;
    const int UB = a.T * pieces_per_tok;
    const int ub0 = range_begin(wg, UB, G), ub1 = range_begin(wg + 1, UB, G);
    const int nq = nkgF / 4;
    const int NRB = (k + 1) * nq;
    const int b_gl = lane / 16, b_half = (lane / 8) % 2, b_row = lane % kDecPiece;
    auto b_round = [&](int u, int rho, float& wj, int& hoff) -> Slice {
        const int t = u / pieces_per_tok, r0 = (u - t * pieces_per_tok) * kDecPiece;
        const int j = rho / nq, gq = rho - j * nq;
        const bool sh = (j == k);
        const int e = sh ? 0 : s_ids[t * k + j];
        wj = sh ? 1.0f : s_w[t * k + j];
        hoff = (j * F + (4 * gq + b_gl) * kGroup + b_half * 32) / 2;
        const char* stack = sh ? a.sh_down : a.down;
        const Rsrc rs = make_rsrc(
            stack + ((size_t)(e * nsH + r0 / kPackRows) * nkgF + 4 * gq) * kPackBlock,
            4 * kPackBlock);
        const int rr = r0 % kPackRows + b_row;
        return load_slice(rs, b_gl * kPackBlock + (b_half * kPackRows + rr) * 16,
                          b_gl * kPackBlock + kPackQ + rr * 2, 0);
    };

    // Loads, in the order they are waited for: the first phase A round, the
    // first phase B rounds. Rounds past the end are clamped onto valid data
    // (results unused), so that no load is conditional and the waits can
    // leave the later loads in flight.
    float accp[kDecPieces];
#pragma unroll
    for (int p = 0; p < kDecPieces; ++p) accp[p] = 0.0f;
    Slice pb[kDecBRounds];
    float pw[kDecBRounds];
    int ph[kDecBRounds];
    const int ub_first = ub0 < ub1 ? ub0 : 0;
    for (int bb = b0; bb < b1; bb += kDecBatch) {
        const int nb = min(kDecBatch, b1 - bb);
        // (segment, group) of each block of the round, stepped from the first
        Slice sl[kDecBatch];
        int piece[kDecBatch], xoff[kDecBatch];
        int sg = bb / nkg, g = bb - sg * nkg, t;
        Rsrc rs = seg_rsrc(sg, t);
#pragma unroll
        for (int n = 0; n < kDecBatch; ++n) {
            sl[n] = load_slice(rs, a_voff_q, a_voff_s, g * kPackBlock);
            piece[n] = sg - seg0;
            xoff[n] = (t - t_lo) * (H / 2) + g * 32 + hh * 16;
            if (n + 1 < nb && ++g == nkg) {
                g = 0;
                rs = seg_rsrc(++sg, t);
            }
        }
        if (bb == b0) {
#pragma unroll
            for (int n = 0; n < kDecBRounds; ++n)
                pb[n] = b_round(ub_first, min(wv + 4 * n, NRB - 1), pw[n], ph[n]);
        }
#pragma unroll
        for (int n = 0; n < kDecBatch; ++n) {
            if (n < nb) {
                const float d = dot_slice(sl[n], s_buf + xoff[n]);
#pragma unroll
                for (int p = 0; p < kDecPieces; ++p)
                    if (p == piece[n]) accp[p] += d;
            }
        }
    }

    // Partial sums of the range's segments (the two K halves added), stored
    // device-coherent.
    const int npieces = (b1 - 1) / nkg - seg0 + 1;
    if (hh == 1) {
#pragma unroll
        for (int p = 0; p < kDecPieces; ++p) s_red[p][i] = accp[p];
    }
    __syncthreads();
    if (hh == 0) {
#pragma unroll
        for (int p = 0; p < kDecPieces; ++p)
            if (p < npieces)
                __hip_atomic_store(a.pa + ((size_t)wg * kDecPieces + p) * kPackRows + i,
                                   accp[p] + s_red[p][i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // Count this range's segments in; the last contribution to a (row, slab)
    // (of its gate and up segments) builds that slab of h.
    if (tid == 0) {
        for (int p = 0; p < npieces; ++p) {
            const int sg = seg0 + p;
            const int r = sg / (2 * nsf), s = sg % nsf;
            int total = 0;
            for (int m = 0; m < 2; ++m) {
                const int msg = (r * 2 + m) * nsf + s;
                total += range_owner(msg * nkg + nkg - 1, NB, G) - range_owner(msg * nkg, NB, G) + 1;
            }
            int32_t* c = a.ctr + r * nsf + s;
            const int prev = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last[p] = (prev == total - 1);
            if (prev == total - 1) __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    for (int p = 0; p < npieces; ++p) {
        if (!s_last[p] || tid >= kPackRows / 2) continue;
        const int sg = seg0 + p;
        const int r = sg / (2 * nsf), s = sg % nsf;
        // every partial of both rows of this thread, gate and up, loaded at once
        float v[2][2][kDecContrib];
        int nw[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int msg = (r * 2 + m) * nsf + s;
            const int w_first = range_owner(msg * nkg, NB, G);
            nw[m] = range_owner(msg * nkg + nkg - 1, NB, G) - w_first + 1;
#pragma unroll
            for (int c = 0; c < kDecContrib; ++c) {
                const int w = w_first + min(c, nw[m] - 1);
                const int piece = msg - range_begin(w, NB, G) / nkg;
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    v[q][m][c] = __hip_atomic_load(
                        a.pa + ((size_t)w * kDecPieces + piece) * kPackRows + 2 * tid + q,
                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        float hv[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float sum[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                float acc = 0.0f;
#pragma unroll
                for (int c = 0; c < kDecContrib; ++c)
                    if (c < nw[m]) acc += v[q][m][c];
                sum[m] = acc;
            }
            hv[q] = silu(sum[0]) * sum[1];
        }
        __hip_atomic_store(reinterpret_cast<uint32_t*>(a.h + (size_t)r * F + s * kPackRows) + tid,
                           pack_bf16x2(hv[0], hv[1]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    device_barrier(a.bar, G, a.err);

    // Phase B: out[t, rows] = bf16(sum over slots j of w_j * (W_down_j rows . h_j)).
    // A thread's sum covers output row lane % 8.
    const int h_words = (k + 1) * F / 2;
    int t_staged = -1;
    for (int u = ub0; u < ub1; ++u) {
        const int t = u / pieces_per_tok;
        if (t != t_staged) {
            __syncthreads();  // earlier readers of s_buf are done
            const uint32_t* hg = reinterpret_cast<const uint32_t*>(a.h + (size_t)t * (k + 1) * F);
            uint32_t hr[kDecHWords];
#pragma unroll
            for (int n = 0; n < kDecHWords; ++n)
                hr[n] = __hip_atomic_load(hg + min(tid + n * kDecThreads, h_words - 1),
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int n = 0; n < kDecHWords; ++n)
                if (tid + n * kDecThreads < h_words) s_buf[tid + n * kDecThreads] = hr[n];
            __syncthreads();
            t_staged = t;
        }
        float acc = 0.0f;
        for (int n0 = 0; wv + 4 * n0 < NRB; n0 += kDecBRounds) {
            if (n0 > 0) {
#pragma unroll
                for (int n = 0; n < kDecBRounds; ++n)
                    pb[n] = b_round(u, min(wv + 4 * (n0 + n), NRB - 1), pw[n], ph[n]);
            }
#pragma unroll
            for (int n = 0; n < kDecBRounds; ++n)
                if (wv + 4 * (n0 + n) < NRB) acc = fmaf(pw[n], dot_slice(pb[n], s_buf + ph[n]), acc);
        }
        // the next unit's first rounds, in flight during this unit's sums
        if (u + 1 < ub1) {
#pragma unroll
            for (int n = 0; n < kDecBRounds; ++n)
                pb[n] = b_round(u + 1, min(wv + 4 * n, NRB - 1), pw[n], ph[n]);
        }
        // Lanes 8 apart share an output row; then across the wavefronts.
        acc += __shfl_xor(acc, 8);
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        if (tid % kWave < kDecPiece) s_bred[wave][tid % kWave] = acc;
        __syncthreads();
        if (tid < kDecPiece) {
            float o = 0.0f;
#pragma unroll
            for (int v = 0; v < kDecThreads / kWave; ++v) o += s_bred[v][tid];
            const int p = u - t * pieces_per_tok;
            a.out[(size_t)t * H + p * kDecPiece + tid] = float_to_bf16_bits(o);
        }
        __syncthreads();
    }

    // Every workgroup has passed the barrier before it counts here; the last
    // one clears the counters for the next launch.
    if (tid == 0 &&
        __hip_atomic_fetch_add(a.bar + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == G - 1) {
        __hip_atomic_store(a.bar, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.bar + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

static long decode_blocks(const lily_moe_dims& d) {
    return (long)d.T * (d.topk + 1) * 2 * (d.F / kPackRows) * (d.H / kGroup);
}

// One workgroup per compute unit (at most kDecMaxGrid), each range at least
// ceil(nkg / (kDecContrib - 1)) blocks long, so that a segment spans at most
// kDecContrib ranges.
static int decode_grid(const lily_moe_dims& d) {
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n = 0;
        cus[dev] = n > 0 ? n : 1;
    }
    const long nkg = d.H / kGroup;
    const long span_min = (nkg + kDecContrib - 2) / (kDecContrib - 1);
    long g = cus[dev] < kDecMaxGrid ? cus[dev] : kDecMaxGrid;
    const long lim = decode_blocks(d) / span_min;
    if (lim < g) g = lim;
    return (int)(g > 0 ? g : 1);
}

size_t decode_workspace_bytes(const lily_moe_dims& d) {
    if (d.T > kDecodeMaxT) return 0;
    const size_t R = (size_t)d.T * (d.topk + 1);
    return (size_t)kDecMaxGrid * kDecPieces * kPackRows * sizeof(float) +
           R * d.F * sizeof(uint16_t);
}

int decode_supported(const lily_moe_dims& d) {
    if (d.T > kDecodeMaxT)
        return set_error(LILY_ERR_UNSUPPORTED, "T = %d; lily_moe_decode serves T <= %d", d.T,
                         kDecodeMaxT);
    if (d.H % (2 * kDecThreads) || d.H > kDecXWords * kDecThreads)
        return set_error(LILY_ERR_UNSUPPORTED, "H = %d must be a multiple of 512, at most %d",
                         d.H, kDecXWords * kDecThreads);
    if (d.F % (4 * kGroup) || (long)(d.topk + 1) * d.F > 2L * kDecLdsWords)
        return set_error(LILY_ERR_UNSUPPORTED,
                         "F = %d must be a multiple of 256 with (topk + 1) * F <= %d", d.F,
                         2 * kDecLdsWords);
    const long R = (long)d.T * (d.topk + 1);
    if (R * (d.F / kPackRows) > kTileCounters)
        return set_error(LILY_ERR_UNSUPPORTED, "T * (topk + 1) * F / 128 = %ld exceeds %d",
                         R * (d.F / kPackRows), kTileCounters);
    if (decode_blocks(d) * kDecMaxGrid >= (1L << 31))
        return set_error(LILY_ERR_UNSUPPORTED, "decode: %ld blocks are too many", decode_blocks(d));
    return LILY_OK;
}

int launch_decode(const lily_moe_dims& d, const lily_moe_weights& w, const float* logits,
                  const uint16_t* x, const lily_moe_routing& r, uint16_t* out, void* workspace,
                  hipStream_t stream) {
    DecodeArgs a{};
    a.logits = logits;
    a.x = x;
    a.T = d.T;
    a.H = d.H;
    a.F = d.F;
    a.E = d.E;
    a.k = d.topk;
    a.gate = static_cast<const char*>(w.gate);
    a.up = static_cast<const char*>(w.up);
    a.down = static_cast<const char*>(w.down);
    a.sh_gate = static_cast<const char*>(w.sh_gate);
    a.sh_up = static_cast<const char*>(w.sh_up);
    a.sh_down = static_cast<const char*>(w.sh_down);
    a.topk_ids = r.topk_ids;
    a.topk_w = r.topk_w;
    a.pa = static_cast<float*>(workspace);
    a.h = reinterpret_cast<uint16_t*>(a.pa + (size_t)kDecMaxGrid * kDecPieces * kPackRows);
    a.out = out;
    a.ctr = r.sched + kQueueInts;
    a.bar = r.sched + kDecodeBarrier;
    a.err = r.sched + kDecodeBarrier + 2;
    // A phase A range touches at most kDecPieces segments and two tokens; a
    // segment spans at most kDecContrib ranges.
    const long nb = decode_blocks(d), g = decode_grid(d), nkg = d.H / kGroup;
    const long span_max = (nb + g - 1) / g, span_min = nb / g;
    if (span_min < 1 || (span_max + nkg - 1) / nkg + 1 > kDecPieces || span_max > nb / d.T ||
        (nkg + span_min - 1) / span_min + 1 > kDecContrib)
        return set_error(LILY_ERR_UNSUPPORTED, "decode ranges of %ld..%ld blocks over %ld groups",
                         span_min, span_max, nkg);
    // At most one workgroup per compute unit, each needing a fraction of a
    // compute unit's registers and LDS: all are resident at once, which the
    // device-wide barrier relies on.
    hipLaunchKernelGGL(moe_decode_kernel, dim3((unsigned)g), dim3(kDecThreads), 0, stream, a);
    return check_launch("decode");
}

}  // namespace lily
