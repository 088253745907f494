// Fused decode: routing and the whole MoE layer for a few tokens in one
// launch (gfx950).
//
// At one or a few tokens the layer is a stream of weights: each of the k
// routed experts and the shared expert is used by one row, so every weight
// is read once and multiplied once (Lily articles, section "Decode": the
// cost per token is the bytes moved). The grouped GEMM's tiles would put a
// 32-row MFMA and a long K loop on a handful of workgroups; here the weights
// are spread evenly over one workgroup per compute unit as matrix-vector
// products on the VALU (bf16 dot2 instructions on the 4-bit values, scale
// and bias applied to each 32-weight dot product):
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
constexpr int kDecXChunks = 4;       // x 16-byte chunks staged per thread: 2 tokens of H <= 4096
constexpr int kDecHChunks = kDecLdsWords / 4 / kDecThreads;  // h chunks staged per thread
constexpr int kDecSums = kDecLdsWords / 16;  // sums of 32 staged values
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
    float* pa;            // [segments][kDecContrib][128] phase A partial sums
    uint16_t* h;          // [R][F] bf16
    uint16_t* out;        // [T, H]
    int32_t* ctr;         // arrivals per (row, slab), ctr_stride apart: zero on entry, left zero
    int ctr_stride;       // ints between counters (up to a 128-byte line each)
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

// Vectors are staged in LDS as bf16 pairs permuted within each chunk of 8
// elements: word j of chunk c holds elements (8c + j, 8c + j + 4). From
// natural pairs p0..p3 of the chunk:
__device__ __forceinline__ u32x4 permute_chunk(u32x4 p) {
    u32x4 o;
    o[0] = (p[0] & 0xFFFFu) | (p[2] << 16);
    o[1] = (p[0] >> 16) | (p[2] & 0xFFFF0000u);
    o[2] = (p[1] & 0xFFFFu) | (p[3] << 16);
    o[3] = (p[1] >> 16) | (p[3] & 0xFFFF0000u);
    return o;
}

// Dot product of a slice's 32 weights w = scale * q + bias with 32 staged
// values v (16 permuted words) whose sum is vsum: scale * sum(q v) +
// bias * vsum. The nibbles j and j + 4 of a weight word become the bf16 pair
// (128 + q_j, 128 + q_j+4) with one byte permute each (exact: the exponent
// byte 0x43 sets the scale to 1 on [128, 256)), so that
// sum(q v) = sum((128 + q) v) - 128 vsum comes from bf16 dot2 instructions.
// The weights enter exactly (fp32 scale and bias), not rounded to bf16 as in
// the GEMMs.
__device__ __forceinline__ float dot_slice(const Slice& s, const uint32_t* v, float vsum) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t lo = s.q[w] & 0x0F0F0F0Fu;         // elements 0, 2, 4, 6
        const uint32_t hi = (s.q[w] >> 4) & 0x0F0F0F0Fu;  // elements 1, 3, 5, 7
        // bytes: 0-3 from the second operand, 4-7 from the first (0x43 each)
        const uint32_t wt[4] = {__builtin_amdgcn_perm(0x43434343u, lo, 0x04020400u),   // 0, 4
                                __builtin_amdgcn_perm(0x43434343u, hi, 0x04020400u),   // 1, 5
                                __builtin_amdgcn_perm(0x43434343u, lo, 0x04030401u),   // 2, 6
                                __builtin_amdgcn_perm(0x43434343u, hi, 0x04030401u)};  // 3, 7
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wt[e]),
                                                  __builtin_bit_cast(bf16x2, v[4 * w + e]), acc,
                                                  false);
    }
    const float scale = bf16_bits_to_float(s.sc), bias = bf16_bits_to_float(s.bi);
    return fmaf(scale, acc, fmaf(-128.0f, scale, bias) * vsum);
}

// Sum of the 32 bf16 values in 16 LDS words (fp32).
__device__ __forceinline__ float sum32(const uint32_t* v) {
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
        a += bf16_bits_to_float(v[n] & 0xFFFFu);
        b += bf16_bits_to_float(v[n] >> 16);
    }
    return a + b;
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
    __shared__ float s_vsum[kDecSums];  // sums of 32 consecutive staged values
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
    u32x4 xr[kDecXChunks];
#pragma unroll
    for (int n = 0; n < kDecXChunks; ++n)  // chunks past the end read 0
        if (n * kDecThreads * 4 < x_words)
            xr[n] = __builtin_amdgcn_raw_buffer_load_b128(x_rs, (tid + n * kDecThreads) * 16, 0, 0);

    // Phase 0: every workgroup routes every token (wave t takes token t).
    if (wave < a.T) topk_one_token(a.logits, wave, a.E, k, s_ids, s_w);
#pragma unroll
    for (int n = 0; n < kDecXChunks; ++n) {
        const int c = tid + n * kDecThreads;
        if (c * 4 < x_words) *reinterpret_cast<u32x4*>(s_buf + 4 * c) = permute_chunk(xr[n]);
    }
    __syncthreads();
    if (tid < x_words / 16) s_vsum[tid] = sum32(s_buf + 16 * tid);
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
                const float d = dot_slice(sl[n], s_buf + xoff[n], s_vsum[xoff[n] / 16]);
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
    // slot of this range among the contributors of segment seg0 + p: the
    // first piece may continue a segment that earlier ranges started
    const int c0 = wg - range_owner(seg0 * nkg, NB, G);
    if (hh == 0) {
#pragma unroll
        for (int p = 0; p < kDecPieces; ++p)
            if (p < npieces)
                __hip_atomic_store(
                    a.pa + ((size_t)(seg0 + p) * kDecContrib + (p == 0 ? c0 : 0)) * kPackRows + i,
                    accp[p] + s_red[p][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // Count this range's segments in (thread p counts piece p); the last
    // contribution to a (row, slab) (of its gate and up segments) builds that
    // slab of h.
    if (tid < npieces) {
        const int sg = seg0 + tid;
        const int r = sg / (2 * nsf), s = sg % nsf;
        int total = 0;
        for (int m = 0; m < 2; ++m) {
            const int msg = (r * 2 + m) * nsf + s;
            total += range_owner(msg * nkg + nkg - 1, NB, G) - range_owner(msg * nkg, NB, G) + 1;
        }
        int32_t* c = a.ctr + (r * nsf + s) * a.ctr_stride;
        const int prev = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last[tid] = (prev == total - 1);
        if (prev == total - 1) __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    // thread (m, row): the partials of row `row` of the gate (m = 0) or up
    // segment of each slab this workgroup builds, all loaded before any h
    // store, added in workgroup order
    const int m = tid / kPackRows, row = tid % kPackRows;
    float sums[kDecPieces];
#pragma unroll
    for (int p = 0; p < kDecPieces; ++p) {
        sums[p] = 0.0f;
        if (p < npieces && s_last[p]) {  // the same in every thread
            const int sg = seg0 + p;
            const int r = sg / (2 * nsf), s = sg % nsf;
            const int msg = (r * 2 + m) * nsf + s;
            const int nw = range_owner(msg * nkg + nkg - 1, NB, G) - range_owner(msg * nkg, NB, G) + 1;
            const float* src = a.pa + (size_t)msg * kDecContrib * kPackRows + row;
            float v[kDecContrib];
#pragma unroll
            for (int c = 0; c < kDecContrib; ++c)
                v[c] = __hip_atomic_load(src + min(c, nw - 1) * kPackRows, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int c = 0; c < kDecContrib; ++c)
                if (c < nw) sums[p] += v[c];
        }
    }
#pragma unroll
    for (int p = 0; p < kDecPieces; ++p) {
        if (p < npieces && s_last[p]) {
            const int sg = seg0 + p;
            const int r = sg / (2 * nsf), s = sg % nsf;
            s_red[m][row] = sums[p];
            __syncthreads();
            if (tid < kPackRows / 2) {
                const float h0 = silu(s_red[0][2 * tid]) * s_red[1][2 * tid];
                const float h1 = silu(s_red[0][2 * tid + 1]) * s_red[1][2 * tid + 1];
                __hip_atomic_store(
                    reinterpret_cast<uint32_t*>(a.h + (size_t)r * F + s * kPackRows) + tid,
                    pack_bf16x2(h0, h1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
        }
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
            u32x4 hr[kDecHChunks];
#pragma unroll
            for (int n = 0; n < kDecHChunks; ++n) {
                if (n * kDecThreads < h_words / 4) {
                    const int c = min(tid + n * kDecThreads, h_words / 4 - 1);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        hr[n][e] = __hip_atomic_load(hg + 4 * c + e, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                }
            }
#pragma unroll
            for (int n = 0; n < kDecHChunks; ++n) {
                const int c = tid + n * kDecThreads;
                if (c < h_words / 4) *reinterpret_cast<u32x4*>(s_buf + 4 * c) = permute_chunk(hr[n]);
            }
            __syncthreads();
            for (int q = tid; q < h_words / 16; q += kDecThreads) s_vsum[q] = sum32(s_buf + 16 * q);
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
                if (wv + 4 * (n0 + n) < NRB)
                    acc = fmaf(pw[n], dot_slice(pb[n], s_buf + ph[n], s_vsum[ph[n] / 16]), acc);
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
    const size_t segments = R * 2 * (d.F / kPackRows);
    return segments * kDecContrib * kPackRows * sizeof(float) + R * d.F * sizeof(uint16_t);
}

int decode_supported(const lily_moe_dims& d) {
    if (d.T > kDecodeMaxT)
        return set_error(LILY_ERR_UNSUPPORTED, "T = %d; lily_moe_decode serves T <= %d", d.T,
                         kDecodeMaxT);
    if (d.H % (2 * kDecThreads) || d.H > kDecXChunks * 4 * kDecThreads)
        return set_error(LILY_ERR_UNSUPPORTED, "H = %d must be a multiple of 512, at most %d",
                         d.H, kDecXChunks * 4 * kDecThreads);
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
    const size_t segments = (size_t)d.T * (d.topk + 1) * 2 * (d.F / kPackRows);
    a.h = reinterpret_cast<uint16_t*>(a.pa + segments * kDecContrib * kPackRows);
    a.out = out;
    // Counters on lines of their own where the sched array has room: device
    // scope atomics on one line are serialised.
    a.ctr = r.sched + kQueueInts;
    const long n_ctr = (long)d.T * (d.topk + 1) * (d.F / kPackRows);
    a.ctr_stride = 1;
    while (a.ctr_stride < 32 && 2 * a.ctr_stride * n_ctr <= kSchedInts - kQueueInts)
        a.ctr_stride *= 2;
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
