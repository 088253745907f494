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
//   phase A  gate/up: unit = (row, 8 features): the 8 gate and 8 up weight
//            rows of those features over all of K, split over the four
//            wavefronts of a workgroup by K slices; their part sums meet in
//            LDS and form h = bf16(silu(gate) * up);
//   one device-wide barrier;
//   phase B  down and combine: unit = (token, 8 output rows); the unit's
//            W_down slices of the k + 1 rows times their h, weighted by the
//            routing weights (1 for the shared expert), summed in fp32 and
//            written as bf16.
// The loads of a workgroup's first phase B unit are issued once it has
// counted in at the barrier, so that they arrive while it waits.
// Row r of the layer is token r / (k + 1), slot r % (k + 1): slots 0..k-1
// are the routed experts in top-k order, slot k the shared expert.
#include <mutex>

#include "common.hpp"
#include "topk.hpp"
#include "w4.hpp"

namespace lily {

constexpr int kDecThreads = 256;
constexpr int kDecodeMaxT = 4;       // lily_moe_decode serves T <= this
constexpr int kDecMaxGrid = 512;     // workgroups: at most one per compute unit and this
constexpr int kDecXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round robin over them
constexpr int kDecASlices = 8;       // phase A slices per lane and weight matrix loaded at once
constexpr int kDecMaxUnits = 16;     // lily_moe_decode: gate/up units per workgroup
constexpr int kDecUnitBatch = 4;     // lily_moe_decode: units whose slices are loaded at once
constexpr int kDecItBatch = 2;       // lily_moe_decode: slices per row and wavefront loaded at once
constexpr int kDecBRounds = 6;       // phase B rounds per wavefront loaded at once
constexpr int kDecLdsWords = 8192;   // LDS: x rows (phase A) or h rows (phase B), bf16 pairs
constexpr int kDecXChunks = 8;       // x 16-byte chunks staged per thread: T * H <= 16384
constexpr int kDecHChunks = kDecLdsWords / 4 / kDecThreads;  // h chunks staged per thread
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
    uint16_t* h;          // [R][F] bf16
    uint16_t* out;        // [T, H]
    int32_t* bar;         // [2] groups arrived, groups exited: zero on entry, left zero
    int32_t* grp;         // per barrier group: arrivals, exits, kBarLine ints apart; zero on
                          // entry, left zero
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

// Dot product of a slice's 32 weights with 32 staged values v (16 permuted
// words). Each weight is rebuilt as w = bf16(scale * q + bias) exactly as
// the grouped GEMMs do (one fp32 fma on q * 2^-9 from v_cvt_pk_f32_fp8, then
// RNE to bf16), and the bf16 pairs (w_j, w_j+4) meet the staged words in
// bf16 dot2 instructions with fp32 accumulation. (Using the exact fp32
// weights instead, applying scale and bias to each 32-weight sum, is cheaper
// but misses the tolerance on tokens whose layer output is small next to
// its terms: a systematic 2^-9 per weight then survives the cancellation.)
__device__ __forceinline__ float dot_slice(const Slice& s, const uint32_t* v) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const float s512 = bf16_bits_to_float(s.sc) * 512.0f, b = bf16_bits_to_float(s.bi);
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t lo = s.q[w] & 0x0F0F0F0Fu;         // elements 0, 2, 4, 6
        const uint32_t hi = (s.q[w] >> 4) & 0x0F0F0F0Fu;  // elements 1, 3, 5, 7
        const f2 e02 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
        const f2 e46 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
        const f2 e13 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
        const f2 e57 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
        const uint32_t wt[4] = {pack_bf16x2(fmaf(s512, e02[0], b), fmaf(s512, e46[0], b)),   // 0, 4
                                pack_bf16x2(fmaf(s512, e13[0], b), fmaf(s512, e57[0], b)),   // 1, 5
                                pack_bf16x2(fmaf(s512, e02[1], b), fmaf(s512, e46[1], b)),   // 2, 6
                                pack_bf16x2(fmaf(s512, e13[1], b), fmaf(s512, e57[1], b))};  // 3, 7
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

// Device-wide barrier in two levels. Device-scope atomics on one address
// are serialised (256 arrivals on one counter took ~7 us), so workgroup w
// counts in at the counter of its group w % kBarGroups (counters on separate
// 128-byte lines) and the last of a group counts the group in at `bar`;
// everyone waits for all groups there. Every global store of the workgroup
// is complete before it counts. The wait is bounded in time: on a timeout it
// flags the error and goes on, so no wave can wait forever.
constexpr int kBarGroups = 8;
constexpr int kBarLine = 32;  // ints between group counters: one 128-byte line each
__device__ __forceinline__ int bar_groups(int G) { return G < kBarGroups ? G : kBarGroups; }
__device__ __forceinline__ int bar_group_size(int G, int g) {
    return (G - g + kBarGroups - 1) / kBarGroups;
}
// Split in two: between barrier_arrive and barrier_wait a workgroup may
// issue loads, which stay in flight through the wait. The counters only
// grow within a launch, so one launch can pass several barriers: the
// instance-th barrier (from 0) is passed when `bar` reaches (instance + 1)
// groups, and a group counts in when its counter reaches a multiple of the
// group's size. Every workgroup arrives at every instance.
// lead: the thread that counts the workgroup in; every wavefront waits for
// its own stores first, or only the lead's wavefront when it made all of
// the stores the barrier publishes (the others' loads stay in flight).
__device__ __forceinline__ void barrier_arrive(int32_t* bar, int32_t* grp, int lead = 0,
                                               bool all_stored = true) {
    const int G = gridDim.x, g = blockIdx.x % kBarGroups;
    if (all_stored || threadIdx.x / kWave == lead / kWave)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (threadIdx.x == lead) {
        const int prev = __hip_atomic_fetch_add(grp + g * kBarLine, 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        if ((prev + 1) % bar_group_size(G, g) == 0)
            __hip_atomic_fetch_add(bar, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}
// poll: the polling thread. Its loads return in order, so it should belong
// to a wavefront with no loads in flight.
__device__ __forceinline__ void barrier_wait(int32_t* bar, int32_t* err, int instance = 0,
                                             int poll = 0) {
    if (threadIdx.x == poll) {
        const int target = (instance + 1) * bar_groups(gridDim.x);
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(2);
            if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > kSpinTicks) {
                __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    lds_barrier();
}

// Every workgroup has passed every barrier wait before it counts out here,
// in the same two levels: the last of a group clears the group's counters,
// the last group clears `bar` for the next launch. lead: the thread that
// made the workgroup's last arrival, so that its count-out follows it.
__device__ __forceinline__ void barrier_exit(int32_t* bar, int32_t* grp, int lead = 0) {
    const int G = gridDim.x;
    if (threadIdx.x == lead) {
        const int g = blockIdx.x % kBarGroups;
        int32_t* gc = grp + g * kBarLine;
        if (__hip_atomic_fetch_add(gc + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            bar_group_size(G, g) - 1) {
            __hip_atomic_store(gc, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(gc + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (__hip_atomic_fetch_add(bar + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                bar_groups(G) - 1) {
                __hip_atomic_store(bar, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(bar + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// Phase B ranges: workgroup w of G takes units [w NB / G, (w + 1) NB / G)
// (NB * G < 2^31 on the host's checks).
__device__ __forceinline__ int range_begin(int w, int nb, int g) { return (unsigned)(w * nb) / (unsigned)g; }

__global__ void __launch_bounds__(kDecThreads) moe_decode_kernel(DecodeArgs a) {
    __shared__ float s_pa[kDecMaxUnits][kDecThreads / kWave][16];  // phase A part sums
    __shared__ int32_t s_ids[kDecodeMaxT * kMaxTopk];
    __shared__ float s_w[kDecodeMaxT * kMaxTopk];
    __shared__ __attribute__((aligned(16))) uint32_t s_buf[kDecLdsWords];
    __shared__ float s_bred[kDecThreads / kWave][kDecPiece];

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int G = gridDim.x;
    const int wg = blockIdx.x;
    // Units are dealt by this index, which numbers the workgroups XCD by
    // XCD (workgroup w runs on XCD w % 8): consecutive units, which share
    // the scale and bias lines of their packed blocks, meet in one L2.
    const int vw = G % kDecXcds == 0 ? (wg % kDecXcds) * (G / kDecXcds) + wg / kDecXcds : wg;
    const int k = a.k;
    const int R = a.T * (k + 1);
    const int H = a.H, F = a.F;
    const int nkg = H / kGroup;        // groups along K of gate/up
    const int nsf = F / kPackRows;     // 128-row slabs of gate/up
    const int nkgF = F / kGroup;       // groups along K of down
    const int nsH = H / kPackRows;     // 128-row slabs of down

    // x of every token, staged in LDS as permuted bf16 pairs, loaded first so
    // that it arrives together with the router logits.
    const int x_words = a.T * (H / 2);
    const Rsrc x_rs = make_rsrc(a.x, x_words * 4);
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
    if (wg == 0 && tid < a.T * k) {
        a.topk_ids[tid] = s_ids[tid];
        a.topk_w[tid] = s_w[tid];
    }

    // Phase B units of this workgroup: wavefront v takes rounds v, v + 4, ...
    // of each. Round rho of a unit: slot j = rho / nq, groups 4 gq .. 4 gq + 3
    // with gq = rho % nq; lane l: group 4 gq + l / 16, half (l / 8) % 2,
    // output row l % 8.
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int pieces_per_tok = H / kDecPiece;
    const int UB = a.T * pieces_per_tok;
    const int ub0 = range_begin(vw, UB, G), ub1 = range_begin(vw + 1, UB, G);
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
    // Rounds past the end of a phase B unit are clamped onto valid data
    // (results unused).
    Slice pb[kDecBRounds];
    float pw[kDecBRounds];
    int ph[kDecBRounds];
    const int ub_first = ub0 < ub1 ? ub0 : 0;
    auto prefetch_b = [&]() {
#pragma unroll
        for (int n = 0; n < kDecBRounds; ++n)
            pb[n] = b_round(ub_first, min(wv + 4 * n, NRB - 1), pw[n], ph[n]);
    };

    // Phase A: unit u = (row r, features f0 .. f0 + 7): the 8 gate rows and
    // the 8 up rows of those features over all of K. Units are dealt to the
    // workgroup with vw = u % G; wavefront w takes the K slices i = w + 4 m
    // of every unit of its workgroup, so the four wavefronts share each
    // unit's dequantisation and dot products (one wavefront per unit left
    // half of a compute unit's SIMDs idle in this VALU-heavy phase).
    // Lane l covers feature f0 + l % 8 and the 32-weight slices c = l / 8 +
    // 8 i of its rows (group c / 2, half c % 2): each load instruction reads
    // whole 128-byte lines (8 rows x 16 bytes of one block half). A
    // wavefront's sums per unit (its 8 lanes of a feature added by shuffles)
    // go to LDS; then threads add the four parts in wavefront order and form
    // h = bf16(silu(gate) * up).
    const int UA = R * (F / 8);
    const int spr8 = H / 256;  // slices per lane per weight row
    const int l8 = lane % 8, lc = lane / 8;
    const int n_u = vw < UA ? (UA - vw + G - 1) / G : 0;  // <= kDecMaxUnits (host check)
    const int n_it = (spr8 - wv + 3) / 4;                 // this wavefront's slices per row
    const int qoff = (lc >> 1) * kPackBlock;
    for (int ub = 0; ub < n_u; ub += kDecUnitBatch) {
        float pg[kDecUnitBatch], pu[kDecUnitBatch];
        Rsrc rg[kDecUnitBatch], ru[kDecUnitBatch];
        int xb[kDecUnitBatch], rrs[kDecUnitBatch];
#pragma unroll
        for (int b = 0; b < kDecUnitBatch; ++b) {
            pg[b] = pu[b] = 0.0f;
            const int u = vw + G * min(ub + b, n_u - 1);  // past the end: a valid unit, unused
            const int r = u / (F / 8), f0 = (u - r * (F / 8)) * 8;
            const int t = r / (k + 1), j = r - t * (k + 1);
            const bool sh = (j == k);
            const int e = sh ? 0 : s_ids[t * k + j];
            const size_t seg = ((size_t)e * nsf + f0 / kPackRows) * nkg * kPackBlock;
            rg[b] = make_rsrc((sh ? a.sh_gate : a.gate) + seg, nkg * kPackBlock);
            ru[b] = make_rsrc((sh ? a.sh_up : a.up) + seg, nkg * kPackBlock);
            rrs[b] = f0 % kPackRows + l8;
            xb[b] = t * (H / 2) + (lc >> 1) * 32 + (lc & 1) * 16;
        }
        for (int m0 = 0; m0 < n_it; m0 += kDecItBatch) {
            Slice sg[kDecUnitBatch][kDecItBatch], su[kDecUnitBatch][kDecItBatch];
#pragma unroll
            for (int b = 0; b < kDecUnitBatch; ++b)
#pragma unroll
                for (int m = 0; m < kDecItBatch; ++m) {
                    // slices past the row's end are clamped onto its last one
                    const int soff = min(wv + 4 * (m0 + m), spr8 - 1) * 4 * kPackBlock;
                    const int vq = qoff + ((lc & 1) * kPackRows + rrs[b]) * 16;
                    const int vs = qoff + kPackQ + rrs[b] * 2;
                    sg[b][m] = load_slice(rg[b], vq, vs, soff);
                    su[b][m] = load_slice(ru[b], vq, vs, soff);
                }
#pragma unroll
            for (int b = 0; b < kDecUnitBatch; ++b)
#pragma unroll
                for (int m = 0; m < kDecItBatch; ++m)
                    if (ub + b < n_u && m0 + m < n_it) {
                        const int xo = xb[b] + (wv + 4 * (m0 + m)) * 128;
                        pg[b] += dot_slice(sg[b][m], s_buf + xo);
                        pu[b] += dot_slice(su[b][m], s_buf + xo);
                    }
        }
#pragma unroll
        for (int b = 0; b < kDecUnitBatch; ++b) {
            pg[b] += __shfl_xor(pg[b], 8);
            pg[b] += __shfl_xor(pg[b], 16);
            pg[b] += __shfl_xor(pg[b], 32);
            pu[b] += __shfl_xor(pu[b], 8);
            pu[b] += __shfl_xor(pu[b], 16);
            pu[b] += __shfl_xor(pu[b], 32);
            if (lane < 8 && ub + b < n_u) {
                s_pa[ub + b][wv][lane] = pg[b];
                s_pa[ub + b][wv][8 + lane] = pu[b];
            }
        }
    }
    lds_barrier();
    // thread (unit ui, pair q): features 2q, 2q + 1 of the unit
    if (tid < 4 * n_u) {
        const int ui = tid / 4, q = tid % 4;
        const int u = vw + G * ui;
        const int r = u / (F / 8), f0 = (u - r * (F / 8)) * 8;
        float hv[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float g = 0.0f, up = 0.0f;
#pragma unroll
            for (int w = 0; w < kDecThreads / kWave; ++w) {
                g += s_pa[ui][w][2 * q + c];
                up += s_pa[ui][w][8 + 2 * q + c];
            }
            hv[c] = silu(g) * up;
        }
        __hip_atomic_store(reinterpret_cast<uint32_t*>(a.h + (size_t)r * F + f0 + 2 * q),
                           pack_bf16x2(hv[0], hv[1]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Phase B's first rounds are loaded once this workgroup has counted in
    // at the barrier, so that they do not compete with phase A's loads; they
    // arrive during the wait.
    barrier_arrive(a.bar, a.grp);
    prefetch_b();
    barrier_wait(a.bar, a.err);

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
                    acc = fmaf(pw[n], dot_slice(pb[n], s_buf + ph[n]), acc);
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

    barrier_exit(a.bar, a.grp);
}

constexpr int kStackMaxIds = 2048;  // n_layers * topk routing entries held in LDS

// Batch-1 decode through a stack of MoE layers in one launch (T = 1): the
// layers of one decode step chained by the residual glue (r_0 = x_0;
// x_l = bf16(r_l / rms(r_l)); r_{l+1} = r_l + out_l), which the pages run as
// one concurrent pass per step (Lily articles, section "Decode"). Per layer
// the phases of moe_decode_kernel, with two device-wide barriers: after the
// gate/up phase (h complete) and after the down phase (out and r complete).
// The launch routes every layer first (the logits are inputs); the next
// layer's gate/up weight loads do not depend on this layer's output, so they
// are issued between this layer's h barrier arrival and wait and stream
// while this layer's down phase runs.
struct StackArgs {
    int L, H, F, E, k;
    const lily_moe_weights* layers;  // device array [L]
    const float* logits;             // [L][E]
    const uint16_t* x0;              // [H] bf16
    float* r;                        // [H] fp32 residual; r_L on exit
    uint16_t* outs;                  // [L][H] bf16 layer outputs
    int32_t* topk_ids;               // [L][k]
    float* topk_w;                   // [L][k]
    uint16_t* h;                     // kDecXcds copies of [k + 1][F] bf16
    float* rr;                       // kDecXcds copies of r_l [H]
    float eps;
    int32_t* bar;
    int32_t* grp;
    int32_t* err;
};

__global__ void __launch_bounds__(kDecThreads) moe_decode_stack_kernel(StackArgs a) {
    __shared__ int32_t s_ids[kStackMaxIds];  // [L][k]: every layer's routing
    __shared__ float s_w[kStackMaxIds];
    __shared__ __attribute__((aligned(16))) uint32_t s_buf[kDecLdsWords];
    __shared__ float s_bred[kDecThreads / kWave][kDecPiece];
    __shared__ float s_part[kDecThreads / kWave];
    __shared__ float s_r[kDecASlices * 256];  // r_l (H <= 2048)
    __shared__ float s_pa[kDecUnitBatch][kDecThreads / kWave][16];  // phase A part sums

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int G = gridDim.x;
    const int wg = blockIdx.x;
    const int vw = G % kDecXcds == 0 ? (wg % kDecXcds) * (G / kDecXcds) + wg / kDecXcds : wg;
    // r and h are kept in one copy per XCD (written by their producers to
    // all copies): every workgroup reads them with device-coherent loads,
    // which go past the XCD's L2, and 256 readers of one copy load its
    // memory channels with the same lines.
    const int xc = wg % kDecXcds;
    const int k = a.k, E = a.E, H = a.H, F = a.F;
    const int R = k + 1;
    const int nkg = H / kGroup, nsf = F / kPackRows, nkgF = F / kGroup, nsH = H / kPackRows;

    // Phase A units of this workgroup (at most kDecUnitBatch: the host
    // checks R * F / 8 <= 4 G): unit u = (row j, features f0 .. f0 + 7) for
    // u = vw + G i. As in moe_decode_kernel, wavefront w takes the K slices
    // w, w + 4, ... of each of them (at most kDecItBatch: H <= 2048), and the
    // part sums meet in LDS.
    const int UA = R * (F / 8);
    const int n_u = vw < UA ? (UA - vw + G - 1) / G : 0;
    const int l8 = lane % 8, lc = lane / 8;
    const int spr8 = H / 256;
    const int n_it = (spr8 - wv + 3) / 4;
    const int qoff = (lc >> 1) * kPackBlock;
    const int xbase = (lc >> 1) * 32 + (lc & 1) * 16;
    Slice sg[kDecUnitBatch][kDecItBatch], su[kDecUnitBatch][kDecItBatch];

    // Phase B unit range (output rows of 8).
    const int UB = H / kDecPiece;
    const int ub0 = range_begin(vw, UB, G), ub1 = range_begin(vw + 1, UB, G);
    const int nq = nkgF / 4;
    const int NRB = R * nq;
    const int b_gl = lane / 16, b_half = (lane / 8) % 2, b_row = lane % kDecPiece;
    Slice pb[kDecBRounds];
    float pw[kDecBRounds];
    int ph[kDecBRounds];

    // Routing of every layer first: its logits are inputs of the launch.
    // Wavefront v takes layers v, v + 4, ...; workgroup 0 writes them out.
    for (int l = wave; l < a.L; l += kDecThreads / kWave)
        topk_one_token(a.logits, l, E, k, s_ids, s_w);
    lds_barrier();
    if (wg == 0)
        for (int i = tid; i < a.L * k; i += kDecThreads) {
            a.topk_ids[i] = s_ids[i];
            a.topk_w[i] = s_w[i];
        }
    // Gate/up weight loads of this wavefront's slices for layer l (units and
    // slices past the end are clamped onto valid ones: loaded, not used).
    auto issue_a = [&](int l) {
        if (n_u == 0) return;
        const lily_moe_weights& w = a.layers[l];
#pragma unroll
        for (int b = 0; b < kDecUnitBatch; ++b) {
            const int u = vw + G * min(b, n_u - 1);
            const int j = u / (F / 8), f0 = (u - j * (F / 8)) * 8;
            const bool sh = j == k;
            const int e = sh ? 0 : s_ids[l * k + j];
            const size_t seg = ((size_t)e * nsf + f0 / kPackRows) * nkg * kPackBlock;
            const Rsrc rg = make_rsrc(static_cast<const char*>(sh ? w.sh_gate : w.gate) + seg,
                                      nkg * kPackBlock);
            const Rsrc ru = make_rsrc(static_cast<const char*>(sh ? w.sh_up : w.up) + seg,
                                      nkg * kPackBlock);
            const int rr = f0 % kPackRows + l8;
            const int vq = qoff + ((lc & 1) * kPackRows + rr) * 16;
            const int vs = qoff + kPackQ + rr * 2;
#pragma unroll
            for (int m = 0; m < kDecItBatch; ++m) {
                const int soff = min(wv + 4 * m, spr8 - 1) * 4 * kPackBlock;
                sg[b][m] = load_slice(rg, vq, vs, soff);
                su[b][m] = load_slice(ru, vq, vs, soff);
            }
        }
    };
    // One phase B round: slot j = rho / nq, groups 4 gq .. 4 gq + 3 of unit ub.
    auto b_round = [&](int l, int ub, int rho, float& wj, int& hoff) -> Slice {
        const lily_moe_weights& w = a.layers[l];
        const int r0 = ub * kDecPiece;
        const int j = rho / nq, gq = rho - j * nq;
        const bool sh = (j == k);
        const int e = sh ? 0 : s_ids[l * k + j];
        wj = sh ? 1.0f : s_w[l * k + j];
        hoff = (j * F + (4 * gq + b_gl) * kGroup + b_half * 32) / 2;
        const char* stack = static_cast<const char*>(sh ? w.sh_down : w.down);
        const Rsrc rs = make_rsrc(
            stack + ((size_t)(e * nsH + r0 / kPackRows) * nkgF + 4 * gq) * kPackBlock,
            4 * kPackBlock);
        const int rrb = r0 % kPackRows + b_row;
        return load_slice(rs, b_gl * kPackBlock + (b_half * kPackRows + rrb) * 16,
                          b_gl * kPackBlock + kPackQ + rrb * 2, 0);
    };
    const int ub_first = ub0 < ub1 ? ub0 : 0;

    // The last wavefront loads r and h for the workgroup, stores each
    // layer's out and r, counts the workgroup in and polls.
    constexpr int kLeadWave = kDecThreads / kWave - 1;
    constexpr int kLead = kLeadWave * kWave;
    int inst = 0;  // barrier instances passed or arrived at
    issue_a(0);
    for (int l = 0; l < a.L; ++l) {
        if (l > 0) barrier_wait(a.bar, a.err, inst - 1, kLead);  // layer l - 1's out and r

        // x_l = bf16(r_l / sqrt(mean(r_l^2) + eps)), r_0 = x_0. The lead
        // wavefront, which has no gate/up loads in flight (a load returns
        // after every earlier one of its wavefront), brings r_l into LDS;
        // then thread t takes elements 4t + 1024 i .. + 3 and the sum of
        // squares runs in the order of residual_norm_kernel (same result bit
        // for bit).
        {
            if (wave == kLeadWave) {
                // all of r in flight at once: pairs of floats, 16 per lane
                constexpr int kPairs = kDecASlices * 256 / 2 / kWave;
                uint64_t t[kPairs];
#pragma unroll
                for (int j = 0; j < kPairs; ++j) {
                    const int p = min(lane + j * kWave, H / 2 - 1);
                    t[j] = l == 0 ? (uint64_t)reinterpret_cast<const uint32_t*>(a.x0)[p]
                                  : __hip_atomic_load(
                                        reinterpret_cast<const uint64_t*>(a.rr + (size_t)xc * H) + p,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int j = 0; j < kPairs; ++j) {
                    const int p = lane + j * kWave;
                    if (p < H / 2) {
                        if (l == 0) {  // two bf16 of x0
                            s_r[2 * p] = bf16_bits_to_float((uint32_t)t[j] & 0xFFFFu);
                            s_r[2 * p + 1] = bf16_bits_to_float(((uint32_t)t[j]) >> 16);
                        } else {
                            s_r[2 * p] = __uint_as_float((uint32_t)t[j]);
                            s_r[2 * p + 1] = __uint_as_float((uint32_t)(t[j] >> 32));
                        }
                    }
                }
            }
            lds_barrier();
            float v[kDecXChunks][4];
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < kDecXChunks; ++i) {
                const int n = tid * 4 + i * kDecThreads * 4;
                if (n < H) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[i][c] = s_r[n + c];
                    ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] +
                          v[i][3] * v[i][3];
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
            if (lane == 0) s_part[wave] = ss;
            lds_barrier();
            float tot = 0.0f;
#pragma unroll
            for (int w = 0; w < kDecThreads / kWave; ++w) tot += s_part[w];
            const float inv = 1.0f / sqrtf(tot / (float)H + a.eps);
#pragma unroll
            for (int i = 0; i < kDecXChunks; ++i) {
                const int n = tid * 4 + i * kDecThreads * 4;
                if (n < H) {
                    s_buf[n / 2] = pack_bf16x2(v[i][0] * inv, v[i][1] * inv);
                    s_buf[n / 2 + 1] = pack_bf16x2(v[i][2] * inv, v[i][3] * inv);
                }
            }
            lds_barrier();
            // natural bf16 pairs -> the permuted chunks dot_slice reads
            for (int c = tid; c < H / 8; c += kDecThreads) {
                const u32x4 p = *reinterpret_cast<const u32x4*>(s_buf + 4 * c);
                *reinterpret_cast<u32x4*>(s_buf + 4 * c) = permute_chunk(p);
            }
            lds_barrier();
        }

        // This layer's down weights: they arrive during phase A and its
        // barrier.
#pragma unroll
        for (int n = 0; n < kDecBRounds; ++n)
            pb[n] = b_round(l, ub_first, min(wv + 4 * n, NRB - 1), pw[n], ph[n]);
        // Phase A of layer l: the slices' loads were issued earlier.
#pragma unroll
        for (int b = 0; b < kDecUnitBatch; ++b) {
            float pg = 0.0f, pu = 0.0f;
#pragma unroll
            for (int m = 0; m < kDecItBatch; ++m)
                if (b < n_u && m < n_it) {
                    const int xo = xbase + (wv + 4 * m) * 128;
                    pg += dot_slice(sg[b][m], s_buf + xo);
                    pu += dot_slice(su[b][m], s_buf + xo);
                }
            pg += __shfl_xor(pg, 8);
            pg += __shfl_xor(pg, 16);
            pg += __shfl_xor(pg, 32);
            pu += __shfl_xor(pu, 8);
            pu += __shfl_xor(pu, 16);
            pu += __shfl_xor(pu, 32);
            if (lane < 8 && b < n_u) {
                s_pa[b][wv][lane] = pg;
                s_pa[b][wv][8 + lane] = pu;
            }
        }
        lds_barrier();
        if (tid < 4 * n_u) {  // thread (unit ui, pair q): features 2q, 2q + 1
            const int ui = tid / 4, q = tid % 4;
            const int u = vw + G * ui;
            const int j = u / (F / 8), f0 = (u - j * (F / 8)) * 8;
            float hv[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float g = 0.0f, up = 0.0f;
#pragma unroll
                for (int w = 0; w < kDecThreads / kWave; ++w) {
                    g += s_pa[ui][w][2 * q + c];
                    up += s_pa[ui][w][8 + 2 * q + c];
                }
                hv[c] = silu(g) * up;
            }
            const uint32_t hw = pack_bf16x2(hv[0], hv[1]);
#pragma unroll
            for (int c = 0; c < kDecXcds; ++c)
                __hip_atomic_store(
                    reinterpret_cast<uint32_t*>(a.h + ((size_t)c * R + j) * F + f0 + 2 * q), hw,
                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        barrier_arrive(a.bar, a.grp, kLead, true);
        const int inst_h = inst++;
        // While the others finish phase A: the next layer's gate/up weights,
        // which stream during this layer's down phase.
        if (l + 1 < a.L) issue_a(l + 1);
        barrier_wait(a.bar, a.err, inst_h, kLead);

        // Phase B of layer l: out_l rows and r_{l+1} = r_l + out_l. h comes
        // into LDS through the lead wavefront, for the same reason as r.
        const int h_words = R * F / 2;
        if (wave == kLeadWave) {
            // 16-byte chunks as two 8-byte loads, 12 chunks per lane in flight
            const uint64_t* hg = reinterpret_cast<const uint64_t*>(a.h + (size_t)xc * R * F);
            constexpr int kC = 12;
            for (int c0 = lane; c0 < h_words / 4; c0 += kC * kWave) {
                uint64_t t[kC][2];
#pragma unroll
                for (int j = 0; j < kC; ++j) {
                    const int c = min(c0 + j * kWave, h_words / 4 - 1);
                    t[j][0] = __hip_atomic_load(hg + 2 * c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    t[j][1] = __hip_atomic_load(hg + 2 * c + 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int j = 0; j < kC; ++j)
                    if (c0 + j * kWave < h_words / 4) {
                        const u32x4 hr = {(uint32_t)t[j][0], (uint32_t)(t[j][0] >> 32),
                                          (uint32_t)t[j][1], (uint32_t)(t[j][1] >> 32)};
                        *reinterpret_cast<u32x4*>(s_buf + 4 * (c0 + j * kWave)) = permute_chunk(hr);
                    }
            }
        }
        lds_barrier();
        for (int ub = ub0; ub < ub1; ++ub) {
            float acc = 0.0f;
            for (int n0 = 0; wv + 4 * n0 < NRB; n0 += kDecBRounds) {
                if (n0 > 0) {
#pragma unroll
                    for (int n = 0; n < kDecBRounds; ++n)
                        pb[n] = b_round(l, ub, min(wv + 4 * (n0 + n), NRB - 1), pw[n], ph[n]);
                }
#pragma unroll
                for (int n = 0; n < kDecBRounds; ++n)
                    if (wv + 4 * (n0 + n) < NRB)
                        acc = fmaf(pw[n], dot_slice(pb[n], s_buf + ph[n]), acc);
            }
            if (ub + 1 < ub1) {
#pragma unroll
                for (int n = 0; n < kDecBRounds; ++n)
                    pb[n] = b_round(l, ub + 1, min(wv + 4 * n, NRB - 1), pw[n], ph[n]);
            }
            acc += __shfl_xor(acc, 8);
            acc += __shfl_xor(acc, 16);
            acc += __shfl_xor(acc, 32);
            if (lane < kDecPiece) s_bred[wave][lane] = acc;
            lds_barrier();
            if (tid >= kLead && tid < kLead + kDecPiece) {
                float o = 0.0f;
#pragma unroll
                for (int v = 0; v < kDecThreads / kWave; ++v) o += s_bred[v][tid - kLead];
                const int n = ub * kDecPiece + tid - kLead;
                const uint16_t ob = float_to_bf16_bits(o);
                a.outs[(size_t)l * H + n] = ob;
                const float rn = s_r[n] + bf16_bits_to_float(ob);  // r_l, staged for the norm
#pragma unroll
                for (int c = 0; c < kDecXcds; ++c)
                    __hip_atomic_store(a.rr + (size_t)c * H + n, rn, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                if (l == a.L - 1) a.r[n] = rn;
            }
            lds_barrier();
        }
        barrier_arrive(a.bar, a.grp, kLead, false);
        ++inst;
    }
    barrier_exit(a.bar, a.grp, kLead);
}

// One workgroup per compute unit, at most kDecMaxGrid.
static int decode_grid() {
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n = 0;
        cus[dev] = n > 0 ? n : 1;
    }
    return cus[dev] < kDecMaxGrid ? cus[dev] : kDecMaxGrid;
}

// lily_moe_decode: h, bf16 [T (k + 1), F]. lily_moe_decode_stack (T = 1):
// kDecXcds copies of h, then kDecXcds copies of r [H] fp32.
static size_t stack_h_bytes(const lily_moe_dims& d) {
    return ((size_t)kDecXcds * (d.topk + 1) * d.F * sizeof(uint16_t) + 255) & ~(size_t)255;
}
size_t decode_workspace_bytes(const lily_moe_dims& d) {
    if (d.T > kDecodeMaxT) return 0;
    const size_t one = (size_t)d.T * (d.topk + 1) * d.F * sizeof(uint16_t);
    if (d.T != 1) return one;
    const size_t stack = stack_h_bytes(d) + (size_t)kDecXcds * d.H * sizeof(float);
    return one > stack ? one : stack;
}

constexpr int kDecMaxH = 4096;  // x of kDecodeMaxT tokens fills the LDS staging area
static_assert(kDecodeMaxT * kDecMaxH / 2 <= kDecLdsWords, "x staging");
static_assert(kDecodeMaxT * kDecMaxH / 2 <= kDecXChunks * 4 * kDecThreads, "x chunks");

int decode_supported(const lily_moe_dims& d) {
    if (d.T > kDecodeMaxT)
        return set_error(LILY_ERR_UNSUPPORTED, "T = %d; lily_moe_decode serves T <= %d", d.T,
                         kDecodeMaxT);
    if (d.H % (2 * kDecThreads) || d.H > kDecMaxH)
        return set_error(LILY_ERR_UNSUPPORTED, "H = %d must be a multiple of 512, at most %d",
                         d.H, kDecMaxH);
    if (d.F % (4 * kGroup) || (long)(d.topk + 1) * d.F > 2L * kDecLdsWords)
        return set_error(LILY_ERR_UNSUPPORTED,
                         "F = %d must be a multiple of 256 with (topk + 1) * F <= %d", d.F,
                         2 * kDecLdsWords);
    return LILY_OK;
}

// The launch of lily_moe_decode and lily_moe_decode_noalloc: h [T (k + 1),
// F] bf16 scratch, bar / grp / err the device-wide barrier's counters (zero
// on entry, left zero) and its give-up flag.
static int launch_decode_with(const lily_moe_dims& d, const lily_moe_weights& w,
                              const float* logits, const uint16_t* x, int32_t* topk_ids,
                              float* topk_w, uint16_t* out, uint16_t* h, int32_t* bar,
                              int32_t* grp, int32_t* err, hipStream_t stream) {
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
    a.topk_ids = topk_ids;
    a.topk_w = topk_w;
    a.h = h;
    a.out = out;
    a.bar = bar;
    a.grp = grp;
    a.err = err;
    const int g = decode_grid();
    // (checked here, after the arguments: it depends on the device)
    const long units = (long)d.T * (d.topk + 1) * (d.F / 8);
    if (units > (long)kDecMaxUnits * g)
        return set_error(LILY_ERR_UNSUPPORTED,
                         "T * (topk + 1) * F / 8 = %ld gate/up units exceed %d per compute unit",
                         units, kDecMaxUnits);
    // At most one workgroup per compute unit, each needing a fraction of a
    // compute unit's registers and LDS: all are resident at once, which the
    // device-wide barrier relies on.
    hipLaunchKernelGGL(moe_decode_kernel, dim3((unsigned)g), dim3(kDecThreads), 0, stream, a);
    return check_launch("decode");
}

int launch_decode(const lily_moe_dims& d, const lily_moe_weights& w, const float* logits,
                  const uint16_t* x, const lily_moe_routing& r, uint16_t* out, void* workspace,
                  hipStream_t stream) {
    static_assert(kQueueInts + kBarGroups * kBarLine <= kSchedInts, "barrier group counters");
    return launch_decode_with(d, w, logits, x, r.topk_ids, r.topk_w, out,
                              static_cast<uint16_t*>(workspace), r.sched + kDecodeBarrier,
                              r.sched + kQueueInts, r.sched + kDecodeBarrier + 2, stream);
}

// Scratch of lily_moe_decode_noalloc, for callers that cannot allocate: the
// barrier counters (kNoAllocCtrInts ints, laid out as in a routing's sched
// array), then h of up to kDecodeMaxT tokens. Each GPU the library runs on
// holds its own copy until the process ends. Host code never uses the
// array's name as an address: the device address of each GPU's copy comes
// from hipGetSymbolAddress, once per device.
constexpr int kNoAllocCtrInts = 1024;
constexpr size_t kNoAllocHBytes = (size_t)kDecodeMaxT * 2 * kDecLdsWords * sizeof(uint16_t);
constexpr size_t kNoAllocBytes = kNoAllocCtrInts * sizeof(int32_t) + kNoAllocHBytes;
static_assert(kQueueInts + kBarGroups * kBarLine <= kNoAllocCtrInts &&
                  kDecodeBarrier + 3 <= kNoAllocCtrInts, "no-alloc barrier counters");
static __device__ __align__(256) char scratch[kNoAllocBytes];

constexpr int kNoAllocMaxDevices = 64;
static std::mutex g_scratch_mu;
static char* g_scratch[kNoAllocMaxDevices];

static int scratch_of_device(char** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices)
        return set_error(LILY_ERR_HIP, "decode_noalloc: no current device below %d",
                         kNoAllocMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return set_error(LILY_ERR_HIP, "decode_noalloc: hipGetSymbolAddress: %s",
                             hipGetErrorString(e));
        g_scratch[dev] = static_cast<char*>(p);
    }
    *out = g_scratch[dev];
    return LILY_OK;
}

// Clears the barrier counters (a kernel rather than a memset, so that the
// call also behaves under graph capture) and the caller's status word.
__global__ void __launch_bounds__(256) clear_ints_kernel(int32_t* p, int n, int32_t* status) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
    if (status && threadIdx.x == 0) *status = 0;
}

int launch_decode_noalloc(const lily_moe_dims& d, const lily_moe_weights& w, const float* logits,
                          const uint16_t* x, int32_t* topk_ids, float* topk_w, uint16_t* out,
                          int32_t* status, hipStream_t stream) {
    const size_t need = (size_t)d.T * (d.topk + 1) * d.F * sizeof(uint16_t);
    if (need > kNoAllocHBytes)
        return set_error(LILY_ERR_UNSUPPORTED,
                         "decode_noalloc: h of T * (topk + 1) * F = %zu bytes exceeds the %zu-byte "
                         "scratch", need, kNoAllocHBytes);
    char* base = nullptr;
    int rc = scratch_of_device(&base);
    if (rc) return rc;
    int32_t* ctr = reinterpret_cast<int32_t*>(base);
    uint16_t* h = reinterpret_cast<uint16_t*>(base + kNoAllocCtrInts * sizeof(int32_t));
    hipLaunchKernelGGL(clear_ints_kernel, dim3(1), dim3(256), 0, stream, ctr, kNoAllocCtrInts,
                       status);
    if ((rc = check_launch("decode_noalloc clear"))) return rc;
    return launch_decode_with(d, w, logits, x, topk_ids, topk_w, out, h, ctr + kDecodeBarrier,
                              ctr + kQueueInts, status ? status : ctr + kDecodeBarrier + 2, stream);
}

int decode_stack_supported(const lily_moe_dims& d, int n_layers) {
    if (n_layers < 1) return set_error(LILY_ERR_INVALID_ARG, "n_layers = %d must be >= 1", n_layers);
    if ((long)n_layers * d.topk > kStackMaxIds)
        return set_error(LILY_ERR_UNSUPPORTED, "n_layers * topk = %ld exceeds %d",
                         (long)n_layers * d.topk, kStackMaxIds);
    if (d.T != 1)
        return set_error(LILY_ERR_UNSUPPORTED, "T = %d; lily_moe_decode_stack serves T = 1", d.T);
    if (d.H % (2 * kDecThreads) || d.H > kDecASlices * 256)
        return set_error(LILY_ERR_UNSUPPORTED, "H = %d must be a multiple of 512, at most %d",
                         d.H, kDecASlices * 256);
    if (d.F % (4 * kGroup) || (long)(d.topk + 1) * d.F > 2L * kDecLdsWords)
        return set_error(LILY_ERR_UNSUPPORTED,
                         "F = %d must be a multiple of 256 with (topk + 1) * F <= %d", d.F,
                         2 * kDecLdsWords);
    const long units = (long)(d.topk + 1) * (d.F / 8);
    if (units > 4L * decode_grid())
        return set_error(LILY_ERR_UNSUPPORTED,
                         "(topk + 1) * F / 8 = %ld gate/up units exceed 4 per compute unit", units);
    return LILY_OK;
}

int launch_decode_stack(const lily_moe_dims& d, int n_layers, const lily_moe_weights* layers,
                        const float* logits, const uint16_t* x0, float* r, uint16_t* outs,
                        int32_t* topk_ids, float* topk_w, int32_t* sched, float eps,
                        void* workspace, hipStream_t stream) {
    StackArgs a{};
    a.L = n_layers;
    a.H = d.H;
    a.F = d.F;
    a.E = d.E;
    a.k = d.topk;
    a.layers = layers;
    a.logits = logits;
    a.x0 = x0;
    a.r = r;
    a.outs = outs;
    a.topk_ids = topk_ids;
    a.topk_w = topk_w;
    a.h = static_cast<uint16_t*>(workspace);
    a.rr = reinterpret_cast<float*>(static_cast<char*>(workspace) + stack_h_bytes(d));
    a.eps = eps;
    a.bar = sched + kDecodeBarrier;
    a.grp = sched + kQueueInts;
    a.err = sched + kDecodeBarrier + 2;
    // At most one workgroup per compute unit, each needing a fraction of a
    // compute unit's registers and LDS: all are resident at once, which the
    // device-wide barriers rely on.
    hipLaunchKernelGGL(moe_decode_stack_kernel, dim3((unsigned)decode_grid()), dim3(kDecThreads),
                       0, stream, a);
    return check_launch("decode_stack");
}

}  // namespace lily
