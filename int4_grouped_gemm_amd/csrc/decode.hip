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
//            rows of those features over all of K, split over the eight
//            wavefronts of a workgroup (two per SIMD) by K slices; their part
//            sums meet in LDS and form h = bf16(silu(gate) * up);
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

constexpr int kDecWaves = 8;         // two wavefronts per SIMD: the phases are VALU bound
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kDecodeMaxT = 4;       // lily_moe_decode serves T <= this
constexpr int kDecMaxGrid = 512;     // workgroups: at most one per compute unit and this
constexpr int kDecXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round robin over them
constexpr int kDecMaxUnits = 16;     // lily_moe_decode: gate/up units per workgroup
constexpr int kDecUnitBatch = 4;     // lily_moe_decode: units whose slices are loaded at once
constexpr int kDecItBatch = 1;       // lily_moe_decode: slices per row and wavefront loaded at once
constexpr int kDecBRounds = 3;       // lily_moe_decode: phase B rounds per wavefront loaded at once
constexpr int kDecLdsWords = 8192;   // LDS: x rows (phase A) or h rows (phase B), bf16 pairs
constexpr int kDecXChunks = 4;       // x 16-byte chunks staged per thread: T * H <= 16384
constexpr int kDecHChunks = kDecLdsWords / 4 / kDecThreads;  // h chunks staged per thread
constexpr int kDecPiece = 8;         // output rows per phase B unit
constexpr long kSpinTicks = 50000000;  // device-wide barrier wait limit: 0.5 s at 100 MHz

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

    // Phase B units of this workgroup: wavefront v takes rounds v, v + 8, ...
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
            pb[n] = b_round(ub_first, min(wv + kDecWaves * n, NRB - 1), pw[n], ph[n]);
    };

    // Phase A: unit u = (row r, features f0 .. f0 + 7): the 8 gate rows and
    // the 8 up rows of those features over all of K. Units are dealt to the
    // workgroup with vw = u % G; wavefront w takes the K slices of quads
    // i = w + 8 m of every unit of its workgroup (i numbers the quads of four
    // groups along K), so the eight wavefronts share each unit's
    // dequantisation and dot products (one wavefront per unit left most of a
    // compute unit's SIMDs idle in this VALU-heavy phase).
    // Lane l covers feature f0 + l % 8 and the 32-weight slices c = l / 8 +
    // 8 i of its rows (group c / 2, half c % 2): each load instruction reads
    // whole 128-byte lines (8 rows x 16 bytes of one block half). A
    // wavefront's sums per unit (its 8 lanes of a feature added by shuffles)
    // go to LDS; then threads add the eight parts in wavefront order and form
    // h = bf16(silu(gate) * up).
    const int UA = R * (F / 8);
    const int spr8 = H / 256;  // slices per lane per weight row
    const int l8 = lane % 8, lc = lane / 8;
    const int n_u = vw < UA ? (UA - vw + G - 1) / G : 0;  // <= kDecMaxUnits (host check)
    const int n_it = (spr8 - wv + kDecWaves - 1) / kDecWaves;  // this wavefront's quads
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
                    const int soff = min(wv + kDecWaves * (m0 + m), spr8 - 1) * 4 * kPackBlock;
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
                        const int xo = xb[b] + (wv + kDecWaves * (m0 + m)) * 128;
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
        for (int n0 = 0; wv + kDecWaves * n0 < NRB; n0 += kDecBRounds) {
            if (n0 > 0) {
#pragma unroll
                for (int n = 0; n < kDecBRounds; ++n)
                    pb[n] = b_round(u, min(wv + kDecWaves * (n0 + n), NRB - 1), pw[n], ph[n]);
            }
#pragma unroll
            for (int n = 0; n < kDecBRounds; ++n)
                if (wv + kDecWaves * (n0 + n) < NRB)
                    acc = fmaf(pw[n], dot_slice(pb[n], s_buf + ph[n]), acc);
        }
        // the next unit's first rounds, in flight during this unit's sums
        if (u + 1 < ub1) {
#pragma unroll
            for (int n = 0; n < kDecBRounds; ++n)
                pb[n] = b_round(u + 1, min(wv + kDecWaves * n, NRB - 1), pw[n], ph[n]);
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

constexpr int kStackMaxIds = 1024;  // n_layers * topk routing entries held in LDS

// Batch-1 decode through a stack of MoE layers in one launch (T = 1): the
// layers of one decode step chained by the residual glue (r_0 = x_0;
// x_l = bf16(r_l / rms(r_l)); r_{l+1} = r_l + out_l), which the pages run as
// one concurrent pass per step (Lily articles, section "Decode"). Per layer
// the phases of moe_decode_kernel with the same split of the sums over the
// eight wavefronts, so that both kernels add in the same order, and the
// norm in residual_norm_kernel's order: the outputs equal those of the
// chain of per-layer launches bit for bit.
//
// A workgroup has three roles, each a loop of its own over the layers:
//  - eight compute wavefronts (two per SIMD) run the two phases from LDS,
//    read the h exchange into LDS between them and (wavefront 0) make the
//    out stores;
//  - one lead wavefront keeps r in LDS, makes the h stores, reads the out
//    exchange, adds out_l to r and computes the norm (its lane l takes the
//    parts of residual_norm_kernel's threads l, l + 64, l + 128, l + 192:
//    elements 4 l + 256 m + c), writing x into LDS;
//  - seven DMA wavefronts stream the weights.
// The roles meet at two workgroup barriers per layer (x ready; h staged
// with the layer's down weights landed); the other hand-offs (phase A or B
// done) go through LDS counters, so that a wavefront stalled on memory
// holds up only those that need it.
//
// The weights do not depend on the activations, so they are copied into LDS
// (LDS DMA, global_load_lds_dwordx4) ahead of the layer that uses them: a
// workgroup's gate/up share into one of two buffers, its down share into a
// single buffer, each share in parts issued at four points of the layers
// before (so that no burst of weight loads meets an exchange at once). A
// wavefront keeps only about four LDS DMA loads in flight (more stall at
// issue, and the stall holds up the compute unit's other memory accesses
// too), and a compute unit needs some 16-32 KB in flight to stream at the
// memory's rate: hence seven DMA wavefronts. Loads and stores complete in
// order within a wavefront: the lead issues no weight loads, so its
// latency-bound exchange reads never queue behind them; the out stores are
// made by a compute wavefront, so that the lead's next exchange reads do not
// wait for them; and the DMA wavefronts, whose loop has no other vector
// memory access, wait for a share only where its buffer is read
// (hand-counted vmcnt).
//
// The two exchanges per layer (h after phase A, out after phase B: each
// workgroup makes a piece, every workgroup needs all of it) carry their own
// completion: each 8-byte word holds 4 bytes of data (two bf16) and a 4-byte
// tag (the layer + 1), written with one 64-bit store, so the readers poll
// the data itself until every word bears this layer's tag. One memory round
// trip per exchange replaces a barrier (counters and a poll) and the data
// read behind it. The tag words are cleared at the start of the launch,
// before a device-wide barrier that every workgroup passes before its first
// exchange store. A word's next store waits for every reader of the last
// one: a workgroup stores layer l + 1's h only after reading all of out_l,
// which each workgroup stores after reading all of layer l's h (and likewise
// for out), so a word holds this layer's tag or the previous one's. Both
// exchanges are kept in one copy per XCD, read by that XCD's workgroups with
// device-coherent loads.
constexpr int kStkLeadWave = kDecWaves;   // after the compute wavefronts
constexpr int kStkLead = kStkLeadWave * kWave;
constexpr int kStkDmaWaves = 7;
constexpr int kStkWaves = kDecWaves + 1 + kStkDmaWaves;
constexpr int kStkIssuers = kStkDmaWaves;  // wavefronts issuing weight loads
constexpr int kStkThreads = kStkWaves * kWave;
constexpr int kStkMaxUnits = 4;           // gate/up units per workgroup
constexpr int kStkGuBytes = 55296;        // one gate/up buffer (3 units at H = 2048)
constexpr int kStkDBytes = 21504;         // the down buffer ((k + 1) F <= 4608)
constexpr int kStkMaxH = 2048;
constexpr int kStkMaxRF = 4608;           // (k + 1) * F
constexpr int kStkBufWords = kStkMaxRF / 2;  // x (H / 2 words), then h ((k + 1) F / 2 words)
constexpr int kStkRSlots = kStkMaxH / 256;   // r slots m per lead lane (four elements each)
static_assert(kStkWaves * kWave <= 1024, "workgroup size");
constexpr int kStkHSlots = (kStkMaxRF / 8 + kWave * kDecWaves - 1) / (kWave * kDecWaves);  // h chunks (4 words) per compute lane
constexpr int kNormThreads = 256;         // residual_norm_kernel's threads
static_assert(kStkMaxH / 2 <= kStkBufWords, "x staging");

struct StackArgs {
    int L, H, F, E, k;
    const lily_moe_weights* layers;  // device array [L]
    const float* logits;             // [L][E]
    const uint16_t* x0;              // [H] bf16
    float* r;                        // [H] fp32 residual; r_L on exit
    uint16_t* outs;                  // [L][H] bf16 layer outputs
    int32_t* topk_ids;               // [L][k]
    float* topk_w;                   // [L][k]
    uint64_t* hx;                    // kDecXcds copies of [(k + 1) F / 2] tagged bf16 pairs of h
    uint64_t* ox;                    // kDecXcds copies of [H / 2] tagged bf16 pairs of out
    float eps;
    int32_t* bar;
    int32_t* grp;
    int32_t* err;
};

__device__ __forceinline__ uint64_t tagged(uint32_t v, uint32_t tag) {
    return (uint64_t)tag << 32 | v;
}
__device__ __forceinline__ void store_tagged(uint64_t* p, uint64_t w) {
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The lead wavefront's wait for an exchange of n tagged words at p: slot
// (m, e) of this lane reads word w0 + m * wm + e (words past n count as
// present) until every word bears `tag`, reloading only the words still
// missing. Buffer loads with the device-coherence bit (sc1), as the
// device-scope atomic loads are: the lane's offset in a VGPR, m's in an
// SGPR, e's in the instruction. Bounded in time like the barrier wait: on a
// timeout it flags the error and goes on.
template <int M, int EP>
__device__ __forceinline__ void gather_tagged(const uint64_t* p, int n, uint32_t tag,
                                              uint64_t (&t)[M * EP], int w0, int wm,
                                              int32_t* err) {
    const Rsrc rs = make_rsrc(p, n * 8);
    auto load = [&](int m, int e) {
        return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(
                                                rs, (w0 + e) * 8, m * wm * 8, kCoherentLoad));
    };
#pragma unroll
    for (int s = 0; s < M * EP; ++s)
        t[s] = w0 + (s / EP) * wm + s % EP < n ? load(s / EP, s % EP) : tagged(0, tag);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        bool missing = false;
#pragma unroll
        for (int s = 0; s < M * EP; ++s) missing |= (uint32_t)(t[s] >> 32) != tag;
        if (!__any(missing)) break;
        if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > kSpinTicks) {
            if (threadIdx.x % kWave == 0)
                __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int s = 0; s < M * EP; ++s)
            if ((uint32_t)(t[s] >> 32) != tag) t[s] = load(s / EP, s % EP);
    }
}

// Word `word` of all kDecXcds copies (copy_words apart) of an exchange,
// stored as the device-scope atomic stores are (sc1): buffer stores whose
// copy offset sits in an SGPR, so that no per-copy address is kept.
__device__ __forceinline__ void store_copies(Rsrc rs, int word, int copy_words, uint64_t w) {
#pragma unroll
    for (int c = 0; c < kDecXcds; ++c)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, w), rs, word * 8,
                                              c * copy_words * 8, kCoherentLoad);
}

// Global -> LDS copy of 16 bytes per lane from a per-lane address; lane l
// lands at lds_addr + 16 l. Counted in vmcnt like any load; its waits are
// counted by hand (wait_vmcnt_upto).
__device__ __forceinline__ void dma16_lane(const void* p, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane((int)lds_addr)), "v"(p) : "memory");
}
// s_waitcnt vmcnt(n) for a wave-uniform n (an immediate in the
// instruction): n above 15 waits for 15, which waits longer, never shorter.
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
    switch (n < 15 ? n : 15) {
#define LILY_VMCNT_CASE(N) case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
        LILY_VMCNT_CASE(0) LILY_VMCNT_CASE(1) LILY_VMCNT_CASE(2) LILY_VMCNT_CASE(3)
        LILY_VMCNT_CASE(4) LILY_VMCNT_CASE(5) LILY_VMCNT_CASE(6) LILY_VMCNT_CASE(7)
        LILY_VMCNT_CASE(8) LILY_VMCNT_CASE(9) LILY_VMCNT_CASE(10) LILY_VMCNT_CASE(11)
        LILY_VMCNT_CASE(12) LILY_VMCNT_CASE(13) LILY_VMCNT_CASE(14)
        default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
#undef LILY_VMCNT_CASE
    }
}

// Workgroup-local hand-offs through LDS counters (a wait here holds up only
// the waiting wavefront, unlike a barrier).
__device__ __forceinline__ void count_done(int* c) {
    __hip_atomic_fetch_add(c, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void wait_count(const int* c, int target) {
    while (__hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
        __builtin_amdgcn_s_sleep(1);
}

// A slice staged in LDS: q at `q`, the scale at `sb` and the bias 16 bytes on.
__device__ __forceinline__ Slice lds_slice(const char* q, const char* sb) {
    Slice s;
    s.q = *reinterpret_cast<const u32x4*>(q);
    s.sc = *reinterpret_cast<const uint16_t*>(sb);
    s.bi = *reinterpret_cast<const uint16_t*>(sb + 16);
    return s;
}

// The loads of one issuing wavefront (index dw of kStkIssuers) among the
// loads [lo, hi) of a share: loads t = dw, dw + kStkIssuers, ...
__device__ __forceinline__ int loads_of(int dw, int lo, int hi) {
    auto upto = [&](int x) { return (x - dw + kStkIssuers - 1) / kStkIssuers; };
    return upto(hi) - upto(lo);
}

#ifdef LILY_TRACE_ITEMS
// Phase trace of moe_decode_stack_kernel, compiled into the tracing build of
// the library only (liblily_moe_trace.so): per workgroup and layer, the wall
// clock (s_memrealtime, 100 MHz) at eight points, written by lane 0 of the
// wavefront that reaches them. Lead wavefront: 0 layer start, 1 previous
// output gathered and added to r, 2 x staged (norm done), 3 phase A part sums
// of the workgroup ready, 4 h words stored, 5 h gathered by the compute
// wavefronts. Compute wavefront 0: 6 its h gathered, 7 phase B sums of the
// workgroup ready (only in workgroups with a phase B unit).
constexpr int kTraceStackWgs = 256, kTraceStackLayers = 64;
__device__ unsigned long long g_stack_trace[kTraceStackWgs][kTraceStackLayers][8];
#define STACK_TRACE(l, i)                                                                       \
    do {                                                                                        \
        if (lane == 0 && blockIdx.x < kTraceStackWgs && (l) < kTraceStackLayers)                \
            g_stack_trace[blockIdx.x][(l)][(i)] = __builtin_amdgcn_s_memrealtime();             \
    } while (0)
#else
#define STACK_TRACE(l, i) \
    do {                  \
    } while (0)
#endif

__global__ void __launch_bounds__(kStkThreads) moe_decode_stack_kernel(StackArgs a) {
    // Gate/up buffer of a layer: per unit (slot s), the gate then the up
    // weights: q as [quad i][lane][16 bytes] (the lane's slice of quad i),
    // then the scales and biases as [group g][scale 16 B | bias 16 B] (8 rows).
    __shared__ __attribute__((aligned(16))) char s_gu[2][kStkGuBytes];
    // Down buffer: q as [round rho][lane][16 bytes], then [slot j][group][scale
    // 16 B | bias 16 B].
    __shared__ __attribute__((aligned(16))) char s_d[kStkDBytes];
    // x (permuted bf16 pairs) for phase A, then h for phase B.
    __shared__ __attribute__((aligned(16))) uint32_t s_buf[kStkBufWords];
    __shared__ int32_t s_ids[kStackMaxIds];  // [L][k]: every layer's routing
    __shared__ float s_w[kStackMaxIds];
    __shared__ float s_pa[kStkMaxUnits][kDecWaves][16];
    __shared__ float s_bred[kDecWaves][kDecPiece];
    __shared__ __attribute__((aligned(16))) float s_r[kStkMaxH];  // r_l
    __shared__ int s_hflag;  // the layer + 1 whose h stores the lead has issued
    // Compute wavefronts done with phase A / phase B, 8 per layer: the
    // workgroup's other hand-offs wait on these instead of on a barrier.
    __shared__ int s_done_a, s_done_b;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int G = gridDim.x;
    const int wg = blockIdx.x;
    const int vw = G % kDecXcds == 0 ? (wg % kDecXcds) * (G / kDecXcds) + wg / kDecXcds : wg;
    const int xc = wg % kDecXcds;
    const int L = a.L, k = a.k, E = a.E, H = a.H, F = a.F;
    const int R = k + 1;
    const int nkg = H / kGroup, nsf = F / kPackRows, nkgF = F / kGroup, nsH = H / kPackRows;
    const int l8 = lane % 8, lc = lane / 8;
    const int b_gl = lane / 16, b_half = (lane / 8) % 2, b_row = lane % kDecPiece;

    // Phase A units: u = vw + G s, s < n_u (the host checks n_u <= kStkMaxUnits
    // and that they fit a buffer). Per unit and matrix: nqh quads of q, then
    // nsbh KB of scales and biases.
    const int UA = R * (F / 8);
    const int n_u = vw < UA ? (UA - vw + G - 1) / G : 0;
    const int nqh = H / 256;
    const int nsbh = (nkg + 31) / 32;
    const int per_mat = nqh + nsbh;
    const int unit_bytes = 2 * per_mat * 1024;
    // Phase B unit: output rows r0 .. r0 + 7 (at most one per workgroup: the
    // host checks H / 8 <= G). NRB rounds of q, then nsbd KB of scales/biases.
    const int UB = H / kDecPiece;
    const int ub0 = range_begin(vw, UB, G);
    const bool has_b = ub0 < range_begin(vw + 1, UB, G);
    const int r0 = ub0 * kDecPiece;
    const int nq = nkgF / 4;
    const int NRB = R * nq;

    // Weight loads: a layer's gate/up share is NGU loads in four parts
    // [GP(p), GP(p + 1)), its down share ND loads in two parts [DP(p),
    // DP(p + 1)); DMA wavefront dw takes loads dw, dw + 7, ... of each.
    const int dw = wv - kStkLeadWave - 1;
    const int NGU = n_u * 2 * per_mat;
    const int nsbd = (R * nkgF * 2 + 63) / 64;
    const int ND = has_b ? NRB + nsbd : 0;
    auto GP = [&](int p) { return NGU * p / 4; };
    auto DP = [&](int p) { return ND * p / 2; };
    int gcnt[4], dcnt[2];  // this wavefront's loads per part
#pragma unroll
    for (int p = 0; p < 4; ++p) gcnt[p] = loads_of(dw, GP(p), GP(p + 1));
#pragma unroll
    for (int p = 0; p < 2; ++p) dcnt[p] = loads_of(dw, DP(p), DP(p + 1));
    // The layer table through the constant address space: scalar loads,
    // which neither count among nor wait for the weight loads in flight.
    typedef const __attribute__((address_space(4))) lily_moe_weights ConstWeights;
    ConstWeights* layers = (ConstWeights*)a.layers;
    // Part p of layer l's gate/up share into s_gu[l & 1].
    auto issue_gu = [&](int l, int p) {
        if (l >= L) return;
        ConstWeights& w = layers[l];
        const char* gate = static_cast<const char*>(uniform_ptr(w.gate));
        const char* up = static_cast<const char*>(uniform_ptr(w.up));
        const char* sh_gate = static_cast<const char*>(uniform_ptr(w.sh_gate));
        const char* sh_up = static_cast<const char*>(uniform_ptr(w.sh_up));
        char* buf = s_gu[l & 1];
        const int lo = GP(p), hi = GP(p + 1);
        for (int t = lo + (dw - lo % kStkIssuers + kStkIssuers) % kStkIssuers; t < hi;
             t += kStkIssuers) {
            const int s = t / (2 * per_mat), rem = t - s * 2 * per_mat;
            const int mt = rem / per_mat, kk = rem - mt * per_mat;
            const int u = vw + G * s;
            const int j = u / (F / 8), f0 = (u - j * (F / 8)) * 8;
            const bool sh = j == k;
            const int e = sh ? 0 : s_ids[l * k + j];
            const char* stack = mt == 0 ? (sh ? sh_gate : gate) : (sh ? sh_up : up);
            const char* seg = stack + ((size_t)e * nsf + f0 / kPackRows) * nkg * kPackBlock;
            char* ub = buf + s * unit_bytes;
            if (kk < nqh) {  // lane: row f0 + l8, group 4 kk + lc / 2, half lc % 2
                dma16_lane(seg + (size_t)(4 * kk + (lc >> 1)) * kPackBlock +
                               ((lc & 1) * kPackRows + f0 % kPackRows + l8) * 16,
                           (uint32_t)(size_t)(ub + (mt * nqh + kk) * 1024));
            } else {  // lane: group 32 q + lane / 2, scale (even) or bias (odd)
                const int q = kk - nqh, g = 32 * q + lane / 2;
                if (g < nkg)
                    dma16_lane(seg + (size_t)g * kPackBlock + kPackQ + (lane & 1) * 2 * kPackRows +
                                   (f0 % kPackRows) * 2,
                               (uint32_t)(size_t)(ub + (2 * nqh + mt * nsbh + q) * 1024));
            }
        }
    };
    // Part p of layer l's down share into s_d.
    auto issue_d = [&](int l, int p) {
        if (l >= L) return;
        ConstWeights& w = layers[l];
        const char* down = static_cast<const char*>(uniform_ptr(w.down));
        const char* sh_down = static_cast<const char*>(uniform_ptr(w.sh_down));
        const int lo = DP(p), hi = DP(p + 1);
        for (int t = lo + (dw - lo % kStkIssuers + kStkIssuers) % kStkIssuers; t < hi;
             t += kStkIssuers) {
            if (t < NRB) {  // round t: slot j, groups 4 gq + b_gl
                const int j = t / nq, gq = t - j * nq;
                const bool sh = j == k;
                const int e = sh ? 0 : s_ids[l * k + j];
                dma16_lane((sh ? sh_down : down) +
                               ((size_t)(e * nsH + r0 / kPackRows) * nkgF + 4 * gq + b_gl) *
                                   kPackBlock +
                               (b_half * kPackRows + r0 % kPackRows + b_row) * 16,
                           (uint32_t)(size_t)(s_d + t * 1024));
            } else {  // lane: entry x = (slot j, group g, scale or bias)
                const int x = (t - NRB) * kWave + lane;
                if (x < R * nkgF * 2) {
                    const int jg = x >> 1, j = jg / nkgF, g = jg - j * nkgF;
                    const bool sh = j == k;
                    const int e = sh ? 0 : s_ids[l * k + j];
                    dma16_lane((sh ? sh_down : down) +
                                   ((size_t)(e * nsH + r0 / kPackRows) * nkgF + g) * kPackBlock +
                                   kPackQ + (x & 1) * 2 * kPackRows + (r0 % kPackRows) * 2,
                               (uint32_t)(size_t)(s_d + t * 1024));
                }
            }
        }
    };
    // The DMA wavefronts' side of the layer loop, at its four barriers
    // (x ready, part sums of phase A, h staged, part sums of phase B). Issue
    // order per layer l: after phase A: gate/up part 0 of layer l + 2; after
    // h: part 1; after phase B: down part 0 of layer l + 1, gate/up part 2;
    // after x (of layer l + 1): down part 1, gate/up part 3.
    auto issue_first = [&]() {  // in the order the loop would have issued them
        for (int p = 0; p < 4; ++p) issue_gu(0, p);
        issue_gu(1, 0);
        issue_gu(1, 1);
        issue_d(0, 0);
        issue_gu(1, 2);
    };
    // Before x of layer l is released: layer l's gate/up share has landed
    // (what was issued after its last part may still be in flight).
    auto wait_gu = [&](int l) {
        wait_vmcnt_upto((l + 1 < L ? gcnt[0] + gcnt[1] + gcnt[2] : 0) + dcnt[0]);
    };
    // Before h of layer l is released: layer l's down share has landed.
    auto wait_d = [&](int l) {
        wait_vmcnt_upto((l + 1 < L ? gcnt[3] : 0) + (l + 2 < L ? gcnt[0] : 0));
    };

    // Routing of every layer first (its logits are inputs of the launch):
    // wavefront v takes layers v, v + 11, ...
    if (tid == 0) s_hflag = s_done_a = s_done_b = 0;
    for (int l = wave; l < L; l += kStkWaves) topk_one_token(a.logits, l, E, k, s_ids, s_w);
    lds_barrier();

    if (wv < kDecWaves) {
        // ---- compute wavefronts: the two phases, from LDS ----
        if (wg == 0)  // the routing out
            for (int i = tid; i < L * k; i += kDecWaves * kWave) {
                a.topk_ids[i] = s_ids[i];
                a.topk_w[i] = s_w[i];
            }
        for (int l = 0; l < L; ++l) {
            lds_barrier();  // x ready (lead); layer l's gate/up share landed
            {
                // Phase A: wavefront w takes quads i = w + 8 m of each unit,
                // like moe_decode_kernel.
                const char* gub = s_gu[l & 1];
                float pg[kStkMaxUnits], pu[kStkMaxUnits];
#pragma unroll
                for (int s = 0; s < kStkMaxUnits; ++s) pg[s] = pu[s] = 0.0f;
                for (int i = wv; i < nqh; i += kDecWaves) {
                    uint32_t xv[16];
                    const uint32_t* xp = s_buf + i * 128 + (lc >> 1) * 32 + (lc & 1) * 16;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        *reinterpret_cast<u32x4*>(xv + 4 * c) =
                            *reinterpret_cast<const u32x4*>(xp + 4 * c);
                    const int gsb = (2 * (4 * i + (lc >> 1))) * 16 + l8 * 2;
#pragma unroll
                    for (int s = 0; s < kStkMaxUnits; ++s)
                        if (s < n_u) {
                            const char* ub = gub + s * unit_bytes;
                            const Slice sg = lds_slice(ub + i * 1024 + lane * 16,
                                                       ub + 2 * nqh * 1024 + gsb);
                            const Slice su = lds_slice(ub + (nqh + i) * 1024 + lane * 16,
                                                       ub + (2 * nqh + nsbh) * 1024 + gsb);
                            pg[s] += dot_slice(sg, xv);
                            pu[s] += dot_slice(su, xv);
                        }
                }
#pragma unroll
                for (int s = 0; s < kStkMaxUnits; ++s)
                    if (s < n_u) {
                        pg[s] += __shfl_xor(pg[s], 8);
                        pg[s] += __shfl_xor(pg[s], 16);
                        pg[s] += __shfl_xor(pg[s], 32);
                        pu[s] += __shfl_xor(pu[s], 8);
                        pu[s] += __shfl_xor(pu[s], 16);
                        pu[s] += __shfl_xor(pu[s], 32);
                        if (lane < 8) {
                            s_pa[s][wv][lane] = pg[s];
                            s_pa[s][wv][8 + lane] = pu[s];
                        }
                    }
            }
            if (lane == 0) count_done(&s_done_a);  // part sums written, x read
            // h of the layer (the lead's stores, and every other workgroup's)
            // into LDS as permuted chunks: wavefront w, lane l takes chunks
            // l + 64 (w + 8 m), four words each. The lead raises the flag after
            // all eight wavefronts are done with phase A (x, which h replaces)
            // and its h stores are issued.
            wait_count(&s_hflag, l + 1);
            {
                const int nh = R * F / 2;
                uint64_t t[kStkHSlots * 4];
                gather_tagged<kStkHSlots, 4>(a.hx + (size_t)xc * nh, nh, (uint32_t)l + 1, t,
                                             4 * (kWave * wv + lane), 4 * kWave * kDecWaves, a.err);
#pragma unroll
                for (int m = 0; m < kStkHSlots; ++m) {
                    const int c = lane + kWave * (wv + kDecWaves * m);
                    if (4 * c < nh) {
                        const u32x4 hr = {(uint32_t)t[4 * m], (uint32_t)t[4 * m + 1],
                                          (uint32_t)t[4 * m + 2], (uint32_t)t[4 * m + 3]};
                        *reinterpret_cast<u32x4*>(s_buf + 4 * c) = permute_chunk(hr);
                    }
                }
            }
            if (wv == 0) STACK_TRACE(l, 6);
            lds_barrier();  // h staged; layer l's down share landed
            if (has_b) {
                // Phase B: rounds rho = w + 8 n of the workgroup's unit, like
                // moe_decode_kernel.
                float acc = 0.0f;
                for (int rho = wv; rho < NRB; rho += kDecWaves) {
                    const int j = rho / nq, gq = rho - j * nq;
                    const float wj = j == k ? 1.0f : s_w[l * k + j];
                    const int hoff = (j * F + (4 * gq + b_gl) * kGroup + b_half * 32) / 2;
                    const Slice sl =
                        lds_slice(s_d + rho * 1024 + lane * 16,
                                  s_d + NRB * 1024 + (2 * (j * nkgF + 4 * gq + b_gl)) * 16 + b_row * 2);
                    acc = fmaf(wj, dot_slice(sl, s_buf + hoff), acc);
                }
                acc += __shfl_xor(acc, 8);
                acc += __shfl_xor(acc, 16);
                acc += __shfl_xor(acc, 32);
                if (lane < kDecPiece) s_bred[wv][lane] = acc;
            }
            if (lane == 0) count_done(&s_done_b);  // part sums written, h and s_d read
            // out_l rows into the exchange (pairs from lanes 2p, 2p + 1) and
            // out; r_L of the rows after the last layer. A compute wavefront
            // makes these stores, so that the lead's next loads (the out
            // exchange) do not wait for them: a wavefront's loads and stores
            // complete in order.
            if (wv == 0 && has_b) {
                wait_count(&s_done_b, kDecWaves * (l + 1));
                STACK_TRACE(l, 7);
                float o = 0.0f;
                if (lane < kDecPiece)
#pragma unroll
                    for (int v = 0; v < kDecWaves; ++v) o += s_bred[v][lane];
                const uint32_t ob = float_to_bf16_bits(o);
                const uint32_t pair = ob | (__shfl_xor(ob, 1) << 16);
                if (lane < kDecPiece) {
                    const int n = r0 + lane;
                    a.outs[(size_t)l * H + n] = (uint16_t)ob;
                    if (l == L - 1) a.r[n] = s_r[n] + bf16_bits_to_float(ob);
                    if (lane % 2 == 0)
                        store_copies(make_rsrc(a.ox, kDecXcds * (H / 2) * 8), n / 2, H / 2,
                                     tagged(pair, (uint32_t)l + 1));
                }
            }
        }
    } else if (wv > kStkLeadWave) {
        // ---- DMA wavefronts ----
        // Nothing of the routing is in flight any more; said with the
        // builtin (not asm), so that the compiler knows it and adds no wait
        // of its own (which would wait for the weight loads too) below.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        issue_first();
        for (int l = 0; l < L; ++l) {
            wait_gu(l);
            lds_barrier();  // x ready
            issue_d(l, 1);
            issue_gu(l + 1, 3);
            wait_count(&s_done_a, kDecWaves * (l + 1));  // phase A done: the gate/up buffer is free
            issue_gu(l + 2, 0);
            wait_d(l);
            lds_barrier();  // h staged
            issue_gu(l + 2, 1);
            wait_count(&s_done_b, kDecWaves * (l + 1));  // phase B done: the down buffer is free
            issue_d(l + 1, 0);
            issue_gu(l + 2, 2);
        }
    } else {
        // ---- lead: r, the norm and the exchanges ----
        const int nh = R * F / 2, no = H / 2;
        const int nhx = kDecXcds * nh, nox = kDecXcds * no;
        for (int i = wg * kWave + lane; i < nhx + nox; i += G * kWave)  // this workgroup's share
            store_tagged(i < nhx ? a.hx + i : a.ox + (i - nhx), 0);      // of the tag clears
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // Device-wide barrier 0, counted in now and waited for before the
        // first exchange store.
        if (lane == 0) {
            const int g = wg % kBarGroups;
            const int prev = __hip_atomic_fetch_add(a.grp + g * kBarLine, 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            if ((prev + 1) % bar_group_size(G, g) == 0)
                __hip_atomic_fetch_add(a.bar, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // r_0 = x0. Lane l takes elements 4 l + 256 m + c (slot m, c).
#pragma unroll
        for (int m = 0; m < kStkRSlots; ++m) {
            const int n = 4 * lane + 256 * m;
            if (n < H) {
                const u32x2 v = *reinterpret_cast<const u32x2*>(a.x0 + n);
                const f32x4 f = {bf16_bits_to_float(v[0] & 0xFFFFu), bf16_bits_to_float(v[0] >> 16),
                                 bf16_bits_to_float(v[1] & 0xFFFFu), bf16_bits_to_float(v[1] >> 16)};
                *reinterpret_cast<f32x4*>(s_r + n) = f;
            }
        }
        for (int l = 0; l < L; ++l) {
            const uint32_t tag = (uint32_t)l + 1;
            STACK_TRACE(l, 0);
            if (l > 0) {
                // out_{l-1} (tag l), elements 4 l + 256 m .. + 3 as two pairs;
                // r_l = r_{l-1} + out_{l-1}.
                uint64_t t[kStkRSlots * 2];
                gather_tagged<kStkRSlots, 2>(a.ox + (size_t)xc * no, no, (uint32_t)l, t, 2 * lane,
                                             128, a.err);
#pragma unroll
                for (int m = 0; m < kStkRSlots; ++m)
                    if (4 * lane + 256 * m < H) {
                        const uint32_t p0 = (uint32_t)t[2 * m], p1 = (uint32_t)t[2 * m + 1];
                        f32x4 f = *reinterpret_cast<const f32x4*>(s_r + 4 * lane + 256 * m);
                        f[0] += bf16_bits_to_float(p0 & 0xFFFFu);
                        f[1] += bf16_bits_to_float(p0 >> 16);
                        f[2] += bf16_bits_to_float(p1 & 0xFFFFu);
                        f[3] += bf16_bits_to_float(p1 >> 16);
                        *reinterpret_cast<f32x4*>(s_r + 4 * lane + 256 * m) = f;
                    }
            }
            STACK_TRACE(l, 1);
            float rv[kStkRSlots][4];
#pragma unroll
            for (int m = 0; m < kStkRSlots; ++m)
                if (4 * lane + 256 * m < H) {
                    const f32x4 f = *reinterpret_cast<const f32x4*>(s_r + 4 * lane + 256 * m);
                    for (int c = 0; c < 4; ++c) rv[m][c] = f[c];
                }
            // x_l = bf16(r_l / sqrt(mean(r_l^2) + eps)) in residual_norm_kernel's
            // order: its thread t = l + 64 v sums elements 4 t + 1024 i + c
            // (slots m = v + 4 i of this lane), then each of its wavefronts v
            // reduces over lanes, and the four parts are added in order.
            float part[kNormThreads / kWave];
#pragma unroll
            for (int v = 0; v < kNormThreads / kWave; ++v) {
                float ss = 0.0f;
#pragma unroll
                for (int i = 0; i < kStkRSlots / (kNormThreads / kWave); ++i) {
                    const int m = v + (kNormThreads / kWave) * i;
                    if (4 * lane + 256 * m < H)
                        ss += rv[m][0] * rv[m][0] + rv[m][1] * rv[m][1] + rv[m][2] * rv[m][2] +
                              rv[m][3] * rv[m][3];
                }
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
                part[v] = ss;
            }
            float tot = 0.0f;
#pragma unroll
            for (int v = 0; v < kNormThreads / kWave; ++v) tot += part[v];
            const float inv = 1.0f / sqrtf(tot / (float)H + a.eps);
            // x replaces h of the layer before in LDS: phase B must be done.
            wait_count(&s_done_b, kDecWaves * l);
            // Permuted chunks: word j of chunk c holds elements (8c + j, 8c + j
            // + 4). Lanes 2p and 2p + 1 hold the two halves of chunk p + 32 m:
            // the even lane writes words 0, 1, the odd lane words 2, 3.
#pragma unroll
            for (int m = 0; m < kStkRSlots; ++m) {
                const uint32_t p0 = pack_bf16x2(rv[m][0] * inv, rv[m][1] * inv);
                const uint32_t p1 = pack_bf16x2(rv[m][2] * inv, rv[m][3] * inv);
                const uint32_t q0 = __shfl_xor(p0, 1), q1 = __shfl_xor(p1, 1);
                if (4 * lane + 256 * m < H) {
                    const bool odd = lane & 1;
                    const uint32_t lo = odd ? q1 : p0, hi = odd ? p1 : q0;  // (low, high) sources
                    u32x2 wd;
                    wd[0] = (lo & 0xFFFFu) | (hi << 16);
                    wd[1] = (lo >> 16) | (hi & 0xFFFF0000u);
                    *reinterpret_cast<u32x2*>(s_buf + 4 * (lane / 2 + 32 * m) + 2 * odd) = wd;
                }
            }
            lds_barrier();  // x ready
            STACK_TRACE(l, 2);
            wait_count(&s_done_a, kDecWaves * (l + 1));  // part sums of phase A ready
            STACK_TRACE(l, 3);
            if (l == 0) {   // every workgroup's tag clears have landed
                if (lane == 0) {
                    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                    while (__hip_atomic_load(a.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                           bar_groups(G)) {
                        __builtin_amdgcn_s_sleep(2);
                        if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > kSpinTicks) {
                            __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
            // h of this workgroup's units into the exchange: lane = (unit
            // ui = lane / 4, features 2q, 2q + 1 with q = lane % 4).
            if (lane < 4 * n_u) {
                const int ui = lane / 4, q = lane % 4;
                const int u = vw + G * ui;
                const int j = u / (F / 8), f0 = (u - j * (F / 8)) * 8;
                float hv[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float g = 0.0f, up = 0.0f;
#pragma unroll
                    for (int w = 0; w < kDecWaves; ++w) {
                        g += s_pa[ui][w][2 * q + c];
                        up += s_pa[ui][w][8 + 2 * q + c];
                    }
                    hv[c] = silu(g) * up;
                }
                store_copies(make_rsrc(a.hx, nhx * 8), (j * F + f0) / 2 + q, nh,
                             tagged(pack_bf16x2(hv[0], hv[1]), tag));
            }
            // The compute wavefronts poll h once these stores are issued: polls
            // issued before them would hold them up in the compute unit's
            // memory queue.
            asm volatile("" ::: "memory");
            if (lane == 0) __hip_atomic_store(&s_hflag, (int)tag, __ATOMIC_RELEASE,
                                              __HIP_MEMORY_SCOPE_WORKGROUP);
            STACK_TRACE(l, 4);
            lds_barrier();  // h staged (compute wavefronts)
            STACK_TRACE(l, 5);
        }
        barrier_exit(a.bar, a.grp, kStkLead);
    }
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
// the exchanges, kDecXcds copies of h as (k + 1) F / 2 tagged words, then
// kDecXcds copies of out as H / 2 tagged words.
static size_t stack_hx_bytes(const lily_moe_dims& d) {
    return ((size_t)kDecXcds * ((d.topk + 1) * d.F / 2) * sizeof(uint64_t) + 255) & ~(size_t)255;
}
size_t decode_workspace_bytes(const lily_moe_dims& d) {
    if (d.T > kDecodeMaxT) return 0;
    const size_t one = (size_t)d.T * (d.topk + 1) * d.F * sizeof(uint16_t);
    if (d.T != 1) return one;
    const size_t stack = stack_hx_bytes(d) + (size_t)kDecXcds * (d.H / 2) * sizeof(uint64_t);
    return one > stack ? one : stack;
}

constexpr int kDecMaxH = 4096;  // x of kDecodeMaxT tokens fills the LDS staging area
static_assert(kDecodeMaxT * kDecMaxH / 2 <= kDecLdsWords, "x staging");
static_assert(kDecodeMaxT * kDecMaxH / 2 <= kDecXChunks * 4 * kDecThreads, "x chunks");

int decode_supported(const lily_moe_dims& d) {
    if (d.T > kDecodeMaxT)
        return set_error(LILY_ERR_UNSUPPORTED, "T = %d; lily_moe_decode serves T <= %d", d.T,
                         kDecodeMaxT);
    if (d.H % 512 || d.H > kDecMaxH)
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
                              r.sched + kQueueInts, r.sched + kGiveUpFlag, stream);
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
                              ctr + kQueueInts, status ? status : ctr + kGiveUpFlag, stream);
}

int decode_stack_supported(const lily_moe_dims& d, int n_layers) {
    if (n_layers < 1) return set_error(LILY_ERR_INVALID_ARG, "n_layers = %d must be >= 1", n_layers);
    if ((long)n_layers * d.topk > kStackMaxIds)
        return set_error(LILY_ERR_UNSUPPORTED, "n_layers * topk = %ld exceeds %d",
                         (long)n_layers * d.topk, kStackMaxIds);
    if (d.T != 1)
        return set_error(LILY_ERR_UNSUPPORTED, "T = %d; lily_moe_decode_stack serves T = 1", d.T);
    if (d.H % (2 * kNormThreads) || d.H > kStkMaxH)
        return set_error(LILY_ERR_UNSUPPORTED, "H = %d must be a multiple of 512, at most %d",
                         d.H, kStkMaxH);
    if (d.F % (4 * kGroup) || (long)(d.topk + 1) * d.F > kStkMaxRF)
        return set_error(LILY_ERR_UNSUPPORTED,
                         "F = %d must be a multiple of 256 with (topk + 1) * F <= %d", d.F,
                         kStkMaxRF);
    const int g = decode_grid();
    if (d.H / kDecPiece > g)
        return set_error(LILY_ERR_UNSUPPORTED, "H / 8 = %d down units exceed one per compute unit",
                         d.H / kDecPiece);
    const long units = (long)(d.topk + 1) * (d.F / 8);
    const long per_wg = (units + g - 1) / g;
    const long unit_bytes = 2L * (d.H / 256 + (d.H / kGroup + 31) / 32) * 1024;
    if (per_wg > kStkMaxUnits || per_wg * unit_bytes > kStkGuBytes)
        return set_error(LILY_ERR_UNSUPPORTED,
                         "(topk + 1) * F / 8 = %ld gate/up units: %ld per compute unit exceed the "
                         "LDS buffer", units, per_wg);
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
    a.hx = static_cast<uint64_t*>(workspace);
    a.ox = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + stack_hx_bytes(d));
    a.eps = eps;
    a.bar = sched + kDecodeBarrier;
    a.grp = sched + kQueueInts;
    a.err = sched + kGiveUpFlag;
    // One workgroup per compute unit (its LDS fills the compute unit): all
    // are resident at once, which the device-wide barrier and the exchanges
    // rely on.
    hipLaunchKernelGGL(moe_decode_stack_kernel, dim3((unsigned)decode_grid()), dim3(kStkThreads),
                       0, stream, a);
    return check_launch("decode_stack");
}

// Copies the phase trace of the last lily_moe_decode_stack launch (tracing
// build only): [min(max_wgs, 256)][64][8] ticks.
int trace_decode_stack(unsigned long long* dst, int max_wgs, hipStream_t stream) {
#ifdef LILY_TRACE_ITEMS
    if (!dst || max_wgs < 1)
        return set_error(LILY_ERR_INVALID_ARG, "trace_decode_stack: dst non-NULL, max_wgs >= 1");
    const int n = max_wgs < kTraceStackWgs ? max_wgs : kTraceStackWgs;
    if (hipStreamSynchronize(stream) != hipSuccess ||
        hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_stack_trace), sizeof(g_stack_trace[0]) * n, 0,
                            hipMemcpyDeviceToHost) != hipSuccess)
        return set_error(LILY_ERR_HIP, "trace_decode_stack: copy failed");
    return n;
#else
    (void)dst;
    (void)max_wgs;
    (void)stream;
    return set_error(LILY_ERR_UNSUPPORTED,
                     "trace_decode_stack: this library was built without the phase trace "
                     "(liblily_moe_trace.so has it)");
#endif
}

}  // namespace lily
