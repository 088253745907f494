/*
 * lily_moe.h: C ABI of the int4 grouped-GEMM MoE layer for MI355X (gfx950).
 *
 * The layer is the prefill Mixture-of-Experts block described in the Lily
 * articles (news.ainew.jp, "Perplexity, Apple Silicon向け推論エンジン「Lily」を
 * オープンソース化"):
 *   - the router picks k of E experts per token and a shared expert also
 *     processes every token (section on the three workload shapes);
 *   - the weights are groupwise-affine 4-bit: 64 weights share one bf16
 *     scale and one bf16 bias; they are rebuilt as bf16 tile by tile inside
 *     the grouped GEMM, kept on chip, and the products accumulate in FP32
 *     (section "Prefill");
 *   - the routing histogram, prefix scan, scatter and block map stay on the
 *     GPU, in one stream, with no host synchronisation inside the layer
 *     (section "Prefill").
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless stated. The caller allocates and
 *     owns every buffer and keeps it alive until the stream work completes.
 *     The library allocates no device memory and keeps no per-call state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls enqueue work and return; none synchronises the host.
 *   - Return value 0 (LILY_OK) or a negative LILY_ERR_* code. Argument checks
 *     are done on the host before anything is enqueued; on an error nothing is
 *     enqueued and lily_last_error() describes it. Faults inside a kernel
 *     surface at the caller's next synchronisation. No C++ exception crosses
 *     this interface.
 *   - The calls are re-entrant for distinct buffers and streams.
 *   - Device pointers must be 16-byte aligned.
 *
 * Readings of points the pages leave open (the same readings the CPU oracle
 * takes): groups of 64 run along K, the input dimension of an [N, K]
 * (out x in) matrix, and byte i of a row packs element 2i in its low nibble;
 * w = scale*q + bias rounded to bf16; ties in top-k go to the lower expert
 * index (-0.0 ties +0.0); routing weights are a softmax over the k selected
 * logits; each expert is a SwiGLU FFN h = bf16(silu(x Wg^T) * (x Wu^T)),
 * y = h Wd^T in fp32; the shared expert has weight 1; the output is
 * bf16(y_shared + sum_j w_j y_j) summed in slot order.
 */
#ifndef LILY_MOE_H
#define LILY_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LILY_OK 0
#define LILY_ERR_INVALID_ARG (-1) /* null pointer, bad size, misaligned pointer */
#define LILY_ERR_UNSUPPORTED (-2) /* a shape or tile the kernels do not cover */
#define LILY_ERR_WORKSPACE (-3)   /* workspace smaller than required */
#define LILY_ERR_HIP (-4)         /* a HIP launch error; text from hipGetErrorString */

/* Layer sizes. T tokens, hidden size H, expert FFN size F, E routed experts,
   topk experts per token, group = 64 (the only supported group), tile_m =
   rows per block of the block map (16, 32, 64 or 128 for lily_moe_forward;
   any value >= 1 for lily_moe_route). H and F must be multiples of 64;
   1 <= topk <= E <= 512; T >= 1. */
typedef struct {
    int32_t T, H, F, E, topk, group, tile_m;
} lily_moe_dims;

/* One groupwise-affine int4 matrix per expert, stacked over n experts
   (n = E for routed, 1 for the shared expert), for a matrix of N rows
   (outputs) and K columns (inputs), in the plain layout:
     q:     uint8 [n, N, K/2]; byte i of a row = element 2i (low nibble)
            and element 2i+1 (high nibble), values 0..15;
     scale: bf16 bits [n, N, K/64];
     bias:  bf16 bits [n, N, K/64];
   weight (e, row, col) = bf16(scale[e,row,col/64] * q + bias[e,row,col/64]).
   lily_w4_pack converts this layout into the packed one the GEMMs read. */
typedef struct {
    const uint8_t* q;
    const uint16_t* scale;
    const uint16_t* bias;
} lily_w4;

/* Packed layout of the same matrix stack (N a multiple of 128, K a
   multiple of 64): one 4608-byte block per (expert e, 128-row slab s, group
   g), block index (e * N/128 + s) * K/64 + g; inside a block, for slab row
   r = 0..127 (matrix row 128 s + r) and half h = 0, 1:
     bytes 16 (128 h + r) .. +15:  q bytes 32 g + 16 h .. +15 of the row
                                   (elements 64 g + 32 h .. +31);
     bytes 4096 + 2 r:             scale of (row, group g);
     bytes 4352 + 2 r:             bias of (row, group g).
   Same size as the plain layout: n * N * K * 9 / 16 bytes. A workgroup's
   weights for one k-step are two contiguous 4 KB runs plus 512-byte scale
   and bias runs, so every load is a full, coalesced line. */

/* gate, up: N = F, K = H.  down: N = H, K = F. Each pointer is a packed
   matrix stack (16-byte aligned) written by lily_w4_pack. */
typedef struct {
    const void* gate;
    const void* up;
    const void* down;     /* routed experts, n = E */
    const void* sh_gate;
    const void* sh_up;
    const void* sh_down;  /* shared expert, n = 1 */
} lily_moe_weights;

/* Outputs of lily_moe_route (inputs of lily_moe_forward). P = T * topk.
   topk_ids  int32 [T, topk]  chosen experts, descending logit;
   topk_w    fp32  [T, topk]  softmax of the chosen logits;
   counts    int32 [E]        rows per expert (histogram);
   offsets   int32 [E + 1]    exclusive scan of counts, offsets[E] = P;
   sorted_pairs int32 [P]     row r of the expert-ordered layout holds pair
                              p = t * topk + j; rows of one expert are in
                              ascending p (stable);
   pair_rows int32 [P]        inverse: pair_rows[sorted_pairs[r]] = r;
   block_expert, block_row0 int32 [lily_moe_max_blocks(dims)]
                              block b covers rows block_row0[b] ..
                              min(block_row0[b] + tile_m, offsets[e+1]) - 1 of
                              expert e = block_expert[b]; experts ascending;
                              entries at and past num_blocks are unspecified;
   num_blocks int32 [1]       number of valid blocks (stays on the device);
   block_order int32 [lily_moe_max_blocks(dims)]
                              schedule of the grouped GEMMs (not part of the
                              method's result): the full blocks (tile_m
                              rows) in block order, then each expert's last,
                              partial block by descending size class
                              ceil(4 rows / tile_m), ties in expert order;
   block_info int32 [lily_moe_max_blocks(dims)][4]
                              the same schedule resolved: entry i holds
                              (expert, first row, rows, block) of block
                              block_order[i], so that a GEMM workgroup
                              learns a block's extent with one load;
   sched int32 [LILY_SCHED_INTS]
                              work-queue and split-K tile counters of the
                              grouped GEMMs (the first 1632 ints), then the
                              route's per-span expert histograms (64 rows of
                              512 counts and an arrival counter). Zero the
                              whole array once after allocating;
                              lily_moe_route clears the counters and leaves
                              the histograms zero, and every GEMM launch
                              leaves its counters zero when it completes.
                              sched[30] is the give-up flag of the bounded
                              device-wide waits (lily_moe_ffn's one launch,
                              the decode kernels): set to 1 when one gave up
                              (the outputs of that call are not valid), and
                              sticky: no call clears it, the caller does.
                              Launches that share a routing buffer must be
                              ordered on one stream. */
#define LILY_SCHED_INTS (1632 + 64 * 512 + 1)
typedef struct {
    int32_t* topk_ids;
    float* topk_w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted_pairs;
    int32_t* pair_rows;
    int32_t* block_expert;
    int32_t* block_row0;
    int32_t* num_blocks;
    int32_t* block_order;
    int32_t* sched;
    int32_t* block_info;
} lily_moe_routing;

/* Host, pure. Capacity of the block map: ceil(P / tile_m) + min(E, P).
   Returns a negative LILY_ERR_* code for invalid dims. */
int32_t lily_moe_max_blocks(const lily_moe_dims* dims);

/* Host, pure. Bytes of device workspace lily_moe_forward needs for dims
   (0 for invalid dims). Layout, each part starting on a 256-byte boundary:
     h     bf16 [P + T, F]: the SwiGLU intermediate (routed rows in expert
           order, then the shared expert's rows by token);
     y     fp32 [P + T, H]: the per-row expert outputs, same row order;
     part  fp32 partial sums of the GEMMs that split K, present only for
           small block maps (few tokens), where a tile's K is spread over
           several workgroups. */
size_t lily_moe_workspace_bytes(const lily_moe_dims* dims);

/* Host, pure. Bytes of the packed layout of an n-expert stack of [N, K]
   matrices (0 if N is not a multiple of 128, K not a multiple of 64, group
   not 64, or a size is < 1). */
size_t lily_w4_packed_bytes(int32_t n, int32_t N, int32_t K, int32_t group);

/* Rearranges a plain-layout matrix stack into the packed layout (a pure
   permutation of bytes: no value changes). packed: lily_w4_packed_bytes
   bytes of device memory, not overlapping the inputs. Errors:
   LILY_ERR_INVALID_ARG (null or misaligned pointer, bad sizes),
   LILY_ERR_HIP. */
int lily_w4_pack(const lily_w4* w, int32_t n, int32_t N, int32_t K, int32_t group, void* packed,
                 void* stream);

/* Router projection, the step before lily_moe_route when a layer starts
   from its activations: logits[t, e] = sum_h x[t, h] * w_router[e, h]
   (the router scores every expert for each token: Lily articles, section on
   the three workload shapes). x bf16 [T, H], w_router bf16 [E, H] (row e
   scores expert e), logits fp32 [T, E], all row-major device memory. The
   bf16 products are exact in fp32 and summed in fp32 (in another order than
   a sequential loop). Only T, H, E of dims are used beyond the common
   checks; H must be a multiple of 256. Errors: LILY_ERR_INVALID_ARG (null
   or misaligned pointer, bad dims), LILY_ERR_UNSUPPORTED (H), LILY_ERR_HIP. */
int lily_moe_router(const lily_moe_dims* dims, const uint16_t* w_router, const uint16_t* x,
                    float* logits, void* stream);

/* Routing of one MoE layer: top-k and softmax per token, histogram,
   exclusive scan, stable scatter and block map, all enqueued on `stream`
   with no host synchronisation. The router keeps k of E experts per token
   (Lily articles, section on the three workload shapes: 256 experts, top 8);
   the histogram, prefix scan, scatter and block map run on the GPU in one
   command stream without a CPU round trip (section "Prefill").
   logits: fp32 [T, E] router scores. Deterministic and bit-exact for
   finite logits; non-finite logits give unspecified (but in-bounds) output.
   Errors: LILY_ERR_INVALID_ARG (null pointer, bad dims, misalignment),
   LILY_ERR_UNSUPPORTED (E > 512 or topk > 64), LILY_ERR_HIP. */
int lily_moe_route(const lily_moe_dims* dims, const float* logits,
                   const lily_moe_routing* routing, void* stream);

/* Ablation twin of lily_moe_route with CPU-synchronised routing (the Lily
   articles, section "Prefill", credit GPU-resident routing with a large
   prefill speed-up over this): the top-k and softmax run on the GPU as in
   lily_moe_route; the ids are then copied to the host, the stream is
   synchronised, the host computes the histogram, scan, stable scatter,
   block map and GEMM schedule with the same definitions, uploads them and
   zeroes sched, and the stream is synchronised again before returning.
   The routing written is bit-identical to lily_moe_route's. Blocks the
   calling thread; allocates host memory only. Same arguments and errors as
   lily_moe_route. */
int lily_moe_route_host(const lily_moe_dims* dims, const float* logits,
                        const lily_moe_routing* routing, void* stream);

/* Expert computation of one MoE layer from a routing produced by
   lily_moe_route with the same dims: grouped gate/up GEMM with the int4 ->
   bf16 dequantisation fused into the tile loads, SwiGLU, grouped down GEMM,
   the shared expert, and the weighted gather-combine. The weights are
   groupwise-affine 4-bit (64 share a bf16 scale and bias) and are rebuilt as
   bf16 inside the grouped GEMM, on chip, with FP32 accumulation (Lily
   articles, section "Prefill"); a shared expert processes every token besides
   the routed ones (section on the three workload shapes).
   x: bf16 bits [T, H]; out: bf16 bits [T, H]; workspace: at least
   lily_moe_workspace_bytes(dims) bytes of device memory (contents on entry
   are ignored). The routing is trusted (ids in range, block map as produced
   by lily_moe_route). Run-to-run deterministic: no floating-point atomics.
   Errors: LILY_ERR_INVALID_ARG, LILY_ERR_UNSUPPORTED (tile_m not 16/32/64/128,
   H not a multiple of 256, F not a multiple of 128, or x [T, H], h
   [T * (topk + 1), F] or one [F, H] matrix as bf16 reaching 4 GiB: the
   kernels address rows with 32-bit byte offsets), LILY_ERR_WORKSPACE,
   LILY_ERR_HIP. */
int lily_moe_forward(const lily_moe_dims* dims, const lily_moe_weights* weights,
                     const uint16_t* x, const lily_moe_routing* routing, uint16_t* out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The stages of lily_moe_forward, callable one at a time (for example to
   time each stage), on the same workspace (layout under
   lily_moe_workspace_bytes). lily_moe_forward runs lily_moe_ffn, then
   lily_moe_combine.
   P = T * topk; rows 0..P-1 are the routed (token, expert) pairs in expert
   order (row r = pair sorted_pairs[r]); rows P..P+T-1 are the shared
   expert's rows for tokens 0..T-1.
   lily_moe_gate_up: h[r] = bf16(silu(x Wg^T) * (x Wu^T)) with the weights
     dequantised tile by tile on chip;
   lily_moe_down: y[r] = h[r] Wd^T in fp32;
   lily_moe_ffn: both of them, h then y, bit for bit as the two calls in
     turn. When neither GEMM splits K (large T; the split depends on the
     sizes only) and the schedule has at most 1024 blocks, it is one launch
     in which a workgroup moves from gate/up tiles to down tiles as the
     gate/up work runs out; a down tile waits for its block's gate/up tiles
     (a bounded wait that can only give up on a faulty device: then it sets
     routing->sched[30] and the output is not valid). Otherwise it is the
     two launches;
   lily_moe_combine: out[t] = bf16(y[P + t] + sum_j topk_w[t, j] *
     y[pair_rows[t * topk + j]]), fp32 sum in slot order; out: bf16 [T, H].
   Errors as for lily_moe_forward. */
int lily_moe_gate_up(const lily_moe_dims* dims, const lily_moe_weights* weights,
                     const uint16_t* x, const lily_moe_routing* routing, void* workspace,
                     size_t workspace_bytes, void* stream);
int lily_moe_down(const lily_moe_dims* dims, const lily_moe_weights* weights,
                  const lily_moe_routing* routing, void* workspace, size_t workspace_bytes,
                  void* stream);
int lily_moe_ffn(const lily_moe_dims* dims, const lily_moe_weights* weights, const uint16_t* x,
                 const lily_moe_routing* routing, void* workspace, size_t workspace_bytes,
                 void* stream);
int lily_moe_combine(const lily_moe_dims* dims, const lily_moe_routing* routing,
                     void* workspace, size_t workspace_bytes, uint16_t* out, void* stream);

/* Ablation twin of the fused dequantisation (the Lily articles, section
   "Prefill", rebuild the 4-bit weights as bf16 inside the grouped GEMM and
   credit that with a large prefill speed-up over expanding them first):
   writes the bf16 weights w = bf16(scale * q + bias) of every expert with
   routing->counts[e] > 0 and of the shared expert to device memory, for
   lily_moe_forward_bf16. packed: the layer's packed stacks, as for
   lily_moe_forward; bf16: six caller-owned bf16 [n][N][K] row-major stacks
   with the same roles (gate and up [E][F][H], down [E][H][F], shared ones
   n = 1); entries of experts with no rows are left untouched. The values
   are the ones the fused GEMMs multiply with, bit for bit. Errors as
   lily_moe_forward. */
int lily_moe_dequant(const lily_moe_dims* dims, const lily_moe_weights* packed,
                     const lily_moe_routing* routing, const lily_moe_weights* bf16,
                     void* stream);

/* The forward of lily_moe_forward reading the bf16 stacks that
   lily_moe_dequant wrote instead of the packed int4 ones: the same grouped
   GEMM with its weight tiles loaded as bf16 (nothing dequantised), the same
   SwiGLU and combine. The output is bit-identical to lily_moe_forward's for
   the same routing. tile_m must be 32 or 64. Errors as lily_moe_forward,
   plus LILY_ERR_UNSUPPORTED for tile_m 128. */
int lily_moe_forward_bf16(const lily_moe_dims* dims, const lily_moe_weights* bf16,
                          const uint16_t* x, const lily_moe_routing* routing, uint16_t* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Route and forward of one MoE layer for a few tokens (T <= 4, decode) in
   one launch: the routing of lily_moe_route (same ids and weights) and the
   output of lily_moe_forward up to the order of the fp32 sums (the same
   bf16 weights bf16(scale * q + bias), bf16 h and fp32 accumulation). Every weight of the k routed experts and of the
   shared expert is read once, spread over one workgroup per compute unit
   as matrix-vector products: gate/up by one wavefront per (row, 8 features)
   over all of K, which forms that part of h itself; one device-wide
   barrier; then down and the weighted combine. The launch relies on all of
   its workgroups (at most one per compute unit) being resident together,
   as they are when no other work holds the device's compute units.
   logits fp32 [T, E], x bf16 [T, H]; out bf16 [T, H]. Of the routing only
   topk_ids, topk_w (written) and sched are used: sched[28..29] and
   sched[32 + 32 g], sched[33 + 32 g] for g < 8 (the barrier's counters) are
   zero on entry and left zero; sched[30] is set to 1 if the barrier wait
   gave up after half a second, which makes out invalid.
   Needs H a multiple of 512 (at most 4096) and F a multiple of 256 with
   (topk + 1) * F <= 16384.
   workspace: lily_moe_workspace_bytes(dims) bytes.
   Errors: LILY_ERR_INVALID_ARG, LILY_ERR_UNSUPPORTED (T > 4, sizes),
   LILY_ERR_WORKSPACE, LILY_ERR_HIP. */
int lily_moe_decode(const lily_moe_dims* dims, const lily_moe_weights* weights,
                    const float* logits, const uint16_t* x, const lily_moe_routing* routing,
                    uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* lily_moe_decode for callers that cannot allocate device memory (code
   under HIP graph capture, serving loops and harnesses that forbid hipMalloc):
   the same routing and output (the same kernel), but the scratch that
   lily_moe_decode takes from its workspace and routing.sched (the h rows and
   the device-wide barrier's counters) lives in a static device array of the
   library, LILY_DECODE_NOALLOC_SCRATCH_BYTES per GPU, which each GPU holds
   from its first call until the process ends. The call allocates nothing and
   clears the counters itself (a small kernel, no memset). Every call on a GPU
   shares that GPU's array: calls that overlap on one GPU (several streams or
   threads) race and give wrong results; order them on one stream.
   logits fp32 [T, E], x bf16 [T, H]; topk_ids int32 [T, topk] and topk_w fp32
   [T, topk] receive the routing; out bf16 [T, H]; status: NULL or one int32
   of device memory, set to 0 and then to 1 if the barrier wait gave up after
   half a second (the outputs are then invalid). Sizes as lily_moe_decode;
   T * (topk + 1) * F bf16 must fit the scratch's 131072-byte h area (which
   the size rules of lily_moe_decode already ensure). Errors:
   LILY_ERR_INVALID_ARG, LILY_ERR_UNSUPPORTED, LILY_ERR_HIP. */
#define LILY_DECODE_NOALLOC_SCRATCH_BYTES (4096 + 131072)
int lily_moe_decode_noalloc(const lily_moe_dims* dims, const lily_moe_weights* weights,
                            const float* logits, const uint16_t* x, int32_t* topk_ids,
                            float* topk_w, uint16_t* out, int32_t* status, void* stream);

/* Batch-1 decode through a stack of MoE layers in one launch (T = 1): for
   l = 0 .. n_layers - 1, x_l = bf16(r_l / sqrt(mean(r_l^2) + eps)) with
   r_0 = x0, out_l = the MoE layer l of lily_moe_decode on x_l, and
   r_{l+1} = r_l + out_l (fp32): the chain of lily_moe_decode and
   lily_residual_norm launches (bit for bit), in one launch whose workgroups
   (one per compute unit, all resident) exchange h and out through the
   workspace twice per layer, while each layer's weights stream into LDS a
   layer or more ahead (the pages run a decode step as one concurrent pass:
   Lily articles, section "Decode").
   layers: device array of n_layers lily_moe_weights (packed stacks, as for
   lily_moe_decode); logits fp32 [n_layers][E]; x0 bf16 [H]; r fp32 [H]
   (ignored on entry, r_{n_layers} on exit); outs bf16 [n_layers][H] (each
   layer's output); topk_ids int32 and topk_w fp32 [n_layers][topk] (each
   layer's routing); sched: as in lily_moe_routing (its barrier counters are
   zero on entry and left zero; sched[30] is set to 1 if a wait, for the
   start barrier or an exchange, gave up after half a second, which makes the
   outputs invalid). workspace: lily_moe_workspace_bytes(dims) bytes; its
   exchange area is cleared by the launch itself.
   Needs T = 1, n_layers * topk <= 1024, H a multiple of 512 (at most 2048
   and at most 8 per compute unit), F a multiple of 256 with
   (topk + 1) * F <= 4608, and the gate/up units ((topk + 1) * F / 8 sets of
   8 features, dealt over the compute units) at most 4 per compute unit and
   within a 54 KB LDS buffer (3 at H = 2048).
   Errors: LILY_ERR_INVALID_ARG, LILY_ERR_UNSUPPORTED, LILY_ERR_WORKSPACE,
   LILY_ERR_HIP. */
int lily_moe_decode_stack(const lily_moe_dims* dims, int32_t n_layers,
                          const lily_moe_weights* layers, const float* logits, const uint16_t* x0,
                          float* r, uint16_t* outs, int32_t* topk_ids, float* topk_w,
                          int32_t* sched, float eps, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Residual stream between stacked MoE layers (the pages describe a stack of
   layers but not this glue; the reading is a pre-norm residual with a
   unit-gain RMSNorm): r += out (fp32), then
   x_next = bf16(r / sqrt(mean(r^2) + eps)) per token.
   r: fp32 [T, H] in/out; out: bf16 bits [T, H], or NULL to only normalise;
   x_next: bf16 bits [T, H]. Errors: LILY_ERR_INVALID_ARG, LILY_ERR_HIP. */
int lily_residual_norm(int32_t T, int32_t H, float* r, const uint16_t* out,
                       uint16_t* x_next, float eps, void* stream);

/* Text of the last error on the calling thread ("" if none). */
const char* lily_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LILY_MOE_H */
