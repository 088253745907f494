// C ABI of the MoE layer: argument checks on the host, then launches.
#include <stdarg.h>
#include <stdio.h>

#include "common.hpp"
#include "lily_trace.h"

namespace lily {

static thread_local char g_last_error[512] = "";

int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

int check_launch(const char* what) {
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return set_error(LILY_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
    return LILY_OK;
}

int launch_route(const lily_moe_dims& d, const float* logits, const lily_moe_routing& r,
                 hipStream_t stream);
int launch_route_host(const lily_moe_dims& d, const float* logits, const lily_moe_routing& r,
                      hipStream_t stream);
int launch_gate_up(const lily_moe_dims& d, const lily_moe_weights& w, const uint16_t* x,
                   const lily_moe_routing& r, int max_blocks, const ForwardWorkspace& ws,
                   hipStream_t stream, bool w4);
int launch_down(const lily_moe_dims& d, const lily_moe_weights& w, const lily_moe_routing& r,
                int max_blocks, const ForwardWorkspace& ws, hipStream_t stream, bool w4);
int launch_ffn(const lily_moe_dims& d, const lily_moe_weights& w, const uint16_t* x,
               const lily_moe_routing& r, int max_blocks, const ForwardWorkspace& ws,
               hipStream_t stream);
int launch_dequant(const void* packed, int n, int N, int K, const int32_t* counts, void* out,
                   hipStream_t stream);
int decode_stack_supported(const lily_moe_dims& d, int n_layers);
int launch_decode_stack(const lily_moe_dims& d, int n_layers, const lily_moe_weights* layers,
                        const float* logits, const uint16_t* x0, float* r, uint16_t* outs,
                        int32_t* topk_ids, float* topk_w, int32_t* sched, float eps,
                        void* workspace, hipStream_t stream);
int launch_combine(const lily_moe_dims& d, const ForwardWorkspace& ws, const lily_moe_routing& r,
                   uint16_t* out, hipStream_t stream);
size_t forward_workspace_bytes(const lily_moe_dims& d, int max_blocks);
ForwardWorkspace forward_workspace_split(const lily_moe_dims& d, void* ws);
size_t packed_w4_bytes(int n, int N, int K);
int launch_pack(const lily_w4& w, int n, int N, int K, void* packed, hipStream_t stream);
int decode_supported(const lily_moe_dims& d);
int launch_decode_noalloc(const lily_moe_dims& d, const lily_moe_weights& w, const float* logits,
                          const uint16_t* x, int32_t* topk_ids, float* topk_w, uint16_t* out,
                          int32_t* status, hipStream_t stream);
int launch_decode(const lily_moe_dims& d, const lily_moe_weights& w, const float* logits,
                  const uint16_t* x, const lily_moe_routing& r, uint16_t* out, void* workspace,
                  hipStream_t stream);
int launch_residual_norm(int T, int H, float* r, const uint16_t* out, uint16_t* x_next,
                         float eps, hipStream_t stream);
int launch_router(const lily_moe_dims& d, const uint16_t* w_router, const uint16_t* x,
                  float* logits, hipStream_t stream);

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE_PTR(p)                                                                   \
    do {                                                                                 \
        if (!(p)) return set_error(LILY_ERR_INVALID_ARG, "%s is NULL", #p);              \
        if (!aligned16(p)) return set_error(LILY_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
    } while (0)

static int check_dims(const lily_moe_dims* d) {
    if (!d) return set_error(LILY_ERR_INVALID_ARG, "dims is NULL");
    if (d->T < 1) return set_error(LILY_ERR_INVALID_ARG, "T = %d < 1", d->T);
    if (d->E < 1) return set_error(LILY_ERR_INVALID_ARG, "E = %d < 1", d->E);
    if (d->topk < 1 || d->topk > d->E)
        return set_error(LILY_ERR_INVALID_ARG, "topk = %d not in [1, E = %d]", d->topk, d->E);
    if (d->group != kGroup)
        return set_error(LILY_ERR_INVALID_ARG, "group = %d; only 64 is supported", d->group);
    if (d->H < kGroup || d->H % kGroup)
        return set_error(LILY_ERR_INVALID_ARG, "H = %d is not a positive multiple of 64", d->H);
    if (d->F < kGroup || d->F % kGroup)
        return set_error(LILY_ERR_INVALID_ARG, "F = %d is not a positive multiple of 64", d->F);
    if (d->tile_m < 1) return set_error(LILY_ERR_INVALID_ARG, "tile_m = %d < 1", d->tile_m);
    if ((int64_t)d->T * d->topk + d->T > (int64_t)1 << 30)
        return set_error(LILY_ERR_UNSUPPORTED, "T * (topk + 1) too large");
    if (d->E > kMaxExperts)
        return set_error(LILY_ERR_UNSUPPORTED, "E = %d > %d", d->E, kMaxExperts);
    if (d->topk > kMaxTopk)
        return set_error(LILY_ERR_UNSUPPORTED, "topk = %d > %d", d->topk, kMaxTopk);
    return LILY_OK;
}

static int32_t max_blocks_of(const lily_moe_dims& d) {
    const int64_t P = (int64_t)d.T * d.topk;
    const int64_t nb = (P + d.tile_m - 1) / d.tile_m + (P < d.E ? P : d.E);
    return (int32_t)nb;
}

static int check_routing(const lily_moe_routing* r) {
    if (!r) return set_error(LILY_ERR_INVALID_ARG, "routing is NULL");
    REQUIRE_PTR(r->topk_ids);
    REQUIRE_PTR(r->topk_w);
    REQUIRE_PTR(r->counts);
    REQUIRE_PTR(r->offsets);
    REQUIRE_PTR(r->sorted_pairs);
    REQUIRE_PTR(r->pair_rows);
    REQUIRE_PTR(r->block_expert);
    REQUIRE_PTR(r->block_row0);
    REQUIRE_PTR(r->num_blocks);
    REQUIRE_PTR(r->block_order);
    REQUIRE_PTR(r->sched);
    REQUIRE_PTR(r->block_info);
    return LILY_OK;
}

static int check_packed(const void* p, const char* name) {
    if (!p) return set_error(LILY_ERR_INVALID_ARG, "weights.%s is NULL", name);
    if (!aligned16(p)) return set_error(LILY_ERR_INVALID_ARG, "weights.%s is not 16-byte aligned", name);
    return LILY_OK;
}

static int check_pack_sizes(int32_t n, int32_t N, int32_t K, int32_t group) {
    if (n < 1 || N < 1 || K < 1)
        return set_error(LILY_ERR_INVALID_ARG, "n = %d, N = %d, K = %d must be >= 1", n, N, K);
    if (group != kGroup)
        return set_error(LILY_ERR_INVALID_ARG, "group = %d; only 64 is supported", group);
    if (N % 128) return set_error(LILY_ERR_INVALID_ARG, "N = %d is not a multiple of 128", N);
    if (K % kGroup) return set_error(LILY_ERR_INVALID_ARG, "K = %d is not a multiple of 64", K);
    if ((int64_t)n * N * K > ((int64_t)1 << 40))
        return set_error(LILY_ERR_INVALID_ARG, "n * N * K too large");
    return LILY_OK;
}

static int check_forward_args(const lily_moe_dims* dims, const lily_moe_weights* weights,
                              const lily_moe_routing* routing) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!weights) return set_error(LILY_ERR_INVALID_ARG, "weights is NULL");
    if ((rc = check_packed(weights->gate, "gate")) || (rc = check_packed(weights->up, "up")) ||
        (rc = check_packed(weights->down, "down")) ||
        (rc = check_packed(weights->sh_gate, "sh_gate")) ||
        (rc = check_packed(weights->sh_up, "sh_up")) ||
        (rc = check_packed(weights->sh_down, "sh_down")))
        return rc;
    rc = check_routing(routing);
    if (rc) return rc;
    if (dims->tile_m != 16 && dims->tile_m != 32 && dims->tile_m != 64 && dims->tile_m != 128)
        return set_error(LILY_ERR_UNSUPPORTED, "tile_m = %d; forward supports 16, 32, 64, 128",
                         dims->tile_m);
    if (dims->H % 256)
        return set_error(LILY_ERR_UNSUPPORTED, "H = %d must be a multiple of 256", dims->H);
    if (dims->F % 128)
        return set_error(LILY_ERR_UNSUPPORTED, "F = %d must be a multiple of 128", dims->F);
    // The grouped GEMMs address their A rows (x [T, H] for gate/up, h
    // [T * (topk + 1), F] for down) with 32-bit byte offsets, and the bf16
    // weight rows of the unfused twin likewise within one [F, H] matrix.
    const int64_t kMax = (int64_t)1 << 32;
    const int64_t rows = (int64_t)dims->T * dims->topk + dims->T;
    if ((int64_t)dims->T * dims->H * 2 >= kMax)
        return set_error(LILY_ERR_UNSUPPORTED, "x [T = %d, H = %d] bf16 is 4 GiB or more", dims->T,
                         dims->H);
    if (rows * dims->F * 2 >= kMax)
        return set_error(LILY_ERR_UNSUPPORTED,
                         "h [T * (topk + 1) = %lld, F = %d] bf16 is 4 GiB or more",
                         (long long)rows, dims->F);
    if ((int64_t)dims->F * dims->H * 2 >= kMax)
        return set_error(LILY_ERR_UNSUPPORTED, "an [F, H] bf16 matrix is 4 GiB or more");
    return LILY_OK;
}

static int check_workspace(const lily_moe_dims& d, const void* workspace, size_t workspace_bytes) {
    const size_t need = forward_workspace_bytes(d, max_blocks_of(d));
    if (!workspace) return set_error(LILY_ERR_INVALID_ARG, "workspace is NULL");
    if (!aligned16(workspace))
        return set_error(LILY_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    if (workspace_bytes < need)
        return set_error(LILY_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
                         workspace_bytes, need);
    return LILY_OK;
}

}  // namespace lily

using namespace lily;

extern "C" {

int32_t lily_moe_max_blocks(const lily_moe_dims* dims) {
    int rc = check_dims(dims);
    if (rc) return rc;
    return max_blocks_of(*dims);
}

size_t lily_moe_workspace_bytes(const lily_moe_dims* dims) {
    if (check_dims(dims)) return 0;
    return forward_workspace_bytes(*dims, max_blocks_of(*dims));
}

size_t lily_w4_packed_bytes(int32_t n, int32_t N, int32_t K, int32_t group) {
    if (check_pack_sizes(n, N, K, group)) return 0;
    return packed_w4_bytes(n, N, K);
}

int lily_w4_pack(const lily_w4* w, int32_t n, int32_t N, int32_t K, int32_t group, void* packed,
                 void* stream) {
    int rc = check_pack_sizes(n, N, K, group);
    if (rc) return rc;
    if (!w) return set_error(LILY_ERR_INVALID_ARG, "w is NULL");
    REQUIRE_PTR(w->q);
    REQUIRE_PTR(w->scale);
    REQUIRE_PTR(w->bias);
    REQUIRE_PTR(packed);
    return launch_pack(*w, n, N, K, packed, reinterpret_cast<hipStream_t>(stream));
}

int lily_moe_router(const lily_moe_dims* dims, const uint16_t* w_router, const uint16_t* x,
                    float* logits, void* stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->H % 256)
        return set_error(LILY_ERR_UNSUPPORTED, "router: H = %d is not a multiple of 256", dims->H);
    REQUIRE_PTR(w_router);
    REQUIRE_PTR(x);
    REQUIRE_PTR(logits);
    return launch_router(*dims, w_router, x, logits, reinterpret_cast<hipStream_t>(stream));
}

int lily_moe_route(const lily_moe_dims* dims, const float* logits,
                   const lily_moe_routing* routing, void* stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    REQUIRE_PTR(logits);
    rc = check_routing(routing);
    if (rc) return rc;
    return launch_route(*dims, logits, *routing, reinterpret_cast<hipStream_t>(stream));
}

int lily_moe_route_host(const lily_moe_dims* dims, const float* logits,
                        const lily_moe_routing* routing, void* stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    REQUIRE_PTR(logits);
    rc = check_routing(routing);
    if (rc) return rc;
    return launch_route_host(*dims, logits, *routing, reinterpret_cast<hipStream_t>(stream));
}

// G1-G3: one launch where it applies, else gate/up then down.
static int run_ffn(const lily_moe_dims& d, const lily_moe_weights& w, const uint16_t* x,
                   const lily_moe_routing& r, const ForwardWorkspace& ws, hipStream_t s) {
    const int mb = max_blocks_of(d);
    const int rc = launch_ffn(d, w, x, r, mb, ws, s);
    if (rc <= 0) return rc;  // launched (0) or failed; 1: not applicable
    const int rg = launch_gate_up(d, w, x, r, mb, ws, s, true);
    return rg ? rg : launch_down(d, w, r, mb, ws, s, true);
}

int lily_moe_forward(const lily_moe_dims* dims, const lily_moe_weights* weights,
                     const uint16_t* x, const lily_moe_routing* routing, uint16_t* out,
                     void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_forward_args(dims, weights, routing);
    if (rc) return rc;
    REQUIRE_PTR(x);
    REQUIRE_PTR(out);
    if ((rc = check_workspace(*dims, workspace, workspace_bytes))) return rc;
    const ForwardWorkspace ws = forward_workspace_split(*dims, workspace);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if ((rc = run_ffn(*dims, *weights, x, *routing, ws, s))) return rc;
    return launch_combine(*dims, ws, *routing, out, s);
}

int lily_moe_dequant(const lily_moe_dims* dims, const lily_moe_weights* packed,
                     const lily_moe_routing* routing, const lily_moe_weights* bf16, void* stream) {
    int rc = check_forward_args(dims, packed, routing);
    if (rc) return rc;
    if (!bf16) return set_error(LILY_ERR_INVALID_ARG, "bf16 is NULL");
    REQUIRE_PTR(bf16->gate);
    REQUIRE_PTR(bf16->up);
    REQUIRE_PTR(bf16->down);
    REQUIRE_PTR(bf16->sh_gate);
    REQUIRE_PTR(bf16->sh_up);
    REQUIRE_PTR(bf16->sh_down);
    // The weight struct's pointers are const; here they name the outputs.
    const lily_moe_dims& d = *dims;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int32_t* c = routing->counts;
    if ((rc = launch_dequant(packed->gate, d.E, d.F, d.H, c, const_cast<void*>(bf16->gate), s)) ||
        (rc = launch_dequant(packed->up, d.E, d.F, d.H, c, const_cast<void*>(bf16->up), s)) ||
        (rc = launch_dequant(packed->down, d.E, d.H, d.F, c, const_cast<void*>(bf16->down), s)) ||
        (rc = launch_dequant(packed->sh_gate, 1, d.F, d.H, nullptr, const_cast<void*>(bf16->sh_gate), s)) ||
        (rc = launch_dequant(packed->sh_up, 1, d.F, d.H, nullptr, const_cast<void*>(bf16->sh_up), s)))
        return rc;
    return launch_dequant(packed->sh_down, 1, d.H, d.F, nullptr, const_cast<void*>(bf16->sh_down), s);
}

int lily_moe_forward_bf16(const lily_moe_dims* dims, const lily_moe_weights* bf16,
                          const uint16_t* x, const lily_moe_routing* routing, uint16_t* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_forward_args(dims, bf16, routing);
    if (rc) return rc;
    REQUIRE_PTR(x);
    REQUIRE_PTR(out);
    if (dims->tile_m != 32 && dims->tile_m != 64)
        return set_error(LILY_ERR_UNSUPPORTED, "tile_m = %d; the bf16 GEMMs take 32 or 64",
                         dims->tile_m);
    if ((rc = check_workspace(*dims, workspace, workspace_bytes))) return rc;
    const ForwardWorkspace ws = forward_workspace_split(*dims, workspace);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int mb = max_blocks_of(*dims);
    if ((rc = launch_gate_up(*dims, *bf16, x, *routing, mb, ws, s, false))) return rc;
    if ((rc = launch_down(*dims, *bf16, *routing, mb, ws, s, false))) return rc;
    return launch_combine(*dims, ws, *routing, out, s);
}

int lily_moe_gate_up(const lily_moe_dims* dims, const lily_moe_weights* weights,
                     const uint16_t* x, const lily_moe_routing* routing, void* workspace,
                     size_t workspace_bytes, void* stream) {
    int rc = check_forward_args(dims, weights, routing);
    if (rc) return rc;
    REQUIRE_PTR(x);
    if ((rc = check_workspace(*dims, workspace, workspace_bytes))) return rc;
    return launch_gate_up(*dims, *weights, x, *routing, max_blocks_of(*dims),
                          forward_workspace_split(*dims, workspace),
                          reinterpret_cast<hipStream_t>(stream), true);
}

int lily_moe_down(const lily_moe_dims* dims, const lily_moe_weights* weights,
                  const lily_moe_routing* routing, void* workspace, size_t workspace_bytes,
                  void* stream) {
    int rc = check_forward_args(dims, weights, routing);
    if (rc) return rc;
    if ((rc = check_workspace(*dims, workspace, workspace_bytes))) return rc;
    return launch_down(*dims, *weights, *routing, max_blocks_of(*dims),
                       forward_workspace_split(*dims, workspace),
                       reinterpret_cast<hipStream_t>(stream), true);
}

int lily_moe_ffn(const lily_moe_dims* dims, const lily_moe_weights* weights, const uint16_t* x,
                 const lily_moe_routing* routing, void* workspace, size_t workspace_bytes,
                 void* stream) {
    int rc = check_forward_args(dims, weights, routing);
    if (rc) return rc;
    REQUIRE_PTR(x);
    if ((rc = check_workspace(*dims, workspace, workspace_bytes))) return rc;
    return run_ffn(*dims, *weights, x, *routing, forward_workspace_split(*dims, workspace),
                   reinterpret_cast<hipStream_t>(stream));
}

int lily_moe_combine(const lily_moe_dims* dims, const lily_moe_routing* routing,
                     void* workspace, size_t workspace_bytes, uint16_t* out, void* stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    rc = check_routing(routing);
    if (rc) return rc;
    REQUIRE_PTR(out);
    if (dims->H % 4) return set_error(LILY_ERR_UNSUPPORTED, "H = %d must be a multiple of 4", dims->H);
    if ((rc = check_workspace(*dims, workspace, workspace_bytes))) return rc;
    return launch_combine(*dims, forward_workspace_split(*dims, workspace), *routing, out,
                          reinterpret_cast<hipStream_t>(stream));
}

int lily_moe_decode(const lily_moe_dims* dims, const lily_moe_weights* weights,
                    const float* logits, const uint16_t* x, const lily_moe_routing* routing,
                    uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if ((rc = decode_supported(*dims))) return rc;
    if (!weights) return set_error(LILY_ERR_INVALID_ARG, "weights is NULL");
    if ((rc = check_packed(weights->gate, "gate")) || (rc = check_packed(weights->up, "up")) ||
        (rc = check_packed(weights->down, "down")) ||
        (rc = check_packed(weights->sh_gate, "sh_gate")) ||
        (rc = check_packed(weights->sh_up, "sh_up")) ||
        (rc = check_packed(weights->sh_down, "sh_down")))
        return rc;
    if (!routing) return set_error(LILY_ERR_INVALID_ARG, "routing is NULL");
    REQUIRE_PTR(routing->topk_ids);
    REQUIRE_PTR(routing->topk_w);
    REQUIRE_PTR(routing->sched);
    REQUIRE_PTR(logits);
    REQUIRE_PTR(x);
    REQUIRE_PTR(out);
    if ((rc = check_workspace(*dims, workspace, workspace_bytes))) return rc;
    return launch_decode(*dims, *weights, logits, x, *routing, out, workspace,
                         reinterpret_cast<hipStream_t>(stream));
}

int lily_moe_decode_noalloc(const lily_moe_dims* dims, const lily_moe_weights* weights,
                            const float* logits, const uint16_t* x, int32_t* topk_ids,
                            float* topk_w, uint16_t* out, int32_t* status, void* stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if ((rc = decode_supported(*dims))) return rc;
    if (!weights) return set_error(LILY_ERR_INVALID_ARG, "weights is NULL");
    if ((rc = check_packed(weights->gate, "gate")) || (rc = check_packed(weights->up, "up")) ||
        (rc = check_packed(weights->down, "down")) ||
        (rc = check_packed(weights->sh_gate, "sh_gate")) ||
        (rc = check_packed(weights->sh_up, "sh_up")) ||
        (rc = check_packed(weights->sh_down, "sh_down")))
        return rc;
    REQUIRE_PTR(logits);
    REQUIRE_PTR(x);
    REQUIRE_PTR(topk_ids);
    REQUIRE_PTR(topk_w);
    REQUIRE_PTR(out);
    if (status && ((uintptr_t)status & 3))
        return set_error(LILY_ERR_INVALID_ARG, "status is not 4-byte aligned");
    return launch_decode_noalloc(*dims, *weights, logits, x, topk_ids, topk_w, out, status,
                                 reinterpret_cast<hipStream_t>(stream));
}

int lily_residual_norm(int32_t T, int32_t H, float* r, const uint16_t* out, uint16_t* x_next,
                       float eps, void* stream) {
    if (T < 1 || H < 4 || H % 4)
        return set_error(LILY_ERR_INVALID_ARG, "T = %d, H = %d (need T >= 1, H %% 4 == 0)", T, H);
    if (!(eps >= 0.0f)) return set_error(LILY_ERR_INVALID_ARG, "eps must be >= 0");
    REQUIRE_PTR(r);
    REQUIRE_PTR(x_next);
    if (out && !aligned16(out))
        return set_error(LILY_ERR_INVALID_ARG, "out is not 16-byte aligned");
    return launch_residual_norm(T, H, r, out, x_next, eps, reinterpret_cast<hipStream_t>(stream));
}

int lily_moe_decode_stack(const lily_moe_dims* dims, int32_t n_layers,
                          const lily_moe_weights* layers, const float* logits, const uint16_t* x0,
                          float* r, uint16_t* outs, int32_t* topk_ids, float* topk_w,
                          int32_t* sched, float eps, void* workspace, size_t workspace_bytes,
                          void* stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    REQUIRE_PTR(layers);
    REQUIRE_PTR(logits);
    REQUIRE_PTR(x0);
    REQUIRE_PTR(r);
    REQUIRE_PTR(outs);
    REQUIRE_PTR(topk_ids);
    REQUIRE_PTR(topk_w);
    REQUIRE_PTR(sched);
    if (!(eps >= 0.0f)) return set_error(LILY_ERR_INVALID_ARG, "eps must be >= 0");
    if ((rc = decode_stack_supported(*dims, n_layers))) return rc;
    if ((rc = check_workspace(*dims, workspace, workspace_bytes))) return rc;
    return launch_decode_stack(*dims, n_layers, layers, logits, x0, r, outs, topk_ids, topk_w,
                               sched, eps, workspace, reinterpret_cast<hipStream_t>(stream));
}

int lily_trace_ffn_items(unsigned long long* dst, int32_t max_wgs, void* stream) {
    return trace_ffn_items(dst, max_wgs, reinterpret_cast<hipStream_t>(stream));
}

int lily_trace_decode_stack(unsigned long long* dst, int32_t max_wgs, void* stream) {
    return trace_decode_stack(dst, max_wgs, reinterpret_cast<hipStream_t>(stream));
}

const char* lily_last_error(void) { return g_last_error; }

}  // extern "C"
