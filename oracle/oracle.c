/*
 * CPU oracle for the int4 grouped-GEMM MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code with
 * the GPU path and is deliberately plain and slow: one token at a time, one
 * expert at a time, sums in index order.
 *
 * What it computes (sources are the Lily articles; "ainew" is the Japanese
 * news.ainew.jp article "Perplexity, Apple Silicon向け推論エンジン「Lily」を
 * オープンソース化", whose sections are named below):
 *
 *  - Weights are groupwise-affine 4-bit: every 64 consecutive weights of a
 *    row share one bf16 scale and one bf16 bias (ainew, section "Prefill").
 *    A weight is w = scale*q + bias with q in 0..15. The tensor units consume
 *    bf16, so the weights are rebuilt as bf16 before the product, and the
 *    products accumulate in FP32 (same section).
 *  - The router scores E experts and picks k of them; a shared expert also
 *    processes every token (ainew, section on the three workload shapes).
 *    Where the scores come from x, they are the router projection x.Wr^T
 *    (bf16 inputs, summed in double here).
 *  - Per MoE layer the route is: a per-expert histogram, a prefix scan, a
 *    scatter of tokens into expert order and a block map for the grouped
 *    GEMM (ainew, section "Prefill").
 *
 * The pages leave these steps open; the readings taken here are:
 *  - q sits in the low nibble for even k, high nibble for odd k; groups run
 *    along K, the input dimension of an [N, K] (out x in) matrix.
 *  - top-k keeps the k largest logits; an equal logit goes to the lower
 *    expert index (-0.0 equals +0.0). The routing weights are a softmax over
 *    the k selected logits.
 *  - Each expert is a SwiGLU FFN: h = bf16(silu(g) * u), g = x.Wg^T,
 *    u = x.Wu^T, y = h.Wd^T kept in fp32. The shared expert has weight 1.
 *  - Combine: out = bf16(y_shared + sum_j w_j * y_j), summed in j order.
 *  - Scatter order inside an expert's segment is ascending token, then
 *    ascending slot j (a stable counting sort of the (t, j) pairs).
 *  - Block map: for each non-empty expert in ascending order, one block per
 *    M rows of its segment.
 *
 * Rounding: bf16 round-to-nearest-even at the dequantised weight, at h and
 * at the output; everything else is fp32. Built without fast-math and
 * without FP contraction so that every operation rounds as written.
 *
 * Parity: the functions here are pinned by the CPU tests against closed
 * forms, routing invariants, hand-worked fixtures and a dense float64
 * formulation on small inputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_NONFINITE (-2)
#define ORACLE_ERR_NOMEM (-3)

#define GROUP 64

/* ------------------------------------------------------------------ bf16 */

static float bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a finite float to the nearest bf16, ties to even. */
static uint16_t float_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

static float round_bf16(float f) { return bf16_to_float(float_to_bf16(f)); }

/* --------------------------------------------------------------- dequant */

/* Element kk of row `row` of an int4 matrix with K columns. */
static float dequant_one(const uint8_t* q, const uint16_t* scale, const uint16_t* bias,
                         int K, int row, int kk) {
    uint8_t byte = q[(size_t)row * (K / 2) + kk / 2];
    int nib = (kk % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    int g = kk / GROUP;
    float s = bf16_to_float(scale[(size_t)row * (K / GROUP) + g]);
    float b = bf16_to_float(bias[(size_t)row * (K / GROUP) + g]);
    float w = fmaf(s, (float)nib, b);
    return round_bf16(w);
}

/* Dequantise a whole [N, K] matrix into bf16 bit patterns. */
int oracle_dequant(const uint8_t* q, const uint16_t* scale, const uint16_t* bias,
                   int N, int K, uint16_t* w_out) {
    if (!q || !scale || !bias || !w_out || N < 1 || K < GROUP || K % GROUP) return ORACLE_ERR_ARG;
    for (int n = 0; n < N; ++n)
        for (int kk = 0; kk < K; ++kk)
            w_out[(size_t)n * K + kk] = float_to_bf16(dequant_one(q, scale, bias, K, n, kk));
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- route */

/* Is logit a (expert ea) ranked above logit b (expert eb)? */
static int ranks_above(float a, int ea, float b, int eb) {
    if (a > b) return 1;
    if (a < b) return 0;
    return ea < eb; /* equal values, including -0.0 vs +0.0 */
}

int oracle_route(int T, int E, int k, int M, const float* logits,
                 int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_pairs, int32_t* pair_rows,
                 int32_t* block_expert, int32_t* block_row0, int32_t* num_blocks) {
    if (T < 1 || E < 1 || k < 1 || k > E || M < 1 || !logits || !topk_ids || !topk_w ||
        !counts || !offsets || !sorted_pairs || !pair_rows || !block_expert || !block_row0 ||
        !num_blocks)
        return ORACLE_ERR_ARG;
    for (size_t i = 0; i < (size_t)T * E; ++i)
        if (!isfinite(logits[i])) return ORACLE_ERR_NONFINITE;

    /* top-k by repeated selection of the best remaining expert, then a
       softmax over the k selected logits. */
    char* taken = (char*)malloc((size_t)E);
    float* ex = (float*)malloc((size_t)k * sizeof(float));
    if (!taken || !ex) { free(taken); free(ex); return ORACLE_ERR_NOMEM; }
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_above(l[e], e, l[best], best)) best = e;
            }
            taken[best] = 1;
            topk_ids[(size_t)t * k + j] = best;
        }
        float lmax = l[topk_ids[(size_t)t * k]];
        float sum = 0.0f;
        for (int j = 0; j < k; ++j) {
            ex[j] = expf(l[topk_ids[(size_t)t * k + j]] - lmax);
            sum += ex[j];
        }
        for (int j = 0; j < k; ++j) topk_w[(size_t)t * k + j] = ex[j] / sum;
    }
    free(taken);
    free(ex);

    /* histogram of rows per expert */
    const int P = T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int p = 0; p < P; ++p) counts[topk_ids[p]] += 1;

    /* exclusive prefix scan */
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];

    /* stable scatter: pairs visited in (t, j) order */
    int32_t* cursor = (int32_t*)malloc((size_t)E * sizeof(int32_t));
    if (!cursor) return ORACLE_ERR_NOMEM;
    for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int p = 0; p < P; ++p) {
        int e = topk_ids[p];
        int row = cursor[e]++;
        sorted_pairs[row] = p;
        pair_rows[p] = row;
    }
    free(cursor);

    /* block map: M rows per block, experts in ascending order */
    int nb = 0;
    for (int e = 0; e < E; ++e) {
        for (int r0 = offsets[e]; r0 < offsets[e + 1]; r0 += M) {
            block_expert[nb] = e;
            block_row0[nb] = r0;
            ++nb;
        }
    }
    *num_blocks = nb;
    return ORACLE_OK;
}

/* --------------------------------------------------------------- forward */

/* One int4 matrix per expert. Index E is the shared expert. An entry may be
   NULL for an expert that none of the requested tokens uses. */
typedef struct {
    const uint8_t* const* q;
    const uint16_t* const* scale;
    const uint16_t* const* bias;
} oracle_w4_set;

static float silu(float z) { return z / (1.0f + expf(-z)); }

/* The SwiGLU FFN of one expert on one token row, from dequantised weights.
   wg, wu: [F, H] float (bf16 values); wd: [H, F]. y: [H] fp32 out. */
static void expert_ffn(const float* xrow, int H, int F, const float* wg, const float* wu,
                       const float* wd, float* hbuf, float* y) {
    for (int f = 0; f < F; ++f) {
        float g = 0.0f, u = 0.0f;
        for (int kk = 0; kk < H; ++kk) {
            g = g + xrow[kk] * wg[(size_t)f * H + kk];
            u = u + xrow[kk] * wu[(size_t)f * H + kk];
        }
        hbuf[f] = round_bf16(silu(g) * u);
    }
    for (int n = 0; n < H; ++n) {
        float acc = 0.0f;
        for (int f = 0; f < F; ++f) acc = acc + hbuf[f] * wd[(size_t)n * F + f];
        y[n] = acc;
    }
}

static float* dequant_to_float(const uint8_t* q, const uint16_t* s, const uint16_t* b, int N,
                               int K) {
    float* w = (float*)malloc((size_t)N * K * sizeof(float));
    if (!w) return NULL;
    for (int n = 0; n < N; ++n)
        for (int kk = 0; kk < K; ++kk) w[(size_t)n * K + kk] = dequant_one(q, s, b, K, n, kk);
    return w;
}

/*
 * Layer output for the tokens listed in `tokens` (n_tok entries; NULL means
 * tokens 0..n_tok-1). x: bf16 [T_all, H]; topk_ids/topk_w: [T_all, k].
 * acc_out: fp32 [n_tok, H] (the sum before the final rounding);
 * out_bf16: bf16 [n_tok, H]. Either output may be NULL.
 * Phase 1 marks the experts used, phase 2 dequantises them, phase 3 runs
 * one token at a time.
 */
int oracle_forward(int H, int F, int E, int k, const uint16_t* x, const int32_t* topk_ids,
                   const float* topk_w, const int32_t* tokens, int n_tok,
                   oracle_w4_set gate, oracle_w4_set up, oracle_w4_set down,
                   float* acc_out, uint16_t* out_bf16, int n_threads) {
    if (H < GROUP || H % GROUP || F < GROUP || F % GROUP || E < 1 || k < 1 || k > E ||
        n_tok < 0 || !x || !topk_ids || !topk_w)
        return ORACLE_ERR_ARG;
    if (n_tok == 0) return ORACLE_OK;

    char* used = (char*)calloc((size_t)E + 1, 1);
    float** wg = (float**)calloc((size_t)E + 1, sizeof(float*));
    float** wu = (float**)calloc((size_t)E + 1, sizeof(float*));
    float** wd = (float**)calloc((size_t)E + 1, sizeof(float*));
    int rc = ORACLE_OK;
    if (!used || !wg || !wu || !wd) { rc = ORACLE_ERR_NOMEM; goto done; }

    used[E] = 1;
    for (int i = 0; i < n_tok; ++i) {
        int t = tokens ? tokens[i] : i;
        for (int j = 0; j < k; ++j) {
            int e = topk_ids[(size_t)t * k + j];
            if (e < 0 || e >= E) { rc = ORACLE_ERR_ARG; goto done; }
            used[e] = 1;
        }
    }
    for (int e = 0; e <= E; ++e) {
        if (!used[e]) continue;
        if (!gate.q[e] || !gate.scale[e] || !gate.bias[e] || !up.q[e] || !up.scale[e] ||
            !up.bias[e] || !down.q[e] || !down.scale[e] || !down.bias[e]) {
            rc = ORACLE_ERR_ARG;
            goto done;
        }
    }

#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

    int nomem = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int e = 0; e <= E; ++e) {
        if (!used[e]) continue;
        wg[e] = dequant_to_float(gate.q[e], gate.scale[e], gate.bias[e], F, H);
        wu[e] = dequant_to_float(up.q[e], up.scale[e], up.bias[e], F, H);
        wd[e] = dequant_to_float(down.q[e], down.scale[e], down.bias[e], H, F);
        if (!wg[e] || !wu[e] || !wd[e]) {
#pragma omp atomic write
            nomem = 1;
        }
    }
    if (nomem) { rc = ORACLE_ERR_NOMEM; goto done; }

#pragma omp parallel
    {
        float* xrow = (float*)malloc((size_t)H * sizeof(float));
        float* hbuf = (float*)malloc((size_t)F * sizeof(float));
        float* y = (float*)malloc((size_t)H * sizeof(float));
        float* acc = (float*)malloc((size_t)H * sizeof(float));
        if (!xrow || !hbuf || !y || !acc) {
#pragma omp atomic write
            nomem = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int i = 0; i < n_tok; ++i) {
                int t = tokens ? tokens[i] : i;
                for (int kk = 0; kk < H; ++kk) xrow[kk] = bf16_to_float(x[(size_t)t * H + kk]);
                /* shared expert, weight 1 */
                expert_ffn(xrow, H, F, wg[E], wu[E], wd[E], hbuf, y);
                for (int n = 0; n < H; ++n) acc[n] = y[n];
                /* routed experts in selection order */
                for (int j = 0; j < k; ++j) {
                    int e = topk_ids[(size_t)t * k + j];
                    float w = topk_w[(size_t)t * k + j];
                    expert_ffn(xrow, H, F, wg[e], wu[e], wd[e], hbuf, y);
                    for (int n = 0; n < H; ++n) acc[n] = acc[n] + w * y[n];
                }
                for (int n = 0; n < H; ++n) {
                    if (acc_out) acc_out[(size_t)i * H + n] = acc[n];
                    if (out_bf16) out_bf16[(size_t)i * H + n] = float_to_bf16(acc[n]);
                }
            }
        }
        free(xrow);
        free(hbuf);
        free(y);
        free(acc);
    }
    if (nomem) rc = ORACLE_ERR_NOMEM;

done:
    if (wg)
        for (int e = 0; e <= E; ++e) free(wg[e]);
    if (wu)
        for (int e = 0; e <= E; ++e) free(wu[e]);
    if (wd)
        for (int e = 0; e <= E; ++e) free(wd[e]);
    free(wg);
    free(wu);
    free(wd);
    free(used);
    return rc;
}

/* ------------------------------------------------- glue for layer stacks */

/*
 * Residual stream between stacked layers. The pages describe a stack of 40
 * layers but not the glue between MoE layers; the reading taken is the
 * standard pre-norm residual with a unit-gain RMSNorm:
 *   r <- r + out (fp32);  x_next = bf16(r / sqrt(mean(r^2) + eps)).
 * r: fp32 [T, H] in/out; out_bf16: [T, H] or NULL (then r is only
 * normalised); x_next: bf16 [T, H].
 */
int oracle_residual_norm(int T, int H, float* r, const uint16_t* out_bf16, uint16_t* x_next,
                         float eps) {
    if (T < 1 || H < 1 || !r || !x_next) return ORACLE_ERR_ARG;
    for (int t = 0; t < T; ++t) {
        float* rr = r + (size_t)t * H;
        if (out_bf16)
            for (int n = 0; n < H; ++n) rr[n] = rr[n] + bf16_to_float(out_bf16[(size_t)t * H + n]);
        float ss = 0.0f;
        for (int n = 0; n < H; ++n) ss = ss + rr[n] * rr[n];
        float inv = 1.0f / sqrtf(ss / (float)H + eps);
        for (int n = 0; n < H; ++n) x_next[(size_t)t * H + n] = float_to_bf16(rr[n] * inv);
    }
    return ORACLE_OK;
}

/* Expose the oracle's own rounding for the pins. */
/* Router projection (the router scores every expert for each token: ainew,
   section on the three workload shapes): logits[t, e] = sum_h x[t, h] *
   w[e, h] with bf16 inputs, summed in double and rounded once to float.
   absdot[t, e] = sum_h |x[t, h] * w[e, h]| (double, then float) bounds the
   error of any fp32 summation order; either output may be NULL. */
int oracle_router(int T, int H, int E, const uint16_t* x, const uint16_t* w, float* logits,
                  float* absdot) {
    if (T < 1 || H < 1 || E < 1 || !x || !w) return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0, mag = 0.0;
            for (int h = 0; h < H; ++h) {
                const double p = (double)bf16_to_float(x[(size_t)t * H + h]) *
                                 (double)bf16_to_float(w[(size_t)e * H + h]);
                acc += p;
                mag += fabs(p);
            }
            if (logits) logits[(size_t)t * E + e] = (float)acc;
            if (absdot) absdot[(size_t)t * E + e] = (float)mag;
        }
    }
    return 0;
}

uint16_t oracle_float_to_bf16(float f) { return float_to_bf16(f); }
int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
