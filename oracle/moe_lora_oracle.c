/*
 * Plain CPU reference of the multi-LoRA Mixture-of-Experts expert layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no code, header,
 * table or helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes (AWS ML Blog post "Efficiently serve dozens of fine-tuned
 * models with vLLM on Amazon SageMaker AI and Amazon Bedrock"):
 *  - a router sends each token to its most relevant experts and their
 *    outputs are aggregated (section "Implementing multi-LoRA inference for
 *    MoE models in vLLM");
 *  - each expert is a two-stage feed-forward block: gate_up widens the hidden
 *    state to the intermediate size and down maps it back; with LoRA each of
 *    the two projections gets a shrink (x.A, rank r) and an expand ((x.A).B)
 *    that is added to the base projection's output (Korean summary on
 *    agentlenshq.com, section "Multi-LoRA serving for MoE"; section "Kernel
 *    optimizations" of the AWS post for shrink = xA and the fused add);
 *  - the adapter is chosen per request, frozen base weights are shared
 *    (AWS post, first section).
 * The activation between the projections is not named on the pages; this
 * reference takes SwiGLU: h_i = silu(g_i) * g_{I+i}, silu(z) = z / (1 + e^-z),
 * with gate rows 0..I-1 and up rows I..2I-1 of the gate_up weight.
 * Routing: the k largest logits (ties -> lower expert id), weights = softmax
 * over the selected logits (equal to softmax over all E, top-k, renormalise).
 * LoRA scaling is 1; an adapter id outside [0, L) means "no adapter".
 *
 * Precision: inputs are bf16 (exactly representable in double); every
 * product, sum, exponential and intermediate is double, with no rounding
 * between stages.
 *
 * Layouts (row-major):
 *   x [T][H] bf16 bits, logits [T][E] f32, adapter_ids [T] i32,
 *   w_gu [E][2I][H], w_d [E][H][I], a_gu [L][E][r][H], b_gu [L][E][2I][r],
 *   a_d [L][E][r][I], b_d [L][E][H][r]   (all bf16 bits)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double widen_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Top-k selection on the logits plus renormalised softmax weights. */
int oracle_route(int32_t T, int32_t E, int32_t k, const float *logits,
                 int32_t *ids, double *w) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
    char *taken = (char *)malloc((size_t)E);
    if (!taken) return -2;
    for (int32_t t = 0; t < T; ++t) {
        const float *row = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                /* strictly greater: an equal later expert never displaces the
                   earlier (lower id) one */
                if (best < 0 || row[e] > row[best]) best = e;
            }
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        double m = (double)row[ids[(size_t)t * k]];
        double s = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            double v = exp((double)row[ids[(size_t)t * k + j]] - m);
            w[(size_t)t * k + j] = v;
            s += v;
        }
        for (int32_t j = 0; j < k; ++j) w[(size_t)t * k + j] /= s;
    }
    free(taken);
    return 0;
}

/* out_row = M[rows][cols] . v  (M in bf16 bits, v double) */
static void matvec_bf16(const uint16_t *M, int64_t rows, int64_t cols,
                        const double *v, double *out_row) {
    for (int64_t n = 0; n < rows; ++n) {
        const uint16_t *m = M + n * cols;
        double acc = 0.0;
        for (int64_t q = 0; q < cols; ++q) acc += widen_bf16(m[q]) * v[q];
        out_row[n] = acc;
    }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * Evaluate the layer for the tokens listed in toks[0..ntok) using the given
 * routing (ids, w: [T][k]). out is [ntok][H] (overwritten). The optional stage
 * buffers receive, per listed token and choice j (row = i*k + j):
 *   st_s1 [r] gate_up shrink, st_g [2I] gate_up output incl. LoRA,
 *   st_h [I] activation, st_s2 [r] down shrink, st_d [H] down output incl. LoRA.
 * Shrink rows of pairs without an adapter are written as 0.
 */
int oracle_forward(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                   int32_t L, int32_t r,
                   const uint16_t *x, const int32_t *ids, const double *w,
                   const int32_t *adapter_ids,
                   const uint16_t *w_gu, const uint16_t *w_d,
                   const uint16_t *a_gu, const uint16_t *b_gu,
                   const uint16_t *a_d, const uint16_t *b_d,
                   int32_t ntok, const int32_t *toks, double *out,
                   double *st_s1, double *st_g, double *st_h, double *st_s2,
                   double *st_d, int32_t nthreads) {
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || L < 0 || r <= 0) return -1;
    for (int32_t i = 0; i < ntok; ++i)
        if (toks[i] < 0 || toks[i] >= T) return -1;
    const int64_t H64 = H, I64 = I, r64 = r, E64 = E;
    int failed = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double *xd = (double *)malloc(sizeof(double) * H64);
        double *g = (double *)malloc(sizeof(double) * 2 * I64);
        double *t2 = (double *)malloc(sizeof(double) * 2 * I64);
        double *h = (double *)malloc(sizeof(double) * I64);
        double *d = (double *)malloc(sizeof(double) * H64);
        double *d2 = (double *)malloc(sizeof(double) * H64);
        double *s = (double *)malloc(sizeof(double) * r64);
        const int ok = xd && g && t2 && h && d && d2 && s;
#pragma omp for schedule(dynamic, 1)
            for (int32_t i = 0; i < ntok; ++i) {
                if (!ok) {
#pragma omp atomic write
                    failed = 1;
                    continue;
                }
                const int32_t t = toks[i];
                double *o = out + (int64_t)i * H64;
                for (int64_t n = 0; n < H64; ++n) o[n] = 0.0;
                for (int64_t q = 0; q < H64; ++q) xd[q] = widen_bf16(x[t * H64 + q]);
                int32_t a = adapter_ids[t];
                if (a < 0 || a >= L) a = -1;
                for (int32_t j = 0; j < k; ++j) {
                    const int64_t e = ids[(int64_t)t * k + j];
                    const int64_t row = (int64_t)i * k + j;
                    /* gate_up: base projection */
                    matvec_bf16(w_gu + e * 2 * I64 * H64, 2 * I64, H64, xd, g);
                    if (a >= 0) {
                        const int64_t ae = (int64_t)a * E64 + e;
                        /* shrink s = A x, expand g += B s */
                        matvec_bf16(a_gu + ae * r64 * H64, r64, H64, xd, s);
                        matvec_bf16(b_gu + ae * 2 * I64 * r64, 2 * I64, r64, s, t2);
                        for (int64_t n = 0; n < 2 * I64; ++n) g[n] += t2[n];
                        if (st_s1) memcpy(st_s1 + row * r64, s, sizeof(double) * r64);
                    } else if (st_s1) {
                        memset(st_s1 + row * r64, 0, sizeof(double) * r64);
                    }
                    if (st_g) memcpy(st_g + row * 2 * I64, g, sizeof(double) * 2 * I64);
                    for (int64_t q = 0; q < I64; ++q) h[q] = silu(g[q]) * g[I64 + q];
                    if (st_h) memcpy(st_h + row * I64, h, sizeof(double) * I64);
                    /* down: base projection */
                    matvec_bf16(w_d + e * H64 * I64, H64, I64, h, d);
                    if (a >= 0) {
                        const int64_t ae = (int64_t)a * E64 + e;
                        matvec_bf16(a_d + ae * r64 * I64, r64, I64, h, s);
                        matvec_bf16(b_d + ae * H64 * r64, H64, r64, s, d2);
                        for (int64_t n = 0; n < H64; ++n) d[n] += d2[n];
                        if (st_s2) memcpy(st_s2 + row * r64, s, sizeof(double) * r64);
                    } else if (st_s2) {
                        memset(st_s2 + row * r64, 0, sizeof(double) * r64);
                    }
                    if (st_d) memcpy(st_d + row * H64, d, sizeof(double) * H64);
                    /* aggregate with the routing weight */
                    const double wj = w[(int64_t)t * k + j];
                    for (int64_t n = 0; n < H64; ++n) o[n] += wj * d[n];
                }
            }
        free(xd); free(g); free(t2); free(h); free(d); free(d2); free(s);
    }
    return failed ? -2 : 0;
}
