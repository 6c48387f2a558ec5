/*
 * ORACLE — test infrastructure only.
 *
 * A plain, slow CPU evaluation of one autoregressive decode step of a
 * Llama-style decoder, the computation that the persistent megakernel must
 * reproduce.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load it; the GPU path never calls it and shares no code with it.
 *
 * The pages describe the megakernel as an execution strategy for a model they
 * take as given: fused "RMSNorm + QKV + RoPE", attention, and the MLP
 * instructions of the Llama-1B forward (yaoshibet.com news page on the Hazy
 * Research megakernel, section 4 "design": fusion of about a hundred
 * operations; section 5 breakdown: RMS norm and matrix-vector products), and
 * insist that fusing must not change the model's result beyond floating-point
 * reordering (cloud.baidu.com explainer, sections 7 and 8).  So this file is
 * the definition of the standard Llama decoder step, written out sequentially:
 *
 *   x  = E[token]                                   (embedding row)
 *   per layer:  xn = rmsnorm(x, g1)
 *               q, k, v = Wq xn, Wk xn, Wv xn
 *               q, k rotated by RoPE at the step's position
 *               k, v stored into the bf16 cache slot `position`
 *               a_i = softmax(q_i K^T / sqrt(d)) V   (GQA, causal 0..pos)
 *               x  = x + Wo a
 *               xn = rmsnorm(x, g2)
 *               x  = x + Wd (silu(Wg xn) * (Wu xn))   (dense SwiGLU)
 *                 or the top-k routed mixture of SwiGLU experts (MoE)
 *   hidden = x;  logits = Wlm rmsnorm(x, gf);  next = argmax(logits)
 *
 * Precision: every activation is double; every dot product, sum of squares and
 * softmax sum accumulates in double, in index order.  Weights are bf16 (exact
 * in double).  Two decisions take a rounding that the GPU path also takes:
 * a cache write rounds double -> float -> bf16 (round to nearest even), and the
 * argmax (and the MoE expert choice) is taken over logits rounded to float,
 * lowest index winning ties.
 *
 * Readings where the pages are silent (all are the plain Llama convention):
 * RoPE pairs (j, j + d/2) of each head, frequency theta^(-2j/d), no scaling;
 * eps inside the square root, gain after normalising; attention scale
 * 1/sqrt(d); query head i uses KV head floor(i / (n_q / n_kv)).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t n_layers, hidden, n_q, n_kv, head_dim, ffn, vocab;
    int32_t n_experts, top_k, expert_ffn; /* n_experts == 0: dense FFN */
    double eps, theta;
} orc_cfg;

typedef struct {
    const uint16_t *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
    const uint16_t *router, *exp_gate, *exp_up, *exp_down; /* MoE: [E][f][h], [E][f][h], [E][h][f] */
} orc_layer;

/* ---- scalar helpers ---------------------------------------------------- */

double orc_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* double -> float (C cast, round to nearest even) -> bf16 (round to nearest even) */
uint16_t orc_f64_to_bf16(double x) {
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* ---- vector operations -------------------------------------------------- */

/* out = x * g / sqrt(mean(x^2) + eps) */
void orc_rmsnorm(const double *x, const uint16_t *g, int32_t n, double eps, double *out) {
    double ss = 0.0;
    for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int32_t i = 0; i < n; ++i) out[i] = x[i] * r * orc_bf16_to_f64(g[i]);
}

/* y = W x, W row-major bf16 [rows][cols] */
void orc_gemv(const uint16_t *W, int32_t rows, int32_t cols, const double *x, double *y) {
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < rows; ++r) {
        const uint16_t *w = W + (size_t)r * cols;
        double acc = 0.0;
        for (int32_t c = 0; c < cols; ++c) acc += orc_bf16_to_f64(w[c]) * x[c];
        y[r] = acc;
    }
}

/* Rotate each head of v (n_heads x d) by the position angle:
 * (v_j, v_{j+d/2}) -> (v_j cos a - v_{j+d/2} sin a, v_j sin a + v_{j+d/2} cos a),
 * a = pos * theta^(-2j/d), j < d/2. */
void orc_rope(double *v, int32_t n_heads, int32_t d, int32_t pos, double theta) {
    int32_t half = d / 2;
    for (int32_t h = 0; h < n_heads; ++h) {
        double *u = v + (size_t)h * d;
        for (int32_t j = 0; j < half; ++j) {
            double a = (double)pos * pow(theta, -2.0 * (double)j / (double)d);
            double c = cos(a), s = sin(a);
            double lo = u[j], hi = u[j + half];
            u[j] = lo * c - hi * s;
            u[j + half] = lo * s + hi * c;
        }
    }
}

/* One query head over positions 0..n_pos-1 of one KV head.
 * K, V: bf16 [n_pos rows, stride d].  If cur_k/cur_v are non-NULL they replace
 * row n_pos-1 (the current token) with unrounded values. */
void orc_attention_head(const double *q, const uint16_t *K, const uint16_t *V, int32_t d, int32_t n_pos,
                        const double *cur_k, const double *cur_v, double *out) {
    double *s = (double *)malloc(sizeof(double) * (size_t)n_pos);
    double scale = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int32_t p = 0; p < n_pos; ++p) {
        double acc = 0.0;
        for (int32_t t = 0; t < d; ++t) {
            double kv = (cur_k && p == n_pos - 1) ? cur_k[t] : orc_bf16_to_f64(K[(size_t)p * d + t]);
            acc += q[t] * kv;
        }
        s[p] = acc * scale;
        if (s[p] > m) m = s[p];
    }
    double z = 0.0;
    for (int32_t p = 0; p < n_pos; ++p) {
        s[p] = exp(s[p] - m);
        z += s[p];
    }
    for (int32_t t = 0; t < d; ++t) out[t] = 0.0;
    for (int32_t p = 0; p < n_pos; ++p) {
        double w = s[p] / z;
        for (int32_t t = 0; t < d; ++t) {
            double vv = (cur_v && p == n_pos - 1) ? cur_v[t] : orc_bf16_to_f64(V[(size_t)p * d + t]);
            out[t] += w * vv;
        }
    }
    free(s);
}

/* Lowest index among the maxima of the float-rounded values; -1 if any NaN. */
int32_t orc_argmax_f32(const double *v, int32_t n) {
    int32_t best = 0;
    float bv = (float)v[0];
    for (int32_t i = 0; i < n; ++i) {
        float f = (float)v[i];
        if (f != f) return -1;
        if (f > bv) {
            bv = f;
            best = i;
        }
    }
    return best;
}

/* Top-k of float-rounded router logits (ties -> lower id), softmax over the k selected. */
void orc_topk_softmax(const double *logits, int32_t n, int32_t k, int32_t *ids, double *w) {
    char *taken = (char *)calloc((size_t)n, 1);
    for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        float bv = 0.0f;
        for (int32_t e = 0; e < n; ++e) {
            if (taken[e]) continue;
            float f = (float)logits[e];
            if (best < 0 || f > bv) {
                best = e;
                bv = f;
            }
        }
        taken[best] = 1;
        ids[j] = best;
    }
    double m = -INFINITY, z = 0.0;
    for (int32_t j = 0; j < k; ++j)
        if (logits[ids[j]] > m) m = logits[ids[j]];
    for (int32_t j = 0; j < k; ++j) {
        w[j] = exp(logits[ids[j]] - m);
        z += w[j];
    }
    for (int32_t j = 0; j < k; ++j) w[j] /= z;
    free(taken);
}

/* ---- the decode step ------------------------------------------------------ */

/* SwiGLU FFN: out = Wd (silu(Wg xn) * (Wu xn)); Wg, Wu [f][h], Wd [h][f] */
static void swiglu(const uint16_t *wg, const uint16_t *wu, const uint16_t *wd, int32_t h, int32_t f, const double *xn,
                   double *out) {
    double *g = (double *)malloc(sizeof(double) * (size_t)f);
    double *u = (double *)malloc(sizeof(double) * (size_t)f);
    orc_gemv(wg, f, h, xn, g);
    orc_gemv(wu, f, h, xn, u);
    for (int32_t i = 0; i < f; ++i) g[i] = orc_silu(g[i]) * u[i];
    orc_gemv(wd, h, f, g, out);
    free(g);
    free(u);
}

/*
 * One decode step for `batch` independent sequences.
 *   tokens[b], positions[b]: the token fed at this step and its position P_b
 *     (= number of tokens already in the cache); the step writes cache slot P_b.
 *   k_cache, v_cache: bf16 [n_layers][batch][n_kv][max_ctx][head_dim], updated.
 *   kv_round: 1 = the current token's K/V enter attention as stored (bf16);
 *             0 = they enter unrounded (used only to compare with fp64 references).
 *   hidden_out [batch][h], logits [batch][vocab], next [batch];
 *   layer_out (optional) [n_layers][batch][h]: the residual after each layer;
 *   expert_ids (optional, MoE) [n_layers][batch][top_k];
 *   router_out (optional, MoE) [n_layers][batch][n_experts]: the router logits.
 */
int32_t orc_decode_step(const orc_cfg *cfg, const orc_layer *layers, const uint16_t *embed, const uint16_t *lm_head,
                        const uint16_t *final_norm, int32_t batch, const int32_t *tokens, const int32_t *positions,
                        uint16_t *k_cache, uint16_t *v_cache, int32_t max_ctx, int32_t kv_round, double *hidden_out,
                        double *logits, int32_t *next, double *layer_out, int32_t *expert_ids,
                        double *router_out) {
    const int32_t h = cfg->hidden, nq = cfg->n_q, nkv = cfg->n_kv, d = cfg->head_dim, L = cfg->n_layers;
    const int32_t grp = nq / nkv;
    for (int32_t b = 0; b < batch; ++b) {
        if (tokens[b] < 0 || tokens[b] >= cfg->vocab) return -1;
        if (positions[b] < 0 || positions[b] >= max_ctx) return -2;
    }
    double *x = (double *)malloc(sizeof(double) * (size_t)h);
    double *xn = (double *)malloc(sizeof(double) * (size_t)h);
    double *q = (double *)malloc(sizeof(double) * (size_t)nq * d);
    double *k = (double *)malloc(sizeof(double) * (size_t)nkv * d);
    double *v = (double *)malloc(sizeof(double) * (size_t)nkv * d);
    double *a = (double *)malloc(sizeof(double) * (size_t)nq * d);
    double *t = (double *)malloc(sizeof(double) * (size_t)h);
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t P = positions[b];
        for (int32_t i = 0; i < h; ++i) x[i] = orc_bf16_to_f64(embed[(size_t)tokens[b] * h + i]);
        for (int32_t l = 0; l < L; ++l) {
            const orc_layer *W = &layers[l];
            /* attention block */
            orc_rmsnorm(x, W->attn_norm, h, cfg->eps, xn);
            orc_gemv(W->wq, nq * d, h, xn, q);
            orc_gemv(W->wk, nkv * d, h, xn, k);
            orc_gemv(W->wv, nkv * d, h, xn, v);
            orc_rope(q, nq, d, P, cfg->theta);
            orc_rope(k, nkv, d, P, cfg->theta);
            for (int32_t g = 0; g < nkv; ++g) {
                size_t base = ((((size_t)l * batch + b) * nkv + g) * (size_t)max_ctx + P) * d;
                for (int32_t j = 0; j < d; ++j) {
                    k_cache[base + j] = orc_f64_to_bf16(k[(size_t)g * d + j]);
                    v_cache[base + j] = orc_f64_to_bf16(v[(size_t)g * d + j]);
                }
            }
            for (int32_t i = 0; i < nq; ++i) {
                int32_t g = i / grp;
                size_t base = (((size_t)l * batch + b) * nkv + g) * (size_t)max_ctx * d;
                orc_attention_head(q + (size_t)i * d, k_cache + base, v_cache + base, d, P + 1,
                                   kv_round ? NULL : k + (size_t)g * d, kv_round ? NULL : v + (size_t)g * d,
                                   a + (size_t)i * d);
            }
            orc_gemv(W->wo, h, nq * d, a, t);
            for (int32_t i = 0; i < h; ++i) x[i] += t[i];
            /* feed-forward block */
            orc_rmsnorm(x, W->ffn_norm, h, cfg->eps, xn);
            if (cfg->n_experts == 0) {
                swiglu(W->w_gate, W->w_up, W->w_down, h, cfg->ffn, xn, t);
                for (int32_t i = 0; i < h; ++i) x[i] += t[i];
            } else {
                const int32_t E = cfg->n_experts, K = cfg->top_k, fe = cfg->expert_ffn;
                double *rl = (double *)malloc(sizeof(double) * (size_t)E);
                int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
                double *wt = (double *)malloc(sizeof(double) * (size_t)K);
                orc_gemv(W->router, E, h, xn, rl);
                orc_topk_softmax(rl, E, K, ids, wt);
                if (router_out)
                    for (int32_t e = 0; e < E; ++e) router_out[((size_t)l * batch + b) * E + e] = rl[e];
                double *acc = (double *)calloc((size_t)h, sizeof(double));
                for (int32_t j = 0; j < K; ++j) {
                    size_t e = (size_t)ids[j];
                    swiglu(W->exp_gate + e * fe * h, W->exp_up + e * fe * h, W->exp_down + e * h * fe, h, fe, xn, t);
                    for (int32_t i = 0; i < h; ++i) acc[i] += wt[j] * t[i];
                    if (expert_ids) expert_ids[((size_t)l * batch + b) * K + j] = ids[j];
                }
                for (int32_t i = 0; i < h; ++i) x[i] += acc[i];
                free(acc);
                free(rl);
                free(ids);
                free(wt);
            }
            if (layer_out)
                for (int32_t i = 0; i < h; ++i) layer_out[((size_t)l * batch + b) * h + i] = x[i];
        }
        for (int32_t i = 0; i < h; ++i) hidden_out[(size_t)b * h + i] = x[i];
        orc_rmsnorm(x, final_norm, h, cfg->eps, xn);
        double *lg = logits + (size_t)b * cfg->vocab;
        orc_gemv(lm_head, cfg->vocab, h, xn, lg);
        next[b] = orc_argmax_f32(lg, cfg->vocab);
    }
    free(x);
    free(xn);
    free(q);
    free(k);
    free(v);
    free(a);
    free(t);
    return 0;
}
