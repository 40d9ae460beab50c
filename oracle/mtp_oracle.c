/*
 * mtp_oracle.c -- plain CPU reference of the MTP draft chain and verify step.
 *
 * TEST INFRASTRUCTURE ONLY (see mtp_oracle.h).  Every function follows the
 * pages' statement of the method, in the order and notation they use, with no
 * blocking, fusion or reordering: loops run in natural index order and
 * accumulate in double.  OpenMP only runs independent (row, sequence, kv head)
 * units side by side; each unit's arithmetic is the same at any thread count.
 *
 * Sources (page title, section):
 *   [G4]  "Gemma 4 MTP -- Multi-Token Prediction speculative decoding":
 *         s.1 (what MTP is), s.3 (pre/post projection shapes), s.4 (per-step
 *         graph), s.5 (KV sharing and the single mask), s.6 (step positions),
 *         s.8 (h_idx rule).
 *   [MTP] "MTP decoding (--mtp)": intro and "How it is wired" (greedy
 *         acceptance of the longest argmax-matching prefix).
 *   [AUD] "opus-mtp-turbo: Track 1 report": s.4 (exact temp>0 speculative
 *         sampling after Leviathan et al. 2023 s.2.3; sampling chain order
 *         top-k, penalties over history + input[0..i], temp, min-p, top-p).
 *   [FUS] "Fused NextN draft graph": on-device argmax -> embed -> next step.
 *   SplitMix64: Steele, Lea & Flood, "Fast splittable pseudorandom number
 *         generators", OOPSLA 2014 (mixing function and golden-gamma step).
 */
#include "mtp_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* element access: every stored format widens exactly to double              */
/* ------------------------------------------------------------------------ */
static double half_to_double(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 31, mant = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)mant, -24);
    else if (e == 31) v = mant ? NAN : INFINITY;
    else v = ldexp((double)(mant | 1024), e - 25);
    return sign ? -v : v;
}

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Element (row, col) of a row-major [rows, ncols] matrix.  Q8_0 ("Q8_0
   block: 32 int8 values plus one fp16 scale"): value = fp16(d) * q. */
double orc_load(const void *base, int32_t dtype, int64_t row, int64_t col, int64_t ncols) {
    switch (dtype) {
    case ORC_F32: return (double)((const float *)base)[row * ncols + col];
    case ORC_BF16: return bf16_to_double(((const uint16_t *)base)[row * ncols + col]);
    case ORC_Q8_0: {
        const uint8_t *blk = (const uint8_t *)base + (row * (ncols / 32) + col / 32) * 34;
        double d = half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
        return d * (double)(int8_t)blk[2 + col % 32];
    }
    }
    return NAN;
}

static double kv_load(const orc_model *m, const orc_kv *kv, const void *base, int64_t cell, int32_t kvh,
                      int32_t i) {
    return orc_load(base, m->kv_dtype, 0, cell * kv->cell_stride + (int64_t)kvh * m->head_dim + i, 0);
}

/* ------------------------------------------------------------------------ */
/* building blocks                                                           */
/* ------------------------------------------------------------------------ */
/* RMSNorm with gain: y = x / sqrt(mean(x^2) + eps) * g  ([G4] s.4 block) */
void orc_rmsnorm(int32_t n, const double *x, const float *g, double eps, double *y) {
    double ss = 0.0;
    for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / n + eps);
    for (int32_t i = 0; i < n; ++i) y[i] = x[i] * r * (double)g[i];
}

/* Rotary position embedding, half-split pairing (i, i + hd/2), frequency
   theta^(-2i/hd), applied to the query at the step position ([G4] s.4:
   "Q-norm -> RoPE"; s.6: step k runs at attn_pos + 1 + k). */
void orc_rope(int32_t hd, int64_t pos, double theta, const double *x, double *y) {
    int32_t half = hd / 2;
    for (int32_t i = 0; i < half; ++i) {
        double freq = pow(theta, -2.0 * (double)i / (double)hd);
        double ang = (double)pos * freq;
        double c = cos(ang), s = sin(ang);
        double a = x[i], b = x[i + half];
        y[i] = a * c - b * s;
        y[i + half] = a * s + b * c;
    }
}

static double silu(double u) { return u / (1.0 + exp(-u)); }

/* y[s][r] = sum_c W[r][c] * x[s][c] for all sequences; each row of W is
   widened once and dotted with every sequence's vector in column order. */
static void gemv_batch(const void *W, int32_t dtype, int64_t rows, int64_t cols, int32_t S, const double *x,
                       int64_t xstride, double *y, int64_t ystride) {
#pragma omp parallel
    {
        double *wrow = (double *)malloc(sizeof(double) * (size_t)cols);
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            for (int64_t c = 0; c < cols; ++c) wrow[c] = orc_load(W, dtype, r, c, cols);
            for (int32_t s = 0; s < S; ++s) {
                const double *xs = x + (int64_t)s * xstride;
                double acc = 0.0;
                for (int64_t c = 0; c < cols; ++c) acc += wrow[c] * xs[c];
                y[(int64_t)s * ystride + r] = acc;
            }
        }
        free(wrow);
    }
}

/* Cross-attention of the g query heads sharing kv head kvh into one KV source
   of the target ([G4] s.1 twist 2, s.4 "Cross-attention", s.5): the drafter
   owns no KV, reads K and V (V from its own slot, never from the rotated K),
   and its mask admits every position <= attn_pos.  A sliding-window source
   holds position p at ring cell p mod n_cells and admits the last swa_window
   positions up to attn_pos.  o_h = sum_c softmax_c(scale * q_h . K_c) V_c. */
int64_t orc_visible_cells(const orc_model *m, const orc_seq *seq, int32_t src, int64_t *cells, int64_t cap) {
    const orc_kv *kv = &seq->src[src];
    const int64_t hi = seq->attn_pos;
    int64_t n = 0;
    if (hi < 0 || !kv->k || !kv->v) return -1;
    if (src == ORC_SRC_FULL) {
        if (hi >= kv->n_cells) return -2;
        for (int64_t p = 0; p <= hi; ++p) {
            if (n >= cap) return -3;
            cells[n++] = p;
        }
    } else if (src == ORC_SRC_SWA) {
        if (m->swa_window <= 0 || kv->n_cells < m->swa_window) return -2;
        int64_t lo = hi - m->swa_window + 1;
        if (lo < 0) lo = 0;
        for (int64_t p = lo; p <= hi; ++p) {
            if (n >= cap) return -3;
            cells[n++] = p % kv->n_cells;
        }
    } else if (src == ORC_SRC_SINK_WINDOW) {
        /* the draft attention's id list [0 .. min(sink, first) - 1] ++
           [first .. cell0], first moved up to the valid run's start */
        if (m->sw_window <= 0 || m->sw_sink < 0 || hi >= kv->n_cells) return -2;
        int64_t first = hi - m->sw_window + 1;
        if (first < seq->run_lo) first = seq->run_lo;
        if (first < 0) first = 0;
        if (first > hi) return -2;
        const int64_t ns = m->sw_sink < first ? m->sw_sink : first;
        for (int64_t p = 0; p < ns; ++p) {
            if (n >= cap) return -3;
            cells[n++] = p;
        }
        for (int64_t p = first; p <= hi; ++p) {
            if (n >= cap) return -3;
            cells[n++] = p;
        }
    } else {
        return -1;
    }
    return n;
}

int orc_attend_group(const orc_model *m, const orc_seq *seq, int32_t src, int32_t kvh, const double *q_group,
                     double *o_group) {
    const orc_kv *kv = &seq->src[src];
    const int32_t hd = m->head_dim, g = m->n_head_q / m->n_head_kv;
    const int64_t cap = (int64_t)seq->attn_pos + 1;
    if (cap <= 0) return -1;
    int64_t *cells = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
    if (!cells) return -4;
    const int64_t n = orc_visible_cells(m, seq, src, cells, cap);
    if (n <= 0) {
        free(cells);
        return n < 0 ? (int)n : -2;
    }
    double *sc = (double *)malloc(sizeof(double) * (size_t)(n * g));
    if (!sc) { free(cells); return -4; }
    for (int64_t c = 0; c < n; ++c)
        for (int32_t j = 0; j < g; ++j) {
            double dot = 0.0;
            for (int32_t i = 0; i < hd; ++i) dot += q_group[j * hd + i] * kv_load(m, kv, kv->k, cells[c], kvh, i);
            sc[j * n + c] = dot * m->attn_scale;
        }
    for (int32_t j = 0; j < g; ++j) {
        double mx = -INFINITY;
        for (int64_t c = 0; c < n; ++c) mx = fmax(mx, sc[j * n + c]);
        double den = 0.0;
        for (int64_t c = 0; c < n; ++c) {
            sc[j * n + c] = exp(sc[j * n + c] - mx);
            den += sc[j * n + c];
        }
        for (int32_t i = 0; i < hd; ++i) o_group[j * hd + i] = 0.0;
        for (int64_t c = 0; c < n; ++c) {
            const double wgt = sc[j * n + c];
            for (int32_t i = 0; i < hd; ++i) o_group[j * hd + i] += wgt * kv_load(m, kv, kv->v, cells[c], kvh, i);
        }
        for (int32_t i = 0; i < hd; ++i) o_group[j * hd + i] /= den;
    }
    free(sc);
    free(cells);
    return 0;
}

/* Greedy argmax over an fp32 logit row, lowest index on ties ([G4] s.4
   "In-graph greedy argmax").  margin = best - second best. */
int32_t orc_argmax_f32(int64_t n, const float *z, double *margin) {
    int64_t best = 0;
    double second = -INFINITY;
    for (int64_t t = 1; t < n; ++t) {
        if (z[t] > z[best]) {
            second = z[best];
            best = t;
        } else if ((double)z[t] > second) {
            second = z[t];
        }
    }
    if (margin) *margin = (n > 1) ? (double)z[best] - second : INFINITY;
    return (int32_t)best;
}

/* Draft confidence ("MTP decoding", section "Stopping early when the head is
   unsure"; "Fused NextN draft graph", risks: the per-step softmax maximum
   read back beside the argmax).  The largest softmax probability is
   exp(max - max) / sum exp(z - max) = 1 / sum exp(z - max). */
double orc_confidence(int64_t n, const float *z) {
    double m = -INFINITY;
    for (int64_t t = 0; t < n; ++t)
        if ((double)z[t] > m) m = z[t];
    double sum = 0.0;
    for (int64_t t = 0; t < n; ++t) sum += exp((double)z[t] - m);
    return 1.0 / sum;
}

/* p_min trim ("MTP decoding", "Stopping early ...": drafting stops as soon
   as the confidence falls below p_min; at 0 it never stops; the step that
   falls below is not proposed).  The chain itself always runs every step
   (one captured launch); the trim is applied to what it returns. */
int orc_pmin_trim(int32_t n_seq, int32_t n_steps, const double *conf, double p_min, double tol, int32_t *drafts,
                  int32_t *out_n_keep, int32_t *out_near) {
    if (n_seq <= 0 || n_steps <= 0 || !conf || !drafts || !out_n_keep) return -1;
    for (int32_t s = 0; s < n_seq; ++s) {
        int32_t keep = n_steps, near = 0;
        for (int32_t k = 0; k < n_steps; ++k) {
            const double c = conf[(int64_t)s * n_steps + k];
            if (fabs(c - p_min) <= tol) near = 1;
            if (c < p_min) {
                keep = k;
                break;
            }
        }
        for (int32_t k = keep; k < n_steps; ++k) drafts[(int64_t)s * n_steps + k] = -1;
        out_n_keep[s] = keep;
        if (out_near) out_near[s] = near;
    }
    return 0;
}

/* Centroid / ordered-embeddings LM head ("Gemma 4 MTP" s.3): steps 1-5 of
   the page, in its order.  The top-k choice is taken on fp32-rounded
   centroid logits (the precision the GPU decides in). */
double orc_centroid_logits(const orc_model *m, const orc_weights *w, const double *f, float *z_out) {
    const int32_t d = m->d_model, V = m->n_vocab, nc = m->n_centroids, k = m->centroid_top_k;
    const int32_t vsc = V / nc;
    float *cl = malloc(sizeof(float) * (size_t)nc);
    char *taken = calloc((size_t)nc, 1);
    if (!cl || !taken) { free(cl); free(taken); return -1.0; }
    /* 1. centroid logits */
    for (int32_t c = 0; c < nc; ++c) {
        double acc = 0.0;
        for (int32_t j = 0; j < d; ++j) acc += orc_load(w->centroids, m->w_dtype, c, j, d) * f[j];
        cl[c] = (float)acc;
    }
    /* 5 (prefill). the full row the verifier expects */
    for (int32_t t = 0; t < V; ++t) z_out[t] = -1e30f;
    double boundary = INFINITY;
    float last = 0.0f;
    for (int32_t i = 0; i < k; ++i) {
        /* 2. next best centroid: largest logit, lowest id among equals */
        int32_t best = -1;
        for (int32_t c = 0; c < nc; ++c)
            if (!taken[c] && (best < 0 || cl[c] > cl[best])) best = c;
        taken[best] = 1;
        last = cl[best];
        /* 3. its candidate token ids; 4. their logits E[t] . f */
        for (int32_t r = 0; r < vsc; ++r) {
            const int32_t t = w->token_ordering[(int64_t)best * vsc + r];
            double acc = 0.0;
            for (int32_t j = 0; j < d; ++j) acc += orc_load(w->head, m->head_dtype, t, j, d) * f[j];
            z_out[t] = (float)acc;
        }
    }
    for (int32_t c = 0; c < nc; ++c)
        if (!taken[c] && (double)last - (double)cl[c] < boundary) boundary = (double)last - (double)cl[c];
    free(cl);
    free(taken);
    return boundary;
}

/* ------------------------------------------------------------------------ */
/* draft chain ([G4] s.4 steps 1-8, s.6 positions; [FUS] on-device chain)    */
/* ------------------------------------------------------------------------ */
static int check_model(const orc_model *m, const orc_weights *w) {
    if (!m || !w) return -1;
    if (m->n_centroids < 0) return -2;
    if (m->n_centroids > 0) {
        if (m->n_vocab % m->n_centroids || m->centroid_top_k < 1 || m->centroid_top_k > m->n_centroids) return -2;
        if (!w->centroids || !w->token_ordering) return -1;
        for (int32_t t = 0; t < m->n_vocab; ++t)
            if (w->token_ordering[t] < 0 || w->token_ordering[t] >= m->n_vocab) return -2;
    }
    if (m->d_model <= 0 || m->d_hprev <= 0 || m->n_blocks <= 0 || m->n_blocks > ORC_MAX_BLOCKS) return -2;
    if (m->n_head_kv <= 0 || m->n_head_q % m->n_head_kv || m->head_dim <= 0 || m->head_dim % 2) return -2;
    if (m->head_dtype == ORC_Q8_0 && m->d_model % 32) return -2;
    if (!w->w_pre || !w->w_post || !w->head || !w->g_final) return -1;
    for (int l = 0; l < m->n_blocks; ++l)
        if (!w->g_attn[l] || !w->w_q[l] || !w->g_q[l] || !w->w_o[l] || !w->g_mlp[l] || !w->w_up[l] || !w->w_down[l])
            return -1;
    return 0;
}

int orc_draft_block(const orc_model *m, const orc_weights *w, int32_t n_seq, const orc_seq *seqs,
                    const int32_t *last_tok, const float *h_prev, int32_t n_steps, int32_t *out_drafts,
                    float *out_h_last, float *out_logits, double *out_margin, double *out_conf) {
    int rc = check_model(m, w);
    if (rc) return rc;
    if (n_seq <= 0 || n_steps <= 0 || !seqs || !last_tok || !h_prev || !out_drafts) return -1;
    const int32_t d = m->d_model, dh = m->d_hprev, Hq = m->n_head_q, Hkv = m->n_head_kv, hd = m->head_dim;
    const int32_t F = m->d_ff, V = m->n_vocab, qd = Hq * hd, g = Hq / Hkv, din = d + dh;
    const int32_t S = n_seq;
    for (int32_t s = 0; s < S; ++s)
        if (last_tok[s] < 0 || last_tok[s] >= V) return -1;

    double *in = calloc((size_t)S * din, sizeof(double));
    double *x = calloc((size_t)S * d, sizeof(double));
    double *a = calloc((size_t)S * d, sizeof(double));
    double *tmp = calloc((size_t)S * d, sizeof(double));
    double *q = calloc((size_t)S * qd, sizeof(double));
    double *qn = calloc((size_t)S * qd, sizeof(double));
    double *o = calloc((size_t)S * qd, sizeof(double));
    double *u = calloc((size_t)S * F, sizeof(double));
    double *f = calloc((size_t)S * d, sizeof(double));
    double *h = calloc((size_t)S * dh, sizeof(double));
    double *zd = calloc((size_t)S * V, sizeof(double));
    float *zf = calloc((size_t)V, sizeof(float));
    int32_t *tok = calloc((size_t)S, sizeof(int32_t));
    int bad = !in || !x || !a || !tmp || !q || !qn || !o || !u || !f || !h || !zd || !zf || !tok;
    int err = 0;
    if (bad) { err = -4; goto done; }

    for (int32_t s = 0; s < S; ++s) {
        tok[s] = last_tok[s];
        for (int32_t j = 0; j < dh; ++j) h[(int64_t)s * dh + j] = (double)h_prev[(int64_t)s * dh + j];
    }

    for (int32_t k = 0; k < n_steps; ++k) {
        /* 1. input: target token embedding (tied head rows) scaled by
              embed_scale, concatenated with h_prev, projected back to d
              ([G4] s.4 steps 2-3; s.3 pre_projection) */
        for (int32_t s = 0; s < S; ++s) {
            double *is = in + (int64_t)s * din;
            for (int32_t j = 0; j < d; ++j) is[j] = m->embed_scale * orc_load(w->head, m->head_dtype, tok[s], j, d);
            for (int32_t j = 0; j < dh; ++j) is[d + j] = h[(int64_t)s * dh + j];
        }
        gemv_batch(w->w_pre, m->w_dtype, d, din, S, in, din, x, d);

        /* 2. transformer blocks ([G4] s.4 step 4) */
        for (int32_t l = 0; l < m->n_blocks; ++l) {
            for (int32_t s = 0; s < S; ++s) orc_rmsnorm(d, x + (int64_t)s * d, w->g_attn[l], m->rms_eps, a + (int64_t)s * d);
            gemv_batch(w->w_q[l], m->w_dtype, qd, d, S, a, d, q, qd);
            for (int32_t s = 0; s < S; ++s) {
                int64_t pos = (int64_t)seqs[s].pos0 + k;
                for (int32_t hh = 0; hh < Hq; ++hh) {
                    double *qh = q + (int64_t)s * qd + (int64_t)hh * hd;
                    double *tmph = qn + (int64_t)s * qd + (int64_t)hh * hd;
                    orc_rmsnorm(hd, qh, w->g_q[l], m->rms_eps, tmph);
                    orc_rope(hd, pos, m->rope_theta, tmph, qh);
                }
            }
            int32_t src = m->block_src[l];
#pragma omp parallel for collapse(2) schedule(dynamic)
            for (int32_t s = 0; s < S; ++s)
                for (int32_t j = 0; j < Hkv; ++j) {
                    int r = orc_attend_group(m, &seqs[s], src, j, q + (int64_t)s * qd + (int64_t)j * g * hd,
                                             o + (int64_t)s * qd + (int64_t)j * g * hd);
                    if (r) {
#pragma omp atomic write
                        err = r;
                    }
                }
            if (err) goto done;
            gemv_batch(w->w_o[l], m->w_dtype, d, qd, S, o, qd, tmp, d);
            for (int64_t i = 0; i < (int64_t)S * d; ++i) x[i] += tmp[i];
            for (int32_t s = 0; s < S; ++s) orc_rmsnorm(d, x + (int64_t)s * d, w->g_mlp[l], m->rms_eps, a + (int64_t)s * d);
            gemv_batch(w->w_up[l], m->w_dtype, F, d, S, a, d, u, F);
            for (int64_t i = 0; i < (int64_t)S * F; ++i) u[i] = silu(u[i]);
            gemv_batch(w->w_down[l], m->w_dtype, d, F, S, u, F, tmp, d);
            for (int64_t i = 0; i < (int64_t)S * d; ++i) x[i] += tmp[i];
        }

        /* 3. final norm; tied LM head over the full vocabulary; greedy
              argmax; post-projection gives the next step's h_prev
              ([G4] s.4 steps 5, 6, 8) */
        for (int32_t s = 0; s < S; ++s) orc_rmsnorm(d, x + (int64_t)s * d, w->g_final, m->rms_eps, f + (int64_t)s * d);
        if (m->n_centroids == 0) gemv_batch(w->head, m->head_dtype, V, d, S, f, d, zd, V);
        double *hn = calloc((size_t)S * dh, sizeof(double));
        if (!hn) { err = -4; goto done; }
        gemv_batch(w->w_post, m->w_dtype, dh, d, S, f, d, hn, dh);
        for (int32_t s = 0; s < S; ++s) {
            double cmargin = INFINITY;
            if (m->n_centroids == 0) {
                for (int32_t t = 0; t < V; ++t) zf[t] = (float)zd[(int64_t)s * V + t];
            } else {
                cmargin = orc_centroid_logits(m, w, f + (int64_t)s * d, zf);
                if (cmargin < 0) { err = -4; free(hn); goto done; }
            }
            double margin;
            int32_t nt = orc_argmax_f32(V, zf, &margin);
            if (cmargin < margin) margin = cmargin;   /* a near tie at either decision */
            if (out_logits) memcpy(out_logits + ((int64_t)s * n_steps + k) * V, zf, sizeof(float) * (size_t)V);
            if (out_margin) out_margin[(int64_t)s * n_steps + k] = margin;
            if (out_conf) out_conf[(int64_t)s * n_steps + k] = orc_confidence(V, zf);
            out_drafts[(int64_t)s * n_steps + k] = nt;
            tok[s] = nt;   /* the argmax feeds the next step ([FUS] chain) */
            /* h is handed over as F32 ([G4] s.4 input inp_h_prev F32) */
            for (int32_t j = 0; j < dh; ++j) h[(int64_t)s * dh + j] = (double)(float)hn[(int64_t)s * dh + j];
        }
        free(hn);
    }
    if (out_h_last)
        for (int64_t i = 0; i < (int64_t)S * dh; ++i) out_h_last[i] = (float)h[i];

done:
    free(in); free(x); free(a); free(tmp); free(q); free(qn); free(o); free(u); free(f); free(h); free(zd);
    free(zf); free(tok);
    return err;
}

/* ------------------------------------------------------------------------ */
/* greedy verify ([MTP] "How it is wired"; [G4] s.8)                         */
/* ------------------------------------------------------------------------ */
/* rows 0..N of the target's logits; t_i = argmax row i; accept the longest
   prefix of drafts with d_j == t_j; emit t_0..t_a (t_a is the free token from
   the first unverified row); n_accept = a is also the batch row that seeds
   the next round's h_prev.  Slots past a hold -1. */
int orc_verify_greedy(int32_t n_seq, int32_t n_draft, int32_t n_vocab, const float *logits, const int32_t *drafts,
                      int32_t *out_tokens, int32_t *out_n_accept) {
    if (n_seq <= 0 || n_draft < 0 || n_vocab <= 0 || !logits || (n_draft && !drafts) || !out_tokens || !out_n_accept)
        return -1;
    const int32_t R = n_draft + 1;
    for (int32_t s = 0; s < n_seq; ++s) {
        int32_t a = 0;
        while (a < n_draft &&
               drafts[(int64_t)s * n_draft + a] == orc_argmax_f32(n_vocab, logits + ((int64_t)s * R + a) * n_vocab, NULL))
            ++a;
        for (int32_t i = 0; i < R; ++i)
            out_tokens[(int64_t)s * R + i] =
                (i <= a) ? orc_argmax_f32(n_vocab, logits + ((int64_t)s * R + i) * n_vocab, NULL) : -1;
        out_n_accept[s] = a;
    }
    return 0;
}

/* The target's logit rows from its final hidden rows ("MTP decoding", "Why
   a wider decode can be faster": the 1 + N verify rows meet the target's head
   weights in one pass).  Row r is the final hidden state h; f = rmsnorm(h; g)
   (f = h when g is NULL: the caller already normed it), z = W_head f in fp64,
   rounded to fp32 as the target's logit row is.  Returns a malloc'd
   [rows, n_vocab] array, or NULL when out of memory. */
static float *hidden_logits(int64_t rows, int32_t n_vocab, int32_t d, const float *hidden, const void *head,
                            int32_t head_dtype, const float *g, double eps) {
    double *f = (double *)malloc(sizeof(double) * (size_t)(rows * d));
    double *z = (double *)malloc(sizeof(double) * (size_t)(rows * n_vocab));
    float *z32 = (float *)malloc(sizeof(float) * (size_t)(rows * n_vocab));
    if (!f || !z || !z32) {
        free(f); free(z); free(z32);
        return NULL;
    }
    for (int64_t r = 0; r < rows; ++r) {
        double *fr = f + r * d;
        for (int32_t c = 0; c < d; ++c) fr[c] = (double)hidden[r * d + c];
        if (g) orc_rmsnorm(d, fr, g, eps, fr);
    }
    gemv_batch(head, head_dtype, n_vocab, d, (int32_t)rows, f, d, z, n_vocab);
    for (int64_t i = 0; i < rows * n_vocab; ++i) z32[i] = (float)z[i];
    free(f); free(z);
    return z32;
}

/* Hidden-state greedy verify: the logit rows of hidden_logits, then the
   greedy acceptance of orc_verify_greedy.  out_margin[row] (optional) is the
   row's top-2 gap. */
int orc_verify_greedy_hidden(int32_t n_seq, int32_t n_draft, int32_t n_vocab, int32_t d, const float *hidden,
                             const void *head, int32_t head_dtype, const float *g, double eps,
                             const int32_t *drafts, int32_t *out_tokens, int32_t *out_n_accept,
                             double *out_margin) {
    if (n_seq <= 0 || n_draft < 0 || n_vocab <= 0 || d <= 0 || !hidden || !head || (n_draft && !drafts) ||
        !out_tokens || !out_n_accept)
        return -1;
    if (head_dtype == ORC_Q8_0 && d % 32) return -1;
    const int64_t rows = (int64_t)n_seq * (n_draft + 1);
    float *z32 = hidden_logits(rows, n_vocab, d, hidden, head, head_dtype, g, eps);
    if (!z32) return -4;
    if (out_margin)
        for (int64_t r = 0; r < rows; ++r) orc_argmax_f32(n_vocab, z32 + r * n_vocab, &out_margin[r]);
    const int rc = orc_verify_greedy(n_seq, n_draft, n_vocab, z32, drafts, out_tokens, out_n_accept);
    free(z32);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* counter-based uniforms (SplitMix64)                                       */
/* ------------------------------------------------------------------------ */
/* one SplitMix64 step: advance the state by the golden gamma, then apply the
   64-bit finaliser (shift-xor-multiply, 30/27/31) */
uint64_t orc_splitmix64_next(uint64_t *state) {
    uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* key derivation: start from seed, then fold in each coordinate with xor and
   take one SplitMix64 step per coordinate */
uint64_t orc_rng_u64(uint64_t seed, uint64_t s, uint64_t round, uint64_t i, uint64_t stream, uint64_t t) {
    uint64_t st = seed;
    uint64_t h = orc_splitmix64_next(&st);
    const uint64_t coord[5] = {s, round, i, stream, t};
    for (int c = 0; c < 5; ++c) {
        st = h ^ coord[c];
        h = orc_splitmix64_next(&st);
    }
    return h;
}

/* uniform in (0,1), exactly representable in fp32: ((h >> 41) + 1/2) / 2^23 */
float orc_uniform(uint64_t seed, uint64_t s, uint64_t round, uint64_t i, uint64_t stream, uint64_t t) {
    uint64_t h = orc_rng_u64(seed, s, round, i, stream, t);
    return (float)(((double)(h >> 41) + 0.5) * (1.0 / 8388608.0));
}

/* ------------------------------------------------------------------------ */
/* sampling chain ([AUD] s.4: top-k, penalties over history + input[0..i],   */
/* temperature, min-p, top-p)                                                */
/* ------------------------------------------------------------------------ */
typedef struct { double key; int32_t id; } kv_pair;

static int cmp_desc(const void *pa, const void *pb) {
    const kv_pair *a = (const kv_pair *)pa, *b = (const kv_pair *)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->id > b->id) - (a->id < b->id);   /* ties: lower id first */
}

int orc_sample_dist(int32_t V, const float *z, const int32_t *ctx, int32_t n_ctx, const orc_sampler *sp,
                    double *p_out, int32_t *flags) {
    if (V <= 0 || !z || !sp || !p_out || sp->temp <= 0.0 || (n_ctx > 0 && !ctx)) return -1;
    double *zz = (double *)malloc(sizeof(double) * (size_t)V);
    char *keep = (char *)malloc((size_t)V);
    int32_t *cnt = (int32_t *)calloc((size_t)V, sizeof(int32_t));
    kv_pair *srt = (kv_pair *)malloc(sizeof(kv_pair) * (size_t)V);
    int32_t fl = 0, n_keep = 0;
    if (!zz || !keep || !cnt || !srt) { free(zz); free(keep); free(cnt); free(srt); return -4; }
    for (int32_t t = 0; t < V; ++t) { zz[t] = z[t]; keep[t] = 1; }

    /* top-k on the raw logits (ties -> lower id) */
    if (sp->top_k > 0 && sp->top_k < V) {
        for (int32_t t = 0; t < V; ++t) { srt[t].key = z[t]; srt[t].id = t; }
        qsort(srt, (size_t)V, sizeof(kv_pair), cmp_desc);
        for (int32_t t = 0; t < V; ++t) keep[t] = 0;
        for (int32_t j = 0; j < sp->top_k; ++j) keep[srt[j].id] = 1;
        if (srt[sp->top_k - 1].key == srt[sp->top_k].key) fl |= ORC_NEAR_TOPK;
    }
    /* penalties, once per distinct context token: repetition (divide a
       positive logit, multiply a negative one), then presence and frequency */
    for (int32_t j = 0; j < n_ctx; ++j)
        if (ctx[j] >= 0 && ctx[j] < V) cnt[ctx[j]]++;
    for (int32_t t = 0; t < V; ++t) {
        if (!cnt[t]) continue;
        zz[t] = zz[t] > 0.0 ? zz[t] / sp->rep_penalty : zz[t] * sp->rep_penalty;
        zz[t] -= sp->presence_penalty + sp->freq_penalty * (double)cnt[t];
    }
    /* temperature and softmax over the kept set; e_t = pi_t / max pi */
    double mx = -INFINITY;
    for (int32_t t = 0; t < V; ++t) {
        zz[t] /= sp->temp;
        if (keep[t]) mx = fmax(mx, zz[t]);
    }
    for (int32_t t = 0; t < V; ++t) zz[t] = keep[t] ? exp(zz[t] - mx) : 0.0;
    /* min-p: keep pi_t >= min_p * max pi, decided in fp32 */
    if (sp->min_p > 0.0) {
        for (int32_t t = 0; t < V; ++t) {
            if (!keep[t]) continue;
            if (fabs(zz[t] - sp->min_p) <= 1e-5 * sp->min_p) fl |= ORC_NEAR_MINP;
            if (!((float)zz[t] >= (float)sp->min_p)) { keep[t] = 0; zz[t] = 0.0; }
        }
    }
    double den = 0.0;
    for (int32_t t = 0; t < V; ++t) den += zz[t];
    /* top-p: by probability, descending (ties -> lower id), keep the shortest
       prefix whose cumulative probability reaches top_p, crossing token
       included; decided in fp32 */
    if (sp->top_p < 1.0) {
        int32_t n = 0;
        for (int32_t t = 0; t < V; ++t)
            if (keep[t]) { srt[n].key = zz[t]; srt[n].id = t; ++n; }
        qsort(srt, (size_t)n, sizeof(kv_pair), cmp_desc);
        double cum = 0.0;
        int32_t cut = n;
        for (int32_t j = 0; j < n; ++j) {
            double prev = cum;
            cum += srt[j].key / den;
            if ((float)cum >= (float)sp->top_p) {
                if (fabs(cum - sp->top_p) <= 1e-5 || fabs(prev - sp->top_p) <= 1e-5) fl |= ORC_NEAR_TOPP;
                cut = j + 1;
                break;
            }
        }
        for (int32_t j = cut; j < n; ++j) { keep[srt[j].id] = 0; zz[srt[j].id] = 0.0; }
        den = 0.0;
        for (int32_t t = 0; t < V; ++t) den += zz[t];
    }
    for (int32_t t = 0; t < V; ++t) {
        p_out[t] = keep[t] ? zz[t] / den : 0.0;
        n_keep += keep[t] ? 1 : 0;
    }
    if (flags) *flags |= fl;
    free(zz); free(keep); free(cnt); free(srt);
    return n_keep;
}

/* Gumbel-max draw from weights w >= 0 (exact sampling proportional to w):
   argmax_t ln w_t - ln(-ln U_t) over w_t > 0, keys rounded to fp32, lowest id
   on ties.  err_t bounds the fp32 rounding of key t; the draw is flagged when
   the two best keys are closer than their bounds. */
static int32_t gumbel_pick(int32_t V, const double *w, const double *wsum_for_err, uint64_t seed, uint64_t s,
                           uint64_t round, uint64_t i, uint64_t stream, int32_t *flags) {
    int32_t best = -1;
    float bestk = -INFINITY, secondk = -INFINITY;
    double besterr = 0.0, seconderr = 0.0;
    for (int32_t t = 0; t < V; ++t) {
        if (!(w[t] > 0.0)) continue;
        double uu = (double)orc_uniform(seed, s, round, i, stream, (uint64_t)t);
        double gk = -log(-log(uu));
        double key = log(w[t]) + gk;
        double err = 4e-6 * (wsum_for_err[t] / w[t]) + 4e-6 * (1.0 + fabs(gk) + fabs(log(w[t])));
        float kf = (float)key;
        if (best < 0 || kf > bestk) {
            secondk = bestk; seconderr = besterr;
            bestk = kf; besterr = err; best = t;
        } else if (kf > secondk) {
            secondk = kf; seconderr = err;
        }
    }
    if (flags && best >= 0 && isfinite(secondk) && (double)bestk - (double)secondk <= besterr + seconderr)
        *flags |= ORC_NEAR_GUMBEL;
    return best;
}

/* context of row i: the last penalty_last_n tokens of history ++ drafts[0..i) */
static int32_t row_ctx(const int32_t *hist, int32_t hlen, const int32_t *dr, int32_t i, int32_t last_n, int32_t *ctx) {
    int32_t total = hlen + i, start = (last_n > 0 && total > last_n) ? total - last_n : 0, n = 0;
    if (last_n == 0) return 0;
    for (int32_t j = start; j < total; ++j) ctx[n++] = (j < hlen) ? hist[j] : dr[j - hlen];
    return n;
}

/* Exact speculative sampling ([AUD] s.4, after Leviathan et al. 2023 s.2.3):
   for rows i < N accept draft d_i when u * q_i(d_i) < p_i(d_i) (probability
   min(1, p/q)); at the first rejection emit a sample of norm(max(p_i - q_i, 0))
   and stop; when all N are accepted emit a sample of p_N.  A NULL q means the
   drafts are deterministic (q one-hot at d_i): then the test is u < p_i(d_i)
   and the residual is p_i with d_i removed, the pages' exact statement. */
int orc_verify_sample(int32_t n_seq, int32_t n_draft, int32_t V, const float *p_logits, const float *q_logits,
                      const int32_t *drafts, const int32_t *history, int32_t history_stride,
                      const int32_t *history_len, const orc_sampler *sp, uint64_t round, int32_t *out_tokens,
                      int32_t *out_n_accept, int32_t *out_flags) {
    if (n_seq <= 0 || n_draft < 0 || V <= 0 || !p_logits || (n_draft && !drafts) || !sp || !out_tokens ||
        !out_n_accept)
        return -1;
    const int32_t N = n_draft, R = N + 1;
    int err = 0;
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)V);
        double *q = (double *)malloc(sizeof(double) * (size_t)V);
        double *r = (double *)malloc(sizeof(double) * (size_t)V);
        double *e = (double *)malloc(sizeof(double) * (size_t)V);
        int32_t *ctx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(sp->penalty_last_n > 0 ? sp->penalty_last_n : 1));
        if (!p || !q || !r || !e || !ctx) {
#pragma omp atomic write
            err = -4;
        }
#pragma omp for schedule(dynamic)
        for (int32_t s = 0; s < n_seq; ++s) {
            if (err) continue;
            const int32_t *hist = history ? history + (int64_t)s * history_stride : NULL;
            /* the boundary's contract: a history length reads as clamped to
               [0, history_stride] */
            int32_t hlen = history_len ? history_len[s] : 0;
            hlen = hlen < 0 ? 0 : (hlen > history_stride ? history_stride : hlen);
            const int32_t *dr = drafts ? drafts + (int64_t)s * N : NULL;
            int32_t fl = 0, a = N;
            for (int32_t j = 0; j < R; ++j) out_tokens[(int64_t)s * R + j] = -1;
            for (int32_t i = 0; i <= N; ++i) {
                int32_t nctx = row_ctx(hist, hlen, dr, i, sp->penalty_last_n, ctx);
                if (orc_sample_dist(V, p_logits + ((int64_t)s * R + i) * V, ctx, nctx, sp, p, &fl) < 0) {
#pragma omp atomic write
                    err = -1;
                    break;
                }
                if (i == N) {
                    for (int32_t t = 0; t < V; ++t) e[t] = p[t] + p[t];
                    out_tokens[(int64_t)s * R + N] = gumbel_pick(V, p, e, sp->seed, (uint64_t)s, round, (uint64_t)N,
                                                                 ORC_STREAM_BONUS, &fl);
                    break;
                }
                int32_t dtok = dr[i];
                if (q_logits) {
                    if (orc_sample_dist(V, q_logits + ((int64_t)s * N + i) * V, ctx, nctx, sp, q, &fl) < 0) {
#pragma omp atomic write
                        err = -1;
                        break;
                    }
                } else {
                    for (int32_t t = 0; t < V; ++t) q[t] = 0.0;
                    if (dtok >= 0 && dtok < V) q[dtok] = 1.0;
                }
                float pf = (dtok >= 0 && dtok < V) ? (float)p[dtok] : 0.0f;
                float qf = (dtok >= 0 && dtok < V) ? (float)q[dtok] : 0.0f;
                float u = orc_uniform(sp->seed, (uint64_t)s, round, (uint64_t)i, ORC_STREAM_ACCEPT, 0);
                double big = fmax((double)pf, (double)qf);
                if (fabs((double)u * qf - pf) < 1e-5 * big) fl |= ORC_NEAR_ACCEPT;
                if (u * qf < pf) {
                    out_tokens[(int64_t)s * R + i] = dtok;
                    continue;
                }
                for (int32_t t = 0; t < V; ++t) {
                    r[t] = p[t] - q[t] > 0.0 ? p[t] - q[t] : 0.0;
                    e[t] = p[t] + q[t];
                }
                out_tokens[(int64_t)s * R + i] =
                    gumbel_pick(V, r, e, sp->seed, (uint64_t)s, round, (uint64_t)i, ORC_STREAM_RESIDUAL, &fl);
                a = i;
                break;
            }
            out_n_accept[s] = a;
            if (out_flags) out_flags[s] = fl;
        }
        free(p); free(q); free(r); free(e); free(ctx);
    }
    return err;
}

/* Hidden-state sampling verify: the logit rows of hidden_logits, then the
   exact speculative sampling of orc_verify_sample on them. */
int orc_verify_sample_hidden(int32_t n_seq, int32_t n_draft, int32_t n_vocab, int32_t d, const float *hidden,
                             const void *head, int32_t head_dtype, const float *g, double eps,
                             const float *q_logits, const int32_t *drafts, const int32_t *history,
                             int32_t history_stride, const int32_t *history_len, const orc_sampler *sp,
                             uint64_t round, int32_t *out_tokens, int32_t *out_n_accept, int32_t *out_flags) {
    if (n_seq <= 0 || n_draft < 0 || n_vocab <= 0 || d <= 0 || !hidden || !head) return -1;
    if (head_dtype == ORC_Q8_0 && d % 32) return -1;
    float *z32 = hidden_logits((int64_t)n_seq * (n_draft + 1), n_vocab, d, hidden, head, head_dtype, g, eps);
    if (!z32) return -4;
    const int rc = orc_verify_sample(n_seq, n_draft, n_vocab, z32, q_logits, drafts, history, history_stride,
                                     history_len, sp, round, out_tokens, out_n_accept, out_flags);
    free(z32);
    return rc;
}

int orc_verify_greedy_match(int32_t n_seq, int32_t n_draft, int32_t V, const float *p_logits, const int32_t *drafts,
                            const int32_t *history, int32_t history_stride, const int32_t *history_len,
                            const orc_sampler *sp, uint64_t round, int32_t *out_tokens, int32_t *out_n_accept) {
    if (n_seq <= 0 || n_draft < 0 || V <= 0 || !p_logits || !sp || !out_tokens || !out_n_accept) return -1;
    const int32_t N = n_draft, R = N + 1;
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *e = (double *)malloc(sizeof(double) * (size_t)V);
    int32_t *ctx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(sp->penalty_last_n > 0 ? sp->penalty_last_n : 1));
    if (!p || !e || !ctx) { free(p); free(e); free(ctx); return -4; }
    for (int32_t s = 0; s < n_seq; ++s) {
        const int32_t *hist = history ? history + (int64_t)s * history_stride : NULL;
        const int32_t hlen = history_len ? history_len[s] : 0;
        const int32_t *dr = drafts + (int64_t)s * N;
        int32_t a = 0;
        while (a < N && dr[a] == orc_argmax_f32(V, p_logits + ((int64_t)s * R + a) * V, NULL)) ++a;
        for (int32_t j = 0; j < R; ++j) out_tokens[(int64_t)s * R + j] = (j < a) ? dr[j] : -1;
        int32_t nctx = row_ctx(hist, hlen, dr, a, sp->penalty_last_n, ctx);
        orc_sample_dist(V, p_logits + ((int64_t)s * R + a) * V, ctx, nctx, sp, p, NULL);
        for (int32_t t = 0; t < V; ++t) e[t] = p[t] + p[t];
        out_tokens[(int64_t)s * R + a] = gumbel_pick(V, p, e, sp->seed, (uint64_t)s, round, (uint64_t)a, ORC_STREAM_BONUS, NULL);
        out_n_accept[s] = a;
    }
    free(p); free(e); free(ctx);
    return 0;
}

int32_t orc_sample_row(int32_t V, const float *z, const int32_t *ctx, int32_t n_ctx, const orc_sampler *sp,
                       uint64_t s, uint64_t round, uint64_t i, uint64_t stream) {
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *e = (double *)malloc(sizeof(double) * (size_t)V);
    if (!p || !e) { free(p); free(e); return -4; }
    int32_t t = -1;
    if (orc_sample_dist(V, z, ctx, n_ctx, sp, p, NULL) > 0) {
        for (int32_t j = 0; j < V; ++j) e[j] = p[j] + p[j];
        t = gumbel_pick(V, p, e, sp->seed, s, round, i, stream, NULL);
    }
    free(p); free(e);
    return t;
}
