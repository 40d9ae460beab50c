/*
 * mtp_oracle.h -- plain, slow CPU reference of the MTP draft chain and verify.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this library; only the tests, the smoke check and the bench's cpu_baseline
 * leg do.  It shares no code or header with the GPU library.
 *
 * Arithmetic is IEEE double throughout, in natural index order, except where
 * the pages fix a storage precision: the hidden state handed from one draft
 * step to the next is F32 (the drafter's h_prev input, "Gemma 4 MTP" design
 * doc section 4, inputs of the one-token graph), and the logit row is F32 (the
 * t_logits row of the same section).  A decision that turns floating point
 * into an integer (argmax, sampling tests) is taken on fp32-rounded operands,
 * the precision the GPU kernels decide in.
 */
#ifndef MTP_ORACLE_H
#define MTP_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_Q8_0 = 2 };
enum { ORC_SRC_FULL = 0, ORC_SRC_SWA = 1, ORC_SRC_SINK_WINDOW = 2 };
enum { ORC_STREAM_ACCEPT = 0, ORC_STREAM_RESIDUAL = 1, ORC_STREAM_BONUS = 2 };
#define ORC_MAX_BLOCKS 8

typedef struct {
    int32_t d_model, d_hprev, n_blocks, n_head_q, n_head_kv, head_dim, d_ff, n_vocab;
    int32_t w_dtype, head_dtype, kv_dtype, swa_window;
    int32_t block_src[ORC_MAX_BLOCKS];
    double rms_eps, rope_theta, attn_scale, embed_scale;
    /* centroid ("ordered embeddings") LM head: 0 = dense tied head */
    int32_t n_centroids, centroid_top_k;
    /* sink + window source: window length and sink cells */
    int32_t sw_window, sw_sink;
} orc_model;

typedef struct {
    const void *w_pre, *w_post, *head;
    const float *g_final;
    const float *g_attn[ORC_MAX_BLOCKS];
    const void *w_q[ORC_MAX_BLOCKS];
    const float *g_q[ORC_MAX_BLOCKS];
    const void *w_o[ORC_MAX_BLOCKS];
    const float *g_mlp[ORC_MAX_BLOCKS];
    const void *w_up[ORC_MAX_BLOCKS], *w_down[ORC_MAX_BLOCKS];
    const void *centroids;          /* [n_centroids, d] (w_dtype), centroid head only */
    const int32_t *token_ordering;  /* [n_vocab], centroid head only */
} orc_weights;

typedef struct { const void *k, *v; int64_t n_cells, cell_stride; } orc_kv;
/* src[ORC_SRC_*]; run_lo = first cell of the valid run of a sink + window
   source (cells below it, outside the sink, are stale) */
typedef struct { orc_kv src[3]; int32_t attn_pos, pos0, run_lo; } orc_seq;

/* Cells a block attends to, in order; returns the count (<= cap) or < 0.
   full: 0..attn_pos.  SWA ring: positions max(0, attn_pos-W+1)..attn_pos at
   cell p mod n_cells.  sink + window ("opus-mtp-turbo" report s.2): first =
   max(attn_pos - W + 1, run_lo, 0), cells [0, min(sink, first)) ++
   [first, attn_pos]. */
int64_t orc_visible_cells(const orc_model *m, const orc_seq *seq, int32_t src, int64_t *cells, int64_t cap);

typedef struct {
    double temp, top_p, min_p, rep_penalty, presence_penalty, freq_penalty;
    int32_t top_k, penalty_last_n;
    uint64_t seed;
} orc_sampler;

/* flags written by the sampling routines (bitwise OR per sequence) */
enum {
    ORC_NEAR_MINP = 1,      /* a token's ratio to the row max lies within 1e-5 (rel.) of min_p */
    ORC_NEAR_TOPP = 2,      /* the top-p cumulative sum lies within 1e-5 of top_p at the cut */
    ORC_NEAR_ACCEPT = 4,    /* |u*q(d) - p(d)| < 1e-5 * max(p(d), q(d)) */
    ORC_NEAR_GUMBEL = 8,    /* the two best Gumbel keys lie within their rounding bound */
    ORC_NEAR_TOPK = 16      /* a tie straddles the top-k cut */
};

/* ---- pieces, exported so the tests can pin each one ---- */
double orc_load(const void *base, int32_t dtype, int64_t row, int64_t col, int64_t ncols);
void orc_rmsnorm(int32_t n, const double *x, const float *g, double eps, double *y);
void orc_rope(int32_t hd, int64_t pos, double theta, const double *x, double *y);
/* o[g*hd] for the g = Hq/Hkv query heads that share kv head kvh */
int orc_attend_group(const orc_model *m, const orc_seq *seq, int32_t src, int32_t kvh,
                     const double *q_group, double *o_group);
int32_t orc_argmax_f32(int64_t n, const float *z, double *margin);
uint64_t orc_splitmix64_next(uint64_t *state);
uint64_t orc_rng_u64(uint64_t seed, uint64_t s, uint64_t round, uint64_t i, uint64_t stream, uint64_t t);
float orc_uniform(uint64_t seed, uint64_t s, uint64_t round, uint64_t i, uint64_t stream, uint64_t t);

/* ---- the path ---- */
/* out_conf (nullable): per-step draft confidence [S, n_steps], see
   orc_confidence */
int orc_draft_block(const orc_model *m, const orc_weights *w, int32_t n_seq, const orc_seq *seqs,
                    const int32_t *last_tok, const float *h_prev, int32_t n_steps,
                    int32_t *out_drafts, float *out_h_last, float *out_logits, double *out_margin,
                    double *out_conf);

/* Centroid LM head of one final-normed vector f ("Gemma 4 MTP" s.3,
   centroid / ordered-embeddings head): centroid logits C f, the top_k
   centroids (ties -> lower id), their token lists ordering[c*vsc ..
   (c+1)*vsc) with vsc = V / n_centroids, candidate logits E[t] f, scattered
   into a full row z_out[V] prefilled with -1e30.  Returns the boundary
   margin of the top-k choice (k-th minus (k+1)-th centroid logit, fp32),
   +inf when every centroid is chosen. */
double orc_centroid_logits(const orc_model *m, const orc_weights *w, const double *f, float *z_out);

/* Draft confidence of one step: the largest probability of the draft head's
   softmax over its (fp32) logit row, 1 / sum_t exp(z_t - max z). */
double orc_confidence(int64_t n, const float *z);

/* p_min trim of a drafted block: drafting stops at the first step whose
   confidence is below p_min, so n_keep[s] = number of leading steps with
   conf >= p_min (n_steps if none falls below; p_min <= 0 never trims).
   Drafts at k >= n_keep[s] become -1.  near[s] = 1 when some conf of the
   sequence up to and including its stopping step lies within tol of p_min. */
int orc_pmin_trim(int32_t n_seq, int32_t n_steps, const double *conf, double p_min, double tol,
                  int32_t *drafts, int32_t *out_n_keep, int32_t *out_near);

int orc_verify_greedy(int32_t n_seq, int32_t n_draft, int32_t n_vocab, const float *logits,
                      const int32_t *drafts, int32_t *out_tokens, int32_t *out_n_accept);

/* greedy verify from the target's final hidden rows [n_seq, n_draft+1, d]
   through rmsnorm(.; g) (skipped when g is NULL) and the head [n_vocab, d] */
int orc_verify_greedy_hidden(int32_t n_seq, int32_t n_draft, int32_t n_vocab, int32_t d, const float *hidden,
                             const void *head, int32_t head_dtype, const float *g, double eps,
                             const int32_t *drafts, int32_t *out_tokens, int32_t *out_n_accept,
                             double *out_margin);

/* processed sampling distribution of one row; returns the number of tokens
   with non-zero probability, or < 0 on error */
int orc_sample_dist(int32_t n_vocab, const float *z, const int32_t *ctx, int32_t n_ctx,
                    const orc_sampler *sp, double *p_out, int32_t *flags);

int orc_verify_sample(int32_t n_seq, int32_t n_draft, int32_t n_vocab, const float *p_logits,
                      const float *q_logits, const int32_t *drafts, const int32_t *history,
                      int32_t history_stride, const int32_t *history_len, const orc_sampler *sp,
                      uint64_t round, int32_t *out_tokens, int32_t *out_n_accept, int32_t *out_flags);
/* the logit rows of the hidden-state greedy verify, then orc_verify_sample */
int orc_verify_sample_hidden(int32_t n_seq, int32_t n_draft, int32_t n_vocab, int32_t d, const float *hidden,
                             const void *head, int32_t head_dtype, const float *g, double eps,
                             const float *q_logits, const int32_t *drafts, const int32_t *history,
                             int32_t history_stride, const int32_t *history_len, const orc_sampler *sp,
                             uint64_t round, int32_t *out_tokens, int32_t *out_n_accept, int32_t *out_flags);

/* the old temperature>0 rule the pages replace: drafts kept while they equal
   the raw argmax, only the first non-matching row sampled (negative control) */
int orc_verify_greedy_match(int32_t n_seq, int32_t n_draft, int32_t n_vocab, const float *p_logits,
                            const int32_t *drafts, const int32_t *history, int32_t history_stride,
                            const int32_t *history_len, const orc_sampler *sp, uint64_t round,
                            int32_t *out_tokens, int32_t *out_n_accept);

/* draw one token from the processed distribution of a row (Gumbel-max on
   the given stream); used by tests to make drafts that follow q exactly */
int32_t orc_sample_row(int32_t n_vocab, const float *z, const int32_t *ctx, int32_t n_ctx,
                       const orc_sampler *sp, uint64_t s, uint64_t round, uint64_t i, uint64_t stream);

#ifdef __cplusplus
}
#endif
#endif
