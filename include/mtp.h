/*
 * mtp.h -- C ABI of the MI355X (gfx950) library for the data-parallel hot path
 * of Multi-Token-Prediction speculative decoding: the fused on-device draft
 * chain and the verify step.
 *
 * Sources (page title, section):
 *   [G4]  "Gemma 4 MTP -- Multi-Token Prediction speculative decoding":
 *         s.1 (assistant drafter fed the target's h_prev and last token, B-1
 *         chained steps, cross-attention into the target KV, no draft KV),
 *         s.3 (pre/post projection shapes, n_embd_backbone check),
 *         s.4 (per-step graph, in-graph argmax), s.5 (KV read contract),
 *         s.6 (async submit/wait, step positions), s.8 (h_idx rule).
 *   [FUS] "Fused NextN draft graph": N steps as one launch sequence with an
 *         on-device argmax -> embed -> hidden chain and one readback
 *         (I32[N] + embedding).
 *   [MTP] "MTP decoding (--mtp)": "How it is wired" (greedy acceptance of the
 *         longest argmax-matching prefix; the free token of the first
 *         unverified row; next h_prev from row min(n_accepted, n_rows-1)).
 *   [AUD] "opus-mtp-turbo: Track 1 report": findings item 2 (sink +
 *         window draft attention over the drafter's valid cell run), s.4
 *         (exact temperature>0 speculative sampling, sampling chain order).
 *
 * Conventions for every entry point
 *   - All tensors are caller-owned DEVICE memory unless marked "host".  The
 *     library never writes weights, KV caches or inputs.
 *   - Matrices are row-major [out, in].  bf16 is stored as raw 16-bit bf16
 *     patterns.  A Q8_0 matrix is row-major blocks of 34 bytes: a
 *     little-endian fp16 scale d followed by 32 int8 values q (value = d*q).
 *   - Every call enqueues work on the context's HIP stream and returns
 *     without waiting (the stream-ordered form of [G4] s.6's async submit;
 *     the caller's stream synchronisation is the "wait").  Inputs are read
 *     when the work runs.
 *   - Errors are negative mtp_status codes.  Every check runs on the host
 *     BEFORE anything is enqueued: a failing call has no device side effects.
 *     A context is used by one host thread at a time.
 */
#ifndef MTP_H
#define MTP_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MTP_MAX_BLOCKS 8
#define MTP_MAX_SPLITS 128   /* split-K partitions per (sequence, kv head) */

typedef struct mtp_ctx mtp_ctx;

typedef enum mtp_status {
    MTP_OK = 0,
    MTP_E_INVAL = -1,       /* null pointer, bad enum, bad scalar */
    MTP_E_SHAPE = -2,       /* dimension mismatch or limit exceeded */
    MTP_E_DTYPE = -3,       /* unsupported dtype combination */
    MTP_E_NOMEM = -4,       /* device or pinned allocation failed */
    MTP_E_DEVICE = -5,      /* HIP runtime error */
    MTP_E_NOWEIGHTS = -6,   /* draft call on a verify-only context */
    MTP_E_BUSY = -7         /* reserved: second in-flight request ([G4] s.6) */
} mtp_status;

typedef enum mtp_dtype { MTP_F32 = 0, MTP_BF16 = 1, MTP_Q8_0 = 2 } mtp_dtype;

/* KV source kinds ([G4] s.1 twist 2: each drafter block reads the last target
   layer of its own attention type).  MTP_SRC_SINK_WINDOW is the attention
   sink + sliding window of [AUD] item 2: the drafter sees
   the first sw_sink positions and the last sw_window positions of a linear
   cache, the window starting no earlier than the sequence's valid run. */
typedef enum mtp_src { MTP_SRC_FULL = 0, MTP_SRC_SWA = 1, MTP_SRC_SINK_WINDOW = 2 } mtp_src;
#define MTP_N_SRC 3

/* Drafter description ([G4] s.3-4).  d_hprev is the target's backbone width
   (n_embd_backbone); the pre-projection maps [embed_scale*E[tok]; h_prev]
   (d_model + d_hprev) to d_model, the post-projection maps the final-normed
   d_model vector to the next step's h_prev (d_hprev). */
typedef struct mtp_model_desc {
    int32_t d_model, d_hprev, n_blocks, n_head_q, n_head_kv, head_dim, d_ff, n_vocab;
    int32_t w_dtype;      /* MTP_F32 | MTP_BF16: w_pre, w_post, block matrices */
    int32_t head_dtype;   /* MTP_F32 | MTP_BF16 | MTP_Q8_0: tied LM head = token embedding [n_vocab, d_model] */
    int32_t kv_dtype;     /* MTP_F32 | MTP_BF16: target K and V */
    int32_t swa_window;   /* positions visible through an SWA source (0: no SWA block) */
    int32_t block_src[MTP_MAX_BLOCKS];   /* an mtp_src per block */
    float rms_eps;        /* RMSNorm epsilon */
    float rope_theta;     /* RoPE base (half-split pairs (i, i + head_dim/2)) */
    float attn_scale;     /* softmax scale, normally 1/sqrt(head_dim) */
    float embed_scale;    /* token-embedding scale, sqrt(d_model) in [G4] s.4 */
    int32_t max_seqs;     /* largest n_seq of any later call (sizes scratch) */
    int32_t max_steps;    /* largest n_steps / n_draft of any later call */
    /* Centroid ("ordered embeddings") LM head ([G4] s.3): 0 = the dense tied
       head.  Otherwise the step's logits are the token-embedding rows of the
       centroid_top_k best centroids' token lists (n_vocab / n_centroids ids
       each) applied to f, every other token -1e30.  Requires n_vocab %
       n_centroids == 0, n_centroids <= 8192, 1 <= centroid_top_k <=
       min(n_centroids, 64), head_dtype MTP_F32 or MTP_BF16. */
    int32_t n_centroids;
    int32_t centroid_top_k;
    /* Sink + window source (MTP_SRC_SINK_WINDOW blocks only): window length
       (> 0) and number of leading sink positions (>= 0). */
    int32_t sw_window;
    int32_t sw_sink;
    /* Verifies from the target's hidden rows (mtp_verify_greedy_hidden,
       mtp_verify_sample_hidden): the widest target head width d of any later
       such call (0: those calls are refused with MTP_E_SHAPE; otherwise a
       multiple of 256, <= 16384), and whether mtp_verify_sample_hidden will be
       called (nonzero: its logit rows, max_seqs * (max_steps + 1) * n_vocab
       floats, are allocated at create).  Both apply to verify-only contexts
       too. */
    int32_t hidden_d_max;
    int32_t hidden_sample;
} mtp_model_desc;

/* Borrowed device pointers; must stay valid and unchanged for the context's
   lifetime.  Gains are fp32 [n] vectors.  w_q [n_head_q*head_dim, d_model],
   g_q [head_dim] (per-head query RMSNorm), w_o [d_model, n_head_q*head_dim],
   w_up [d_ff, d_model], w_down [d_model, d_ff]. */
typedef struct mtp_weights {
    const void *w_pre;          /* [d_model, d_model + d_hprev] */
    const void *w_post;         /* [d_hprev, d_model] */
    const void *head;           /* [n_vocab, d_model] in head_dtype */
    const float *g_final;       /* [d_model] */
    const float *g_attn[MTP_MAX_BLOCKS];
    const void *w_q[MTP_MAX_BLOCKS];
    const float *g_q[MTP_MAX_BLOCKS];
    const void *w_o[MTP_MAX_BLOCKS];
    const float *g_mlp[MTP_MAX_BLOCKS];
    const void *w_up[MTP_MAX_BLOCKS];
    const void *w_down[MTP_MAX_BLOCKS];
    const void *centroids;          /* [n_centroids, d_model] in w_dtype (centroid head only) */
    const int32_t *token_ordering;  /* [n_vocab] token ids in [0, n_vocab): centroid c lists entries
                                       [c*vsc, (c+1)*vsc), vsc = n_vocab / n_centroids (centroid head only) */
} mtp_weights;

/* One KV source of one sequence, read-only.  K and V hold n_cells cells;
   cell c of kv head j starts at element c*cell_stride + j*head_dim.  A full
   or sink + window source holds position p at cell p; an SWA ring holds
   position p at cell p mod n_cells (n_cells >= swa_window). */
typedef struct mtp_kv_view {
    const void *k, *v;
    int64_t n_cells;
    int64_t cell_stride;        /* elements; >= n_head_kv * head_dim */
} mtp_kv_view;

/* Host-side per-sequence draft descriptor ([G4] s.5): the drafter attends to
   every position <= attn_pos (full), the last swa_window of them (SWA), or,
   through a sink + window source, positions [0, min(sw_sink, first)) and
   [first, attn_pos] with first = max(attn_pos - sw_window + 1, run_lo, 0)
   ([AUD] item 2: cells before run_lo hold stale entries of an earlier
   context and are never read).  Step k runs RoPE at position
   pos0 + k (pos0 = attn_pos + 1 in [G4] s.6). */
typedef struct mtp_seq {
    mtp_kv_view src[MTP_N_SRC];  /* indexed by mtp_src; unused ones may be zero */
    int32_t attn_pos;
    int32_t pos0;
    int32_t run_lo;             /* first valid position (sink + window source only; <= attn_pos) */
    int32_t pad;
} mtp_seq;

/* Sampling chain of the temperature>0 verify ([AUD] s.4): top-k, penalties
   over the context window, temperature, min-p, top-p. */
typedef struct mtp_sampler {
    float temp, top_p, min_p;
    float rep_penalty, presence_penalty, freq_penalty;
    int32_t top_k;              /* 0 = off */
    int32_t penalty_last_n;     /* context window length (0 = no penalties) */
    uint64_t seed;
} mtp_sampler;

/* Create a context on the current HIP device, bound to hip_stream (a
   hipStream_t; NULL = the null stream).  Allocates all scratch once
   (vocabulary-sized buffers included); no later call allocates device
   memory.  weights == NULL makes a verify-only context (then only n_vocab,
   max_seqs, max_steps, hidden_d_max and hidden_sample of desc are used).
   A Q8_0 head is re-laid out once into a context-owned copy (int8 plane plus
   fp16 scale plane, the same bytes per weight).  Returns MTP_OK and *out. */
int mtp_ctx_create(const mtp_model_desc *desc, const mtp_weights *weights, void *hip_stream, mtp_ctx **out);

/* Waits for the context's stream, then frees everything the context owns. */
void mtp_ctx_destroy(mtp_ctx *ctx);

/* Draft chain ([G4] s.4; [FUS]): for every sequence s, n_steps chained steps
   starting from token last_tok[s] and hidden state h_prev[s, :d_hprev] (fp32).
   Step k: x = W_pre [embed_scale*E[tok_k]; h_k]; per block: RMSNorm -> Q ->
   per-head RMSNorm -> RoPE(pos0+k) -> cross-attention into the block's KV
   source -> W_o + residual -> RMSNorm -> W_down silu(W_up .) + residual; final
   RMSNorm f; logits z = E f; tok_{k+1} = argmax z (lowest id on ties);
   h_{k+1} = W_post f.  No host round trip between steps.
     seqs       host array [n_seq]
     last_tok   int32 [n_seq]
     h_prev     fp32 [n_seq, d_hprev]
     out_drafts int32 [n_seq, n_steps]      tok_1 .. tok_n_steps
     out_h_last fp32 [n_seq, d_hprev] or NULL  (h_{n_steps})
     out_logits fp32 [n_seq, n_steps, n_vocab] or NULL
   Requires 1 <= n_seq <= max_seqs, 1 <= n_steps <= max_steps,
   0 <= attn_pos < n_cells for each full or sink + window source read,
   n_cells >= swa_window for each SWA source read, and run_lo <= attn_pos
   where a sink + window source is read.  The KV must not be rewritten at positions <=
   attn_pos until the work completes; appending past attn_pos is allowed. */
int mtp_draft_block(mtp_ctx *ctx, int32_t n_seq, const mtp_seq *seqs, const int32_t *last_tok,
                    const float *h_prev, int32_t n_steps, int32_t *out_drafts, float *out_h_last,
                    float *out_logits);

/* Draft chain with per-step confidence and the p_min trim ("MTP decoding",
   section "Stopping early when the head is unsure"; "Fused NextN draft
   graph", risks: the per-step softmax maximum read back beside the argmax,
   then the draft block trimmed by p_min before verify).  The same chain as
   mtp_draft_block, always n_steps steps in one launch sequence, plus:
     out_conf   fp32 [n_seq, n_steps]  conf[s, k] = the largest softmax
                probability of step k's logits, 1 / sum_t exp(z_t - max z)
                (required whenever p_min > 0 or out_n_keep is given)
     p_min      trim threshold: drafting stops at the first step whose
                confidence is below p_min and that step is not proposed;
                out_drafts[s, k] = -1 for k >= n_keep[s] (-1 never matches
                in mtp_verify_greedy).  p_min <= 0 keeps every draft.
     out_n_keep int32 [n_seq] or NULL  leading drafts kept
   Returns MTP_E_INVAL for a NaN p_min or a trim request without out_conf. */
int mtp_draft_block_conf(mtp_ctx *ctx, int32_t n_seq, const mtp_seq *seqs, const int32_t *last_tok,
                         const float *h_prev, int32_t n_steps, int32_t *out_drafts, float *out_h_last,
                         float *out_logits, float *out_conf, float p_min, int32_t *out_n_keep);

/* Greedy verify ([MTP] "How it is wired"; [G4] s.8).  logits fp32
   [n_seq, n_draft+1, n_vocab] are the target's rows for [confirmed, drafts...];
   t_i = argmax row i (lowest id on ties); a = the longest prefix with
   drafts[s, j] == t_j; out_tokens[s, 0..a] = t_0..t_a and -1 after;
   out_n_accept[s] = a, which is also the target row whose hidden state seeds
   the next round's h_prev.  drafts int32 [n_seq, n_draft]. */
int mtp_verify_greedy(mtp_ctx *ctx, int32_t n_seq, int32_t n_draft, int32_t n_vocab, const float *logits,
                      const int32_t *drafts, int32_t *out_tokens, int32_t *out_n_accept);

/* Greedy verify for callers that cannot allocate device memory (code under
   HIP graph capture, tight serving loops, harnesses that forbid
   allocation): the same operation, kernels and results as
   mtp_verify_greedy, without a context.  Its scratch (one argmax key per
   verified row) is a static device array of MTP_NOALLOC_MAX_ROWS keys
   (128 KiB) that every GPU the library runs on keeps until the process
   ends; nothing is allocated or freed, and the call clears the keys it uses
   with a kernel (no memset).  All calls on one GPU share that array: calls
   that overlap on one GPU (on different streams, or from several threads)
   race and must be serialised by the caller.
     hip_stream  a hipStream_t (NULL = the null stream) of the current device
     logits, drafts, out_tokens, out_n_accept: as for mtp_verify_greedy
   Returns MTP_E_SHAPE, with nothing enqueued, when n_seq * (n_draft + 1)
   exceeds MTP_NOALLOC_MAX_ROWS; MTP_E_DEVICE if the scratch array's device
   address cannot be looked up. */
#define MTP_NOALLOC_MAX_ROWS 16384
int mtp_verify_greedy_noalloc(void *hip_stream, int32_t n_seq, int32_t n_draft, int32_t n_vocab,
                              const float *logits, const int32_t *drafts, int32_t *out_tokens,
                              int32_t *out_n_accept);

/* The target's LM head, for the verify from hidden states: row-major
   [n_vocab, d] bf16 weights (dtype MTP_BF16; others are MTP_E_DTYPE) and
   the gain of the target's final RMSNorm. */
typedef struct mtp_lm_head {
    const void *w;          /* [n_vocab, d], 16-byte aligned */
    const float *g_final;   /* [d] fp32, or NULL: the hidden rows are already final-normed */
    int32_t d;              /* multiple of 256, <= 16384 */
    int32_t n_vocab;
    int32_t dtype;
    float rms_eps;
} mtp_lm_head;

/* Greedy verify from the target's final hidden rows ([MTP] "Why a wider
   decode can be faster": the head weights are read once for all 1 + n_draft
   rows of every sequence; [MTP] "How it is wired" for the acceptance).  Row
   i of sequence s is hidden[s, i, :]; its logits are z = W rmsnorm(h; g_final)
   (z = W h when g_final is NULL), t_i = argmax z (lowest id on ties), and
   the acceptance is that of mtp_verify_greedy.  No logit row is written:
   the head runs on the matrix cores with an argmax epilogue, 64 rows per
   pass over the weights (more rows take more passes).
     head        host pointer; its w and g_final are device pointers
     hidden      fp32 [n_seq, n_draft+1, head->d], 16-byte aligned
     drafts      int32 [n_seq, n_draft]
     out_tokens  int32 [n_seq, n_draft+1] (-1 past the emitted ones); out_n_accept int32 [n_seq]
   head->d must not exceed the context's hidden_d_max (else MTP_E_SHAPE,
   nothing enqueued); the staging scratch (256 * hidden_d_max bytes) was
   allocated at create. */
int mtp_verify_greedy_hidden(mtp_ctx *ctx, int32_t n_seq, int32_t n_draft, const mtp_lm_head *head,
                             const float *hidden, const int32_t *drafts, int32_t *out_tokens,
                             int32_t *out_n_accept);

/* Exact temperature>0 verify ([AUD] s.4, after Leviathan et al. 2023 s.2.3).
   Row i's context is the last penalty_last_n tokens of history[s, :history_len[s]]
   ++ drafts[s, :i]; p_i and q_i are the sampling chain applied to p_logits
   row i and q_logits row i (q_logits == NULL: q_i one-hot at drafts[s, i]).
   Draft i is accepted when u * q_i(d_i) < p_i(d_i) with u = U(seed, s, round,
   i, 0); at the first rejection the emitted token is drawn from
   max(p_i - q_i, 0) and the round stops; if all are accepted a bonus token is
   drawn from p_n_draft.  Draws use Gumbel-max over SplitMix64 counters
   (stream 1 residual, 2 bonus).
     p_logits fp32 [n_seq, n_draft+1, n_vocab]; q_logits fp32 [n_seq, n_draft, n_vocab]
     history int32 [n_seq, history_stride]; history_len int32 [n_seq], each
             read as clamped to [0, history_stride] (history may be NULL when
             history_stride is 0; history_len may be NULL when
             penalty_last_n is 0)
     sampler host pointer
   Logit rows are expected finite.  A row none of whose tokens survives the
   chain (no finite maximum) has an empty distribution: its draft is
   rejected and a draw from it emits -1.
     out_tokens int32 [n_seq, n_draft+1] (-1 past the emitted ones); out_n_accept int32 [n_seq] */
int mtp_verify_sample(mtp_ctx *ctx, int32_t n_seq, int32_t n_draft, int32_t n_vocab, const float *p_logits,
                      const float *q_logits, const int32_t *drafts, const int32_t *history,
                      int32_t history_stride, const int32_t *history_len, const mtp_sampler *sampler,
                      uint64_t round, int32_t *out_tokens, int32_t *out_n_accept);

/* Exact temperature>0 verify from the target's final hidden rows ("MTP
   decoding", why a wider decode can be faster; [AUD] s.4): the 1 + N rows of
   every sequence meet the target's LM head in one pass over its weights, as
   in mtp_verify_greedy_hidden, and the resulting logit rows go through the
   sampling chain and acceptance rule of mtp_verify_sample (same draws, same
   outputs as mtp_verify_sample called on those rows).
     head        host pointer (bf16 head, as for mtp_verify_greedy_hidden);
                 head->n_vocab must not exceed the context's n_vocab
     hidden      fp32 [n_seq, n_draft+1, head->d], 16-byte aligned
     q_logits    fp32 [n_seq, n_draft, head->n_vocab] or NULL (one-hot drafts)
     drafts, history, history_stride, history_len, sampler, round, out_tokens,
     out_n_accept: as for mtp_verify_sample
   The logit rows go to a context-owned buffer allocated at create (requires
   hidden_sample nonzero and head->d <= hidden_d_max, else MTP_E_SHAPE with
   nothing enqueued); the caller never sees them. */
int mtp_verify_sample_hidden(mtp_ctx *ctx, int32_t n_seq, int32_t n_draft, const mtp_lm_head *head,
                             const float *hidden, const float *q_logits, const int32_t *drafts,
                             const int32_t *history, int32_t history_stride, const int32_t *history_len,
                             const mtp_sampler *sampler, uint64_t round, int32_t *out_tokens,
                             int32_t *out_n_accept);

/* Optional HIP-event timing of the kernels one context launches, for
   measurement tools.  mtp_profile_enable waits for the stream, clears all
   counters and enables the classes whose bit (1 << class) is set in mask
   (0 disables timing).  While enabled, calls launch their kernels one by one
   (not as a replayed graph) and every kernel of an enabled class carries a
   start and a stop event that the runtime sets when that kernel starts and
   finishes running, so a duration holds no dispatch time.  mtp_profile_read
   waits for the stream, returns the summed duration (ms) and the number of
   kernels of one class since the last enable/read, and resets that class. */
typedef enum mtp_prof_class {
    MTP_PROF_HEAD = 0,      /* final norm + LM head + argmax + post-projection */
    MTP_PROF_ATTN = 1,      /* split-K attention (partials per split) */
    MTP_PROF_GEMV = 2,      /* pre-projection, Q, O, up, down GEMVs */
    MTP_PROF_VERIFY = 3,    /* greedy or sampling verify */
    MTP_PROF_MERGE = 4,     /* log-sum-exp merge of the attention splits */
    MTP_PROF_N = 5
} mtp_prof_class;
int mtp_profile_enable(mtp_ctx *ctx, int mask);
int mtp_profile_read(mtp_ctx *ctx, int cls, double *total_ms, int64_t *count);

/* Static string for a status code. */
const char *mtp_strerror(int code);

/* Text of the last HIP failure seen by this thread (the HIP call and its
   error string), or "" if none. */
const char *mtp_last_error(void);

/* Host-only validation of a drafter description (no device calls); the same
   checks mtp_ctx_create runs first. */
int mtp_check_desc(const mtp_model_desc *desc);

#ifdef __cplusplus
}
#endif
#endif
