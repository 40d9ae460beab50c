// mtp_internal.h -- structures shared by the host runtime and the kernels.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mtp.h"

namespace mtp {

// Per-(sequence, source) attention geometry, computed on the host per call and
// copied to the device once per call.  n_vis cells are visible: visible index
// j < n_sink reads cell j (the sink), and j >= n_sink reads cell
// c0 + j - n_sink, wrapped once at n_cells (an SWA ring).
struct SrcParams {
    const void *k;
    const void *v;
    int64_t cell_stride;
    int32_t n_cells;
    int32_t n_sink;
    int32_t n_vis;
    int32_t c0;
    int32_t split_len;
    int32_t n_split;
    int32_t heads_wg;       // kv heads one attention workgroup serves (1, or 2 at long context)
    int32_t pad;
};

struct SeqParams {
    SrcParams src[MTP_N_SRC];
    int32_t pos0;
    int32_t pad[3];
};

// cell holding visible index j of a source
__device__ __forceinline__ int src_cell(const SrcParams &sp, int j) {
    int c = j < sp.n_sink ? j : sp.c0 + (j - sp.n_sink);
    return c >= sp.n_cells ? c - sp.n_cells : c;
}

// Caller buffers of one draft call.  They sit in device memory at a fixed
// address (followed by the SeqParams array), so the kernels of a captured
// chain never change: each call only rewrites this block.
struct CallIO {
    const int32_t *last_tok;
    const float *h_prev;
    int32_t *out_drafts;
    float *out_h_last;
    float *out_logits;
    float *out_conf;        // [S, N] per-step draft confidence (or null)
    int32_t *out_n_keep;    // [S] drafts kept by the p_min trim (or null)
    float p_min;            // trim threshold; <= 0 keeps every draft
    int32_t pad;
};
static_assert(sizeof(CallIO) == 64, "the parameter block layout is fixed");

// Per-workgroup partials of the draft confidence: (max, sum exp(z - max))
// of the workgroup's logits, per (step, sequence) in slots [kConfSlots].
static constexpr int kConfSlots = 2048;
// A split partial row: m, l, 30 pad floats, then acc[hd].  The 128-byte
// header keeps every row and every 64- or 256-byte piece of acc that a
// merge workgroup reads inside whole 128-byte lines (head_dim is a multiple
// of 64); with a 16-byte header those pieces straddled lines and the merge
// fetched 1.7x (four dims per lane) to 3.4x (one dim per lane) its bytes.
static constexpr int kPartHead = 32;
struct ConfPart {
    float m, s;
};

// Input transforms applied while a GEMV stages its input vector.
enum GemvIn : int { IN_PLAIN = 0, IN_NORM = 1, IN_EMBED = 2 };
// Output transforms.
enum GemvEpi : int { EPI_STORE = 0, EPI_ADD = 1, EPI_SILU = 2 };

struct GemvArgs {
    const void *W;          // [M, K] row-major
    int32_t M, K, S;
    int32_t rows_per_wg;
    // input
    const float *src;       // [S, src_stride] (IN_PLAIN / IN_NORM)
    int32_t src_stride;
    const float *gain;      // IN_NORM
    float eps;
    // IN_EMBED: [embed_scale * E[tok]; h]
    const void *embed;      // head / embedding table [V, d]
    int32_t embed_dtype, d_embed, embed_rows;
    const int8_t *embed_q;  // Q8_0 plane [V, d]
    const uint16_t *embed_qs;   // Q8_0 scales [V, d/32]
    float embed_scale;
    const CallIO *io;       // caller buffers (IN_EMBED)
    int32_t step;           // draft step: 0 reads io->last_tok / io->h_prev
    const int32_t *tok_in;  // resolved in the kernel from io / step
    const uint64_t *key_in; // later steps: argmax keys of the previous step
    const float *h;         // [S, dh] hidden state of later steps
    int32_t dh;
    uint64_t *key_reset;    // keys to clear for this step's head
    int32_t *drafts_out;    // resolved in the kernel: io->out_drafts for step > 0
    int32_t drafts_stride, drafts_col;
    // output
    float *dst;             // [S, dst_stride]
    int32_t dst_stride;
    // several sequences (matrix-core path): the input / output also in operand
    // order, [K / 4][16][4] floats (value k of sequence s at (k / 4 * 16 + s) * 4
    // + k % 4), so a consumer's wave loads read 256 contiguous bytes per lane group
    const float *src_op;    // read instead of src when set (IN_PLAIN, IN_NORM)
    float *dst_op;          // written besides dst when set
};

// index of value k of sequence s in an operand-order buffer
__host__ __device__ __forceinline__ int64_t op_index(int k, int s) { return ((int64_t)(k >> 2) * 16 + s) * 4 + (k & 3); }

struct HeadArgs {
    // final norm
    const float *x;         // [S, d]
    const float *g_final;
    float eps;
    int32_t d, S, V;
    // head
    const void *head;       // bf16 / f32 [V, d]
    const int8_t *head_q;   // Q8_0 plane [V, d]
    const uint16_t *head_qs;    // Q8_0 scales [V, d/32]
    const uint8_t *head_qt; // Q8_0 head in unit order (several-sequence head), or null
    int32_t rows_per_wg, n_head_wg;
    uint64_t *keys;         // [S] argmax keys (cleared before)
    const CallIO *io;       // io->out_logits (nullable), io->out_h_last (nullable)
    int32_t step, n_steps;  // logits land at out_logits[s, step, :]
    // post-projection: h = W_post f
    const void *w_post;     // [dh, d] (w dtype)
    int32_t dh, post_rows_per_wg;
    float *h_out;           // [S, dh] context buffer (the last step writes io->out_h_last when given)
    float *sink;            // [64] target of stores that carry nothing (matrix-core head)
    ConfPart *conf;         // this step's confidence partials [S][kConfSlots] (or null)
    // centroid head: candidate rows of sequence s are ordering[cand[s, i] * vsc + r]
    const int32_t *cand;    // [S, n_cand] chosen centroids
    const int32_t *ordering;
    int32_t n_cand, vsc;
};

static constexpr int kMaxCentroids = 8192;
static constexpr int kMaxCentroidTopK = 64;

struct AttnArgs {
    const float *q;         // [S, Hq*hd] raw projections
    const float *g_q;       // [hd]
    const double *inv_freq; // [hd/2] RoPE frequencies theta^(-2i/hd)
    float eps, theta, scale;
    int32_t Hq, Hkv, hd, S, src, step;
    const SeqParams *seqs;
    float *part;            // [S, Hq, MTP_MAX_SPLITS, kPartHead + hd]  (m, l, pad..., o[hd])
    int32_t stream_kv;      // a step's KV exceeds the last-level cache: non-temporal KV loads
    int32_t wide;           // sequences with heads_wg 2 for this source: 0 none, 1 some, 2 all
};

// Visible cells from which a sequence's bf16 attention workgroups serve two
// kv heads each (the waves then read whole cell rows of both heads together)
// and its split count is at most 64.  Measured over 8 sequences x 131072
// cells, 2 kv heads x 256 dims: 328.5 us per launch with one head and
// 1024-cell splits, 324.5 us with two heads and 2048-cell splits; with
// 4096-cell splits 344 us.  Shorter contexts keep one head per workgroup
// (one sequence over 8192 cells: 8.4 -> 11.8 us with two).
static constexpr int32_t kWideCtx = 65536;

// kv heads per attention workgroup for a sequence of n_vis visible cells:
// 2 on the bf16 matrix-core path at long context with an even kv head count
// (not at head_dim 256 with 8 query heads per kv head, whose registers would
// not fit two waves per SIMD).
inline int attn_heads_per_wg(int kv_dtype, int hd, int n_head_q, int n_head_kv, int64_t n_vis) {
    const int G = n_head_kv > 0 ? n_head_q / n_head_kv : 0;
    const bool mm = kv_dtype == MTP_BF16 && ((hd == 256 && (G == 1 || G == 2 || G == 4)) ||
                                             (hd == 128 && (G == 1 || G == 2 || G == 4 || G == 8)));
    return (mm && n_head_kv % 2 == 0 && n_vis >= kWideCtx) ? 2 : 1;
}

// KV bytes per draft step above which the attention streams its KV with
// non-temporal loads: past this a step's KV cannot stay in the device's
// 256 MiB last-level cache until the next step reads it again.
static constexpr int64_t kStreamKvBytes = (int64_t)192 << 20;

struct MergeArgs {
    const float *part;
    float *o;               // [S, Hq*hd]
    float *o_op;            // o in operand order as well (or null)
    int32_t Hq, Hkv, hd, S, src;
    const SeqParams *seqs;
};

// Kernel timing (mtp_profile_enable).  While a timed kernel class is being
// enqueued on this thread, g_launch_timer is set and every launch takes a
// start and a stop event of its own, which the runtime sets when that
// kernel starts and finishes running (no dispatch time between them).
struct LaunchTimer;
extern thread_local LaunchTimer *g_launch_timer;
bool launch_timer_take(LaunchTimer *t, hipEvent_t *start, hipEvent_t *stop);
void launch_timer_done(LaunchTimer *t, hipEvent_t start, hipEvent_t stop);

// Every kernel of the library is launched through here (arguments converted
// to the kernel's parameter types).
template <typename... P, typename... A>
inline void mtp_launch(void (*kernel)(P...), const dim3 &grid, const dim3 &block, size_t shmem, hipStream_t st,
                       A &&...args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    LaunchTimer *t = g_launch_timer;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (t && launch_timer_take(t, &e0, &e1)) {
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, st, e0, e1, 0u, static_cast<P>(args)...);
        launch_timer_done(t, e0, e1);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shmem, st, static_cast<P>(args)...);
    }
}

// launchers (defined with their kernels; all enqueue on `st`)
hipError_t launch_gemv(int w_dtype, int in_mode, int epi, const GemvArgs &a, int n_wg, hipStream_t st);
hipError_t launch_head(int head_dtype, int w_dtype, const HeadArgs &a, int n_post_wg, bool logits, hipStream_t st);
hipError_t launch_attn(int kv_dtype, const AttnArgs &a, int max_split, hipStream_t st);
hipError_t launch_merge(const MergeArgs &a, hipStream_t st);
hipError_t launch_finish_drafts(const uint64_t *keys, int32_t S, const CallIO *io, int32_t stride, int32_t col,
                                hipStream_t st);
hipError_t launch_q8_repack(const uint8_t *blocks, int64_t rows, int32_t cols, int8_t *q, uint16_t *s,
                            hipStream_t st);
// Unit order of a Q8_0 matrix [rows, cols] (cols % 256 == 0) for the
// several-sequence head: unit (t, c) = rows 16t .. 16t+15 x columns 256c ..
// 256c+255 is kQ8UnitBytes contiguous bytes at (t * cols / 256 + c) *
// kQ8UnitBytes.  Bytes 1024 p + 16 l (p < 4, lane l = 16 g + j) hold the 8
// quants of row 16t + j at columns 256c + 32 (2p) + 8g .. +7, then those at
// 256c + 32 (2p + 1) + 8g .. +7: a wave's 16-byte load at its lane offset is
// two K steps of the matrix-core operand.  Bytes 4096 + 16 j hold the fp16
// scales of row 16t + j's blocks 8c .. 8c+7.  Rows past the end are zero.
static constexpr int kQ8UnitBytes = 4352;
size_t q8_unit_order_bytes(int64_t rows, int32_t cols);
hipError_t launch_q8_unit_order(const uint8_t *blocks, int64_t rows, int32_t cols, uint8_t *out, hipStream_t st);
hipError_t launch_clear_u64(uint64_t *p, int64_t n, hipStream_t st);
hipError_t launch_conf_finish(const ConfPart *part, int32_t S, int32_t N, int32_t n_part, int64_t step_stride,
                              const CallIO *io, hipStream_t st);
hipError_t launch_rope_init(double *inv_freq, int32_t hd, float theta, hipStream_t st);

// centroid LM head: top-k centroids per sequence, then the candidate rows
hipError_t launch_centroid_topk(const float *cl, int32_t n_centroids, int32_t k, int32_t S, int32_t *cand,
                                hipStream_t st);
int cand_head_groups(const HeadArgs &a);    // candidate workgroups per sequence (confidence partials)
hipError_t launch_fill_logits(const CallIO *io, int32_t S, int32_t N, int32_t V, int32_t step, float v,
                              hipStream_t st);
hipError_t launch_cand_head(int head_dtype, int w_dtype, const HeadArgs &a, int n_post_wg, bool logits,
                            hipStream_t st);

// several sequences: GEMVs and the LM head on the matrix cores
static constexpr int kMmMinSeqs = 2;
bool mm_gemv_supported(int w_dtype, const GemvArgs &a);
hipError_t launch_mm_gemv(int in_mode, int epi, const GemvArgs &a, hipStream_t st);
bool mm_head_supported(int head_dtype, int w_dtype, const HeadArgs &a);
hipError_t launch_mm_head(int head_dtype, const HeadArgs &a, bool logits, hipStream_t st);
int mm_head_groups(int head_dtype, const HeadArgs &a);   // head workgroups (confidence partials) of one launch

// verify from hidden states: the target's final norm + LM head + argmax over
// rows [row0, row0 + R) of hidden, in passes of up to 64 rows
struct HvArgs {
    const float *hidden;    // [rows, d] fp32 final hidden rows
    const float *g;         // [d] final-norm gain, or null (rows already normed)
    float eps;
    int32_t d, V, row0, R;
    const void *head;       // [V, d] bf16
    void *plane;            // scratch: hv_plane_bytes(d) bytes
    uint64_t *keys;         // [rows] argmax keys, zero before; indexed by row
    float *logits;          // [rows, V] logit rows instead of keys (or null)
};
size_t hv_plane_bytes(int32_t d);
hipError_t launch_verify_hidden(const HvArgs &a, int32_t rows, hipStream_t st);
hipError_t launch_verify_prefix(const int32_t *drafts, int32_t S, int32_t N, uint64_t *keys, int32_t *out_tokens,
                                int32_t *out_n_accept, hipStream_t st);

// device address of the current device's static key scratch of
// mtp_verify_greedy_noalloc (MTP_NOALLOC_MAX_ROWS keys)
hipError_t noalloc_scratch(uint64_t **out);

// verify
hipError_t launch_verify_greedy(const float *logits, const int32_t *drafts, int32_t S, int32_t N, int32_t V,
                                uint64_t *keys, int32_t *out_tokens, int32_t *out_n_accept, hipStream_t st);

struct SampleArgs {
    const float *p_logits;  // [S, N+1, V]
    const float *q_logits;  // [S, N, V] or nullptr
    const int32_t *drafts;  // [S, N]
    const int32_t *history; // [S, hstride]
    const int32_t *history_len;
    int32_t hstride, S, N, V;
    float temp, top_p, min_p, rep, presence, freq;
    double ln_min_p;        // log(min_p) (-inf for min_p = 0), once per call on the host
    int32_t top_k, last_n;
    uint64_t seed, round;
    // scratch, per row (S*(N+1) target rows, then S*N draft rows)
    uint32_t *row_maxkey;   // [rows * kRowCtrStride], zero between calls
    uint64_t *topk_key;
    int32_t *cand_n;        // [rows * kRowCtrStride], zero between calls
    int32_t *cand_id;       // [rows, cap]
    float *cand_v;          // [rows, cap]
    void *row_state;        // [rows] RowState
    int32_t cap;
    int32_t *out_tokens, *out_n_accept;
};
// Every chunk workgroup of a row updates the row's max and list length with
// device-scope atomics; atomics on one line are applied one after another,
// so each row's counter sits alone on a 256-byte stretch (row r at r * 64).
static constexpr int kRowCtrStride = 64;
hipError_t launch_verify_sample(const SampleArgs &a, hipStream_t st);
size_t sample_row_state_bytes();

}  // namespace mtp
