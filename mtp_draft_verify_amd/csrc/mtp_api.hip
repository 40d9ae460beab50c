// mtp_api.hip -- host runtime behind include/mtp.h.
//
// Responsibilities: validate every argument on the host before anything is
// enqueued, own the scratch (allocated once at create, sized by max_seqs,
// max_steps and the drafter shape), compute the per-call attention geometry
// (visible positions, split-K partition) and hand it to the device in one
// small copy, then enqueue the kernel sequence of the draft chain or verify
// step on the context's stream.  No device-to-host traffic happens inside a
// call.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <utility>
#include <vector>

#include "mtp_internal.h"

using namespace mtp;

namespace {

constexpr int kParamSlots = 8;
constexpr size_t kMaxGraphs = 16;       // captured chains kept per context

thread_local char g_last_error[256] = "";

// Record a failing HIP call (readable through mtp_last_error) and map it to
// MTP_E_DEVICE.
int hip_fail(const char *what, hipError_t e) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
    return MTP_E_DEVICE;
}

int elem_size(int dt) { return dt == MTP_F32 ? 4 : 2; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

bool attn_supported(int kv_dtype, int hd, int g) {
    if (kv_dtype == MTP_BF16) {
        if (hd == 256) return g == 1 || g == 2 || g == 4 || g == 8;
        if (hd == 128) return g == 1 || g == 2 || g == 4 || g == 8;
        return false;
    }
    if (kv_dtype == MTP_F32) {
        if (hd == 64) return g == 1 || g == 2 || g == 4 || g == 8;
        if (hd == 128 || hd == 256) return g == 4;
        return false;
    }
    return false;
}

int64_t pow2ceil(int64_t v) {
    int64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}

}  // namespace

struct mtp_ctx {
    mtp_model_desc desc{};
    mtp_weights w{};
    bool has_weights = false;
    int device = 0;
    int n_cu = 256;                     // compute units of the device
    hipStream_t stream = nullptr;
    // draft scratch
    float *x = nullptr, *q = nullptr, *o = nullptr, *u = nullptr, *h = nullptr, *part = nullptr;
    float *o_op = nullptr, *u_op = nullptr, *x_op = nullptr;    // o, u, x in operand order (several sequences)
    float *sink = nullptr;              // [64] stores that carry nothing land here
    ConfPart *conf_part = nullptr;      // [max_steps][max_seqs][kConfSlots] confidence partials
    float *cl = nullptr;                // [max_seqs, n_centroids] centroid logits (centroid head)
    int32_t *cand = nullptr;            // [max_seqs, centroid_top_k] chosen centroids
    uint64_t *dkeys = nullptr;          // [2][max_seqs]
    double *inv_freq = nullptr;         // [head_dim / 2] RoPE frequencies
    int8_t *head_q = nullptr;           // Q8_0 head re-laid out: int8 plane
    uint16_t *head_qs = nullptr;        //   and fp16 scale plane
    uint8_t *head_qt = nullptr;         // Q8_0 head in unit order (several-sequence head)
    // per-call parameter block: CallIO then SeqParams[max_seqs], at one fixed
    // device address; staged through a ring of pinned host slots
    uint8_t *d_block = nullptr;
    uint8_t *h_block = nullptr;         // [kParamSlots][block_bytes], pinned
    size_t block_bytes = 0;
    hipEvent_t ev[kParamSlots]{};
    bool ev_pending[kParamSlots]{};
    int slot = 0;
    // captured draft chains, one per launch shape, least recently used evicted
    // past kMaxGraphs; an evicted graph may still be queued on the stream, so
    // it is destroyed only once an event recorded behind it has completed
    hipStream_t cap_stream = nullptr;
    struct Graph { int key[11]; hipGraph_t g; hipGraphExec_t exec; uint64_t last_use; };
    std::vector<Graph> graphs;
    uint64_t use_clock = 0;
    struct Retired { hipGraph_t g; hipGraphExec_t exec; hipEvent_t done; };
    std::vector<Retired> retired;
    bool graph_failed = false;          // capture unsupported: launch directly
    // optional event timing per kernel class
    int prof_mask = 0;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_pool;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_pending[MTP_PROF_N];
    // verify scratch
    uint64_t *vkeys = nullptr;          // [max_seqs][max_steps + 1]
    void *hv_plane = nullptr;           // verify from hidden states: staged rows (hidden_d_max wide)
    size_t hv_plane_size = 0;
    float *hv_logits = nullptr;         // sampling verify from hidden states: logit rows (hidden_sample)
    size_t hv_logits_size = 0;
    // temperature>0 verify scratch, per row (target rows then draft rows)
    int32_t s_cap = 0;                  // candidate slots per row
    uint32_t *s_maxkey = nullptr;
    uint64_t *s_topk = nullptr;
    int32_t *s_cand_n = nullptr, *s_cand_id = nullptr;
    float *s_cand_v = nullptr;
    void *s_state = nullptr;
};

extern "C" const char *mtp_last_error(void) { return g_last_error; }

extern "C" const char *mtp_strerror(int code) {
    switch (code) {
    case MTP_OK: return "ok";
    case MTP_E_INVAL: return "invalid argument";
    case MTP_E_SHAPE: return "shape mismatch or limit exceeded";
    case MTP_E_DTYPE: return "unsupported dtype combination";
    case MTP_E_NOMEM: return "out of device or pinned memory";
    case MTP_E_DEVICE: return "HIP runtime error";
    case MTP_E_NOWEIGHTS: return "draft call on a verify-only context";
    case MTP_E_BUSY: return "context busy";
    default: return "unknown status";
    }
}

// Limits of the hidden-state verifies' scratch, sized at create.
static int check_hidden_desc(const mtp_model_desc *d) {
    if (d->hidden_d_max < 0 || d->hidden_d_max > 16384 || d->hidden_d_max % 256) return MTP_E_SHAPE;
    if (d->hidden_sample && d->hidden_d_max == 0) return MTP_E_SHAPE;
    return MTP_OK;
}

extern "C" int mtp_check_desc(const mtp_model_desc *d) {
    if (!d) return MTP_E_INVAL;
    if (check_hidden_desc(d) != MTP_OK) return MTP_E_SHAPE;
    if (d->d_model <= 0 || d->d_hprev <= 0 || d->n_blocks <= 0 || d->n_head_q <= 0 || d->n_head_kv <= 0 ||
        d->head_dim <= 0 || d->d_ff <= 0 || d->n_vocab <= 0 || d->max_seqs <= 0 || d->max_steps <= 0)
        return MTP_E_SHAPE;
    if (d->n_blocks > MTP_MAX_BLOCKS || d->n_head_q % d->n_head_kv) return MTP_E_SHAPE;
    if (d->w_dtype != MTP_F32 && d->w_dtype != MTP_BF16) return MTP_E_DTYPE;
    if (d->kv_dtype != MTP_F32 && d->kv_dtype != MTP_BF16) return MTP_E_DTYPE;
    if (d->head_dtype != MTP_F32 && d->head_dtype != MTP_BF16 && d->head_dtype != MTP_Q8_0) return MTP_E_DTYPE;
    if (!attn_supported(d->kv_dtype, d->head_dim, d->n_head_q / d->n_head_kv)) return MTP_E_SHAPE;
    // 16-byte vectors over every matrix row; Q8_0 blocks of 32
    if (d->d_model % 32 || d->d_hprev % 8 || d->d_ff % 8) return MTP_E_SHAPE;
    const int64_t qd = (int64_t)d->n_head_q * d->head_dim;
    const int64_t kmax = d->w_dtype == MTP_BF16 ? 4096 : 2048;        // <= 8 vectors per lane
    if (d->d_model + d->d_hprev > kmax || d->d_ff > kmax || qd > kmax || d->d_model > kmax) return MTP_E_SHAPE;
    const int64_t hmax = d->head_dtype == MTP_F32 ? 2048 : 4096;        // head kernel: <= 8 vectors per lane
    if (d->d_model > hmax) return MTP_E_SHAPE;
    if (d->max_seqs > 16 || (int64_t)d->max_seqs * d->d_model > 16384) return MTP_E_SHAPE;
    if (d->max_steps > 64) return MTP_E_SHAPE;
    bool swa = false, sw = false;
    for (int l = 0; l < d->n_blocks; ++l) {
        const int b = d->block_src[l];
        if (b != MTP_SRC_FULL && b != MTP_SRC_SWA && b != MTP_SRC_SINK_WINDOW) return MTP_E_INVAL;
        swa |= b == MTP_SRC_SWA;
        sw |= b == MTP_SRC_SINK_WINDOW;
    }
    if (swa && d->swa_window <= 0) return MTP_E_SHAPE;
    if (sw && (d->sw_window <= 0 || d->sw_sink < 0)) return MTP_E_SHAPE;
    if (!(d->rms_eps >= 0.f) || !(d->attn_scale > 0.f) || !(d->rope_theta > 0.f) || !std::isfinite(d->embed_scale))
        return MTP_E_INVAL;
    if (d->n_centroids < 0) return MTP_E_SHAPE;
    if (d->n_centroids > 0) {
        if (d->n_centroids > kMaxCentroids || d->n_vocab % d->n_centroids) return MTP_E_SHAPE;
        if (d->centroid_top_k < 1 || d->centroid_top_k > std::min(d->n_centroids, kMaxCentroidTopK)) return MTP_E_SHAPE;
        if (d->head_dtype == MTP_Q8_0) return MTP_E_DTYPE;
    }
    return MTP_OK;
}

static int check_weights(const mtp_model_desc *d, const mtp_weights *w) {
    const void *mats[] = {w->w_pre, w->w_post, w->head};
    for (const void *p : mats)
        if (!p || !aligned16(p)) return MTP_E_INVAL;
    if (!w->g_final) return MTP_E_INVAL;
    for (int l = 0; l < d->n_blocks; ++l) {
        const void *bm[] = {w->w_q[l], w->w_o[l], w->w_up[l], w->w_down[l]};
        for (const void *p : bm)
            if (!p || !aligned16(p)) return MTP_E_INVAL;
        if (!w->g_attn[l] || !w->g_q[l] || !w->g_mlp[l]) return MTP_E_INVAL;
    }
    if (d->n_centroids > 0 && (!w->centroids || !aligned16(w->centroids) || !w->token_ordering)) return MTP_E_INVAL;
    return MTP_OK;
}

// Destroy the evicted graphs whose last launch has completed (all of them
// when `all`, after the stream has been drained).
static void reap_graphs(mtp_ctx *c, bool all) {
    size_t keep = 0;
    for (size_t i = 0; i < c->retired.size(); ++i) {
        mtp_ctx::Retired &r = c->retired[i];
        if (all || hipEventQuery(r.done) == hipSuccess) {
            (void)hipGraphExecDestroy(r.exec);
            (void)hipGraphDestroy(r.g);
            (void)hipEventDestroy(r.done);
        } else {
            c->retired[keep++] = r;
        }
    }
    c->retired.resize(keep);
    (void)hipGetLastError();            // a pending query is not an error
}

static void free_ctx(mtp_ctx *c) {
    if (!c) return;
    reap_graphs(c, true);
    for (auto &g : c->graphs) {
        (void)hipGraphExecDestroy(g.exec);
        (void)hipGraphDestroy(g.g);
    }
    if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
    void *bufs[] = {c->x, c->q, c->o, c->u, c->h, c->part, c->sink, c->conf_part, c->cl, c->cand, c->dkeys, c->inv_freq, c->head_q, c->head_qs, c->head_qt, c->d_block,
                    c->vkeys, c->s_maxkey, c->s_topk, c->s_cand_n, c->s_cand_id, c->s_cand_v, c->s_state, c->hv_plane,
                    c->o_op, c->u_op, c->x_op, c->hv_logits};
    for (void *b : bufs)
        if (b) (void)hipFree(b);
    if (c->h_block) (void)hipHostFree(c->h_block);
    for (int i = 0; i < kParamSlots; ++i)
        if (c->ev[i]) (void)hipEventDestroy(c->ev[i]);
    for (int k = 0; k < MTP_PROF_N; ++k)
        for (auto &pr : c->prof_pending[k]) c->prof_pool.push_back(pr);
    for (auto &pr : c->prof_pool) {
        (void)hipEventDestroy(pr.first);
        (void)hipEventDestroy(pr.second);
    }
    delete c;
}

template <typename T>
static bool dalloc(T **p, size_t n) {
    return hipMalloc((void **)p, sizeof(T) * std::max<size_t>(n, 1)) == hipSuccess;
}

extern "C" int mtp_ctx_create(const mtp_model_desc *desc, const mtp_weights *weights, void *hip_stream,
                              mtp_ctx **out) {
    if (!desc || !out) return MTP_E_INVAL;
    *out = nullptr;
    if (weights) {
        int rc = mtp_check_desc(desc);
        if (rc) return rc;
        rc = check_weights(desc, weights);
        if (rc) return rc;
    } else if (desc->n_vocab <= 0 || desc->max_seqs <= 0 || desc->max_steps <= 0 || desc->max_steps > 64 ||
               check_hidden_desc(desc) != MTP_OK) {
        return MTP_E_SHAPE;
    }
    mtp_ctx *c = new (std::nothrow) mtp_ctx();
    if (!c) return MTP_E_NOMEM;
    c->desc = *desc;
    c->stream = (hipStream_t)hip_stream;
    g_last_error[0] = 0;
    {
        const hipError_t e = hipGetDevice(&c->device);
        if (e != hipSuccess) { free_ctx(c); return hip_fail("hipGetDevice", e); }
        const hipError_t e2 = hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, c->device);
        if (e2 != hipSuccess) { free_ctx(c); return hip_fail("hipDeviceGetAttribute", e2); }
    }
    const mtp_model_desc &d = c->desc;
    const size_t S = d.max_seqs, R = (size_t)d.max_steps + 1;
    bool ok = dalloc(&c->vkeys, S * R);
    {
        const size_t rows = S * (2 * (size_t)d.max_steps + 1);
        // candidate slots per row: a row's min-p survivors up to this many are
        // kept as a list (sorted when there are at most 4096); at least 4096,
        // at most 65536, within 64 MiB of lists for all rows
        const size_t fit = ((size_t)8 << 20) / rows;
        const size_t cap = std::max<size_t>(4096, std::min<size_t>(65536, fit)) & ~(size_t)255;
        c->s_cap = (int32_t)std::min<size_t>(cap, (size_t)d.n_vocab);
        ok = ok && dalloc(&c->s_maxkey, rows * kRowCtrStride) && dalloc(&c->s_topk, rows) &&
             dalloc(&c->s_cand_n, rows * kRowCtrStride) &&
             dalloc(&c->s_cand_id, rows * c->s_cap) && dalloc(&c->s_cand_v, rows * c->s_cap) &&
             dalloc((uint8_t **)&c->s_state, rows * sample_row_state_bytes());
    }
    // verifies from hidden rows: the staging plane for the widest head, and
    // the logit rows of the sampling form (every row of a largest call)
    if (ok && d.hidden_d_max > 0) {
        c->hv_plane_size = hv_plane_bytes(d.hidden_d_max);
        ok = dalloc((uint8_t **)&c->hv_plane, c->hv_plane_size);
    }
    if (ok && d.hidden_sample) {
        c->hv_logits_size = sizeof(float) * S * R * (size_t)d.n_vocab;
        ok = dalloc(&c->hv_logits, S * R * (size_t)d.n_vocab);
    }
    if (weights) {
        c->w = *weights;
        c->has_weights = true;
        const size_t qd = (size_t)d.n_head_q * d.head_dim;
        ok = ok && dalloc(&c->x, S * d.d_model) && dalloc(&c->q, S * qd) && dalloc(&c->o, S * qd) &&
             dalloc(&c->u, S * d.d_ff) && dalloc(&c->h, S * d.d_hprev) &&
             dalloc(&c->o_op, 16 * qd) && dalloc(&c->u_op, 16 * (size_t)d.d_ff) && dalloc(&c->x_op, 16 * (size_t)d.d_model) &&
             dalloc(&c->part, S * d.n_head_q * MTP_MAX_SPLITS * (size_t)(d.head_dim + kPartHead)) &&
             dalloc(&c->dkeys, 2 * S) && dalloc(&c->inv_freq, (size_t)d.head_dim / 2) && dalloc(&c->sink, 64) &&
             dalloc(&c->conf_part, (size_t)d.max_steps * S * kConfSlots);
        if (ok && d.n_centroids > 0)
            ok = dalloc(&c->cl, S * d.n_centroids) && dalloc(&c->cand, S * d.centroid_top_k);
        c->block_bytes = sizeof(CallIO) + sizeof(SeqParams) * S;
        ok = ok && dalloc(&c->d_block, c->block_bytes);
        if (ok && d.head_dtype == MTP_Q8_0)
            ok = dalloc(&c->head_q, (size_t)d.n_vocab * d.d_model) &&
                 dalloc(&c->head_qs, (size_t)d.n_vocab * (d.d_model / 32));
        // the several-sequence head streams the Q8_0 head in unit order: each
        // 16-row x 256-column unit is one contiguous run already in operand order
        if (ok && d.head_dtype == MTP_Q8_0 && d.max_seqs >= kMmMinSeqs && d.d_model % 256 == 0)
            ok = dalloc(&c->head_qt, q8_unit_order_bytes(d.n_vocab, d.d_model));
        if (ok) ok = hipHostMalloc((void **)&c->h_block, c->block_bytes * kParamSlots) == hipSuccess;
        if (ok) ok = hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking) == hipSuccess;
        for (int i = 0; ok && i < kParamSlots; ++i)
            ok = hipEventCreateWithFlags(&c->ev[i], hipEventDisableTiming) == hipSuccess;
    }
    if (!ok) {
        std::snprintf(g_last_error, sizeof(g_last_error), "allocation failed: %s", hipGetErrorString(hipGetLastError()));
        free_ctx(c);
        return MTP_E_NOMEM;
    }
    {
        const size_t rows = S * (2 * (size_t)d.max_steps + 1);
        hipError_t e = hipMemset(c->vkeys, 0, sizeof(uint64_t) * S * R);
        if (e == hipSuccess) e = hipMemset(c->s_maxkey, 0, sizeof(uint32_t) * rows * kRowCtrStride);
        if (e == hipSuccess) e = hipMemset(c->s_cand_n, 0, sizeof(int32_t) * rows * kRowCtrStride);
        if (e != hipSuccess) { free_ctx(c); return hip_fail("hipMemset (verify scratch)", e); }
    }
    if (c->has_weights) {
        hipError_t e = hipMemset(c->dkeys, 0, sizeof(uint64_t) * 2 * S);
        if (e != hipSuccess) { free_ctx(c); return hip_fail("hipMemset (draft keys)", e); }
        // the operand-order slots of sequences >= S are read (their MFMA
        // columns are discarded) but never written: keep them finite
        const size_t qd = (size_t)d.n_head_q * d.head_dim;
        e = hipMemset(c->o_op, 0, sizeof(float) * 16 * qd);
        if (e == hipSuccess) e = hipMemset(c->u_op, 0, sizeof(float) * 16 * (size_t)d.d_ff);
        if (e == hipSuccess) e = hipMemset(c->x_op, 0, sizeof(float) * 16 * (size_t)d.d_model);
        if (e != hipSuccess) { free_ctx(c); return hip_fail("hipMemset (operand buffers)", e); }
        e = launch_rope_init(c->inv_freq, d.head_dim, d.rope_theta, c->stream);
        if (e != hipSuccess) { free_ctx(c); return hip_fail("rope table kernel", e); }
        if (d.head_dtype == MTP_Q8_0) {
            e = launch_q8_repack((const uint8_t *)c->w.head, d.n_vocab, d.d_model, c->head_q, c->head_qs, c->stream);
            if (e == hipSuccess && c->head_qt)
                e = launch_q8_unit_order((const uint8_t *)c->w.head, d.n_vocab, d.d_model, c->head_qt, c->stream);
            if (e != hipSuccess) { free_ctx(c); return hip_fail("Q8_0 re-layout kernel", e); }
        }
    }
    *out = c;
    return MTP_OK;
}

extern "C" void mtp_ctx_destroy(mtp_ctx *c) {
    if (!c) return;
    (void)hipStreamSynchronize(c->stream);
    free_ctx(c);
}

// ---------------------------------------------------------------------------
// optional event timing
// ---------------------------------------------------------------------------
namespace mtp {
struct LaunchTimer {
    mtp_ctx *c;
    int cls;
};
thread_local LaunchTimer *g_launch_timer = nullptr;

bool launch_timer_take(LaunchTimer *t, hipEvent_t *start, hipEvent_t *stop) {
    mtp_ctx *c = t->c;
    if (c->prof_pool.empty()) {
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess) return false;
        if (hipEventCreate(&b) != hipSuccess) {
            (void)hipEventDestroy(a);
            return false;
        }
        c->prof_pool.emplace_back(a, b);
    }
    *start = c->prof_pool.back().first;
    *stop = c->prof_pool.back().second;
    c->prof_pool.pop_back();
    return true;
}

void launch_timer_done(LaunchTimer *t, hipEvent_t start, hipEvent_t stop) {
    t->c->prof_pending[t->cls].emplace_back(start, stop);
}
}  // namespace mtp

namespace {
// Times every kernel launched in its scope as class k (when k is enabled).
struct ProfScope {
    LaunchTimer timer;
    LaunchTimer *prev;
    bool on;
    ProfScope(mtp_ctx *ctx, int k) : timer{ctx, k}, prev(g_launch_timer), on((ctx->prof_mask >> k) & 1) {
        if (on) g_launch_timer = &timer;
    }
    ~ProfScope() {
        if (on) g_launch_timer = prev;
    }
};
}  // namespace

extern "C" int mtp_profile_enable(mtp_ctx *c, int mask) {
    if (!c) return MTP_E_INVAL;
    if (hipStreamSynchronize(c->stream) != hipSuccess) return MTP_E_DEVICE;
    for (int k = 0; k < MTP_PROF_N; ++k) {
        for (auto &pr : c->prof_pending[k]) c->prof_pool.push_back(pr);
        c->prof_pending[k].clear();
    }
    c->prof_mask = mask & ((1 << MTP_PROF_N) - 1);
    return MTP_OK;
}

extern "C" int mtp_profile_read(mtp_ctx *c, int cls, double *total_ms, int64_t *count) {
    if (!c || cls < 0 || cls >= MTP_PROF_N || !total_ms || !count) return MTP_E_INVAL;
    if (hipStreamSynchronize(c->stream) != hipSuccess) return MTP_E_DEVICE;
    double t = 0.0;
    for (auto &pr : c->prof_pending[cls]) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess) return MTP_E_DEVICE;
        t += ms;
        c->prof_pool.push_back(pr);
    }
    *total_ms = t;
    *count = (int64_t)c->prof_pending[cls].size();
    c->prof_pending[cls].clear();
    return MTP_OK;
}

// ---------------------------------------------------------------------------
// draft chain
// ---------------------------------------------------------------------------
// Split-K geometry of one sequence's visible cells: at most MTP_MAX_SPLITS
// power-of-two splits of at least 64 cells (one 16-cell tile per wave), and
// at most MTP_MAX_SPLITS / 2 when its workgroups serve two kv heads each
// (kWideCtx).  It depends on the sequence alone (and on whether it is alone
// in the batch), so a sequence gets the same partition and the same
// arithmetic whatever else is in the batch.  In a
// batch, sequences of 2048 or more visible cells split no finer than 128
// cells, so that each wave overlaps one tile's loads with the other's
// arithmetic; workgroups are plentiful there (measured, attention + merge:
// 16 sequences x 8192 cells 74 -> 58 us, 16 x 4096 42 -> 36 us, 2 x 8192
// 16.9 -> 16.5 us), while short windows keep the finer split for
// parallelism (8 sequences x 321 cells lose 2% with 128).
static int src_geometry(const mtp_model_desc &d, const mtp_seq &sq, int src, bool batched, SrcParams &p) {
    const mtp_kv_view &kv = sq.src[src];
    const int es = elem_size(d.kv_dtype);
    if (!kv.k || !kv.v || !aligned16(kv.k) || !aligned16(kv.v)) return MTP_E_INVAL;
    if (kv.n_cells <= 0 || kv.n_cells > 0x7FFFFFFF) return MTP_E_SHAPE;
    if (kv.cell_stride < (int64_t)d.n_head_kv * d.head_dim || (kv.cell_stride * es) % 16) return MTP_E_SHAPE;
    p.k = kv.k;
    p.v = kv.v;
    p.cell_stride = kv.cell_stride;
    p.n_cells = (int32_t)kv.n_cells;
    p.n_sink = 0;
    if (src == MTP_SRC_FULL) {
        if (sq.attn_pos >= kv.n_cells) return MTP_E_SHAPE;
        p.n_vis = sq.attn_pos + 1;
        p.c0 = 0;
    } else if (src == MTP_SRC_SWA) {
        if (kv.n_cells < d.swa_window) return MTP_E_SHAPE;
        const int32_t lo = std::max(0, sq.attn_pos - d.swa_window + 1);
        p.n_vis = sq.attn_pos - lo + 1;
        p.c0 = (int32_t)(lo % kv.n_cells);
    } else {
        // sink + window over a linear cache: [0, min(sink, first)) ++ [first, attn_pos]
        if (sq.attn_pos >= kv.n_cells) return MTP_E_SHAPE;
        if (sq.run_lo > sq.attn_pos) return MTP_E_INVAL;
        const int32_t first = std::max({sq.attn_pos - d.sw_window + 1, sq.run_lo, 0});
        p.n_sink = std::min(d.sw_sink, first);
        p.c0 = first;
        p.n_vis = p.n_sink + (sq.attn_pos - first + 1);
    }
    p.heads_wg = attn_heads_per_wg(d.kv_dtype, d.head_dim, d.n_head_q, d.n_head_kv, p.n_vis);
    const int64_t max_split = p.heads_wg == 2 ? MTP_MAX_SPLITS / 2 : MTP_MAX_SPLITS;
    const int64_t per = (p.n_vis + max_split - 1) / max_split;
    const int64_t min_split = (batched && p.n_vis >= 2048) ? 128 : 64;
    p.split_len = (int32_t)std::max<int64_t>(min_split, pow2ceil(per));
    p.n_split = (p.n_vis + p.split_len - 1) / p.split_len;
    return MTP_OK;
}

static int gemv_rows_per_wg(int M) {
    int r = (M + 511) / 512;
    r = ((r + 3) / 4) * 4;
    return std::max(4, r);
}

static hipError_t run_gemv(mtp_ctx *c, int in_mode, int epi, GemvArgs a, hipStream_t st) {
    ProfScope ps(c, MTP_PROF_GEMV);
    if (mm_gemv_supported(c->desc.w_dtype, a)) return launch_mm_gemv(in_mode, epi, a, st);
    if (a.src_op || a.dst_op) return hipErrorInvalidValue;     // operand order is a matrix-core path layout
    a.rows_per_wg = gemv_rows_per_wg(a.M);
    const int n_wg = (a.M + a.rows_per_wg - 1) / a.rows_per_wg;
    return launch_gemv(c->desc.w_dtype, in_mode, epi, a, n_wg, st);
}

// Launch shape of one draft call: everything the kernel sequence depends on
// besides the parameter block.
struct ChainShape {
    int S, N, split[MTP_N_SRC];
    int logits;     // the caller asked for draft logits
    int conf;       // the caller asked for per-step confidence / the p_min trim
    int stream_kv;  // a step's visible KV exceeds kStreamKvBytes (non-temporal KV loads)
    int wide[MTP_N_SRC];    // sequences whose attention workgroups serve two kv heads: 0 none, 1 some, 2 all
};

// Enqueue the whole draft chain (N steps of a1..a7, then the hand-off of the
// last draft ids) on `st`.  Every argument is a context-owned or weight
// address, so the same sequence can be captured once and replayed.
static hipError_t enqueue_chain(mtp_ctx *c, const ChainShape &sh, hipStream_t st) {
    const mtp_model_desc &d = c->desc;
    const int D = d.d_model, DH = d.d_hprev, QD = d.n_head_q * d.head_dim, F = d.d_ff, V = d.n_vocab;
    const int S = sh.S, N = sh.N;
    const CallIO *io = (const CallIO *)c->d_block;
    const SeqParams *dp = (const SeqParams *)(c->d_block + sizeof(CallIO));
    hipError_t e = hipSuccess;
    int n_part = 0;                     // confidence partials per (step, sequence)
    // Several sequences: the residual stream x, the attention output and the
    // MLP hidden units also go to operand-order buffers, read by the GEMVs
    // that consume them (all of which then take the matrix-core path).
    bool mm_io;
    {
        GemvArgs t{};
        t.S = S;
        t.K = QD;
        mm_io = mm_gemv_supported(d.w_dtype, t);
        t.K = D;
        mm_io = mm_io && mm_gemv_supported(d.w_dtype, t);
        t.K = F;
        mm_io = mm_io && mm_gemv_supported(d.w_dtype, t);
        t.K = D + DH;
        mm_io = mm_io && mm_gemv_supported(d.w_dtype, t);
    }
    for (int k = 0; k < N && e == hipSuccess; ++k) {
        uint64_t *key_cur = c->dkeys + (size_t)(k & 1) * d.max_seqs;
        uint64_t *key_prev = c->dkeys + (size_t)((k + 1) & 1) * d.max_seqs;
        // a1: x = W_pre [embed_scale * E[tok]; h]
        GemvArgs ga{};
        ga.W = c->w.w_pre; ga.M = D; ga.K = D + DH; ga.S = S;
        ga.embed = c->w.head; ga.embed_dtype = d.head_dtype; ga.d_embed = D; ga.embed_rows = V;
        ga.embed_q = c->head_q; ga.embed_qs = c->head_qs; ga.embed_scale = d.embed_scale;
        ga.io = io; ga.step = k;
        ga.key_in = key_prev;
        ga.h = c->h; ga.dh = DH;
        ga.key_reset = key_cur;
        ga.drafts_stride = N; ga.drafts_col = k - 1;
        ga.dst = c->x; ga.dst_stride = D;
        ga.dst_op = mm_io ? c->x_op : nullptr;
        e = run_gemv(c, IN_EMBED, EPI_STORE, ga, st);
        for (int l = 0; l < d.n_blocks && e == hipSuccess; ++l) {
            // a2: q = W_q rmsnorm(x)
            GemvArgs gq{};
            gq.W = c->w.w_q[l]; gq.M = QD; gq.K = D; gq.S = S;
            gq.src = c->x; gq.src_stride = D; gq.gain = c->w.g_attn[l]; gq.eps = d.rms_eps;
            gq.dst = c->q; gq.dst_stride = QD;
            gq.src_op = mm_io ? c->x_op : nullptr;
            e = run_gemv(c, IN_NORM, EPI_STORE, gq, st);
            // a3: split-K attention + merge
            const int src = d.block_src[l];
            {
                ProfScope ps_attn(c, MTP_PROF_ATTN);
                if (e == hipSuccess) {
                    AttnArgs aa{};
                    aa.q = c->q; aa.g_q = c->w.g_q[l]; aa.inv_freq = c->inv_freq; aa.eps = d.rms_eps;
                    aa.theta = d.rope_theta;
                    aa.scale = d.attn_scale; aa.Hq = d.n_head_q; aa.Hkv = d.n_head_kv; aa.hd = d.head_dim;
                    aa.S = S; aa.src = src; aa.step = k; aa.seqs = dp; aa.part = c->part;
                    aa.stream_kv = sh.stream_kv;
                    aa.wide = sh.wide[src];
                    e = launch_attn(d.kv_dtype, aa, sh.split[src], st);
                }
            }
            {
                ProfScope ps_merge(c, MTP_PROF_MERGE);
                if (e == hipSuccess) {
                    MergeArgs ma{};
                    ma.part = c->part; ma.o = c->o; ma.o_op = mm_io ? c->o_op : nullptr;
                    ma.Hq = d.n_head_q; ma.Hkv = d.n_head_kv;
                    ma.hd = d.head_dim; ma.S = S; ma.src = src; ma.seqs = dp;
                    e = launch_merge(ma, st);
                }
            }
            // a4: x += W_o o
            if (e == hipSuccess) {
                GemvArgs go{};
                go.W = c->w.w_o[l]; go.M = D; go.K = QD; go.S = S;
                go.src = c->o; go.src_stride = QD; go.dst = c->x; go.dst_stride = D;
                go.src_op = mm_io ? c->o_op : nullptr;
                go.dst_op = mm_io ? c->x_op : nullptr;
                e = run_gemv(c, IN_PLAIN, EPI_ADD, go, st);
            }
            // a5: u = silu(W_up rmsnorm(x)); x += W_down u
            if (e == hipSuccess) {
                GemvArgs gu{};
                gu.W = c->w.w_up[l]; gu.M = F; gu.K = D; gu.S = S;
                gu.src = c->x; gu.src_stride = D; gu.gain = c->w.g_mlp[l]; gu.eps = d.rms_eps;
                gu.dst = c->u; gu.dst_stride = F;
                gu.dst_op = mm_io ? c->u_op : nullptr;
                gu.src_op = mm_io ? c->x_op : nullptr;
                e = run_gemv(c, IN_NORM, EPI_SILU, gu, st);
            }
            if (e == hipSuccess) {
                GemvArgs gd{};
                gd.W = c->w.w_down[l]; gd.M = D; gd.K = F; gd.S = S;
                gd.src = c->u; gd.src_stride = F; gd.dst = c->x; gd.dst_stride = D;
                gd.src_op = mm_io ? c->u_op : nullptr;
                gd.dst_op = mm_io ? c->x_op : nullptr;
                e = run_gemv(c, IN_PLAIN, EPI_ADD, gd, st);
            }
        }
        // a6 (centroid head): centroid logits C rmsnorm(x; g_final), top-k
        if (e == hipSuccess && d.n_centroids > 0) {
            GemvArgs gc{};
            gc.W = c->w.centroids; gc.M = d.n_centroids; gc.K = D; gc.S = S;
            gc.src = c->x; gc.src_stride = D; gc.gain = c->w.g_final; gc.eps = d.rms_eps;
            gc.dst = c->cl; gc.dst_stride = d.n_centroids;
            gc.src_op = mm_io && mm_gemv_supported(d.w_dtype, gc) ? c->x_op : nullptr;
            e = run_gemv(c, IN_NORM, EPI_STORE, gc, st);
            if (e == hipSuccess) e = launch_centroid_topk(c->cl, d.n_centroids, d.centroid_top_k, S, c->cand, st);
        }
        // a6 + a7: final norm, LM head + argmax, post-projection
        if (e == hipSuccess) {
            HeadArgs ha{};
            ha.x = c->x; ha.g_final = c->w.g_final; ha.eps = d.rms_eps; ha.d = D; ha.S = S; ha.V = V;
            ha.head = c->w.head; ha.head_q = c->head_q; ha.head_qs = c->head_qs; ha.head_qt = c->head_qt;
            // one sequence: one workgroup per compute unit, each streaming a
            // contiguous block of rows with the next rows always in flight
            const int64_t wg_cap = S == 1 ? c->n_cu : 2048;
            const int n_head_wg = (int)std::min<int64_t>(wg_cap, std::max<int64_t>(1, (V + 15) / 16));
            int rpw = (V + n_head_wg - 1) / n_head_wg;
            rpw = ((rpw + 15) / 16) * 16;
            ha.rows_per_wg = rpw;
            ha.n_head_wg = (V + rpw - 1) / rpw;
            ha.keys = key_cur;
            ha.io = io; ha.step = k; ha.n_steps = N;
            ha.w_post = c->w.w_post; ha.dh = DH;
            ha.post_rows_per_wg = 4;
            ha.h_out = c->h;
            ha.sink = c->sink;
            ha.conf = sh.conf ? c->conf_part + (size_t)k * d.max_seqs * kConfSlots : nullptr;
            const int n_post_wg = (DH + ha.post_rows_per_wg - 1) / ha.post_rows_per_wg;
            ProfScope ps(c, MTP_PROF_HEAD);
            if (d.n_centroids > 0) {
                ha.cand = c->cand; ha.ordering = c->w.token_ordering;
                ha.n_cand = d.centroid_top_k; ha.vsc = V / d.n_centroids;
                n_part = cand_head_groups(ha);
                e = launch_cand_head(d.head_dtype, d.w_dtype, ha, n_post_wg, sh.logits, st);
            } else {
                const bool mm = mm_head_supported(d.head_dtype, d.w_dtype, ha);
                n_part = mm ? mm_head_groups(d.head_dtype, ha) : ha.n_head_wg;
                e = mm ? launch_mm_head(d.head_dtype, ha, sh.logits, st)
                       : launch_head(d.head_dtype, d.w_dtype, ha, n_post_wg, sh.logits, st);
            }
        }
    }
    if (e == hipSuccess)
        e = launch_finish_drafts(c->dkeys + (size_t)((N - 1) & 1) * d.max_seqs, S, io, N, N - 1, st);
    if (e == hipSuccess && sh.conf)
        e = launch_conf_finish(c->conf_part, S, N, n_part, (int64_t)d.max_seqs * kConfSlots, io, st);
    return e;
}

// The captured chain for a launch shape (built on first use).
static hipGraphExec_t chain_graph(mtp_ctx *c, const ChainShape &sh) {
    const int key[11] = {sh.S, sh.N, sh.split[0], sh.split[1], sh.split[2], sh.logits, sh.conf, sh.stream_kv,
                         sh.wide[0], sh.wide[1], sh.wide[2]};
    ++c->use_clock;
    reap_graphs(c, false);
    for (auto &g : c->graphs)
        if (std::memcmp(g.key, key, sizeof(key)) == 0) {
            g.last_use = c->use_clock;
            return g.exec;
        }
    if (c->graph_failed) return nullptr;
    if (hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeRelaxed) != hipSuccess) {
        c->graph_failed = true;
        return nullptr;
    }
    const hipError_t e = enqueue_chain(c, sh, c->cap_stream);
    hipGraph_t g = nullptr;
    const hipError_t e2 = hipStreamEndCapture(c->cap_stream, &g);
    if (e != hipSuccess || e2 != hipSuccess || !g) {
        if (g) (void)hipGraphDestroy(g);
        (void)hipGetLastError();
        c->graph_failed = true;
        return nullptr;
    }
    hipGraphExec_t exec = nullptr;
    if (hipGraphInstantiate(&exec, g, nullptr, nullptr, 0) != hipSuccess) {
        (void)hipGraphDestroy(g);
        (void)hipGetLastError();
        c->graph_failed = true;
        return nullptr;
    }
    if (c->graphs.size() >= kMaxGraphs) {
        // evict the least recently used chain; everything enqueued so far on
        // the stream (its launches included) precedes the event
        size_t lru = 0;
        for (size_t i = 1; i < c->graphs.size(); ++i)
            if (c->graphs[i].last_use < c->graphs[lru].last_use) lru = i;
        hipEvent_t done = nullptr;
        if (hipEventCreateWithFlags(&done, hipEventDisableTiming) != hipSuccess ||
            hipEventRecord(done, c->stream) != hipSuccess) {
            // cannot tell when the old chain is idle: keep it, and drop the
            // new one (never launched); this call launches kernel by kernel
            if (done) (void)hipEventDestroy(done);
            (void)hipGetLastError();
            (void)hipGraphExecDestroy(exec);
            (void)hipGraphDestroy(g);
            return nullptr;
        }
        c->retired.push_back({c->graphs[lru].g, c->graphs[lru].exec, done});
        c->graphs.erase(c->graphs.begin() + (long)lru);
    }
    mtp_ctx::Graph ent;
    std::memcpy(ent.key, key, sizeof(key));
    ent.g = g;
    ent.exec = exec;
    ent.last_use = c->use_clock;
    c->graphs.push_back(ent);
    return exec;
}

extern "C" int mtp_draft_block(mtp_ctx *c, int32_t n_seq, const mtp_seq *seqs, const int32_t *last_tok,
                               const float *h_prev, int32_t n_steps, int32_t *out_drafts, float *out_h_last,
                               float *out_logits) {
    return mtp_draft_block_conf(c, n_seq, seqs, last_tok, h_prev, n_steps, out_drafts, out_h_last, out_logits,
                                nullptr, 0.0f, nullptr);
}

extern "C" int mtp_draft_block_conf(mtp_ctx *c, int32_t n_seq, const mtp_seq *seqs, const int32_t *last_tok,
                                    const float *h_prev, int32_t n_steps, int32_t *out_drafts, float *out_h_last,
                                    float *out_logits, float *out_conf, float p_min, int32_t *out_n_keep) {
    if (!c) return MTP_E_INVAL;
    if (!(p_min == p_min) || ((p_min > 0.0f || out_n_keep) && !out_conf)) return MTP_E_INVAL;
    if (!c->has_weights) return MTP_E_NOWEIGHTS;
    const mtp_model_desc &d = c->desc;
    if (n_seq < 1 || n_seq > d.max_seqs || n_steps < 1 || n_steps > d.max_steps) return MTP_E_SHAPE;
    if (!seqs || !last_tok || !h_prev || !out_drafts) return MTP_E_INVAL;
    if (!aligned16(h_prev)) return MTP_E_INVAL;
    bool use_src[MTP_N_SRC] = {false, false, false};
    for (int l = 0; l < d.n_blocks; ++l) use_src[d.block_src[l]] = true;

    // per-call parameter block into the next pinned slot
    const int slot = c->slot;
    if (c->ev_pending[slot] && hipEventSynchronize(c->ev[slot]) != hipSuccess) return MTP_E_DEVICE;
    c->ev_pending[slot] = false;
    uint8_t *hb = c->h_block + (size_t)slot * c->block_bytes;
    CallIO *hio = (CallIO *)hb;
    SeqParams *hp = (SeqParams *)(hb + sizeof(CallIO));
    std::memset(hio, 0, sizeof(CallIO));
    ChainShape sh{n_seq, n_steps, {0, 0, 0}, out_logits != nullptr, out_conf != nullptr, 0, {0, 0, 0}};
    int64_t kv_step_bytes = 0;          // visible K + V bytes one draft step reads
    for (int s = 0; s < n_seq; ++s) {
        const mtp_seq &sq = seqs[s];
        SeqParams &p = hp[s];
        std::memset(&p, 0, sizeof(p));
        if (sq.attn_pos < 0 || sq.pos0 < 0 || (int64_t)sq.pos0 + n_steps > 0x7FFFFFFF) return MTP_E_INVAL;
        p.pos0 = sq.pos0;
        for (int src = 0; src < MTP_N_SRC; ++src) {
            if (!use_src[src]) continue;
            int rc = src_geometry(d, sq, src, n_seq > 1, p.src[src]);
            if (rc) return rc;
            sh.split[src] = std::max(sh.split[src], p.src[src].n_split);
            sh.wide[src] += p.src[src].heads_wg == 2;       // counted here, coded after the loop
        }
        for (int l = 0; l < d.n_blocks; ++l)
            kv_step_bytes += (int64_t)p.src[d.block_src[l]].n_vis * d.n_head_kv * d.head_dim * 2 * elem_size(d.kv_dtype);
    }
    sh.stream_kv = kv_step_bytes > kStreamKvBytes;
    for (int src = 0; src < MTP_N_SRC; ++src)
        sh.wide[src] = sh.wide[src] == 0 ? 0 : sh.wide[src] == n_seq ? 2 : 1;
    // grids are sized for a power-of-two split count so one captured chain
    // serves a range of context lengths (surplus workgroups exit at once)
    for (int src = 0; src < MTP_N_SRC; ++src)
        if (sh.split[src]) sh.split[src] = (int)std::min<int64_t>(MTP_MAX_SPLITS, pow2ceil(sh.split[src]));
    hio->last_tok = last_tok;
    hio->h_prev = h_prev;
    hio->out_drafts = out_drafts;
    hio->out_h_last = out_h_last;
    hio->out_logits = out_logits;
    hio->out_conf = out_conf;
    hio->out_n_keep = out_n_keep;
    hio->p_min = p_min;
    const size_t bytes = sizeof(CallIO) + sizeof(SeqParams) * n_seq;
    {
        hipError_t e0 = hipMemcpyAsync(c->d_block, hb, bytes, hipMemcpyHostToDevice, c->stream);
        if (e0 != hipSuccess) return hip_fail("hipMemcpyAsync (parameter block)", e0);
        e0 = hipEventRecord(c->ev[slot], c->stream);
        if (e0 != hipSuccess) return hip_fail("hipEventRecord", e0);
    }
    c->ev_pending[slot] = true;
    c->slot = (slot + 1) % kParamSlots;

    hipError_t e;
    if (c->prof_mask) {
        e = enqueue_chain(c, sh, c->stream);        // kernel timing takes individual launches
    } else {
        hipGraphExec_t exec = chain_graph(c, sh);
        e = exec ? hipGraphLaunch(exec, c->stream) : enqueue_chain(c, sh, c->stream);
    }
    return e == hipSuccess ? MTP_OK : hip_fail("draft chain launch", e);
}

// ---------------------------------------------------------------------------
// verify
// ---------------------------------------------------------------------------
extern "C" int mtp_verify_greedy(mtp_ctx *c, int32_t n_seq, int32_t n_draft, int32_t n_vocab, const float *logits,
                                 const int32_t *drafts, int32_t *out_tokens, int32_t *out_n_accept) {
    if (!c) return MTP_E_INVAL;
    if (n_seq < 1 || n_seq > c->desc.max_seqs || n_draft < 0 || n_draft > c->desc.max_steps || n_vocab < 1)
        return MTP_E_SHAPE;
    if (!logits || (n_draft > 0 && !drafts) || !out_tokens || !out_n_accept) return MTP_E_INVAL;
    ProfScope ps(c, MTP_PROF_VERIFY);
    hipError_t e = launch_verify_greedy(logits, drafts, n_seq, n_draft, n_vocab, c->vkeys, out_tokens, out_n_accept,
                                        c->stream);
    return e == hipSuccess ? MTP_OK : hip_fail("greedy verify launch", e);
}

extern "C" int mtp_verify_greedy_noalloc(void *hip_stream, int32_t n_seq, int32_t n_draft, int32_t n_vocab,
                                         const float *logits, const int32_t *drafts, int32_t *out_tokens,
                                         int32_t *out_n_accept) {
    if (n_seq < 1 || n_draft < 0 || n_vocab < 1) return MTP_E_SHAPE;
    const int64_t rows = (int64_t)n_seq * (n_draft + 1);
    if (rows > MTP_NOALLOC_MAX_ROWS) {
        std::snprintf(g_last_error, sizeof(g_last_error),
                      "mtp_verify_greedy_noalloc: %lld verified rows exceed the static scratch of %d rows",
                      (long long)rows, MTP_NOALLOC_MAX_ROWS);
        return MTP_E_SHAPE;
    }
    if (!logits || (n_draft > 0 && !drafts) || !out_tokens || !out_n_accept) return MTP_E_INVAL;
    uint64_t *keys = nullptr;
    hipError_t e = noalloc_scratch(&keys);
    if (e != hipSuccess) return hip_fail("scratch symbol lookup", e);
    const hipStream_t st = (hipStream_t)hip_stream;
    // the keys start at zero: an earlier call may have been cut short
    e = launch_clear_u64(keys, rows, st);
    if (e == hipSuccess) e = launch_verify_greedy(logits, drafts, n_seq, n_draft, n_vocab, keys, out_tokens,
                                                  out_n_accept, st);
    return e == hipSuccess ? MTP_OK : hip_fail("greedy verify launch (no-alloc)", e);
}

// Checks of a caller's LM head and hidden rows shared by both hidden-state
// verifies; the head must fit the staging plane allocated at create.
static int prepare_hidden_head(mtp_ctx *c, int32_t n_seq, int32_t n_draft, const mtp_lm_head *head,
                               const float *hidden, const int32_t *drafts, int32_t *out_tokens,
                               int32_t *out_n_accept) {
    if (!c || !head) return MTP_E_INVAL;
    if (n_seq < 1 || n_seq > c->desc.max_seqs || n_draft < 0 || n_draft > c->desc.max_steps) return MTP_E_SHAPE;
    if (head->dtype != MTP_BF16) return MTP_E_DTYPE;
    if (head->d < 256 || head->d > 16384 || head->d % 256 || head->n_vocab < 1 || head->n_vocab > 0x7FFFFFF0)
        return MTP_E_SHAPE;
    if (!head->w || !aligned16(head->w) || (head->g_final && !aligned16(head->g_final)) || !hidden ||
        !aligned16(hidden) || (n_draft > 0 && !drafts) || !out_tokens || !out_n_accept)
        return MTP_E_INVAL;
    if (!(head->rms_eps >= 0.f) || !std::isfinite(head->rms_eps)) return MTP_E_INVAL;
    if (!c->hv_plane || hv_plane_bytes(head->d) > c->hv_plane_size) return MTP_E_SHAPE;
    return MTP_OK;
}

static HvArgs hidden_args(mtp_ctx *c, const mtp_lm_head *head, const float *hidden) {
    HvArgs a{};
    a.hidden = hidden;
    a.g = head->g_final;
    a.eps = head->rms_eps;
    a.d = head->d;
    a.V = head->n_vocab;
    a.head = head->w;
    a.plane = c->hv_plane;
    a.keys = c->vkeys;
    return a;
}

extern "C" int mtp_verify_greedy_hidden(mtp_ctx *c, int32_t n_seq, int32_t n_draft, const mtp_lm_head *head,
                                        const float *hidden, const int32_t *drafts, int32_t *out_tokens,
                                        int32_t *out_n_accept) {
    const int rc = prepare_hidden_head(c, n_seq, n_draft, head, hidden, drafts, out_tokens, out_n_accept);
    if (rc != MTP_OK) return rc;
    ProfScope ps(c, MTP_PROF_VERIFY);
    const HvArgs a = hidden_args(c, head, hidden);
    hipError_t e = launch_verify_hidden(a, n_seq * (n_draft + 1), c->stream);
    if (e == hipSuccess) e = launch_verify_prefix(drafts, n_seq, n_draft, c->vkeys, out_tokens, out_n_accept, c->stream);
    return e == hipSuccess ? MTP_OK : hip_fail("hidden-state verify launch", e);
}

// Sampler checks and the launch arguments of the sampling verify.
static int sample_args(mtp_ctx *c, int32_t n_seq, int32_t n_draft, int32_t n_vocab, const float *p_logits,
                       const float *q_logits, const int32_t *drafts, const int32_t *history, int32_t history_stride,
                       const int32_t *history_len, const mtp_sampler *sp, uint64_t round, int32_t *out_tokens,
                       int32_t *out_n_accept, SampleArgs *out) {
    if (q_logits && n_draft == 0) q_logits = nullptr;
    if (!(sp->temp > 0.f) || !(sp->top_p > 0.f && sp->top_p <= 1.f) || !(sp->min_p >= 0.f && sp->min_p < 1.f) ||
        !(sp->rep_penalty > 0.f) || !std::isfinite(sp->presence_penalty) || !std::isfinite(sp->freq_penalty) ||
        sp->top_k < 0 || sp->penalty_last_n < 0 || sp->penalty_last_n > 1024)
        return MTP_E_INVAL;
    if (sp->penalty_last_n > 0 && (!history_len || (history_stride > 0 && !history) || history_stride < 0))
        return MTP_E_INVAL;
    SampleArgs a{};
    a.p_logits = p_logits; a.q_logits = q_logits; a.drafts = drafts;
    a.history = history; a.history_len = sp->penalty_last_n > 0 ? history_len : nullptr;
    a.hstride = history_stride; a.S = n_seq; a.N = n_draft; a.V = n_vocab;
    a.temp = sp->temp; a.top_p = sp->top_p; a.min_p = sp->min_p;
    a.ln_min_p = std::log((double)a.min_p);
    a.rep = sp->rep_penalty; a.presence = sp->presence_penalty; a.freq = sp->freq_penalty;
    a.top_k = sp->top_k; a.last_n = sp->penalty_last_n; a.seed = sp->seed; a.round = round;
    a.row_maxkey = c->s_maxkey; a.topk_key = c->s_topk; a.cand_n = c->s_cand_n; a.cand_id = c->s_cand_id;
    a.cand_v = c->s_cand_v; a.row_state = c->s_state; a.cap = std::min(c->s_cap, n_vocab);
    a.out_tokens = out_tokens; a.out_n_accept = out_n_accept;
    *out = a;
    return MTP_OK;
}

extern "C" int mtp_verify_sample(mtp_ctx *c, int32_t n_seq, int32_t n_draft, int32_t n_vocab, const float *p_logits,
                                 const float *q_logits, const int32_t *drafts, const int32_t *history,
                                 int32_t history_stride, const int32_t *history_len, const mtp_sampler *sp,
                                 uint64_t round, int32_t *out_tokens, int32_t *out_n_accept) {
    if (!c || !sp) return MTP_E_INVAL;
    const mtp_model_desc &d = c->desc;
    if (n_seq < 1 || n_seq > d.max_seqs || n_draft < 0 || n_draft > d.max_steps || n_vocab < 1 ||
        n_vocab > d.n_vocab)
        return MTP_E_SHAPE;
    if (!p_logits || (n_draft > 0 && !drafts) || !out_tokens || !out_n_accept) return MTP_E_INVAL;
    SampleArgs a;
    const int rc = sample_args(c, n_seq, n_draft, n_vocab, p_logits, q_logits, drafts, history, history_stride,
                               history_len, sp, round, out_tokens, out_n_accept, &a);
    if (rc != MTP_OK) return rc;
    ProfScope ps(c, MTP_PROF_VERIFY);
    const hipError_t e = launch_verify_sample(a, c->stream);
    return e == hipSuccess ? MTP_OK : hip_fail("sampling verify launch", e);
}

extern "C" int mtp_verify_sample_hidden(mtp_ctx *c, int32_t n_seq, int32_t n_draft, const mtp_lm_head *head,
                                        const float *hidden, const float *q_logits, const int32_t *drafts,
                                        const int32_t *history, int32_t history_stride, const int32_t *history_len,
                                        const mtp_sampler *sp, uint64_t round, int32_t *out_tokens,
                                        int32_t *out_n_accept) {
    if (!sp) return MTP_E_INVAL;
    int rc = prepare_hidden_head(c, n_seq, n_draft, head, hidden, drafts, out_tokens, out_n_accept);
    if (rc != MTP_OK) return rc;
    // the sampling scratch and the logit rows are sized by desc.n_vocab
    if (head->n_vocab > c->desc.n_vocab || !c->hv_logits) return MTP_E_SHAPE;
    SampleArgs sa;
    rc = sample_args(c, n_seq, n_draft, head->n_vocab, nullptr, q_logits, drafts, history, history_stride,
                     history_len, sp, round, out_tokens, out_n_accept, &sa);
    if (rc != MTP_OK) return rc;
    const int32_t rows = n_seq * (n_draft + 1);
    if (sizeof(float) * (size_t)rows * head->n_vocab > c->hv_logits_size) return MTP_E_SHAPE;
    sa.p_logits = c->hv_logits;
    ProfScope ps(c, MTP_PROF_VERIFY);
    HvArgs a = hidden_args(c, head, hidden);
    a.logits = c->hv_logits;
    hipError_t e = launch_verify_hidden(a, rows, c->stream);
    if (e == hipSuccess) e = launch_verify_sample(sa, c->stream);
    return e == hipSuccess ? MTP_OK : hip_fail("hidden-state sampling verify launch", e);
}
