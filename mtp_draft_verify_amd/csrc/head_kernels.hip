// head_kernels.hip -- final RMSNorm + tied LM head + greedy argmax, fused with
// the post-projection ("Gemma 4 MTP" doc s.4 steps 5-8; "Fused NextN draft
// graph": the argmax stays on the device and feeds the next step).
//
// The head is the largest stream of a step (V x d weights).  Rows are read
// with non-temporal 16-byte loads (so the block weights and the KV cache keep
// their cache residency), several rows in flight per wave, and each workgroup
// folds its best (value, lowest index) per sequence into one 64-bit key with
// atomicMax.  Workgroups past n_head_wg compute h' = W_post f instead.  With
// one sequence there is one head workgroup per compute unit, each streaming a
// contiguous block of rows and always holding the next 4 rows per wave in
// flight; measured, that streams a 512 MiB head faster than eight shorter
// workgroups per CU that rely on occupancy for their loads.
#include <algorithm>

#include "widen.h"

namespace mtp {

template <typename WT>
__device__ void post_rows(const HeadArgs &a, const float *fs, float *h_out) {
    constexpr int EPV = WTr<WT>::EPV, CPW = 64 * EPV;
    const int d = a.d, S = a.S;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int r0 = ((int)blockIdx.x - a.n_head_wg) * a.post_rows_per_wg;
    const int r1 = min(a.dh, r0 + a.post_rows_per_wg);
    for (int r = r0 + wid; r < r1; r += 4) {
        const uint4 *wr = (const uint4 *)((const WT *)a.w_post + (int64_t)r * d);
        for (int s = 0; s < S; ++s) {
            float acc = 0.f;
            for (int col = lane * EPV; col < d; col += CPW) {
                float w[EPV];
                widen(wr[col / EPV], w);
                const float4 *fp = (const float4 *)(fs + s * d + col);
#pragma unroll
                for (int e4 = 0; e4 < EPV / 4; ++e4) {
                    const float4 f4 = fp[e4];
                    acc = fmaf(w[4 * e4 + 0], f4.x, acc);
                    acc = fmaf(w[4 * e4 + 1], f4.y, acc);
                    acc = fmaf(w[4 * e4 + 2], f4.z, acc);
                    acc = fmaf(w[4 * e4 + 3], f4.w, acc);
                }
            }
            const float y = wave_sum(acc);
            if (lane == 0) h_out[(int64_t)s * a.dh + r] = y;
        }
    }
}

template <typename HT, int NV, bool ONE, bool CONF, bool LOGITS>
__global__ __launch_bounds__(256) void head_kernel(HeadArgs a, int w_dtype) {
    constexpr int EPV = WTr<HT>::EPV, CPW = 64 * EPV;
    constexpr int RU = ONE ? 4 : 2;        // rows in flight per wave
    extern __shared__ float fs[];          // [S][d] final-normed activations
    __shared__ float rs[kMaxSeqGroup];
    __shared__ uint64_t wbest[4][kMaxSeqGroup];
    __shared__ float wcm[4][kMaxSeqGroup], wcs[4][kMaxSeqGroup];   // confidence partials per wave
    const int d = a.d, S = a.S;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int r0 = blockIdx.x * a.rows_per_wg;
    const int r1 = min(a.V, r0 + a.rows_per_wg);
    const int nblk = d / 32;
    uint4 wv[RU][NV];
    float sc[RU][NV];
    // Loads are unconditional, from clamped addresses (row r1 - 1, the last
    // vector of the row), so that the compiler can count them and wait for
    // exactly the rows it is about to use; rows past r1 are never used and
    // columns past d are zeroed where the weights are consumed.
    auto load_head_rows = [&](int rb, uint4 (&dw)[RU][NV], float (&ds)[RU][NV]) {
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int r = min(rb + u, r1 - 1);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int col = min(v * CPW + lane * EPV, d - EPV);
                if constexpr (sizeof(HT) == 1) {
                    dw[u][v] = ld_nt((const uint4 *)(a.head_q + (int64_t)r * d + col));
                    ds[u][v] = half_to_f(a.head_qs[(int64_t)r * nblk + col / 32]);
                } else {
                    dw[u][v] = ld_nt((const uint4 *)((const HT *)a.head + (int64_t)r * d + col));
                    ds[u][v] = 1.f;
                }
            }
        }
    };
    // the first rows' weights do not depend on x: request them before the prologue
    const bool head_wg = (int)blockIdx.x < a.n_head_wg;
    if (head_wg) load_head_rows(r0 + wid * RU, wv, sc);

    float fr[ONE ? NV : 1][EPV];
    if (ONE && head_wg) {
        // f = rmsnorm(x; g_final) for the one sequence, in registers: every
        // wave loads its lanes' slices of x and of the gain at once and
        // reduces the sum of squares itself (no LDS, no barrier)
        float xr[NV][EPV], gr[NV][EPV];
#pragma unroll
        for (int v = 0; v < (ONE ? NV : 1); ++v) {
            const int col = min(v * CPW + lane * EPV, d - EPV);     // clamped; tail columns zeroed by mask
            const uint32_t m = v * CPW + lane * EPV < d ? 0xFFFFFFFFu : 0u;
#pragma unroll
            for (int e4 = 0; e4 < EPV / 4; ++e4) {
                const float4 x4 = *(const float4 *)(a.x + col + 4 * e4);
                const float4 g4 = *(const float4 *)(a.g_final + col + 4 * e4);
                xr[v][4 * e4 + 0] = __uint_as_float(__float_as_uint(x4.x) & m);
                xr[v][4 * e4 + 1] = __uint_as_float(__float_as_uint(x4.y) & m);
                xr[v][4 * e4 + 2] = __uint_as_float(__float_as_uint(x4.z) & m);
                xr[v][4 * e4 + 3] = __uint_as_float(__float_as_uint(x4.w) & m);
                gr[v][4 * e4 + 0] = g4.x; gr[v][4 * e4 + 1] = g4.y; gr[v][4 * e4 + 2] = g4.z; gr[v][4 * e4 + 3] = g4.w;
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int v = 0; v < (ONE ? NV : 1); ++v)
#pragma unroll
            for (int e = 0; e < EPV; ++e) ss = fmaf(xr[v][e], xr[v][e], ss);
        const float r = 1.0f / sqrtf(wave_sum(ss) / (float)d + a.eps);
#pragma unroll
        for (int v = 0; v < (ONE ? NV : 1); ++v)
#pragma unroll
            for (int e = 0; e < EPV; ++e) fr[ONE ? v : 0][e] = xr[v][e] * r * gr[v][e];
    } else {
        // f = rmsnorm(x; g_final) staged in LDS for every sequence
        for (int j = wid; j < S; j += 4) {
            const float *x = a.x + (int64_t)j * d;
            float ss = 0.f;
            for (int c = lane; c < d; c += 64) ss = fmaf(x[c], x[c], ss);
            ss = wave_sum(ss);
            if (lane == 0) rs[j] = 1.0f / sqrtf(ss / (float)d + a.eps);
        }
        if (tid < 4 * kMaxSeqGroup) {
            wbest[tid / kMaxSeqGroup][tid % kMaxSeqGroup] = 0ull;
            wcm[tid / kMaxSeqGroup][tid % kMaxSeqGroup] = -INFINITY;
            wcs[tid / kMaxSeqGroup][tid % kMaxSeqGroup] = 0.f;
        }
        __syncthreads();
        for (int i = tid; i < S * d; i += kBlock) {
            const int j = i / d, c = i - j * d;
            fs[i] = a.x[i] * rs[j] * a.g_final[c];
        }
        __syncthreads();
        if (!head_wg) {
            float *h_out = (a.step == a.n_steps - 1 && a.io->out_h_last) ? a.io->out_h_last : a.h_out;
            if (w_dtype == MTP_BF16) post_rows<uint16_t>(a, fs, h_out);
            else post_rows<float>(a, fs, h_out);
            return;
        }
    }
    float *logits = LOGITS && a.io->out_logits ? a.io->out_logits + (int64_t)a.step * a.V : nullptr;
    const int64_t logits_stride = (int64_t)a.n_steps * a.V;

    uint64_t best1 = 0ull;                  // one-sequence path keeps its best in a register
    float cm1 = -INFINITY, cs1 = 0.f;       // and its confidence partial
    constexpr bool conf = CONF;             // confidence partials requested
    if constexpr (ONE) {
        // The next rows are requested before these are used (one workgroup
        // per CU: the wave itself keeps its loads in flight).  Between the
        // loads and their use there are no branches or stores, so the
        // compiler waits for exactly the rows in use: columns past d are
        // masked with an AND (a select could become a branch), the last
        // group of rows is peeled instead of guarding the prefetch, and rows
        // past r1 (clamped loads) are dropped after the dot products.  A
        // scheduling barrier stops the compiler from sinking the prefetch
        // below the arithmetic.
        uint32_t cmask[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) cmask[v] = v * CPW + lane * EPV < d ? 0xFFFFFFFFu : 0u;
        auto rows = [&](int rb) {
            float z[RU];
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                float acc = 0.f;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const uint4 q = wv[u][v];
                    float w[EPV];
                    widen(make_uint4(q.x & cmask[v], q.y & cmask[v], q.z & cmask[v], q.w & cmask[v]), w);
                    float part = 0.f;
#pragma unroll
                    for (int e = 0; e < EPV; ++e) part = fmaf(w[e], fr[v][e], part);
                    acc = fmaf(part, sc[u][v], acc);
                }
                z[u] = wave_sum(acc);
            }
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const int r = rb + u;
                if (r < r1) {                   // wave-uniform
                    const uint64_t k = argmax_key(z[u], (uint32_t)r);
                    best1 = k > best1 ? k : best1;
                    if (conf) conf_add(cm1, cs1, z[u]);
                    if (LOGITS && logits && lane == 0) logits[r] = z[u];
                }
            }
        };
        int rb = r0 + wid * RU;
        for (; rb + 4 * RU < r1; rb += 4 * RU) {
            uint4 wn[RU][NV];
            float sn[RU][NV];
            load_head_rows(rb + 4 * RU, wn, sn);
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the dot products
            rows(rb);
#pragma unroll
            for (int u = 0; u < RU; ++u)
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    wv[u][v] = wn[u][v];
                    sc[u][v] = sn[u][v];
                }
        }
        if (rb < r1) rows(rb);
    } else {
        for (int rb = r0 + wid * RU; rb < r1; rb += 4 * RU) {
            if (rb != r0 + wid * RU) load_head_rows(rb, wv, sc);
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const int r = rb + u;
                if (r >= r1) break;             // wave-uniform
                float w[NV][EPV];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const bool col_ok = v * CPW + lane * EPV < d;
                    widen(col_ok ? wv[u][v] : make_uint4(0, 0, 0, 0), w[v]);
                }
                for (int j = 0; j < S; ++j) {
                    float acc = 0.f;
#pragma unroll
                    for (int v = 0; v < NV; ++v) {
                        float part = 0.f;
                        const int col = v * CPW + lane * EPV;
                        if (col < d) {
                            const float4 *fp = (const float4 *)(fs + j * d + col);
#pragma unroll
                            for (int e4 = 0; e4 < EPV / 4; ++e4) {
                                const float4 f4 = fp[e4];
                                part = fmaf(w[v][4 * e4 + 0], f4.x, part);
                                part = fmaf(w[v][4 * e4 + 1], f4.y, part);
                                part = fmaf(w[v][4 * e4 + 2], f4.z, part);
                                part = fmaf(w[v][4 * e4 + 3], f4.w, part);
                            }
                        }
                        acc = fmaf(part, sc[u][v], acc);
                    }
                    const float z = wave_sum(acc);
                    if (logits && lane == 0) logits[(int64_t)j * logits_stride + r] = z;
                    const uint64_t k = argmax_key(z, (uint32_t)r);
                    if (lane == 0) {            // only lane 0 of this wave touches these slots
                        if (k > wbest[wid][j]) wbest[wid][j] = k;
                        if (conf) conf_add(wcm[wid][j], wcs[wid][j], z);
                    }
                }
            }
        }
    }
    if (ONE && lane == 0) {
        wbest[wid][0] = best1;
        wcm[wid][0] = cm1;
        wcs[wid][0] = cs1;
    }
    __syncthreads();
    if (tid < S) {
        uint64_t k = wbest[0][tid];
        for (int w = 1; w < 4; ++w) k = wbest[w][tid] > k ? wbest[w][tid] : k;
        atomicMax((unsigned long long *)&a.keys[tid], (unsigned long long)k);
        if (conf) {
            float m = wcm[0][tid], sm = wcs[0][tid];
            for (int w = 1; w < 4; ++w) conf_merge(m, sm, wcm[w][tid], wcs[w][tid]);
            a.conf[(int64_t)tid * kConfSlots + blockIdx.x] = ConfPart{m, sm};
        }
    }
}

template <typename HT, bool ONE, bool CONF, bool LOGITS>
static hipError_t launch_head_c(const HeadArgs &a, int w_dtype, int n_post_wg, hipStream_t st) {
    constexpr int CPW = 64 * WTr<HT>::EPV;
    const int nv = (a.d + CPW - 1) / CPW;
    const size_t lds = sizeof(float) * (size_t)a.S * a.d;
    dim3 grid(a.n_head_wg + n_post_wg);
#define MTP_HEAD_CASE(N)                                                                               \
    if (nv <= N) {                                                                                     \
        hipError_t e0 = allow_dynamic_lds(head_kernel<HT, N, ONE, CONF, LOGITS>, lds);                 \
        if (e0 != hipSuccess) return e0;                                                               \
        mtp_launch((head_kernel<HT, N, ONE, CONF, LOGITS>), grid, dim3(kBlock), lds, st, a,     \
                           w_dtype);                                                                   \
        return hipGetLastError();                                                                      \
    }
    MTP_HEAD_CASE(1)
    MTP_HEAD_CASE(2)
    MTP_HEAD_CASE(4)
    MTP_HEAD_CASE(8)
#undef MTP_HEAD_CASE
    return hipErrorInvalidValue;
}

// LOGITS: the call may write logit rows (the one-sequence kernel without it
// has no store in its row loop); several sequences always check at run time.
template <typename HT, bool ONE>
static hipError_t launch_head_t(const HeadArgs &a, int w_dtype, int n_post_wg, bool logits, hipStream_t st) {
    if (ONE && !logits)
        return a.conf ? launch_head_c<HT, ONE, true, false>(a, w_dtype, n_post_wg, st)
                      : launch_head_c<HT, ONE, false, false>(a, w_dtype, n_post_wg, st);
    return a.conf ? launch_head_c<HT, ONE, true, true>(a, w_dtype, n_post_wg, st)
                  : launch_head_c<HT, ONE, false, true>(a, w_dtype, n_post_wg, st);
}

// ----------------------------------------------------------------------------
// Centroid head steps 3-5 ("Gemma 4 MTP" s.3): the candidate rows.
// ----------------------------------------------------------------------------
// Workgroup = (sequence, chunk of kCandChunk candidate rows).  The lane's
// slice of f = rmsnorm(x_s; g_final) lives in registers; each wave takes
// rows two at a time, looks up the token id through the chosen centroid's
// list, gathers that embedding row with 16-byte loads and reduces the dot
// across the wave.  Keys, confidence partials and (optionally) the logit
// scatter follow the dense head.  Workgroups past S * chunks run the
// post-projection exactly as in head_kernel.
static constexpr int kCandChunk = 32;

template <typename HT, int NV, bool CONF>
__global__ __launch_bounds__(256) void cand_head_kernel(HeadArgs a, int w_dtype, int chunks) {
    constexpr int EPV = WTr<HT>::EPV, CPW = 64 * EPV;
    constexpr int RU = 2;
    extern __shared__ float fs[];
    __shared__ float rs[kMaxSeqGroup];
    __shared__ uint64_t wbest[4];
    __shared__ float wcm[4], wcs[4];
    const int d = a.d, S = a.S;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    if ((int)blockIdx.x >= S * chunks) {         // post-projection rows
        for (int j = wid; j < S; j += 4) {
            const float *x = a.x + (int64_t)j * d;
            float ss = 0.f;
            for (int c = lane; c < d; c += 64) ss = fmaf(x[c], x[c], ss);
            ss = wave_sum(ss);
            if (lane == 0) rs[j] = 1.0f / sqrtf(ss / (float)d + a.eps);
        }
        __syncthreads();
        for (int i = tid; i < S * d; i += kBlock) {
            const int j = i / d, c = i - j * d;
            fs[i] = a.x[i] * rs[j] * a.g_final[c];
        }
        __syncthreads();
        float *h_out = (a.step == a.n_steps - 1 && a.io->out_h_last) ? a.io->out_h_last : a.h_out;
        if (w_dtype == MTP_BF16) post_rows<uint16_t>(a, fs, h_out);
        else post_rows<float>(a, fs, h_out);
        return;
    }
    const int s = blockIdx.x / chunks, ch = blockIdx.x - s * chunks;
    const int total = a.n_cand * a.vsc;
    const int r0 = ch * kCandChunk, r1 = min(total, r0 + kCandChunk);
    const int32_t *cand = a.cand + (int64_t)s * a.n_cand;
    auto row_of = [&](int r) {                  // ids outside the vocabulary are clamped into it
        const int q = r / a.vsc;
        return min(max(a.ordering[(int64_t)cand[q] * a.vsc + (r - q * a.vsc)], 0), a.V - 1);
    };
    uint4 wv[RU][NV];
    int tok[RU];
    auto load_rows = [&](int rb) {
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int r = rb + 4 * u;
            tok[u] = r < r1 ? row_of(r) : 0;
            const HT *er = (const HT *)a.head + (int64_t)tok[u] * d;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int col = v * CPW + lane * EPV;
                wv[u][v] = (r < r1 && col < d) ? *(const uint4 *)(er + col) : make_uint4(0, 0, 0, 0);
            }
        }
    };
    load_rows(r0 + wid);
    // f slice of this lane (all waves compute the norm of sequence s)
    float fr[NV][EPV];
    {
        const float *x = a.x + (int64_t)s * d;
        float ss = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int col = v * CPW + lane * EPV;
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                fr[v][e] = (col < d) ? x[col + e] : 0.f;
                ss = fmaf(fr[v][e], fr[v][e], ss);
            }
        }
        const float r = 1.0f / sqrtf(wave_sum(ss) / (float)d + a.eps);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int col = v * CPW + lane * EPV;
#pragma unroll
            for (int e = 0; e < EPV; ++e) fr[v][e] = (col < d) ? fr[v][e] * r * a.g_final[col + e] : 0.f;
        }
    }
    float *logits = a.io->out_logits ? a.io->out_logits + ((int64_t)s * a.n_steps + a.step) * a.V : nullptr;
    uint64_t best = 0ull;
    float cm = -INFINITY, cs = 0.f;
    for (int rb = r0 + wid; rb < r1; rb += 4 * RU) {
        if (rb != r0 + wid) load_rows(rb);
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int r = rb + 4 * u;
            if (r >= r1) break;                  // wave-uniform
            float acc = 0.f;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float w[EPV];
                widen(wv[u][v], w);
#pragma unroll
                for (int e = 0; e < EPV; ++e) acc = fmaf(w[e], fr[v][e], acc);
            }
            const float z = wave_sum(acc);
            const uint64_t k = argmax_key(z, (uint32_t)tok[u]);
            best = k > best ? k : best;
            if (CONF) conf_add(cm, cs, z);
            if (logits && lane == 0) logits[tok[u]] = z;
        }
    }
    if (lane == 0) {
        wbest[wid] = best;
        wcm[wid] = cm;
        wcs[wid] = cs;
    }
    __syncthreads();
    if (tid == 0) {
        uint64_t k = wbest[0];
        for (int w = 1; w < 4; ++w) k = wbest[w] > k ? wbest[w] : k;
        atomicMax((unsigned long long *)&a.keys[s], (unsigned long long)k);
        if (CONF) {
            float m = wcm[0], sm = wcs[0];
            for (int w = 1; w < 4; ++w) conf_merge(m, sm, wcm[w], wcs[w]);
            a.conf[(int64_t)s * kConfSlots + ch] = ConfPart{m, sm};
        }
    }
}

int cand_head_groups(const HeadArgs &a) {
    return std::min(kConfSlots, (a.n_cand * a.vsc + kCandChunk - 1) / kCandChunk);
}

template <typename HT, bool CONF>
static hipError_t launch_cand_t(const HeadArgs &a_in, int w_dtype, int n_post_wg, hipStream_t st) {
    constexpr int CPW = 64 * WTr<HT>::EPV;
    HeadArgs a = a_in;
    const int chunks = cand_head_groups(a);
    if ((int64_t)chunks * kCandChunk < (int64_t)a.n_cand * a.vsc) return hipErrorInvalidValue;
    a.n_head_wg = a.S * chunks;                 // post rows follow the candidate workgroups
    const int nv = (a.d + CPW - 1) / CPW;
    const size_t lds = sizeof(float) * (size_t)a.S * a.d;
    const dim3 grid(a.n_head_wg + n_post_wg);
#define MTP_CAND_CASE(N)                                                                               \
    if (nv <= N) {                                                                                     \
        hipError_t e0 = allow_dynamic_lds(cand_head_kernel<HT, N, CONF>, lds);                         \
        if (e0 != hipSuccess) return e0;                                                               \
        mtp_launch((cand_head_kernel<HT, N, CONF>), grid, dim3(kBlock), lds, st, a, w_dtype, chunks); \
        return hipGetLastError();                                                                      \
    }
    MTP_CAND_CASE(1)
    MTP_CAND_CASE(2)
    MTP_CAND_CASE(4)
    MTP_CAND_CASE(8)
#undef MTP_CAND_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_cand_head(int head_dtype, int w_dtype, const HeadArgs &a, int n_post_wg, bool logits,
                            hipStream_t st) {
    if (logits) {
        const hipError_t e = launch_fill_logits(a.io, a.S, a.n_steps, a.V, a.step, -1e30f, st);
        if (e != hipSuccess) return e;
    }
    const bool conf = a.conf != nullptr;
    if (head_dtype == MTP_BF16) return conf ? launch_cand_t<uint16_t, true>(a, w_dtype, n_post_wg, st)
                                            : launch_cand_t<uint16_t, false>(a, w_dtype, n_post_wg, st);
    if (head_dtype == MTP_F32) return conf ? launch_cand_t<float, true>(a, w_dtype, n_post_wg, st)
                                           : launch_cand_t<float, false>(a, w_dtype, n_post_wg, st);
    return hipErrorInvalidValue;
}

hipError_t launch_head(int head_dtype, int w_dtype, const HeadArgs &a, int n_post_wg, bool logits, hipStream_t st) {
    const bool one = a.S == 1;
    if (head_dtype == MTP_BF16) return one ? launch_head_t<uint16_t, true>(a, w_dtype, n_post_wg, logits, st)
                                           : launch_head_t<uint16_t, false>(a, w_dtype, n_post_wg, logits, st);
    if (head_dtype == MTP_Q8_0) return one ? launch_head_t<int8_t, true>(a, w_dtype, n_post_wg, logits, st)
                                           : launch_head_t<int8_t, false>(a, w_dtype, n_post_wg, logits, st);
    if (head_dtype == MTP_F32) return one ? launch_head_t<float, true>(a, w_dtype, n_post_wg, logits, st)
                                          : launch_head_t<float, false>(a, w_dtype, n_post_wg, logits, st);
    return hipErrorInvalidValue;
}

}  // namespace mtp
