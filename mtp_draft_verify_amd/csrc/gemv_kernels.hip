// gemv_kernels.hip -- GEMVs of the draft chain (pre-projection, Q, O, up, down).
//
// dst[s, r] (op)= sum_c W[r, c] in[s, c] for all sequences of the call.  Each
// weight row is read once per sequence group with 16-byte coalesced loads; the
// transformed input (plain, RMSNorm with gain, or the token-embedding /
// hidden-state concat of the "Gemma 4 MTP" doc s.4 steps 2-3) is staged in LDS.
// HBM-bound: about one flop per weight byte per sequence.  With one sequence
// the input slice of each lane lives in registers for the whole row loop.
#include "widen.h"

namespace mtp {

// Column slice of lane `lane` in a row of K values: vectors v = 0..NV-1 of EPV
// consecutive values starting at v*64*EPV + lane*EPV.  Every sum of squares
// (RMSNorm) runs over these slices in this order and finishes with wave_sum,
// whether the input sits in registers (one sequence) or in LDS (several), so
// a sequence gets the same bits alone or in a batch.
template <int NV, int EPV>
__device__ __forceinline__ float slice_sumsq(const float *x, int K, int lane) {
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int col = v * 64 * EPV + lane * EPV;
        if (col < K)
#pragma unroll
            for (int e = 0; e < EPV; ++e) ss = fmaf(x[col + e], x[col + e], ss);
    }
    return wave_sum(ss);
}

__device__ __forceinline__ float embed_value(const GemvArgs &a, int s, int c) {
    const int d = a.d_embed;
    if (c >= d) return a.h[(int64_t)s * a.dh + (c - d)];
    const int32_t tok = a.tok_in ? a.tok_in[s] : key_index(a.key_in[s]);
    float e;
    if (tok < 0 || tok >= a.embed_rows) e = 0.f;   // ids outside the vocabulary embed to zero
    else if (a.embed_dtype == MTP_F32) e = ((const float *)a.embed)[(int64_t)tok * d + c];
    else if (a.embed_dtype == MTP_BF16) e = bf16_to_f(((const uint16_t *)a.embed)[(int64_t)tok * d + c]);
    else e = half_to_f(a.embed_qs[(int64_t)tok * (d / 32) + c / 32]) * (float)a.embed_q[(int64_t)tok * d + c];
    return a.embed_scale * e;
}

// Token whose embedding row sequence s gathers: the caller's id at step 0,
// the previous step's argmax afterwards.
__device__ __forceinline__ int32_t embed_token(const GemvArgs &a, int s) {
    return a.tok_in ? a.tok_in[s] : key_index(a.key_in[s]);
}

// embed_scale * E[tok, col .. col + EPV) with vector loads (col < d_embed,
// a multiple of EPV); the same values embed_value gives element by element.
template <int EPV>
__device__ __forceinline__ void load_embed_slice(const GemvArgs &a, int32_t tok, int col, float (&x)[EPV]) {
    if (tok < 0 || tok >= a.embed_rows) {   // ids outside the vocabulary embed to zero
#pragma unroll
        for (int e = 0; e < EPV; ++e) x[e] = 0.f;
        return;
    }
    const int64_t off = (int64_t)tok * a.d_embed + col;
    if (a.embed_dtype == MTP_F32) {
        const float4 *p = (const float4 *)((const float *)a.embed + off);
#pragma unroll
        for (int e4 = 0; e4 < EPV / 4; ++e4) {
            const float4 v = p[e4];
            x[4 * e4 + 0] = v.x; x[4 * e4 + 1] = v.y; x[4 * e4 + 2] = v.z; x[4 * e4 + 3] = v.w;
        }
    } else if (a.embed_dtype == MTP_BF16) {
        const uint32_t *p = (const uint32_t *)((const uint16_t *)a.embed + off);
#pragma unroll
        for (int e2 = 0; e2 < EPV / 2; ++e2) {
            const uint32_t w = p[e2];
            x[2 * e2] = bf16_lo(w);
            x[2 * e2 + 1] = bf16_hi(w);
        }
    } else {
        const float sc = half_to_f(a.embed_qs[(int64_t)tok * (a.d_embed / 32) + col / 32]);
        const int8_t *q = a.embed_q + off;
#pragma unroll
        for (int e = 0; e < EPV; ++e) x[e] = sc * (float)q[e];
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) x[e] *= a.embed_scale;
}

// The EPV input values of sequence s at columns [col, col + EPV), loaded with
// 16-byte vectors (EPV is 4 or 8 and divides d_model, so a slice never
// straddles the embedding / hidden-state boundary).
template <int IN, int EPV>
__device__ __forceinline__ void load_x_slice(const GemvArgs &a, int s, int col, float (&x)[EPV]) {
    if (IN != IN_EMBED) {
        const float4 *p = (const float4 *)(a.src + (int64_t)s * a.src_stride + col);
#pragma unroll
        for (int e4 = 0; e4 < EPV / 4; ++e4) {
            const float4 v = p[e4];
            x[4 * e4 + 0] = v.x; x[4 * e4 + 1] = v.y; x[4 * e4 + 2] = v.z; x[4 * e4 + 3] = v.w;
        }
        return;
    }
    const int d = a.d_embed;
    if (col >= d) {
        const float4 *p = (const float4 *)(a.h + (int64_t)s * a.dh + (col - d));
#pragma unroll
        for (int e4 = 0; e4 < EPV / 4; ++e4) {
            const float4 v = p[e4];
            x[4 * e4 + 0] = v.x; x[4 * e4 + 1] = v.y; x[4 * e4 + 2] = v.z; x[4 * e4 + 3] = v.w;
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) x[e] = embed_value(a, s, col + e);
}

// Stage the transformed inputs of sequences s0 .. s0+sg-1 into LDS (several
// sequences per call).
template <int IN, int NV, int EPV>
__device__ void stage_input(const GemvArgs &a, float *xs, float *rs, int s0, int sg) {
    const int K = a.K, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    for (int i = tid; i < sg * K; i += kBlock) {
        const int j = i / K, c = i - j * K;
        xs[i] = (IN == IN_EMBED) ? embed_value(a, s0 + j, c) : a.src[(int64_t)(s0 + j) * a.src_stride + c];
    }
    if (IN == IN_NORM) {
        __syncthreads();
        for (int j = wid; j < sg; j += 4) {
            const float ss = slice_sumsq<NV, EPV>(xs + j * K, K, lane);
            if (lane == 0) rs[j] = 1.0f / sqrtf(ss / (float)K + a.eps);
        }
        __syncthreads();
        for (int i = tid; i < sg * K; i += kBlock) {
            const int j = i / K, c = i - j * K;
            xs[i] = xs[i] * rs[j] * a.gain[c];
        }
    }
}

template <int EPI>
__device__ __forceinline__ void gemv_store(const GemvArgs &a, int s, int r, float y) {
    float *dp = a.dst + (int64_t)s * a.dst_stride + r;
    if (EPI == EPI_STORE) *dp = y;
    else if (EPI == EPI_ADD) *dp = *dp + y;
    else *dp = silu_f(y);
}

template <typename WT, int NV, int RU>
__device__ __forceinline__ void load_rows(const GemvArgs &a, int rb, int row1, int lane, uint4 (&wv)[RU][NV]) {
    constexpr int EPV = WTr<WT>::EPV, CPW = 64 * EPV;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        const int r = rb + 4 * u;
        const uint4 *wr = (const uint4 *)((const WT *)a.W + (int64_t)r * a.K);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int col = v * CPW + lane * EPV;
            wv[u][v] = (r < row1 && col < a.K) ? wr[col / EPV] : make_uint4(0, 0, 0, 0);
        }
    }
}

// One workgroup = 4 waves over rows [row0, row1); wave w takes rows
// row0 + w, row0 + w + 4, ... two at a time.  The first rows' weights are
// requested before the input is read, so the two latencies overlap.
template <typename WT, int NV, int IN, int EPI, bool ONE>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a_in) {
    GemvArgs a = a_in;
    if (IN == IN_EMBED) {   // caller buffers of this call
        a.tok_in = a.step == 0 ? a.io->last_tok : nullptr;
        if (a.step == 0) a.h = a.io->h_prev;
        a.drafts_out = a.step > 0 ? a.io->out_drafts : nullptr;
    }
    constexpr int EPV = WTr<WT>::EPV;
    constexpr int CPW = 64 * EPV;
    constexpr int RU = 2;                  // rows in flight per wave
    extern __shared__ float xs[];
    __shared__ float rs[kMaxSeqGroup];
    const int K = a.K, M = a.M, S = a.S;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

    if (IN == IN_EMBED && blockIdx.x == 0 && tid < S) {
        if (a.drafts_out) a.drafts_out[(int64_t)tid * a.drafts_stride + a.drafts_col] = key_index(a.key_in[tid]);
        if (a.key_reset) a.key_reset[tid] = 0ull;
    }
    const int row0 = blockIdx.x * a.rows_per_wg;
    const int row1 = min(M, row0 + a.rows_per_wg);

    if constexpr (ONE) {
        // One sequence: the lane's input slice lives in registers, no LDS.
        // Every load this wave needs (weights of its first rows, input slice,
        // gains, residual) is issued before any arithmetic.
        int rb = row0 + wid;
        uint4 wv[RU][NV];
        load_rows<WT, NV, RU>(a, rb, row1, lane, wv);
        float xr[NV][EPV], gr[NV][EPV];
        if (IN == IN_EMBED) {
            // the hidden-state part first: it does not wait for the token
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int col = v * CPW + lane * EPV;
                if (col < K && col >= a.d_embed) load_x_slice<IN, EPV>(a, 0, col, xr[v]);
            }
            const int32_t tok = embed_token(a, 0);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int col = v * CPW + lane * EPV;
                if (col < a.d_embed) load_embed_slice<EPV>(a, tok, col, xr[v]);
                else if (col >= K)
#pragma unroll
                    for (int e = 0; e < EPV; ++e) xr[v][e] = 0.f;
            }
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int col = v * CPW + lane * EPV;
            if (IN == IN_EMBED) continue;
            if (col < K) {
                load_x_slice<IN, EPV>(a, 0, col, xr[v]);
                if (IN == IN_NORM) {
                    const float4 *gp = (const float4 *)(a.gain + col);
#pragma unroll
                    for (int e4 = 0; e4 < EPV / 4; ++e4) {
                        const float4 g4 = gp[e4];
                        gr[v][4 * e4 + 0] = g4.x; gr[v][4 * e4 + 1] = g4.y;
                        gr[v][4 * e4 + 2] = g4.z; gr[v][4 * e4 + 3] = g4.w;
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPV; ++e) xr[v][e] = gr[v][e] = 0.f;
            }
        }
        float res[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u)
            res[u] = (EPI == EPI_ADD && lane == 0 && rb + 4 * u < row1) ? a.dst[rb + 4 * u] : 0.f;
        if (IN == IN_NORM) {
            float ss = 0.f;
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int e = 0; e < EPV; ++e) ss = fmaf(xr[v][e], xr[v][e], ss);
            const float r = 1.0f / sqrtf(wave_sum(ss) / (float)K + a.eps);
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int e = 0; e < EPV; ++e) xr[v][e] = xr[v][e] * r * gr[v][e];
        }
        for (; rb < row1; rb += 4 * RU) {
            uint4 wn[RU][NV];
            if (rb + 4 * RU < row1) load_rows<WT, NV, RU>(a, rb + 4 * RU, row1, lane, wn);
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const int r = rb + 4 * u;
                if (r >= row1) break;          // wave-uniform
                float acc = 0.f;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    float w[EPV];
                    widen(wv[u][v], w);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) acc = fmaf(w[e], xr[v][e], acc);
                }
                const float y = wave_sum(acc);
                if (lane == 0) {
                    if (EPI == EPI_ADD) a.dst[r] = res[u] + y;
                    else gemv_store<EPI>(a, 0, r, y);
                }
            }
#pragma unroll
            for (int u = 0; u < RU; ++u) {
#pragma unroll
                for (int v = 0; v < NV; ++v) wv[u][v] = wn[u][v];
                res[u] = (EPI == EPI_ADD && lane == 0 && rb + 4 * RU + 4 * u < row1) ? a.dst[rb + 4 * RU + 4 * u] : 0.f;
            }
        }
        return;
    } else {
        const int Sg = min(kMaxSeqGroup, max(1, kLdsFloats / K));
        for (int s0 = 0; s0 < S; s0 += Sg) {
            const int sg = min(Sg, S - s0);
            int rb = row0 + wid;
            uint4 wv[RU][NV];
            load_rows<WT, NV, RU>(a, rb, row1, lane, wv);
            __syncthreads();
            stage_input<IN, NV, EPV>(a, xs, rs, s0, sg);
            __syncthreads();
            for (; rb < row1; rb += 4 * RU) {
                uint4 wn[RU][NV];
                if (rb + 4 * RU < row1) load_rows<WT, NV, RU>(a, rb + 4 * RU, row1, lane, wn);
#pragma unroll
                for (int u = 0; u < RU; ++u) {
                    const int r = rb + 4 * u;
                    if (r >= row1) break;          // wave-uniform
                    float w[NV][EPV];
#pragma unroll
                    for (int v = 0; v < NV; ++v) widen(wv[u][v], w[v]);
                    for (int j = 0; j < sg; ++j) {
                        float acc = 0.f;
#pragma unroll
                        for (int v = 0; v < NV; ++v) {
                            const int col = v * CPW + lane * EPV;
                            if (col < K) {
                                const float4 *xp = (const float4 *)(xs + j * K + col);
#pragma unroll
                                for (int e4 = 0; e4 < EPV / 4; ++e4) {
                                    const float4 xv = xp[e4];
                                    acc = fmaf(w[v][4 * e4 + 0], xv.x, acc);
                                    acc = fmaf(w[v][4 * e4 + 1], xv.y, acc);
                                    acc = fmaf(w[v][4 * e4 + 2], xv.z, acc);
                                    acc = fmaf(w[v][4 * e4 + 3], xv.w, acc);
                                }
                            }
                        }
                        const float y = wave_sum(acc);
                        if (lane == 0) gemv_store<EPI>(a, s0 + j, r, y);
                    }
                }
#pragma unroll
                for (int u = 0; u < RU; ++u)
#pragma unroll
                    for (int v = 0; v < NV; ++v) wv[u][v] = wn[u][v];
            }
        }
    }
}

template <typename WT, int NV, bool ONE>
static hipError_t launch_gemv_nv(int in_mode, int epi, const GemvArgs &a, int n_wg, hipStream_t st) {
    const int Sg = ONE ? 1 : std::min(kMaxSeqGroup, std::max(1, kLdsFloats / a.K));
    const size_t lds = sizeof(float) * (size_t)Sg * a.K;
#define MTP_GEMV_CASE(I, E)                                                                             \
    if (in_mode == I && epi == E) {                                                                     \
        hipError_t e0 = allow_dynamic_lds(gemv_kernel<WT, NV, I, E, ONE>, lds);                         \
        if (e0 != hipSuccess) return e0;                                                                \
        mtp_launch((gemv_kernel<WT, NV, I, E, ONE>), dim3(n_wg), dim3(kBlock), lds, st, a);    \
        return hipGetLastError();                                                                       \
    }
    MTP_GEMV_CASE(IN_EMBED, EPI_STORE)
    MTP_GEMV_CASE(IN_NORM, EPI_STORE)
    MTP_GEMV_CASE(IN_NORM, EPI_SILU)
    MTP_GEMV_CASE(IN_PLAIN, EPI_ADD)
#undef MTP_GEMV_CASE
    return hipErrorInvalidValue;
}

template <typename WT, bool ONE>
static hipError_t launch_gemv_t(int in_mode, int epi, const GemvArgs &a, int n_wg, hipStream_t st) {
    constexpr int CPW = 64 * WTr<WT>::EPV;
    const int nv = (a.K + CPW - 1) / CPW;
    if (nv <= 1) return launch_gemv_nv<WT, 1, ONE>(in_mode, epi, a, n_wg, st);
    if (nv <= 2) return launch_gemv_nv<WT, 2, ONE>(in_mode, epi, a, n_wg, st);
    if (nv <= 4) return launch_gemv_nv<WT, 4, ONE>(in_mode, epi, a, n_wg, st);
    if (nv <= 8) return launch_gemv_nv<WT, 8, ONE>(in_mode, epi, a, n_wg, st);
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(int w_dtype, int in_mode, int epi, const GemvArgs &a, int n_wg, hipStream_t st) {
    const bool one = a.S == 1;
    if (w_dtype == MTP_F32) return one ? launch_gemv_t<float, true>(in_mode, epi, a, n_wg, st)
                                       : launch_gemv_t<float, false>(in_mode, epi, a, n_wg, st);
    if (w_dtype == MTP_BF16) return one ? launch_gemv_t<uint16_t, true>(in_mode, epi, a, n_wg, st)
                                        : launch_gemv_t<uint16_t, false>(in_mode, epi, a, n_wg, st);
    return hipErrorInvalidValue;
}

}  // namespace mtp
