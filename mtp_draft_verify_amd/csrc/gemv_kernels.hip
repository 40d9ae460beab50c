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

template <int IN>
__device__ void stage_input(const GemvArgs &a, float *xs, float *rs, int s0, int sg) {
    const int K = a.K, tid = threadIdx.x;
    if (IN == IN_NORM) {
        // 1 / rms per sequence: wave w reduces sequences w, w+4, ... (fixed order)
        const int lane = tid & 63, wid = tid >> 6;
        for (int j = wid; j < sg; j += 4) {
            const float *x = a.src + (int64_t)(s0 + j) * a.src_stride;
            float ss = 0.f;
            for (int c = lane; c < K; c += 64) ss = fmaf(x[c], x[c], ss);
            ss = wave_sum(ss);
            if (lane == 0) rs[j] = 1.0f / sqrtf(ss / (float)K + a.eps);
        }
        __syncthreads();
        for (int i = tid; i < sg * K; i += kBlock) {
            const int j = i / K, c = i - j * K;
            xs[i] = a.src[(int64_t)(s0 + j) * a.src_stride + c] * rs[j] * a.gain[c];
        }
    } else if (IN == IN_PLAIN) {
        for (int i = tid; i < sg * K; i += kBlock) {
            const int j = i / K, c = i - j * K;
            xs[i] = a.src[(int64_t)(s0 + j) * a.src_stride + c];
        }
    } else {   // IN_EMBED: [embed_scale * E[tok]; h]
        const int d = a.d_embed;
        for (int i = tid; i < sg * K; i += kBlock) {
            const int j = i / K, c = i - j * K, s = s0 + j;
            float v;
            if (c < d) {
                const int32_t tok = a.tok_in ? a.tok_in[s] : key_index(a.key_in[s]);
                float e;
                if (tok < 0 || tok >= a.embed_rows) e = 0.f;   // ids outside the vocabulary embed to zero
                else if (a.embed_dtype == MTP_F32) e = ((const float *)a.embed)[(int64_t)tok * d + c];
                else if (a.embed_dtype == MTP_BF16) e = bf16_to_f(((const uint16_t *)a.embed)[(int64_t)tok * d + c]);
                else e = half_to_f(a.embed_qs[(int64_t)tok * (d / 32) + c / 32]) * (float)a.embed_q[(int64_t)tok * d + c];
                v = a.embed_scale * e;
            } else {
                v = a.h[(int64_t)s * a.dh + (c - d)];
            }
            xs[i] = v;
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

template <typename WT, int NV, int IN, int EPI, bool ONE>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
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
    const int Sg = ONE ? 1 : min(kMaxSeqGroup, max(1, kLdsFloats / K));
    const int row0 = blockIdx.x * a.rows_per_wg;
    const int row1 = min(M, row0 + a.rows_per_wg);

    for (int s0 = 0; s0 < S; s0 += Sg) {
        const int sg = min(Sg, S - s0);
        __syncthreads();
        stage_input<IN>(a, xs, rs, s0, sg);
        __syncthreads();
        float xr[ONE ? NV : 1][EPV];
        if (ONE) {
#pragma unroll
            for (int v = 0; v < (ONE ? NV : 1); ++v) {
                const int col = v * CPW + lane * EPV;
#pragma unroll
                for (int e = 0; e < EPV; ++e) xr[v][e] = (col < K) ? xs[col + e] : 0.f;
            }
        }
        for (int rb = row0 + wid; rb < row1; rb += 4 * RU) {
            uint4 wv[RU][NV];
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const int r = rb + 4 * u;
                const uint4 *wr = (const uint4 *)((const WT *)a.W + (int64_t)r * K);
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int col = v * CPW + lane * EPV;
                    wv[u][v] = (r < row1 && col < K) ? wr[col / EPV] : make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const int r = rb + 4 * u;
                if (r >= row1) break;          // wave-uniform
                float w[NV][EPV];
#pragma unroll
                for (int v = 0; v < NV; ++v) widen(wv[u][v], w[v]);
                if (ONE) {
                    float acc = 0.f;
#pragma unroll
                    for (int v = 0; v < NV; ++v)
#pragma unroll
                        for (int e = 0; e < EPV; ++e) acc = fmaf(w[v][e], xr[ONE ? v : 0][e], acc);
                    const float y = wave_sum(acc);
                    if (lane == 0) gemv_store<EPI>(a, s0, r, y);
                } else {
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
        hipLaunchKernelGGL((gemv_kernel<WT, NV, I, E, ONE>), dim3(n_wg), dim3(kBlock), lds, st, a);    \
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
