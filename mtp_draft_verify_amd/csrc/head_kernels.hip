// head_kernels.hip -- final RMSNorm + tied LM head + greedy argmax, fused with
// the post-projection ("Gemma 4 MTP" doc s.4 steps 5-8; "Fused NextN draft
// graph": the argmax stays on the device and feeds the next step).
//
// The head is the largest stream of a step (V x d weights).  Rows are read
// with non-temporal 16-byte loads (so the block weights and the KV cache keep
// their cache residency), several rows in flight per wave, and each workgroup
// folds its best (value, lowest index) per sequence into one 64-bit key with
// atomicMax.  Workgroups past n_head_wg compute h' = W_post f instead.
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

template <typename HT, int NV, bool ONE, bool CONF>
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
    auto load_head_rows = [&](int rb) {
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int r = rb + u;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int col = v * CPW + lane * EPV;
                const bool ok = (r < r1) && (col < d);
                if constexpr (sizeof(HT) == 1) {
                    wv[u][v] = ok ? ld_nt((const uint4 *)(a.head_q + (int64_t)r * d + col)) : make_uint4(0, 0, 0, 0);
                    sc[u][v] = ok ? half_to_f(a.head_qs[(int64_t)r * nblk + col / 32]) : 0.f;
                } else {
                    wv[u][v] = ok ? ld_nt((const uint4 *)((const HT *)a.head + (int64_t)r * d + col))
                                  : make_uint4(0, 0, 0, 0);
                    sc[u][v] = 1.f;
                }
            }
        }
    };
    // the first rows' weights do not depend on x: request them before the prologue
    const bool head_wg = (int)blockIdx.x < a.n_head_wg;
    if (head_wg) load_head_rows(r0 + wid * RU);

    // f = rmsnorm(x; g_final)
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

    if ((int)blockIdx.x >= a.n_head_wg) {
        float *h_out = (a.step == a.n_steps - 1 && a.io->out_h_last) ? a.io->out_h_last : a.h_out;
        if (w_dtype == MTP_BF16) post_rows<uint16_t>(a, fs, h_out);
        else post_rows<float>(a, fs, h_out);
        return;
    }
    float *logits = a.io->out_logits ? a.io->out_logits + (int64_t)a.step * a.V : nullptr;
    const int64_t logits_stride = (int64_t)a.n_steps * a.V;

    float fr[ONE ? NV : 1][EPV];
    if (ONE) {
#pragma unroll
        for (int v = 0; v < (ONE ? NV : 1); ++v) {
            const int col = v * CPW + lane * EPV;
#pragma unroll
            for (int e = 0; e < EPV; ++e) fr[v][e] = (col < d) ? fs[col + e] : 0.f;
        }
    }
    uint64_t best1 = 0ull;                  // one-sequence path keeps its best in a register
    float cm1 = -INFINITY, cs1 = 0.f;       // and its confidence partial
    constexpr bool conf = CONF;             // confidence partials requested
    for (int rb = r0 + wid * RU; rb < r1; rb += 4 * RU) {
        if (rb != r0 + wid * RU) load_head_rows(rb);
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int r = rb + u;
            if (r >= r1) break;                 // wave-uniform
            float w[NV][EPV];
#pragma unroll
            for (int v = 0; v < NV; ++v) widen(wv[u][v], w[v]);
            for (int j = 0; j < (ONE ? 1 : S); ++j) {
                float acc = 0.f;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    float part = 0.f;
                    if (ONE) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) part = fmaf(w[v][e], fr[ONE ? v : 0][e], part);
                    } else {
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
                    }
                    acc = fmaf(part, sc[u][v], acc);
                }
                const float z = wave_sum(acc);
                if (logits && lane == 0) logits[(int64_t)j * logits_stride + r] = z;
                const uint64_t k = argmax_key(z, (uint32_t)r);
                if (ONE) {
                    best1 = k > best1 ? k : best1;
                    if (conf) conf_add(cm1, cs1, z);
                } else if (lane == 0) {         // only lane 0 of this wave touches these slots
                    if (k > wbest[wid][j]) wbest[wid][j] = k;
                    if (conf) conf_add(wcm[wid][j], wcs[wid][j], z);
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

template <typename HT, bool ONE, bool CONF>
static hipError_t launch_head_c(const HeadArgs &a, int w_dtype, int n_post_wg, hipStream_t st) {
    constexpr int CPW = 64 * WTr<HT>::EPV;
    const int nv = (a.d + CPW - 1) / CPW;
    const size_t lds = sizeof(float) * (size_t)a.S * a.d;
    dim3 grid(a.n_head_wg + n_post_wg);
#define MTP_HEAD_CASE(N)                                                                               \
    if (nv <= N) {                                                                                     \
        hipError_t e0 = allow_dynamic_lds(head_kernel<HT, N, ONE, CONF>, lds);                         \
        if (e0 != hipSuccess) return e0;                                                               \
        hipLaunchKernelGGL((head_kernel<HT, N, ONE, CONF>), grid, dim3(kBlock), lds, st, a, w_dtype);  \
        return hipGetLastError();                                                                      \
    }
    MTP_HEAD_CASE(1)
    MTP_HEAD_CASE(2)
    MTP_HEAD_CASE(4)
    MTP_HEAD_CASE(8)
#undef MTP_HEAD_CASE
    return hipErrorInvalidValue;
}

template <typename HT, bool ONE>
static hipError_t launch_head_t(const HeadArgs &a, int w_dtype, int n_post_wg, hipStream_t st) {
    return a.conf ? launch_head_c<HT, ONE, true>(a, w_dtype, n_post_wg, st)
                  : launch_head_c<HT, ONE, false>(a, w_dtype, n_post_wg, st);
}

hipError_t launch_head(int head_dtype, int w_dtype, const HeadArgs &a, int n_post_wg, hipStream_t st) {
    const bool one = a.S == 1;
    if (head_dtype == MTP_BF16) return one ? launch_head_t<uint16_t, true>(a, w_dtype, n_post_wg, st)
                                           : launch_head_t<uint16_t, false>(a, w_dtype, n_post_wg, st);
    if (head_dtype == MTP_Q8_0) return one ? launch_head_t<int8_t, true>(a, w_dtype, n_post_wg, st)
                                           : launch_head_t<int8_t, false>(a, w_dtype, n_post_wg, st);
    if (head_dtype == MTP_F32) return one ? launch_head_t<float, true>(a, w_dtype, n_post_wg, st)
                                          : launch_head_t<float, false>(a, w_dtype, n_post_wg, st);
    return hipErrorInvalidValue;
}

}  // namespace mtp
