// verify_kernels.hip -- gfx950 kernels of the greedy verify step.
//
// "MTP decoding (--mtp)", How it is wired: the target decodes [confirmed,
// drafts...] with logits at every position; the longest prefix of drafts that
// equals the per-row argmax is accepted and the first unverified row supplies
// the next token.  Pass 1 streams the fp32 logits once (8192 values per
// workgroup, 16-byte loads) and folds each chunk's (max, lowest index) into a
// 64-bit key per row with atomicMax; pass 2 does the prefix match per
// sequence, writes the outputs and clears the keys for the next call.
#include "dev_common.h"

namespace mtp {

static constexpr int kVerifyChunk = 8192;

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t o = shfl_xor_u64(k, m);
        k = o > k ? o : k;
    }
    return k;
}

__global__ __launch_bounds__(256) void verify_argmax_kernel(const float *logits, int32_t n_chunk, int32_t V,
                                                            uint64_t *keys) {
    __shared__ uint64_t wk[4];
    const int chunk = blockIdx.x % n_chunk;
    const int64_t row_id = blockIdx.x / n_chunk;     // s * R + r
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const float *row = logits + row_id * V;
    const int c0 = chunk * kVerifyChunk;
    const int c1 = min(V, c0 + kVerifyChunk);
    uint64_t best = 0ull;
    if ((V & 3) == 0 && ((uintptr_t)logits & 15) == 0) {
        // all 8 vectors of the thread are requested at once (clamped into the
        // chunk; those past its end are dropped), then folded
        constexpr int NI = kVerifyChunk / (kBlock * 4);
        float4 v[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) v[i] = ld_nt((const float4 *)(row + min(c0 + tid * 4 + kBlock * 4 * i, c1 - 4)));
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = c0 + tid * 4 + kBlock * 4 * i;
            uint64_t k0 = argmax_key(v[i].x, c), k1 = argmax_key(v[i].y, c + 1);
            uint64_t k2 = argmax_key(v[i].z, c + 2), k3 = argmax_key(v[i].w, c + 3);
            k0 = k1 > k0 ? k1 : k0;
            k2 = k3 > k2 ? k3 : k2;
            k0 = k2 > k0 ? k2 : k0;
            best = (c < c1 && k0 > best) ? k0 : best;
        }
    } else {
        for (int c = c0 + tid; c < c1; c += kBlock) {
            const uint64_t k = argmax_key(row[c], c);
            best = k > best ? k : best;
        }
    }
    best = wave_max_u64(best);
    if (lane == 0) wk[wid] = best;
    __syncthreads();
    if (tid == 0) {
        uint64_t k = wk[0];
        for (int w = 1; w < 4; ++w) k = wk[w] > k ? wk[w] : k;
        atomicMax((unsigned long long *)&keys[row_id], (unsigned long long)k);
    }
}

__global__ void verify_prefix_kernel(const int32_t *drafts, int32_t S, int32_t N, uint64_t *keys, int32_t *out_tokens,
                                     int32_t *out_n_accept) {
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= S) return;
    const int R = N + 1;
    uint64_t *k = keys + (int64_t)s * R;
    int a = 0;
    while (a < N && drafts[(int64_t)s * N + a] == key_index(k[a])) ++a;
    for (int i = 0; i < R; ++i) {
        out_tokens[(int64_t)s * R + i] = (i <= a) ? key_index(k[i]) : -1;
        k[i] = 0ull;
    }
    out_n_accept[s] = a;
}

hipError_t launch_verify_greedy(const float *logits, const int32_t *drafts, int32_t S, int32_t N, int32_t V,
                                uint64_t *keys, int32_t *out_tokens, int32_t *out_n_accept, hipStream_t st) {
    const int64_t n_chunk = (V + kVerifyChunk - 1) / kVerifyChunk;
    const int64_t n_wg = n_chunk * (int64_t)(N + 1) * S;
    if (n_wg > 0x7FFFFFFF) return hipErrorInvalidValue;
    mtp_launch(verify_argmax_kernel, dim3((unsigned)n_wg), dim3(kBlock), 0, st, logits, (int32_t)n_chunk, V,
                       keys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_verify_prefix(drafts, S, N, keys, out_tokens, out_n_accept, st);
}

hipError_t launch_verify_prefix(const int32_t *drafts, int32_t S, int32_t N, uint64_t *keys, int32_t *out_tokens,
                                int32_t *out_n_accept, hipStream_t st) {
    mtp_launch(verify_prefix_kernel, dim3((S + 63) / 64), dim3(64), 0, st, drafts, S, N, keys, out_tokens,
                       out_n_accept);
    return hipGetLastError();
}

}  // namespace mtp
