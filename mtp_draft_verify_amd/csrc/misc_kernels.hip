// misc_kernels.hip -- small helpers of the draft chain: draft-id hand-off, Q8_0
// re-layout at context creation, key clearing.
#include "widen.h"

namespace mtp {

// ----------------------------------------------------------------------------
// small helpers
// ----------------------------------------------------------------------------
__global__ void finish_drafts_kernel(const uint64_t *keys, int32_t S, const CallIO *io, int32_t stride, int32_t col) {
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s < S) io->out_drafts[(int64_t)s * stride + col] = key_index(keys[s]);
}

hipError_t launch_finish_drafts(const uint64_t *keys, int32_t S, const CallIO *io, int32_t stride, int32_t col,
                                hipStream_t st) {
    hipLaunchKernelGGL(finish_drafts_kernel, dim3((S + 63) / 64), dim3(64), 0, st, keys, S, io, stride, col);
    return hipGetLastError();
}

// Q8_0 blocks (fp16 scale + 32 int8) -> int8 plane [rows, cols] + fp16 scale plane [rows, cols/32]
__global__ void q8_repack_kernel(const uint8_t *blocks, int64_t n_blocks, int8_t *q, uint16_t *s) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    const uint8_t *src = blocks + b * 34;
    s[b] = (uint16_t)(src[0] | (src[1] << 8));
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        w[i] = (uint32_t)src[2 + 4 * i] | ((uint32_t)src[3 + 4 * i] << 8) | ((uint32_t)src[4 + 4 * i] << 16) |
               ((uint32_t)src[5 + 4 * i] << 24);
    uint4 *dst = (uint4 *)(q + b * 32);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

hipError_t launch_q8_repack(const uint8_t *blocks, int64_t rows, int32_t cols, int8_t *q, uint16_t *s,
                            hipStream_t st) {
    const int64_t nb = rows * (cols / 32);
    hipLaunchKernelGGL(q8_repack_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, blocks, nb, q, s);
    return hipGetLastError();
}

__global__ void clear_u64_kernel(uint64_t *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0ull;
}

hipError_t launch_clear_u64(uint64_t *p, int64_t n, hipStream_t st) {
    hipLaunchKernelGGL(clear_u64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

// Per-step draft confidence and the p_min trim ("MTP decoding", stopping
// early when the head is unsure; "Fused NextN draft graph", risks: the
// per-step softmax maximum read back with the argmax).  One workgroup per
// sequence.  For each step the head workgroups' (max, sum exp) partials are
// merged in a fixed order -- thread t takes slots t, t + 256, ..., then a
// tree over the threads -- and conf = 1 / sum exp(z - max).  Thread 0 then
// keeps the leading steps with conf >= p_min and writes -1 over the rest.
__global__ __launch_bounds__(256) void conf_finish_kernel(const ConfPart *part, int32_t N, int32_t n_part,
                                                          int64_t step_stride, const CallIO *io) {
    __shared__ float tm[256], ts[256];
    __shared__ float conf_s[64];
    const int s = blockIdx.x, tid = threadIdx.x;
    for (int k = 0; k < N; ++k) {
        const ConfPart *p = part + k * step_stride + (int64_t)s * kConfSlots;
        float m = -INFINITY, sm = 0.f;
        for (int i = tid; i < n_part; i += 256) conf_merge(m, sm, p[i].m, p[i].s);
        tm[tid] = m;
        ts[tid] = sm;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if (tid < w) {
                float a = tm[tid], b = ts[tid];
                conf_merge(a, b, tm[tid + w], ts[tid + w]);
                tm[tid] = a;
                ts[tid] = b;
            }
            __syncthreads();
        }
        if (tid == 0) conf_s[k] = 1.0f / ts[0];
        __syncthreads();
    }
    if (tid == 0) {
        const float p_min = io->p_min;
        int keep = N;
        for (int k = 0; k < N; ++k) {
            if (io->out_conf) io->out_conf[(int64_t)s * N + k] = conf_s[k];
            if (keep == N && conf_s[k] < p_min) keep = k;
        }
        for (int k = keep; k < N; ++k) io->out_drafts[(int64_t)s * N + k] = -1;
        if (io->out_n_keep) io->out_n_keep[s] = keep;
    }
}

hipError_t launch_conf_finish(const ConfPart *part, int32_t S, int32_t N, int32_t n_part, int64_t step_stride,
                              const CallIO *io, hipStream_t st) {
    if (N > 64 || n_part > kConfSlots) return hipErrorInvalidValue;
    hipLaunchKernelGGL(conf_finish_kernel, dim3(S), dim3(256), 0, st, part, N, n_part, step_stride, io);
    return hipGetLastError();
}

// RoPE frequencies theta^(-2i/hd), i < hd/2, in fp64 (once per context)
__global__ void rope_init_kernel(double *inv_freq, int32_t hd, double theta) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < hd / 2) inv_freq[i] = pow(theta, -2.0 * (double)i / (double)hd);
}

hipError_t launch_rope_init(double *inv_freq, int32_t hd, float theta, hipStream_t st) {
    hipLaunchKernelGGL(rope_init_kernel, dim3((hd / 2 + 63) / 64), dim3(64), 0, st, inv_freq, hd, (double)theta);
    return hipGetLastError();
}

}  // namespace mtp
