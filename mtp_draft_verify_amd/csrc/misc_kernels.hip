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
    mtp_launch(finish_drafts_kernel, dim3((S + 63) / 64), dim3(64), 0, st, keys, S, io, stride, col);
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
    mtp_launch(q8_repack_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, blocks, nb, q, s);
    return hipGetLastError();
}

// Q8_0 blocks -> unit order (layout in mtp_internal.h): one thread per
// 16-byte piece of the output.
__global__ void q8_unit_order_kernel(const uint8_t *blocks, int64_t rows, int32_t cols, int64_t n_pieces,
                                     uint8_t *out) {
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= n_pieces) return;
    constexpr int kPieces = kQ8UnitBytes / 16;
    const int upc = cols / 256, nblk = cols / 32;
    const int64_t unit = id / kPieces;
    const int w = (int)(id - unit * kPieces);
    const int64_t t = unit / upc;
    const int c = (int)(unit - t * upc);
    auto byte_at = [&](int64_t row, int b, int off) -> uint32_t { return blocks[(row * nblk + b) * 34 + off]; };
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    if (w < 256) {
        const int p = w >> 6, l = w & 63, g = l >> 4, j = l & 15;
        const int64_t row = 16 * t + j;
        if (row < rows) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int b = 8 * c + 2 * p + h;
#pragma unroll
                for (int wd = 0; wd < 2; ++wd) {
                    const int off = 2 + 8 * g + 4 * wd;
                    v[2 * h + wd] = byte_at(row, b, off) | (byte_at(row, b, off + 1) << 8) |
                                    (byte_at(row, b, off + 2) << 16) | (byte_at(row, b, off + 3) << 24);
                }
            }
        }
    } else {
        const int j = w - 256;
        const int64_t row = 16 * t + j;
        if (row < rows) {
#pragma unroll
            for (int k = 0; k < 8; k += 2)
                v[k / 2] = byte_at(row, 8 * c + k, 0) | (byte_at(row, 8 * c + k, 1) << 8) |
                           (byte_at(row, 8 * c + k + 1, 0) << 16) | (byte_at(row, 8 * c + k + 1, 1) << 24);
        }
    }
    *(uint4 *)(out + id * 16) = make_uint4(v[0], v[1], v[2], v[3]);
}

size_t q8_unit_order_bytes(int64_t rows, int32_t cols) {
    return (size_t)((rows + 15) / 16) * (size_t)(cols / 256) * kQ8UnitBytes;
}

hipError_t launch_q8_unit_order(const uint8_t *blocks, int64_t rows, int32_t cols, uint8_t *out, hipStream_t st) {
    if (cols % 256 != 0) return hipErrorInvalidValue;
    const int64_t n_pieces = (int64_t)(q8_unit_order_bytes(rows, cols) / 16);
    mtp_launch(q8_unit_order_kernel, dim3((unsigned)((n_pieces + 255) / 256)), dim3(256), 0, st, blocks, rows,
                       cols, n_pieces, out);
    return hipGetLastError();
}

__global__ void clear_u64_kernel(uint64_t *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0ull;
}

hipError_t launch_clear_u64(uint64_t *p, int64_t n, hipStream_t st) {
    mtp_launch(clear_u64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
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
    mtp_launch(conf_finish_kernel, dim3(S), dim3(256), 0, st, part, N, n_part, step_stride, io);
    return hipGetLastError();
}

// Centroid head step 2 ("Gemma 4 MTP" s.3): the top-k centroids of each
// sequence, one workgroup per sequence.  Centroid c gets the argmax key
// (ordered logit << 32 | ~c): larger logit first, lower id first among equal
// logits, and every key distinct.  A radix select from the top byte down
// finds the k-th largest key -- per byte, a histogram of the keys that still
// match the chosen prefix, then one wave scans the 256 bins from the top --
// stopping as soon as the chosen bin holds exactly the keys still needed.
// The k keys at or above it are gathered and sorted (bitonic, one wave), so
// the chosen centroids come out best first whatever order the gather took.
static constexpr int kTopkPerThread = kMaxCentroids / 256;

__global__ __launch_bounds__(256) void centroid_topk_kernel(const float *cl, int32_t nc, int32_t k, int32_t *cand) {
    __shared__ uint32_t hist[256];
    __shared__ uint64_t sel[kMaxCentroidTopK];
    __shared__ uint64_t s_prefix, s_mask;
    __shared__ int32_t s_need, s_done, s_nsel;
    const int s = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    uint64_t key[kTopkPerThread];
#pragma unroll
    for (int i = 0; i < kTopkPerThread; ++i) {
        const int c = tid + 256 * i;
        key[i] = c < nc ? argmax_key(cl[(int64_t)s * nc + c], (uint32_t)c) : 0ull;
    }
    if (tid == 0) {
        s_prefix = 0ull;
        s_mask = 0ull;
        s_need = k;
        s_done = 0;
        s_nsel = 0;
    }
    for (int shift = 56; shift >= 0; shift -= 8) {
        hist[tid] = 0u;
        __syncthreads();
        const uint64_t prefix = s_prefix, mask = s_mask;
        if (s_done) break;                       // uniform: read after the barrier
#pragma unroll
        for (int i = 0; i < kTopkPerThread; ++i)
            if (tid + 256 * i < nc && (key[i] & mask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
        __syncthreads();
        if (tid < 64) {
            // lane l holds bins 255-4l .. 252-4l (top down); inclusive scan over lanes
            uint32_t part = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) part += hist[255 - 4 * lane - j];
            uint32_t cum = part;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_up(cum, off);
                if (lane >= off) cum += o;
            }
            const uint32_t need = (uint32_t)s_need;
            const uint64_t hit = __ballot(cum >= need);
            const int l0 = __ffsll((unsigned long long)hit) - 1;     // first lane reaching need
            if (lane == l0) {
                uint32_t c = cum - part;                 // keys in higher bins
                for (int j = 0; j < 4; ++j) {
                    const int bin = 255 - 4 * lane - j;
                    const uint32_t h = hist[bin];
                    if (c + h >= need) {
                        s_prefix = prefix | ((uint64_t)bin << shift);
                        s_mask = mask | (255ull << shift);
                        s_need = (int32_t)(need - c);
                        s_done = (h == need - c) ? 1 : 0;
                        break;
                    }
                    c += h;
                }
            }
        }
        __syncthreads();
    }
    // keys whose masked prefix is at or above the final prefix: exactly k
    {
        const uint64_t prefix = s_prefix, mask = s_mask;
#pragma unroll
        for (int i = 0; i < kTopkPerThread; ++i)
            if (tid + 256 * i < nc && (key[i] & mask) >= prefix) {
                const int slot = atomicAdd(&s_nsel, 1);
                if (slot < kMaxCentroidTopK) sel[slot] = key[i];
            }
    }
    __syncthreads();
    if (tid < 64) {
        uint64_t v = lane < k ? sel[lane] : 0ull;
        // bitonic sort of 64 keys across the wave, descending
        for (int size = 2; size <= 64; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                const uint32_t lo = __shfl_xor((uint32_t)v, stride), hi = __shfl_xor((uint32_t)(v >> 32), stride);
                const uint64_t o = ((uint64_t)hi << 32) | lo;
                const bool desc = (lane & size) == 0;
                const bool first = (lane & stride) == 0;
                const bool keep_max = desc == first;
                v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
            }
        }
        if (lane < k) cand[(int64_t)s * k + lane] = key_index(v);
    }
}

hipError_t launch_centroid_topk(const float *cl, int32_t n_centroids, int32_t k, int32_t S, int32_t *cand,
                                hipStream_t st) {
    if (n_centroids > kMaxCentroids || k < 1 || k > n_centroids || k > kMaxCentroidTopK) return hipErrorInvalidValue;
    mtp_launch(centroid_topk_kernel, dim3(S), dim3(256), 0, st, cl, n_centroids, k, cand);
    return hipGetLastError();
}

// The full logit row of a centroid head starts at -1e30 for every token
// that is not a candidate ("Gemma 4 MTP" s.3 step 5); only when the caller
// asked for logits.
__global__ void fill_logits_kernel(const CallIO *io, int32_t S, int32_t N, int32_t V, int32_t step, float v) {
    float *z = io->out_logits;
    if (!z) return;
    const int64_t n = (int64_t)S * V;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = i / V, t = i - s * V;
        z[(s * N + step) * V + t] = v;
    }
}

hipError_t launch_fill_logits(const CallIO *io, int32_t S, int32_t N, int32_t V, int32_t step, float v,
                              hipStream_t st) {
    mtp_launch(fill_logits_kernel, dim3(1024), dim3(256), 0, st, io, S, N, V, step, v);
    return hipGetLastError();
}

// RoPE frequencies theta^(-2i/hd), i < hd/2, in fp64 (once per context)
__global__ void rope_init_kernel(double *inv_freq, int32_t hd, double theta) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < hd / 2) inv_freq[i] = pow(theta, -2.0 * (double)i / (double)hd);
}

hipError_t launch_rope_init(double *inv_freq, int32_t hd, float theta, hipStream_t st) {
    mtp_launch(rope_init_kernel, dim3((hd / 2 + 63) / 64), dim3(64), 0, st, inv_freq, hd, (double)theta);
    return hipGetLastError();
}

}  // namespace mtp
