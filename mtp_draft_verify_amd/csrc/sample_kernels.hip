// sample_kernels.hip -- exact temperature>0 speculative verification on gfx950.
//
// "opus-mtp-turbo: Track 1 report" s.4 (after Leviathan et al. 2023 s.2.3):
// row i's distribution p_i is the sampling chain (top-k, penalties over the
// history plus drafts[0..i), temperature, min-p, top-p) of the target's row;
// draft d_i is accepted when u * q_i(d_i) < p_i(d_i); at the first rejection
// the emitted token is drawn from max(p_i - q_i, 0); if every draft is
// accepted, a bonus token is drawn from p_N.  A missing q means the drafts
// are deterministic (q one-hot at d_i).
//
// Kernels (rows = S*(N+1) target rows followed by S*N draft rows):
//   topk   (only when top_k > 0) one workgroup per row: radix select of the
//          k-th largest raw (logit, -id) key
//   chunk  per (row, 8192-token chunk), one read of the logits: the chunk's
//          max of the penalised, tempered logits v goes into the row max
//          (atomic max; the row max published so far comes back), then every
//          token with exp(v - ref) >= min_p, ref = the larger of the two
//          maxima, joins the row's list with its v.  ref never exceeds the
//          row max M, so the list is a superset of the min-p survivors
//   row    one workgroup per row: each listed v becomes e = exp(v - M), or 0
//          when it does not survive min-p; up to 4096 survivors are sorted by (prob
//          desc, id asc), with cumulative sums in a fixed tree order, top-p
//          cut and normaliser; more candidates that still fit the row's list
//          keep it unsorted (list form: the top-p threshold key by radix
//          select over the list, fixed-point sums); beyond the list the row
//          switches to an implicit form (radix select over the whole row).
//          Every form is exact for any distribution
//   seq    one workgroup per sequence: accept tests (all drafts at once),
//          residual or bonus draw by Gumbel-max over counter-based SplitMix64
//          uniforms, outputs, and the reset of the per-row scratch for the
//          next call
// All floating point is fp32; every sum runs in a fixed order, so a call is
// deterministic.
#include <cfloat>

#include "dev_common.h"

namespace mtp {

static constexpr int kChunk = 8192;     // tokens per chunk workgroup, held in registers
static constexpr int32_t kImplicitForm = -1, kListForm = -2;
static constexpr int kMaxCtx = 1024;
static constexpr int kMaxDrafts = 64;     // drafts per sequence (the context's max_steps bound)

struct RowState {
    float M;          // max of the penalised, tempered logits (kept set)
    float Z;          // normaliser of the final kept set
    uint64_t tau;     // kept iff key(e, id) >= tau (after the min-p test)
    int32_t n_keep;   // compact form: number of kept entries in the sorted list; kListForm: the
                      // unsorted list of cand_n entries, kept iff key >= tau; kImplicitForm: the whole row
    int32_t pad;
};

// ---------------------------------------------------------------------------
// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): golden-gamma step and the
// 30/27/31 shift-xor-multiply finaliser.  A coordinate tuple is folded in by
// xor into the state, one step per coordinate.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t sm64_step(uint64_t state) {
    uint64_t z = state + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
__device__ __forceinline__ float counter_uniform(uint64_t seed, uint64_t s, uint64_t round, uint64_t i, uint64_t stream,
                                                 uint64_t t) {
    uint64_t h = sm64_step(seed);
    h = sm64_step(h ^ s);
    h = sm64_step(h ^ round);
    h = sm64_step(h ^ i);
    h = sm64_step(h ^ stream);
    h = sm64_step(h ^ t);
    return ((float)(h >> 41) + 0.5f) * (1.0f / 8388608.0f);   // (k + 1/2) / 2^23, exact in fp32
}

__device__ __forceinline__ uint32_t fkey(float v) {            // monotone fp32 -> u32
    const uint32_t b = __float_as_uint(v + 0.0f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t tok_key(float v, int32_t id) {  // larger value, then lower id
    return ((uint64_t)fkey(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

struct RowRef {
    const float *z;   // logits row
    int kind;         // 0: target row, 1: draft row
    int s, i;
};

__device__ __forceinline__ RowRef row_ref(const SampleArgs &a, int row) {
    RowRef r;
    const int np = a.S * (a.N + 1);
    if (row < np) {
        r.kind = 0;
        r.s = row / (a.N + 1);
        r.i = row - r.s * (a.N + 1);
        r.z = a.p_logits + (int64_t)row * a.V;
    } else {
        const int qr = row - np;
        r.kind = 1;
        r.s = qr / a.N;
        r.i = qr - r.s * a.N;
        r.z = a.q_logits + (int64_t)qr * a.V;
    }
    return r;
}

// context of row (s, i): the last last_n tokens of history[s] ++ drafts[s][0..i)
// (a history length outside [0, hstride] reads as clamped into it)
__device__ __forceinline__ int hist_len(const SampleArgs &a, int s) {
    return a.history_len ? min(max(a.history_len[s], 0), a.hstride) : 0;
}
__device__ __forceinline__ int ctx_len(const SampleArgs &a, int s, int i) {
    const int total = hist_len(a, s) + i;
    return a.last_n <= 0 ? 0 : min(a.last_n, total);
}
__device__ __forceinline__ int32_t ctx_token(const SampleArgs &a, int s, int i, int n_ctx, int j) {
    const int hlen = hist_len(a, s);
    const int pos = hlen + i - n_ctx + j;
    return pos < hlen ? a.history[(int64_t)s * a.hstride + pos] : a.drafts[(int64_t)s * a.N + (pos - hlen)];
}

__device__ __forceinline__ float chain_value(const SampleArgs &a, float z, int cnt) {
    if (cnt > 0) {
        z = z > 0.f ? z / a.rep : z * a.rep;
        z -= a.presence + a.freq * (float)cnt;
    }
    return z / a.temp;
}

// block-wide helpers (NT threads, NT / 64 waves; red holds NT / 64 floats)
template <int NT = kBlock>
__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wid] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
    return m;
}
template <int NT = kBlock>
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wid] = v;
    __syncthreads();
    // pairwise in a fixed order: (0 + 1) + (2 + 3), then those sums in order
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; w += 4) tot += (red[w] + red[w + 1]) + (red[w + 2] + red[w + 3]);
    return tot;
}

template <int NT>
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t *red) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_u64(v, m);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wid] = v;
    __syncthreads();
    uint64_t t = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) t += red[w];
    return t;
}

// Context of one row in LDS: token list, and a bitmap over [c0, c0 + nbits).
struct CtxLds {
    int32_t tok[kMaxCtx];
    uint32_t bits[kChunk / 32];
    uint16_t cnt[kChunk];   // occurrences in the context of the token at each chunk position (where bits is set)
};

// Scalar load of a value whose address is the same in every lane.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T *p) {
    return *(const __attribute__((address_space(4))) T *)p;
}

// The penalty context of row (s, i), in two parts around the chunk's logit
// loads.  A wave's vector loads return in order, so context reads issued
// behind the logits would wait for all of them: ctx_request reads the
// context's length (one scalar load) and requests its tokens (thread j
// holds tokens j, j + kBlock, ...) before the logits are requested;
// ctx_store then writes them to LDS (cl.tok) with the bitmap of those
// inside the chunk [c0, c0 + nbits) and their counts.
struct CtxReq {
    int32_t t[kMaxCtx / kBlock];
    int n;
};

__device__ __forceinline__ void ctx_request(const SampleArgs &a, int s, int i, CtxReq &r) {
    const int hlen = a.history_len ? min(max(ld_uniform(a.history_len + s), 0), a.hstride) : 0;
    const int total = hlen + i;
    r.n = a.last_n <= 0 ? 0 : min(a.last_n, total);
    const int p0 = total - r.n;             // the context's first position
#pragma unroll
    for (int u = 0; u < kMaxCtx / kBlock; ++u) {
        const int j = (int)threadIdx.x + kBlock * u;
        r.t[u] = 0;
        if (j < r.n) {
            const int pos = p0 + j;
            r.t[u] = pos < hlen ? a.history[(int64_t)s * a.hstride + pos] : a.drafts[(int64_t)s * a.N + (pos - hlen)];
        }
    }
}

__device__ void ctx_store(const CtxReq &r, int c0, int nbits, CtxLds &cl) {
    for (int w = threadIdx.x; w < kChunk / 32; w += kBlock) cl.bits[w] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kMaxCtx / kBlock; ++u) {
        const int j = (int)threadIdx.x + kBlock * u, t = r.t[u];
        if (j < r.n) {
            cl.tok[j] = t;
            if (t >= c0 && t < c0 + nbits) atomicOr(&cl.bits[(t - c0) >> 5], 1u << ((t - c0) & 31));
        }
    }
    __syncthreads();
    // each in-chunk occurrence counts its token once (equal tokens store
    // equal counts), so a penalised logit later costs one LDS read
#pragma unroll
    for (int u = 0; u < kMaxCtx / kBlock; ++u) {
        const int j = (int)threadIdx.x + kBlock * u, t = r.t[u];
        if (j < r.n && t >= c0 && t < c0 + nbits) {
            int c = 0;
            for (int jj = 0; jj < r.n; ++jj) c += cl.tok[jj] == t;
            cl.cnt[t - c0] = (uint16_t)c;
        }
    }
    __syncthreads();
}

__device__ __forceinline__ int32_t shfl_xor_key(int32_t v, int m) { return __shfl_xor(v, m); }
__device__ __forceinline__ uint64_t shfl_xor_key(uint64_t v, int m) { return shfl_xor_u64(v, m); }

// Bitonic sorting network, descending when DESC: stage (k, j) orders each
// pair (x, x ^ j) of the keys the way x's block of k keys runs.  A wave holds
// the 128 keys x = xb + lane + 64 h (xb a multiple of 128) in v[h]; a stage
// with j <= 64 runs inside the wave: partners 64 apart sit in one lane,
// closer ones are exchanged across lanes, so it needs no barrier.
template <bool DESC, typename T>
__device__ __forceinline__ void wave_stage(T (&v)[2], int lane, int xb, int k, int j) {
    if (j == 64) {
        // (x, x + 64), k >= 128: both in the same block of k
        const bool up = (((xb + lane) & k) == 0) != DESC;
        const T hi = v[0] > v[1] ? v[0] : v[1], lo = v[0] > v[1] ? v[1] : v[0];
        v[0] = up ? lo : hi;
        v[1] = up ? hi : lo;
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int x = xb + lane + 64 * h;
            const T o = shfl_xor_key(v[h], j);
            const bool up = ((x & k) == 0) != DESC;     // x's block is sorted ascending
            const bool first = (x & j) == 0;            // x is the lower of the pair
            const T hi = v[h] > o ? v[h] : o, lo = v[h] > o ? o : v[h];
            v[h] = (up == first) ? lo : hi;
        }
    }
}
// the wave's 128 keys sorted (blocks up to k = 128)
template <bool DESC, typename T>
__device__ __forceinline__ void wave_sort128(T (&v)[2], int lane, int xb = 0) {
#pragma unroll
    for (int k = 2; k <= 128; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) wave_stage<DESC>(v, lane, xb, k, j);
}

// Descending sort of keys[0, np2) in LDS (256 <= np2 <= 2048, a power of
// two, padded with zeros) by np2 / 128 waves of the workgroup, 128 keys per
// wave in registers: stages with partners more than 64 apart exchange through
// LDS, alternating between keys[0, 2048) and keys[2048, 4096), one workgroup
// barrier each; the others run inside the waves.  Every thread of the
// workgroup calls it; keys is visible to the workgroup on entry and on return.
__device__ void block_sort_desc(uint64_t *keys, int np2) {
    const int lane = threadIdx.x & 63, xb = 128 * (threadIdx.x >> 6);
    const bool act = xb < np2;
    uint64_t v[2] = {0ull, 0ull};
    if (act) {
        v[0] = keys[xb + lane];
        v[1] = keys[xb + lane + 64];
        wave_sort128<true>(v, lane, xb);
    }
    int buf = 0;
    for (int k = 256; k <= np2; k <<= 1) {
        for (int j = k >> 1; j >= 128; j >>= 1) {
            uint64_t *bk = keys + 2048 * buf;
            if (act) {
                bk[xb + lane] = v[0];
                bk[xb + lane + 64] = v[1];
            }
            __syncthreads();
            if (act) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int x = xb + lane + 64 * h;
                    const uint64_t o = bk[x ^ j];
                    const bool up = (x & k) != 0, first = (x & j) == 0;
                    const uint64_t hi = v[h] > o ? v[h] : o, lo = v[h] > o ? o : v[h];
                    v[h] = (up == first) ? lo : hi;
                }
            }
            buf ^= 1;
        }
        if (act) {
            wave_stage<true>(v, lane, xb, k, 64);
            wave_stage<true>(v, lane, xb, k, 32);
            wave_stage<true>(v, lane, xb, k, 16);
            wave_stage<true>(v, lane, xb, k, 8);
            wave_stage<true>(v, lane, xb, k, 4);
            wave_stage<true>(v, lane, xb, k, 2);
            wave_stage<true>(v, lane, xb, k, 1);
        }
    }
    __syncthreads();
    if (act) {
        keys[xb + lane] = v[0];
        keys[xb + lane + 64] = v[1];
    }
    __syncthreads();
}

// sort a context list of n <= kMaxCtx tokens ascending in place (LDS):
// up to 128 in one wave's registers, more by a bitonic network over the
// workgroup.  The list is visible to the workgroup on entry and on return.
template <int NT>
__device__ void sort_ctx(int32_t *tok, int n) {
    if (n <= 128) {
        if (threadIdx.x < 64) {
            const int l = threadIdx.x;
            int32_t v[2] = {l < n ? tok[l] : 0x7FFFFFFF, l + 64 < n ? tok[l + 64] : 0x7FFFFFFF};
            wave_sort128<false>(v, l);
            if (l < n) tok[l] = v[0];
            if (l + 64 < n) tok[l + 64] = v[1];
        }
        __syncthreads();
        return;
    }
    int np2 = 1;
    while (np2 < n) np2 <<= 1;
    for (int j = n + threadIdx.x; j < np2; j += NT) tok[j] = 0x7FFFFFFF;
    __syncthreads();
    for (int k = 2; k <= np2; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int x = threadIdx.x; x < np2; x += NT) {
                const int y = x ^ j;
                if (y > x) {
                    const bool up = (x & k) == 0;
                    const int32_t a = tok[x], b = tok[y];
                    if (up ? (a > b) : (a < b)) { tok[x] = b; tok[y] = a; }
                }
            }
            __syncthreads();
        }
}
// occurrences of t in a sorted list
__device__ __forceinline__ int sorted_count(const int32_t *tok, int n, int32_t t) {
    int lo = 0, hi = n;
    while (lo < hi) { const int m = (lo + hi) >> 1; if (tok[m] < t) lo = m + 1; else hi = m; }
    int c = 0;
    while (lo + c < n && tok[lo + c] == t) ++c;
    return c;
}

// value of token t of a row (raw logit `raw`) after top-k and penalties (NaN
// when top-k drops it); member: t is in the penalty context, whose counts
// ctx_store left per position of the chunk starting at c0
__device__ __forceinline__ float raw_value(const SampleArgs &a, float raw, int32_t t, bool member, const CtxLds &cl,
                                           int c0, uint64_t topk_key) {
    if (a.top_k > 0 && tok_key(raw, t) < topk_key) return __int_as_float(0x7FC00000);
    return chain_value(a, raw, member ? (int)cl.cnt[t - c0] : 0);
}

// The chunk kernel holds its kChunk tokens in registers, in batches of
// KB = 32 / E loads per thread, each load E consecutive logits (E = 4 when
// rows are 16-byte aligned: one wave load then moves 1 KiB).  Every batch is
// requested at once (clamped into the chunk), right after the context's
// tokens.
template <int E> struct ChunkShape {
    static constexpr int KB = E == 4 ? 4 : 8;           // loads per thread per batch
    static constexpr int BT = E * kBlock * KB;          // tokens per batch
    static constexpr int NB = kChunk / BT;              // batches per chunk
};
template <int E, int KB>
__device__ __forceinline__ void load_batch(const float *z, int b0, int c1, float (&raw)[KB][E]) {
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int t = min(b0 + E * ((int)threadIdx.x + kBlock * k), c1 - E);
        if constexpr (E == 4) {
            const float4 v = *(const float4 *)(z + t);
            raw[k][0] = v.x; raw[k][1] = v.y; raw[k][2] = v.z; raw[k][3] = v.w;
        } else {
            raw[k][0] = z[t];
        }
    }
}

// ---------------------------------------------------------------------------
// radix select over one row: the largest 64-bit key K with W(key >= K) >= target,
// where W sums weight(t) over the row's eligible tokens.  8 passes of 8 bits.
// ---------------------------------------------------------------------------
template <int NT, typename KeyW>
__device__ uint64_t radix_select(int V, uint64_t target, KeyW key_weight, uint64_t *hist /* [256] LDS */,
                                 uint64_t *scal /* [4] LDS */) {
    uint64_t prefix = 0, mask = 0;
    for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        for (int b = threadIdx.x; b < 256; b += NT) hist[b] = 0;
        __syncthreads();
        for (int t = threadIdx.x; t < V; t += NT) {
            uint64_t k, wgt;
            if (!key_weight(t, k, wgt)) continue;
            if ((k & mask) != prefix) continue;
            atomicAdd((unsigned long long *)&hist[(k >> shift) & 0xFF], (unsigned long long)wgt);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            uint64_t above = 0;
            int dsel = 0;
            for (int b = 255; b >= 0; --b) {
                if (above + hist[b] >= target) { dsel = b; break; }
                above += hist[b];
            }
            scal[0] = (uint64_t)dsel;
            scal[1] = above;
        }
        __syncthreads();
        prefix |= scal[0] << shift;
        mask |= (uint64_t)0xFF << shift;
        target -= scal[1];
        __syncthreads();
    }
    return prefix;
}

// top-k threshold on raw logits (ties: lower id first)
__global__ __launch_bounds__(256) void sample_topk_kernel(SampleArgs a) {
    __shared__ uint64_t hist[256], scal[4];
    const int row = blockIdx.x;
    const RowRef rr = row_ref(a, row);
    if (a.top_k >= a.V) {
        if (threadIdx.x == 0) a.topk_key[row] = 0;
        return;
    }
    auto kw = [&](int t, uint64_t &k, uint64_t &w) {
        k = tok_key(rr.z[t], t);
        w = 1;
        return true;
    };
    const uint64_t K = radix_select<kBlock>(a.V, (uint64_t)a.top_k, kw, hist, scal);
    if (threadIdx.x == 0) a.topk_key[row] = K;
}

// The single pass over the logits: the chunk's row max contribution, then
// its part of a superset of the row's min-p survivors (token, v).
template <int E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(E == 4 ? 6 : 3))) void sample_chunk_kernel(SampleArgs a, int n_chunk) {
    constexpr int KB = ChunkShape<E>::KB, BT = ChunkShape<E>::BT, NB = ChunkShape<E>::NB;
    __shared__ CtxLds cl;
    __shared__ float red[4];
    __shared__ float ref_sh;
    const int row = blockIdx.x / n_chunk, chunk = blockIdx.x - row * n_chunk;
    const RowRef rr = row_ref(a, row);
    const int c0 = chunk * kChunk, c1 = min(a.V, c0 + kChunk);
    // the penalty context's tokens are requested first, then the whole chunk
    // (into registers)
    CtxReq creq;
    ctx_request(a, rr.s, rr.i, creq);
    float raw[NB][KB][E];
#pragma unroll
    for (int b = 0; b < NB; ++b) load_batch<E, KB>(rr.z, c0 + b * BT, c1, raw[b]);
    ctx_store(creq, c0, c1 - c0, cl);
    // which of the thread's NB * KB * E tokens are in the context (bit =
    // position, as for kmask below): read from the bitmap once, so the
    // passes below test a register instead of waiting on LDS per token.  A
    // load's E tokens start at a multiple of E and share one bitmap word.
    static_assert(NB * KB * E <= 32, "one bit per token of the thread");
    uint32_t mmask = 0u;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int off = b * BT + E * ((int)threadIdx.x + kBlock * k);
            const uint32_t w = cl.bits[off >> 5] >> (off & 31);
            mmask |= (w & ((1u << E) - 1u)) << ((b * KB + k) * E);
        }
    const uint64_t tk = a.top_k > 0 ? a.topk_key[row] : 0;
    // Positions p = (b * KB + k) * E + e of the thread's tokens: `ok` holds
    // those that are tokens of the row (the last chunk's loads are clamped)
    // and survive top-k; of them, context tokens (memb) take the full chain
    // and every other token (plain) is valued fl(z / temp).
    constexpr int NP = NB * KB * E;
    constexpr uint32_t kAll = (uint32_t)((1ull << NP) - 1u);
    auto tok_at = [&](int b, int k, int e) { return c0 + b * BT + E * ((int)threadIdx.x + kBlock * k) + e; };
    uint32_t ok = kAll;
    if (c1 - c0 < kChunk || a.top_k > 0) {
        ok = 0u;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int k = 0; k < KB; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int t = tok_at(b, k, e);
                    const bool keep = t < c1 && !(a.top_k > 0 && tok_key(raw[b][k][e], t) < tk);
                    ok |= (uint32_t)keep << ((b * KB + k) * E + e);
                }
    }
    const uint32_t memb = ok & mmask, plain = ok & ~mmask;
    // fl(z / temp) does not decrease as z grows, so the largest plain value
    // is that of the largest plain raw logit: those tokens only need a
    // running max of z.
    float mz = -INFINITY;
    if (plain == kAll) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int k = 0; k < KB; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e) mz = fmaxf(mz, raw[b][k][e]);
    } else {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int k = 0; k < KB; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    mz = fmaxf(mz, (plain >> ((b * KB + k) * E + e)) & 1u ? raw[b][k][e] : -INFINITY);
    }
    float mx = -INFINITY;
    if (memb) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int k = 0; k < KB; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if ((memb >> ((b * KB + k) * E + e)) & 1u) {
                        const float v = raw_value(a, raw[b][k][e], tok_at(b, k, e), true, cl, c0, tk);
                        if (v == v) mx = fmaxf(mx, v);
                    }
    }
    const float mz_thread = mz;
    if (mz > -INFINITY) mx = fmaxf(mx, chain_value(a, mz, 0));
    mx = block_max(mx, red);
    if (threadIdx.x == 0) {
        float ref = mx;
        if (mx > -INFINITY) {
            const uint32_t old = atomicMax(&a.row_maxkey[row * kRowCtrStride], fkey(mx));
            if (old != 0u) ref = fmaxf(mx, fkey_inv(old));
        }
        ref_sh = ref;
    }
    __syncthreads();
    const float ref = ref_sh;
    // exp(fl(v - M)) >= min_p implies exp(fl(v - ref)) >= min_p for ref <= M
    // (rounding and exp do not decrease with their argument), so testing
    // against ref keeps every survivor.  A plain token passes only if
    // z / temp >= ref + ln(min_p) - 1e-5 (1 + |ref|) at the least (fp32
    // rounding and expf's error), so every plain token with a raw logit of at
    // least zlo = temp * (ref + ln(min_p) - 0.01 - 1e-5 |ref|) (rounded down)
    // is listed, untested: the list stays a superset, and the row kernel
    // takes the exact decision.  A token of value -inf never survives (its
    // weight is 0), so zlo is at least -FLT_MAX.
    float zlo = -FLT_MAX;
    if (a.min_p > 0.f && ref > -INFINITY) {
        const double zl = (double)a.temp * ((double)ref + a.ln_min_p - 0.01 - 1e-5 * fabs((double)ref));
        zlo = fmaxf(nextafterf((float)zl, -INFINITY), -FLT_MAX);
    }
    // which of the thread's tokens are listed (bit = position)
    uint32_t kmask = 0u;
    if (mz_thread >= zlo) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int k = 0; k < KB; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e) kmask |= (uint32_t)(raw[b][k][e] >= zlo) << ((b * KB + k) * E + e);
        kmask &= plain;
    }
    if (memb) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int k = 0; k < KB; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if ((memb >> ((b * KB + k) * E + e)) & 1u) {
                        const float v = raw_value(a, raw[b][k][e], tok_at(b, k, e), true, cl, c0, tk);
                        if (v == v && expf(v - ref) >= a.min_p) kmask |= 1u << ((b * KB + k) * E + e);
                    }
    }
    // Slots: an exclusive prefix sum of the threads' counts over the wave
    // and one reservation per wave (each row's counter has a line of its
    // own), so no wave waits on an atomic inside the token loop or on the
    // other waves.  Slot order within the list does not matter: the row
    // kernel sorts it or sums it in fixed point.
    const int lane = threadIdx.x & 63;
    const int cnt = __popc(kmask);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    const int wtot = __shfl(incl, 63);
    if (wtot == 0) return;
    int wbase = 0;
    if (lane == 0) wbase = atomicAdd(&a.cand_n[row * kRowCtrStride], wtot);
    int slot = __shfl(wbase, 0) + incl - cnt;
    // each thread walks the set bits of its kmask (the slots follow position
    // order); the listed value is picked out of the registers by position
    for (uint32_t m = kmask; m != 0u; m &= m - 1u) {
        const int p = __builtin_ctz(m);
        float z = 0.f;
#pragma unroll
        for (int q = 0; q < NP; ++q) z = p == q ? raw[q / (KB * E)][(q / E) % KB][q % E] : z;
        const int t = tok_at(p / (KB * E), (p / E) % KB, p % E);
        if (slot < a.cap) {
            a.cand_id[(int64_t)row * a.cap + slot] = t;
            a.cand_v[(int64_t)row * a.cap + slot] = raw_value(a, z, t, (mmask >> p) & 1u, cl, c0, tk);
        }
        ++slot;
    }
}

// ---------------------------------------------------------------------------
// row finalisation
// ---------------------------------------------------------------------------
static constexpr int kSortMax = 4096;
// The row and sequence kernels run one workgroup per row / sequence; a
// broad row (more candidates than kSortMax) makes them walk the whole
// vocabulary several times, so they take 16 waves.
static constexpr int kRowThreads = 1024;

__global__ __launch_bounds__(kRowThreads) void sample_row_kernel(SampleArgs a) {
    constexpr int NT = kRowThreads;
    __shared__ uint64_t keys[kSortMax];
    __shared__ float red[NT / 64];
    __shared__ int cut_sh, nkey_sh;
    __shared__ uint64_t hist[256], scal[4], red64[NT / 64];
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int n_all = a.cand_n[row * kRowCtrStride];
    const float M = fkey_inv(a.row_maxkey[row * kRowCtrStride]);
    RowState st;
    st.M = M;
    st.pad = 0;
    // The chunk pass listed a superset of the min-p survivors with their
    // chain values v: each entry becomes e = exp(v - M) when it survives and
    // 0 when it does not (an entry of weight 0 takes part in no sum and no
    // draw).  The survivors are counted; beyond the list's slots the row
    // takes the implicit form below, which does not read the list.
    // A list of at most RU * NT entries stays in registers through the
    // count: it always takes the compact form, which then needs no second
    // read of it.  A longer one is rewritten in place.
    constexpr int RU = 4;
    static_assert(RU * NT <= kSortMax, "a list held in registers is always sorted");
    const bool inreg = n_all <= RU * NT;
    float er[RU];
    int32_t ir[RU];
    if (tid == 0) nkey_sh = 0;
    int n_surv = 0;
    if (n_all > 0 && n_all <= a.cap) {
        float *lv = a.cand_v + (int64_t)row * a.cap;
        const int32_t *li = a.cand_id + (int64_t)row * a.cap;
        float cnt = 0.f;
        auto filter = [&](float v) {
            const float e = expf(v - M);
            const bool keep = e >= a.min_p && e > 0.f;     // a zero weight is never drawn
            cnt += keep ? 1.f : 0.f;
            return keep ? e : 0.f;
        };
        if (inreg) {
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const int j = tid + NT * u;
                er[u] = 0.f;
                ir[u] = 0;
                if (j < n_all) {
                    er[u] = filter(lv[j]);
                    ir[u] = li[j];
                }
            }
        } else {
            for (int j = tid; j < n_all; j += NT) lv[j] = filter(lv[j]);
        }
        n_surv = (int)block_sum<NT>(cnt, red);     // exact: at most 65536 ones
        __syncthreads();                           // the rewritten list is visible to the whole workgroup
    }
    if (n_all == 0 || (n_all <= a.cap && n_surv == 0)) {
        // no token survives (a row without a finite maximum): the row's
        // distribution is empty, every probability reads 0 and a draw from it
        // emits -1
        if (tid == 0) {
            st.Z = 1.f;
            st.tau = ~0ull;
            st.n_keep = 0;
            ((RowState *)a.row_state)[row] = st;
        }
        return;
    }
    if (n_all <= a.cap && n_surv <= kSortMax) {
        // ---- compact form: sort the survivors ----
        const int n = n_surv;
        int np2 = 1;
        while (np2 < n) np2 <<= 1;
        if (inreg) {
#pragma unroll
            for (int u = 0; u < RU; ++u)
                if (er[u] > 0.f) keys[atomicAdd(&nkey_sh, 1)] = tok_key(er[u], ir[u]);
        } else {
            for (int j = tid; j < n_all; j += NT) {
                const float e = a.cand_v[(int64_t)row * a.cap + j];
                if (e > 0.f) keys[atomicAdd(&nkey_sh, 1)] = tok_key(e, a.cand_id[(int64_t)row * a.cap + j]);
            }
        }
        if (np2 <= 128) np2 = 128;                     // the one-wave sort below takes 128 keys
        for (int j = n + tid; j < np2; j += NT) keys[j] = 0ull;
        __syncthreads();
        if (np2 == 128) {
            // sorted descending in one wave's registers
            if (tid < 64) {
                uint64_t v[2] = {keys[tid], keys[tid + 64]};
                wave_sort128<true>(v, tid);
                keys[tid] = v[0];
                keys[tid + 64] = v[1];
            }
            __syncthreads();
        } else if (np2 <= 2048) {
            block_sort_desc(keys, np2);
        } else {
            for (int k = 2; k <= np2; k <<= 1) {       // bitonic sort, descending
                for (int j = k >> 1; j > 0; j >>= 1) {
                    for (int x = tid; x < np2; x += NT) {
                        const int y = x ^ j;
                        if (y > x) {
                            const bool desc = (x & k) == 0;
                            const uint64_t kx = keys[x], ky = keys[y];
                            if (desc ? (kx < ky) : (kx > ky)) { keys[x] = ky; keys[y] = kx; }
                        }
                    }
                    __syncthreads();
                }
            }
        }
        // prefix sums of e in sorted order, in a fixed order: thread tid sums
        // its contiguous block of `per` entries, the block sums are scanned
        // within each wave (shuffles) and across the waves (LDS), and the
        // top-p cut and the kept prefix's normaliser both come from that one
        // running sum
        const int per = (n + NT - 1) / NT;
        const int b0 = min(n, tid * per), b1 = min(n, b0 + per);
        const int lane = tid & 63, wid = tid >> 6;
        float bs = 0.f;
        for (int j = b0; j < b1; ++j) bs += fkey_inv((uint32_t)(keys[j] >> 32));
        float inc = bs;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(inc, off);
            if (lane >= off) inc += y;
        }
        float excl = __shfl_up(inc, 1);
        if (lane == 0) excl = 0.f;
        if (lane == 63) red[wid] = inc;
        if (tid == 0) cut_sh = n - 1;
        __syncthreads();
        float base = 0.f, Z2 = 0.f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            if (w < wid) base += red[w];
            Z2 += red[w];
        }
        const float start = base + excl;    // the sum of all entries before this thread's block
        if (a.top_p < 1.f) {
            float cum = start;
            for (int j = b0; j < b1; ++j) {
                cum += fkey_inv((uint32_t)(keys[j] >> 32));
                if (cum / Z2 >= a.top_p) { atomicMin(&cut_sh, j); break; }
            }
        }
        __syncthreads();
        const int cut = cut_sh;
        // normaliser of the kept prefix: the running sum at the cut
        if (cut >= b0 && cut < b1) {
            float z = start;
            for (int j = b0; j <= cut; ++j) z += fkey_inv((uint32_t)(keys[j] >> 32));
            st.Z = z;
            st.tau = keys[cut];
            st.n_keep = cut + 1;
            ((RowState *)a.row_state)[row] = st;
        }
        for (int j = tid; j <= cut; j += NT) {
            a.cand_id[(int64_t)row * a.cap + j] = (int32_t)(0xFFFFFFFFu - (uint32_t)keys[j]);
            a.cand_v[(int64_t)row * a.cap + j] = fkey_inv((uint32_t)(keys[j] >> 32));
        }
        return;
    }
    const double scale = 1099511627776.0;   // 2^40: fixed-point weights (e <= 1), exact sums in any order
    if (n_all <= a.cap) {
        // ---- list form: every min-p survivor is in the row's (unordered)
        // list (beside entries of weight 0); the top-p threshold is a radix
        // select over the list, and the sums are fixed-point so that they do
        // not depend on its order
        const int n = n_all;
        const int32_t *lid = a.cand_id + (int64_t)row * a.cap;
        const float *lv = a.cand_v + (int64_t)row * a.cap;
        uint64_t z2 = 0;
        for (int j = tid; j < n; j += NT) z2 += (uint64_t)((double)lv[j] * scale);
        const uint64_t Z2 = block_sum_u64<NT>(z2, red64);
        uint64_t tau = 0;
        if (a.top_p < 1.f) {
            const uint64_t target = (uint64_t)ceil((double)a.top_p * (double)Z2);
            auto kw = [&](int j, uint64_t &k, uint64_t &w) {
                const float e = lv[j];
                k = tok_key(e, lid[j]);
                w = (uint64_t)((double)e * scale);
                return true;
            };
            tau = radix_select<NT>(n, target, kw, hist, scal);
        }
        uint64_t z3 = 0;
        for (int j = tid; j < n; j += NT)
            if (tok_key(lv[j], lid[j]) >= tau) z3 += (uint64_t)((double)lv[j] * scale);
        const uint64_t Z3 = block_sum_u64<NT>(z3, red64);
        if (tid == 0) {
            st.Z = (float)((double)Z3 / scale);
            st.tau = tau;
            st.n_keep = kListForm;
            ((RowState *)a.row_state)[row] = st;
        }
        return;
    }
    // ---- implicit form: thresholds over the whole row ----
    const RowRef rr = row_ref(a, row);
    __shared__ int32_t ctx_tok[kMaxCtx];
    const int n_ctx = ctx_len(a, rr.s, rr.i);
    for (int j = tid; j < n_ctx; j += NT) ctx_tok[j] = ctx_token(a, rr.s, rr.i, n_ctx, j);
    __syncthreads();
    sort_ctx<NT>(ctx_tok, n_ctx);
    const uint64_t tk = a.top_k > 0 ? a.topk_key[row] : 0;
    auto e_of = [&](int t, float &e) {
        const float raw = rr.z[t];
        if (a.top_k > 0 && tok_key(raw, t) < tk) return false;
        e = expf(chain_value(a, raw, sorted_count(ctx_tok, n_ctx, t)) - M);
        return e >= a.min_p;
    };
    float z2 = 0.f;
    for (int t = tid; t < a.V; t += NT) {
        float e;
        if (e_of(t, e)) z2 += e;
    }
    const float Z2 = block_sum<NT>(z2, red);
    uint64_t tau = 0;
    if (a.top_p < 1.f) {
        // fixed-point weights (scale = 2^40 per unit) keep the histogram sums exact
        const uint64_t target = (uint64_t)ceil((double)a.top_p * (double)Z2 * scale);
        auto kw = [&](int t, uint64_t &k, uint64_t &w) {
            float e;
            if (!e_of(t, e)) return false;
            k = tok_key(e, t);
            w = (uint64_t)((double)e * scale);
            return true;
        };
        tau = radix_select<NT>(a.V, target, kw, hist, scal);
    }
    float z3 = 0.f;
    for (int t = tid; t < a.V; t += NT) {
        float e;
        if (e_of(t, e) && tok_key(e, t) >= tau) z3 += e;
    }
    const float Z3 = block_sum<NT>(z3, red);
    if (tid == 0) {
        st.Z = Z3;
        st.tau = tau;
        st.n_keep = kImplicitForm;
        ((RowState *)a.row_state)[row] = st;
    }
}

// ---------------------------------------------------------------------------
// per-sequence accept / resample
// ---------------------------------------------------------------------------
// Probability of token t under row `row` (its RowState final), t occurring
// cnt times in the row's context, in two halves: tok_prob_load issues the
// reads (the row's state, its logit at t and top-k key), tok_prob_value
// finishes once the count is known.
struct TokProbIn {
    RowState st;
    float raw;
    uint64_t tk;
    bool in_vocab;
};
__device__ __forceinline__ TokProbIn tok_prob_load(const SampleArgs &a, int row, int32_t t) {
    TokProbIn r;
    r.in_vocab = t >= 0 && t < a.V;
    r.st = ((const RowState *)a.row_state)[row];
    r.raw = r.in_vocab ? row_ref(a, row).z[t] : 0.f;
    r.tk = a.top_k > 0 ? a.topk_key[row] : 0;
    return r;
}
__device__ __forceinline__ float tok_prob_value(const SampleArgs &a, const TokProbIn &r, int32_t t, int cnt) {
    if (!r.in_vocab) return 0.f;
    if (a.top_k > 0 && tok_key(r.raw, t) < r.tk) return 0.f;
    const float e = expf(chain_value(a, r.raw, cnt) - r.st.M);
    if (!(e >= a.min_p) || tok_key(e, t) < r.st.tau) return 0.f;
    return e / r.st.Z;
}
__device__ float row_prob_cnt(const SampleArgs &a, int row, int32_t t, int cnt) {
    return tok_prob_value(a, tok_prob_load(a, row, t), t, cnt);
}
// the same with the row's context as a sorted list
__device__ float row_prob(const SampleArgs &a, int row, int32_t t, const int32_t *ctx_tok, int n_ctx) {
    if (t < 0 || t >= a.V) return 0.f;
    return row_prob_cnt(a, row, t, sorted_count(ctx_tok, n_ctx, t));
}

__global__ __launch_bounds__(kRowThreads) void sample_seq_kernel(SampleArgs a) {
    constexpr int NT = kRowThreads;
    __shared__ int32_t seq_tok[kMaxCtx + kMaxDrafts];
    __shared__ int32_t ctx_tok[kMaxCtx];
    __shared__ uint64_t best_w[NT / 64];
    __shared__ int accept[kMaxDrafts];
    __shared__ RowState pstate[kMaxDrafts + 1];
    const int s = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int N = a.N, R = N + 1;
    // Every row's penalty context lies in positions [p_lo, hlen + N) of
    // history[s] ++ drafts[s]: read once into LDS.  Row i's context starts
    // at hlen + i - n_ctx(i), which does not decrease with i.
    const int hlen = hist_len(a, s);
    const int p_lo = hlen - ctx_len(a, s, 0);
    const int n_seq = hlen + N - p_lo;
    // The accept test of draft i needs only the final states of its p and q
    // rows, the draft's count in row i's context and its own uniform, none
    // of the earlier outcomes: all the tests run at once, one wave per draft
    // (the reads at the draft are issued with the context's).
    constexpr int kWaves = NT / 64;
    static_assert(kMaxDrafts <= 4 * kWaves, "drafts per wave");
    int32_t dr[4];
    TokProbIn pin[4], qin[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = wid + kWaves * u;
        dr[u] = i < N ? a.drafts[(int64_t)s * N + i] : -1;
    }
    for (int j = tid; j < n_seq; j += NT) {
        const int pos = p_lo + j;
        seq_tok[j] = pos < hlen ? a.history[(int64_t)s * a.hstride + pos] : a.drafts[(int64_t)s * N + (pos - hlen)];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = wid + kWaves * u;
        if (i < N) {
            pin[u] = tok_prob_load(a, s * R + i, dr[u]);
            if (a.q_logits) qin[u] = tok_prob_load(a, a.S * R + s * N + i, dr[u]);
        }
    }
    // the bonus row's state, for the draw below
    if (tid == 0) pstate[N] = ((const RowState *)a.row_state)[s * R + N];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = wid + kWaves * u;
        if (i >= N) continue;
        const int32_t d = dr[u];
        const int n_ctx = ctx_len(a, s, i), c0 = hlen + i - n_ctx - p_lo;
        float c = 0.f;
        if (d >= 0 && d < a.V)
            for (int j = lane; j < n_ctx; j += 64) c += seq_tok[c0 + j] == d ? 1.f : 0.f;
        const int cnt = (int)wave_sum(c);         // exact: at most kMaxCtx ones
        if (lane == 0) {
            const float pd = tok_prob_value(a, pin[u], d, cnt);
            const float qd = a.q_logits ? tok_prob_value(a, qin[u], d, cnt) : ((d >= 0 && d < a.V) ? 1.f : 0.f);
            const float uu = counter_uniform(a.seed, s, a.round, i, 0, 0);
            accept[i] = (uu * qd < pd) ? 1 : 0;
            pstate[i] = pin[u].st;
        }
    }
    __syncthreads();
    int i = 0;
    while (i < N && accept[i]) ++i;              // first rejection, or N
    const int n_acc = i;
    for (int j = tid; j < n_acc; j += NT) a.out_tokens[(int64_t)s * R + j] = a.drafts[(int64_t)s * N + j];
    {
        const int prow = s * R + i;
        const int n_ctx = ctx_len(a, s, i), c0 = hlen + i - n_ctx - p_lo;
        for (int j = tid; j < n_ctx; j += NT) ctx_tok[j] = seq_tok[c0 + j];
        __syncthreads();
        sort_ctx<NT>(ctx_tok, n_ctx);
        const int32_t d = i < N ? a.drafts[(int64_t)s * N + i] : -1;
        const int qrow = a.q_logits ? a.S * R + s * N + i : -1;
        // draw from max(p - q, 0) (rejection at row i) or from p_N (bonus)
        const uint64_t stream = i < N ? 1 : 2;
        const RowState st = pstate[i];
        uint64_t best = 0;
        auto consider = [&](int32_t t, float pt) {
            float r = pt;
            if (i < N) r -= a.q_logits ? row_prob(a, qrow, t, ctx_tok, n_ctx) : (t == d ? 1.f : 0.f);
            if (!(r > 0.f)) return;
            const float u = counter_uniform(a.seed, s, a.round, i, stream, (uint64_t)t);
            const float key = logf(r) - logf(-logf(u));
            const uint64_t k = tok_key(key, t);
            best = k > best ? k : best;
        };
        if (st.n_keep >= 0) {
            for (int j = tid; j < st.n_keep; j += NT)
                consider(a.cand_id[(int64_t)prow * a.cap + j], a.cand_v[(int64_t)prow * a.cap + j] / st.Z);
        } else if (st.n_keep == kListForm) {
            const int n = a.cand_n[prow * kRowCtrStride];
            for (int j = tid; j < n; j += NT) {
                const int32_t t = a.cand_id[(int64_t)prow * a.cap + j];
                const float e = a.cand_v[(int64_t)prow * a.cap + j];
                if (tok_key(e, t) >= st.tau) consider(t, e / st.Z);
            }
        } else {
            for (int t = tid; t < a.V; t += NT) {
                const float pt = row_prob(a, prow, t, ctx_tok, n_ctx);
                if (pt > 0.f) consider(t, pt);
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const uint64_t o = shfl_xor_u64(best, m);
            best = o > best ? o : best;
        }
        if (lane == 0) best_w[wid] = best;
        __syncthreads();
        if (tid == 0) {
            uint64_t b = best_w[0];
            for (int w = 1; w < NT / 64; ++w) b = best_w[w] > b ? best_w[w] : b;
            a.out_tokens[(int64_t)s * R + i] = b ? (int32_t)(0xFFFFFFFFu - (uint32_t)b) : -1;
        }
        if (i < N) {
            for (int j = i + 1 + tid; j < R; j += NT) a.out_tokens[(int64_t)s * R + j] = -1;
        }
    }
    if (tid == 0) a.out_n_accept[s] = n_acc;
    // clear this sequence's row scratch for the next call
    for (int i = tid; i < R; i += NT) {
        a.row_maxkey[(s * R + i) * kRowCtrStride] = 0u;
        a.cand_n[(s * R + i) * kRowCtrStride] = 0;
    }
    if (a.q_logits)
        for (int i = tid; i < N; i += NT) {
            a.row_maxkey[(a.S * R + s * N + i) * kRowCtrStride] = 0u;
            a.cand_n[(a.S * R + s * N + i) * kRowCtrStride] = 0;
        }
}

hipError_t launch_verify_sample(const SampleArgs &a, hipStream_t st) {
    const int rows = a.S * (a.N + 1) + (a.q_logits ? a.S * a.N : 0);
    const int n_chunk = (a.V + kChunk - 1) / kChunk;
    if ((int64_t)rows * n_chunk > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (a.top_k > 0) {
        mtp_launch(sample_topk_kernel, dim3(rows), dim3(kBlock), 0, st, a);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    // 4 logits per load when every row starts on a 16-byte boundary
    const bool v4 = a.V % 4 == 0 && ((uintptr_t)a.p_logits & 15) == 0 && ((uintptr_t)a.q_logits & 15) == 0;
    if (v4) mtp_launch(sample_chunk_kernel<4>, dim3(rows * n_chunk), dim3(kBlock), 0, st, a, n_chunk);
    else mtp_launch(sample_chunk_kernel<1>, dim3(rows * n_chunk), dim3(kBlock), 0, st, a, n_chunk);
    mtp_launch(sample_row_kernel, dim3(rows), dim3(kRowThreads), 0, st, a);
    mtp_launch(sample_seq_kernel, dim3(a.S), dim3(kRowThreads), 0, st, a);
    return hipGetLastError();
}

size_t sample_row_state_bytes() { return sizeof(RowState); }

}  // namespace mtp
