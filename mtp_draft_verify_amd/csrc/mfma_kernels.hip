// mfma_kernels.hip -- the draft chain's GEMVs and LM head for several
// sequences at once, on the gfx950 matrix cores.
//
// With S >= 2 sequences a weight pass is a real (if skinny) contraction,
// Y[s, r] = sum_c W[r, c] X[s, c], so each 16-row weight tile meets all S
// sequences in v_mfma_f32_16x16x32_bf16 instead of S wave reductions.  The
// fp32 activations enter as an exact-to-2^-18 pair of bf16 halves (hi + lo,
// two MFMAs, two fp32 accumulators), so the products keep fp32 accuracy; bf16
// weights enter as they are and Q8_0 quants widen exactly to bf16, the block
// scale being applied to each 32-column MFMA result in fp32.
//
// Operand layout of the 16x16x32 bf16 MFMA (one wave, lane l = 16 g + j):
//   A: lane l holds row j, columns 8 g .. 8 g + 7 of the 32-column step
//   B: lane l holds column j (a sequence), the same 8 step columns
//   D: lane l holds rows 4 g .. 4 g + 3 of column j
// Each output column is a separate dot product, so a sequence gets the same
// bits whatever else is in the batch.
#include <algorithm>
#include <type_traits>

#include "widen.h"

namespace mtp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mfma(const bf16x8_t a, const bf16x8_t b, const f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v ~= hi + lo with |v - hi - lo| <= 2^-18 |v| (both halves round to nearest).
__device__ __forceinline__ void split_bf16(const float (&v)[8], u32x4_t &hi, u32x4_t &lo) {
    bf16x8_t h, l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const __bf16 b = (__bf16)v[i];
        h[i] = b;
        l[i] = (__bf16)(v[i] - (float)b);
    }
    hi = __builtin_bit_cast(u32x4_t, h);
    lo = __builtin_bit_cast(u32x4_t, l);
}

// Signed byte B of w as fp32, in one instruction (the convert's own byte
// select and sign extension; left to itself the compiler extracts bytes 1
// and 3 with an extra 16-bit shift each).
template <int B>
__device__ __forceinline__ float sbyte_to_f32(uint32_t w) {
    float f;
    if constexpr (B == 0)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(f) : "v"(w));
    else if constexpr (B == 1)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(f) : "v"(w));
    else if constexpr (B == 2)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(f) : "v"(w));
    else
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(f) : "v"(w));
    return f;
}

// 8 Q8_0 quants (one lane's share of a step) as exact bf16 values: each
// integer goes to fp32 exactly and every |q| <= 128 has at most 8
// significant bits, so the pairwise fp32 -> bf16 conversion (one
// instruction per pair on gfx950) is exact too.
__device__ __forceinline__ u32x4_t q8_to_bf16(const u32x2_t q) {
    bf16x8_t r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w = q[h];
        r[4 * h + 0] = (__bf16)sbyte_to_f32<0>(w);
        r[4 * h + 1] = (__bf16)sbyte_to_f32<1>(w);
        r[4 * h + 2] = (__bf16)sbyte_to_f32<2>(w);
        r[4 * h + 3] = (__bf16)sbyte_to_f32<3>(w);
    }
    return __builtin_bit_cast(u32x4_t, r);
}

__device__ __forceinline__ u32x4_t ld_nt4(const void *p) { return __builtin_nontemporal_load((const u32x4_t *)p); }
__device__ __forceinline__ u32x2_t ld_nt2(const void *p) { return __builtin_nontemporal_load((const u32x2_t *)p); }

// ============================================================================
// GEMV tile kernel: one 16-row tile per workgroup, the K steps dealt out
// round-robin to the NW waves (step t = w + NW i), partial tiles summed over
// the waves in a fixed order.  All weight loads are issued first.
// ============================================================================
static constexpr int kMmSteps = 8;     // K steps per wave (K <= NW * 8 * 32)

template <int IN>
__device__ __forceinline__ void mm_load_x(const GemvArgs &a, int s, int col, float (&x)[8]) {
    if (IN != IN_EMBED) {
        const float4 *p = (const float4 *)(a.src + (int64_t)s * a.src_stride + col);
        const float4 u = p[0], v = p[1];
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
        return;
    }
    const int d = a.d_embed;
    if (col >= d) {
        const float4 *p = (const float4 *)(a.h + (int64_t)s * a.dh + (col - d));
        const float4 u = p[0], v = p[1];
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
        return;
    }
    const int32_t tok = a.tok_in ? a.tok_in[s] : key_index(a.key_in[s]);
    if (tok < 0 || tok >= a.embed_rows) {   // ids outside the vocabulary embed to zero
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.f;
        return;
    }
    float e[8];
    if (a.embed_dtype == MTP_F32) {
        const float4 *p = (const float4 *)((const float *)a.embed + (int64_t)tok * d + col);
        const float4 u = p[0], v = p[1];
        e[0] = u.x; e[1] = u.y; e[2] = u.z; e[3] = u.w; e[4] = v.x; e[5] = v.y; e[6] = v.z; e[7] = v.w;
    } else if (a.embed_dtype == MTP_BF16) {
        widen(*(const uint4 *)((const uint16_t *)a.embed + (int64_t)tok * d + col), e);
    } else {
        const float sc = half_to_f(a.embed_qs[(int64_t)tok * (d / 32) + col / 32]);
        const uint2 q = *(const uint2 *)(a.embed_q + (int64_t)tok * d + col);
        const uint32_t qw[2] = {q.x, q.y};
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = sc * (float)(int8_t)((qw[i / 4] >> (8 * (i % 4))) & 0xFF);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = a.embed_scale * e[i];
}

// ROWS < 16: a workgroup's tile holds ROWS weight rows (operand rows ROWS ..
// 15 are zero), so short matrices spread over more workgroups (M = 1024 in
// 16-row tiles would leave three CUs in four idle).  Each output row is its
// own MFMA dot product: its value does not depend on the tile height.
template <int NW, int IN, int EPI, int ROWS>
__global__ __launch_bounds__(NW * 64) void mm_gemv_kernel(GemvArgs a_in) {
    static_assert(ROWS == 16 || ROWS == 8 || ROWS == 4 || ROWS == 2, "a tile is a power-of-two part of an operand");
    GemvArgs a = a_in;
    if (IN == IN_EMBED) {   // caller buffers of this call
        a.tok_in = a.step == 0 ? a.io->last_tok : nullptr;
        if (a.step == 0) a.h = a.io->h_prev;
        a.drafts_out = a.step > 0 ? a.io->out_drafts : nullptr;
    }
    __shared__ float ssw[NW][16];
    __shared__ f32x4_t red[NW][64];
    const int K = a.K, M = a.M, S = a.S, KS = K / 32;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int j16 = lane & 15, g = lane >> 4;
    const int R0 = blockIdx.x * ROWS;

    if (IN == IN_EMBED && blockIdx.x == 0 && tid < S) {
        if (a.drafts_out) a.drafts_out[(int64_t)tid * a.drafts_stride + a.drafts_col] = key_index(a.key_in[tid]);
        if (a.key_reset) a.key_reset[tid] = 0ull;
    }

    // weights of this wave's steps (row R0 + j16)
    u32x4_t wa[kMmSteps];
    {
        const int row = R0 + j16;
        const bool rok = j16 < ROWS && row < M;
        const uint16_t *wr = (const uint16_t *)a.W + (int64_t)row * K + 8 * g;
#pragma unroll
        for (int i = 0; i < kMmSteps; ++i) {
            const int t = wid + NW * i;
            wa[i] = (rok && t < KS) ? ld_nt4(wr + 32 * t) : u32x4_t{0, 0, 0, 0};
        }
    }
    // activations of sequence j16 at the same columns
    const bool sok = j16 < S;
    float x[kMmSteps][8];
    float gn[IN == IN_NORM ? kMmSteps : 1][8];
#pragma unroll
    for (int i = 0; i < kMmSteps; ++i) {
        const int t = wid + NW * i;
        const int col = 32 * t + 8 * g;
        if (sok && t < KS) {
            if (IN != IN_EMBED && a.src_op) {
                // operand order: the 16 lanes of a group read 256 contiguous bytes
                const float4 u = *(const float4 *)(a.src_op + op_index(col, j16));
                const float4 v = *(const float4 *)(a.src_op + op_index(col + 4, j16));
                x[i][0] = u.x; x[i][1] = u.y; x[i][2] = u.z; x[i][3] = u.w;
                x[i][4] = v.x; x[i][5] = v.y; x[i][6] = v.z; x[i][7] = v.w;
            } else {
                mm_load_x<IN>(a, j16, col, x[i]);
            }
            if (IN == IN_NORM) {
                const float4 *gp = (const float4 *)(a.gain + col);
                const float4 u = gp[0], v = gp[1];
                float *gi = gn[IN == IN_NORM ? i : 0];
                gi[0] = u.x; gi[1] = u.y; gi[2] = u.z; gi[3] = u.w; gi[4] = v.x; gi[5] = v.y; gi[6] = v.z; gi[7] = v.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
            if (IN == IN_NORM)
#pragma unroll
                for (int e = 0; e < 8; ++e) gn[IN == IN_NORM ? i : 0][e] = 0.f;
        }
    }
    if (IN == IN_NORM) {
        // sum of squares of sequence j16: lane (steps, then values), then the
        // four lane groups, then the waves in order
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < kMmSteps; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(x[i][e], x[i][e], ss);
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        if (g == 0) ssw[wid][j16] = ss;
        __syncthreads();
        float tot = 0.f;
        for (int w = 0; w < NW; ++w) tot += ssw[w][j16];
        const float r = 1.0f / sqrtf(tot / (float)K + a.eps);
#pragma unroll
        for (int i = 0; i < kMmSteps; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = x[i][e] * r * gn[IN == IN_NORM ? i : 0][e];
    }
    f32x4_t acc_h = {0.f, 0.f, 0.f, 0.f}, acc_l = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMmSteps; ++i) {
        if (wid + NW * i >= KS) break;     // wave-uniform
        u32x4_t bh, bl;
        split_bf16(x[i], bh, bl);
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, wa[i]);
        acc_h = mfma(av, __builtin_bit_cast(bf16x8_t, bh), acc_h);
        acc_l = mfma(av, __builtin_bit_cast(bf16x8_t, bl), acc_l);
    }
    red[wid][lane] = acc_h + acc_l;
    __syncthreads();
    // thread -> (sequence s, row rho): 16 consecutive threads own 16 consecutive rows
    for (int o = tid; o < 256; o += NW * 64) {
        const int s = o >> 4, rho = o & 15;
        const int row = R0 + rho;
        if (s >= S || rho >= ROWS || row >= M) continue;
        const int l = s + 16 * (rho >> 2), q = rho & 3;
        float y = 0.f;
        for (int w = 0; w < NW; ++w) y += red[w][l][q];
        float *dp = a.dst + (int64_t)s * a.dst_stride + row;
        const float out = EPI == EPI_STORE ? y : EPI == EPI_ADD ? *dp + y : silu_f(y);
        *dp = out;
        if (a.dst_op) a.dst_op[op_index(row, s)] = out;
    }
}

// ============================================================================
// LM head tile kernel: f = rmsnorm(x; g_final) is staged once per workgroup
// in LDS as the A operand (hi and lo halves); the four waves then stream
// their 16-row head tiles with several 8-step units of weights in flight,
// store the logits, and keep a per-sequence argmax key; the post-projection
// h' = W_post f runs in the same workgroups over the same staged f.
// ============================================================================
static constexpr int kHeadUnit = 8;     // K steps per unit: 16 rows x 256 columns
// bf16 units in flight per wave in head_tiles (a unit carries 8 KiB)
static constexpr int kHeadDepth = 4;

// A bf16 unit in operand order: step k of lane (g, j16) holds row j16's
// 8 columns 32k + 8g .. +7.
template <typename HT>
struct HeadUnit;
template <> struct HeadUnit<uint16_t> {
    u32x4_t w[kHeadUnit];
};

// Staged-activation slot of (step t, half h, lane group g, sequence s): one
// 1 KiB block per (t, h) in lane order, so a wave reads it with a single
// conflict-free ds_read_b128 at a compile-time offset from its lane base.
__device__ __forceinline__ int bslot(int t, int h, int g, int s) { return ((2 * t + h) * 4 + g) * 16 + s; }
// Packed form for at most 8 sequences: one block per step t whose operand
// rows j < 8 hold the hi half of sequence j and rows j >= 8 the lo half of
// sequence j - 8, so one MFMA forms both halves' products (in separate
// output rows, added once per tile).
__device__ __forceinline__ int pslot(int t, int g, int j) { return (t * 4 + g) * 16 + j; }

// Weights of unit c (steps 8c .. 8c+7, 256 columns) of the 16-row tile at
// row0, as loaded.  A wave load that touches 16 rows (the operand order, lane
// l holds row l % 16) streams at ~5.2 TB/s on gfx950, one that touches 4 rows
// x 256 contiguous bytes at ~7.0 TB/s, so a bf16 unit is loaded in that
// second form and put into operand order through a small LDS tile
// (transpose_unit); rows are clamped into the matrix (rows past the end are
// computed but never stored).  A Q8_0 unit comes from the head's unit-order
// copy, where it is one contiguous run already in operand order: four 1 KiB
// wave loads of quants and one of its 256 bytes of scales, no transpose.
template <typename HT>
struct RawUnit;
template <> struct RawUnit<uint16_t> {
    u32x4_t r[8];           // load q: rows 4 (q % 4) + lane / 16, columns 128 (q / 4) + 8 (lane % 16)
};
template <> struct RawUnit<int8_t> {
    u32x4_t r[4];           // load p: K steps 2p and 2p + 1 of the lane's operand
    u32x4_t sc;             // fp16 scales of the lane's row j16 for the unit's 8 blocks
};

template <typename HT>
__device__ __forceinline__ void raw_load_unit(const void *W, int rows, int d, int row0, int c, int lane,
                                              RawUnit<HT> &u) {
    if constexpr (sizeof(HT) == 2) {
        const int rq = lane >> 4, col16 = lane & 15;
        const uint16_t *wc = (const uint16_t *)W + 256 * c + 8 * col16;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            u.r[q] = ld_nt4(wc + (int64_t)min(row0 + 4 * (q & 3) + rq, rows - 1) * d + 128 * (q >> 2));
    } else {
        // W: the unit-order copy, padded to whole tiles (row0 is a tile start).
        // Plain (cached) loads, measured in the draft round of 8 sequences x
        // 131072 cells (285 MB head, V = 262144, d = 1024): 51.6 us with
        // non-temporal loads, 48.8 us plain.  With plain KV loads in the
        // round as well the head takes 55.4 us, so the gain goes with the KV
        // stream's non-temporal loads leaving the last-level cache to the
        // head between steps; holding a fixed 140-240 MB of it cached (the
        // rest non-temporal) gains nothing more.
        const uint8_t *ub = (const uint8_t *)W + ((int64_t)(row0 >> 4) * (d >> 8) + c) * kQ8UnitBytes;
#pragma unroll
        for (int p = 0; p < 4; ++p) u.r[p] = *(const u32x4_t *)(ub + 1024 * p + 16 * lane);
        u.sc = *(const u32x4_t *)(ub + 4096 + 16 * (lane & 15));
    }
}

// Transpose tile of one wave: 16 rows of 256 bytes, rows padded to 272
// bytes so the operand reads (16 rows, one 16- or 8-byte piece each) hit
// distinct banks.  LDS operations of one wave execute in order, so the tile
// is reused unit after unit without waits beyond the data dependences.
static constexpr int kTrStride = 17;        // 16-byte slots per row
static constexpr int kTrSlots = 16 * kTrStride;

template <typename HT>
__device__ __forceinline__ void transpose_unit(const RawUnit<HT> &raw, u32x4_t *tr, int lane, HeadUnit<HT> &u) {
    static_assert(sizeof(HT) == 2, "bf16 units only: Q8_0 units load in operand order");
    const int j16 = lane & 15, g = lane >> 4;
    u32x4_t *wrow = tr + (lane >> 4) * kTrStride + j16;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int q = 0; q < 4; ++q) wrow[4 * q * kTrStride] = raw.r[4 * hf + q];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) u.w[4 * hf + kk] = tr[j16 * kTrStride + 4 * kk + g];
    }
}

__device__ __forceinline__ float sc_at(const u32x4_t &v, int k) {
    const uint32_t w = v[k >> 1];
    return half_to_f((uint16_t)((k & 1) ? (w >> 16) : (w & 0xFFFF)));
}

// MFMAs of one bf16 unit with its activation operands xv (hi, lo per step,
// read from LDS beforehand); acc_h / acc_l carry the tile's running sums.
// The activations are the A operand (rows = sequences) and the weights the B
// operand (columns = vocabulary rows), so a lane's four results share its
// weight row j16.
template <typename HT>
__device__ __forceinline__ void head_unit_mma(const HeadUnit<HT> &u, const u32x4_t (&xv)[2 * kHeadUnit],
                                              f32x4_t &acc_h, f32x4_t &acc_l) {
    static_assert(sizeof(HT) == 2, "bf16 units only");
#pragma unroll
    for (int k = 0; k < kHeadUnit; ++k) {
        const bf16x8_t wv = __builtin_bit_cast(bf16x8_t, u.w[k]);
        acc_h = mfma(__builtin_bit_cast(bf16x8_t, xv[2 * k]), wv, acc_h);
        acc_l = mfma(__builtin_bit_cast(bf16x8_t, xv[2 * k + 1]), wv, acc_l);
    }
}

// The 16-row tiles [T0, T1) of one workgroup: wave w takes T0 + w, T0 + w + 4,
// ...  Units go through a ring of DEPTH raw units (loaded DEPTH units
// ahead); unit u + 1 is transposed into operand order while unit u's
// MFMAs run.  UPT units make a tile and DEPTH is a multiple of UPT, so
// a tile's epilogue sits at a fixed ring position; loads and stores are
// unconditional (tiles past the wave's last one load the matrix's first unit
// and store to `sink`), which keeps the loop body straight-line and lets the
// compiler wait for exactly the unit it is about to use.
//   HEAD: argmax key over valid rows, logits to `out` when LOGITS
//   else: rows stored to `out` (the post-projection)
// stage() (the workgroup's activation staging, with its barriers) runs once
// the ring's first loads are issued.
template <typename HT, int UPT, bool HEAD, bool LOGITS, typename Stage>
__device__ void head_tiles(const HeadArgs &a, const void *W, int rows, int T0, int T1,
                           const u32x4_t *bsm, u32x4_t *tr, float *out, int64_t out_stride, uint64_t (&best)[4],
                           float (&cm)[4], float (&cs)[4], Stage &&stage) {
    const bool conf = HEAD && a.conf != nullptr;
    static_assert(sizeof(HT) == 2, "bf16 heads only: the Q8_0 head runs q8_head_tiles");
    constexpr int DEPTH = kHeadDepth;
    constexpr int TPI = DEPTH / UPT;        // tiles per loop iteration
    static_assert(DEPTH % UPT == 0, "ring must hold whole tiles");
    static_assert(DEPTH % 2 == 0, "operand buffers alternate with the ring position");
    const int d = a.d, S = a.S;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j16 = lane & 15, g = lane >> 4;
    const int nt = T1 - T0 > wid ? (T1 - T0 - wid + 3) / 4 : 0;
    const int nit = (nt + TPI - 1) / TPI;
    auto load = [&](int i, int c, RawUnit<HT> &dst) {
        const bool real = i < nt;
        raw_load_unit<HT>(W, rows, d, real ? 16 * (T0 + wid + 4 * i) : 0, real ? c : 0, lane, dst);
    };
    RawUnit<HT> raw[DEPTH];
    HeadUnit<HT> op[2];
#pragma unroll
    for (int p = 0; p < DEPTH; ++p) load(p / UPT, p % UPT, raw[p]);
    stage();                                // the activations, while the first weights arrive
    transpose_unit<HT>(raw[0], tr, lane, op[0]);
    load(TPI, 0, raw[0]);
    f32x4_t acc_h = {0.f, 0.f, 0.f, 0.f}, acc_l = {0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < nit; ++it) {
#pragma unroll
        for (int p = 0; p < DEPTH; ++p) {
            const int i = it * TPI + p / UPT, c = p % UPT;
            // unit u + 1 into operand order, then its ring slot refills with
            // unit u + 1 + DEPTH
            const int pn = (p + 1) % DEPTH;
            const int un_i = it * TPI + (p + 1) / UPT + TPI, un_c = pn % UPT;
            // this unit's activation operands first: they arrive while the
            // next unit is transposed
            u32x4_t xv[2 * kHeadUnit];
            const u32x4_t *xb = bsm + bslot(c * kHeadUnit, 0, g, j16);
#pragma unroll
            for (int k = 0; k < kHeadUnit; ++k) {
                xv[2 * k] = xb[128 * k];
                xv[2 * k + 1] = xb[128 * k + 64];
            }
            transpose_unit<HT>(raw[pn], tr, lane, op[(p + 1) & 1]);
            load(un_i, un_c, raw[pn]);
            head_unit_mma<HT>(op[p & 1], xv, acc_h, acc_l);
            if (c == UPT - 1) {
                // lane (j16, g) holds row 16 tile + j16 for sequences 4g .. 4g+3
                const int r = 16 * (T0 + wid + 4 * i) + j16;
                const f32x4_t z = acc_h + acc_l;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int sq = 4 * g + q;
                    const bool ok = i < nt && sq < S && r < rows;
                    if (HEAD) {
                        const uint64_t k = ok ? argmax_key(z[q], (uint32_t)r) : 0ull;
                        best[q] = k > best[q] ? k : best[q];
                        if (conf && ok) conf_add(cm[q], cs[q], z[q]);
                    }
                    if (!HEAD || LOGITS) *(ok ? out + (int64_t)sq * out_stride + r : a.sink + lane) = z[q];
                }
                acc_h = f32x4_t{0.f, 0.f, 0.f, 0.f};
                acc_l = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
            // issue order within the unit: activation reads, the next unit's
            // transpose, its ring refill, then the MFMAs (left alone, the
            // compiler reads each activation operand just before its MFMA)
            constexpr int n_ld = 8;
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kHeadUnit, 0);     // LDS reads: activations
            __builtin_amdgcn_sched_group_barrier(0x300, 16, 0);                // LDS writes / reads: transpose
            __builtin_amdgcn_sched_group_barrier(0x020, n_ld, 0);              // global loads
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * kHeadUnit, 0);     // MFMA
            __builtin_amdgcn_sched_barrier(0);  // keep each unit's transpose and loads next to its MFMAs
        }
    }
}

// Q8_0 units in flight per wave in the Q8_0 head (a multiple of 4, so of
// every units-per-tile count; 8 measured slower than 4 at 8 sequences).
static constexpr int kQ8Depth = 4;

// MFMAs of one Q8_0 unit, straight from the ring: per block the hi and lo
// activation products go into one accumulation (hi first), which the block's
// scale then adds to the tile's running sums, in block order.  xb: the
// unit's first activation slot.  The schedule is pinned block by block (the
// empty volatile asm statements: each block's operands are complete there
// and nothing of a later block moves above it): the next block's activations
// are read while this block converts its quants and issues its MFMAs, and a
// block is scaled in while the next one's MFMAs run.  Left free, the
// compiler converts and reads ahead for every block at once and the wave
// needs more than its half of the register file.
// PACK: the activations in the packed form (one MFMA per block; a lane's
// results are the hi or the lo products of its four sequences).
template <bool PACK>
__device__ __forceinline__ void q8_unit_mma(const RawUnit<int8_t> &u, const u32x4_t *xb, f32x4_t &acc) {
    constexpr int XS = PACK ? 64 : 128;     // slots per step
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    u32x4_t xh = xb[0], xl = PACK ? xh : xb[64];
    f32x4_t pp = z;
    float spp = 0.f;
#pragma unroll
    for (int k = 0; k < kHeadUnit; ++k) {
        const u32x4_t &r = u.r[k >> 1];
        u32x2_t q = (k & 1) ? u32x2_t{r[2], r[3]} : u32x2_t{r[0], r[1]};
        if constexpr (PACK) asm volatile("" : "+v"(q), "+v"(xh) : : "memory");
        else asm volatile("" : "+v"(q), "+v"(xh), "+v"(xl) : : "memory");
        u32x4_t nxh = xh, nxl = xl;
        if (k + 1 < kHeadUnit) {
            nxh = xb[XS * (k + 1)];
            if constexpr (!PACK) nxl = xb[XS * (k + 1) + 64];
        }
        const bf16x8_t wv = __builtin_bit_cast(bf16x8_t, q8_to_bf16(q));
        f32x4_t pk = mfma(__builtin_bit_cast(bf16x8_t, xh), wv, z);
        if constexpr (!PACK) pk = mfma(__builtin_bit_cast(bf16x8_t, xl), wv, pk);
        if (k > 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = fmaf(spp, pp[i], acc[i]);
        }
        pp = pk;
        spp = sc_at(u.sc, k);
        xh = nxh;
        xl = nxl;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(spp, pp[i], acc[i]);
    // the unit's scaling is done here: sunk to the tile's end, it would keep
    // every unit's scales out of the ring slots being refilled
    asm volatile("" : "+v"(acc));
}

// The 16-row tiles [T0, T1) of one workgroup for a Q8_0 head: wave w takes
// T0 + w, T0 + w + 4, ...; its units (UPT per tile) stream through a ring of
// kQ8Depth slots, each refilled as soon as its unit's MFMAs are issued.  The
// unit-order copy is already in operand order, so nothing goes through LDS
// but the activations.  Loads past the wave's last unit read the first unit
// of the matrix and their results are never stored (as in head_tiles).  The
// last ring pass is peeled: it refills nothing, and before it last() requests
// what the workgroup needs after the head (the post-projection's weights),
// into the registers the ring is about to free.
template <int UPT, bool LOGITS, bool PACK, typename StageLoad, typename StageFinish, typename Last>
__device__ void q8_head_tiles(const HeadArgs &a, int T0, int T1, const u32x4_t *bsm, float *out, int64_t out_stride,
                              uint64_t (&best)[4], float (&cm)[4], float (&cs)[4], StageLoad &&stage_load,
                              StageFinish &&stage_finish, Last &&last) {
    constexpr int DEPTH = kQ8Depth;
    static_assert(DEPTH % UPT == 0, "ring must hold whole tiles");
    constexpr int TPI = DEPTH / UPT;        // tiles per loop iteration
    const bool conf = a.conf != nullptr;
    const int d = a.d, S = a.S;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j16 = lane & 15, g = lane >> 4;
    const int nt = T1 - T0 > wid ? (T1 - T0 - wid + 3) / 4 : 0;
    const int nit = (nt + TPI - 1) / TPI;
    auto load = [&](int i, int c, RawUnit<int8_t> &dst) {
        const bool real = i < nt;
        raw_load_unit<int8_t>(a.head_qt, a.V, d, real ? 16 * (T0 + wid + 4 * i) : 0, real ? c : 0, lane, dst);
    };
    RawUnit<int8_t> raw[DEPTH];
    stage_load();                           // x and the gain (from L2) ahead of the weights
    asm volatile("" : : : "memory");        // keeps them first in the load queue
#pragma unroll
    for (int p = 0; p < DEPTH; ++p) load(p / UPT, p % UPT, raw[p]);
    stage_finish();                         // the activations, while the first weights arrive
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    auto pass = [&](int it, auto refill) {
#pragma unroll
        for (int p = 0; p < DEPTH; ++p) {
            const int i = it * TPI + p / UPT, c = p % UPT;
            // the activations are the same for every tile: left visible, the
            // compiler hoists all of them out of the loop and spills.  Only the
            // lane's base offset is hidden; the rest stays an immediate.
            int lb = PACK ? pslot(0, g, j16) : bslot(0, 0, g, j16);
            asm volatile("" : "+v"(lb));
            q8_unit_mma<PACK>(raw[p], bsm + lb + (PACK ? pslot(c * kHeadUnit, 0, 0) : bslot(c * kHeadUnit, 0, 0, 0)),
                              acc);
            if constexpr (decltype(refill)::value) load(i + TPI, c, raw[p]);
            if (c == UPT - 1) {
                // lane (j16, g) holds row 16 tile + j16 for sequences 4g .. 4g+3;
                // packed: lanes g < 2 the hi products, lanes g + 2 the lo ones
                const int r = 16 * (T0 + wid + 4 * i) + j16;
                f32x4_t zt = acc;
                if constexpr (PACK) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) zt[q] = acc[q] + __shfl_xor(acc[q], 32);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int sq = 4 * g + q;
                    const bool ok = (!PACK || g < 2) && i < nt && sq < S && r < a.V;
                    const uint64_t k = ok ? argmax_key(zt[q], (uint32_t)r) : 0ull;
                    best[q] = k > best[q] ? k : best[q];
                    if (conf && ok) conf_add(cm[q], cs[q], zt[q]);
                    if (LOGITS) *(ok ? out + (int64_t)sq * out_stride + r : a.sink + lane) = zt[q];
                }
                acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
            __builtin_amdgcn_sched_barrier(0);  // no instruction moves across units
        }
    };
    for (int it = 0; it + 1 < nit; ++it) pass(it, std::true_type{});
    last();
    if (nit > 0) pass(nit - 1, std::false_type{});
}

// A bf16 unit loaded straight in operand order (lane l: row l % 16, 8
// columns per step): the post-projection of the Q8_0 head, whose few units do
// not need the faster row-block loads and whose workgroups keep no transpose
// tile.
__device__ __forceinline__ void direct_load_unit(const void *W, int rows, int d, int row0, int c, int lane,
                                                 HeadUnit<uint16_t> &u) {
    const uint16_t *wr = (const uint16_t *)W + (int64_t)min(row0 + (lane & 15), rows - 1) * d + 256 * c + 8 * (lane >> 4);
#pragma unroll
    for (int k = 0; k < kHeadUnit; ++k) u.w[k] = ld_nt4(wr + 32 * k);
}

// The several-sequence LM head.  A Q8_0 head keeps no transpose tile, so two
// workgroups fit a CU and each wave has half the register file.
template <typename HT, int UPT, bool LOGITS, bool PACK>
__device__ __forceinline__ void mm_head_body(const HeadArgs &a, int tiles_per_wg) {
    constexpr bool Q8 = sizeof(HT) == 1;
    static_assert(Q8 || !PACK, "the packed activations serve the Q8_0 head");
    extern __shared__ u32x4_t mm_bsm[];     // activation halves: [KS][2][4][16] (bslot), packed [KS][4][16] (pslot)
    __shared__ u32x4_t mm_tr[Q8 ? 1 : 4 * kTrSlots];    // one weight transpose tile per wave (bf16)
    __shared__ float rsw[4][16];            // per-wave partial sums of squares of each sequence
    __shared__ uint64_t wbest[4][16];
    __shared__ float wcm[4][16], wcs[4][16];
    __shared__ f32x4_t post_part[4][64];    // per-wave partial sums of a post-projection tile
    const int d = a.d, S = a.S;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int hb = blockIdx.x;

    // f = rmsnorm(x; g_final) -> activation halves (sequences >= S stay zero),
    // run by head_tiles once its first weights are requested.  Thread tid
    // stages the slots tid + 256 k, all of sequence s = tid % 16: it loads
    // its 16 * UPT column groups of x and of the gain at once, sums its
    // squares, and the 16 threads of a sequence (4 lanes of each wave) add
    // theirs in a fixed order, so the stage costs one memory round trip.
    // (stage_load requests x and the gain; stage_finish waits for them and
    // fills the LDS.  The Q8_0 kernel requests its first weights between the
    // two, so that its staging waits for x alone, not for those weights.)
    constexpr int NIT = 2 * UPT;            // KS * 64 / 256 slots per thread
    const int s_st = tid & 15;
    const int sx = PACK ? (s_st & 7) : s_st;    // the sequence this thread stages (packed: rows s, s + 8)
    float v[NIT][8], gv[NIT][8];
    auto stage_load = [&]() {
        const float *xs = a.x + (int64_t)min(sx, S - 1) * d;
#pragma unroll
        for (int k = 0; k < NIT; ++k) {
            const int it = tid + 256 * k, t = it >> 6, g = (it >> 4) & 3;
            const int col = 32 * t + 8 * g;
            const float4 x0 = *(const float4 *)(xs + col), x1 = *(const float4 *)(xs + col + 4);
            v[k][0] = x0.x; v[k][1] = x0.y; v[k][2] = x0.z; v[k][3] = x0.w;
            v[k][4] = x1.x; v[k][5] = x1.y; v[k][6] = x1.z; v[k][7] = x1.w;
            const float4 g0 = *(const float4 *)(a.g_final + col), g1 = *(const float4 *)(a.g_final + col + 4);
            gv[k][0] = g0.x; gv[k][1] = g0.y; gv[k][2] = g0.z; gv[k][3] = g0.w;
            gv[k][4] = g1.x; gv[k][5] = g1.y; gv[k][6] = g1.z; gv[k][7] = g1.w;
        }
    };
    auto stage_finish = [&]() {
        const int s = s_st;
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < NIT; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(v[k][e], v[k][e], ss);
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        if (lane < 16) rsw[wid][lane] = ss;
        __syncthreads();
        const float r = 1.0f / sqrtf(((rsw[0][s] + rsw[1][s]) + (rsw[2][s] + rsw[3][s])) / (float)d + a.eps);
#pragma unroll
        for (int k = 0; k < NIT; ++k) {
            const int it = tid + 256 * k, t = it >> 6, g = (it >> 4) & 3;
            u32x4_t hi = {0, 0, 0, 0}, lo = {0, 0, 0, 0};
            if (sx < S) {
                float f[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = v[k][e] * r * gv[k][e];
                split_bf16(f, hi, lo);
            }
            if constexpr (PACK) {
                mm_bsm[pslot(t, g, s)] = s < 8 ? hi : lo;
            } else {
                mm_bsm[bslot(t, 0, g, s)] = hi;
                mm_bsm[bslot(t, 1, g, s)] = lo;
            }
        }
        __syncthreads();
    };
    auto stage = [&]() {
        stage_load();
        stage_finish();
    };

    uint64_t best[4] = {0ull, 0ull, 0ull, 0ull};   // sequences 4g .. 4g+3 of this lane
    float cm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, cs[4] = {0.f, 0.f, 0.f, 0.f};
    // Post-projection h' = W_post f: one 16-row tile for each of the first
    // ceil(dh / 16) workgroups, its K chunks (units) dealt out to the waves,
    // one unit each, the partial sums added in wave order.  The tile's
    // weights are requested before the head's and used after them, so the
    // projection costs a unit of streaming per wave and no extra latency.
    const int n_post_tiles = (a.dh + 15) / 16;
    const bool post_unit = wid < UPT;
    std::conditional_t<Q8, HeadUnit<uint16_t>, RawUnit<uint16_t>> praw;
    auto load_post = [&](int tb) {
        if constexpr (Q8) direct_load_unit(a.w_post, a.dh, d, 16 * tb, wid, lane, praw);
        else raw_load_unit<uint16_t>(a.w_post, a.dh, d, 16 * tb, wid, lane, praw);
    };
    // (the Q8_0 kernel's half register file has no room to hold them through
    // the head: it requests them before its last ring pass)
    auto post_first = [&]() {
        if (hb < n_post_tiles && post_unit) load_post(hb);
    };
    if (!Q8) post_first();
    {
        float *logits = a.io->out_logits ? a.io->out_logits + (int64_t)a.step * a.V : a.sink;
        const int64_t logits_stride = (int64_t)a.n_steps * a.V;
        const int n_tiles = (a.V + 15) / 16;
        const int T0 = hb * tiles_per_wg, T1 = min(n_tiles, T0 + tiles_per_wg);
        if constexpr (Q8)
            q8_head_tiles<UPT, LOGITS, PACK>(a, T0, T1, mm_bsm, logits, logits_stride, best, cm, cs, stage_load,
                                             stage_finish, post_first);
        else
            head_tiles<HT, UPT, true, LOGITS>(a, a.head, a.V, T0, T1, mm_bsm, mm_tr + wid * kTrSlots, logits,
                                              logits_stride, best, cm, cs, stage);
        // best over the 16 rows of each lane group: xor-shuffles within 16 lanes
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) {
                const uint64_t o = shfl_xor_u64(best[q], m);
                best[q] = o > best[q] ? o : best[q];
            }
        }
        const bool conf = a.conf != nullptr;
        if (conf) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int m = 1; m < 16; m <<= 1) {
                    const float om = __shfl_xor(cm[q], m), os = __shfl_xor(cs[q], m);
                    conf_merge(cm[q], cs[q], om, os);
                }
            }
        }
        if ((lane & 15) == 0)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wbest[wid][4 * (lane >> 4) + q] = best[q];
                wcm[wid][4 * (lane >> 4) + q] = cm[q];
                wcs[wid][4 * (lane >> 4) + q] = cs[q];
            }
    }
    // The post-projection tile(s) of this workgroup: tb = hb, hb + the grid,
    // ...  Each wave multiplies its unit as soon as its head tiles are done
    // and leaves the partial sums in LDS; the first tile shares the barrier of
    // the argmax reduction, so its sum and store go out beside the atomics.
    float *h_out = (a.step == a.n_steps - 1 && a.io->out_h_last) ? a.io->out_h_last : a.h_out;
    const int j16 = lane & 15, g = lane >> 4;
    auto post_mma = [&](int tb) {
        if (tb != hb && post_unit) load_post(tb);
        f32x4_t ph = {0.f, 0.f, 0.f, 0.f}, pl = {0.f, 0.f, 0.f, 0.f};
        if (post_unit) {
            HeadUnit<uint16_t> u;
            if constexpr (Q8) u = praw;
            else transpose_unit<uint16_t>(praw, mm_tr + wid * kTrSlots, lane, u);
            if constexpr (PACK) {
                // hi products in lanes g < 2, lo products in lanes g + 2
                const u32x4_t *xb = mm_bsm + pslot(wid * kHeadUnit, g, j16);
#pragma unroll
                for (int k = 0; k < kHeadUnit; ++k)
                    ph = mfma(__builtin_bit_cast(bf16x8_t, xb[64 * k]), __builtin_bit_cast(bf16x8_t, u.w[k]), ph);
            } else {
                u32x4_t xv[2 * kHeadUnit];
                const u32x4_t *xb = mm_bsm + bslot(wid * kHeadUnit, 0, g, j16);
#pragma unroll
                for (int k = 0; k < kHeadUnit; ++k) {
                    xv[2 * k] = xb[128 * k];
                    xv[2 * k + 1] = xb[128 * k + 64];
                }
                head_unit_mma<uint16_t>(u, xv, ph, pl);
            }
        }
        post_part[wid][lane] = PACK ? ph : ph + pl;
    };
    auto post_store = [&](int tb) {
        if (wid == 0 && (!PACK || lane < 32)) {
            // lane (j16, g) holds row 16 tb + j16 for sequences 4g .. 4g+3
            // (packed: hi + lo of the same wave first, as unpacked)
            auto part = [&](int w) { return PACK ? post_part[w][lane] + post_part[w][lane + 32] : post_part[w][lane]; };
            f32x4_t z = part(0);
            for (int w = 1; w < UPT; ++w) z += part(w);
            const int r = 16 * tb + j16;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (r < a.dh && 4 * g + q < S) h_out[(int64_t)(4 * g + q) * a.dh + r] = z[q];
        }
    };
    if (hb < n_post_tiles) post_mma(hb);
    __syncthreads();
    if (tid < S) {
        uint64_t k = wbest[0][tid];
        for (int w = 1; w < 4; ++w) k = wbest[w][tid] > k ? wbest[w][tid] : k;
        atomicMax((unsigned long long *)&a.keys[tid], (unsigned long long)k);
        if (a.conf) {
            float m = wcm[0][tid], sm = wcs[0][tid];
            for (int w = 1; w < 4; ++w) conf_merge(m, sm, wcm[w][tid], wcs[w][tid]);
            a.conf[(int64_t)tid * kConfSlots + hb] = ConfPart{m, sm};
        }
    }
    if (hb < n_post_tiles) post_store(hb);
    for (int tb = hb + (int)gridDim.x; tb < n_post_tiles; tb += (int)gridDim.x) {
        __syncthreads();        // the previous tile's partial sums are read
        post_mma(tb);
        __syncthreads();
        post_store(tb);
    }
}

// bf16: one workgroup per CU at d = 1024 (the LDS holds one), so the register
// file may hold one wave per SIMD: the activation operands of a whole unit
// are read ahead of its MFMAs.
template <typename HT, int UPT, bool LOGITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void mm_head_kernel(HeadArgs a,
                                                                                                 int tiles_per_wg) {
    mm_head_body<HT, UPT, LOGITS, false>(a, tiles_per_wg);
}

// Q8_0: two workgroups per CU, two waves per SIMD; PACK for at most 8
// sequences.
template <int UPT, bool LOGITS, bool PACK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void mm_q8_head_kernel(HeadArgs a,
                                                                                                    int tiles_per_wg) {
    mm_head_body<int8_t, UPT, LOGITS, PACK>(a, tiles_per_wg);
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------
bool mm_gemv_supported(int w_dtype, const GemvArgs &a) {
    return w_dtype == MTP_BF16 && a.S >= kMmMinSeqs && a.S <= 16 && a.K % 32 == 0 && a.K <= 16 * kMmSteps * 32;
}

// Weight rows per workgroup tile: halved from 16 (down to 2) while the
// matrix has fewer than 256 tiles, one per CU.  Measured against 16-row tiles
// with the M = 1024 down projection split over K (4 runs + a reduce): rounds
// of 8 sequences x 131072 cells 5.99 -> 5.96 ms, 16 sequences over SWA + full
// KV 1.213 -> 1.185 ms, 8 sequences over a sink + window 0.789 -> 0.755 ms;
// with 512 tiles as the target (2- and 4-row tiles) all three got slower
// (6.13, 1.357, 0.893 ms).
static int mm_gemv_rows(const GemvArgs &a) {
    int rows = 16;
    while (rows > 2 && (a.M + rows - 1) / rows < 256) rows /= 2;
    return rows;
}

hipError_t launch_mm_gemv(int in_mode, int epi, const GemvArgs &a, hipStream_t st) {
    const int KS = a.K / 32;
    const int nw = KS <= 4 * kMmSteps ? 4 : KS <= 8 * kMmSteps ? 8 : 16;
    const int rows = mm_gemv_rows(a);
    const dim3 grid((a.M + rows - 1) / rows);
#define MTP_MM_CASE_R(NW, I, E, R)                                                                     \
    if (nw == NW && in_mode == I && epi == E && rows == R) {                                           \
        mtp_launch((mm_gemv_kernel<NW, I, E, R>), grid, dim3(NW * 64), 0, st, a);               \
        return hipGetLastError();                                                                      \
    }
#define MTP_MM_CASE(NW, I, E)   \
    MTP_MM_CASE_R(NW, I, E, 16) \
    MTP_MM_CASE_R(NW, I, E, 8)  \
    MTP_MM_CASE_R(NW, I, E, 4)  \
    MTP_MM_CASE_R(NW, I, E, 2)
#define MTP_MM_NW(NW)                          \
    MTP_MM_CASE(NW, IN_EMBED, EPI_STORE)       \
    MTP_MM_CASE(NW, IN_NORM, EPI_STORE)        \
    MTP_MM_CASE(NW, IN_NORM, EPI_SILU)         \
    MTP_MM_CASE(NW, IN_PLAIN, EPI_ADD)
    MTP_MM_NW(4)
    MTP_MM_NW(8)
    MTP_MM_NW(16)
#undef MTP_MM_NW
#undef MTP_MM_CASE
#undef MTP_MM_CASE_R
    return hipErrorInvalidValue;
}

bool mm_head_supported(int head_dtype, int w_dtype, const HeadArgs &a) {
    const int upt = a.d / (32 * kHeadUnit);
    return w_dtype == MTP_BF16 && (head_dtype == MTP_BF16 || (head_dtype == MTP_Q8_0 && a.head_qt)) && a.S >= kMmMinSeqs &&
           a.S <= 16 && a.d % (32 * kHeadUnit) == 0 && (upt == 1 || upt == 2 || upt == 4) && a.sink;
}

template <typename K>
static hipError_t launch_head_k(K kernel, const HeadArgs &a, int tiles_per_wg, dim3 grid, size_t lds, hipStream_t st) {
    hipError_t e = allow_dynamic_lds(kernel, lds);
    if (e != hipSuccess) return e;
    mtp_launch(kernel, grid, dim3(256), lds, st, a, tiles_per_wg);
    return hipGetLastError();
}

template <typename HT, int UPT>
static hipError_t launch_mm_head_t(const HeadArgs &a, int tiles_per_wg, dim3 grid, size_t lds, bool logits,
                                   hipStream_t st) {
    if constexpr (sizeof(HT) == 1) {
        if (a.S <= 8)
            return logits ? launch_head_k(mm_q8_head_kernel<UPT, true, true>, a, tiles_per_wg, grid, lds, st)
                          : launch_head_k(mm_q8_head_kernel<UPT, false, true>, a, tiles_per_wg, grid, lds, st);
        return logits ? launch_head_k(mm_q8_head_kernel<UPT, true, false>, a, tiles_per_wg, grid, lds, st)
                      : launch_head_k(mm_q8_head_kernel<UPT, false, false>, a, tiles_per_wg, grid, lds, st);
    } else {
        return logits ? launch_head_k(mm_head_kernel<HT, UPT, true>, a, tiles_per_wg, grid, lds, st)
                      : launch_head_k(mm_head_kernel<HT, UPT, false>, a, tiles_per_wg, grid, lds, st);
    }
}

// Head workgroups of a launch and the 16-row tiles each takes.
// Dynamic LDS of a launch: the staged activations.
static size_t mm_head_lds(int head_dtype, const HeadArgs &a) {
    const bool pack = head_dtype == MTP_Q8_0 && a.S <= 8;
    return sizeof(u32x4_t) * (size_t)(pack ? 64 : 128) * (a.d / 32);
}

static void mm_head_grid(int head_dtype, const HeadArgs &a, int &n_wg, int &tiles_per_wg) {
    // activations + the static transpose tiles (bf16) and reduction slots; the
    // Q8_0 kernel's registers hold two workgroups per CU at most
    const bool q8 = head_dtype == MTP_Q8_0;
    const size_t tr = q8 ? 1 : 4 * kTrSlots;
    const size_t lds = mm_head_lds(head_dtype, a) + sizeof(u32x4_t) * (tr + 4 * 64) + 2048;
    const int per_cu = (int)std::max<size_t>(1, std::min<size_t>(q8 ? 2 : 4, (160 * 1024) / lds));
    const int n_tiles = (a.V + 15) / 16;
    n_wg = std::min(256 * per_cu, (n_tiles + 3) / 4);
    tiles_per_wg = (n_tiles + n_wg - 1) / n_wg;
    n_wg = (n_tiles + tiles_per_wg - 1) / tiles_per_wg;
}

int mm_head_groups(int head_dtype, const HeadArgs &a) {
    int n_wg, tpw;
    mm_head_grid(head_dtype, a, n_wg, tpw);
    return n_wg;
}

hipError_t launch_mm_head(int head_dtype, const HeadArgs &a_in, bool logits, hipStream_t st) {
    HeadArgs a = a_in;
    const int upt = a.d / (32 * kHeadUnit);
    const size_t lds = mm_head_lds(head_dtype, a);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    int n_wg, tiles_per_wg;
    mm_head_grid(head_dtype, a, n_wg, tiles_per_wg);
    a.n_head_wg = n_wg;
    const dim3 grid(n_wg);
#define MTP_MMH(HT, U)                                                                                 \
    if (upt == U) return launch_mm_head_t<HT, U>(a, tiles_per_wg, grid, lds, logits, st);
    if (head_dtype == MTP_BF16) {
        MTP_MMH(uint16_t, 1)
        MTP_MMH(uint16_t, 2)
        MTP_MMH(uint16_t, 4)
    } else {
        MTP_MMH(int8_t, 1)
        MTP_MMH(int8_t, 2)
        MTP_MMH(int8_t, 4)
    }
#undef MTP_MMH
    return hipErrorInvalidValue;
}

}  // namespace mtp
