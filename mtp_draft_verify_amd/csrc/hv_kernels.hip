// hv_kernels.hip -- greedy verify from the target's final hidden rows: its
// final RMSNorm, its LM head over the R = S (N + 1) verify rows, and the
// argmax, with no logit row ever written to memory.
//
// Verifying the 1 + N positions of a round reads the head weights once for
// all of them ("MTP decoding", why a wider decode can be faster), so this is
// a real (skinny) contraction Z[row, v] = sum_c W[v, c] f[row, c] and runs on
// the matrix cores (v_mfma_f32_16x16x32_bf16; operand layout as in
// mfma_kernels.hip: activations are the A operand, one 16-row group of verify
// rows; weights the B operand, one 16-row vocabulary tile).  The fp32 rows
// enter as an exact-to-2^-18 pair of bf16 halves, so the products keep fp32
// accuracy.
//
// Up to 64 rows (RG groups of 16) share one pass over the head.  Staged
// whole, the rows would need R * d * 4 bytes of LDS (720 KiB for 64 rows of
// 2816), so they are staged in chunks of 256 columns, double-buffered:
// while the waves multiply chunk c of their tiles, the next chunk's
// activations (from an L2-resident plane written once by hv_prep_kernel) and
// weights are already loading.
#include <algorithm>

#include "widen.h"

namespace mtp {

typedef __bf16 hv_bf16x8_t __attribute__((ext_vector_type(8)));

static constexpr int kHvTW = 2;        // 16-row vocabulary tiles per wave in a tile group
static constexpr int kHvChunk = 8;     // K steps of 32 columns per staged chunk (256 columns)
static constexpr int kHvMaxRG = 4;     // row groups of 16 per pass (64 rows)

// Staged slot of (step t, half h, row group rg, lane l = 16 g + s) in one
// chunk: each (t, h, rg) owns a 1 KiB block in lane order, so a wave reads
// its A operand with one conflict-free ds_read_b128.
template <int RG>
__device__ __forceinline__ int hv_slot(int t, int h, int rg, int l) { return ((t * 2 + h) * RG + rg) * 64 + l; }

template <int RG>
__host__ __device__ constexpr int hv_chunk_slots() { return kHvChunk * 2 * RG * 64; }

// f = rmsnorm(x; g) (or x when g is null) for the 16 RG rows of a pass, as
// bf16 hi / lo halves in the per-chunk slot order; rows >= R are zero.
template <int RG>
__global__ __launch_bounds__(256) void hv_prep_kernel(HvArgs a) {
    __shared__ float red[4];
    constexpr int CS = hv_chunk_slots<RG>();
    const int row = blockIdx.x, rg = row >> 4, s = row & 15;
    const int d = a.d, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const bool real = row < a.R;
    const float *x = a.hidden + (int64_t)(a.row0 + (real ? row : 0)) * d;     // rows >= R read row 0, unused
    float r = 1.0f;
    if (a.g) {
        float ss = 0.f;
        for (int c = tid; c < d; c += 256) ss = fmaf(x[c], x[c], ss);
        ss = wave_sum(ss);
        if (lane == 0) red[wid] = ss;
        __syncthreads();
        r = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + a.eps);
    }
    for (int j = tid; j < d / 8; j += 256) {
        const int col = 8 * j, c = col >> 8, t = (col >> 5) & 7, g = (col >> 3) & 3;
        u32x4_t hi = {0, 0, 0, 0}, lo = {0, 0, 0, 0};
        if (real) {
            const float4 x0 = ((const float4 *)(x + col))[0], x1 = ((const float4 *)(x + col))[1];
            float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            if (a.g) {
                const float4 g0 = ((const float4 *)(a.g + col))[0], g1 = ((const float4 *)(a.g + col))[1];
                const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = v[i] * r * gv[i];
            }
            hv_bf16x8_t h8, l8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const __bf16 b = (__bf16)v[i];
                h8[i] = b;
                l8[i] = (__bf16)(v[i] - (float)b);
            }
            hi = __builtin_bit_cast(u32x4_t, h8);
            lo = __builtin_bit_cast(u32x4_t, l8);
        }
        u32x4_t *plane = (u32x4_t *)a.plane + (int64_t)c * CS;
        plane[hv_slot<RG>(t, 0, rg, 16 * g + s)] = hi;
        plane[hv_slot<RG>(t, 1, rg, 16 * g + s)] = lo;
    }
}

// One workgroup owns tile groups [G0, G1) (a group is 4 waves x TW tiles
// of 16 vocabulary rows) and walks (group, chunk) pairs in order; the
// accumulators of a wave's tiles live across the chunks of a group, and the
// group's last chunk folds them into per-row argmax keys.
//
// Weights.  A load instruction that touches 16 rows (the MFMA operand order:
// lane l holds row l % 16) streams at ~5.2 TB/s on gfx950; one that touches
// 4 rows x 256 contiguous bytes streams at ~7.0 TB/s.  So a tile's half chunk
// (16 rows x 4 steps x 32 columns) is loaded as 4 such instructions into a
// raw register ring, a chunk ahead, then passed through a small wave-private
// LDS tile into operand order: 4 writes of 4 rows, 4 reads of one step each.
// Each half chunk of the next chunk is transposed while the MFMAs of this
// chunk's other half run.
// LOGITS: write the logit rows to a.logits instead of argmax keys (for the
// sampling verify, which needs every row's whole distribution).
template <int RG, int TW, bool LOGITS>
__global__ __launch_bounds__(256) void hv_head_kernel(HvArgs a, int groups_per_wg) {
    static_assert(TW == 2, "the transpose schedule spreads two tiles over a half chunk's four steps");
    constexpr int TS = 17;                  // transpose tile row stride in 16-byte slots (256 B + 16 B pad)
    extern __shared__ u32x4_t hv_lds[];     // [2][CS]
    __shared__ u32x4_t hv_tr[4][16 * TS];   // one transpose tile per wave
    __shared__ uint64_t wbest[4][16 * RG];
    constexpr int CS = hv_chunk_slots<RG>();
    constexpr int SPT = CS / 256;           // staged slots per thread per chunk
    const int d = a.d, NC = d / (32 * kHvChunk);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j16 = lane & 15, g = lane >> 4;
    const int n_tiles = (a.V + 15) / 16;
    const int n_groups = (n_tiles + 4 * TW - 1) / (4 * TW);
    const int G0 = blockIdx.x * groups_per_wg, G1 = min(n_groups, G0 + groups_per_wg);
    const uint16_t *W = (const uint16_t *)a.head;
    const u32x4_t *plane = (const u32x4_t *)a.plane;
    u32x4_t *tr = hv_tr[wid];

    // Raw load q of half hf of tile i of (group, chunk): rows 4 q + lane / 16
    // of the tile, columns 128 hf + 8 (lane % 16) of the chunk.  Past the
    // last group the loads read chunk 0 of group G0 (rows clamped into the
    // matrix): issued, never used.
    auto raw_load = [&](int grp, int c, int i, int hf, u32x4_t (&r)[4]) {
        const bool real = grp < G1;
        const int row0 = 16 * (((real ? grp : G0) * TW + i) * 4 + wid) + (lane >> 4);
        const uint16_t *wc = W + 256 * (real ? c : 0) + 128 * hf + 8 * j16;
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = ld_global_nt<u32x4_t>(wc + (int64_t)min(row0 + 4 * q, a.V - 1) * d);
    };
    auto tr_write = [&](const u32x4_t (&r)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) tr[(4 * q + (lane >> 4)) * TS + j16] = r[q];
    };
    // operand of step kk of the half: lane (g, j16) takes row j16, columns 32 kk + 8 g
    auto tr_read = [&](u32x4_t (&m)[4]) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) m[kk] = tr[j16 * TS + 4 * kk + g];
    };
    // the (group, chunk) after (grp, c)
    auto next = [&](int &grp, int &c) {
        if (++c == NC) {
            c = 0;
            ++grp;
        }
    };

    uint64_t best[RG][4];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) best[rg][0] = best[rg][1] = best[rg][2] = best[rg][3] = 0ull;

    // ring: raw[i][1] holds half 1 of the current chunk, raw[i][0] half 0 of
    // the next one; m[0] holds the current chunk's half 0 in operand order
    u32x4_t raw[TW][2][4], m[2][TW][4];
    u32x4_t st[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) st[j] = ld_global<u32x4_t>(plane + tid + 256 * j);
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        raw_load(G0, 0, i, 0, raw[i][0]);
        raw_load(G0, 0, i, 1, raw[i][1]);
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j) hv_lds[tid + 256 * j] = st[j];
    {
        int g1 = G0, c1 = 0;
        next(g1, c1);
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            tr_write(raw[i][0]);
            tr_read(m[0][i]);
            raw_load(g1, c1, i, 0, raw[i][0]);
        }
    }
    __syncthreads();

    int buf = 0;
    for (int grp = G0; grp < G1; ++grp) {
        // one fp32 accumulator per (tile, row group) takes both halves' products
        f32x4_t acc[TW][RG];
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) acc[i][rg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < NC; ++c) {
            // step k's A operands are read during step k - 1 (step 0's right
            // after the barrier).  The scheduling barriers keep loads and LDS
            // traffic where they are written (left alone, the compiler sinks
            // the loads below the MFMAs).
            const u32x4_t *xb = hv_lds + buf * CS + lane;
            u32x4_t x[2][2][RG];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int rg = 0; rg < RG; ++rg) x[0][h][rg] = xb[hv_slot<RG>(0, h, rg, 0)];
            int g1 = grp, c1 = c;
            next(g1, c1);
            int g2 = g1, c2 = c1;
            next(g2, c2);
            // the next chunk's activations (from L2, stored before the barrier)
            const int cs = g1 < G1 ? c1 : 0;
#pragma unroll
            for (int j = 0; j < SPT; ++j) st[j] = ld_global<u32x4_t>(plane + (int64_t)cs * CS + tid + 256 * j);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < kHvChunk; ++k) {
                const int hf = k >> 2, kk = k & 3, ti = kk >> 1;
                if (k + 1 < kHvChunk)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int rg = 0; rg < RG; ++rg) x[(k + 1) & 1][h][rg] = xb[hv_slot<RG>(k + 1, h, rg, 0)];
                // transpose work of this step: half 1 of this chunk during
                // half 0's steps, half 0 of the next chunk during half 1's
                if ((kk & 1) == 0) {
                    tr_write(raw[ti][1 - hf]);
                } else {
                    tr_read(m[1 - hf][ti]);
                    if (hf == 0) raw_load(g1, c1, ti, 1, raw[ti][1]);
                    else raw_load(g2, c2, ti, 0, raw[ti][0]);
                }
#pragma unroll
                for (int i = 0; i < TW; ++i) {
                    const hv_bf16x8_t wv = __builtin_bit_cast(hv_bf16x8_t, m[hf][i][kk]);
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int rg = 0; rg < RG; ++rg)
                            acc[i][rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(hv_bf16x8_t, x[k & 1][h][rg]), wv, acc[i][rg], 0, 0, 0);
                }
                // issue order: LDS traffic interleaved with the first MFMAs,
                // the other MFMAs, then the raw refills
                if (k + 1 < kHvChunk) {
#pragma unroll
                    for (int j2 = 0; j2 < 2 * RG + 4; ++j2) {
                        __builtin_amdgcn_sched_group_barrier(0x300, 1, 0);     // LDS read / write
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 2 * RG * TW - 2 * RG - 4, 0);
                } else {
#pragma unroll
                    for (int j2 = 0; j2 < 4; ++j2) {
                        __builtin_amdgcn_sched_group_barrier(0x300, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 2 * RG * TW - 4, 0);
                }
                if (kk & 1) __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);  // global loads
                __builtin_amdgcn_sched_barrier(0);
            }
            buf ^= 1;
            u32x4_t *dst = hv_lds + buf * CS + tid;
#pragma unroll
            for (int j = 0; j < SPT; ++j) dst[256 * j] = st[j];
            __syncthreads();
        }
        // lane (j16, g) holds vocabulary row 16 tile + j16 for rows 16 rg + 4 g .. + 3
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int v = 16 * ((grp * TW + i) * 4 + wid) + j16;
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const f32x4_t z = acc[i][rg];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = 16 * rg + 4 * g + q;
                    const bool ok = v < a.V && row < a.R;
                    if (LOGITS) {
                        if (ok) a.logits[(int64_t)(a.row0 + row) * a.V + v] = z[q];
                    } else {
                        const uint64_t key = ok ? argmax_key(z[q], (uint32_t)v) : 0ull;
                        best[rg][q] = key > best[rg][q] ? key : best[rg][q];
                    }
                }
            }
        }
    }
    if (LOGITS) return;

    // best over the 16 vocabulary lanes of each lane group, then the 4 waves
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) {
                const uint64_t o = shfl_xor_u64(best[rg][q], m);
                best[rg][q] = o > best[rg][q] ? o : best[rg][q];
            }
    if (j16 == 0)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int q = 0; q < 4; ++q) wbest[wid][16 * rg + 4 * g + q] = best[rg][q];
    __syncthreads();
    if (tid < a.R) {
        uint64_t k = wbest[0][tid];
        for (int w2 = 1; w2 < 4; ++w2) k = wbest[w2][tid] > k ? wbest[w2][tid] : k;
        atomicMax((unsigned long long *)&a.keys[a.row0 + tid], (unsigned long long)k);
    }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------
size_t hv_plane_bytes(int32_t d) { return sizeof(u32x4_t) * (size_t)hv_chunk_slots<kHvMaxRG>() * (d / 256); }

template <int RG, bool LOGITS>
static hipError_t launch_hv_pass(const HvArgs &a, hipStream_t st) {
    mtp_launch(hv_prep_kernel<RG>, dim3(16 * RG), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = 2 * sizeof(u32x4_t) * (size_t)hv_chunk_slots<RG>();
    e = allow_dynamic_lds(hv_head_kernel<RG, kHvTW, LOGITS>, lds);
    if (e != hipSuccess) return e;
    // up to 16 rows the register file and LDS hold two workgroups per CU,
    // beyond that one
    const int per_cu = RG == 1 ? 2 : 1;
    const int n_groups = ((a.V + 15) / 16 + 4 * kHvTW - 1) / (4 * kHvTW);
    int n_wg = std::min(256 * per_cu, n_groups);
    const int gpw = (n_groups + n_wg - 1) / n_wg;
    n_wg = (n_groups + gpw - 1) / gpw;
    mtp_launch((hv_head_kernel<RG, kHvTW, LOGITS>), dim3(n_wg), dim3(256), lds, st, a, gpw);
    return hipGetLastError();
}

hipError_t launch_verify_hidden(const HvArgs &a_in, int32_t rows, hipStream_t st) {
    if (a_in.d % 256 || a_in.d <= 0) return hipErrorInvalidValue;
    for (int32_t row0 = 0; row0 < rows; row0 += 16 * kHvMaxRG) {
        HvArgs a = a_in;
        a.row0 = row0;
        a.R = std::min<int32_t>(16 * kHvMaxRG, rows - row0);
        const int rg = (a.R + 15) / 16;
        hipError_t e;
        if (a.logits)
            e = rg == 1 ? launch_hv_pass<1, true>(a, st)
              : rg == 2 ? launch_hv_pass<2, true>(a, st)
              : rg == 3 ? launch_hv_pass<3, true>(a, st)
                        : launch_hv_pass<4, true>(a, st);
        else
            e = rg == 1 ? launch_hv_pass<1, false>(a, st)
              : rg == 2 ? launch_hv_pass<2, false>(a, st)
              : rg == 3 ? launch_hv_pass<3, false>(a, st)
                        : launch_hv_pass<4, false>(a, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mtp
