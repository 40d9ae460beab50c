// attn_kernels.hip -- split-K GQA decode cross-attention of the drafter query
// into the target's read-only KV cache ("Gemma 4 MTP" doc s.1, s.4-5), and the
// log-sum-exp merge of the split partials.
#include "widen.h"

namespace mtp {

// ----------------------------------------------------------------------------
// split-K GQA cross-attention into the target KV ("Gemma 4 MTP" s.4-5)
// ----------------------------------------------------------------------------
// Workgroup = (split, kv head, sequence).  With one sequence the kv head runs
// fastest in the grid, so the workgroups of a split read the kv heads' parts
// of the same cell rows at about the same time (measured: one sequence over
// 8192 cells 8.8 -> 8.4 us); with several the split runs fastest (with the
// kv head fastest, 8 sequences x 131072 cells lost 3% of a round).  The
// first chunk of K/V is loaded
// before anything else (it does not depend on the query), so its HBM latency
// overlaps the prologue: per-head RMSNorm of the G = Hq/Hkv query heads of
// this kv head, then RoPE at pos0 + step (angle pos * inv_freq in fp64, reduced
// mod 2*pi in fp64, sin/cos in fp32), staged in LDS.  Main loop: 16 lane
// groups of 16 lanes; a group scores one cell at a time (each lane holds
// DPL = hd/16 dims; the dot finishes with a 16-lane DPP sum) and keeps an
// online softmax (m, l, acc) in base 2.  Groups merge through shuffles and
// LDS; the workgroup writes one partial (m, l, acc[hd]) per query head.
static constexpr float kLog2e = 1.4426950408889634f;

template <typename KT> struct KVTr;
template <> struct KVTr<float> { static constexpr int EPV = 4; };
template <> struct KVTr<uint16_t> { static constexpr int EPV = 8; };

template <typename KT, int DPL, int G>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
    constexpr int EPV = KVTr<KT>::EPV;
    constexpr int NVL = DPL / EPV;          // 16-byte vectors per lane per row
    constexpr int HD = DPL * 16;
    constexpr int T = 4;                    // cells per group per chunk
    static_assert(DPL % EPV == 0, "lane slice must be whole 16-byte vectors");
    __shared__ float qs[G][HD];
    __shared__ float cs[HD / 2], sn[HD / 2];
    // per lane-group state, merged in LDS; padded (lane stride DPL+1, group
    // stride +16) so the 64 lanes of a store hit 64 different banks
    constexpr int JS = 16 * (DPL + 1), GS = G * JS + 16;
    __shared__ float gm[16][G], gl[16][G], gw[16][G], gL[G], gM[G];
    __shared__ float gacc[16 * GS];

    const bool kv_fast = a.S == 1;
    const int kvh = kv_fast ? blockIdx.x : blockIdx.y, split = kv_fast ? blockIdx.y : blockIdx.x, s = blockIdx.z;
    const SeqParams &sqp = a.seqs[s];
    const SrcParams &sp = sqp.src[a.src];
    if (split >= sp.n_split) return;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int gi = tid >> 4, li = tid & 15;

    const int pbeg = split * sp.split_len;
    const int npos = min(sp.split_len, sp.n_vis - pbeg);
    const KT *kbase = (const KT *)sp.k + (int64_t)kvh * HD + li * DPL;
    const KT *vbase = (const KT *)sp.v + (int64_t)kvh * HD + li * DPL;
    uint4 kv[T][NVL], vv[T][NVL];
    bool ok[T];
    auto load_chunk = [&](int cb) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int pi = cb + t * 16 + gi;
            ok[t] = pi < npos;
            const int64_t off = (int64_t)src_cell(sp, pbeg + pi) * sp.cell_stride;
#pragma unroll
            for (int v = 0; v < NVL; ++v) {
                kv[t][v] = ok[t] ? *(const uint4 *)(kbase + off + v * EPV) : make_uint4(0, 0, 0, 0);
                vv[t][v] = ok[t] ? *(const uint4 *)(vbase + off + v * EPV) : make_uint4(0, 0, 0, 0);
            }
        }
    };
    load_chunk(0);

    // --- prologue: per-head q RMSNorm, RoPE (all its loads issued first) -----
    constexpr int QPL = (HD + 63) / 64;     // query values per lane per head
    constexpr int GW = (G + 3) / 4;         // heads per wave
    float qv[GW][QPL], gq[QPL];
#pragma unroll
    for (int i = 0; i < QPL; ++i) gq[i] = (lane + 64 * i < HD) ? a.g_q[lane + 64 * i] : 0.f;
#pragma unroll
    for (int jj = 0; jj < GW; ++jj) {
        const int j = wid + 4 * jj;
        const float *qh = a.q + ((int64_t)s * a.Hq + (int64_t)kvh * G + min(j, G - 1)) * HD;
#pragma unroll
        for (int i = 0; i < QPL; ++i) qv[jj][i] = (lane + 64 * i < HD) ? qh[lane + 64 * i] : 0.f;
    }
    const double invf = (tid < HD / 2) ? a.inv_freq[tid] : 0.0;
    const int64_t pos = (int64_t)sqp.pos0 + a.step;
    if (tid < HD / 2) {
        const double kTwoPi = 6.283185307179586476925;
        const double ang = (double)pos * invf;
        const double red = ang - kTwoPi * rint(ang * (1.0 / kTwoPi));
        float sv, cv;
        sincosf((float)red, &sv, &cv);
        cs[tid] = cv;
        sn[tid] = sv;
    }
#pragma unroll
    for (int jj = 0; jj < GW; ++jj) {
        const int j = wid + 4 * jj;
        if (j < G) {                        // wave-uniform
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < QPL; ++i) ss = fmaf(qv[jj][i], qv[jj][i], ss);
            ss = wave_sum(ss);
            const float r = 1.0f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
            for (int i = 0; i < QPL; ++i)
                if (lane + 64 * i < HD) qs[j][lane + 64 * i] = qv[jj][i] * r * gq[i];
        }
    }
    __syncthreads();
    for (int i = tid; i < G * (HD / 2); i += kBlock) {
        const int j = i / (HD / 2), c = i - j * (HD / 2);
        const float x0 = qs[j][c], x1 = qs[j][c + HD / 2];
        const float y0 = x0 * cs[c] - x1 * sn[c];
        const float y1 = x0 * sn[c] + x1 * cs[c];
        qs[j][c] = y0;            // each (j, c) pair is owned by one thread
        qs[j][c + HD / 2] = y1;
    }
    __syncthreads();

    float qr[G][DPL];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < DPL; ++e) qr[j][e] = qs[j][li * DPL + e] * (a.scale * kLog2e);

    float m[G], l[G], acc[G][DPL];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[j][e] = 0.f;
    }

    for (int cb = 0; cb < npos; cb += 16 * T) {
        if (cb > 0) load_chunk(cb);
        float sc[T][G];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float part[G];
#pragma unroll
            for (int j = 0; j < G; ++j) part[j] = 0.f;
#pragma unroll
            for (int v = 0; v < NVL; ++v) {
                float kf[EPV];
                widen(kv[t][v], kf);
#pragma unroll
                for (int j = 0; j < G; ++j)
#pragma unroll
                    for (int e = 0; e < EPV; ++e) part[j] = fmaf(qr[j][v * EPV + e], kf[e], part[j]);
            }
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float r = row_sum16(part[j]);   // all lanes take part in the DPP sum
                sc[t][j] = ok[t] ? r : -INFINITY;
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float mx = sc[0][j];
#pragma unroll
            for (int t = 1; t < T; ++t) mx = fmaxf(mx, sc[t][j]);
            const float mn = fmaxf(m[j], mx);
            if (mn == -INFINITY) continue;          // nothing visible yet in this group
            const float corr = exp2f(m[j] - mn);    // m = -inf gives 0
            m[j] = mn;
            l[j] *= corr;
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[j][e] *= corr;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const float p = exp2f(sc[t][j] - mn);
                l[j] += p;
#pragma unroll
                for (int v = 0; v < NVL; ++v) {
                    float vf[EPV];
                    widen(vv[t][v], vf);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) acc[j][v * EPV + e] = fmaf(p, vf[e], acc[j][v * EPV + e]);
                }
            }
        }
    }

    // merge the 16 lane groups through LDS: each group stores (m, l, acc),
    // 64 threads turn the m's into per-group weights 2^(m_g - M) and the
    // normaliser, then every thread writes merged (head, dim) outputs
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) gacc[gi * GS + j * JS + li * (DPL + 1) + e] = acc[j][e];
        if (li == 0) {
            gm[gi][j] = m[j];
            gl[gi][j] = l[j];
        }
    }
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
        for (int g = 0; g < 16; ++g) M = fmaxf(M, gm[g][tid]);
        float L = 0.f;
        for (int g = 0; g < 16; ++g) {
            const float w = (gm[g][tid] == -INFINITY) ? 0.f : exp2f(gm[g][tid] - M);
            gw[g][tid] = w;
            L += gl[g][tid] * w;
        }
        gM[tid] = M;
        gL[tid] = L;
    }
    __syncthreads();
    for (int i = tid; i < G * HD; i += kBlock) {
        const int j = i / HD, c = i - j * HD;
        float av = 0.f;
        const int cl = (c / DPL) * (DPL + 1) + (c % DPL);
#pragma unroll
        for (int g = 0; g < 16; ++g) av = fmaf(gw[g][j], gacc[g * GS + j * JS + cl], av);
        float *pp = a.part + (((int64_t)s * a.Hq + (int64_t)kvh * G + j) * MTP_MAX_SPLITS + split) * (HD + kPartHead);
        pp[kPartHead + c] = av;
        if (c == 0) {
            pp[0] = gM[j];
            pp[1] = gL[j];
        }
    }
}

// ----------------------------------------------------------------------------
// bf16 KV: scores on the matrix cores, softmax and P.V on the vector ALUs
// ----------------------------------------------------------------------------
// Workgroup = (split, kv head group, sequence), serving nh kv heads of the
// group (nh = the sequence's heads_wg: 1, or 2 at long context).  Its four
// waves are dealt out head-fastest: wave w serves kv head w % nh of the
// group and the split's 16-cell tiles w / nh, w / nh + 4 / nh, ...  With
// nh = 2 the waves of a workgroup read both heads' halves of the same cell
// rows together, one contiguous run of 2 * hd * 2 bytes per cell.  Per tile
// the G query heads of a wave's kv head meet the 16 K rows in
// v_mfma_f32_16x16x32_bf16 (A = K, cells as rows, loaded in operand order,
// or through LDS when streaming; B = the scaled query as bf16 hi and lo
// halves, 2G of the 16 columns), so a score costs no vector work.  Lane j < G of each 16-lane row then owns
// head j for 4 cells: it adds the lo column, keeps the online softmax
// (m, l) in base 2; every lane then accumulates P.V for its HD/64 dims of
// all G heads from the tile's V rows, which it loads as one coalesced row
// per cell.  The next tile's K and V are loaded before the current one is
// used.  Positions past the split end are clamped to its last position
// (never an unseen cell) and masked to -inf.  NHM is the largest nh the
// instantiation serves; a sequence with nh = 1 takes the same operations in
// the same order in either instantiation.
// STREAM: the KV a draft step reads is far larger than the last-level
// cache, so nothing read now is still cached when the next step reads it:
// the tile loads are non-temporal (measured with loads alone over 8 x 131072
// cells: 351.6 -> 310.0 us).  Otherwise plain loads let the next step's
// reads of the same cells hit in cache.
typedef __bf16 abf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t au32x2_t __attribute__((ext_vector_type(2)));

template <int DPL> struct VRow;
template <> struct VRow<4> { typedef au32x2_t T; };   // 4 bf16 per lane per cell
template <> struct VRow<2> { typedef uint32_t T; };   // 2 bf16

// KV addresses come from the per-call parameter block, so the compiler
// cannot see that they are global memory: the tile loads use ld_global.
template <int HD, int G>
struct AttnTile {
    static constexpr int KS = HD / 32, DPL = HD / 64;
    u32x4_t k[KS];
    typename VRow<DPL>::T v[16];
};

template <bool STREAM, typename T>
__device__ __forceinline__ T kv_load(const void *p) {
    if constexpr (STREAM) return ld_global_nt<T>(p);
    else return ld_global<T>(p);
}

__device__ __forceinline__ void bf16_pair(uint32_t w, float &lo, float &hi) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xFFFF0000u);
}

// K tile staging in LDS: each wave's 16 rows of hd bf16, rows padded by 16
// bytes so that a wave's operand-order reads (16 rows x 16 bytes per lane
// group) fall on 16 different 4-bank groups.
template <int HD>
struct KStage {
    static constexpr int ROWB = 2 * HD + 16;
    alignas(16) char w[4][16 * ROWB];
};

// LDS of one attention workgroup, sized for NHM kv heads.  The K staging is
// used only by the main loop and the wave partials only after it.
template <int HD, int G, int NHM>
struct AttnSmem {
    static constexpr int KS = HD / 32;
    alignas(16) float qs[G * NHM][HD];
    alignas(16) float cs[HD / 2];
    alignas(16) float sn[HD / 2];
    float wm[4][G], wl[4][G];
    union {
        KStage<HD> kst;
        float wacc[4][G][HD];
    };
    abf16x8_t qbs[NHM][KS][64];
};

// One workgroup's split for NH kv heads (NH <= NHM, compile time).
template <int HD, int G, int NH, int NHM, bool STREAM>
__device__ __forceinline__ void attn_mm_body(const AttnArgs &a, AttnSmem<HD, G, NHM> &sm, int kvg, int split, int s) {
    constexpr int KS = HD / 32, DPL = HD / 64;
    const SeqParams &sqp = a.seqs[s];
    const SrcParams &sp = sqp.src[a.src];
    constexpr int nh = NH, wph = 4 / NH, nqh = G * NH;     // kv heads, waves per kv head, query heads
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hw = wid % NH, wt = wid / NH;                     // head in the group, first tile
    const int kvh = kvg * nh + hw;
    const int j16 = lane & 15, g = lane >> 4;
    const int pbeg = split * sp.split_len;
    const int npos = min(sp.split_len, sp.n_vis - pbeg);
    const int ntile = (npos + 15) / 16;
    const int nt = ntile > wt ? (ntile - wt + wph - 1) / wph : 0;   // this wave's tiles

    const uint16_t *kb = (const uint16_t *)sp.k + (int64_t)kvh * HD;
    const uint16_t *vb = (const uint16_t *)sp.v + (int64_t)kvh * HD;
    auto cell_of = [&](int pi) { return src_cell(sp, pbeg + min(pi, npos - 1)); };
    // STREAM: K rows are loaded whole, instruction q taking rows RPI q ..
    // RPI q + RPI - 1 of the tile, lane l the 16-byte chunk l % CPR of row
    // RPI q + l / CPR, and go into operand order through LDS (measured with
    // loads alone, 8 sequences x 131072 cells: 322 us with the 16 rows x 64
    // bytes per instruction that the operand order needs, 315 us this way
    // with the LDS transpose; in the kernel, 16 sequences of 4096-32768
    // cells 39.8 -> 38.0 us).  Otherwise each lane loads its operand (row j16,
    // 16 bytes per step) directly: with one or two tiles per wave the LDS
    // round trip would sit on the critical path (one sequence over 8192
    // cells 7.8 -> 8.3 us with it).
    constexpr int CPR = HD / 8, RPI = 64 / CPR;
    const int krow = STREAM ? lane / CPR : j16, kchunk = lane % CPR;
    auto load = [&](int i, AttnTile<HD, G> &t) {
        const int p0 = i < nt ? 16 * (wt + wph * i) : 16 * wt;
        if constexpr (STREAM) {
#pragma unroll
            for (int q = 0; q < KS; ++q)
                t.k[q] = kv_load<STREAM, u32x4_t>(kb + (int64_t)cell_of(p0 + RPI * q + krow) * sp.cell_stride + 8 * kchunk);
        } else {
            const uint16_t *kp = kb + (int64_t)cell_of(p0 + krow) * sp.cell_stride + 8 * g;
#pragma unroll
            for (int u = 0; u < KS; ++u) t.k[u] = kv_load<STREAM, u32x4_t>(kp + 32 * u);
        }
#pragma unroll
        for (int c = 0; c < 16; ++c)
            t.v[c] = kv_load<STREAM, typename VRow<DPL>::T>(vb + (int64_t)cell_of(p0 + c) * sp.cell_stride + DPL * lane);
    };
    char *kst = sm.kst.w[wid];
    // the first two tiles do not depend on the query: request them first
    AttnTile<HD, G> buf[2];
    if (nt > 0) load(0, buf[0]);
    if (nt > 1) load(1, buf[1]);

    // --- prologue: per-head q RMSNorm; RoPE follows in the operand build ---
    constexpr int QPL = (HD + 63) / 64;
    constexpr int GW = (G * NH + 3) / 4;
    float qv[GW][QPL], gq[QPL];
#pragma unroll
    for (int i = 0; i < QPL; ++i) gq[i] = (lane + 64 * i < HD) ? a.g_q[lane + 64 * i] : 0.f;
#pragma unroll
    for (int jj = 0; jj < GW; ++jj) {
        const int j = wid + 4 * jj;
        const float *qh = a.q + ((int64_t)s * a.Hq + (int64_t)kvg * nqh + min(j, nqh - 1)) * HD;
#pragma unroll
        for (int i = 0; i < QPL; ++i) qv[jj][i] = (lane + 64 * i < HD) ? qh[lane + 64 * i] : 0.f;
    }
    const double invf = (tid < HD / 2) ? a.inv_freq[tid] : 0.0;
    const int64_t pos = (int64_t)sqp.pos0 + a.step;
    if (tid < HD / 2) {
        const double kTwoPi = 6.283185307179586476925;
        const double ang = (double)pos * invf;
        const double red = ang - kTwoPi * rint(ang * (1.0 / kTwoPi));
        float sv, cv;
        sincosf((float)red, &sv, &cv);
        sm.cs[tid] = cv;
        sm.sn[tid] = sv;
    }
#pragma unroll
    for (int jj = 0; jj < GW; ++jj) {
        const int j = wid + 4 * jj;
        if (j < nqh) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < QPL; ++i) ss = fmaf(qv[jj][i], qv[jj][i], ss);
            ss = wave_sum(ss);
            const float r = 1.0f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
            for (int i = 0; i < QPL; ++i)
                if (lane + 64 * i < HD) sm.qs[j][lane + 64 * i] = qv[jj][i] * r * gq[i];
        }
    }
    __syncthreads();

    // B operand of each kv head of the workgroup: column h < G holds the hi
    // half of its query head h after RoPE, column 8 + h its lo half (scaled
    // by scale * log2(e)); the other columns are zero.  Each wave builds
    // nh * KS / 4 of the nh * KS steps and puts them in LDS, where every wave
    // reads its head's operand back.  A lane's 8 values of a step are 8
    // consecutive dims inside one rotation half (which half depends on the
    // step only); it reads them and their partners from a clamped head row
    // with 16-byte LDS reads and zeroes dead columns afterwards: a per-lane
    // guard on the reads would turn into a branch and a wait around each of
    // them.
    {
        const int h = j16 & 7;
        const bool live = h < G;
        const float sc = a.scale * kLog2e;
#pragma unroll
        for (int uu = 0; uu < NH * KS / 4; ++uu) {
            const int v = wid * (NH * KS / 4) + uu;
            const int hb = v / KS, u = v % KS;
            const float *qrow = sm.qs[hb * G + min(h, G - 1)];
            const bool first = 32 * u < HD / 2;             // rotation half, uniform per step
            const int c0 = (32 * u + 8 * g) % (HD / 2);
            float x0[8], x1[8], cv[8], sv[8];
            auto rd8 = [](const float *src, float (&d)[8]) {
                const float4 lo = *(const float4 *)src, hi = *(const float4 *)(src + 4);
                d[0] = lo.x; d[1] = lo.y; d[2] = lo.z; d[3] = lo.w;
                d[4] = hi.x; d[5] = hi.y; d[6] = hi.z; d[7] = hi.w;
            };
            rd8(qrow + c0, x0);
            rd8(qrow + c0 + HD / 2, x1);
            rd8(sm.cs + c0, cv);
            rd8(sm.sn + c0, sv);
            abf16x8_t qv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float r0 = x0[e] * cv[e] - x1[e] * sv[e], r1 = x0[e] * sv[e] + x1[e] * cv[e];
                const float x = live ? (first ? r0 : r1) * sc : 0.f;
                const __bf16 hbf = (__bf16)x;
                qv[e] = j16 < 8 ? hbf : (__bf16)(x - (float)hbf);
            }
            sm.qbs[hb][u][lane] = qv;
        }
    }
    __syncthreads();
    abf16x8_t qb[KS];
#pragma unroll
    for (int u = 0; u < KS; ++u) qb[u] = sm.qbs[hw][u][lane];

    float m = -INFINITY, l = 0.f;           // head j16 (lanes j16 < G)
    float acc[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;

    // (x, y) of lanes l and l ^ 32 (and l ^ 16) in the same order in both lanes
    auto xmax = [](float v) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
        r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    auto xsum = [](float v) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    };
    auto tile = [&](int i, const AttnTile<HD, G> &t) {
        // STREAM: K through the wave's LDS rows into operand order (step u of
        // lane (j16, g) is row j16, dims 32 u + 8 g .. + 7).  A wave's LDS
        // operations complete in order, so the next tile's stores cannot
        // overtake these reads.
        constexpr int ROWB = KStage<HD>::ROWB;
        u32x4_t ko[KS];
        if constexpr (STREAM) {
#pragma unroll
            for (int q = 0; q < KS; ++q) *(u32x4_t *)(kst + (RPI * q + krow) * ROWB + 16 * kchunk) = t.k[q];
#pragma unroll
            for (int u = 0; u < KS; ++u) ko[u] = *(const u32x4_t *)(kst + j16 * ROWB + 64 * u + 16 * g);
        } else {
#pragma unroll
            for (int u = 0; u < KS; ++u) ko[u] = t.k[u];
        }
        // two independent MFMA chains over the even / odd head-dim steps
        f32x4_t d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < KS; u += 2) {
            d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(abf16x8_t, ko[u]), qb[u], d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(abf16x8_t, ko[u + 1]), qb[u + 1], d1, 0, 0, 0);
        }
        const f32x4_t d = d0 + d1;
        // lane (j16 < G, g): head j16, cells 4g .. 4g+3; its lo column sits
        // 8 lanes away in the same row (a rotate by 8 either way)
        const int pt = 16 * (wt + wph * i) + 4 * g;
        float sc[4], mt = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            sc[q] = (pt + q < npos) ? d[q] + dpp<0x128>(d[q]) : -INFINITY;
            mt = fmaxf(mt, sc[q]);
        }
        mt = xmax(mt);
        const float mn = fmaxf(m, mt);
        const float corr = mn == -INFINITY ? 1.f : exp2f(m - mn);
        float p[4], ps = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            p[q] = mn == -INFINITY ? 0.f : exp2f(sc[q] - mn);
            ps += p[q];
        }
        l = l * corr + xsum(ps);
        m = mn;
        // P.V: p and the rescale are read out of the owning lanes as scalars
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float cr = lane_read(corr, h);
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] *= cr;
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float vf[DPL];
            if constexpr (DPL == 4) {
                bf16_pair(t.v[c][0], vf[0], vf[1]);
                bf16_pair(t.v[c][1], vf[2], vf[3]);
            } else {
                bf16_pair(t.v[c], vf[0], vf[1]);
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float ph = lane_read(p[c & 3], h + 16 * (c >> 2));
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
            }
        }
    };
    // Two tiles in flight.  The steady-state body issues its loads without
    // conditions; the last one to three tiles are peeled, so no load is
    // issued past the wave's last tile.
    int i = 0;
    // (STREAM: the scheduling fences keep the next tile's loads behind the
    // current tile, whose staged K then reuses the registers its raw K held)
    for (; i + 3 < nt; i += 2) {
        tile(i, buf[0]);
        if constexpr (STREAM) __builtin_amdgcn_sched_barrier(0);
        load(i + 2, buf[0]);
        tile(i + 1, buf[1]);
        if constexpr (STREAM) __builtin_amdgcn_sched_barrier(0);
        load(i + 3, buf[1]);
    }
    if (i < nt) tile(i, buf[0]);
    if (i + 2 < nt) load(i + 2, buf[0]);
    if (i + 1 < nt) tile(i + 1, buf[1]);
    if (i + 2 < nt) tile(i + 2, buf[0]);

    // --- merge the states of each kv head's waves -> one partial per query head
    __syncthreads();                        // the wave partials reuse the K staging
    if (j16 < G && g == 0) {
        sm.wm[wid][j16] = m;
        sm.wl[wid][j16] = l;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < DPL; ++e) sm.wacc[wid][h][DPL * lane + e] = acc[h][e];
    __syncthreads();
    for (int i = tid; i < nqh * HD; i += kBlock) {
        const int j = i / HD, c = i - j * HD;
        const int hh = j / G, jh = j - hh * G;          // kv head in the workgroup, query head of it
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < wph; ++k) M = fmaxf(M, sm.wm[hh + nh * k][jh]);
        float L = 0.f, av = 0.f;
#pragma unroll
        for (int k = 0; k < wph; ++k) {
            const int w = hh + nh * k;
            const float wt = sm.wm[w][jh] == -INFINITY ? 0.f : exp2f(sm.wm[w][jh] - M);
            L = fmaf(sm.wl[w][jh], wt, L);
            av = fmaf(sm.wacc[w][jh][c], wt, av);
        }
        float *pp = a.part + (((int64_t)s * a.Hq + (int64_t)kvg * nqh + j) * MTP_MAX_SPLITS + split) * (HD + kPartHead);
        pp[kPartHead + c] = av;
        if (c == 0) {
            pp[0] = M;
            pp[1] = L;
        }
    }
}

template <int HD, int G, int NHM, bool STREAM>
__global__ __launch_bounds__(256) void attn_mm_kernel(AttnArgs a) {
    static_assert(2 * G <= 16, "hi and lo query columns must fit one MFMA tile");
    static_assert(NHM == 1 || NHM == 2, "one or two kv heads per workgroup");
    static_assert((HD / 32) % 4 == 0, "every wave builds the same number of operand steps");
    __shared__ AttnSmem<HD, G, NHM> sm;
    // Grid: (kv head, split) for one sequence, so the kv heads of a split run
    // together; (split, kv head, sequence) for several; and (split, sequence,
    // kv head) when some sequence's workgroups serve two kv heads.  There the
    // second kv head's workgroups of such a sequence have nothing to do: they
    // come last instead of between the working ones, and the grid leaves
    // them out when every sequence of the launch serves two.
    int kvg, split, s;
    if (NHM == 2) {
        split = blockIdx.x; s = blockIdx.y; kvg = blockIdx.z;
    } else if (a.S == 1) {
        kvg = blockIdx.x; split = blockIdx.y; s = 0;
    } else {
        split = blockIdx.x; kvg = blockIdx.y; s = blockIdx.z;
    }
    const SrcParams &sp = a.seqs[s].src[a.src];
    if (split >= sp.n_split) return;
    if (NHM == 2 && sp.heads_wg == 2) {             // uniform per workgroup
        if (2 * kvg < a.Hkv) attn_mm_body<HD, G, (NHM == 2 ? 2 : 1), NHM, STREAM>(a, sm, kvg, split, s);
    } else {
        attn_mm_body<HD, G, 1, NHM, STREAM>(a, sm, kvg, split, s);
    }
}

hipError_t launch_attn(int kv_dtype, const AttnArgs &a, int max_split, hipStream_t st) {
    const dim3 grid = a.S == 1 ? dim3(a.Hkv, max_split, 1) : dim3(max_split, a.Hkv, a.S);
    const dim3 grid_wide(max_split, a.S, a.wide == 2 ? a.Hkv / 2 : a.Hkv);
    const int G = a.Hq / a.Hkv;
#define MTP_ATTN_CASE(KT, HDV, GV)                                                                  \
    if (a.hd == HDV && G == GV) {                                                                   \
        mtp_launch((attn_kernel<KT, HDV / 16, GV>), grid, dim3(kBlock), 0, st, a);          \
        return hipGetLastError();                                                                   \
    }
#define MTP_ATTN_MM_NH(HDV, GV, NHV)                                                                \
    if (a.stream_kv)                                                                                \
        mtp_launch((attn_mm_kernel<HDV, GV, NHV, true>), NHV == 2 ? grid_wide : grid, dim3(kBlock), 0, st, a); \
    else                                                                                            \
        mtp_launch((attn_mm_kernel<HDV, GV, NHV, false>), NHV == 2 ? grid_wide : grid, dim3(kBlock), 0, st, a); \
    return hipGetLastError();
#define MTP_ATTN_MM(HDV, GV)                                                                        \
    if (a.hd == HDV && G == GV) {                                                                   \
        if (a.wide) { MTP_ATTN_MM_NH(HDV, GV, 2) }                                                  \
        MTP_ATTN_MM_NH(HDV, GV, 1)                                                                  \
    }
#define MTP_ATTN_MM1(HDV, GV)                                                                       \
    if (a.hd == HDV && G == GV) {                                                                   \
        MTP_ATTN_MM_NH(HDV, GV, 1)                                                                  \
    }
    if (kv_dtype == MTP_BF16) {
        MTP_ATTN_MM(256, 4)
        MTP_ATTN_MM(256, 2)
        MTP_ATTN_MM(256, 1)
        MTP_ATTN_MM1(256, 8)      // two heads of 8 query heads each would not fit two waves per SIMD
        MTP_ATTN_MM(128, 8)
        MTP_ATTN_MM(128, 4)
        MTP_ATTN_MM(128, 2)
        MTP_ATTN_MM(128, 1)
    }
#undef MTP_ATTN_MM_NH
#undef MTP_ATTN_MM1
#undef MTP_ATTN_MM
    if (kv_dtype == MTP_BF16) {
        MTP_ATTN_CASE(uint16_t, 256, 4)
        MTP_ATTN_CASE(uint16_t, 256, 2)
        MTP_ATTN_CASE(uint16_t, 256, 1)
        MTP_ATTN_CASE(uint16_t, 128, 8)
        MTP_ATTN_CASE(uint16_t, 128, 4)
        MTP_ATTN_CASE(uint16_t, 128, 2)
        MTP_ATTN_CASE(uint16_t, 128, 1)
    } else if (kv_dtype == MTP_F32) {
        MTP_ATTN_CASE(float, 64, 4)
        MTP_ATTN_CASE(float, 64, 8)
        MTP_ATTN_CASE(float, 64, 2)
        MTP_ATTN_CASE(float, 64, 1)
        MTP_ATTN_CASE(float, 128, 4)
        MTP_ATTN_CASE(float, 256, 4)
    }
#undef MTP_ATTN_CASE
    return hipErrorInvalidValue;
}

// Log-sum-exp merge of the split partials of one query head, online form:
// (m, l, acc) <- (M, l*2^(m-M) + l_j*2^(m_j-M), acc*2^(m-M) + acc_j*2^(m_j-M)),
// M = max(m, m_j).  Workgroup = (chunk of 16 * DPT dims, query head,
// sequence): 16 thread slices take every 16th split (at most 8 each, all
// loads in flight at once); a lane holds DPT consecutive dims and reads
// (m, l) as one 8-byte load.  Then the 16 lanes of slice 0 combine the slices
// through LDS in a fixed order.  Every dim sees the same operations in the
// same order whatever DPT is.  DPT = 4 (one wave load = 4 partial rows x 256
// contiguous bytes) serves several sequences; one sequence keeps DPT = 1,
// whose 4x more workgroups finish its few partials sooner.
template <int DPT>
__device__ __forceinline__ void lse_combine(float &m, float &l, float (&acc)[DPT], float mj, float lj,
                                            const float (&aj)[DPT]) {
    const float mn = fmaxf(m, mj);
    if (mn == -INFINITY) return;
    const float c0 = exp2f(m - mn), c1 = exp2f(mj - mn);
    l = l * c0 + lj * c1;
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = acc[e] * c0 + aj[e] * c1;
    m = mn;
}

template <int DPT>
__device__ __forceinline__ void ld_dims(const float *p, float (&v)[DPT]) {
    if constexpr (DPT == 4) {
        const float4 t = *(const float4 *)p;
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
        v[0] = *p;
    }
}

template <int DPT>
__device__ __forceinline__ void st_dims(float *p, const float (&v)[DPT]) {
    if constexpr (DPT == 4) *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
    else *p = v[0];
}

template <int DPT>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
    constexpr int DC = 16 * DPT, SL = 16, U = MTP_MAX_SPLITS / SL;
    __shared__ float sm[SL][16], sl[SL][16];
    __shared__ float sa[SL][16][DPT];
    // Workgroup w takes (sequence, head) w % n_sh and dim chunk w / n_sh:
    // consecutive workgroups go to different XCDs, so all chunks of one
    // head then share an XCD and its L2 fetches the head's partial rows
    // once (the chunk-fastest order fetched their header lines once per XCD).
    const int n_sh = a.S * a.Hq;
    const int sh = blockIdx.x % n_sh, chunk = blockIdx.x / n_sh;
    const int s = sh / a.Hq, h = sh - s * a.Hq;
    const int tid = threadIdx.x, dl = tid % 16, slice = tid / 16;
    const int hd = a.hd;
    const int dim = chunk * DC + DPT * dl;      // hd is a multiple of 64
    const int ns = a.seqs[s].src[a.src].n_split;
    const int64_t row = hd + kPartHead;
    const float *base = a.part + ((int64_t)s * a.Hq + h) * MTP_MAX_SPLITS * row;
    float2 ml[U];
    float aj[U][DPT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float *pj = base + (int64_t)min(slice + SL * u, ns - 1) * row;
        ml[u] = *(const float2 *)pj;
        ld_dims<DPT>(pj + kPartHead + dim, aj[u]);
    }
    float m = -INFINITY, l = 0.f, acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) lse_combine<DPT>(m, l, acc, slice + SL * u < ns ? ml[u].x : -INFINITY, ml[u].y, aj[u]);
    sm[slice][dl] = m;
    sl[slice][dl] = l;
#pragma unroll
    for (int e = 0; e < DPT; ++e) sa[slice][dl][e] = acc[e];
    __syncthreads();
    if (slice == 0) {
        for (int k = 1; k < SL; ++k) {
            float ak[DPT];
#pragma unroll
            for (int e = 0; e < DPT; ++e) ak[e] = sa[k][dl][e];
            lse_combine<DPT>(m, l, acc, sm[k][dl], sl[k][dl], ak);
        }
        float ov[DPT];
#pragma unroll
        for (int e = 0; e < DPT; ++e) ov[e] = acc[e] / l;
        st_dims<DPT>(a.o + ((int64_t)s * a.Hq + h) * hd + dim, ov);
        if (a.o_op) st_dims<DPT>(a.o_op + op_index(h * hd + dim, s), ov);   // DPT consecutive k: one run
    }
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t st) {
    if (a.hd % 64) return hipErrorInvalidValue;
    if (a.S == 1) {
        mtp_launch(merge_kernel<1>, dim3((a.hd / 16) * a.Hq * a.S), dim3(kBlock), 0, st, a);
    } else {
        mtp_launch(merge_kernel<4>, dim3((a.hd / 64) * a.Hq * a.S), dim3(kBlock), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace mtp
