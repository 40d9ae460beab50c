// attn_kernels.hip -- split-K GQA decode cross-attention of the drafter query
// into the target's read-only KV cache ("Gemma 4 MTP" doc s.1, s.4-5), and the
// log-sum-exp merge of the split partials.
#include "widen.h"

namespace mtp {

// ----------------------------------------------------------------------------
// split-K GQA cross-attention into the target KV ("Gemma 4 MTP" s.4-5)
// ----------------------------------------------------------------------------
// Workgroup = (split, kv head, sequence).  The first chunk of K/V is loaded
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

    const int split = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
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
            int cell = sp.c0 + pbeg + pi;
            if (cell >= sp.n_cells) cell -= sp.n_cells;
            const int64_t off = (int64_t)cell * sp.cell_stride;
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
        float *pp = a.part + (((int64_t)s * a.Hq + (int64_t)kvh * G + j) * MTP_MAX_SPLITS + split) * (HD + 2);
        pp[2 + c] = av;
        if (c == 0) {
            pp[0] = gM[j];
            pp[1] = gL[j];
        }
    }
}

hipError_t launch_attn(int kv_dtype, const AttnArgs &a, int max_split, hipStream_t st) {
    dim3 grid(max_split, a.Hkv, a.S);
    const int G = a.Hq / a.Hkv;
#define MTP_ATTN_CASE(KT, HDV, GV)                                                                  \
    if (a.hd == HDV && G == GV) {                                                                   \
        hipLaunchKernelGGL((attn_kernel<KT, HDV / 16, GV>), grid, dim3(kBlock), 0, st, a);          \
        return hipGetLastError();                                                                   \
    }
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
// M = max(m, m_j).  Workgroup = (16-dim chunk, query head, sequence): 16
// thread slices take every 16th split (at most 8 each, all loads in flight at
// once), then 16 threads combine the slices through LDS in a fixed order.
__device__ __forceinline__ void lse_combine(float &m, float &l, float &acc, float mj, float lj, float aj) {
    const float mn = fmaxf(m, mj);
    if (mn == -INFINITY) return;
    const float c0 = exp2f(m - mn), c1 = exp2f(mj - mn);
    l = l * c0 + lj * c1;
    acc = acc * c0 + aj * c1;
    m = mn;
}

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
    constexpr int DC = 16, SL = 16, U = MTP_MAX_SPLITS / SL;
    __shared__ float sm[SL][DC], sl[SL][DC], sa[SL][DC];
    const int s = blockIdx.z, h = blockIdx.y, chunk = blockIdx.x;
    const int tid = threadIdx.x, dl = tid % DC, slice = tid / DC;
    const int hd = a.hd;
    const int dim = min(chunk * DC + dl, hd - 1);
    const int ns = a.seqs[s].src[a.src].n_split;
    const float *base = a.part + ((int64_t)s * a.Hq + h) * MTP_MAX_SPLITS * (hd + 2);
    float mj[U], lj[U], aj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = slice + SL * u;
        const float *pj = base + (int64_t)min(j, ns - 1) * (hd + 2);
        mj[u] = (j < ns) ? pj[0] : -INFINITY;
        lj[u] = pj[1];
        aj[u] = pj[2 + dim];
    }
    float m = -INFINITY, l = 0.f, acc = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) lse_combine(m, l, acc, mj[u], lj[u], aj[u]);
    sm[slice][dl] = m;
    sl[slice][dl] = l;
    sa[slice][dl] = acc;
    __syncthreads();
    if (slice == 0 && chunk * DC + dl < hd) {
        for (int k = 1; k < SL; ++k) lse_combine(m, l, acc, sm[k][dl], sl[k][dl], sa[k][dl]);
        a.o[((int64_t)s * a.Hq + h) * hd + chunk * DC + dl] = acc / l;
    }
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t st) {
    dim3 grid((a.hd + 15) / 16, a.Hq, a.S);
    hipLaunchKernelGGL(merge_kernel, grid, dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

}  // namespace mtp
