// widen.h -- 16-byte weight/KV vectors widened to fp32 (bf16, fp32, int8).
#pragma once
#include "dev_common.h"

namespace mtp {


// ----------------------------------------------------------------------------
// weight vectors: 16 bytes per lane, widened to fp32
// ----------------------------------------------------------------------------
template <typename WT> struct WTr;
template <> struct WTr<float> { static constexpr int EPV = 4; };
template <> struct WTr<uint16_t> { static constexpr int EPV = 8; };
template <> struct WTr<int8_t> { static constexpr int EPV = 16; };

__device__ __forceinline__ void widen(const uint4 u, float (&w)[4]) {
    w[0] = __uint_as_float(u.x); w[1] = __uint_as_float(u.y); w[2] = __uint_as_float(u.z); w[3] = __uint_as_float(u.w);
}
__device__ __forceinline__ void widen(const uint4 u, float (&w)[8]) {
    w[0] = bf16_lo(u.x); w[1] = bf16_hi(u.x); w[2] = bf16_lo(u.y); w[3] = bf16_hi(u.y);
    w[4] = bf16_lo(u.z); w[5] = bf16_hi(u.z); w[6] = bf16_lo(u.w); w[7] = bf16_hi(u.w);
}
__device__ __forceinline__ void widen(const uint4 u, float (&w)[16]) {
    const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[4 * i + 0] = (float)(int8_t)(ws[i] & 0xFF);
        w[4 * i + 1] = (float)(int8_t)((ws[i] >> 8) & 0xFF);
        w[4 * i + 2] = (float)(int8_t)((ws[i] >> 16) & 0xFF);
        w[4 * i + 3] = (float)(int8_t)(ws[i] >> 24);
    }
}


static constexpr int kLdsFloats = 16384;   // 64 KiB of staged activations
static constexpr int kMaxSeqGroup = 16;

}  // namespace mtp
