// dev_common.h -- device helpers shared by the gfx950 kernels of the MTP path.
//
// Wave64 reductions use DPP row operations (quad_perm, half-mirror, mirror)
// inside a 16-lane row and readlane across the four rows.  All arithmetic is
// fp32; bf16 and Q8_0 operands widen exactly to fp32 before use.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mtp_internal.h"

namespace mtp {

static constexpr int kWave = 64;
static constexpr int kBlock = 256;   // 4 waves per workgroup

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float half_to_f(uint16_t h) {
    _Float16 x;
    __builtin_memcpy(&x, &h, 2);
    return (float)x;
}

// --- DPP reductions ---------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over each 16-lane row; every lane of the row receives the row sum
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    v += dpp<0x140>(v);   // row_mirror
    return v;
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return v;
}
__device__ __forceinline__ float lane_read(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
// full wave sum, uniform result.  Fixed order: rows 0+1, 2+3, then both.
__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum16(v);
    return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
    v = row_max16(v);
    return fmaxf(fmaxf(lane_read(v, 0), lane_read(v, 16)), fmaxf(lane_read(v, 32), lane_read(v, 48)));
}

// --- argmax keys --------------------------------------------------------------
// Monotone map fp32 -> u32 (-0 folded onto +0 so that equal values tie), packed
// with the complemented index: a larger key is a larger value, then a lower id.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
    uint32_t b = __float_as_uint(v + 0.0f);
    uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ int32_t key_index(uint64_t k) { return (int32_t)(0xFFFFFFFFu - (uint32_t)k); }
__device__ __forceinline__ float key_value(uint64_t k) {
    uint32_t o = (uint32_t)(k >> 32);
    uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(b);
}

__device__ __forceinline__ float silu_f(float u) { return u / (1.0f + __expf(-u)); }

// Running (max m, sum s of exp(z - m)) over a stream of logits, and the merge
// of two such pairs.  The merge is symmetric in its operands, so both lanes
// of a butterfly exchange end with the same bits.
__device__ __forceinline__ void conf_add(float &m, float &s, float z) {
    if (z > m) {
        s = s * __expf(m - z) + 1.0f;
        m = z;
    } else {
        s += __expf(z - m);
    }
}
__device__ __forceinline__ void conf_merge(float &m, float &s, float m2, float s2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
    m = mn;
}

// non-temporal 16-byte loads for data streamed once (weights, logits)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4 *p) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ld_nt(const float4 *p) {
    const f32x4_t v = __builtin_nontemporal_load((const f32x4_t *)p);
    return make_float4(v.x, v.y, v.z, v.w);
}

// Loads through an explicitly global pointer: a generic (flat) load would
// also count against the LDS counter, so every LDS wait would drain it.
template <typename T>
__device__ __forceinline__ T ld_global(const void *p) {
    return *(const __attribute__((address_space(1))) T *)p;
}
template <typename T>
__device__ __forceinline__ T ld_global_nt(const void *p) {
    return __builtin_nontemporal_load((const __attribute__((address_space(1))) T *)p);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m), hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// Raise a kernel's dynamic-LDS limit once (gfx950 has 160 KiB of LDS per CU).
template <typename K>
inline hipError_t allow_dynamic_lds(K kernel, size_t bytes) {
    if (bytes <= 32768) return hipSuccess;
    return hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace mtp
