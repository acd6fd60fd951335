// ckv_device.h -- device helpers shared by the libckv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ckv.h"

namespace ckv {

constexpr int kWave = 64;

// ---- element types ---------------------------------------------------------------
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits_rne(float f) {
    uint32_t b = __float_as_uint(f);
    b = b + 0x7fffu + ((b >> 16) & 1u);
    return static_cast<uint16_t>(b >> 16);
}

// ---- DPP lane exchanges inside a row of 16 lanes ------------------------------------
// quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141,
// row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// All-reduce sum over aligned groups of L lanes (L in {1,2,4,8,16,32,64}).
template <int L>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (L >= 2) x += dpp<0xB1>(x);
    if constexpr (L >= 4) x += dpp<0x4E>(x);
    if constexpr (L >= 8) x += dpp<0x141>(x);
    if constexpr (L >= 16) x += dpp<0x140>(x);
    if constexpr (L >= 32) x += __shfl_xor(x, 16);
    if constexpr (L >= 64) x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load with the nontemporal hint, for data read once per step (the
// selected K/V rows, the centroid stream): it is not kept in the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const void *p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float4 load_nt_f4(const void *p) {
    const uint4 u = load_nt(p);
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                       __uint_as_float(u.w));
}

// DPP move of a float inside 16-lane rows (lanes without a source keep their own
// value), used by the wave reductions below.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_keep(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL,
                                                      ROW_MASK, 0xF, false));
}

// Reductions of a float over the wavefront, as wave-uniform values: row shifts
// 1, 2, 4, 8, then the row totals carried by row_bcast 15 / 31 into the last row.
template <typename Op>
__device__ __forceinline__ float wave_reduce_f(float x, Op op) {
    x = op(x, dpp_keep<0x111>(x));       // row_shr:1
    x = op(x, dpp_keep<0x112>(x));       // row_shr:2
    x = op(x, dpp_keep<0x114>(x));       // row_shr:4
    x = op(x, dpp_keep<0x118>(x));       // row_shr:8
    x = op(x, dpp_keep<0x142, 0xA>(x));  // row_bcast:15
    x = op(x, dpp_keep<0x143, 0xC>(x));  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
}
__device__ __forceinline__ float wave_max_f(float x) {
    return wave_reduce_f(x, [](float a, float b) { return fmaxf(a, b); });
}
// Sum: here lanes without a DPP source must contribute 0, not their own value.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_zero(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, true));
}
__device__ __forceinline__ float wave_sum_f(float x) {
    x += dpp_zero<0x111>(x);
    x += dpp_zero<0x112>(x);
    x += dpp_zero<0x114>(x);
    x += dpp_zero<0x118>(x);
    x += dpp_zero<0x142, 0xA>(x);
    x += dpp_zero<0x143, 0xC>(x);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
}

// Order-preserving map of an fp32 score to u32 (larger score -> larger key);
// -0 and +0 compare equal as floats, so both map to the key of +0.
__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if ((u << 1) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void set_err(int32_t *err, int32_t bit) {
    if (err) atomicOr(err, bit);
}

}  // namespace ckv
