// gdn_device.h -- device-side helpers shared by the gfx950 kernels.
//
// Wave64 cross-lane reductions on DPP, bf16 <-> fp32 conversion, and vector
// loads of 4 consecutive q/k/v elements in either input dtype.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is the top half of an fp32 bit pattern, so widening is
// a shift; narrowing rounds to nearest, ties to even (inputs are finite).

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two fp32 -> one dword of two bf16 (a in the low half), rounded to nearest
// even by the conversion instruction (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// Loads of 4 consecutive elements (8 bytes of bf16 or 16 bytes of fp32) as
// fp32.  The pointer must be aligned to the access size.

template <typename T> struct In;

template <> struct In<uint16_t> {  // bf16 stored as raw 16-bit patterns
    __device__ __forceinline__ static float4 load4(const uint16_t *p) {
        const uint2 w = *reinterpret_cast<const uint2 *>(p);
        return make_float4(bf16_lo_to_f32(w.x), bf16_hi_to_f32(w.x), bf16_lo_to_f32(w.y), bf16_hi_to_f32(w.y));
    }
    __device__ __forceinline__ static float load1(const uint16_t *p) { return __uint_as_float(uint32_t(*p) << 16); }
};

template <> struct In<float> {
    __device__ __forceinline__ static float4 load4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
    __device__ __forceinline__ static float load1(const float *p) { return *p; }
};

// ---------------------------------------------------------------------------
// Cross-lane sums over aligned groups of N lanes (N = 2, 4, 8, 16) with DPP.
// quad_perm [1,0,3,2] and [2,3,0,1] sum within quads; row_half_mirror pairs
// lane i with 7-i inside each 8-lane half row; row_mirror pairs i with 15-i
// inside each 16-lane row.  Every lane of a group ends with the group's sum.

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
    if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
    if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
    return x;
}

// ---------------------------------------------------------------------------
// 16-byte state accesses, optionally non-temporal (streamed past the caches:
// for data touched once per kernel and not again until far more bytes have
// gone by than the last-level cache holds).

typedef float f32x4v_t __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ float4 load_state4(const float *p) {
    if constexpr (NT) {
        const f32x4v_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t *>(p));
        return make_float4(x[0], x[1], x[2], x[3]);
    } else {
        return *reinterpret_cast<const float4 *>(p);
    }
}

template <bool NT>
__device__ __forceinline__ void store_state4(float *p, float4 y) {
    if constexpr (NT) {
        const f32x4v_t x = {y.x, y.y, y.z, y.w};
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4v_t *>(p));
    } else {
        *reinterpret_cast<float4 *>(p) = y;
    }
}

__device__ __forceinline__ float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

__device__ __forceinline__ float4 axpby4(float a, float4 x, float b, float4 y) {
    return make_float4(a * x.x + b * y.x, a * x.y + b * y.y, a * x.z + b * y.z, a * x.w + b * y.w);
}

}  // namespace gdn
