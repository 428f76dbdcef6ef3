// gdn_conv.h -- per-row arithmetic of the pre-processing in front of the
// recurrence, shared by the standalone pre-processing kernel and the fused
// layer's chunk preparation (so that both produce the same bits): the 4-tap
// causal convolution of one row slice of 8 channels, the optional SiLU, the
// L2 norm over a head's lanes, the gate maps, and 8-channel loads and stores.
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename T> struct Vec8;

// Outputs are stored non-temporally (measured about 4% faster on a layer's
// q, k, v at T = 4096, H = 48; non-temporal loads were slower).
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt16(void *p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    __builtin_nontemporal_store(v4u32{a, b, c, d}, reinterpret_cast<v4u32 *>(p));
}

template <> struct Vec8<uint16_t> {  // bf16 bit patterns
    typedef uint4 raw_t;
    __device__ __forceinline__ static raw_t load(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ static raw_t zero() { return make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ static void unpack(const raw_t &w, float (&x)[8]) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo_to_f32(u[i]);
            x[2 * i + 1] = bf16_hi_to_f32(u[i]);
        }
    }
    __device__ __forceinline__ static void store(uint16_t *p, const float (&x)[8]) {
        store_nt16(p, pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7]));
    }
};

template <> struct Vec8<float> {
    struct raw_t {
        float4 a, b;
    };
    __device__ __forceinline__ static raw_t load(const float *p) {
        return raw_t{*reinterpret_cast<const float4 *>(p), *reinterpret_cast<const float4 *>(p + 4)};
    }
    __device__ __forceinline__ static raw_t zero() {
        return raw_t{make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    }
    __device__ __forceinline__ static void unpack(const raw_t &w, float (&x)[8]) {
        x[0] = w.a.x; x[1] = w.a.y; x[2] = w.a.z; x[3] = w.a.w;
        x[4] = w.b.x; x[5] = w.b.y; x[6] = w.b.z; x[7] = w.b.w;
    }
    __device__ __forceinline__ static void store(float *p, const float (&x)[8]) {
        store_nt16(p, __float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
        store_nt16(p + 4, __float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]),
                   __float_as_uint(x[7]));
    }
};

__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float softplusf_(float x) { return x > 0.f ? x + log1pf(__expf(-x)) : log1pf(__expf(x)); }

// The 32 taps of one lane: 8 channels x 4 taps, oldest input first.
__device__ __forceinline__ void load_taps(const float *__restrict__ wp, float (&tap)[8][4]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float4 t = *reinterpret_cast<const float4 *>(wp + 4 * e);
        tap[e][0] = t.x; tap[e][1] = t.y; tap[e][2] = t.z; tap[e][3] = t.w;
    }
}

// One token of one (tensor, head) row slice: convolution over the window
// w0..w2 (oldest first) and the current input, activation, norm (over the
// LPR lanes of the head), into acc.
template <int LPR>
__device__ __forceinline__ void pre_row(const float (&tap)[8][4], const float (&w0)[8], const float (&w1)[8],
                                        const float (&w2)[8], const float (&cur)[8], int act, bool normalise,
                                        float (&acc)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = tap[e][0] * w0[e] + tap[e][1] * w1[e] + tap[e][2] * w2[e] + tap[e][3] * cur[e];
    if (act) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= sigmoidf_(acc[e]);
    }
    if (normalise) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += acc[e] * acc[e];
        ss = group_sum<LPR>(ss);
        const float scale = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 1.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= scale;
    }
}

// The same, stored to dst when `store`.
template <typename TIn, int LPR>
__device__ __forceinline__ void pre_token(const float (&tap)[8][4], const float (&w0)[8], const float (&w1)[8],
                                          const float (&w2)[8], const float (&cur)[8], int act, bool normalise,
                                          bool store, TIn *dst) {
    float acc[8];
    pre_row<LPR>(tap, w0, w1, w2, cur, act, normalise, acc);
    if (store) Vec8<TIn>::store(dst, acc);
}

// The gate maps: beta = sigmoid(b), g = exp(-softplus(a + bias)).
__device__ __forceinline__ float gate_beta(float b) { return sigmoidf_(b); }
__device__ __forceinline__ float gate_g(float a, float bias) { return __expf(-softplusf_(a + bias)); }

}  // namespace gdn
