// gdn_mfma.h -- bf16 MFMA fragments for gfx950 (v_mfma_f32_16x16x32_bf16).
//
// One wave multiplies a 16x32 A tile by a 32x16 B tile into a 16x16 fp32 tile.
// With lane L = 16*g + r (g = 0..3, r = 0..15):
//   A fragment: lane L holds A[r][slot 8g + e], e = 0..7   (16 bytes)
//   B fragment: lane L holds B[slot 8g + e][r], e = 0..7   (16 bytes)
//   accumulator: lane L holds D[4g + e][r], e = 0..3       (4 fp32)
// A B fragment of Y is therefore the A fragment of Y^T.
//
// Slot order.  The 32 k indices of one step are assigned to slots so that two
// accumulator tiles stacked along k ARE a B fragment, lane for lane:
//   slot 8g + e  <->  k = 4g + e        (e < 4, from the first 16-row tile)
//   slot 8g + e  <->  k = 16 + 4g + e-4 (e >= 4, from the second tile)
// Every operand read from memory uses the same slot order, so a product whose
// k runs over rows of an earlier accumulator needs no cross-lane movement.
//
// fp32 operands are split as x = hi + lo with hi = bf16(x), lo = bf16(x - hi);
// hi*hi + lo*hi + hi*lo keeps about 16 significant bits of each product, and a
// product with an exact bf16 operand needs only hi + lo of the other.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// k index (0..31) held in slot 8g + e of a step
__host__ __device__ constexpr int slot_k(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); }

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Two fp32 -> one dword of two bf16 (round to nearest even; a in the low half).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// (a, b) -> hi = bf16(a), bf16(b) and lo = bf16(a - hi_a), bf16(b - hi_b), one dword each.
// a - hi_a is exact in fp32 (hi_a is a rounded to 8 significant bits); it is
// formed as the bf16 dot product (hi_a, hi_b) . (-1, 0) + a, one instruction
// instead of an unpack and a subtraction (likewise (0, -1) for b).  Only a
// value below the smallest normal float could lose its hi part there (a
// flushed bf16 operand), an absolute error under 1.2e-38.  The two constant
// operands are kept opaque (scalar registers): the compiler would otherwise
// encode the pair (-1, 0) as the inline constant -1.0, which the hardware
// does not read as that pair for a packed bf16 operand.
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    uint32_t m_lo = 0x0000BF80u, m_hi = 0xBF800000u;  // (-1, 0) and (0, -1)
    asm("" : "+s"(m_lo), "+s"(m_hi));
    hi = cvt_pk_bf16(a, b);
    const bf16x2_t h = __builtin_bit_cast(bf16x2_t, hi);
    const float la = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2_t, m_lo), a, false);
    const float lb = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2_t, m_hi), b, false);
    lo = cvt_pk_bf16(la, lb);
}

// x[0..7] -> (hi, lo) bf16 fragments
__device__ __forceinline__ void split8(const float (&x)[8], u32x4_t &hi, u32x4_t &lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t h, l;
        split2(x[2 * i], x[2 * i + 1], h, l);
        hi[i] = h;
        lo[i] = l;
    }
}

// x[0..3] -> (hi, lo) halves of a fragment (8 bytes each)
__device__ __forceinline__ void split4(f32x4_t x, u32x2_t &hi, u32x2_t &lo) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        uint32_t h, l;
        split2(x[2 * i], x[2 * i + 1], h, l);
        hi[i] = h;
        lo[i] = l;
    }
}

// Two accumulator tiles stacked along k -> split B fragment.
__device__ __forceinline__ void split_pair(f32x4_t a, f32x4_t b, u32x4_t &hi, u32x4_t &lo) {
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    split8(x, hi, lo);
}

// D += A*B with A split (hi, lo) and B exact bf16
__device__ __forceinline__ f32x4_t mfma2a(u32x4_t ahi, u32x4_t alo, u32x4_t b, f32x4_t d) {
    d = mfma(alo, b, d);
    return mfma(ahi, b, d);
}
// D += A*B with A exact bf16 and B split
__device__ __forceinline__ f32x4_t mfma2b(u32x4_t a, u32x4_t bhi, u32x4_t blo, f32x4_t d) {
    d = mfma(a, blo, d);
    return mfma(a, bhi, d);
}
// D += A*B with both split (lo*lo dropped)
__device__ __forceinline__ f32x4_t mfma3(u32x4_t ahi, u32x4_t alo, u32x4_t bhi, u32x4_t blo, f32x4_t d) {
    d = mfma(alo, bhi, d);
    d = mfma(ahi, blo, d);
    return mfma(ahi, bhi, d);
}

}  // namespace gdn
