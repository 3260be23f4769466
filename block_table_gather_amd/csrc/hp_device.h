// hp_device.h -- small helpers shared by the kernel files: division by a
// launch-invariant divisor, index loads of either index type, wave-uniform
// values, the int8 -> bf16 rounding. Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hp {

// Division by a launch-invariant 32-bit divisor d as a multiply and a shift:
// q = (umulhi(n, mul) + n) >> shift with shift = ceil(log2 d) and
// mul = floor(2^32 (2^shift - d) / d) + 1, exact for every 32-bit n
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).
struct Div {
    uint32_t d, mul, shift;
};

inline Div make_div(uint32_t d) {
    Div f;
    f.d = d;
    f.shift = 0;
    while ((1ull << f.shift) < d)
        ++f.shift;
    const unsigned __int128 num = ((unsigned __int128)1 << 32) * (((uint64_t)1 << f.shift) - d);
    f.mul = (uint32_t)(num / d + 1);
    return f;
}

__device__ __forceinline__ uint64_t min64(uint64_t a, uint64_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t min32(uint32_t a, uint32_t b) { return a < b ? a : b; }

// Wave-uniform copies (the value of the first active lane, in scalar registers).
__device__ __forceinline__ uint32_t uni(uint32_t x) {
    return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ uint64_t uni64(uint64_t x) {
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t udiv32(uint32_t n, Div f) {
    return (uint32_t)(((uint64_t)__umulhi(n, f.mul) + n) >> f.shift);
}
__device__ __forceinline__ uint64_t udiv(uint64_t n, Div f) {
    if ((n >> 32) == 0)
        return udiv32((uint32_t)n, f);
    return n / f.d;
}

template <typename IdxT>
__device__ __forceinline__ uint64_t ld_idx(const void *p, uint64_t i) {
    return (uint64_t)static_cast<const IdxT *>(p)[i];
}

// fp32 -> bf16 bits, round to nearest even (gfx950 converts with IEEE
// rounding for this type). The pair converts as one vector, which maps to a
// single v_cvt_pk_bf16_f32 (lo in the low half). Every int8 -> bf16
// dequantisation in the library (the dequant-gathers and attention over an
// int8 pool) rounds through these, so their results agree bit for bit.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, b2));
}
__device__ __forceinline__ uint16_t to_bf16(float x) {
    __bf16 a = (__bf16)x;
    return __builtin_bit_cast(uint16_t, a);
}
// Signed byte k of w, as a float (exact).
__device__ __forceinline__ float sbyte(uint32_t w, int k) {
    return (float)(int8_t)(w >> (8 * k));
}

} // namespace hp
