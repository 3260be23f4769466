// hp_device.h -- small helpers shared by the kernel files: division by a
// launch-invariant divisor, index loads of either index type, wave-uniform
// values. Not installed; not part of the ABI.
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

} // namespace hp
