// Division by a divisor fixed at launch, with one multiply-high and a shift.
//
// The kernels map their workgroup index (and the backward's step index) onto
// (batch, head, tile) with divisions by sizes known only at run time. A
// plain integer division of wave-uniform values compiles to ~30 scalar
// instructions around a vector reciprocal and a readfirstlane; with the
// multiplier computed on the host it is a scalar multiply-high and a shift.
//
// Method (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, the round-up variant): for a divisor d >= 2
// let l = ceil(log2 d) and m = ceil(2^(31+l) / d), so 2^31 <= m < 2^32 and
// e = m d - 2^(31+l) lies in [0, d). For 0 <= n < 2^31, write n = q d + r:
//   n m / 2^(31+l) = n / d + n e / (d 2^(31+l)),
// and the second term is below n / 2^(31+l) < 1/d, because d <= 2^l; so the
// sum stays below q + (d-1)/d + 1/d = q + 1 and its floor is q. The floor of
// n m / 2^(31+l) is the high word of the 64-bit product shifted right by
// l - 1. d = 1 is kept apart (m would need 33 bits): mul = 0 returns n.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FastDiv {
    uint32_t mul;  // m, or 0 for d == 1
    uint32_t shr;  // l - 1
};

// Host: the multiplier and shift for a divisor d in [1, 2^31).
inline FastDiv make_fastdiv(int d) {
    FastDiv f = {0u, 0u};
    if (d <= 1) return f;
    uint32_t l = 0;
    while ((1ull << l) < (unsigned long long)d) ++l;
    const unsigned long long num = 1ull << (31 + l);
    f.mul = (uint32_t)((num + (unsigned long long)d - 1ull) / (unsigned long long)d);
    f.shr = l - 1;
    return f;
}

// floor(n / d) for 0 <= n < 2^31.
__host__ __device__ __forceinline__ int fast_div(int n, FastDiv f) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t hi = __umulhi((uint32_t)n, f.mul);
#else
    const uint32_t hi = (uint32_t)(((unsigned long long)(uint32_t)n * f.mul) >> 32);
#endif
    return f.mul != 0u ? (int)(hi >> f.shr) : n;
}

}  // namespace fa
