// OCP FP8 E4M3 in software (the FP8 write window): 1 sign bit, 4 exponent bits
// with bias 7, 3 mantissa bits; exponent field 0 holds subnormals, multiples
// of 2^-9; the largest finite value is 448 (exponent field 15, mantissa 6).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace pace {
namespace {

constexpr float E4M3_MAX = 448.f;

// nearest E4M3 code of x (|x| <= 448), ties to even: 3 mantissa bits kept of
// float32's 23; below 2^-6 the quantum is 2^-9
__device__ inline uint8_t e4m3_encode(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fabsf(x);
    if (a < 0.015625f) {  // subnormal range: multiples of 2^-9
        const float m = rintf(a * 512.f);  // exact scaling, nearest even
        return (uint8_t)(sign | (uint32_t)m);
    }
    const uint32_t au = __float_as_uint(a);
    int e = (int)(au >> 23) - 127;
    uint32_t man = au & 0x7fffffu;
    uint32_t r = man >> 20, rem = man & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    if (r == 8u) {
        r = 0;
        ++e;
    }
    return (uint8_t)(sign | ((uint32_t)(e + 7) << 3) | r);
}

// value of an E4M3 code (the low byte of c), without branches: an exponent
// field E > 0 gives (1 + M/8) 2^(E-7), i.e. float32 bits (E + 120) << 23 |
// M << 20; E = 0 gives M 2^-9
__device__ inline float e4m3_decode(uint32_t c) {
    const uint32_t em = c & 0x7fu;
    const float nrm = __uint_as_float((em << 20) + (120u << 23));
    const float sub = (float)em * 0.001953125f;
    const float v = em >= 8u ? nrm : sub;
    return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}

}  // namespace
}  // namespace pace
