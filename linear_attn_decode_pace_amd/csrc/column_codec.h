// Device helpers of the per-column kernels (kernels_v0.hip, kernels_window.hip):
// a thread owns one state column j of one (sequence, head) state; it reads
// and writes only its column's codes (pace_layout.h), so no two threads of a
// launch touch the same byte.
#pragma once

#include "pace_layout.h"

namespace pace {
namespace {

__device__ inline float ld_in(const void *p, size_t idx, int bf16) {
    if (bf16) {
        uint32_t u = ((const uint16_t *)p)[idx];
        return __uint_as_float(u << 16);
    }
    return ((const float *)p)[idx];
}

template <int DK>
__device__ inline void load_column(const uint8_t *codes, int bits, int j, float s, float M[DK]) {
#pragma unroll
    for (int i = 0; i < DK; ++i) {
        int c;
        if (bits == 4) {
            int sh;
            size_t o = loc4(DK, i, j, &sh);
            c = ((int)((uint32_t)codes[o] << (28 - sh))) >> 28;  // sign-extend the nibble
        } else {
            c = (int)(int8_t)codes[loc8(DK, i, j)];
        }
        M[i] = (float)c * s;
    }
}

// Per-column quantizer: s = absmax / qmax (float32, correctly rounded),
// c = rint(M / s) with round-half-even, clamped to +-qmax; s = 0 -> codes 0.
// err (NULL: skipped) receives the sums over the column of (M - c s)^2 and M^2;
// deq2 (NULL: skipped) the sum of (c s)^2.
template <int DK>
__device__ inline float store_column(uint8_t *codes, int bits, int j, const float M[DK],
                                     float *err, float *deq2 = nullptr) {
    float e2 = 0.f, m2 = 0.f, q2 = 0.f;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < DK; ++i) amax = fmaxf(amax, fabsf(M[i]));
    const int qm = bits == 4 ? 7 : 127;
    float s = amax / (float)qm;
    if (bits == 4) {
        // whole bytes: rows (2ks, r) and (2ks+1, r) of one lane group share a byte
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            int rt = i >> 4;
            if (rt & 1) continue;
            int i2 = i + 16;
            int c0 = 0, c1 = 0;
            if (s > 0.f) {
                c0 = (int)fminf(fmaxf(rintf(M[i] / s), -7.f), 7.f);
                c1 = (int)fminf(fmaxf(rintf(M[i2] / s), -7.f), 7.f);
            }
            if (err) {
                const float d0 = M[i] - (float)c0 * s, d1 = M[i2] - (float)c1 * s;
                e2 += d0 * d0 + d1 * d1;
                m2 += M[i] * M[i] + M[i2] * M[i2];
            }
            q2 += (float)(c0 * c0 + c1 * c1);
            int sh;
            size_t o = loc4(DK, i, j, &sh);
            codes[o] = (uint8_t)((c0 & 15) | ((c1 & 15) << 4));
        }
    } else {
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            int c = 0;
            if (s > 0.f) c = (int)fminf(fmaxf(rintf(M[i] / s), -127.f), 127.f);
            codes[loc8(DK, i, j)] = (uint8_t)(int8_t)c;
            if (err) {
                const float d = M[i] - (float)c * s;
                e2 += d * d;
                m2 += M[i] * M[i];
            }
            q2 += (float)(c * c);
        }
    }
    if (err) {
        err[0] = e2;
        err[1] = m2;
    }
    if (deq2) *deq2 = q2 * s * s;
    return s;
}

// sum of x over the block's threads (blockDim.x <= 256), returned to every thread
__device__ inline float block_sum(float x, float *red) {
    for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    float t = 0.f;
    for (int w = 0; w < (int)(blockDim.x + 63) / 64; ++w) t += red[w];
    return t;
}

// max of x over the block's threads (blockDim.x <= 256), returned to every thread
__device__ inline float block_max(float x, float *red) {
    for (int m = 32; m > 0; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    float t = 0.f;
    for (int w = 0; w < (int)(blockDim.x + 63) / 64; ++w) t = fmaxf(t, red[w]);
    return t;
}

}  // namespace
}  // namespace pace
