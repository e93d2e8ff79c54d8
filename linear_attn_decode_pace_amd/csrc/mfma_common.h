// Device helpers shared by the fused decode kernels (decode_mfma.hip for
// chunks of up to 8 tokens, decode_mfma16.hip for 9..16): operand types, bf16
// packing, MFMA wrappers, the code loader / unpacker and byte packing.
#pragma once

#include "pace_mfma.h"
#include "pace_step.h"

namespace pace {

struct MfmaArgs {
    PoolView p;
    const uint16_t *q, *k, *v;
    const float *alpha, *beta;
    float *out;
    const int32_t *heads8;  // slot -> head, 8-bit pool
    const int32_t *heads4;  // slot -> head, 4-bit pool
    int n_tok;
    int tiles8;     // B * n8: work items below this are 8-bit tiles
    int tiles;      // B * H
    int xcd_run;    // K: workgroups per XCD run (see xcd_block)
    int xcd_full;   // workgroups covered by whole groups of 8 K
    StepView step;  // per-step decode only (PACE_STEP_BUFFER)
};

// Workgroup order.  The dispatcher hands workgroup i to XCD i % 8, and each
// XCD reaches memory through its own L2 and fabric port, so the launch runs at
// the pace of the XCD with the most bytes.  Heads of different bit widths move
// different bytes, so a plain order loads XCDs unevenly whenever the head mix
// repeats with the XCD count (e.g. four-tile workgroups over 16 heads: XCDs 3
// and 7 always get heads 12..15).  Instead XCD x takes a run of K consecutive
// workgroups out of every group of 8 K, with K chosen so that K workgroups
// cover whole sequences: every XCD then carries the same head mix, and all
// XCDs still work inside one window of the pools.  Workgroups past the last
// whole group keep their place.
inline int xcd_run_for(int heads, int tiles_per_wg) {
    int a = heads, b = tiles_per_wg;
    while (b) {
        const int t = a % b;
        a = b;
        b = t;
    }
    return heads / a;  // lcm(heads, tiles_per_wg) / tiles_per_wg
}
inline void set_xcd_order(MfmaArgs &a, int tiles_per_wg) {
    const int K = xcd_run_for(a.p.H, tiles_per_wg);
    const long long whole_wgs = a.tiles / tiles_per_wg;
    a.xcd_run = K;
    a.xcd_full = (int)(whole_wgs / (8ll * K) * (8ll * K));
}
__device__ inline int xcd_block(int i, int K, int full) {
    if (i >= full) return i;
    const int G = i / (8 * K), p = i - G * 8 * K;
    return G * 8 * K + (p & 7) * K + (p >> 3);
}

// the 16-token chunk kernel (decode_mfma16.hip), for 9..16 tokens per call
hipError_t launch_decode_mfma16(const MfmaArgs &a, hipStream_t s);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Debug builds may define PACE_MFMA_TRACE(slot, lane, value) to record
// intermediates of the first work item; it is a no-op otherwise.
#ifndef PACE_MFMA_TRACE
#define PACE_MFMA_TRACE(slot, lane, value) \
    do {                                    \
    } while (0)
#endif

// column blocks of codes kept in flight ahead of the one being processed
#ifndef PACE_MFMA_PREFETCH
#define PACE_MFMA_PREFETCH 2
#endif


__device__ inline float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ inline uint32_t pk_bf16(float lo, float hi) {
    f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
__device__ inline float lo_f32(uint32_t pk) { return __uint_as_float(pk << 16); }
__device__ inline float hi_f32(uint32_t pk) { return __uint_as_float(pk & 0xffff0000u); }

// Order this wavefront's LDS accesses (no workgroup barrier: waves of a block
// are independent; LDS operations of one wave execute in issue order).
__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ inline f32x4 mfma_bf16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma_bf16_k16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ inline float xor_max(float x, int mask) {
    return fmaxf(x, __shfl_xor(x, mask));
}

// low bytes of four words -> one word
__device__ inline uint32_t gather_low_bytes(uint32_t y0, uint32_t y1, uint32_t y2, uint32_t y3) {
    uint32_t a = __builtin_amdgcn_perm(y1, y0, 0x0c0c0400u);  // [y0.b0, y1.b0, 0, 0]
    uint32_t b = __builtin_amdgcn_perm(y3, y2, 0x04000c0cu);  // [0, 0, y2.b0, y3.b0]
    return a | b;
}

template <int DK>
struct CodeChunk;
template <>
struct CodeChunk<128> {
    static constexpr int NKS = 4, NRT = 8;
};
template <>
struct CodeChunk<64> {
    static constexpr int NKS = 2, NRT = 4;
};

template <int DK, int BITS>
struct Loader {
    // Codes are streamed: read once and written once per period, with a pool
    // far larger than the last-level cache, so loads and stores are
    // non-temporal.
    // dwords a lane holds per column block: 4-bit: one per k-slice; 8-bit: one per row tile
    static constexpr int ND = BITS == 4 ? DK / 32 : DK / 16;
    uint32_t d[ND];
    __device__ inline void load(const uint8_t *codes, int cb, int lane) {
        if constexpr (BITS == 4) {
            const uint8_t *p = codes + (size_t)cb * (64 * DK / 8) + (size_t)lane * (DK / 8);
            if constexpr (DK == 128) {
                u32x4 x = __builtin_nontemporal_load((const u32x4 *)p);
                d[0] = x[0], d[1] = x[1], d[2] = x[2], d[3] = x[3];
            } else {
                u32x2 x = __builtin_nontemporal_load((const u32x2 *)p);
                d[0] = x[0], d[1] = x[1];
            }
        } else {
            const uint8_t *p = codes + (size_t)cb * (64 * DK / 4) + (size_t)lane * 16;
#pragma unroll
            for (int qd = 0; qd < DK / 64; ++qd) {
                u32x4 x = __builtin_nontemporal_load((const u32x4 *)(p + qd * 1024));
                d[4 * qd + 0] = x[0], d[4 * qd + 1] = x[1], d[4 * qd + 2] = x[2], d[4 * qd + 3] = x[3];
            }
        }
    }
    __device__ inline void store(uint8_t *codes, int cb, int lane) const {
        if constexpr (BITS == 4) {
            uint8_t *p = codes + (size_t)cb * (64 * DK / 8) + (size_t)lane * (DK / 8);
            if constexpr (DK == 128) {
                u32x4 x = {d[0], d[1], d[2], d[3]};
                __builtin_nontemporal_store(x, (u32x4 *)p);
            } else {
                u32x2 x = {d[0], d[1]};
                __builtin_nontemporal_store(x, (u32x2 *)p);
            }
        } else {
            uint8_t *p = codes + (size_t)cb * (64 * DK / 4) + (size_t)lane * 16;
#pragma unroll
            for (int qd = 0; qd < DK / 64; ++qd) {
                u32x4 x = {d[4 * qd], d[4 * qd + 1], d[4 * qd + 2], d[4 * qd + 3]};
                __builtin_nontemporal_store(x, (u32x4 *)(p + qd * 1024));
            }
        }
    }
    // KAPPA * code of (row tile rt, row r in the lane's group) as float.  A
    // 4-bit code is read by v_cvt_off_f32_i4, which takes bits 3:0 of its
    // source (here one byte, or the byte's high half moved down) as a signed
    // 4-bit integer c and returns c / 16: one instruction per code, with the
    // factor KAPPA = 1/16 folded exactly into the scale units.  8-bit codes
    // are one sign-extending byte conversion each.
    static constexpr float KAPPA = BITS == 4 ? 1.f / 16.f : 1.f;
    template <int B>
    __device__ static inline float nibble_f32(uint32_t x) {
        float r;
        if constexpr (B == 0)
            asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(x));
        else if constexpr (B == 1)
            asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(x));
        else if constexpr (B == 2)
            asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(x));
        else
            asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(x));
        return r;
    }
    __device__ inline void codes_f32(f32x4 *acc) const {
        if constexpr (BITS == 4) {
#pragma unroll
            for (int ks = 0; ks < ND; ++ks) {
                const uint32_t lo = d[ks];       // row tile 2 ks: low nibbles
                const uint32_t hi = d[ks] >> 4;  // row tile 2 ks + 1: high nibbles
                acc[2 * ks][0] = nibble_f32<0>(lo);
                acc[2 * ks][1] = nibble_f32<1>(lo);
                acc[2 * ks][2] = nibble_f32<2>(lo);
                acc[2 * ks][3] = nibble_f32<3>(lo);
                acc[2 * ks + 1][0] = nibble_f32<0>(hi);
                acc[2 * ks + 1][1] = nibble_f32<1>(hi);
                acc[2 * ks + 1][2] = nibble_f32<2>(hi);
                acc[2 * ks + 1][3] = nibble_f32<3>(hi);
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < ND; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[rt][r] = (float)(int)__builtin_amdgcn_sbfe(d[rt], 8 * r, 8);
        }
    }
};

// Error statistics of one column at its re-encode: sums over the column's rows
// of (M - c s_new)^2 and M^2, with M = acc * sig and c read back from the
// rounding sum y = acc * ratio + 1.5 * 2^23 (exact: |acc * ratio| <= qmax);
// the four lane groups of the column are combined and lanes g == 0 store.
template <int NRT>
__device__ inline void column_error(const f32x4 *acc, const uint32_t (*y)[4], float sig,
                                    float s_new, float *dst, int g) {
    float e2 = 0.f, m2 = 0.f;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float m = acc[rt][r] * sig;
            const float c = __uint_as_float(y[rt][r]) - 12582912.f;
            const float d = fmaf(-c, s_new, m);
            e2 = fmaf(d, d, e2);
            m2 = fmaf(m, m, m2);
        }
    e2 += __shfl_xor(e2, 16);
    m2 += __shfl_xor(m2, 16);
    e2 += __shfl_xor(e2, 32);
    m2 += __shfl_xor(m2, 32);
    if (g == 0) *(f32x2 *)dst = f32x2{e2, m2};
}

// byte-offset access from a wave-uniform base: keeps per-lane address math in
// 32 bits (the base lives in scalar registers)
template <class T>
__device__ inline T *at(T *base, uint32_t byte_off) {
    return (T *)((char *)base + byte_off);
}
template <class T>
__device__ inline const T *at(const T *base, uint32_t byte_off) {
    return (const T *)((const char *)base + byte_off);
}

}  // namespace
}  // namespace pace
