// Token-only matrices of a 16-token chunk for the 16-token decode kernel
// (decode_mfma16.hip).  One wavefront computes them from the chunk's k_t,
// q_t (bf16 rows in LDS, row stride ROW elements) and alpha_t, beta_t:
//   kk[t][s] = k_t . k_s,  qk[t][s] = q_t . k_s                (Gram on MFMA)
//   Gamma_ts = prod_{s<r<=t} alpha_r, gam[t] = Gamma_t,-1, gamC[t] = Gamma_15,t
//   A = strictly lower (Gamma * kk),  Lq = lower incl. diagonal (Gamma * qk)
//   Zt = ((I + diag(beta) A)^-1)^T, so that T = Z diag(beta)   (UT transform)
//   LqT = Lq T                                                  (float32 MFMA)
// Gates are products of alpha (no log / exp).  All arrays live in LDS; each
// step ends with the wavefront's LDS writes visible to it (wave_sync).
#pragma once

#include "mfma_common.h"

namespace pace {
namespace {

constexpr int CK = 16;  // tokens per chunk
// Row stride (floats) that callers may give the 16 x 16 matrices: rows stay
// 16-byte aligned and a column's 16 entries fall in 16 different LDS banks
// (a stride of 16 puts rows t and t + 4 in the same bank).
constexpr int CKS = 20;

// Gram products kk[t][s] = k_t . k'_s and qk[t][s] = q_t . k'_s, where k_t,
// q_t come from kq_t (rows 0..15 keys, rows 16..31 queries) and k'_s from
// kq_s (rows 0..15): the A row m of the K (Q) block is token 4 (m % 4) + m / 4,
// so output row 4 g + r is token 4 r + g
template <int DK, int ROW, int STR>
__device__ inline void chunk16_gram2(const uint16_t (*kq_t)[ROW], const uint16_t (*kq_s)[ROW],
                                     float (*kk)[STR], float (*qk)[STR], int lane) {
    constexpr int NKS = DK / 32;
    const int g = lane >> 4, n = lane & 15;
    const int tok_n = 4 * (n & 3) + (n >> 2);
    f32x4 GK = {0.f, 0.f, 0.f, 0.f}, GQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const int c0 = 32 * ks + 4 * g, c1 = c0 + 16;
        const u32x2 k0 = *(const u32x2 *)&kq_t[tok_n][c0], k1 = *(const u32x2 *)&kq_t[tok_n][c1];
        const u32x2 q0 = *(const u32x2 *)&kq_t[CK + tok_n][c0], q1 = *(const u32x2 *)&kq_t[CK + tok_n][c1];
        const u32x2 s0 = *(const u32x2 *)&kq_s[n][c0], s1 = *(const u32x2 *)&kq_s[n][c1];
        const bf16x8 BG = __builtin_bit_cast(bf16x8, u32x4{s0[0], s0[1], s1[0], s1[1]});
        GK = mfma_bf16_k32(__builtin_bit_cast(bf16x8, u32x4{k0[0], k0[1], k1[0], k1[1]}), BG, GK);
        GQ = mfma_bf16_k32(__builtin_bit_cast(bf16x8, u32x4{q0[0], q0[1], q1[0], q1[1]}), BG, GQ);
    }
    wave_sync();  // the A operands are read before kk / qk may alias them
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        kk[4 * r + g][n] = GK[r];
        qk[4 * r + g][n] = GQ[r];
    }
    wave_sync();
}

// Gram products of one chunk: kk[t][s] = k_t . k_s, qk[t][s] = q_t . k_s
template <int DK, int ROW, int STR>
__device__ inline void chunk16_gram(const uint16_t (*kq)[ROW], float (*kk)[STR], float (*qk)[STR],
                                    int lane) {
    chunk16_gram2<DK, ROW, STR>(kq, kq, kk, qk, lane);
}

// x from lane n - K (SHR) or n + K (SHL) of the lane's row of 16, 1 where
// that lane lies outside the row
template <int CTRL>
__device__ inline float row_move_or_one(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_SHL = 0x100, DPP_SHR = 0x110;

// gates, A and Lq: lane -> row t = lane / 4, columns s0 .. s0 + 3 with
// s0 = 4 (lane % 4): Gamma_{t,s0+3} as one masked product, then the running
// product down to s0.  gamma_t (prefix products of alpha) and Gamma_{CK-1,t}
// (the product of the alphas after t) come from DPP scans over each row of
// 16 lanes, lane n holding alpha_n.
template <int STR>
__device__ inline void chunk16_gates(const float *alpha, const float (*kk)[STR],
                                     const float (*qk)[STR], float (*A)[STR], float (*Lq)[STR],
                                     float *gam, float *gamC, int lane) {
    float al[CK];
#pragma unroll
    for (int r = 0; r < CK; ++r) al[r] = alpha[r];
    const int t = lane >> 2, s0 = 4 * (lane & 3);
    float gts = 1.f;
#pragma unroll
    for (int r = 1; r < CK; ++r) gts *= (r > s0 + 3 && r <= t) ? al[r] : 1.f;
    float a_row[4], l_row[4];
#pragma unroll
    for (int e = 3; e >= 0; --e) {
        const int s = s0 + e;
        a_row[e] = s < t ? gts * kk[t][s] : 0.f;
        l_row[e] = s <= t ? gts * qk[t][s] : 0.f;
        if (e > 0 && s <= t) gts *= alpha[s];  // Gamma_{t,s-1} = Gamma_{t,s} alpha_s
    }
    const float x = alpha[lane & 15];
    float pre = x, suf = x;
    pre *= row_move_or_one<DPP_SHR + 1>(pre);
    suf *= row_move_or_one<DPP_SHL + 1>(suf);
    pre *= row_move_or_one<DPP_SHR + 2>(pre);
    suf *= row_move_or_one<DPP_SHL + 2>(suf);
    pre *= row_move_or_one<DPP_SHR + 4>(pre);
    suf *= row_move_or_one<DPP_SHL + 4>(suf);
    pre *= row_move_or_one<DPP_SHR + 8>(pre);
    suf *= row_move_or_one<DPP_SHL + 8>(suf);
    const float after = row_move_or_one<DPP_SHL + 1>(suf);  // product over r > t
    wave_sync();  // kk / qk are read before A / Lq may alias them
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        A[t][s0 + e] = a_row[e];
        Lq[t][s0 + e] = l_row[e];
    }
    if (lane < CK) {
        gam[lane] = pre;
        gamC[lane] = after;
    }
    wave_sync();
}

// UT transform in 8 x 8 blocks.  Z = (I + N)^-1 with N = diag(beta) A
// strictly lower is [Z11 0; Z21 Z22] with Z11, Z22 the inverses of the
// diagonal blocks and Z21 = -Z22 N21 Z11.  Lanes 0..15 substitute column
// s = lane of its diagonal block (8 steps); then all 64 lanes form
// Y = N21 Z11 and Z21 = -Z22 Y, one entry each.  Writes Zt[s][t] = Z[t][s]
// (T = Z diag(beta) is left to the readers: T[t][s] = Z[t][s] beta_s).
template <int STR>
__device__ inline void chunk16_ut(const float (*A)[STR], const float *beta, float (*Zt)[STR],
                                  int lane) {
    {
        const int s = lane & 15, rb = s & 8;  // column s, rows rb .. rb + 7 of its diagonal block
        float z[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            float sum = 0.f;
#pragma unroll
            for (int u = 0; u < t; ++u) sum = fmaf(A[rb + t][rb + u], z[u], sum);
            z[t] = (rb + t == s ? 1.f : 0.f) - beta[rb + t] * sum;
        }
        if (lane < CK) {
#pragma unroll
            for (int t = 0; t < 8; ++t) Zt[s][rb + t] = z[t];
        }
    }
    wave_sync();
    const int i = lane >> 3, j = lane & 7;
    // Y[i][j] = beta_{8+i} sum_k A[8+i][k] Z[k][j], kept at Zt[8 + j][i] (the
    // zero block of Z^T: rows s >= 8, columns t < 8)
    float y = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) y = fmaf(A[8 + i][k], Zt[j][k], y);
    Zt[8 + j][i] = beta[8 + i] * y;
    wave_sync();
    // Z21[i][j] = -sum_k Z[8+i][8+k] Y[k][j]; then the zero block is restored
    float zz = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) zz = fmaf(Zt[8 + k][8 + i], Zt[8 + j][k], zz);
    Zt[j][8 + i] = -zz;
    wave_sync();  // every lane has read Y
    Zt[8 + j][i] = 0.f;
    wave_sync();
}

// Lq T on float32 MFMA from Zt = Z^T (T = Z diag(beta)): step st takes
// column / row 4 st + g; the product's column n is scaled by beta_n
template <int STR>
__device__ inline void chunk16_lqt(const float (*Lq)[STR], const float (*Zt)[STR], const float *beta,
                                   float (*LqT)[STR], int lane) {
    const int g = lane >> 4, n = lane & 15;
    f32x4 D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) D = mfma_f32_k4(Lq[n][4 * st + g], Zt[n][4 * st + g], D);
    const float bn = beta[n];
    wave_sync();  // Lq is read before LqT may alias it
#pragma unroll
    for (int r = 0; r < 4; ++r) LqT[4 * g + r][n] = D[r] * bn;
    wave_sync();
}

}  // namespace
}  // namespace pace
