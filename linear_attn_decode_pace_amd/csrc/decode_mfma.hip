// Fused dequant -> chunked gated-delta update -> requant kernel for gfx950.
//
// One 64-wide wavefront owns one (sequence, head) state tile M (d x d, d = 64
// or 128) for the whole period and streams its packed codes and column scales
// through registers once: read, update, re-encode, write.  The period's C = 8
// tokens (fewer are padded with identity tokens alpha = 1, beta = 0) are
// applied as one chunk in the WY / UT form of the gated delta rule, which
// follows from unrolling M_t = alpha_t (M - beta_t k_t k_t^T M) + beta_t k_t v_t^T
// over the chunk (periodic rounding applies a period's tokens in high
// precision before one encode: 'PACE: four-bit recurrent state by rounding
// less often', TL;DR (1) and flowchart):
//
//   gamma_t = prod_{r<=t} alpha_r,  Gamma_ts = prod_{s<r<=t} alpha_r
//   A   = strictly lower (Gamma * K K^T),  T = (I + diag(beta) A)^-1 diag(beta)
//   X   = V - diag(gamma) K M0                 U = T X
//   O   = diag(gamma) Q M0 + lower_incl(Gamma * Q K^T) U
//   M_C = gamma_C M0 + K^T diag(Gamma_C,:) U
//
// with M0 = codes * diag(s).  Dense contractions run on MFMA:
//   * P = [K; Q] . codes  (16 x d x 16 per column block): bf16 MFMA, exact,
//     because codes (|c| <= 127) and bf16 inputs are exact in bf16 and their
//     products exact in float32;
//   * the 8 x 8 chunk matrices applied to X and Y = diag(gamma) Q M0 give W
//     (the update's right factor) and O: float32 MFMA (16x16x4) on X, whose
//     operand layout matches what each lane already holds, and Y (which
//     enters only O, with coefficient 1) added by one bf16 MFMA over two
//     parts of Y;
//   * K^T W (d x 8 x 16 per column block): bf16 MFMA with W in two bf16
//     parts (hi + mid: 16 significant bits, relative error below 2^-17)
//     stacked along the reduction dimension, one 16-deep product per row
//     tile.  A third part (exact W) cost eight more matrix instructions per
//     column block and 3-7% of the kernel's time; its 2^-17 is far below
//     the rounding the re-encode applies.
// The state is accumulated in units of sigma_j = gamma_C s_j:
//   acc = M_C / sigma_j = codes + K^T (W / sigma_j),
// so the accumulator starts from the codes themselves (no per-entry multiply).
// Re-encode (one scale per column: 'PACE: A New 4-Bit Recurrent State
// Quantization Method ...', section 'Channel-Aligned Encoding'):
//   absmax over the column's d rows (in-lane max, then two cross-lane xors),
//   s_new = absmax / qmax, codes = rint(M / s_new) via a fused multiply-add
//   against 1.5 * 2^23 (round to nearest even in one float32 rounding),
//   nibble / byte packing with v_perm and v_bfi, one 16-byte store per lane.
//
// Lane l = 16 g + n owns, in every column block cb, column j = 16 cb + n and
// the rows i with (i / 4) % 4 == g: exactly its rows of a 16 x 16 MFMA
// accumulator tile, and exactly its bytes in the pool layout (pace_layout.h).
#include "mfma_common.h"

namespace pace {
namespace {

constexpr int CH = 8;      // tokens per chunk
constexpr int LROW = 136;  // bf16 elements per LDS token row (128 + 8 padding)
constexpr int OCOL = 32;   // output columns staged before a flush (one 128-byte line per row)
constexpr int OROW = 36;   // floats per LDS output staging row (32 + 4 padding)

// LDS of one tile: its tokens and the chunk's small matrices
struct TileLds {
    uint16_t kq[16][LROW];  // rows 0..7: k_t, rows 8..15: q_t (bf16 bits)
    uint16_t v[CH][LROW];
    float alpha[CH], beta[CH];
    float kk[CH][CH], qk[CH][CH];  // k_t.k_s, q_t.k_s
    float A[CH][CH];               // strictly lower Gamma * K K^T
    float Lq[CH][CH];              // lower incl. diagonal Gamma * Q K^T
    float Tt[CH][CH];              // Tt[s][t] = T[t][s]
    float gam[CH];                 // gamma_t
    float gamC[CH];                // Gamma_{C-1, t}
};
// LDS of one wave: outputs of two column blocks, flushed as full lines
struct WaveOut {
    float o[CH][OROW];
};

// Waves sharing one tile (WPT).  WPT = 1: a wave owns a whole tile and four
// tiles share a workgroup.  WPT > 1 (a workgroup per tile, WPT waves splitting
// its column blocks, the first wave computing the chunk matrices) measured
// slower: the other waves wait at the barrier during that serial step.
#ifndef PACE_MFMA_WPT128
#define PACE_MFMA_WPT128 1
#endif
template <int DK>
struct Split;
template <>
struct Split<128> {
    static constexpr int WPT = PACE_MFMA_WPT128;
};
template <>
struct Split<64> {
    static constexpr int WPT = 1;
};

template <int WPT>
__device__ inline void tile_sync() {
    if constexpr (WPT == 1)
        wave_sync();
    else
        __syncthreads();
}

template <int DK, int BITS, int WPT, bool ERR, bool STEP>
__device__ void process_tile(const MfmaArgs &a, TileLds &L, WaveOut &WO_lds, int b, int h,
                             int slot, int lane, int q, bool trace) {
#define TRACE(slot_, v_)                                        \
    do {                                                        \
        if (trace) PACE_MFMA_TRACE((slot_), lane, (float)(v_)); \
    } while (0)
    constexpr int NKS = CodeChunk<DK>::NKS;  // k-slices of 32 rows
    constexpr int NRT = CodeChunk<DK>::NRT;  // row tiles of 16 rows
    constexpr int NCB = DK / 16;             // column blocks (d_v = d_k)
    constexpr int CPW = NCB / WPT;           // column blocks of this wave
    static_assert(CPW % 2 == 0, "outputs are flushed every two column blocks");
    constexpr float QMAX = BITS == 4 ? 7.f : 127.f;
    const int g = lane >> 4, n = lane & 15;
    // (sequence, head) rows per token; offsets between tokens are 64-bit, so
    // any batch the pools can hold runs here
    const size_t tok_stride = (size_t)a.p.B * (size_t)a.p.H;
    const size_t tile_row = (size_t)b * a.p.H + h;
    const int cb0 = q * CPW;
    // STEP (a PACE_STEP_BUFFER step): the chunk is the state's f buffered
    // tokens plus the step's own token f; only token f's output is written,
    // and the state is updated and re-encoded only when token f ends a period
    static_assert(!STEP || WPT == 1, "steps run one wave per tile");
    const int f = STEP ? __builtin_amdgcn_readfirstlane(a.step.fill[tile_row]) : 0;
    const int n_tok = STEP ? f + 1 : a.n_tok;
    // adaptive period: the step also closes the period once the buffered
    // tokens' summed write norms A exceed tau R (R: the stored state's norm
    // at its last encode)
    const bool adaptive = STEP && a.step.tau > 0.f;
    float adapt_A = 0.f, adapt_R = 0.f;
    if (adaptive) {
        adapt_A = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.step.adapt[2 * tile_row])));
        adapt_R = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.step.adapt[2 * tile_row + 1])));
    }
    const bool pend = !STEP || n_tok == a.step.period || (adaptive && adapt_A > a.step.tau * adapt_R);
    float uacc = 0.f, racc = 0.f;  // adaptive: sum of u_f^2 (mid-period) or of (c s)^2 (encode)
    uint16_t *sbuf = STEP ? (uint16_t *)a.step.kv + tile_row * a.step.slots * (2 * DK) : nullptr;
    float *sab = STEP ? a.step.ab + tile_row * a.step.slots * 2 : nullptr;

    uint8_t *codes = BITS == 4
        ? a.p.codes4 + ((size_t)b * a.p.n4 + slot) * tile_code_bytes(DK, DK, 4)
        : a.p.codes8 + ((size_t)b * a.p.n8 + slot) * tile_code_bytes(DK, DK, 8);
    float *scl = a.p.scales + tile_row * DK;

    // codes and scales of this wave's first column blocks: a ring of PF
    // column blocks kept in flight ahead of the one being processed
    constexpr int PF = CPW < PACE_MFMA_PREFETCH ? CPW : PACE_MFMA_PREFETCH;
    Loader<DK, BITS> ring[PF];
    float sring[PF];
#pragma unroll
    for (int c = 0; c < PF; ++c) {
        ring[c].load(codes, cb0 + c, lane);
        sring[c] = scl[16 * (cb0 + c) + n];
    }

    // ---- stage the chunk's tokens in LDS (padding tokens: k = q = v = 0),
    //      split over the tile's waves; every load before the first write ----
    {
        constexpr int CPR = DK / 8;                         // 16-byte chunks per token row
        constexpr int NL = (24 * CPR + 64 * WPT - 1) / (64 * WPT);  // loads per lane
        const uint16_t *srcs[3] = {a.k + tile_row * DK, a.q + tile_row * DK, a.v + tile_row * DK};
        // load it of this lane reads token row (c / CPR) & 7 with c = lane +
        // 64 (q + WPT it): token lane / CPR plus a wave-uniform step, so one
        // per-lane 64-bit product serves every load
        const size_t tok_elems = tok_stride * DK;
        const size_t lane_off = (size_t)(lane / CPR) * tok_elems + (lane % CPR) * 8;
        u32x4 val[NL];
#pragma unroll
        for (int it = 0; it < NL; ++it) {
            const int c = lane + 64 * (q + WPT * it);
            const int row = c / CPR, col = (c % CPR) * 8;
            const int t = row & 7, which = row >> 3;
            const size_t off = lane_off + (size_t)(((64 / CPR) * (q + WPT * it)) & 7) * tok_elems;
            val[it] = u32x4{0u, 0u, 0u, 0u};
            if constexpr (STEP) {
                // token f from the step's inputs [B, H, d]; earlier tokens (k, v
                // only: their outputs are not needed) from the buffer
                if (row < 24 && t == f)
                    val[it] = __builtin_nontemporal_load(at((const u32x4 *)srcs[which], (uint32_t)col * 2u));
                else if (row < 24 && t < f && which != 1)
                    val[it] = *at((const u32x4 *)sbuf,
                                  (uint32_t)(t * 2 * DK + (which == 2 ? DK : 0) + col) * 2u);
            } else if (row < 24 && t < n_tok) {
                val[it] = __builtin_nontemporal_load((const u32x4 *)(srcs[which] + off));
            }
        }
        float ab = 0.f;
        if (q == 0 && lane < 16) {
            const int t = lane & 7;
            const bool is_beta = lane >= 8;
            ab = is_beta ? 0.f : 1.f;
            if (STEP && t < f)
                ab = sab[2 * t + is_beta];
            else if (t < n_tok)
                ab = (is_beta ? a.beta : a.alpha)[tile_row + (STEP ? 0 : t * tok_stride)];
        }
#pragma unroll
        for (int it = 0; it < NL; ++it) {
            const int c = lane + 64 * (q + WPT * it);
            const int row = c / CPR, col = (c % CPR) * 8;
            const int t = row & 7, which = row >> 3;
            if (row < 24) {
                uint16_t *dst = which < 2 ? &L.kq[which * 8 + t][col] : &L.v[t][col];
                *(u32x4 *)dst = val[it];
                // a token that does not end its period joins the buffer (slot f)
                if (STEP && !pend && t == f && which != 1)
                    *at((u32x4 *)sbuf, (uint32_t)(t * 2 * DK + (which == 2 ? DK : 0) + col) * 2u) = val[it];
            }
        }
        if (q == 0 && lane < 16) {
            if (lane >= 8)
                L.beta[lane & 7] = ab;
            else
                L.alpha[lane & 7] = ab;
            if (STEP && !pend && (lane & 7) == f) sab[2 * f + (lane >> 3)] = ab;
        }
    }
    tile_sync<WPT>();

    // ---- [K;Q] as the MFMA A operand: A row m = 4 gg + rr holds k_gg, k_{4+gg},
    //      q_gg, q_{4+gg} for rr = 0..3; k index e of slice ks is state row
    //      32 ks + 16 (e / 4) + 4 g + e % 4 (this lane's rows of two row tiles) ----
    const int krow = ((n & 3) == 0) ? (n >> 2) : ((n & 3) == 1) ? 4 + (n >> 2)
                   : ((n & 3) == 2) ? 8 + (n >> 2) : 12 + (n >> 2);
    // A operand slice ks of [K;Q] (re-read from LDS where needed: saves registers)
    auto ap_slice = [&](int ks) {
        const int c0 = 32 * ks + 4 * g, c1 = c0 + 16;
        u32x2 r0 = *(const u32x2 *)&L.kq[krow][c0];
        u32x2 r1 = *(const u32x2 *)&L.kq[krow][c1];
        u32x4 w = {r0[0], r0[1], r1[0], r1[1]};
        return __builtin_bit_cast(bf16x8, w);
    };

    // ---- the chunk's small matrices, computed once per tile by its first wave ----
    if (q == 0) {
        {
            bf16x8 AP[NKS];
            bf16x8 BG[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int c0 = 32 * ks + 4 * g, c1 = c0 + 16;
                AP[ks] = ap_slice(ks);
                u32x4 z = {0u, 0u, 0u, 0u};
                if (n < 8) {
                    u32x2 s0 = *(const u32x2 *)&L.kq[n][c0];
                    u32x2 s1 = *(const u32x2 *)&L.kq[n][c1];
                    z = u32x4{s0[0], s0[1], s1[0], s1[1]};
                }
                BG[ks] = __builtin_bit_cast(bf16x8, z);
            }
            // G[m][n] = row m of [K;Q] . k_n
            f32x4 G = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) G = mfma_bf16_k32(AP[ks], BG[ks], G);
            TRACE(0, G[0]); TRACE(1, G[1]); TRACE(2, G[2]); TRACE(3, G[3]);
            if (n < 8) {
                L.kk[g][n] = G[0];
                L.kk[4 + g][n] = G[1];
                L.qk[g][n] = G[2];
                L.qk[4 + g][n] = G[3];
            }
        }
        wave_sync();

        // gates: Gamma_ts as products of alpha (no log / exp), A and Lq
        {
            float al[CH];
#pragma unroll
            for (int r = 0; r < CH; ++r) al[r] = L.alpha[r];
            const int t = lane >> 3, s = lane & 7;
            float gts = 1.f;
#pragma unroll
            for (int r = 1; r < CH; ++r) gts *= (r > s && r <= t) ? al[r] : 1.f;
            L.A[t][s] = s < t ? gts * L.kk[t][s] : 0.f;
            L.Lq[t][s] = s <= t ? gts * L.qk[t][s] : 0.f;
            if (lane < CH) {
                float gm = 1.f, gc = 1.f;
#pragma unroll
                for (int r = 0; r < CH; ++r) {
                    gm *= r <= lane ? al[r] : 1.f;
                    gc *= r > lane ? al[r] : 1.f;
                }
                L.gam[lane] = gm;
                L.gamC[lane] = gc;
            }
        }
        wave_sync();

        // UT transform: column s of Z = (I + diag(beta) A)^-1 by forward
        // substitution; T = Z diag(beta)
        {
            const int s = lane & 7;
            float be[CH], z[CH];
#pragma unroll
            for (int r = 0; r < CH; ++r) be[r] = L.beta[r];
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                float sum = 0.f;
#pragma unroll
                for (int u = 0; u < t; ++u) sum = fmaf(L.A[t][u], z[u], sum);
                z[t] = (t == s ? 1.f : 0.f) - be[t] * sum;
            }
            if (lane < CH) {
#pragma unroll
                for (int t = 0; t < CH; ++t) L.Tt[s][t] = z[t] * be[s];
            }
        }
    }
    tile_sync<WPT>();

    // ---- A operand of the chunk mixing (4 steps over [X tokens 0-3, X 4-7,
    //      Y 0-3, Y 4-7]; float32 16x16x4 MFMA for the X steps):
    //      rows 0..7  -> W_t = Gamma_{C-1,t} (T X)_t          (A = Gamma_C T, 0)
    //      rows 8..15 -> O_t = (Lq T X)_t + Y_t               (A = Lq T, I) ----
    float CA[4];
    {
        const int t = n & 7;
        const bool is_o = n >= 8;
        float r0 = 0.f, r1 = 0.f;
        if (is_o) {
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                const float lq = L.Lq[t][u];
                r0 = fmaf(lq, L.Tt[g][u], r0);
                r1 = fmaf(lq, L.Tt[4 + g][u], r1);
            }
        } else {
            const float gct = L.gamC[t];
            r0 = gct * L.Tt[g][t];
            r1 = gct * L.Tt[4 + g][t];
        }
        CA[0] = r0;
        CA[1] = r1;
        CA[2] = (is_o && t == g) ? 1.f : 0.f;
        CA[3] = (is_o && t == 4 + g) ? 1.f : 0.f;
    }
    // Y enters only the O rows, with coefficient 1: one bf16 16x16x16 product
    // adds it, Y in two parts (k-slots 4 g + [Y0 hi, Y1 hi, Y0 mid, Y1 mid]),
    // in place of the two float32 Y steps (16 instead of 64 matrix-core
    // cycles).  W's rows get exact zeros from it; O gets Y to 2^-17.
    const uint32_t ay = pk_bf16(CA[2], CA[3]);
    const s16x4 AY = __builtin_bit_cast(s16x4, u32x2{ay, ay});
    const float gam_g = L.gam[g], gam_4g = L.gam[4 + g], gamC = L.gam[CH - 1];
    TRACE(4, CA[0]); TRACE(5, CA[1]); TRACE(6, CA[2]); TRACE(7, CA[3]);
    TRACE(10, gam_g); TRACE(11, gam_4g); TRACE(12, gamC);
    TRACE(13, L.A[lane >> 3][lane & 7]); TRACE(14, L.Tt[lane >> 3][lane & 7]);
    TRACE(15, L.kk[lane >> 3][lane & 7]); TRACE(16, L.Lq[lane >> 3][lane & 7]);

    // K^T as the A operand of the update: row i = 16 rt + n, k index 4 g + e is
    // token 4 (g % 2) + e (the same tokens for the hi and mid parts)
    s16x4 AU[NRT];
    {
        const int t0 = 4 * (g & 1);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int i = 16 * rt + n;
            s16x4 x;
            x[0] = (short)L.kq[t0 + 0][i];
            x[1] = (short)L.kq[t0 + 1][i];
            x[2] = (short)L.kq[t0 + 2][i];
            x[3] = (short)L.kq[t0 + 3][i];
            AU[rt] = x;
        }
    }

    // this lane's part of an output flush: token row lane / 8, 16-byte chunk
    // lane % 8 of the 32 staged columns
    float *olane = a.out + (tile_row + (STEP ? 0 : (size_t)(lane >> 3) * tok_stride)) * DK + (lane & 7) * 4;

    // ---- this wave's column blocks (unrolled: ring slots stay in fixed registers) ----
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
        // compiler-only barrier: keeps the per-block LDS re-reads from being
        // hoisted out of the unrolled loop into long-lived registers
        asm volatile("" ::: "memory");
        const int cb = cb0 + cc;
        const int j = 16 * cb + n;
        const int slot = cc % PF;
        const float s = sring[slot];

        // KAPPA * codes -> float32 (the accumulator's start) and bf16 B operands
        constexpr float KAPPA = Loader<DK, BITS>::KAPPA;
        f32x4 acc[NRT];
        ring[slot].codes_f32(acc);
        if (cc + PF < CPW) {
            ring[slot].load(codes, cb + PF, lane);
            sring[slot] = scl[j + 16 * PF];
        }

        f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4 w = {pk_bf16(acc[2 * ks][0], acc[2 * ks][1]), pk_bf16(acc[2 * ks][2], acc[2 * ks][3]),
                       pk_bf16(acc[2 * ks + 1][0], acc[2 * ks + 1][1]),
                       pk_bf16(acc[2 * ks + 1][2], acc[2 * ks + 1][3])};
            P = mfma_bf16_k32(ap_slice(ks), __builtin_bit_cast(bf16x8, w), P);
        }
        // P = KAPPA * [k_g . c, k_{4+g} . c, q_g . c, q_{4+g} . c] for column j
        if (cb == 0) { TRACE(20, P[0]); TRACE(21, P[1]); TRACE(22, P[2]); TRACE(23, P[3]); TRACE(24, s); }
        const float sk = s * (1.f / KAPPA);  // exact: KAPPA is a power of two
        const float sg = gam_g * sk, s4g = gam_4g * sk;
        const float X0 = fmaf(-sg, P[0], bf2f(L.v[g][j]));
        const float X1 = fmaf(-s4g, P[1], bf2f(L.v[4 + g][j]));
        const float Y0 = sg * P[2];
        const float Y1 = s4g * P[3];

        // accumulate M / unit with unit = gamma_C s / KAPPA, so the accumulator
        // starts from the loaded KAPPA * c (unit = 1 / KAPPA for a zero column)
        const float sig_raw = gamC * s;
        const bool tiny = s > 0.f && !(sig_raw >= 1.17549435e-38f);
        const float sig = ((s > 0.f && !tiny) ? sig_raw : 1.f) * (1.f / KAPPA);
        if (__builtin_amdgcn_ballot_w64(tiny)) {
            // decay below float32's normal range: start from gamma_C s c directly
            const float m0 = tiny ? sig_raw : 1.f;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) acc[rt] *= m0;
        }
        const float inv_sig = __builtin_amdgcn_rcpf(sig);

        // one chain: lanes g < 2 get W (tokens 4 g + r), lanes g >= 2 get O
        const uint32_t yh = pk_bf16(Y0, Y1);
        const uint32_t ym = pk_bf16(Y0 - lo_f32(yh), Y1 - hi_f32(yh));
        f32x4 WO = {0.f, 0.f, 0.f, 0.f};
        WO = mfma_f32_k4(CA[0], X0, WO);
        WO = mfma_f32_k4(CA[1], X1, WO);
        WO = mfma_bf16_k16(AY, __builtin_bit_cast(s16x4, u32x2{yh, ym}), WO);
        f32x4 W;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float other = __shfl_xor(WO[r], 32);
            W[r] = (g < 2 ? WO[r] : other) * inv_sig;  // tokens 4 (g % 2) + r, units of sig
        }
        if (cb == 0) {
            TRACE(25, X0); TRACE(26, X1); TRACE(27, Y0); TRACE(28, Y1); TRACE(29, sig);
            for (int r = 0; r < 4; ++r) { TRACE(30 + r, W[r]); TRACE(34 + r, WO[r]); }
        }
        if (g >= 2) {
#pragma unroll
            for (int r = 0; r < 4; ++r) WO_lds.o[4 * (g - 2) + r][j % OCOL] = WO[r];
        }
        if (cc % 2 == 1) {
            // every second column block: flush 8 rows x 128 bytes, one 16-byte
            // chunk per lane (lane -> row lane / 8, chunk lane % 8)
            wave_sync();
            const int t = lane >> 3, c4 = (lane & 7) * 4;
            const f32x4 x = *(const f32x4 *)&WO_lds.o[t][c4];
            if (STEP ? t == f : t < n_tok) __builtin_nontemporal_store(x, (f32x4 *)(olane + 16 * cb - 16));
        }
        if constexpr (STEP) {
            if (adaptive && !pend) {
                // this token's write u_f (column j): row f of W, held by lane group f / 4
                const int r = f & 3;
                const float u = r == 0 ? WO[0] : r == 1 ? WO[1] : r == 2 ? WO[2] : WO[3];
                if (g == (f >> 2)) uacc = fmaf(u, u, uacc);
            }
            if (!pend) continue;  // mid-period step: the stored state is only read
        }

        // W in two bf16 parts: lanes g < 2 give hi (k-slots 0..7), lanes
        // g >= 2 the rounded rest (k-slots 8..15), both for tokens 4 (g % 2) + r
        const uint32_t hi01 = pk_bf16(W[0], W[1]), hi23 = pk_bf16(W[2], W[3]);
        const float r0 = W[0] - lo_f32(hi01), r1 = W[1] - hi_f32(hi01);
        const float r2 = W[2] - lo_f32(hi23), r3 = W[3] - hi_f32(hi23);
        const uint32_t md01 = pk_bf16(r0, r1), md23 = pk_bf16(r2, r3);
        const bool first = g < 2;
        const u32x2 b1 = {first ? hi01 : md01, first ? hi23 : md23};
        const s16x4 B1 = __builtin_bit_cast(s16x4, b1);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) acc[rt] = mfma_bf16_k16(AU[rt], B1, acc[rt]);

        // ---- re-encode the column ----
        float am = 0.f;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) am = fmaxf(am, fabsf(acc[rt][r]));
        am = xor_max(am, 16);
        am = xor_max(am, 32);
        if (cb == 0) {
            for (int rt = 0; rt < NRT; ++rt)
                for (int r = 0; r < 4; ++r) TRACE(40 + 4 * rt + r, acc[rt][r]);
            TRACE(38, am);
        }
        const float absmax = am * sig;
        const float s_new = absmax * (1.f / QMAX);
        const float ratio = s_new > 0.f ? sig * __builtin_amdgcn_rcpf(s_new) : 0.f;
        uint32_t y[NRT][4];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) y[rt][r] = __float_as_uint(fmaf(acc[rt][r], ratio, 12582912.f));
        Loader<DK, BITS> outc;
        if constexpr (BITS == 4) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const uint32_t lo = gather_low_bytes(y[2 * ks][0], y[2 * ks][1], y[2 * ks][2], y[2 * ks][3]);
                const uint32_t hi = gather_low_bytes(y[2 * ks + 1][0], y[2 * ks + 1][1],
                                                     y[2 * ks + 1][2], y[2 * ks + 1][3]);
                outc.d[ks] = (lo & 0x0f0f0f0fu) | ((hi << 4) & 0xf0f0f0f0u);
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) outc.d[rt] = gather_low_bytes(y[rt][0], y[rt][1], y[rt][2], y[rt][3]);
        }
        outc.store(codes, cb, lane);
        if (g == 0) scl[j] = s_new;
        if constexpr (ERR) column_error<NRT>(acc, y, sig, s_new, a.p.colerr + (tile_row * DK + j) * 2, g);
        if constexpr (STEP) {
            if (adaptive) {
                float cc = 0.f;
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float c = __uint_as_float(y[rt][r]) - 12582912.f;
                        cc = fmaf(c, c, cc);
                    }
                racc = fmaf(cc, s_new * s_new, racc);
            }
        }
    }
    if constexpr (STEP) {
        if (adaptive) {
            float v = pend ? racc : uacc;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
            if (lane == 0) {
                if (pend) {
                    a.step.adapt[2 * tile_row] = 0.f;
                    a.step.adapt[2 * tile_row + 1] = sqrtf(v);   // ||decode(new stored)||_F
                } else {
                    a.step.adapt[2 * tile_row] = adapt_A + sqrtf(L.kk[f][f]) * sqrtf(v);
                }
            }
        }
        if (lane == 0) a.step.fill[tile_row] = pend ? 0 : n_tok;
    }
#undef TRACE
}

template <int DK, bool ERR, bool STEP>
__global__ void __launch_bounds__(256) decode_mfma_kernel(MfmaArgs a) {
    constexpr int WPT = Split<DK>::WPT;
    // tiles per workgroup: four for whole periods; one per step, where tiles
    // that end their period (and write codes) run beside tiles that only
    // read, and a workgroup holds its slot until its slowest wave is done
    constexpr int TPB = WPT == 1 && !STEP ? 4 : 1;
    __shared__ TileLds tl[TPB];
    __shared__ WaveOut wo[TPB * WPT];
    const int lane = threadIdx.x & 63;
    // wave-uniform indices (scalar registers: the head lookup below is a
    // scalar-cache load, not a dependent vector load at the head of the tile)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tib = wave / WPT, q = wave - tib * WPT;
    const int w = xcd_block(blockIdx.x, a.xcd_run, a.xcd_full) * TPB + tib;
    if (w >= a.tiles) return;  // whole tiles only: every wave of a workgroup agrees when WPT > 1
    // sequence-major order: the heads of one sequence are neighbours, so
    // workgroups on a CU mix 4-bit and 8-bit tiles and read whole input rows
    const int b = w / a.p.H, h = w - b * a.p.H;
    if (STEP && a.step.active && !a.step.active[b]) return;  // this sequence takes no token
    const int m = a.p.head_map[h];  // slot | bits << 16 (scalar load)
    if ((m >> 16) == 8)
        process_tile<DK, 8, WPT, ERR, STEP>(a, tl[tib], wo[wave], b, h, m & 0xffff, lane, q, w == 0 && q == 0);
    else
        process_tile<DK, 4, WPT, ERR, STEP>(a, tl[tib], wo[wave], b, h, m & 0xffff, lane, q, w == 0 && q == 0);
}

}  // namespace

bool mfma_supported(int dk, int dv, int n_tok, int in_bf16, long long rows_per_token) {
    // periods of 9..16 tokens take the 16-token chunk kernel; offsets between
    // tokens are 64-bit, so the batch is not limited here
    (void)rows_per_token;
    return in_bf16 && dk == dv && (dk == 128 || dk == 64) && n_tok >= 1 && n_tok <= 2 * CH;
}

namespace {

MfmaArgs make_args(const PoolView &p, const int32_t *heads8, const int32_t *heads4, int n_tok,
                   const void *q, const void *k, const void *v, const float *alpha,
                   const float *beta, float *out) {
    MfmaArgs a = {};
    a.p = p;
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.alpha = alpha;
    a.beta = beta;
    a.out = out;
    a.heads8 = heads8;
    a.heads4 = heads4;
    a.n_tok = n_tok;
    a.tiles8 = p.B * p.n8;
    a.tiles = p.B * p.H;
    return a;
}

template <bool STEP>
hipError_t launch(MfmaArgs &a, hipStream_t s) {
    const PoolView &p = a.p;
    const bool err = p.colerr != nullptr;
    set_xcd_order(a, (p.dk == 128 ? Split<128>::WPT : Split<64>::WPT) == 1 && !STEP ? 4 : 1);
    if (p.dk == 128) {
        constexpr int WPT = Split<128>::WPT, TPB = WPT == 1 && !STEP ? 4 : 1;
        const dim3 grid((a.tiles + TPB - 1) / TPB), block(64 * WPT * TPB);
        if (err)
            hipLaunchKernelGGL((decode_mfma_kernel<128, true, STEP>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<128, false, STEP>), grid, block, 0, s, a);
    } else {
        constexpr int WPT = Split<64>::WPT, TPB = WPT == 1 && !STEP ? 4 : 1;
        const dim3 grid((a.tiles + TPB - 1) / TPB), block(64 * WPT * TPB);
        if (err)
            hipLaunchKernelGGL((decode_mfma_kernel<64, true, STEP>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<64, false, STEP>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const PoolView &p, const int32_t *heads8, const int32_t *heads4,
                              int n_tok, const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta, float *out, hipStream_t s) {
    MfmaArgs a = make_args(p, heads8, heads4, n_tok, q, k, v, alpha, beta, out);
    if (n_tok > CH) return launch_decode_mfma16(a, s);
    return launch<false>(a, s);
}

bool mfma_step_supported(int dk, int dv, int period, int in_bf16, long long rows_per_token) {
    return period <= CH && mfma_supported(dk, dv, period, in_bf16, rows_per_token);
}

hipError_t launch_step_mfma(const PoolView &p, const StepView &sv, const int32_t *heads8,
                            const int32_t *heads4, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, float *out, hipStream_t s) {
    MfmaArgs a = make_args(p, heads8, heads4, 0, q, k, v, alpha, beta, out);
    a.step = sv;
    return launch<true>(a, s);
}

}  // namespace pace
