// Fused dequant -> chunked gated-delta update -> requant kernel for periods of
// 9..16 tokens (gfx950).  Same algebra, pool layout and codec as the 8-token
// kernel (decode_mfma.hip); the chunk is C = 16 (shorter periods are padded
// with identity tokens alpha = 1, beta = 0):
//
//   gamma_t = prod_{r<=t} alpha_r,  Gamma_ts = prod_{s<r<=t} alpha_r
//   A   = strictly lower (Gamma * K K^T),  T = (I + diag(beta) A)^-1 diag(beta)
//   X   = V - diag(gamma) K M0,   Y = diag(gamma) Q M0,   U = T X
//   O   = Y + lower_incl(Gamma * Q K^T) U,   M_C = gamma_C M0 + K^T diag(Gamma_C,:) U
//
// Token placement: lane group g (lane = 16 g + n) holds tokens 4 r + g,
// r = 0..3, of the [K.codes; Q.codes] products (the MFMA output rows 4 g + r),
// which is exactly the reduction index the float32 16x16x4 MFMA steps take
// from each lane; the chunk-mixing chain then returns W and O rows 4 g + r,
// i.e. tokens 4 g + r, which are the reduction indices this lane feeds to the
// K^T W update (16x16x16 bf16 MFMA, W in two bf16 parts, hi + mid): no
// cross-lane exchange is needed at C = 16.  W (the update's right factor)
// comes from float32 16x16x4 steps; O, which only leaves as an output, from
// three bf16 16x16x16 products over two parts of each factor (hi.hi + hi.mid
// + mid.hi: relative error near 2^-16 per product, against 1e-4 for the
// outputs), 48 instead of 128 matrix-core cycles per column block.
#include "chunk16.h"

namespace pace {
namespace {

constexpr int C16 = 16;     // tokens per chunk
constexpr int LROW16 = 136;  // bf16 elements per LDS token row (128 + 8 padding)
constexpr int OCOL16 = 32;   // output columns staged before a flush
constexpr int OROW16 = 36;   // floats per LDS output staging row

// One region serves three phases in turn: the staged v rows (read into
// registers right after staging), the chunk matrices (dead once the MFMA
// operands are built), then the output staging of the column loop.  13 KB per
// tile: three waves per SIMD.
struct alignas(16) Tile16Lds {
    uint16_t kq[2 * C16][LROW16];  // rows 0..15: k_t, rows 16..31: q_t (bf16 bits)
    union {
        uint16_t v[C16][LROW16];
        struct {
            // rows padded to CKS floats: a column's 16 entries in 16 banks
            float kkA[C16][CKS];   // k_t.k_s, then A (strictly lower Gamma * K K^T) in place
            float qkLq[C16][CKS];  // q_t.k_s, then Lq, then Lq T in place
            float Zt[C16][CKS];    // Zt[s][t] = Z[t][s], T = Z diag(beta)
        } m;
        float o[C16][OROW16];      // outputs of two column blocks
    } u;
    float alpha[C16], beta[C16];
    float gam[C16];   // gamma_t
    float gamC[C16];  // Gamma_{C-1, t}
};

constexpr int TPB16 = 2;  // tiles (waves) per workgroup

template <int DK, int BITS, bool ERR>
__device__ void process_tile16(const MfmaArgs &a, Tile16Lds &L, int b, int h, int slot, int lane) {
    constexpr int NKS = CodeChunk<DK>::NKS;  // k-slices of 32 rows
    constexpr int NRT = CodeChunk<DK>::NRT;  // row tiles of 16 rows
    constexpr int NCB = DK / 16;             // column blocks (d_v = d_k)
    constexpr float QMAX = BITS == 4 ? 7.f : 127.f;
    constexpr float KAPPA = Loader<DK, BITS>::KAPPA;
    const int g = lane >> 4, n = lane & 15;
    const int n_tok = a.n_tok;
    // (sequence, head) rows per token; offsets between tokens are 64-bit
    const size_t tok_stride = (size_t)a.p.B * (size_t)a.p.H;
    const size_t tok_elems = tok_stride * DK;
    const size_t tile_row = (size_t)b * a.p.H + h;

    uint8_t *codes = BITS == 4
        ? a.p.codes4 + ((size_t)b * a.p.n4 + slot) * tile_code_bytes(DK, DK, 4)
        : a.p.codes8 + ((size_t)b * a.p.n8 + slot) * tile_code_bytes(DK, DK, 8);
    float *scl = a.p.scales + tile_row * DK;

    constexpr int PF = NCB < PACE_MFMA_PREFETCH ? NCB : PACE_MFMA_PREFETCH;
    Loader<DK, BITS> ring[PF];
    float sring[PF];
#pragma unroll
    for (int c = 0; c < PF; ++c) {
        ring[c].load(codes, c, lane);
        sring[c] = scl[16 * c + n];
    }

    // ---- stage the chunk's tokens (48 rows) in LDS.  A padding token
    //      (t >= n_tok, alpha = 1, beta = 0) repeats the last real token's
    //      k, q, v: beta = 0 makes its row and column of T exactly zero, so
    //      finite values there change no output or state entry ----
    {
        constexpr int CPR = DK / 8;                // 16-byte chunks per token row
        constexpr int RPL = 64 / CPR;              // token rows per load
        constexpr int NL = 3 * C16 / RPL;          // loads per lane (12 for d = 128)
        constexpr int NT = C16 / RPL;              // distinct tokens of a lane (4 for d = 128)
        const uint16_t *srcs[3] = {a.k + tile_row * DK, a.q + tile_row * DK, a.v + tile_row * DK};
        // load it reads token row lane / CPR + RPL (it % NT) of source it / NT
        size_t toff[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i)
            toff[i] = (size_t)min(lane / CPR + RPL * i, n_tok - 1) * tok_elems + (lane % CPR) * 8;
        u32x4 val[NL];
#pragma unroll
        for (int it = 0; it < NL; ++it)
            val[it] = __builtin_nontemporal_load((const u32x4 *)(srcs[it / NT] + toff[it % NT]));
        float ab = 0.f;
        if (lane < 32) {
            const int t = lane & 15;
            const bool is_beta = lane >= 16;
            ab = is_beta ? 0.f : 1.f;
            if (t < n_tok)
                ab = (is_beta ? a.beta : a.alpha)[tile_row + t * tok_stride];
        }
#pragma unroll
        for (int it = 0; it < NL; ++it) {
            const int c = lane + 64 * it;
            const int row = c / CPR, col = (c % CPR) * 8;
            const int t = row & 15, which = row >> 4;
            uint16_t *dst = which < 2 ? &L.kq[which * 16 + t][col] : &L.u.v[t][col];
            *(u32x4 *)dst = val[it];
        }
        if (lane < 32) {
            if (lane >= 16)
                L.beta[lane & 15] = ab;
            else
                L.alpha[lane & 15] = ab;
        }
    }
    wave_sync();

    // ---- A operands: A row m of the K block is token 4 (m % 4) + m / 4, so
    //      output row 4 g + r of P_K is token 4 r + g (the mixing steps'
    //      reduction index); the Q block keeps token order, so row 4 g + r of
    //      P_Q is token 4 g + r, the output row this lane holds; k index e of
    //      slice ks is state row 32 ks + 16 (e / 4) + 4 g + e % 4 ----
    const int tok_n = 4 * (n & 3) + (n >> 2);
    auto ap_slice = [&](int blk, int ks) {
        const int c0 = 32 * ks + 4 * g, c1 = c0 + 16;
        const int row = blk == 0 ? tok_n : 16 + n;
        u32x2 r0 = *(const u32x2 *)&L.kq[row][c0];
        u32x2 r1 = *(const u32x2 *)&L.kq[row][c1];
        u32x4 w = {r0[0], r0[1], r1[0], r1[1]};
        return __builtin_bit_cast(bf16x8, w);
    };
    // v_{4 r + g}[16 cb + n] of every column block, two tokens per register
    // (the v rows' LDS then takes the chunk matrices)
    constexpr int NCBV = DK / 16;
    uint32_t vreg[NCBV][2];
#pragma unroll
    for (int cb = 0; cb < NCBV; ++cb)
#pragma unroll
        for (int hp = 0; hp < 2; ++hp)
            vreg[cb][hp] = (uint32_t)L.u.v[4 * (2 * hp) + g][16 * cb + n] |
                           ((uint32_t)L.u.v[4 * (2 * hp + 1) + g][16 * cb + n] << 16);
    wave_sync();

    // ---- the chunk's token-only matrices (chunk16.h) ----
    chunk16_gram<DK, LROW16>(L.kq, L.u.m.kkA, L.u.m.qkLq, lane);
    chunk16_gates(L.alpha, L.u.m.kkA, L.u.m.qkLq, L.u.m.kkA, L.u.m.qkLq, L.gam, L.gamC, lane);
    chunk16_ut(L.u.m.kkA, L.beta, L.u.m.Zt, lane);
    chunk16_lqt(L.u.m.qkLq, L.u.m.Zt, L.beta, L.u.m.qkLq, lane);

    // ---- chunk-mixing operands (step st takes token 4 st + g from lane
    //      group g; 16x16x4 float32 MFMA for W, the same four k-slots of a
    //      16x16x16 bf16 MFMA for O):
    //      W chain, row m = token m: A = Gamma_{C-1,m} T[m][4 st + k]
    //      O chain, row m = token m: A = (Lq T)[m][4 st + k] on X; Y is added
    //      in place, its rows already in output order ----
    float CW[4], CO[4];
    {
        const float gct = L.gamC[n];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int s = 4 * st + g;
            CW[st] = gct * (L.u.m.Zt[s][n] * L.beta[s]);  // Gamma_{C-1,n} T[n][s]
            CO[st] = L.u.m.qkLq[n][s];  // (Lq T)[n][s]
        }
    }
    float gam_r[4], gam_o[4];  // gamma of tokens 4 r + g (X) and 4 g + r (Y)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        gam_r[r] = L.gam[4 * r + g];
        gam_o[r] = L.gam[4 * g + r];
    }
    const float gamC = L.gam[C16 - 1];
    // the O coefficients in two bf16 parts (hi + mid), k-slot 4 g + st
    s16x4 COH, COM;
    {
        const uint32_t h01 = pk_bf16(CO[0], CO[1]), h23 = pk_bf16(CO[2], CO[3]);
        const uint32_t m01 = pk_bf16(CO[0] - lo_f32(h01), CO[1] - hi_f32(h01));
        const uint32_t m23 = pk_bf16(CO[2] - lo_f32(h23), CO[3] - hi_f32(h23));
        COH = __builtin_bit_cast(s16x4, u32x2{h01, h23});
        COM = __builtin_bit_cast(s16x4, u32x2{m01, m23});
    }

    // K^T as the update's A operand: row i = 16 rt + n, k index 4 g + e is token 4 g + e
    s16x4 AU[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int i = 16 * rt + n;
        s16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (short)L.kq[4 * g + e][i];
        AU[rt] = x;
    }
    wave_sync();  // the chunk matrices are dead from here on: their LDS holds outputs

    // this lane's part of an output flush: token rows lane / 8 (+ 8), 16-byte
    // chunk lane % 8 of the 32 staged columns
    float *olane = a.out + (tile_row + (size_t)(lane >> 3) * tok_stride) * DK + (lane & 7) * 4;

#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        asm volatile("" ::: "memory");
        const int j = 16 * cb + n;
        const int slot = cb % PF;
        const float s = sring[slot];
        f32x4 acc[NRT];
        ring[slot].codes_f32(acc);
        if (cb + PF < NCB) {
            ring[slot].load(codes, cb + PF, lane);
            sring[slot] = scl[j + 16 * PF];
        }

        // P_K[r] = KAPPA k_{4r+g} . c_j,  P_Q[r] = KAPPA q_{4g+r} . c_j
        f32x4 PK = {0.f, 0.f, 0.f, 0.f}, PQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4 w = {pk_bf16(acc[2 * ks][0], acc[2 * ks][1]), pk_bf16(acc[2 * ks][2], acc[2 * ks][3]),
                       pk_bf16(acc[2 * ks + 1][0], acc[2 * ks + 1][1]),
                       pk_bf16(acc[2 * ks + 1][2], acc[2 * ks + 1][3])};
            const bf16x8 Bc = __builtin_bit_cast(bf16x8, w);
            PK = mfma_bf16_k32(ap_slice(0, ks), Bc, PK);
            PQ = mfma_bf16_k32(ap_slice(1, ks), Bc, PQ);
        }
        const float sk = s * (1.f / KAPPA);
        const float sig_raw = gamC * s;
        const bool tiny = s > 0.f && !(sig_raw >= 1.17549435e-38f);
        const float sig = ((s > 0.f && !tiny) ? sig_raw : 1.f) * (1.f / KAPPA);
        if (__builtin_amdgcn_ballot_w64(tiny)) {
            const float m0 = tiny ? sig_raw : 1.f;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) acc[rt] *= m0;
        }
        const float inv_sig = __builtin_amdgcn_rcpf(sig);
        float X[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sg = gam_r[r] * sk;
            const uint32_t vv = vreg[cb][r >> 1];
            X[r] = fmaf(-sg, PK[r], bf2f((uint16_t)((r & 1) ? (vv >> 16) : (vv & 0xffffu))));
        }
        f32x4 W = {0.f, 0.f, 0.f, 0.f}, O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) W = mfma_f32_k4(CW[st], X[st] * inv_sig, W);
        {
            const uint32_t xh01 = pk_bf16(X[0], X[1]), xh23 = pk_bf16(X[2], X[3]);
            const uint32_t xm01 = pk_bf16(X[0] - lo_f32(xh01), X[1] - hi_f32(xh01));
            const uint32_t xm23 = pk_bf16(X[2] - lo_f32(xh23), X[3] - hi_f32(xh23));
            const s16x4 XH = __builtin_bit_cast(s16x4, u32x2{xh01, xh23});
            const s16x4 XM = __builtin_bit_cast(s16x4, u32x2{xm01, xm23});
            O = mfma_bf16_k16(COH, XH, O);
            O = mfma_bf16_k16(COH, XM, O);
            O = mfma_bf16_k16(COM, XH, O);
        }
        // + Y = diag(gamma) Q M0, tokens 4 g + r
#pragma unroll
        for (int r = 0; r < 4; ++r) O[r] = fmaf(gam_o[r] * sk, PQ[r], O[r]);

        // outputs: tokens 4 g + r of column j; flush 16 rows x 128 bytes every two blocks
#pragma unroll
        for (int r = 0; r < 4; ++r) L.u.o[4 * g + r][j % OCOL16] = O[r];
        if (cb % 2 == 1) {
            wave_sync();
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int t = (lane >> 3) + 8 * half, c4 = (lane & 7) * 4;
                const f32x4 x = *(const f32x4 *)&L.u.o[t][c4];
                if (t < n_tok)
                    __builtin_nontemporal_store(x, (f32x4 *)(olane + half * 8 * tok_elems + 16 * cb - 16));
            }
        }

        // W (tokens 4 g + r, units of sig) in two bf16 parts (hi + mid)
        const uint32_t hi01 = pk_bf16(W[0], W[1]), hi23 = pk_bf16(W[2], W[3]);
        const float r0 = W[0] - lo_f32(hi01), r1 = W[1] - hi_f32(hi01);
        const float r2 = W[2] - lo_f32(hi23), r3 = W[3] - hi_f32(hi23);
        const uint32_t md01 = pk_bf16(r0, r1), md23 = pk_bf16(r2, r3);
        const s16x4 BH = __builtin_bit_cast(s16x4, u32x2{hi01, hi23});
        const s16x4 BM = __builtin_bit_cast(s16x4, u32x2{md01, md23});
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            acc[rt] = mfma_bf16_k16(AU[rt], BH, acc[rt]);
            acc[rt] = mfma_bf16_k16(AU[rt], BM, acc[rt]);
        }

        // ---- re-encode the column ----
        float am = 0.f;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) am = fmaxf(am, fabsf(acc[rt][r]));
        am = xor_max(am, 16);
        am = xor_max(am, 32);
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
    }
}

template <int DK, bool ERR>
__global__ void __launch_bounds__(64 * TPB16) __attribute__((amdgpu_waves_per_eu(3))) decode_mfma16_kernel(MfmaArgs a) {
    __shared__ Tile16Lds tl[TPB16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = xcd_block(blockIdx.x, a.xcd_run, a.xcd_full) * TPB16 + wave;
    if (w >= a.tiles) return;
    const int b = w / a.p.H, h = w - b * a.p.H;
    const int m = a.p.head_map[h];
    if ((m >> 16) == 8)
        process_tile16<DK, 8, ERR>(a, tl[wave], b, h, m & 0xffff, lane);
    else
        process_tile16<DK, 4, ERR>(a, tl[wave], b, h, m & 0xffff, lane);
}

}  // namespace

hipError_t launch_decode_mfma16(const MfmaArgs &args, hipStream_t s) {
    MfmaArgs a = args;
    set_xcd_order(a, TPB16);
    dim3 grid((a.tiles + TPB16 - 1) / TPB16), block(64 * TPB16);
    const bool err = a.p.colerr != nullptr;
    if (a.p.dk == 128) {
        if (err)
            hipLaunchKernelGGL((decode_mfma16_kernel<128, true>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((decode_mfma16_kernel<128, false>), grid, block, 0, s, a);
    } else {
        if (err)
            hipLaunchKernelGGL((decode_mfma16_kernel<64, true>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((decode_mfma16_kernel<64, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace pace
