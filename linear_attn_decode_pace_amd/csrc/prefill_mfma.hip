// Prompt prefill into the quantized state (gfx950): a period of n_tok tokens,
// any n_tok >= 1, applied to every (sequence, head) state in float32 and
// encoded once at the end (the prefill hand-off: chunked kernels already keep
// the state in high precision across a chunk, and periodic rounding extends
// that to decode: 'PACE: four-bit recurrent state by rounding less often',
// TL;DR point (1)).
//
// Chunks of 32 tokens in the WY / UT form, split into two 16-token halves H1,
// H2 (one MFMA tile of rows each).  One workgroup per state tile, resident
// for the whole prompt:
//   * NCB consumer waves (one per 16-column block) hold the tile's float32
//     state in registers from the first token to the final encode;
//   * two producer waves, on different SIMDs, take alternate chunks.  A
//     producer copies a chunk's keys, queries and gates from HBM straight
//     into LDS (no registers) one interval before it needs them, computes
//     the chunk's Gram blocks and gates (phase A) two chunks ahead of the
//     consumers, then its UT solve and Lq T (phase B) one chunk ahead (four
//     chunk buffers in LDS).  The token matrices are block lower triangular:
//     the diagonal blocks of T come from forward substitution, the
//     off-diagonal one from T21 = -T22 A21 T11;
//   * the consumers read their own v values straight from the inputs, one
//     chunk ahead, build the next chunk's key table by state row, and write
//     the outputs;
//   * one workgroup barrier per chunk, ordering LDS only (global loads and
//     stores stay in flight across it).
// Per chunk and column block:
//   P_K = K M0 and P_Q = Q M0 with M0 in two bf16 parts (hi + mid, 16
//   significant bits: ~1e-5 relative error, far below the final encode's
//   rounding; tie flips of the 4096-token parity cases did not change);
//   X = V - diag(g) P_K; W = diag(G') T X on float32 MFMA; Lq T X on bf16
//   MFMA over two parts of each factor (outputs only: ~1e-5 relative error);
//   O = Lq T X + diag(g) P_Q; M <- g_C M + K^T W (bf16 MFMA, W in two
//   parts, each a 32-deep product over the chunk's tokens).
// While a chunk is applied, lane group g of a consumer holds state rows
// 32 ks + 8 g .. 32 ks + 8 g + 7 of each 32-row slice ks, so its MFMA k-slots
// are eight adjacent key columns (one 16-byte LDS read); the stored pool
// layout is restored for the final encode.  Outputs of a chunk go through
// double-buffered LDS and leave as whole rows.
#include <type_traits>

#include "mfma_common.h"
#include "pace_prefill.h"

namespace pace {
namespace {

// Workgroup barrier for LDS hand-offs only: global loads and stores stay in
// flight across it (a plain __syncthreads waits for every outstanding one)
__device__ inline void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The producers' side of the same barrier.  A memory fence would also wait
// for the producer's buffer-to-LDS loads still in flight (they write LDS),
// which are meant to land an interval later; this waits for its LDS
// instructions only and keeps the compiler from moving memory accesses
// across it.
__device__ inline void producer_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Hide a value's origin from the optimiser: lane-dependent masks, constants
// and offsets are then recomputed where they are used instead of being
// hoisted out of the chunk loop, where they would hold registers for the
// whole prompt.
__device__ inline void launder(int &x) { asm volatile("" : "+v"(x)); }

constexpr int CT = 32;      // tokens per chunk
constexpr int HT = 16;      // tokens per half chunk
constexpr int OPAD = 132;   // floats per LDS output row
constexpr int KS = 18;      // row stride of the Gram / gate blocks (column reads stay
                            // free of bank conflicts)

// 16-byte piece p of key / query row `row` sits in LDS slot p ^ kq_swz(row):
// the 16 rows one MFMA operand read touches then fall in 16 different bank
// groups
template <int DK>
__device__ inline int kq_swz(int row) {
    return DK == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int DK>
__device__ inline u32x4 kq_piece(const uint16_t (*kq)[DK], int row, int p) {
    return *(const u32x4 *)&kq[row][8 * (p ^ kq_swz<DK>(row))];
}

// State row held by MFMA row m of row tile rt in the chunk layout
__device__ inline int chunk_row(int rt, int m) {
    return 32 * (rt >> 1) + 8 * (m >> 2) + 4 * (rt & 1) + (m & 3);
}

// Blocks of a chunk's lower-triangular token matrices: 0 = (H1, H1),
// 1 = (H2, H1), 2 = (H2, H2).
template <int DK>
struct alignas(16) ChunkLds {
    uint16_t kq[2 * CT][DK];  // rows 0..31: k_t, rows 32..63: q_t (bf16, pieces swizzled)
    float TGt[3][HT][HT];     // TGt[b][s][t] = G'_t T_b[t][s]   (diag(G') T, transposed)
    // Lq T in two bf16 parts (hi, mid), as MFMA A operands whose k-slot
    // 4 g + e (16 slots) / 8 g + e (32 slots) is token 4 e + g of the chunk:
    // LqB1[p][t][.] the (H1, H1) block for the first half's outputs,
    // LqB2[p][t][.] the (H2, H1) and (H2, H2) blocks for the second half's
    uint16_t LqB1[2][HT][HT];
    uint16_t LqB2[2][HT][2 * HT];
    float gam[CT];            // gamma_t = alpha_0 ... alpha_t
    float ab[2 * CT];         // alpha_t, then beta_t (padding tokens: 1, 0)
};

struct alignas(16) PrepScratch {
    float gh[2][HT];    // per half: alpha products from the half's start to t
    float gch[2][HT];   // per half: alpha products over (t, half end]
    float gcp[CT];      // G'_t = alpha products over (t, chunk end]
    float kk[3][HT][KS];  // k_t . k_s per block, then A in place
    float qk[3][HT][KS];  // q_t . k_s per block, then Lq in place
    float T[3][HT][HT];   // T blocks, natural layout (block 1 holds A21 T11 first)
};

constexpr int NBUF = 4;  // chunk buffers: applied, prepared (B), prepared (A), loading
constexpr int NPROD = 2; // producer waves

template <int DK>
struct PrefillLds {
    ChunkLds<DK> ch[NBUF];
    // keys by state row for K^T W, built by the consumers one chunk ahead
    // (double buffered): row i holds, per group gg, k[i] of tokens
    // 4 gg .. 4 gg + 3 and 16 + 4 gg .. 16 + 4 gg + 3 (16 bytes), the groups
    // in the order gg ^ ((i / 8) % 4) (conflict-free reads)
    alignas(16) uint16_t kt[2][DK][32];
    PrepScratch ps[NPROD];
    alignas(16) float o[2][CT][OPAD];
};

struct PrefillArgs {
    PoolView p;
    const uint16_t *q, *k, *v;
    const float *alpha, *beta;
    float *out;  // NULL: no outputs
    int n_tok;
    int tiles;
};

// Element x of token t (inside a chunk) of a token-major [T, B, H, d] tensor,
// from that chunk's base: 32-bit lane offsets when a chunk's whole span fits
// in 32 bits (WIDE_OFF = false, fewer instructions in the chunk loop), 64-bit
// otherwise.
template <bool WIDE_OFF, int DK, class T>
__device__ inline T *tok_at(T *base, int t, const PrefillArgs &a, uint32_t x) {
    if constexpr (WIDE_OFF) {
        return base + (size_t)t * ((size_t)a.p.B * (size_t)a.p.H) * DK + x;
    } else {
        const uint32_t tok_stride = (uint32_t)a.p.B * (uint32_t)a.p.H;
        return at(base, (uint32_t)(t * tok_stride * DK + x) * (uint32_t)sizeof(T));
    }
}

// Producer: copy chunk c's k and q rows and its alpha / beta from HBM into
// LDS (buffer-to-LDS loads: lane l of each instruction fills 16 bytes at
// 16 l).  Tokens past the prompt repeat its last token; phase A resets their
// gates.
template <int DK>
__device__ __attribute__((always_inline)) inline void issue_chunk(const PrefillArgs &a, ChunkLds<DK> &N,
                                                                  size_t tile_row, int c, int lane,
                                                                  bool wide) {
    launder(lane);
    constexpr int SPR = DK / 8;    // 16-byte slots per row
    constexpr int RPI = 64 / SPR;  // rows per instruction
    // rows per token (32-bit arithmetic unless the launch needs 64-bit offsets)
    const size_t tok_stride = wide ? (size_t)a.p.B * (size_t)a.p.H
                                   : (size_t)((uint32_t)a.p.B * (uint32_t)a.p.H);
    const int t0 = CT * c, last = a.n_tok - 1 - t0;
    const size_t base = ((size_t)t0 * tok_stride + tile_row) * DK;
#pragma unroll
    for (int it = 0; it < 2 * CT / RPI; ++it) {
        const int row = it * RPI + lane / SPR, slot = lane % SPR;
        const int which = (it * RPI) / CT;  // k rows, then q rows
        const int t = min(row & (CT - 1), last);
        const int piece = slot ^ kq_swz<DK>(row);
        const uint16_t *src = (which == 0 ? a.k : a.q) + base;
        const uint16_t *at_t = wide ? tok_at<true, DK>(src, t, a, 8 * piece)
                                    : tok_at<false, DK>(src, t, a, 8 * piece);
        __builtin_amdgcn_global_load_lds(at_t,
                                         (__attribute__((address_space(3))) void *)&N.kq[it * RPI][0], 16, 0, 0);
    }
    const int t = min(lane & (CT - 1), last);
    const float *gsrc = (lane < CT ? a.alpha : a.beta) + ((size_t)t0 + t) * tok_stride + tile_row;
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)&N.ab[0], 4, 0, 0);
}

// kk[t][s] = k_{t0+t} . k_{s0+s}, qk[t][s] = q_{t0+t} . k_{s0+s} for one
// 16 x 16 block: the A row m is token t0 + 4 (m % 4) + m / 4, so output row
// 4 g + r is token t0 + 4 r + g
template <int DK>
__device__ inline void gram_block(const uint16_t (*kq)[DK], int t0, int s0, float (*kk)[KS],
                                  float (*qk)[KS], int lane) {
    constexpr int NKS = DK / 32;
    const int g = lane >> 4, n = lane & 15;
    const int tok_n = 4 * (n & 3) + (n >> 2);
    f32x4 GK = {0.f, 0.f, 0.f, 0.f}, GQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const int p = 4 * ks + g;
        const bf16x8 AK = __builtin_bit_cast(bf16x8, kq_piece<DK>(kq, t0 + tok_n, p));
        const bf16x8 AQ = __builtin_bit_cast(bf16x8, kq_piece<DK>(kq, CT + t0 + tok_n, p));
        const bf16x8 BS = __builtin_bit_cast(bf16x8, kq_piece<DK>(kq, s0 + n, p));
        GK = mfma_bf16_k32(AK, BS, GK);
        GQ = mfma_bf16_k32(AQ, BS, GQ);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        kk[4 * r + g][n] = GK[r];
        qk[4 * r + g][n] = GQ[r];
    }
}

// D += X Y for 16 x 16 float matrices on float32 MFMA (output row 4 g + r,
// column n), and D += (X Y)^T
template <int XS, int YS>
__device__ inline f32x4 mm16(const float (*X)[XS], const float (*Y)[YS], f32x4 D, int lane) {
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int st = 0; st < 4; ++st) D = mfma_f32_k4(X[n][4 * st + g], Y[4 * st + g][n], D);
    return D;
}
template <int XS, int YS>
__device__ inline f32x4 mm16t(const float (*X)[XS], const float (*Y)[YS], f32x4 D, int lane) {
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int st = 0; st < 4; ++st) D = mfma_f32_k4(Y[4 * st + g][n], X[n][4 * st + g], D);
    return D;
}

// x from the lane CTRL names inside the lane's row of 16 (a DPP row shift),
// 1 where that lane lies outside the row
template <int CTRL>
__device__ inline float row_shift_or_one(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// A = strictly lower (Gamma * kk), Lq = lower (Gamma * qk) of one diagonal
// block in place: lane -> row t = lane / 4, columns s0 .. s0 + 3 with
// s0 = 4 (lane % 4); Gamma_{t, s0+3} as one masked product, then the running
// product down to s0
__device__ inline void diag_gates(const float *alpha, float (*kk)[KS], float (*qk)[KS], int lane) {
    float al[HT];
#pragma unroll
    for (int r = 0; r < HT; ++r) al[r] = alpha[r];
    const int t = lane >> 2, s0 = 4 * (lane & 3);
    float gts = 1.f;
#pragma unroll
    for (int r = 1; r < HT; ++r) gts *= (r > s0 + 3 && r <= t) ? al[r] : 1.f;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
        const int s = s0 + e;
        kk[t][s] = s < t ? gts * kk[t][s] : 0.f;
        qk[t][s] = s <= t ? gts * qk[t][s] : 0.f;
        if (e > 0 && s <= t) gts *= alpha[s];  // Gamma_{t,s-1} = Gamma_{t,s} alpha_s
    }
}

// Producer, phase A: Gram blocks and gates of a loaded chunk.
//   Gamma_{t,s} = prod_{s<r<=t} alpha_r; inside a half from its own gates,
//   across the halves Gamma_{16+t, s} = gch[0][s] gh[1][t].  The per-half
//   prefix products gh and the products over the rest of the half gch come
//   from DPP scans (lane l: token l % 32, one half per row of 16 lanes).
template <int DK>
__device__ __attribute__((always_inline)) inline void prep_a(ChunkLds<DK> &L, PrepScratch &S, int lane) {
    launder(lane);
    wave_sync();
    gram_block<DK>(L.kq, 0, 0, S.kk[0], S.qk[0], lane);
    gram_block<DK>(L.kq, HT, 0, S.kk[1], S.qk[1], lane);
    gram_block<DK>(L.kq, HT, HT, S.kk[2], S.qk[2], lane);
    {
        const float al = L.ab[lane & (CT - 1)];
        float pre = al, suf = al;
        pre *= row_shift_or_one<0x111>(pre);  // row_shr:1
        pre *= row_shift_or_one<0x112>(pre);
        pre *= row_shift_or_one<0x114>(pre);
        pre *= row_shift_or_one<0x118>(pre);
        suf *= row_shift_or_one<0x101>(suf);  // row_shl:1
        suf *= row_shift_or_one<0x102>(suf);
        suf *= row_shift_or_one<0x104>(suf);
        suf *= row_shift_or_one<0x108>(suf);
        const float after = row_shift_or_one<0x101>(suf);  // product over (t, half end]
        const float tot1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pre), HT - 1));
        const float tot2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pre), CT - 1));
        if (lane < CT) {
            const int hb = lane >> 4, t = lane & 15;
            S.gh[hb][t] = pre;
            S.gch[hb][t] = after;
            L.gam[lane] = hb ? tot1 * pre : pre;
            S.gcp[lane] = hb ? after : after * tot2;
        }
    }
    wave_sync();
    diag_gates(L.ab, S.kk[0], S.qk[0], lane);
    diag_gates(L.ab + HT, S.kk[2], S.qk[2], lane);
    {
        const int t = lane >> 2, s0 = 4 * (lane & 3);
        const float gt = S.gh[1][t];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float f = gt * S.gch[0][s0 + e];
            S.kk[1][t][s0 + e] *= f;
            S.qk[1][t][s0 + e] *= f;
        }
    }
    wave_sync();
}

// x - (low / high bf16 of pk) in one instruction: a bf16 dot product with
// (-1, -0) / (0, -1) accumulated onto x (exact: the difference is a float32).
// The low-half factor is (-1, -0), not (-1, 0): the compiler encodes the
// packed (-1, 0) as the inline constant -1.0, which the dot product applies
// to the high half.
__device__ inline float sub_lo(uint32_t pk, float x) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                           __builtin_bit_cast(bf16x2, 0x8000bf80u), x, false);
}
__device__ inline float sub_hi(uint32_t pk, float x) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                           __builtin_bit_cast(bf16x2, 0xbf800000u), x, false);
}

// bf16 parts (hi, mid, lo) of the four floats x[0..3], as two packed dwords
// each: x = hi + mid + lo exactly (8 + 8 + 8 significant bits)
__device__ inline void split3(const f32x4 &x, uint32_t hi[2], uint32_t md[2], uint32_t lo[2]) {
    hi[0] = pk_bf16(x[0], x[1]);
    hi[1] = pk_bf16(x[2], x[3]);
    const float r0 = sub_lo(hi[0], x[0]), r1 = sub_hi(hi[0], x[1]);
    const float r2 = sub_lo(hi[1], x[2]), r3 = sub_hi(hi[1], x[3]);
    md[0] = pk_bf16(r0, r1);
    md[1] = pk_bf16(r2, r3);
    lo[0] = pk_bf16(sub_lo(md[0], r0), sub_hi(md[0], r1));
    lo[1] = pk_bf16(sub_lo(md[1], r2), sub_hi(md[1], r3));
}

// bf16 parts (hi, mid) of the four floats x[0..3]: x = hi + mid to 16
// significant bits
__device__ inline void split2(const f32x4 &x, uint32_t hi[2], uint32_t md[2]) {
    hi[0] = pk_bf16(x[0], x[1]);
    hi[1] = pk_bf16(x[2], x[3]);
    md[0] = pk_bf16(sub_lo(hi[0], x[0]), sub_hi(hi[0], x[1]));
    md[1] = pk_bf16(sub_lo(hi[1], x[2]), sub_hi(hi[1], x[3]));
}

// Producer, part 4 (phase B): T = (I + diag(beta) A)^-1 diag(beta) block by
// block, diag(G') T and Lq T for the consumers.
template <int DK>
__device__ __attribute__((always_inline)) inline void prep_b(ChunkLds<DK> &L, PrepScratch &S, int lane) {
    launder(lane);
    const int g = lane >> 4, n = lane & 15;
    {
        // diagonal blocks by forward substitution, one column s per lane:
        // lanes 0..15 the first half, lanes 32..47 the second (lanes 16..31
        // and 48..63 repeat them and store nothing)
        const int hb = lane >> 5, s = lane & 15;
        const float(*A)[KS] = S.kk[2 * hb];
        const float *be_p = L.ab + CT + HT * hb;
        float be[HT], z[HT];
#pragma unroll
        for (int r = 0; r < HT; ++r) be[r] = be_p[r];
#pragma unroll
        for (int t = 0; t < HT; ++t) {
            float sum = 0.f;
#pragma unroll
            for (int u = 0; u < t; ++u) sum = fmaf(A[t][u], z[u], sum);
            z[t] = (t == s ? 1.f : 0.f) - be[t] * sum;
        }
        if ((lane & 31) < HT) {
            const float bs = be_p[s];
            float(*T)[HT] = S.T[2 * hb];
            float(*TG)[HT] = L.TGt[2 * hb];
            const float *gp = S.gcp + HT * hb;
#pragma unroll
            for (int t = 0; t < HT; ++t) T[t][s] = z[t] * bs;
#pragma unroll
            for (int q = 0; q < HT / 4; ++q)
                *(f32x4 *)&TG[s][4 * q] = f32x4{gp[4 * q] * z[4 * q] * bs, gp[4 * q + 1] * z[4 * q + 1] * bs,
                                                gp[4 * q + 2] * z[4 * q + 2] * bs,
                                                gp[4 * q + 3] * z[4 * q + 3] * bs};
        }
    }
    wave_sync();
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // T21 = -T22 (A21 T11): block 1 of T holds A21 T11 until T21 replaces it
    f32x4 D = mm16(S.kk[1], S.T[0], zero, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) S.T[1][4 * g + r][n] = D[r];
    wave_sync();
    D = mm16(S.T[2], S.T[1], zero, lane);
    wave_sync();  // A21 T11 is read before T21 replaces it
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float x = -D[r];
        S.T[1][4 * g + r][n] = x;
        L.TGt[1][n][4 * g + r] = S.gcp[HT + 4 * g + r] * x;
    }
    wave_sync();
    // Lq T block by block: this lane holds (Lq T)[t = n][s = 4 g + r] of the
    // block (computed transposed), stored as hi and mid bf16 parts at the
    // k-slot of token s
    auto put = [&](uint16_t *hi_row, uint16_t *mid_row, int slot0, int slot_r, const f32x4 &x) {
        uint32_t h[2], m[2], l[2];
        split3(x, h, m, l);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hi_row[slot0 + slot_r * r] = (uint16_t)(h[r >> 1] >> (16 * (r & 1)));
            mid_row[slot0 + slot_r * r] = (uint16_t)(m[r >> 1] >> (16 * (r & 1)));
        }
    };
    D = mm16t(S.qk[0], S.T[0], zero, lane);
    put(L.LqB1[0][n], L.LqB1[1][n], g, 4, D);          // s = 4 g + r -> slot 4 r + g
    D = mm16t(S.qk[2], S.T[2], zero, lane);
    put(L.LqB2[0][n], L.LqB2[1][n], 4 + g, 8, D);      // s = 16 + 4 g + r -> slot 8 r + 4 + g
    D = mm16t(S.qk[2], S.T[1], mm16t(S.qk[1], S.T[0], zero, lane), lane);
    put(L.LqB2[0][n], L.LqB2[1][n], g, 8, D);          // s = 4 g + r -> slot 8 r + g
    wave_sync();
}

// Chunk layout <-> pool layout of a column block's state (lane (g, n); four
// rows per register quad).  Pool layout: acc[2 ks + h][r] is row
// 32 ks + 16 h + 4 g + r; chunk layout: acc[2 ks + h][r] is row
// 32 ks + 8 g + 4 h + r.  Rows move between the four lane groups of column
// n (ds_bpermute), once at the start of a prompt and once before the encode.
template <int NKS>
__device__ inline void to_chunk_layout(f32x4 *acc, int lane) {
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const f32x4 a0 = acc[2 * ks], a1 = acc[2 * ks + 1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int src = 4 * ((((2 * g + h) & 3) << 4) | n);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x0 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(a0[r])));
                const float x1 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(a1[r])));
                acc[2 * ks + h][r] = (g >> 1) ? x1 : x0;
            }
        }
    }
}
template <int NKS>
__device__ inline void to_pool_layout(f32x4 *acc, int lane) {
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const f32x4 c0 = acc[2 * ks], c1 = acc[2 * ks + 1];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int src = 4 * (((2 * t + (g >> 1)) << 4) | n);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x0 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(c0[r])));
                const float x1 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(c1[r])));
                acc[2 * ks + t][r] = (g & 1) ? x1 : x0;
            }
        }
    }
}

template <int DK, int BITS, bool ERR, bool WIDE_OFF>
__device__ void prefill_tile(const PrefillArgs &a, PrefillLds<DK> &L, int b, int h, int slot,
                             int wave, int lane) {
    constexpr int NKS = DK / 32;  // k-slices of 32 rows
    constexpr int NRT = DK / 16;  // row tiles of 16 rows
    constexpr int NCB = DK / 16;  // column blocks = consumer waves
    constexpr float QMAX = BITS == 4 ? 7.f : 127.f;
    constexpr float KAPPA = Loader<DK, BITS>::KAPPA;
    const int g = lane >> 4, n = lane & 15;
    const size_t tile_row = (size_t)b * a.p.H + h;
    // rows per token: 32-bit arithmetic unless the launch needs 64-bit offsets
    using TokStride = typename std::conditional<WIDE_OFF, size_t, uint32_t>::type;
    const TokStride tok_stride = (TokStride)a.p.B * (TokStride)a.p.H;
    const int n_chunks = (a.n_tok + CT - 1) / CT;
    const bool producer = wave >= NCB;
    const int cb = wave, j = 16 * cb + n;

    uint8_t *codes = BITS == 4
        ? a.p.codes4 + ((size_t)b * a.p.n4 + slot) * tile_code_bytes(DK, DK, 4)
        : a.p.codes8 + ((size_t)b * a.p.n8 + slot) * tile_code_bytes(DK, DK, 8);
    float *scl = a.p.scales + tile_row * DK;

    if (producer) {
        // Two producers take alternate chunks.  Chunk c's tokens are copied
        // into LDS during interval c - 3 (at the start of phase B of chunk
        // c - 2, by the same producer), its Gram blocks and gates computed
        // (phase A) while the consumers apply chunk c - 2, its UT solve and
        // Lq T (phase B) while they apply chunk c - 1.  Each producer
        // alternates A and B, so both carry half of the work every interval,
        // on different SIMDs; a producer's only memory operations are its
        // own buffer-to-LDS loads, so waiting for them all at the start of
        // phase A waits for nothing else.  Phase B (the forward substitution
        // is a long serial chain) runs at raised wave priority, ahead of the
        // consumers sharing its SIMD.
        const int p = wave - NCB;
        PrepScratch &ps = L.ps[p];
        auto phase_a = [&](int c) {
            ChunkLds<DK> &N = L.ch[c % NBUF];
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): chunk c is in LDS
            const int nv = a.n_tok - CT * c;
            if (lane < CT && lane >= nv) {  // padding tokens leave the state alone
                N.ab[lane] = 1.f;
                N.ab[CT + lane] = 0.f;
            }
            prep_a<DK>(N, ps, lane);
        };
        auto phase_b = [&](int c) {
            if (c + NPROD < n_chunks) issue_chunk<DK>(a, L.ch[(c + NPROD) % NBUF], tile_row, c + NPROD, lane, WIDE_OFF);
            __builtin_amdgcn_s_setprio(3);
            prep_b<DK>(L.ch[c % NBUF], ps, lane);
            __builtin_amdgcn_s_setprio(0);
        };
        if (p < n_chunks) {
            issue_chunk<DK>(a, L.ch[p], tile_row, p, lane, WIDE_OFF);
            phase_a(p);
            if (p == 0) phase_b(0);
        }
        producer_barrier();
        producer_barrier();  // the consumers' key table of chunk 0
        for (int c = 0; c < n_chunks; ++c) {
            // this interval: phase B of chunk c + 1 (after issuing chunk
            // c + 3's loads) or phase A of chunk c + 2
            if ((c + 1) % NPROD == p) {
                if (c + 1 < n_chunks) phase_b(c + 1);
            } else if (c + 2 < n_chunks) {
                phase_a(c + 2);
            }
            producer_barrier();  // chunk c+1 prepared, chunk c's outputs complete
        }
        return;
    }

    // the column block's starting state: the stored codes decoded (zero after
    // a zero initialisation), in chunk layout
    f32x4 acc[NRT];
    {
        Loader<DK, BITS> ld;
        ld.load(codes, cb, lane);
        ld.codes_f32(acc);
        const float sk = scl[j] * (1.f / KAPPA);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) acc[rt] *= sk;
        to_chunk_layout<NKS>(acc, lane);
    }
    // Output flush of chunk c by the consumers after the barrier that closes
    // it: rows of DK floats, 16 bytes per lane.  Staging buffer c & 1 is
    // written again only in chunk c + 2, after the next barrier, by which
    // every consumer has finished this flush.
    auto flush = [&](int c, int ln) {
        if (!a.out) return;
        constexpr int PER_ROW = DK / 4;          // lanes per output row
        constexpr int ROWS = 64 * NCB / PER_ROW; // rows per pass
        const int e = wave * 64 + ln;
        const int nv = a.n_tok - CT * c;
        float *obase = a.out + ((size_t)CT * c * tok_stride + tile_row) * DK;
#pragma unroll
        for (int t0 = 0; t0 < CT; t0 += ROWS) {
            const int t = t0 + e / PER_ROW, c4 = (e % PER_ROW) * 4;
            if (t < nv) {  // chunk c's real tokens
                const f32x4 x = *(const f32x4 *)&L.o[c & 1][t][c4];
                __builtin_nontemporal_store(x, (f32x4 *)tok_at<WIDE_OFF, DK>(obase, t, a, c4));
            }
        }
    };

    lds_barrier();
    // this wave's 16 rows of a chunk's key table: lane -> (state row, token group)
    auto build_kt = [&](const ChunkLds<DK> &N, uint16_t (*KT)[32], int ln) {
        const int i = 16 * wave + (ln >> 2), gg = ln & 3;
        uint32_t w[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int t = HT * hh + 4 * gg;
            uint32_t e[4];
#pragma unroll
            for (int x = 0; x < 4; ++x)
                e[x] = N.kq[t + x][8 * ((i >> 3) ^ kq_swz<DK>(t + x)) + (i & 7)];
            w[2 * hh] = e[0] | (e[1] << 16);
            w[2 * hh + 1] = e[2] | (e[3] << 16);
        }
        *(u32x4 *)&KT[i][8 * (gg ^ ((i >> 3) & 3))] = u32x4{w[0], w[1], w[2], w[3]};
    };
    build_kt(L.ch[0], L.kt[0], lane);
    lds_barrier();
    // this lane's v values: tokens 4 e + g of a chunk (e = 0..7), column j,
    // read from the inputs one chunk ahead
    // Every chunk issues the same eight loads (past the prompt they repeat
    // its last token: padding tokens have beta = 0, so their v never
    // reaches the state or a real output), which keeps the count of memory
    // operations static and the compiler's waits for them exact.
    auto load_v = [&](int c, uint16_t (&vv)[8], int g, int j) {
        const int cc = min(c, n_chunks - 1), last = a.n_tok - 1 - CT * cc;
        const uint16_t *vbase = a.v + ((size_t)CT * cc * tok_stride + tile_row) * DK;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = min(4 * e + g, last);
            vv[e] = *tok_at<WIDE_OFF, DK>(vbase, t, a, j);
        }
    };
    // v values of the chunk being applied and of the next one, in two
    // register sets that swap roles every chunk (the loop is unrolled by two,
    // so no copies: a copy would have to wait for the loads, and a wait for
    // loads may mean a wait for every memory operation issued after them)
    uint16_t va[8], vb[8];
    load_v(0, va, g, j);
    // the first chunk's v values are waited for here, so that inside the loop
    // the compiler's wait for them is not merged with the prologue's loads
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    auto step = [&](int c, const uint16_t (&vcur)[8], uint16_t (&vnext)[8]) __attribute__((always_inline)) {
        // lane-derived offsets are recomputed per chunk rather than held
        // across the loop (register pressure)
        int ln = lane;
        launder(ln);
        const int g = ln >> 4, n = ln & 15, j = 16 * cb + n;
        // A operand rows: the K blocks' row m is token 4 (m % 4) + m / 4 of
        // its half, so P_K's row 4 g + r is token 4 r + g (the B layout of the
        // float32 chunk MFMAs); the Q blocks' row m is token m, so P_Q's rows
        // line up with O's
        const int tok_n = 4 * (n & 3) + (n >> 2);
        load_v(c + 1, vnext, g, j);
        const ChunkLds<DK> &C = L.ch[c % NBUF];
        const uint16_t(*KT)[32] = L.kt[c & 1];
        if (c + 1 < n_chunks) build_kt(L.ch[(c + 1) % NBUF], L.kt[(c + 1) & 1], ln);
        {
            // P_K = K M0 and P_Q = Q M0 over two bf16 parts of M0 (hi + mid,
            // 16 significant bits; a third part for P_K cost 8 more MFMAs
            // per chunk and 5% of the time without moving a code), both
            // halves of the chunk; k-slot 8 g + e is state row 32 ks + 8 g + e
            f32x4 PK1 = {0.f, 0.f, 0.f, 0.f}, PK2 = PK1, PQ1 = PK1, PQ2 = PK1;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int pc = 4 * ks + g;
                const bf16x8 AK1 = __builtin_bit_cast(bf16x8, kq_piece<DK>(C.kq, tok_n, pc));
                const bf16x8 AK2 = __builtin_bit_cast(bf16x8, kq_piece<DK>(C.kq, HT + tok_n, pc));
                const bf16x8 AQ1 = __builtin_bit_cast(bf16x8, kq_piece<DK>(C.kq, CT + n, pc));
                const bf16x8 AQ2 = __builtin_bit_cast(bf16x8, kq_piece<DK>(C.kq, CT + HT + n, pc));
                uint32_t h0[2], m0[2], h1[2], m1[2];
                split2(acc[2 * ks], h0, m0);
                split2(acc[2 * ks + 1], h1, m1);
                const bf16x8 BH = __builtin_bit_cast(bf16x8, u32x4{h0[0], h0[1], h1[0], h1[1]});
                const bf16x8 BM = __builtin_bit_cast(bf16x8, u32x4{m0[0], m0[1], m1[0], m1[1]});
                PK1 = mfma_bf16_k32(AK1, BH, PK1);
                PK2 = mfma_bf16_k32(AK2, BH, PK2);
                PQ1 = mfma_bf16_k32(AQ1, BH, PQ1);
                PQ2 = mfma_bf16_k32(AQ2, BH, PQ2);
                PK1 = mfma_bf16_k32(AK1, BM, PK1);
                PK2 = mfma_bf16_k32(AK2, BM, PK2);
                PQ1 = mfma_bf16_k32(AQ1, BM, PQ1);
                PQ2 = mfma_bf16_k32(AQ2, BM, PQ2);
            }
            // X for tokens 4 r + g and 16 + 4 r + g (the P_K rows this lane holds)
            float X1[4], X2[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                X1[r] = fmaf(-C.gam[4 * r + g], PK1[r], bf2f(vcur[r]));
                X2[r] = fmaf(-C.gam[HT + 4 * r + g], PK2[r], bf2f(vcur[4 + r]));
            }
            // W = diag(G') T X on float32 MFMA (rows = tokens; step st takes
            // token 4 st + g of each half): the state needs its accuracy
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            f32x4 W1 = zero, W2 = zero;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int s = 4 * st + g;
                W1 = mfma_f32_k4(C.TGt[0][s][n], X1[st], W1);
                W2 = mfma_f32_k4(C.TGt[1][s][n], X1[st], W2);
            }
#pragma unroll
            for (int st = 0; st < 4; ++st) W2 = mfma_f32_k4(C.TGt[2][4 * st + g][n], X2[st], W2);
            // Lq T X on bf16 MFMA with X and Lq T in two parts each (hi hi,
            // hi mid, mid hi: ~1e-5 relative error, outputs only); the
            // lane's k-slots are its own tokens 4 e + g
            uint32_t xh[4], xm[4];
            {
                const f32x4 x1 = {X1[0], X1[1], X1[2], X1[3]}, x2 = {X2[0], X2[1], X2[2], X2[3]};
                uint32_t l_[2];
                split3(x1, xh, xm, l_);
                split3(x2, xh + 2, xm + 2, l_);
            }
            const s16x4 B1h = __builtin_bit_cast(s16x4, u32x2{xh[0], xh[1]});
            const s16x4 B1m = __builtin_bit_cast(s16x4, u32x2{xm[0], xm[1]});
            const bf16x8 B2h = __builtin_bit_cast(bf16x8, u32x4{xh[0], xh[1], xh[2], xh[3]});
            const bf16x8 B2m = __builtin_bit_cast(bf16x8, u32x4{xm[0], xm[1], xm[2], xm[3]});
            const s16x4 A1h = __builtin_bit_cast(s16x4, *(const u32x2 *)&C.LqB1[0][n][4 * g]);
            const s16x4 A1m = __builtin_bit_cast(s16x4, *(const u32x2 *)&C.LqB1[1][n][4 * g]);
            const bf16x8 A2h = __builtin_bit_cast(bf16x8, *(const u32x4 *)&C.LqB2[0][n][8 * g]);
            const bf16x8 A2m = __builtin_bit_cast(bf16x8, *(const u32x4 *)&C.LqB2[1][n][8 * g]);
            f32x4 O1 = mfma_bf16_k16(A1h, B1h, zero);
            f32x4 O2 = mfma_bf16_k32(A2h, B2h, zero);
            O1 = mfma_bf16_k16(A1h, B1m, O1);
            O2 = mfma_bf16_k32(A2h, B2m, O2);
            O1 = mfma_bf16_k16(A1m, B1h, O1);
            O2 = mfma_bf16_k32(A2m, B2h, O2);
            // O += diag(gamma) Q M0: rows 4 g + r of O and P_Q are the same tokens
            const f32x4 gq1 = *(const f32x4 *)&C.gam[4 * g];
            const f32x4 gq2 = *(const f32x4 *)&C.gam[HT + 4 * g];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                L.o[c & 1][4 * g + r][j] = fmaf(gq1[r], PQ1[r], O1[r]);
                L.o[c & 1][HT + 4 * g + r][j] = fmaf(gq2[r], PQ2[r], O2[r]);
            }

            // M <- gamma_C M + K^T W, W in two bf16 parts (hi + mid, relative
            // error below 2^-17; a third part cost 8 more MFMAs per chunk and
            // 3% of the time): the lane's k-slots
            // are tokens 4 g .. 4 g + 3 (first half) and 16 + 4 g .. 16 + 4 g + 3
            // (second half), one 32-deep product per part; MFMA row m of row
            // tile rt is state row chunk_row(rt, m)
            const float gC = C.gam[CT - 1];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) acc[rt] *= gC;
            uint32_t h1[2], m1[2], h2[2], m2[2];
            split2(W1, h1, m1);
            split2(W2, h2, m2);
            const bf16x8 BH = __builtin_bit_cast(bf16x8, u32x4{h1[0], h1[1], h2[0], h2[1]});
            const bf16x8 BM = __builtin_bit_cast(bf16x8, u32x4{m1[0], m1[1], m2[0], m2[1]});
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const int R = chunk_row(rt, n);
                const bf16x8 A2 = __builtin_bit_cast(bf16x8, *(const u32x4 *)&KT[R][8 * (g ^ ((R >> 3) & 3))]);
                acc[rt] = mfma_bf16_k32(A2, BH, acc[rt]);
                acc[rt] = mfma_bf16_k32(A2, BM, acc[rt]);
            }
        }
        lds_barrier();  // chunk c+1 staged, chunk c's outputs complete
        flush(c, ln);
    };
    for (int c = 0; c < n_chunks; c += 2) {
        step(c, va, vb);
        if (c + 1 < n_chunks) step(c + 1, vb, va);
    }

    // ---- encode each column block once: absmax, scale, codes ----
    to_pool_layout<NKS>(acc, lane);
    {
        float am = 0.f;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) am = fmaxf(am, fabsf(acc[rt][r]));
        am = xor_max(am, 16);
        am = xor_max(am, 32);
        const float s_new = am * (1.f / QMAX);
        const float ratio = s_new > 0.f ? __builtin_amdgcn_rcpf(s_new) : 0.f;
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
        if constexpr (ERR) column_error<NRT>(acc, y, 1.f, s_new, a.p.colerr + (tile_row * DK + j) * 2, g);
    }
}

template <int DK, bool ERR, bool WIDE_OFF>
__global__ void __launch_bounds__(64 * (DK / 16 + NPROD)) prefill_mfma_kernel(PrefillArgs a) {
    __shared__ PrefillLds<DK> L;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = blockIdx.x;  // one tile per workgroup, sequence-major
    const int b = w / a.p.H, h = w - b * a.p.H;
    const int m = a.p.head_map[h];
    if ((m >> 16) == 8)
        prefill_tile<DK, 8, ERR, WIDE_OFF>(a, L, b, h, m & 0xffff, wave, lane);
    else
        prefill_tile<DK, 4, ERR, WIDE_OFF>(a, L, b, h, m & 0xffff, wave, lane);
}

}  // namespace

bool prefill_mfma_supported(int dk, int dv, int in_bf16, long long rows_per_token) {
    // any batch: launches whose chunk span exceeds 32-bit offsets take the
    // 64-bit instantiation
    (void)rows_per_token;
    return in_bf16 && dk == dv && (dk == 128 || dk == 64);
}



hipError_t launch_prefill_mfma(const PoolView &p, int n_tok, const void *q, const void *k,
                               const void *v, const float *alpha, const float *beta, float *out,
                               hipStream_t s) {
    PrefillArgs a;
    a.p = p;
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.alpha = alpha;
    a.beta = beta;
    a.out = out;
    a.n_tok = n_tok;
    a.tiles = p.B * p.H;
    const bool err = p.colerr != nullptr;
    // byte span of one chunk's outputs (float32): 32-bit lane offsets suffice below 2^32
    const bool wide = (unsigned long long)CT * a.tiles * p.dk * sizeof(float) >= (1ull << 32);
    const dim3 grid(a.tiles), block(64 * (p.dk / 16 + NPROD));
#define PACE_PREFILL_LAUNCH(DK_, ERR_, WIDE_) \
    hipLaunchKernelGGL((prefill_mfma_kernel<DK_, ERR_, WIDE_>), grid, block, 0, s, a)
    if (p.dk == 128) {
        if (err)
            {
            if (wide) PACE_PREFILL_LAUNCH(128, true, true);
            else PACE_PREFILL_LAUNCH(128, true, false);
        }
        else
            {
            if (wide) PACE_PREFILL_LAUNCH(128, false, true);
            else PACE_PREFILL_LAUNCH(128, false, false);
        }
    } else {
        if (err)
            {
            if (wide) PACE_PREFILL_LAUNCH(64, true, true);
            else PACE_PREFILL_LAUNCH(64, true, false);
        }
        else
            {
            if (wide) PACE_PREFILL_LAUNCH(64, false, true);
            else PACE_PREFILL_LAUNCH(64, false, false);
        }
    }
#undef PACE_PREFILL_LAUNCH
    return hipGetLastError();
}

}  // namespace pace
