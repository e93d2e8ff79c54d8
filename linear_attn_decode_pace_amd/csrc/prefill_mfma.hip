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
//   * DK / 32 consumer waves, two 16-column blocks each, hold the tile's
//     float32 state in registers from the first token to the final encode
//     (the K, Q, T and Lq operands a chunk reads from LDS serve both blocks,
//     and the two blocks' dependency chains interleave in one wave);
//   * two producer waves, on different SIMDs, take alternate chunks.  A
//     producer copies a chunk's keys, queries, values and gates from HBM
//     straight into LDS (no registers; whole rows, so every byte fetched is
//     used) one interval before it needs them, computes the chunk's Gram
//     blocks, gates and gated blocks A and Lq in registers (phase A) two
//     chunks ahead of the consumers, then the diagonal blocks T11, T22 of
//     the UT transform by forward substitution (phase B) one chunk ahead
//     (four chunk buffers in LDS);
//   * the consumers build the next chunk's key table by state row and write
//     the outputs straight from registers;
//   * one workgroup barrier per chunk, ordering LDS only (global loads and
//     stores stay in flight across it).
// Per chunk and column block (T = (I + diag(beta) A)^-1 diag(beta) is block
// lower triangular, T21 = -T22 A21 T11, and is never formed):
//   P_K = K M0 and P_Q = Q M0 with M0 in two bf16 parts (hi + mid, 16
//   significant bits: ~1e-5 relative error, far below the final encode's
//   rounding; tie flips of the 4096-token parity cases did not change);
//   X = V - diag(g) P_K; Y1 = T11 X1, Y2 = T22 (X2 - A21 Y1) on float32 MFMA
//   (Y = T X); W = diag(G') Y; Lq Y on bf16 MFMA over two parts of each
//   factor (outputs only: ~1e-5 relative error); O = Lq Y + diag(g) P_Q;
//   M <- g_C M + K^T W (bf16 MFMA, W in two parts, each a 32-deep product
//   over the chunk's tokens).
// While a chunk is applied, lane group g of a consumer holds state rows
// 32 ks + 8 g .. 32 ks + 8 g + 7 of each 32-row slice ks, so its MFMA k-slots
// are eight adjacent key columns (one 16-byte LDS read); the stored pool
// layout is restored for the final encode.  P_Q and Lq Y are computed
// transposed (the same MFMAs with A and B swapped), so a lane ends a chunk
// holding four adjacent output columns of one token: 16-byte stores, the
// column blocks of a token filling its row together.
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

// Keep memory accesses on their side of this point (the loads above it stay
// ahead of the work below; their waits are placed at first use)
__device__ inline void compiler_fence() { asm volatile("" ::: "memory"); }

// Make y's next uses come after x is computed (an empty asm that reads x and
// redefines both), so that a register y occupied can be reused in place.
__device__ inline void order_after(f32x4 &x, f32x4 &y) { asm volatile("" : "+v"(x), "+v"(y)); }

constexpr int CT = 32;      // tokens per chunk
constexpr int HT = 16;      // tokens per half chunk

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

// 16-byte piece p of value row t sits in LDS slot p ^ v_swz(t): the four
// rows (tokens 4 r + g, g = 0..3) one consumer read touches then fall in
// different bank groups
__device__ inline int v_swz(int t) { return 2 * (t & 3); }

// State row held by MFMA row m of row tile rt in the chunk layout
__device__ inline int chunk_row(int rt, int m) {
    return 32 * (rt >> 1) + 8 * (m >> 2) + 4 * (rt & 1) + (m & 3);
}

// Blocks of a chunk's lower-triangular token matrices over its halves:
// X11 = (H1, H1), X21 = (H2, H1), X22 = (H2, H2).
template <int DK>
struct alignas(16) ChunkLds {
    uint16_t kq[2 * CT][DK];  // rows 0..31: k_t, rows 32..63: q_t (bf16, pieces swizzled)
    uint16_t v[CT][DK];       // v_t (bf16, pieces swizzled)
    float Tt[2][HT][HT];      // T11 and T22 transposed: Tt[b][s][t] = T_bb[t][s]
    // A21 transposed, its rows in the order of the consumers' X2 registers:
    // A21t[s][4 r + g] = A21[4 g + r][s]
    float A21t[HT][HT];
    // Lq blocks in two bf16 parts (hi, mid), as MFMA operands of the outputs:
    // LqB1[p][t][s] = Lq11[t][s]; LqB2[p][t][.] = Lq21 and Lq22 row t, token s
    // of the first half at slot 8 (s / 4) + s % 4 and token 16 + s at slot
    // 8 (s / 4) + 4 + s % 4
    uint16_t LqB1[2][HT][HT];
    uint16_t LqB2[2][HT][2 * HT];
    float gam[CT];            // gamma_t = alpha_0 ... alpha_t
    float gp[CT];             // G'_t = alpha_{t+1} ... alpha_31
    float ab[2 * CT];         // alpha_t, then beta_t (padding tokens: 1, 0)
};

// A producer's hand-off from phase A to its own phase B: the diagonal blocks
// of A, transposed (At[b][s][t] = A_bb[t][s], i.e. column s of A_bb)
struct alignas(16) PrepScratch {
    float At[2][HT][HT];
};

constexpr int NBUF = 4;  // chunk buffers: applied, prepared (B), prepared (A), loading
constexpr int NPROD = 2; // producer waves
constexpr int CPW = 2;   // column blocks per consumer wave

template <int DK>
struct PrefillLds {
    ChunkLds<DK> ch[NBUF];
    // keys by state row for K^T W, built by the consumers one chunk ahead
    // (double buffered): row i holds, per group gg, k[i] of tokens
    // 4 gg .. 4 gg + 3 and 16 + 4 gg .. 16 + 4 gg + 3 (16 bytes), the groups
    // in the order gg ^ ((i / 8) % 4) (conflict-free reads)
    alignas(16) uint16_t kt[2][DK][32];
    PrepScratch ps[NPROD];
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

// Producer: copy chunk c's k, q and v rows and its alpha / beta from HBM into
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
    // k rows, then q rows (N.kq), then v rows (N.v)
#pragma unroll
    for (int it = 0; it < 3 * CT / RPI; ++it) {
        const int row = it * RPI + lane / SPR, slot = lane % SPR;
        const int which = (it * RPI) / CT;
        const int t = min(row & (CT - 1), last);
        const int piece = slot ^ (which < 2 ? kq_swz<DK>(row) : v_swz(row));
        const uint16_t *src = (which == 0 ? a.k : which == 1 ? a.q : a.v) + base;
        const uint16_t *at_t = wide ? tok_at<true, DK>(src, t, a, 8 * piece)
                                    : tok_at<false, DK>(src, t, a, 8 * piece);
        uint16_t *dst = which < 2 ? &N.kq[it * RPI][0] : &N.v[it * RPI - 2 * CT][0];
        __builtin_amdgcn_global_load_lds(at_t, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
    const int t = min(lane & (CT - 1), last);
    const float *gsrc = (lane < CT ? a.alpha : a.beta) + ((size_t)t0 + t) * tok_stride + tile_row;
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)&N.ab[0], 4, 0, 0);
}

// Gram blocks of a chunk in natural order: lane (g, n) gets
// kk[r] = k_{t0+4g+r} . k_{s0+n} and qk[r] = q_{t0+4g+r} . k_{s0+n}
template <int DK>
__device__ inline void gram(const uint16_t (*kq)[DK], int t0, int s0, f32x4 &kk, f32x4 &qk, int lane) {
    constexpr int NKS = DK / 32;
    const int g = lane >> 4, n = lane & 15;
    kk = f32x4{0.f, 0.f, 0.f, 0.f};
    qk = kk;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const int p = 4 * ks + g;
        const bf16x8 AK = __builtin_bit_cast(bf16x8, kq_piece<DK>(kq, t0 + n, p));
        const bf16x8 AQ = __builtin_bit_cast(bf16x8, kq_piece<DK>(kq, CT + t0 + n, p));
        const bf16x8 BS = __builtin_bit_cast(bf16x8, kq_piece<DK>(kq, s0 + n, p));
        kk = mfma_bf16_k32(AK, BS, kk);
        qk = mfma_bf16_k32(AQ, BS, qk);
    }
}

// x from the lane CTRL names inside the lane's row of 16 (a DPP row shift),
// 1 where that lane lies outside the row
template <int CTRL>
__device__ inline float row_shift_or_one(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), CTRL, 0xf, 0xf, false));
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

// bf16 parts (hi, mid) of the four floats x[0..3]: x = hi + mid to 16
// significant bits
__device__ inline void split2(const f32x4 &x, uint32_t hi[2], uint32_t md[2]) {
    hi[0] = pk_bf16(x[0], x[1]);
    hi[1] = pk_bf16(x[2], x[3]);
    md[0] = pk_bf16(sub_lo(hi[0], x[0]), sub_hi(hi[0], x[1]));
    md[1] = pk_bf16(sub_lo(hi[1], x[2]), sub_hi(hi[1], x[3]));
}

// The low (r even) or high half of the packed pair holding element r
__device__ inline uint16_t half_of(const uint32_t pk[2], int r) {
    return (uint16_t)(pk[r >> 1] >> (16 * (r & 1)));
}

// Producer, phase A: Gram blocks, gates and gated blocks of a loaded chunk,
// in registers.  Gamma_{t,s} = prod_{s<u<=t} alpha_u; A_ts = Gamma_ts k_t.k_s
// for s < t and Lq_ts = Gamma_ts q_t.k_s for s <= t (zero above).  Inside a
// half, lane (g, n) multiplies the gates of its own range (n, 4 g + r];
// across the halves Gamma_{16+t, s} = (product over (s, 15]) (product over
// [16, 16 + t]).  Writes gamma and G' and the blocks the consumers read (A21
// and the Lq blocks), and keeps A11 and A22 by column for its own phase B.
template <int DK>
__device__ __attribute__((always_inline)) inline void prep_a(ChunkLds<DK> &L, PrepScratch &S, int lane) {
    launder(lane);
    const int g = lane >> 4, n = lane & 15;
    wave_sync();  // the padding tokens' gates
    f32x4 kk11, qk11, kk21, qk21, kk22, qk22;
    gram<DK>(L.kq, 0, 0, kk11, qk11, lane);
    gram<DK>(L.kq, HT, 0, kk21, qk21, lane);
    gram<DK>(L.kq, HT, HT, kk22, qk22, lane);
    // prefix (pre) and suffix products inside each half by DPP scans (lane
    // l: token l % 32, one half per row of 16 lanes)
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
        const bool h2 = lane >= HT;
        L.gam[lane] = h2 ? tot1 * pre : pre;
        L.gp[lane] = h2 ? after : after * tot2;
    }
    // Gamma inside the halves: running products over u = 0..15 of the gates
    // past column n, kept at u = 4 g + r
    f32x4 G11 = {0.f, 0.f, 0.f, 0.f}, G22 = G11;
    float R1 = 1.f, R2 = 1.f;
    {
        f32x4 a4[CT / 4];  // alpha_0..31, the same in every lane
#pragma unroll
        for (int q = 0; q < CT / 4; ++q) a4[q] = *(const f32x4 *)&L.ab[4 * q];
#pragma unroll
        for (int u = 0; u < HT; ++u) {
            R1 *= u > n ? a4[u >> 2][u & 3] : 1.f;
            R2 *= u > n ? a4[4 + (u >> 2)][u & 3] : 1.f;
            if (g == (u >> 2)) {
                G11[u & 3] = R1;
                G22[u & 3] = R2;
            }
        }
    }
    f32x4 A11, A21, A22, L11, L21, L22;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = 4 * g + r;
        // R1 now holds the product over (n, 15]; pre of token 16 + t is the
        // product over [16, 16 + t]
        const float g21 = R1 * __shfl(pre, HT + t);
        A11[r] = t > n ? G11[r] * kk11[r] : 0.f;
        L11[r] = t >= n ? G11[r] * qk11[r] : 0.f;
        A22[r] = t > n ? G22[r] * kk22[r] : 0.f;
        L22[r] = t >= n ? G22[r] * qk22[r] : 0.f;
        A21[r] = g21 * kk21[r];
        L21[r] = g21 * qk21[r];
    }
    // column n of A11 and A22 for the forward substitution
    *(f32x4 *)&S.At[0][n][4 * g] = A11;
    *(f32x4 *)&S.At[1][n][4 * g] = A22;
#pragma unroll
    for (int r = 0; r < 4; ++r) L.A21t[n][4 * r + g] = A21[r];
    // Lq blocks as bf16 (hi, mid) operands
    uint32_t h[2], m[2];
    split2(L11, h, m);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        L.LqB1[0][4 * g + r][n] = half_of(h, r);
        L.LqB1[1][4 * g + r][n] = half_of(m, r);
    }
    const int slot = 8 * (n >> 2) + (n & 3);
    split2(L21, h, m);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        L.LqB2[0][4 * g + r][slot] = half_of(h, r);
        L.LqB2[1][4 * g + r][slot] = half_of(m, r);
    }
    split2(L22, h, m);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        L.LqB2[0][4 * g + r][slot + 4] = half_of(h, r);
        L.LqB2[1][4 * g + r][slot + 4] = half_of(m, r);
    }
}

// Producer, phase B: the diagonal blocks of T = (I + diag(beta) A)^-1
// diag(beta) by forward substitution, column s of T11 in lanes 0..15 and of
// T22 in lanes 32..47 (lanes 16..31 and 48..63 repeat them and store
// nothing).  With z = column s of (I + diag(beta) A)^-1,
// z_t = [t == s] - beta_t sum_{u<t} A_tu z_u; column u of A is applied to
// the later rows as soon as z_u is known (the same terms in the same order
// as row by row, without the row-by-row dependency chain).
template <int DK>
__device__ __attribute__((always_inline)) inline void prep_b(ChunkLds<DK> &L, PrepScratch &S, int lane) {
    launder(lane);
    const int hb = lane >> 5, s = lane & 15;
    const float(*At)[HT] = S.At[hb];
    float be[HT];
#pragma unroll
    for (int q = 0; q < HT / 4; ++q) {
        const f32x4 x = *(const f32x4 *)&L.ab[CT + HT * hb + 4 * q];
#pragma unroll
        for (int i = 0; i < 4; ++i) be[4 * q + i] = x[i];
    }
    float acc[HT], z[HT];
#pragma unroll
    for (int t = 0; t < HT; ++t) acc[t] = 0.f;
#pragma unroll
    for (int u = 0; u < HT; ++u) {
        z[u] = (u == s ? 1.f : 0.f) - be[u] * acc[u];
#pragma unroll
        for (int q = (u + 1) / 4; q < HT / 4; ++q) {
            const f32x4 col = *(const f32x4 *)&At[u][4 * q];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * q + i > u) acc[4 * q + i] = fmaf(col[i], z[u], acc[4 * q + i]);
        }
    }
    if ((lane & 16) == 0) {
        const float bs = L.ab[CT + HT * hb + s];
        f32x4 *dst = (f32x4 *)&L.Tt[hb][s][0];
#pragma unroll
        for (int q = 0; q < HT / 4; ++q)
            dst[q] = f32x4{z[4 * q] * bs, z[4 * q + 1] * bs, z[4 * q + 2] * bs, z[4 * q + 3] * bs};
    }
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
    constexpr int NCW = DK / 16 / CPW;  // consumer waves
    constexpr float QMAX = BITS == 4 ? 7.f : 127.f;
    constexpr float KAPPA = Loader<DK, BITS>::KAPPA;
    const int g = lane >> 4, n = lane & 15;
    const size_t tile_row = (size_t)b * a.p.H + h;
    // rows per token: 32-bit arithmetic unless the launch needs 64-bit offsets
    using TokStride = typename std::conditional<WIDE_OFF, size_t, uint32_t>::type;
    const TokStride tok_stride = (TokStride)a.p.B * (TokStride)a.p.H;
    const int n_chunks = (a.n_tok + CT - 1) / CT;
    const bool producer = wave >= NCW;
    const int cb0 = CPW * wave;  // a consumer's first column block

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
        // phase A waits for nothing else.  The producers set the pace of the
        // interval (long dependent chains through LDS, the forward
        // substitution), so they run at raised wave priority throughout,
        // ahead of the consumers sharing their SIMDs.
        const int p = wave - NCW;
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
            prep_b<DK>(L.ch[c % NBUF], ps, lane);
        };
        __builtin_amdgcn_s_setprio(3);
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

    // the column blocks' starting state: the stored codes decoded (zero after
    // a zero initialisation), in chunk layout
    f32x4 acc[CPW][NRT];
#pragma unroll
    for (int e = 0; e < CPW; ++e) {
        Loader<DK, BITS> ld;
        ld.load(codes, cb0 + e, lane);
        ld.codes_f32(acc[e]);
        const float sk = scl[16 * (cb0 + e) + n] * (1.f / KAPPA);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) acc[e][rt] *= sk;
        to_chunk_layout<NKS>(acc[e], lane);
    }

    lds_barrier();
    // this wave's DK / NCW rows of a chunk's key table, 16 per pass: lane ->
    // (state row, token group)
    auto build_kt = [&](const ChunkLds<DK> &N, uint16_t (*KT)[32]) {
        constexpr int ROWS = DK / NCW;
#pragma unroll
        for (int pass = 0; pass < ROWS / 16; ++pass) {
            const int i = ROWS * wave + 16 * pass + (lane >> 2), gg = lane & 3;
            uint32_t w[4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int t = HT * hh + 4 * gg;
                uint32_t x4[4];
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    x4[x] = N.kq[t + x][8 * ((i >> 3) ^ kq_swz<DK>(t + x)) + (i & 7)];
                w[2 * hh] = x4[0] | (x4[1] << 16);
                w[2 * hh + 1] = x4[2] | (x4[3] << 16);
            }
            *(u32x4 *)&KT[i][8 * (gg ^ ((i >> 3) & 3))] = u32x4{w[0], w[1], w[2], w[3]};
        }
    };
    build_kt(L.ch[0], L.kt[0]);
    lds_barrier();
    // A operand rows of P_K: the K blocks' row m is token 4 (m % 4) + m / 4 of
    // its half, so P_K's row 4 g + r is token 4 r + g (the B layout of the
    // float32 chunk MFMAs)
    const int tok_n = 4 * (n & 3) + (n >> 2);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < n_chunks; ++c) {
        const ChunkLds<DK> &C = L.ch[c % NBUF];
        const uint16_t(*KT)[32] = L.kt[c & 1];
        if (c + 1 < n_chunks) build_kt(L.ch[(c + 1) % NBUF], L.kt[(c + 1) & 1]);
        // Operands of the X and Y stages, read before the P stage so that
        // their LDS latency hides behind it: the values v (tokens 4 r + g and
        // 16 + 4 r + g of column 16 cb + n: vv[e][r] and vv[e][4 + r]),
        // gamma and G' of the lane's tokens, and its entries of T11, A21t, T22
        uint16_t vv[CPW][8];
        float gk1[4], gk2[4], t11[4], a21[4], t22[4];
        f32x4 gp1, gp2;
        {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                gk1[r] = C.gam[4 * r + g];
                gk2[r] = C.gam[HT + 4 * r + g];
                t11[r] = C.Tt[0][4 * r + g][n];
                a21[r] = C.A21t[4 * g + r][n];
                t22[r] = C.Tt[1][4 * r + g][n];
            }
            gp1 = *(const f32x4 *)&C.gp[4 * g];
            gp2 = *(const f32x4 *)&C.gp[HT + 4 * g];
#pragma unroll
            for (int e = 0; e < CPW; ++e) {
                const uint16_t *vl = &C.v[g][8 * ((2 * (cb0 + e) + (n >> 3)) ^ v_swz(g)) + (n & 7)];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    vv[e][r] = vl[4 * r * DK];
                    vv[e][4 + r] = vl[(HT + 4 * r) * DK];
                }
            }
            compiler_fence();
        }
        // P_K = K M0 and, transposed, P_Q^T = M0^T Q^T over two bf16 parts of
        // M0 (hi + mid, 16 significant bits; a third part for P_K cost 8 more
        // MFMAs per chunk and 5% of the time without moving a code), both
        // halves of the chunk; k-slot 8 g + e is state row 32 ks + 8 g + e.
        // The K and Q operands serve both column blocks.  P_Q^T's lane (g, n)
        // holds P_Q[token n][column 16 cb + 4 g + r].
        // The gated state gamma_C M of the update (M <- gamma_C M + K^T W) is
        // taken as each slice is split, so the split consumes the old values
        // in place (no copies).
        const float gC = C.gam[CT - 1];
        f32x4 PK1[CPW], PK2[CPW], PQ1[CPW], PQ2[CPW];
#pragma unroll
        for (int e = 0; e < CPW; ++e) PK1[e] = PK2[e] = PQ1[e] = PQ2[e] = zero;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int pc = 4 * ks + g;
            const bf16x8 AK1 = __builtin_bit_cast(bf16x8, kq_piece<DK>(C.kq, tok_n, pc));
            const bf16x8 AK2 = __builtin_bit_cast(bf16x8, kq_piece<DK>(C.kq, HT + tok_n, pc));
            const bf16x8 AQ1 = __builtin_bit_cast(bf16x8, kq_piece<DK>(C.kq, CT + n, pc));
            const bf16x8 AQ2 = __builtin_bit_cast(bf16x8, kq_piece<DK>(C.kq, CT + HT + n, pc));
#pragma unroll
            for (int e = 0; e < CPW; ++e) {
                uint32_t h0[2], m0[2], h1[2], m1[2];
                f32x4 x0 = acc[e][2 * ks], x1 = acc[e][2 * ks + 1];
                acc[e][2 * ks] *= gC;
                acc[e][2 * ks + 1] *= gC;
                // the gated copies exist before the split, which then consumes
                // x0 and x1 in place
                order_after(acc[e][2 * ks], x0);
                order_after(acc[e][2 * ks + 1], x1);
                split2(x0, h0, m0);
                split2(x1, h1, m1);
                const bf16x8 BH = __builtin_bit_cast(bf16x8, u32x4{h0[0], h0[1], h1[0], h1[1]});
                const bf16x8 BM = __builtin_bit_cast(bf16x8, u32x4{m0[0], m0[1], m1[0], m1[1]});
                PK1[e] = mfma_bf16_k32(AK1, BH, PK1[e]);
                PK2[e] = mfma_bf16_k32(AK2, BH, PK2[e]);
                PQ1[e] = mfma_bf16_k32(BH, AQ1, PQ1[e]);
                PQ2[e] = mfma_bf16_k32(BH, AQ2, PQ2[e]);
                PK1[e] = mfma_bf16_k32(AK1, BM, PK1[e]);
                PK2[e] = mfma_bf16_k32(AK2, BM, PK2[e]);
                PQ1[e] = mfma_bf16_k32(BM, AQ1, PQ1[e]);
                PQ2[e] = mfma_bf16_k32(BM, AQ2, PQ2[e]);
            }
        }
        // X for tokens 4 r + g and 16 + 4 r + g (the P_K rows this lane
        // holds), column 16 cb + n
        float X1[CPW][4], X2[CPW][4];
#pragma unroll
        for (int e = 0; e < CPW; ++e)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                X1[e][r] = fmaf(-gk1[r], PK1[e][r], bf2f(vv[e][r]));
                X2[e][r] = fmaf(-gk2[r], PK2[e][r], bf2f(vv[e][4 + r]));
            }
        // W = diag(G') T X with T = [T11 0; T21 T22], T21 = -T22 A21 T11:
        // Y1 = T11 X1, X2' = X2 - A21 Y1, Y2 = T22 X2', W = diag(G') [Y1; Y2]
        // (float32 MFMA: the state needs its accuracy).  Y1 and Y2 come out
        // in natural row order (lane (g, n): token 4 g + r of the half)
        f32x4 Y1[CPW], D21[CPW], Y2[CPW];
#pragma unroll
        for (int e = 0; e < CPW; ++e) Y1[e] = D21[e] = Y2[e] = zero;
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int e = 0; e < CPW; ++e) Y1[e] = mfma_f32_k4(t11[st], X1[e][st], Y1[e]);
        // step st takes Y1's own row 4 g + st; A21t's row order puts the
        // product in X2's layout (token 16 + 4 r + g)
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int e = 0; e < CPW; ++e) D21[e] = mfma_f32_k4(a21[st], Y1[e][st], D21[e]);
#pragma unroll
        for (int e = 0; e < CPW; ++e)
#pragma unroll
            for (int r = 0; r < 4; ++r) X2[e][r] -= D21[e][r];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int e = 0; e < CPW; ++e) Y2[e] = mfma_f32_k4(t22[st], X2[e][st], Y2[e]);
        f32x4 W1[CPW], W2[CPW];
        {
#pragma unroll
            for (int e = 0; e < CPW; ++e)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    W1[e][r] = gp1[r] * Y1[e][r];
                    W2[e][r] = gp2[r] * Y2[e][r];
                }
        }
        // key rows of the update, read ahead of the output stage
        u32x4 ktr[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int R = chunk_row(rt, n);
            ktr[rt] = *(const u32x4 *)&KT[R][8 * (g ^ ((R >> 3) & 3))];
        }
        compiler_fence();
        // (Lq T X)^T = ([Lq11 Y1; Lq21 Y1 + Lq22 Y2])^T on bf16 MFMA, Y and Lq
        // in two parts each (hi hi, hi mid, mid hi: ~1e-5 relative error,
        // outputs only); the lane's k-slots are its own tokens 4 g + e.  Then
        // O^T += (diag(gamma) Q M0)^T: this lane's outputs are token n (first
        // half) and 16 + n (second half), columns 16 cb + 4 g .. 16 cb + 4 g + 3
        {
            const s16x4 A1h = __builtin_bit_cast(s16x4, *(const u32x2 *)&C.LqB1[0][n][4 * g]);
            const s16x4 A1m = __builtin_bit_cast(s16x4, *(const u32x2 *)&C.LqB1[1][n][4 * g]);
            const bf16x8 A2h = __builtin_bit_cast(bf16x8, *(const u32x4 *)&C.LqB2[0][n][8 * g]);
            const bf16x8 A2m = __builtin_bit_cast(bf16x8, *(const u32x4 *)&C.LqB2[1][n][8 * g]);
            const float gq1 = C.gam[n], gq2 = C.gam[HT + n];
            const int nv = a.n_tok - CT * c;  // chunk c's real tokens
            float *obase = a.out + ((size_t)CT * c * tok_stride + tile_row) * DK;
#pragma unroll
            for (int e = 0; e < CPW; ++e) {
                uint32_t yh[4], ym[4];
                split2(Y1[e], yh, ym);
                split2(Y2[e], yh + 2, ym + 2);
                const s16x4 B1h = __builtin_bit_cast(s16x4, u32x2{yh[0], yh[1]});
                const s16x4 B1m = __builtin_bit_cast(s16x4, u32x2{ym[0], ym[1]});
                const bf16x8 B2h = __builtin_bit_cast(bf16x8, u32x4{yh[0], yh[1], yh[2], yh[3]});
                const bf16x8 B2m = __builtin_bit_cast(bf16x8, u32x4{ym[0], ym[1], ym[2], ym[3]});
                f32x4 O1 = mfma_bf16_k16(B1h, A1h, zero);
                f32x4 O2 = mfma_bf16_k32(B2h, A2h, zero);
                O1 = mfma_bf16_k16(B1m, A1h, O1);
                O2 = mfma_bf16_k32(B2m, A2h, O2);
                O1 = mfma_bf16_k16(B1h, A1m, O1);
                O2 = mfma_bf16_k32(B2h, A2m, O2);
                if (a.out) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        O1[r] = fmaf(gq1, PQ1[e][r], O1[r]);
                        O2[r] = fmaf(gq2, PQ2[e][r], O2[r]);
                    }
                    // Each store writes 64 bytes of a token's 128-byte line
                    // (the other half comes from the next e): ordinary
                    // stores let L2 merge the two halves before HBM, where
                    // nontemporal ones wrote each half as its own line
                    // (+46% write bytes) and took 1-3% longer
                    const uint32_t x = 16 * (cb0 + e) + 4 * g;
                    if (n < nv) *(f32x4 *)tok_at<WIDE_OFF, DK>(obase, n, a, x) = O1;
                    if (HT + n < nv) *(f32x4 *)tok_at<WIDE_OFF, DK>(obase, HT + n, a, x) = O2;
                }
            }
        }

        // M <- gamma_C M + K^T W (acc already holds gamma_C M), W in two bf16 parts (hi + mid, relative
        // error below 2^-17; a third part cost 8 more MFMAs per chunk and
        // 3% of the time): the lane's k-slots are tokens 4 g .. 4 g + 3 (first
        // half) and 16 + 4 g .. 16 + 4 g + 3 (second half), one 32-deep
        // product per part; MFMA row m of row tile rt is state row
        // chunk_row(rt, m).  The key rows serve both column blocks.
        bf16x8 WH[CPW], WM[CPW];
#pragma unroll
        for (int e = 0; e < CPW; ++e) {
            uint32_t h1[2], m1[2], h2[2], m2[2];
            split2(W1[e], h1, m1);
            split2(W2[e], h2, m2);
            WH[e] = __builtin_bit_cast(bf16x8, u32x4{h1[0], h1[1], h2[0], h2[1]});
            WM[e] = __builtin_bit_cast(bf16x8, u32x4{m1[0], m1[1], m2[0], m2[1]});
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const bf16x8 A2 = __builtin_bit_cast(bf16x8, ktr[rt]);
#pragma unroll
            for (int e = 0; e < CPW; ++e) {
                acc[e][rt] = mfma_bf16_k32(A2, WH[e], acc[e][rt]);
                acc[e][rt] = mfma_bf16_k32(A2, WM[e], acc[e][rt]);
            }
        }
        lds_barrier();  // chunk c+1 prepared and its key table built, chunk c's buffer free
    }

    // ---- encode each column block once: absmax, scale, codes ----
#pragma unroll
    for (int e = 0; e < CPW; ++e) {
        const int cb = cb0 + e, j = 16 * cb + n;
        to_pool_layout<NKS>(acc[e], lane);
        float am = 0.f;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) am = fmaxf(am, fabsf(acc[e][rt][r]));
        am = xor_max(am, 16);
        am = xor_max(am, 32);
        const float s_new = am * (1.f / QMAX);
        const float ratio = s_new > 0.f ? __builtin_amdgcn_rcpf(s_new) : 0.f;
        uint32_t y[NRT][4];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) y[rt][r] = __float_as_uint(fmaf(acc[e][rt][r], ratio, 12582912.f));
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
        if constexpr (ERR) column_error<NRT>(acc[e], y, 1.f, s_new, a.p.colerr + (tile_row * DK + j) * 2, g);
    }
}

template <int DK, bool ERR, bool WIDE_OFF>
__global__ void __launch_bounds__(64 * (DK / 16 / CPW + NPROD)) prefill_mfma_kernel(PrefillArgs a) {
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
    const dim3 grid(a.tiles), block(64 * (p.dk / 16 / CPW + NPROD));
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
