// Prompt prefill into the quantized state (gfx950): a period of n_tok tokens,
// any n_tok >= 1, applied to every (sequence, head) state in float32 and
// encoded once at the end (the prefill hand-off: chunked kernels already keep
// the state in high precision across a chunk, and periodic rounding extends
// that to decode: 'PACE: four-bit recurrent state by rounding less often',
// TL;DR point (1)).
//
// One workgroup per state tile, resident for the whole prompt:
//   * NCB consumer waves (one per 16-column block) hold the tile's float32
//     state in MFMA accumulator layout (the same lane -> (row, column) map as
//     the pool layout) from the first token to the final encode;
//   * two producer waves, on different SIMDs, take alternate chunks: each
//     stages a chunk's keys and queries in LDS and computes its Gram products
//     and gates two chunks ahead of the consumers, then its UT solve and
//     Lq T one chunk ahead (three chunk buffers in LDS); the consumers read
//     their own v values straight from the inputs, one chunk ahead, and
//     build the next chunk's key table by state row for K^T W (16 rows
//     each);
//   * one workgroup barrier per chunk, ordering LDS only (global loads and
//     stores stay in flight across it).
// Per chunk and column block (WY / UT form, as the decode kernels):
//   P_K = K M0 with M0 split exactly into three bf16 parts (hi + mid + lo), so
//   the state update keeps float32 accuracy; P_Q = Q M0 over hi + mid (it
//   only reaches the outputs, and two parts leave ~1e-5 relative error);
//   X = V - diag(g) P_K; W = diag(G_C) T X and Lq T X on float32 MFMA;
//   O = Lq T X + diag(g) P_Q; M <- g_C M + K^T W (bf16 MFMA, W in three parts:
//   hi and mid in one 32-deep product, lo in a second one).
// Outputs of a chunk go through double-buffered LDS and leave as whole
// 512-byte rows.
#include "chunk16.h"
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

constexpr int CT = CK;      // tokens per chunk
constexpr int PROW = 136;   // bf16 elements per LDS token row (128 + 8 padding)
constexpr int OPAD = 132;   // floats per LDS output row

struct alignas(16) ChunkLds {
    uint16_t kq[2 * CT][PROW];  // rows 0..15: k_t, rows 16..31: q_t (bf16 bits)
    float Tt[CT][CT];   // Tt[s][t] = T[t][s]
    float LqT[CT][CT];  // (Lq T)[t][s]
    float gam[CT];      // gamma_t inside the chunk
    float gamC[CT];     // Gamma_{C-1, t}
    // keys by state row for K^T W, built by the consumers: row i holds, per
    // group gg of tokens 4 gg .. 4 gg + 3, their k[i] twice (16 bytes), the
    // groups in the order gg ^ ((i % 16) / 4) (conflict-free row reads)
    uint16_t kt[128][32];
};

struct alignas(16) PrepScratch {
    float alpha[CT], beta[CT];
    float kkA[CT][CT];   // k_t . k_s, then A in place
    float qkLq[CT][CT];  // q_t . k_s, then Lq in place
};

constexpr int NBUF = 3;  // chunk buffers: applied, being prepared, being staged
constexpr int NPROD = 2; // producer waves

template <int DK>
struct PrefillLds {
    ChunkLds ch[NBUF];
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

template <int DK>
struct TokenRegs {
    static constexpr int CPR = DK / 8;            // 16-byte chunks per token row
    static constexpr int NL = 2 * CT * CPR / 64;  // loads per lane (k and q rows)
    u32x4 val[NL];
    float ab;
};

// Producer, part 1: issue the loads of chunk c's tokens (k, q, v rows, then
// alpha / beta) into registers; padding tokens are zero (alpha 1, beta 0).
template <int DK>
__device__ __attribute__((always_inline)) inline void load_chunk(const PrefillArgs &a, TokenRegs<DK> &R, size_t tile_row, int c,
                                  int lane) {
    constexpr int CPR = TokenRegs<DK>::CPR;
    const uint32_t tok_stride = (uint32_t)a.p.B * (uint32_t)a.p.H;
    const int t0 = CT * c, nv = min(CT, a.n_tok - t0);
    const size_t base = ((size_t)t0 * tok_stride + tile_row) * DK;
#pragma unroll
    for (int it = 0; it < TokenRegs<DK>::NL; ++it) {
        const int e = lane + 64 * it;
        const int row = e / CPR, col = (e % CPR) * 8;
        const int t = row & 15;
        // the 32 rows are k, q in blocks of 16: the block is fixed per load
        constexpr int RPL = 64 / CPR;  // rows per load
        const int which = (it * RPL) / CT;
        const uint16_t *src = (which == 0 ? a.k : a.q) + base;
        R.val[it] = u32x4{0u, 0u, 0u, 0u};
        if (t < nv)
            R.val[it] = __builtin_nontemporal_load(
                at((const u32x4 *)src, (uint32_t)(t * tok_stride * DK + col) * 2u));
    }
    R.ab = 0.f;
    if (lane < 32) {
        const int t = lane & 15;
        const bool is_beta = lane >= 16;
        R.ab = is_beta ? 0.f : 1.f;
        if (t < nv) R.ab = (is_beta ? a.beta : a.alpha)[((size_t)t0 + t) * tok_stride + tile_row];
    }
}

// Producer, part 2: write the loaded chunk into LDS.
template <int DK>
__device__ __attribute__((always_inline)) inline void stage_chunk(const TokenRegs<DK> &R, ChunkLds &L, PrepScratch &S, int lane) {
    constexpr int CPR = TokenRegs<DK>::CPR;
#pragma unroll
    for (int it = 0; it < TokenRegs<DK>::NL; ++it) {
        const int e = lane + 64 * it;
        const int row = e / CPR, col = (e % CPR) * 8;
        const int t = row & 15, which = row >> 4;
        uint16_t *dst = &L.kq[which * 16 + t][col];
        *(u32x4 *)dst = R.val[it];
    }
    if (lane < 32) (lane >= 16 ? S.beta : S.alpha)[lane & 15] = R.ab;
}

// Producer, part 3: the staged chunk's token-only matrices, in two phases
// of about equal length (Gram products and gates; UT solve and Lq T).
template <int DK>
__device__ __attribute__((always_inline)) inline void prep_a(ChunkLds &L, PrepScratch &S, int lane) {
    wave_sync();
    chunk16_gram<DK, PROW>(L.kq, S.kkA, S.qkLq, lane);
    chunk16_gates(S.alpha, S.kkA, S.qkLq, S.kkA, S.qkLq, L.gam, L.gamC, lane);
}
__device__ __attribute__((always_inline)) inline void prep_b(ChunkLds &L, PrepScratch &S, int lane) {
    chunk16_ut(S.kkA, S.beta, L.Tt, lane);
    chunk16_lqt(S.qkLq, L.Tt, L.LqT, lane);
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

template <int DK, int BITS, bool ERR>
__device__ void prefill_tile(const PrefillArgs &a, PrefillLds<DK> &L, int b, int h, int slot,
                             int wave, int lane) {
    constexpr int NKS = DK / 32;  // k-slices of 32 rows
    constexpr int NRT = DK / 16;  // row tiles of 16 rows
    constexpr int NCB = DK / 16;  // column blocks = consumer waves
    constexpr float QMAX = BITS == 4 ? 7.f : 127.f;
    constexpr float KAPPA = Loader<DK, BITS>::KAPPA;
    const int g = lane >> 4, n = lane & 15;
    const size_t tile_row = (size_t)b * a.p.H + h;
    const uint32_t tok_stride = (uint32_t)a.p.B * (uint32_t)a.p.H;
    const int n_chunks = (a.n_tok + CT - 1) / CT;
    const bool producer = wave >= NCB;
    const int cb = wave, j = 16 * cb + n;

    uint8_t *codes = BITS == 4
        ? a.p.codes4 + ((size_t)b * a.p.n4 + slot) * tile_code_bytes(DK, DK, 4)
        : a.p.codes8 + ((size_t)b * a.p.n8 + slot) * tile_code_bytes(DK, DK, 8);
    float *scl = a.p.scales + tile_row * DK;

    // the column block's starting state: the stored codes decoded (zero after
    // a zero initialisation)
    f32x4 acc[NRT];
    if (!producer) {
        Loader<DK, BITS> ld;
        ld.load(codes, cb, lane);
        ld.codes_f32(acc);
        const float sk = scl[j] * (1.f / KAPPA);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) acc[rt] *= sk;
    }
    // Output flush of chunk c, shared by every wave after the barrier that
    // closes it: rows of DK floats, 16 bytes per lane.  Staging buffer c & 1
    // is written again only in chunk c + 2, after the next barrier, by which
    // every wave has finished this flush.
    auto flush = [&](int c) {
        if (!a.out) return;
        constexpr int PER_ROW = DK / 4;
        const int e = wave * 64 + lane;
        const int t = e / PER_ROW, c4 = (e % PER_ROW) * 4;
        if (t < CT && t < a.n_tok - CT * c) {  // chunk c's real tokens
            const f32x4 x = *(const f32x4 *)&L.o[c & 1][t][c4];
            __builtin_nontemporal_store(
                x, (f32x4 *)(a.out + (((size_t)CT * c + t) * tok_stride + tile_row) * DK + c4));
        }
    };

    if (producer) {
        // Two producers take alternate chunks.  Chunk c is staged and its
        // Gram products and gates computed (phase A) while the consumers
        // apply chunk c - 2, its UT solve and Lq T (phase B) while they apply
        // chunk c - 1; its tokens were loaded into the producer's registers
        // two intervals earlier.  Each producer alternates A and B, so both
        // carry half of the work every interval, on different SIMDs.
        const int p = wave - NCB;
        PrepScratch &ps = L.ps[p];
        TokenRegs<DK> R;
        auto phase_a = [&](int c) {
            ChunkLds &N = L.ch[c % NBUF];
            stage_chunk<DK>(R, N, ps, lane);
            if (c + NPROD < n_chunks) load_chunk<DK>(a, R, tile_row, c + NPROD, lane);
            prep_a<DK>(N, ps, lane);
        };
        if (p < n_chunks) {
            load_chunk<DK>(a, R, tile_row, p, lane);
            phase_a(p);
            if (p == 0) prep_b(L.ch[0], ps, lane);
        }
        lds_barrier();
        lds_barrier();  // the consumers' key table of chunk 0
        for (int c = 0; c < n_chunks; ++c) {
            // this interval: phase B of chunk c + 1 or phase A of chunk c + 2
            if ((c + 1) % NPROD == p) {
                if (c + 1 < n_chunks) prep_b(L.ch[(c + 1) % NBUF], ps, lane);
            } else if (c + 2 < n_chunks) {
                phase_a(c + 2);
            }
            lds_barrier();  // chunk c+1 prepared, chunk c's outputs complete
            flush(c);
        }
        return;
    }

    lds_barrier();
    // this wave's 16 rows of a chunk's key table: lane -> (row, token group)
    auto build_kt = [&](ChunkLds &N) {
        const int i = 16 * wave + (lane >> 2), gg = lane & 3;
        const uint32_t a01 = (uint32_t)N.kq[4 * gg][i] | ((uint32_t)N.kq[4 * gg + 1][i] << 16);
        const uint32_t a23 = (uint32_t)N.kq[4 * gg + 2][i] | ((uint32_t)N.kq[4 * gg + 3][i] << 16);
        *(u32x4 *)&N.kt[i][8 * (gg ^ ((i & 15) >> 2))] = u32x4{a01, a23, a01, a23};
    };
    build_kt(L.ch[0]);
    lds_barrier();
    // A operand rows: the K block's row m is token 4 (m % 4) + m / 4, so P_K's
    // row 4 g + r is token 4 r + g (the B layout of the float32 chunk MFMAs);
    // the Q block's row m is token m, so P_Q's rows line up with O's
    const int tok_n = 4 * (n & 3) + (n >> 2);
    // this lane's v values (tokens 4 r + g of a chunk, column j), read from
    // the inputs one chunk ahead
    auto load_v = [&](int c, uint32_t (&vv)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = CT * c + 4 * r + g;
            vv[r] = t < a.n_tok ? (uint32_t)a.v[((size_t)t * tok_stride + tile_row) * DK + j] : 0u;
        }
    };
    uint32_t vcur[4], vnext[4];
    load_v(0, vcur);
    for (int c = 0; c < n_chunks; ++c) {
        if (c + 1 < n_chunks) load_v(c + 1, vnext);
        ChunkLds &C = L.ch[c % NBUF];
        if (c + 1 < n_chunks) build_kt(L.ch[(c + 1) % NBUF]);  // staged before the last barrier
        {
            // P_K = K M0 over three bf16 parts of M0 (the state update needs
            // float32 accuracy), P_Q = Q M0 over two (outputs only)
            f32x4 PK = {0.f, 0.f, 0.f, 0.f}, PQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int c0 = 32 * ks + 4 * g, c1 = c0 + 16;
                const u32x2 k0 = *(const u32x2 *)&C.kq[tok_n][c0], k1 = *(const u32x2 *)&C.kq[tok_n][c1];
                const u32x2 q0 = *(const u32x2 *)&C.kq[16 + n][c0], q1 = *(const u32x2 *)&C.kq[16 + n][c1];
                const bf16x8 AK = __builtin_bit_cast(bf16x8, u32x4{k0[0], k0[1], k1[0], k1[1]});
                const bf16x8 AQ = __builtin_bit_cast(bf16x8, u32x4{q0[0], q0[1], q1[0], q1[1]});
                uint32_t h0[2], m0[2], l0[2], h1[2], m1[2], l1[2];
                split3(acc[2 * ks], h0, m0, l0);
                split3(acc[2 * ks + 1], h1, m1, l1);
                const bf16x8 BH = __builtin_bit_cast(bf16x8, u32x4{h0[0], h0[1], h1[0], h1[1]});
                const bf16x8 BM = __builtin_bit_cast(bf16x8, u32x4{m0[0], m0[1], m1[0], m1[1]});
                const bf16x8 BL = __builtin_bit_cast(bf16x8, u32x4{l0[0], l0[1], l1[0], l1[1]});
                PK = mfma_bf16_k32(AK, BH, PK);
                PQ = mfma_bf16_k32(AQ, BH, PQ);
                PK = mfma_bf16_k32(AK, BM, PK);
                PQ = mfma_bf16_k32(AQ, BM, PQ);
                PK = mfma_bf16_k32(AK, BL, PK);
            }
            // X for tokens 4 r + g (the P_K rows this lane holds)
            float X[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) X[r] = fmaf(-C.gam[4 * r + g], PK[r], bf2f((uint16_t)vcur[r]));
            // W (rows = tokens) and Lq T X on float32 MFMA; step st takes token 4 st + g
            f32x4 W = {0.f, 0.f, 0.f, 0.f}, O = {0.f, 0.f, 0.f, 0.f};
            const float gct = C.gamC[n];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int s = 4 * st + g;
                W = mfma_f32_k4(gct * C.Tt[s][n], X[st], W);
                O = mfma_f32_k4(C.LqT[n][s], X[st], O);
            }
            // O += diag(gamma) Q M0: rows 4 g + r of O and P_Q are the same tokens
#pragma unroll
            for (int r = 0; r < 4; ++r) L.o[c & 1][4 * g + r][j] = fmaf(C.gam[4 * g + r], PQ[r], O[r]);

            // M <- gamma_C M + K^T W, W in three bf16 parts: hi and mid of
            // tokens 4 g + e in one 32-deep product, lo (and zeros) in a
            // second one of the same shape.  Both products accumulate into
            // the same registers back to back; a 16-deep product there
            // instead lost the 32-deep one's result on some row tiles (the
            // compiler inserts no wait between the two shapes).
            const float gC = C.gam[CT - 1];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) acc[rt] *= gC;
            uint32_t wh[2], wm[2], wl[2];
            split3(W, wh, wm, wl);
            const bf16x8 BHM = __builtin_bit_cast(bf16x8, u32x4{wh[0], wh[1], wm[0], wm[1]});
            const bf16x8 BL0 = __builtin_bit_cast(bf16x8, u32x4{wl[0], wl[1], 0u, 0u});
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                // k of tokens 4 g .. 4 g + 3 at row 16 rt + n, twice
                const bf16x8 A2 = __builtin_bit_cast(bf16x8, *(const u32x4 *)&C.kt[16 * rt + n][8 * (g ^ (n >> 2))]);
                acc[rt] = mfma_bf16_k32(A2, BHM, acc[rt]);
                acc[rt] = mfma_bf16_k32(A2, BL0, acc[rt]);
            }
        }
        lds_barrier();  // chunk c+1 staged, chunk c's outputs complete
        flush(c);
#pragma unroll
        for (int r = 0; r < 4; ++r) vcur[r] = vnext[r];
    }

    // ---- encode each column block once: absmax, scale, codes ----
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

template <int DK, bool ERR>
__global__ void __launch_bounds__(64 * (DK / 16 + NPROD)) prefill_mfma_kernel(PrefillArgs a) {
    __shared__ PrefillLds<DK> L;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = blockIdx.x;  // one tile per workgroup, sequence-major
    const int b = w / a.p.H, h = w - b * a.p.H;
    const int m = a.p.head_map[h];
    if ((m >> 16) == 8)
        prefill_tile<DK, 8, ERR>(a, L, b, h, m & 0xffff, wave, lane);
    else
        prefill_tile<DK, 4, ERR>(a, L, b, h, m & 0xffff, wave, lane);
}

}  // namespace

bool prefill_mfma_supported(int dk, int dv, int in_bf16, long long rows_per_token) {
    // per-lane token offsets inside a chunk (16 tokens x rows x d x 2 bytes)
    // and the output offsets are kept in 32 bits
    return in_bf16 && dk == dv && (dk == 128 || dk == 64) &&
           (long long)CT * rows_per_token * dk * 4 < (1ll << 31);
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
    if (p.dk == 128) {
        if (err)
            hipLaunchKernelGGL((prefill_mfma_kernel<128, true>), dim3(a.tiles), dim3(64 * (8 + NPROD)), 0, s, a);
        else
            hipLaunchKernelGGL((prefill_mfma_kernel<128, false>), dim3(a.tiles), dim3(64 * (8 + NPROD)), 0, s, a);
    } else {
        if (err)
            hipLaunchKernelGGL((prefill_mfma_kernel<64, true>), dim3(a.tiles), dim3(64 * (4 + NPROD)), 0, s, a);
        else
            hipLaunchKernelGGL((prefill_mfma_kernel<64, false>), dim3(a.tiles), dim3(64 * (4 + NPROD)), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace pace
