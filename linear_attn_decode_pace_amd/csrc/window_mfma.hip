// FP8 write window step for gfx950, one 64-wide wavefront per (sequence,
// head) state (bf16 inputs, d_k = d_v = 64 or 128).  The window is the
// pure-write sliding window of '低比特量化新突破：GGA+PW让线性注意力长文本生成更准更短',
// section 'PW：让近期写入走“纯净通道”': the last S writes (k_e, w_e) of the
// delta rule stay out of the column-quantized history H as E4M3 vectors with
// one float32 scale each and a decay delta_e, the history decays through one
// factor lam, and the write that leaves the window is merged into H.
//
// The state is never rebuilt.  With M = lam H + sum_e delta_e k_e w_e^T:
//   d   = M^T k   = lam s_j (c_j . k) + sum_e delta_e (k_e . k) w_e[j]
//   u_j = beta (v_j - alpha d_j)
//   o_j = ((alpha M + k u^T)^T q)_j = alpha (lam s_j (c_j . q) + sum_e delta_e (k_e . q) w_e[j]) + (k . q) u_j
// so a step reads the codes once for two dot products per column (bf16 MFMA:
// codes and bf16 inputs are exact in bf16, products exact in float32), and
// the window only through S key dot products and S bytes per column.  When
// the window is full the oldest write (k_o, w_o) leaves:
//   H' = lam alpha H + delta_o alpha k_o w_o^T,
// accumulated in units of sigma_j = lam alpha s_j / KAPPA, where the loaded
// codes are already KAPPA c: one fused multiply-add per entry, then the
// column quantizer of the decode kernels (absmax, s = absmax / qmax, codes by
// one rounding against 1.5 * 2^23, one 16-byte store per lane and block).
// Tiles whose window is not full leave the history untouched.
//
// Lane l = 16 g + n owns column 16 cb + n of column block cb and the rows
// 16 rt + 4 g + r (pace_layout.h), as in the decode kernels.
#include "e4m3.h"
#include "mfma_common.h"
#include "pace_window.h"

namespace pace {
namespace {

constexpr int WTPB = 4;     // tiles (wavefronts) per workgroup
constexpr int WMAX_S = 64;  // largest window

struct WinArgs {
    PoolView p;
    WindowView wv;
    const uint16_t *q, *k, *v;
    const float *alpha, *beta;
    float *out;
    int tiles;     // B * H
    int xcd_run;   // see xcd_block
    int xcd_full;
};

template <int DK>
struct alignas(16) WinLds {
    uint16_t k[DK], q[DK], v[DK];  // the token (bf16 bits)
    float kd[WMAX_S], qd[WMAX_S];  // window entry e (oldest first): delta_e (k_e . k), delta_e (k_e . q)
    float fk[WMAX_S], su[WMAX_S];  // entry e: k scale * decay, w scale
    float wk[DK], wq[DK];          // per column: window terms of M^T k and M^T q
    float wo[DK];                  // per column: delta_o alpha w_o (full window)
    float kw[DK];                  // the leaving key k_o (full window)
    float u[DK], o[DK];            // per column: u_t and the output
};

__device__ inline float sfirst(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

template <int DK, int BITS, bool ERR>
__device__ void window_tile(const WinArgs &a, WinLds<DK> &L, int b, int h, int slot, int lane) {
    constexpr int NKS = CodeChunk<DK>::NKS;
    constexpr int NRT = CodeChunk<DK>::NRT;
    constexpr int NCB = DK / 16;
    constexpr int CPL = DK / 64;  // columns (and token elements) per lane in the row passes
    constexpr int BPL = DK / 8;   // key bytes per lane in the window's key dot products
    constexpr float QMAX = BITS == 4 ? 7.f : 127.f;
    constexpr float KAPPA = Loader<DK, BITS>::KAPPA;
    constexpr int PF = 2;
    const int g = lane >> 4, n = lane & 15;
    const size_t tile_row = (size_t)b * a.p.H + h;
    const WindowView &wv = a.wv;
    const int S = wv.S;
    const int cnt = __builtin_amdgcn_readfirstlane(wv.count[tile_row]);
    const int head = __builtin_amdgcn_readfirstlane(wv.head[tile_row]);
    const float lam = sfirst(wv.lam[tile_row]);
    const bool full = cnt == S;
    constexpr size_t ROW = 2 * DK;  // bytes per window entry: k codes, then w codes
    uint8_t *wc = wv.codes + tile_row * S * ROW;
    float *wf = wv.f + tile_row * S * 3;  // per slot: k scale, w scale, decay
    auto slot_of = [&](int e) {
        const int sl = head + e;
        return sl >= S ? sl - S : sl;
    };

    uint8_t *codes = BITS == 4
        ? a.p.codes4 + ((size_t)b * a.p.n4 + slot) * tile_code_bytes(DK, DK, 4)
        : a.p.codes8 + ((size_t)b * a.p.n8 + slot) * tile_code_bytes(DK, DK, 8);
    float *scl = a.p.scales + tile_row * DK;

    // ---- every load of the prologue before its first use: the codes of the
    //      first blocks, the token, each entry's scales and decay, the first
    //      eight entries' key slices and w bytes, the leaving key ----
    Loader<DK, BITS> ring[PF];
    float sring[PF];
#pragma unroll
    for (int c = 0; c < PF; ++c) {
        ring[c].load(codes, c, lane);
        sring[c] = scl[16 * c + n];
    }
    const float al = sfirst(a.alpha[tile_row]), be = sfirst(a.beta[tile_row]);
    uint32_t tk, tq, tv;  // CPL bf16 values each
    {
        const size_t o = tile_row * DK + CPL * lane;
        if constexpr (CPL == 2) {
            tk = *(const uint32_t *)(a.k + o);
            tq = *(const uint32_t *)(a.q + o);
            tv = *(const uint32_t *)(a.v + o);
        } else {
            tk = a.k[o];
            tq = a.q[o];
            tv = a.v[o];
        }
    }
    // entry e = lane (oldest first): k scale, w scale, decay
    float e_sk = 0.f, e_su = 0.f, e_dl = 0.f;
    if (lane < cnt) {
        const int sl = slot_of(lane);
        e_sk = wf[3 * sl];
        e_su = wf[3 * sl + 1];
        e_dl = wf[3 * sl + 2];
    }
    auto load_keys = [&](int e0, uint32_t (&kc)[BPL / 4]) {
        const int e = e0 + (lane >> 3);
        const uint8_t *c = wc + slot_of(e < cnt ? e : 0) * ROW + (lane & 7) * BPL;
        if constexpr (BPL == 16) {
            const u32x4 x = *(const u32x4 *)c;
            kc[0] = x[0], kc[1] = x[1], kc[2] = x[2], kc[3] = x[3];
        } else {
            const u32x2 x = *(const u32x2 *)c;
            kc[0] = x[0], kc[1] = x[1];
        }
    };
    auto load_w = [&](int e0, uint32_t (&cw)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint8_t *c = wc + slot_of(e0 + i < cnt ? e0 + i : 0) * ROW + DK + CPL * lane;
            cw[i] = CPL == 2 ? (uint32_t) * (const uint16_t *)c : (uint32_t)*c;
        }
    };
    uint32_t kc0[BPL / 4], cw0[8];
    uint32_t kwb = 0;  // the leaving key, bytes CPL * lane ..
    if (cnt > 0) {
        load_keys(0, kc0);
        load_w(0, cw0);
        if (full) {
            const uint8_t *c = wc + head * ROW + CPL * lane;
            kwb = CPL == 2 ? (uint32_t) * (const uint16_t *)c : (uint32_t)*c;
        }
    }

    // ---- the token in LDS, k . q ----
    float kq;
    if constexpr (CPL == 2) {
        *(uint32_t *)&L.k[2 * lane] = tk;
        *(uint32_t *)&L.q[2 * lane] = tq;
        *(uint32_t *)&L.v[2 * lane] = tv;
        kq = fmaf(lo_f32(tk), lo_f32(tq), hi_f32(tk) * hi_f32(tq));
    } else {
        L.k[lane] = (uint16_t)tk;
        L.q[lane] = (uint16_t)tq;
        L.v[lane] = (uint16_t)tv;
        kq = bf2f((uint16_t)tk) * bf2f((uint16_t)tq);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) kq += __shfl_xor(kq, m);
    if (lane < cnt) {
        L.fk[lane] = e_sk * e_dl;
        L.su[lane] = e_su;
    }
    if (full) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) L.kw[CPL * lane + c] = e4m3_decode(kwb >> (8 * c)) * sfirst(e_sk);
    }
    wave_sync();

    // ---- window keys against the token: 8 lanes per entry, 8 entries a round ----
    {
        const int p = lane & 7;
        float tkf[BPL], tqf[BPL];
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            tkf[i] = bf2f(L.k[p * BPL + i]);
            tqf[i] = bf2f(L.q[p * BPL + i]);
        }
        for (int e0 = 0; e0 < cnt; e0 += 8) {
            uint32_t kc[BPL / 4];
            if (e0 == 0) {
#pragma unroll
                for (int i = 0; i < BPL / 4; ++i) kc[i] = kc0[i];
            } else {
                load_keys(e0, kc);
            }
            float kd = 0.f, qd = 0.f;
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                const float x = e4m3_decode(kc[i >> 2] >> (8 * (i & 3)));
                kd = fmaf(x, tkf[i], kd);
                qd = fmaf(x, tqf[i], qd);
            }
#pragma unroll
            for (int m = 1; m < 8; m <<= 1) {
                kd += __shfl_xor(kd, m);
                qd += __shfl_xor(qd, m);
            }
            const int e = e0 + (lane >> 3);
            if (p == 0 && e < cnt) {
                L.kd[e] = kd * L.fk[e];
                L.qd[e] = qd * L.fk[e];
            }
        }
    }
    wave_sync();

    // ---- per column: the window's terms, and the leaving write ----
    {
        float wk[CPL] = {}, wq[CPL] = {};
        for (int e0 = 0; e0 < cnt; e0 += 8) {
            uint32_t cw[8];
            if (e0 == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) cw[i] = cw0[i];
            } else {
                load_w(e0, cw);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (e0 + i < cnt) {
                    const float kde = L.kd[e0 + i], qde = L.qd[e0 + i], su = L.su[e0 + i];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const float w = e4m3_decode(cw[i] >> (8 * c)) * su;
                        wk[c] = fmaf(kde, w, wk[c]);
                        wq[c] = fmaf(qde, w, wq[c]);
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            L.wk[CPL * lane + c] = wk[c];
            L.wq[CPL * lane + c] = wq[c];
        }
        if (full) {
            // oldest entry (e = 0): w scale * decay after this step
            const float f = L.su[0] * (sfirst(e_dl) * al);
#pragma unroll
            for (int c = 0; c < CPL; ++c) L.wo[CPL * lane + c] = e4m3_decode(cw0[0] >> (8 * c)) * f;
        }
    }
    // [k; q] as the MFMA A operand: rows 4 gg hold k, rows 4 gg + 1 hold q
    // (every lane group then receives both products of its column); k index
    // e of slice ks is state row 32 ks + 16 (e / 4) + 4 g + e % 4
    bf16x8 AP[NKS];
    {
        const int sel = n & 3;
        const uint16_t *src = sel == 0 ? L.k : L.q;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int c0 = 32 * ks + 4 * g, c1 = c0 + 16;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (sel < 2) {
                const u32x2 r0 = *(const u32x2 *)&src[c0];
                const u32x2 r1 = *(const u32x2 *)&src[c1];
                w = u32x4{r0[0], r0[1], r1[0], r1[1]};
            }
            AP[ks] = __builtin_bit_cast(bf16x8, w);
        }
    }
    wave_sync();

    const float lam_al = lam * al;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        asm volatile("" ::: "memory");
        const int j = 16 * cb + n;
        const int rs = cb % PF;
        const float s = sring[rs];
        f32x4 acc[NRT];
        ring[rs].codes_f32(acc);
        if (cb + PF < NCB) {
            ring[rs].load(codes, cb + PF, lane);
            sring[rs] = scl[j + 16 * PF];
        }
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4 w = {pk_bf16(acc[2 * ks][0], acc[2 * ks][1]), pk_bf16(acc[2 * ks][2], acc[2 * ks][3]),
                       pk_bf16(acc[2 * ks + 1][0], acc[2 * ks + 1][1]),
                       pk_bf16(acc[2 * ks + 1][2], acc[2 * ks + 1][3])};
            P = mfma_bf16_k32(AP[ks], __builtin_bit_cast(bf16x8, w), P);
        }
        // P[0] = KAPPA (c_j . k), P[1] = KAPPA (c_j . q)
        const float hs = lam * s * (1.f / KAPPA);  // exact scaling by a power of two
        const float d = fmaf(hs, P[0], L.wk[j]);
        const float u = be * (bf2f(L.v[j]) - al * d);
        const float o = fmaf(kq, u, al * fmaf(hs, P[1], L.wq[j]));
        if (g == 0) {
            L.u[j] = u;
            L.o[j] = o;
        }
        if (full) {
            // H' / sigma = KAPPA c + (delta_o alpha w_o[j] / sigma) k_o
            const float sig_raw = lam_al * s;
            const bool tiny = s > 0.f && !(sig_raw >= 1.17549435e-38f);
            const float sig = ((s > 0.f && !tiny) ? sig_raw : 1.f) * (1.f / KAPPA);
            if (__builtin_amdgcn_ballot_w64(tiny)) {
                // decay below float32's normal range: start from lam alpha s c directly
                const float m0 = tiny ? sig_raw : 1.f;
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) acc[rt] *= m0;
            }
            const float bco = L.wo[j] * __builtin_amdgcn_rcpf(sig);
            float am = 0.f;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const f32x4 kw = *(const f32x4 *)&L.kw[16 * rt + 4 * g];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[rt][r] = fmaf(bco, kw[r], acc[rt][r]);
                    am = fmaxf(am, fabsf(acc[rt][r]));
                }
            }
            am = xor_max(am, 16);
            am = xor_max(am, 32);
            const float s_new = (am * sig) * (1.f / QMAX);
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
    wave_sync();

    // ---- outputs, and the new write (k_t, u_t) in E4M3 with one scale per vector ----
    const int slot_new = slot_of(cnt);  // == head when the window is full
    {
        float ov[CPL], kv[CPL], uv[CPL];
        float ka = 0.f, ua = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int i = CPL * lane + c;
            ov[c] = L.o[i];
            kv[c] = bf2f(L.k[i]);
            uv[c] = L.u[i];
            ka = fmaxf(ka, fabsf(kv[c]));
            ua = fmaxf(ua, fabsf(uv[c]));
        }
        float *orow = a.out + tile_row * DK + CPL * lane;
        if constexpr (CPL == 2)
            __builtin_nontemporal_store(f32x2{ov[0], ov[1]}, (f32x2 *)orow);
        else
            __builtin_nontemporal_store(ov[0], orow);
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            ka = fmaxf(ka, __shfl_xor(ka, m));
            ua = fmaxf(ua, __shfl_xor(ua, m));
        }
        const float s_k = ka / E4M3_MAX, s_u = ua / E4M3_MAX;
        uint32_t ck = 0, cu = 0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (s_k > 0.f) ck |= (uint32_t)e4m3_encode(fminf(fmaxf(kv[c] / s_k, -E4M3_MAX), E4M3_MAX)) << (8 * c);
            if (s_u > 0.f) cu |= (uint32_t)e4m3_encode(fminf(fmaxf(uv[c] / s_u, -E4M3_MAX), E4M3_MAX)) << (8 * c);
        }
        uint8_t *cn = wc + slot_new * ROW + CPL * lane;
        if constexpr (CPL == 2) {
            *(uint16_t *)cn = (uint16_t)ck;
            *(uint16_t *)(cn + DK) = (uint16_t)cu;
        } else {
            cn[0] = (uint8_t)ck;
            cn[DK] = (uint8_t)cu;
        }
        // decays of the entries that stay (entry e = lane), then the new
        // entry and the window's bookkeeping
        if (lane < cnt && !(full && lane == 0)) wf[3 * slot_of(lane) + 2] = e_dl * al;
        if (lane == 0) {
            wf[3 * slot_new] = s_k;
            wf[3 * slot_new + 1] = s_u;
            wf[3 * slot_new + 2] = 1.f;
            if (full) {
                wv.head[tile_row] = head + 1 == S ? 0 : head + 1;
                wv.lam[tile_row] = 1.f;
            } else {
                wv.count[tile_row] = cnt + 1;
                wv.lam[tile_row] = lam_al;
            }
        }
    }
}

template <int DK, bool ERR>
__global__ void __launch_bounds__(64 * WTPB) __attribute__((amdgpu_waves_per_eu(ERR ? 3 : 4))) window_mfma_kernel(WinArgs a) {
    __shared__ WinLds<DK> lds[WTPB];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = xcd_block(blockIdx.x, a.xcd_run, a.xcd_full) * WTPB + wave;
    if (w >= a.tiles) return;
    const int b = w / a.p.H, h = w - b * a.p.H;
    if (a.wv.active && !a.wv.active[b]) return;  // this sequence takes no token
    const int m = a.p.head_map[h];               // slot | bits << 16
    if ((m >> 16) == 8)
        window_tile<DK, 8, ERR>(a, lds[wave], b, h, m & 0xffff, lane);
    else
        window_tile<DK, 4, ERR>(a, lds[wave], b, h, m & 0xffff, lane);
}

}  // namespace

bool window_mfma_supported(int dk, int dv, int in_bf16, int S) {
    return in_bf16 && dk == dv && (dk == 128 || dk == 64) && S >= 1 && S <= WMAX_S;
}

hipError_t launch_window_step_mfma(const PoolView &p, const WindowView &wv, const void *q,
                                   const void *k, const void *v, const float *alpha,
                                   const float *beta, float *out, hipStream_t s) {
    WinArgs a = {};
    a.p = p;
    a.wv = wv;
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.alpha = alpha;
    a.beta = beta;
    a.out = out;
    a.tiles = p.B * p.H;
    const int K = xcd_run_for(p.H, WTPB);
    const long long whole = a.tiles / WTPB;
    a.xcd_run = K;
    a.xcd_full = (int)(whole / (8ll * K) * (8ll * K));
    const dim3 grid((a.tiles + WTPB - 1) / WTPB), block(64 * WTPB);
    const bool err = p.colerr != nullptr;
    if (p.dk == 128) {
        if (err)
            hipLaunchKernelGGL((window_mfma_kernel<128, true>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((window_mfma_kernel<128, false>), grid, block, 0, s, a);
    } else {
        if (err)
            hipLaunchKernelGGL((window_mfma_kernel<64, true>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((window_mfma_kernel<64, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace pace
