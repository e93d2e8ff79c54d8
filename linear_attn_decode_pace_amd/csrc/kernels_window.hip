// FP8 write window over the low-bit state (PACE_FP8_WINDOW handles), one
// thread per state column: the pure-write sliding window of
// '低比特量化新突破：GGA+PW让线性注意力长文本生成更准更短', section 'PW：让近期写入走“纯净通道”'.
// The last S writes (k_t, u_t) of the delta rule, M_t = alpha_t M_{t-1} +
// k_t u_t^T with u_t = beta_t (v_t - alpha_t M_{t-1}^T k_t), are kept as OCP
// E4M3 vectors with one float32 scale each and a decay factor; the history is
// column-quantized as every other state here and decays through one factor
// lam.  When a write leaves the window it is merged into the history, which
// is then re-encoded.
#include "column_codec.h"
#include "e4m3.h"
#include "pace_window.h"

namespace pace {
namespace {

// one step for the state `tile`: thread j owns column j (blockDim = d_v)
template <int DK>
__global__ void __launch_bounds__(256) window_step_kernel(PoolView p, WindowView wv, const void *q, const void *k,
                                   const void *v, const float *alpha, const float *beta,
                                   float *out, int bf16) {
    __shared__ float sk[DK], sq[DK], kw[DK], red[4];
    const int tile = blockIdx.x, b = tile / p.H, h = tile % p.H, j = threadIdx.x;
    if (wv.active && !wv.active[b]) return;
    const int S = wv.S, cnt = wv.count[tile], head = wv.head[tile];
    const float lam = wv.lam[tile];
    const size_t row = (size_t)DK + p.dv;
    uint8_t *wc = wv.codes + (size_t)tile * S * row;
    float *wf = wv.f + (size_t)tile * S * 3;  // per slot: k scale, u scale, decay
    int bits;
    uint8_t *codes = tile_codes(p, b, h, &bits);
    float *sc = p.scales + (size_t)tile * p.dv;

    // M_{t-1}, column j: lam * history + the decayed FP8 writes of the window
    float M[DK];
    load_column<DK>(codes, bits, j, sc[j], M);
#pragma unroll
    for (int i = 0; i < DK; ++i) M[i] *= lam;
    for (int e = 0; e < cnt; ++e) {
        const int slot = (head + e) % S;
        const uint8_t *c = wc + slot * row;
        __syncthreads();
        for (int i = j; i < DK; i += blockDim.x) kw[i] = e4m3_decode(c[i]) * wf[3 * slot];
        __syncthreads();
        const float w = e4m3_decode(c[DK + j]) * wf[3 * slot + 1] * wf[3 * slot + 2];
#pragma unroll
        for (int i = 0; i < DK; ++i) M[i] = fmaf(kw[i], w, M[i]);
    }
    // this token
    for (int i = j; i < DK; i += blockDim.x) {
        sk[i] = ld_in(k, (size_t)tile * DK + i, bf16);
        sq[i] = ld_in(q, (size_t)tile * DK + i, bf16);
    }
    __syncthreads();
    const float a = alpha[tile], bt = beta[tile];
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < DK; ++i) d = fmaf(sk[i], M[i], d);
    const float u = bt * (ld_in(v, (size_t)tile * p.dv + j, bf16) - a * d);
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < DK; ++i) o = fmaf(sq[i], fmaf(a, M[i], sk[i] * u), o);
    out[(size_t)tile * p.dv + j] = o;

    // decay the history and every window entry; a full window merges its
    // oldest write (already decayed) into the history, which is re-encoded
    const float lam_new = lam * a;
    const int slot_new = (head + cnt) % S;  // == head when the window is full
    if (cnt == S) {
        const uint8_t *c = wc + head * row;
        const float delta_o = wf[3 * head + 2] * a;
        __syncthreads();
        for (int i = j; i < DK; i += blockDim.x) kw[i] = e4m3_decode(c[i]) * wf[3 * head];
        __syncthreads();
        const float w = e4m3_decode(c[DK + j]) * wf[3 * head + 1] * delta_o;
        // M is no longer needed: reuse its registers for the history column
        load_column<DK>(codes, bits, j, sc[j], M);
#pragma unroll
        for (int i = 0; i < DK; ++i) M[i] = fmaf(kw[i], w, lam_new * M[i]);
        sc[j] = store_column<DK>(codes, bits, j, M,
                              p.colerr ? p.colerr + ((size_t)tile * p.dv + j) * 2 : nullptr);
    }
    // the new write (k_t, u_t) in E4M3, one scale per vector
    float ka = 0.f;
    for (int i = j; i < DK; i += blockDim.x) ka = fmaxf(ka, fabsf(sk[i]));
    const float s_k = block_max(ka, red) / E4M3_MAX;
    const float s_u = block_max(fabsf(u), red) / E4M3_MAX;
    uint8_t *cn = wc + slot_new * row;
    for (int i = j; i < DK; i += blockDim.x)
        cn[i] = s_k > 0.f ? e4m3_encode(fminf(fmaxf(sk[i] / s_k, -E4M3_MAX), E4M3_MAX)) : 0;
    cn[DK + j] = s_u > 0.f ? e4m3_encode(fminf(fmaxf(u / s_u, -E4M3_MAX), E4M3_MAX)) : 0;
    __syncthreads();  // every thread has read the window's decay factors
    if (j == 0) {
        for (int e = 0; e < cnt; ++e) {
            const int slot = (head + e) % S;
            if (!(cnt == S && slot == head)) wf[3 * slot + 2] *= a;
        }
        wf[3 * slot_new] = s_k;
        wf[3 * slot_new + 1] = s_u;
        wf[3 * slot_new + 2] = 1.f;
        if (cnt == S) {
            wv.head[tile] = (head + 1) % S;
            wv.lam[tile] = 1.f;
        } else {
            wv.count[tile] = cnt + 1;
            wv.lam[tile] = lam_new;
        }
    }
}

// merge every window entry into the history (oldest first) and encode once
template <int DK>
__global__ void __launch_bounds__(256) window_flush_kernel(PoolView p, WindowView wv) {
    __shared__ float kw[DK];
    const int tile = blockIdx.x, b = tile / p.H, h = tile % p.H, j = threadIdx.x;
    const int S = wv.S, cnt = wv.count[tile], head = wv.head[tile];
    if (cnt == 0) return;
    const float lam = wv.lam[tile];
    const size_t row = (size_t)DK + p.dv;
    const uint8_t *wc = wv.codes + (size_t)tile * S * row;
    const float *wf = wv.f + (size_t)tile * S * 3;
    int bits;
    uint8_t *codes = tile_codes(p, b, h, &bits);
    float *sc = p.scales + (size_t)tile * p.dv;
    float H[DK];
    load_column<DK>(codes, bits, j, sc[j], H);
#pragma unroll
    for (int i = 0; i < DK; ++i) H[i] *= lam;
    for (int e = 0; e < cnt; ++e) {
        const int slot = (head + e) % S;
        const uint8_t *c = wc + slot * row;
        __syncthreads();
        for (int i = j; i < DK; i += blockDim.x) kw[i] = e4m3_decode(c[i]) * wf[3 * slot];
        __syncthreads();
        const float w = e4m3_decode(c[DK + j]) * wf[3 * slot + 1] * wf[3 * slot + 2];
#pragma unroll
        for (int i = 0; i < DK; ++i) H[i] = fmaf(kw[i], w, H[i]);
    }
    sc[j] = store_column<DK>(codes, bits, j, H,
                          p.colerr ? p.colerr + ((size_t)tile * p.dv + j) * 2 : nullptr);
    __syncthreads();
    if (j == 0) {
        wv.count[tile] = 0;
        wv.head[tile] = 0;
        wv.lam[tile] = 1.f;
    }
}

__global__ void window_meta_kernel(WindowView wv, float *out, size_t states) {
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < states) {
        out[2 * t] = wv.lam[t];
        out[2 * t + 1] = (float)wv.head[t];
    }
}

}  // namespace

hipError_t launch_window_meta(const WindowView &wv, float *out, size_t states, hipStream_t s) {
    hipLaunchKernelGGL(window_meta_kernel, dim3((unsigned)((states + 255) / 256)), dim3(256), 0, s,
                       wv, out, states);
    return hipGetLastError();
}

hipError_t launch_window_step(const PoolView &p, const WindowView &wv, const void *q,
                              const void *k, const void *v, const float *alpha,
                              const float *beta, float *out, int in_bf16, hipStream_t s) {
    dim3 grid(p.B * p.H), block(p.dv);
    if (p.dk == 128)
        hipLaunchKernelGGL(window_step_kernel<128>, grid, block, 0, s, p, wv, q, k, v, alpha,
                           beta, out, in_bf16);
    else
        hipLaunchKernelGGL(window_step_kernel<64>, grid, block, 0, s, p, wv, q, k, v, alpha,
                           beta, out, in_bf16);
    return hipGetLastError();
}

hipError_t launch_window_flush(const PoolView &p, const WindowView &wv, hipStream_t s) {
    dim3 grid(p.B * p.H), block(p.dv);
    if (p.dk == 128)
        hipLaunchKernelGGL(window_flush_kernel<128>, grid, block, 0, s, p, wv);
    else
        hipLaunchKernelGGL(window_flush_kernel<64>, grid, block, 0, s, p, wv);
    return hipGetLastError();
}

}  // namespace pace
