// Straightforward HIP kernels: one thread per state column.
//
// These are the reference-shaped device kernels: the period decode applies
// tokens one at a time with the gated delta rule in float32 (the recurrence
// in the form M_t = alpha (M - beta k (k^T M)) + beta k v^T, o_t = M_t^T q_t),
// the encoder implements the per-column absmax quantizer, and the read and
// prefill kernels serve checkpointing and warm-up.  The fused MFMA kernel in
// decode_mfma.hip is the fast path; this file is its second opinion and the
// fallback for shapes it does not cover (float32 inputs, d_v not 128).
//
// A thread owns one column j of one (sequence, head) state, so every code
// byte it reads or writes belongs to its column only (see pace_layout.h) and
// decode can update the pool in place without synchronisation between threads.
#include <mutex>

#include "column_codec.h"
#include "pace_step.h"

namespace pace {
namespace {

// Apply tokens t = 0..n_tok-1 to the column held in M; writes o_t if out != NULL.
template <int DK>
__device__ inline void apply_tokens(float M[DK], float *sk, float *sq, int n_tok, int B, int H,
                                    int dv, int b, int h, int j, const void *q, const void *k,
                                    const void *v, const float *alpha, const float *beta,
                                    float *out, int bf16) {
    for (int t = 0; t < n_tok; ++t) {
        size_t base = (((size_t)t * B + b) * H + h);
        __syncthreads();
        for (int i = threadIdx.x; i < DK; i += blockDim.x) {
            sk[i] = ld_in(k, base * DK + i, bf16);
            sq[i] = ld_in(q, base * DK + i, bf16);
        }
        __syncthreads();
        const float a = alpha[base], bt = beta[base];
        const float vj = ld_in(v, base * dv + j, bf16);
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) d = fmaf(sk[i], M[i], d);
        float o = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            float bk = bt * sk[i];
            M[i] = a * (M[i] - bk * d) + bk * vj;
            o = fmaf(sq[i], M[i], o);
        }
        if (out) out[base * dv + j] = o;
    }
}

template <int DK>
__global__ void __launch_bounds__(256) decode_v0_kernel(PoolView p, int n_tok, const void *q, const void *k,
                                 const void *v, const float *alpha, const float *beta,
                                 float *out, int bf16) {
    __shared__ float sk[DK], sq[DK];
    const int tile = blockIdx.x, b = tile / p.H, h = tile % p.H, j = threadIdx.x;
    int bits;
    uint8_t *codes = tile_codes(p, b, h, &bits);
    float *sc = p.scales + (size_t)tile * p.dv;
    float M[DK];
    load_column<DK>(codes, bits, j, sc[j], M);
    apply_tokens<DK>(M, sk, sq, n_tok, p.B, p.H, p.dv, b, h, j, q, k, v, alpha, beta, out, bf16);
    sc[j] = store_column<DK>(codes, bits, j, M,
                             p.colerr ? p.colerr + ((size_t)tile * p.dv + j) * 2 : nullptr);
}

template <int DK>
__global__ void __launch_bounds__(256) encode_f32_kernel(PoolView p, const float *src) {
    const int tile = blockIdx.x, b = tile / p.H, h = tile % p.H, j = threadIdx.x;
    int bits;
    uint8_t *codes = tile_codes(p, b, h, &bits);
    const float *m = src + (size_t)tile * DK * p.dv;
    float M[DK];
#pragma unroll
    for (int i = 0; i < DK; ++i) M[i] = m[(size_t)i * p.dv + j];
    p.scales[(size_t)tile * p.dv + j] = store_column<DK>(
        codes, bits, j, M, p.colerr ? p.colerr + ((size_t)tile * p.dv + j) * 2 : nullptr);
}

template <int DK>
__global__ void __launch_bounds__(256) prefill_v0_kernel(int B, int H, int dv, int n_tok, int bf16, const void *q,
                                  const void *k, const void *v, const float *alpha,
                                  const float *beta, float *state, float *out) {
    __shared__ float sk[DK], sq[DK];
    const int tile = blockIdx.x, b = tile / H, h = tile % H, j = threadIdx.x;
    float *m = state + (size_t)tile * DK * dv;
    float M[DK];
#pragma unroll
    for (int i = 0; i < DK; ++i) M[i] = m[(size_t)i * dv + j];
    apply_tokens<DK>(M, sk, sq, n_tok, B, H, dv, b, h, j, q, k, v, alpha, beta, out, bf16);
#pragma unroll
    for (int i = 0; i < DK; ++i) m[(size_t)i * dv + j] = M[i];
}

// what: 0 = codes to int8 [B,H,dk,dv] + scales, 1 = dequantized float32
template <int DK>
__global__ void __launch_bounds__(256) read_kernel(PoolView p, int what, void *dst, float *sdst) {
    const int tile = blockIdx.x, b = tile / p.H, h = tile % p.H, j = threadIdx.x;
    int bits;
    const uint8_t *codes = tile_codes(p, b, h, &bits);
    const float s = p.scales[(size_t)tile * p.dv + j];
    for (int i = 0; i < DK; ++i) {
        int c;
        if (bits == 4) {
            int sh;
            size_t o = loc4(DK, i, j, &sh);
            c = ((int)((uint32_t)codes[o] << (28 - sh))) >> 28;
        } else {
            c = (int)(int8_t)codes[loc8(DK, i, j)];
        }
        size_t o = ((size_t)tile * DK + i) * p.dv + j;
        if (what == 0)
            ((int8_t *)dst)[o] = (int8_t)c;
        else
            ((float *)dst)[o] = (float)c * s;
    }
    if (sdst) sdst[(size_t)tile * p.dv + j] = s;
}

__global__ void count_zero_kernel(const float *scales, size_t n, unsigned long long *counter) {
    unsigned int mine = 0;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        mine += scales[i] == 0.f;
    for (int off = 32; off > 0; off >>= 1) mine += __shfl_xor(mine, off);
    if ((threadIdx.x & 63) == 0 && mine) atomicAdd(counter, (unsigned long long)mine);
}

// ---- per-step decode (PACE_STEP_BUFFER) ----------------------------------

__device__ inline void copy_in(void *dst, size_t di, const void *src, size_t si, int bf16) {
    if (bf16)
        ((uint16_t *)dst)[di] = ((const uint16_t *)src)[si];
    else
        ((float *)dst)[di] = ((const float *)src)[si];
}

// Apply buffered tokens 0..f-1 of state `tile` and then, if cur_k != NULL, the
// step's own token (whose output is written); column j per thread, as
// apply_tokens.
// u_cur (if not NULL) receives this thread's entry u_j = beta (v_j - alpha d_j)
// of the step token's write.
template <int DK>
__device__ inline void apply_buffered(float M[DK], float *sk, float *sq, const StepView &sv,
                                      int tile, int dv, int j, int f, const void *q,
                                      const void *cur_k, const void *v, const float *alpha,
                                      const float *beta, float *out, int bf16,
                                      float *u_cur = nullptr) {
    const size_t row = (size_t)DK + dv;  // elements per buffered token
    const int last = cur_k ? f : f - 1;
    for (int t = 0; t <= last; ++t) {
        const bool cur = t == f;
        const size_t slot = (size_t)tile * sv.slots + t;
        __syncthreads();
        for (int i = threadIdx.x; i < DK; i += blockDim.x) {
            sk[i] = cur ? ld_in(cur_k, (size_t)tile * DK + i, bf16) : ld_in(sv.kv, slot * row + i, bf16);
            if (cur) sq[i] = ld_in(q, (size_t)tile * DK + i, bf16);
        }
        __syncthreads();
        const float a = cur ? alpha[tile] : sv.ab[2 * slot];
        const float bt = cur ? beta[tile] : sv.ab[2 * slot + 1];
        const float vj = cur ? ld_in(v, (size_t)tile * dv + j, bf16) : ld_in(sv.kv, slot * row + DK + j, bf16);
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) d = fmaf(sk[i], M[i], d);
        float o = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            float bk = bt * sk[i];
            M[i] = a * (M[i] - bk * d) + bk * vj;
            o = fmaf(sq[i], M[i], o);
        }
        if (cur) {
            out[(size_t)tile * dv + j] = o;
            if (u_cur) *u_cur = bt * (vj - a * d);
        }
    }
}

template <int DK>
__global__ void __launch_bounds__(256) step_v0_kernel(PoolView p, StepView sv, const void *q, const void *k,
                               const void *v, const float *alpha, const float *beta, float *out,
                               int bf16) {
    __shared__ float sk[DK], sq[DK], red[4];
    const int tile = blockIdx.x, b = tile / p.H, h = tile % p.H, j = threadIdx.x;
    if (sv.active && !sv.active[b]) return;
    const int f = sv.fill[tile];
    const bool adaptive = sv.tau > 0.f;
    const float A = adaptive ? sv.adapt[2 * tile] : 0.f, R = adaptive ? sv.adapt[2 * tile + 1] : 0.f;
    const bool close = f + 1 == sv.period || (adaptive && A > sv.tau * R);
    int bits;
    uint8_t *codes = tile_codes(p, b, h, &bits);
    float *sc = p.scales + (size_t)tile * p.dv;
    float M[DK];
    load_column<DK>(codes, bits, j, sc[j], M);
    float u = 0.f;
    apply_buffered<DK>(M, sk, sq, sv, tile, p.dv, j, f, q, k, v, alpha, beta, out, bf16, &u);
    // every thread has read fill[tile] and adapt[] before the first barrier inside apply_buffered
    if (close) {
        float q2 = 0.f;
        sc[j] = store_column<DK>(codes, bits, j, M,
                                 p.colerr ? p.colerr + ((size_t)tile * p.dv + j) * 2 : nullptr, &q2);
        if (adaptive) {
            const float r2 = block_sum(q2, red);
            if (j == 0) {
                sv.adapt[2 * tile] = 0.f;
                sv.adapt[2 * tile + 1] = sqrtf(r2);
            }
        }
        if (j == 0) sv.fill[tile] = 0;
    } else {
        if (adaptive) {
            // A += ||k_f|| ||u_f||; sk still holds k_f
            const float u2 = block_sum(u * u, red);
            if (j == 0) {
                float k2 = 0.f;
                for (int i = 0; i < DK; ++i) k2 = fmaf(sk[i], sk[i], k2);
                sv.adapt[2 * tile] = A + sqrtf(k2) * sqrtf(u2);
            }
        }
        const size_t slot = (size_t)tile * sv.slots + f, row = (size_t)DK + p.dv;
        for (int i = j; i < DK; i += blockDim.x) copy_in(sv.kv, slot * row + i, k, (size_t)tile * DK + i, bf16);
        copy_in(sv.kv, slot * row + DK + j, v, (size_t)tile * p.dv + j, bf16);
        if (j == 0) {
            sv.ab[2 * slot] = alpha[tile];
            sv.ab[2 * slot + 1] = beta[tile];
            sv.fill[tile] = f + 1;
        }
    }
}

template <int DK>
__global__ void __launch_bounds__(256) flush_v0_kernel(PoolView p, StepView sv, int bf16) {
    __shared__ float sk[DK], sq[DK], red[4];
    const int tile = blockIdx.x, b = tile / p.H, h = tile % p.H, j = threadIdx.x;
    const int f = sv.fill[tile];
    if (f == 0) return;
    int bits;
    uint8_t *codes = tile_codes(p, b, h, &bits);
    float *sc = p.scales + (size_t)tile * p.dv;
    float M[DK];
    load_column<DK>(codes, bits, j, sc[j], M);
    apply_buffered<DK>(M, sk, sq, sv, tile, p.dv, j, f, nullptr, nullptr, nullptr, nullptr,
                       nullptr, nullptr, bf16);
    float q2 = 0.f;
    sc[j] = store_column<DK>(codes, bits, j, M,
                             p.colerr ? p.colerr + ((size_t)tile * p.dv + j) * 2 : nullptr, &q2);
    if (sv.tau > 0.f) {
        const float r2 = block_sum(q2, red);
        if (j == 0) {
            sv.adapt[2 * tile] = 0.f;
            sv.adapt[2 * tile + 1] = sqrtf(r2);
        }
    }
    if (j == 0) sv.fill[tile] = 0;
}

// adapt[2 t] = 0, adapt[2 t + 1] = ||decode(stored state t)||_F
template <int DK>
__global__ void __launch_bounds__(256) adapt_init_kernel(PoolView p, float *adapt) {
    __shared__ float red[4];
    const int tile = blockIdx.x, b = tile / p.H, h = tile % p.H, j = threadIdx.x;
    int bits;
    const uint8_t *codes = tile_codes(p, b, h, &bits);
    float M[DK];
    load_column<DK>(codes, bits, j, p.scales[(size_t)tile * p.dv + j], M);
    float m2 = 0.f;
#pragma unroll
    for (int i = 0; i < DK; ++i) m2 = fmaf(M[i], M[i], m2);
    const float r2 = block_sum(m2, red);
    if (j == 0) {
        adapt[2 * tile] = 0.f;
        adapt[2 * tile + 1] = sqrtf(r2);
    }
}

// one block per head; float64 sums over sequences and columns
__global__ void reduce_colerr_kernel(const float *colerr, int B, int H, int dv, double *out) {
    __shared__ double part[2][4];
    const int h = blockIdx.x;
    double e = 0.0, m = 0.0;
    for (long long idx = threadIdx.x; idx < (long long)B * dv; idx += blockDim.x) {
        const long long b = idx / dv, j = idx - b * dv;
        const float *x = colerr + (((size_t)b * H + h) * dv + j) * 2;
        e += (double)x[0];
        m += (double)x[1];
    }
    for (int off = 32; off > 0; off >>= 1) {
        e += __shfl_xor(e, off);
        m += __shfl_xor(m, off);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        part[0][wave] = e;
        part[1][wave] = m;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        out[2 * h] = part[0][0] + part[0][1] + part[0][2] + part[0][3];
        out[2 * h + 1] = part[1][0] + part[1][1] + part[1][2] + part[1][3];
    }
}

}  // namespace

hipError_t launch_decode_v0(const PoolView &p, int n_tok, const void *q, const void *k,
                            const void *v, const float *alpha, const float *beta, float *out,
                            int in_bf16, hipStream_t s) {
    dim3 grid(p.B * p.H), block(p.dv);
    if (p.dk == 128)
        hipLaunchKernelGGL(decode_v0_kernel<128>, grid, block, 0, s, p, n_tok, q, k, v, alpha,
                           beta, out, in_bf16);
    else
        hipLaunchKernelGGL(decode_v0_kernel<64>, grid, block, 0, s, p, n_tok, q, k, v, alpha,
                           beta, out, in_bf16);
    return hipGetLastError();
}

hipError_t launch_encode_f32(const PoolView &p, const float *src, hipStream_t s) {
    dim3 grid(p.B * p.H), block(p.dv);
    if (p.dk == 128)
        hipLaunchKernelGGL(encode_f32_kernel<128>, grid, block, 0, s, p, src);
    else
        hipLaunchKernelGGL(encode_f32_kernel<64>, grid, block, 0, s, p, src);
    return hipGetLastError();
}

hipError_t launch_prefill_v0(int B, int H, int dk, int dv, int n_tok, int in_bf16,
                             const void *q, const void *k, const void *v, const float *alpha,
                             const float *beta, float *state, float *out, hipStream_t s) {
    dim3 grid(B * H), block(dv);
    if (dk == 128)
        hipLaunchKernelGGL(prefill_v0_kernel<128>, grid, block, 0, s, B, H, dv, n_tok, in_bf16,
                           q, k, v, alpha, beta, state, out);
    else
        hipLaunchKernelGGL(prefill_v0_kernel<64>, grid, block, 0, s, B, H, dv, n_tok, in_bf16,
                           q, k, v, alpha, beta, state, out);
    return hipGetLastError();
}

hipError_t launch_read(const PoolView &p, int what, void *dst, float *scales_dst,
                       hipStream_t s) {
    dim3 grid(p.B * p.H), block(p.dv);
    if (p.dk == 128)
        hipLaunchKernelGGL(read_kernel<128>, grid, block, 0, s, p, what, dst, scales_dst);
    else
        hipLaunchKernelGGL(read_kernel<64>, grid, block, 0, s, p, what, dst, scales_dst);
    return hipGetLastError();
}

// Scratch of the statistics entry point that allocates nothing (for callers
// that cannot allocate device memory): word 0 counts zero columns, words
// 1 .. 2 * STATS_SCRATCH_HEADS hold the per-head float64 error sums.  One copy
// per device, held until the process ends; calls that overlap on one device
// share it and race.
static __device__ __align__(256) unsigned long long scratch[1 + 2 * STATS_SCRATCH_HEADS];

hipError_t stats_scratch(int device, unsigned long long **out) {
    // in host code `scratch` names a host-side stand-in: the device address of
    // each device's copy is looked up once, with that device current
    constexpr int MAX_DEVICES = 64;
    static std::mutex mu;
    static unsigned long long *addr[MAX_DEVICES] = {};
    if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != device) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        addr[device] = (unsigned long long *)p;
    }
    *out = addr[device];
    return hipSuccess;
}

hipError_t launch_count_zero_scales(const PoolView &p, unsigned long long *counter,
                                    hipStream_t s) {
    size_t n = (size_t)p.B * p.H * p.dv;
    int blocks = (int)((n + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(count_zero_kernel, dim3(blocks), dim3(256), 0, s, p.scales, n, counter);
    return hipGetLastError();
}

hipError_t launch_reduce_colerr(const PoolView &p, double *out, hipStream_t s) {
    hipLaunchKernelGGL(reduce_colerr_kernel, dim3(p.H), dim3(256), 0, s, p.colerr, p.B, p.H, p.dv,
                       out);
    return hipGetLastError();
}

hipError_t launch_step_v0(const PoolView &p, const StepView &sv, const void *q, const void *k,
                          const void *v, const float *alpha, const float *beta, float *out,
                          int in_bf16, hipStream_t s) {
    dim3 grid(p.B * p.H), block(p.dv);
    if (p.dk == 128)
        hipLaunchKernelGGL(step_v0_kernel<128>, grid, block, 0, s, p, sv, q, k, v, alpha, beta,
                           out, in_bf16);
    else
        hipLaunchKernelGGL(step_v0_kernel<64>, grid, block, 0, s, p, sv, q, k, v, alpha, beta,
                           out, in_bf16);
    return hipGetLastError();
}

hipError_t launch_flush_v0(const PoolView &p, const StepView &sv, int in_bf16, hipStream_t s) {
    dim3 grid(p.B * p.H), block(p.dv);
    if (p.dk == 128)
        hipLaunchKernelGGL(flush_v0_kernel<128>, grid, block, 0, s, p, sv, in_bf16);
    else
        hipLaunchKernelGGL(flush_v0_kernel<64>, grid, block, 0, s, p, sv, in_bf16);
    return hipGetLastError();
}

hipError_t launch_adapt_init(const PoolView &p, float *adapt, hipStream_t s) {
    dim3 grid(p.B * p.H), block(p.dv);
    if (p.dk == 128)
        hipLaunchKernelGGL(adapt_init_kernel<128>, grid, block, 0, s, p, adapt);
    else
        hipLaunchKernelGGL(adapt_init_kernel<64>, grid, block, 0, s, p, adapt);
    return hipGetLastError();
}

}  // namespace pace
