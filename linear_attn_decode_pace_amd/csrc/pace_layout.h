// Device layout of the quantized state pools and the views kernels receive.
//
// One (sequence, head) state M is d_k x d_v (rows = key channels i, columns =
// value channels j).  Its codes are stored in a layout chosen for the MFMA
// decode kernel: the state is cut into column blocks of 16 columns
// (cb = j / 16), and inside a column block into 64 "lane chunks", one per
// lane of a 64-wide wavefront.  Lane l = 16 * g + n owns column n of the block
// and the rows i with (i / 4) % 4 == g, which are exactly the rows a lane holds
// of a 16x16 MFMA accumulator tile, for all d_k / 16 row tiles rt = i / 16.
//
//   4-bit pool: a lane chunk is d_k / 8 bytes = d_k / 32 dwords.  Dword ks
//     (k-slice of 32 rows: row tiles 2ks and 2ks+1) holds, in byte r (0..3),
//     the code of row 16*(2ks) + 4g + r in the low nibble and the code of row
//     16*(2ks+1) + 4g + r in the high nibble.  Codes are two's complement.
//     A column block is 64 * d_k / 8 bytes, contiguous per lane chunk.
//   8-bit pool: a lane chunk is d_k / 4 bytes; byte r of dword rt holds the
//     code of row 16 rt + 4g + r.  Lane chunks are split in quads of 4 dwords
//     (16 bytes) so one 16-byte load per lane reads 1 KiB contiguous:
//     offset = cb * (64 * d_k / 4) + (rt / 4) * 1024 + l * 16 + (rt % 4) * 4 + r.
//   Scales: float32 [B, H, d_v] for all heads, column order.
//
// Pools: codes4 [B, n4, tile4], codes8 [B, n8, tile8] where n4 / n8 are the
// number of 4-bit / 8-bit heads and a head's slot is its rank among heads of
// the same width.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace pace {

struct PoolView {
    uint8_t *codes4;
    uint8_t *codes8;
    float *scales;
    const int32_t *head_map;  // device [H]: slot | (bits << 16)
    // device float32 [B, H, d_v, 2] or NULL: per column, the sums over its
    // rows of (M - c s)^2 and M^2 at the column's last encode (error statistics)
    float *colerr;
    int B, H, dk, dv, n4, n8;
};

__host__ __device__ inline size_t tile_code_bytes(int dk, int dv, int bits) {
    return (size_t)dk * dv * bits / 8;
}

// byte offset and nibble shift of code (i, j) inside a 4-bit tile
__host__ __device__ inline size_t loc4(int dk, int i, int j, int *shift) {
    int cb = j >> 4, n = j & 15, rt = i >> 4, g = (i >> 2) & 3, r = i & 3;
    int lane = g * 16 + n;
    *shift = (rt & 1) * 4;
    return (size_t)cb * (64 * (dk / 8)) + (size_t)lane * (dk / 8) + (rt >> 1) * 4 + r;
}

// byte offset of code (i, j) inside an 8-bit tile
__host__ __device__ inline size_t loc8(int dk, int i, int j) {
    int cb = j >> 4, n = j & 15, rt = i >> 4, g = (i >> 2) & 3, r = i & 3;
    int lane = g * 16 + n;
    return (size_t)cb * (64 * (dk / 4)) + (size_t)(rt >> 2) * 1024 + (size_t)lane * 16 +
           (rt & 3) * 4 + r;
}

__device__ inline uint8_t *tile_codes(const PoolView &p, int b, int h, int *bits) {
    int m = p.head_map[h];
    int slot = m & 0xffff;
    *bits = m >> 16;
    if (*bits == 4)
        return p.codes4 + ((size_t)b * p.n4 + slot) * tile_code_bytes(p.dk, p.dv, 4);
    return p.codes8 + ((size_t)b * p.n8 + slot) * tile_code_bytes(p.dk, p.dv, 8);
}

// ---- launchers (defined in the .hip files) --------------------------------

hipError_t launch_decode_v0(const PoolView &p, int n_tok, const void *q, const void *k,
                            const void *v, const float *alpha, const float *beta, float *out,
                            int in_bf16, hipStream_t s);
hipError_t launch_encode_f32(const PoolView &p, const float *src, hipStream_t s);
hipError_t launch_prefill_v0(int B, int H, int dk, int dv, int n_tok, int in_bf16,
                             const void *q, const void *k, const void *v, const float *alpha,
                             const float *beta, float *state, float *out, hipStream_t s);
hipError_t launch_read(const PoolView &p, int what, void *dst, float *scales_dst,
                       hipStream_t s);
hipError_t launch_count_zero_scales(const PoolView &p, unsigned long long *counter,
                                    hipStream_t s);
// streaming copy of `bytes` (a multiple of 16) between 16-byte aligned buffers
hipError_t launch_stream_copy(void *dst, const void *src, size_t bytes, hipStream_t s);
// heads the statistics scratch of the allocation-free stats entry point holds
constexpr int STATS_SCRATCH_HEADS = 256;
// device address of that scratch on `device` (looked up once per device): a
// zero-column counter, then 2 * STATS_SCRATCH_HEADS float64 error sums
hipError_t stats_scratch(int device, unsigned long long **out);
// per head h: out[2 h] = sum of colerr[b, h, j, 0], out[2 h + 1] = sum of
// colerr[b, h, j, 1] over b and j, in float64
hipError_t launch_reduce_colerr(const PoolView &p, double *out, hipStream_t s);

}  // namespace pace
