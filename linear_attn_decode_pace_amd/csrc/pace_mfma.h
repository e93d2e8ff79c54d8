// Fused MFMA decode kernels for gfx950 (decode_mfma.hip: chunks of up to 8
// tokens; decode_mfma16.hip: 9..16).
#pragma once

#include "pace_layout.h"

namespace pace {

// True when the fused kernel covers this shape (bf16 inputs, d_k = d_v = 128
// or 64, n_tok within the kernel's chunk, B * H small enough for 32-bit lane
// offsets); rows_per_token = B * H.
bool mfma_supported(int dk, int dv, int n_tok, int in_bf16, long long rows_per_token);

// heads8 / heads4: device [n8] / [n4], the head of each slot of the 8-bit /
// 4-bit pool.
hipError_t launch_decode_mfma(const PoolView &p, const int32_t *heads8, const int32_t *heads4,
                              int n_tok, const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta, float *out, hipStream_t s);

}  // namespace pace
