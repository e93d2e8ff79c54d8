// Prompt prefill straight into the quantized pools (prefill_mfma.hip).
#pragma once

#include "pace_layout.h"

namespace pace {

// True when the fused prefill covers this shape (rows_per_token = B * H).
bool prefill_mfma_supported(int dk, int dv, int in_bf16, long long rows_per_token);

// Apply n_tok tokens ([n_tok, B, H, d], bf16) to every stored state in
// float32 and encode once at the end; out ([n_tok, B, H, d_v] float32) may be
// NULL.
hipError_t launch_prefill_mfma(const PoolView &p, int n_tok, const void *q, const void *k,
                               const void *v, const float *alpha, const float *beta, float *out,
                               hipStream_t s);

}  // namespace pace
