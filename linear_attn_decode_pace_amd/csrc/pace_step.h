// Per-step token buffer of a PACE_STEP_BUFFER handle and the launchers that
// use it (kernels_v0.hip: per-column kernels for every shape; decode_mfma.hip:
// the fused kernel for bf16 inputs, d_k = d_v = 64 or 128, periods up to 8).
#pragma once

#include "pace_layout.h"

namespace pace {

struct StepView {
    void *kv;               // in_dtype [B * H][slots][d_k + d_v]: k_t then v_t of each buffered token
    float *ab;              // float32 [B * H][slots][2]: alpha_t, beta_t
    int32_t *fill;          // [B * H]: tokens buffered per state (0 .. slots)
    const uint8_t *active;  // device [B], or NULL: sequences taking a token this step
    int slots;              // period - 1
    int period;             // the maximum period when adaptive
    // adaptive period (tau > 0): per state A (summed write norms of the
    // buffered tokens) and R (norm of the stored state at its last encode)
    float *adapt;           // [B * H][2], or NULL when tau == 0
    float tau;              // 0: fixed period
};

hipError_t launch_step_v0(const PoolView &p, const StepView &sv, const void *q, const void *k,
                          const void *v, const float *alpha, const float *beta, float *out,
                          int in_bf16, hipStream_t s);
hipError_t launch_flush_v0(const PoolView &p, const StepView &sv, int in_bf16, hipStream_t s);
// adapt[2 t] = 0, adapt[2 t + 1] = ||decode(stored state t)||_F for every state
hipError_t launch_adapt_init(const PoolView &p, float *adapt, hipStream_t s);

// True when the fused kernel covers a step of this shape (rows_per_token = B * H).
bool mfma_step_supported(int dk, int dv, int period, int in_bf16, long long rows_per_token);
hipError_t launch_step_mfma(const PoolView &p, const StepView &sv, const int32_t *heads8,
                            const int32_t *heads4, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, float *out, hipStream_t s);

}  // namespace pace
