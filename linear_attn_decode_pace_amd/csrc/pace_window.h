// FP8 write window of a PACE_FP8_WINDOW handle (kernels_window.hip).
#pragma once

#include "pace_layout.h"

namespace pace {

struct WindowView {
    uint8_t *codes;         // [B * H][S][d_k + d_v]: E4M3 codes of k_t, then of u_t
    float *f;               // [B * H][S][3]: k scale, u scale, decay since the write
    int32_t *count;         // [B * H]: writes in the window (0 .. S)
    int32_t *head;          // [B * H]: slot of the oldest write
    float *lam;             // [B * H]: decay of the history since its last encode
    const uint8_t *active;  // device [B] or NULL
    int S;
};

hipError_t launch_window_step(const PoolView &p, const WindowView &wv, const void *q,
                              const void *k, const void *v, const float *alpha,
                              const float *beta, float *out, int in_bf16, hipStream_t s);
// The fused window step (window_mfma.hip): bf16 inputs, d_k = d_v = 64 or
// 128; other shapes take launch_window_step (one thread per column).
bool window_mfma_supported(int dk, int dv, int in_bf16, int S);
hipError_t launch_window_step_mfma(const PoolView &p, const WindowView &wv, const void *q,
                                   const void *k, const void *v, const float *alpha,
                                   const float *beta, float *out, hipStream_t s);
hipError_t launch_window_flush(const PoolView &p, const WindowView &wv, hipStream_t s);
// out[2 t] = lam[t], out[2 t + 1] = head[t] (as float), t < states
hipError_t launch_window_meta(const WindowView &wv, float *out, size_t states, hipStream_t s);

}  // namespace pace
