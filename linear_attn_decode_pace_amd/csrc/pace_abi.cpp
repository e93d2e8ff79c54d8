// C ABI of the PACE decode library: argument validation, pool ownership and
// kernel dispatch.  Every check runs before the first HIP call; HIP errors are
// turned into PACE_EDEVICE / PACE_ENOMEM with a thread-local message.
#include <stdarg.h>
#include <stdio.h>

#include <new>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/pace.h"
#include "pace_layout.h"
#include "pace_mfma.h"
#include "pace_prefill.h"
#include "pace_step.h"
#include "pace_window.h"

#define PACE_API extern "C" __attribute__((visibility("default")))

struct pace_state {
    pace_config cfg;
    std::vector<uint8_t> bits;
    std::vector<int32_t> map;  // host copy of the head map
    int device = 0;
    int n4 = 0, n8 = 0;
    int32_t *d_map = nullptr;
    uint8_t *codes4 = nullptr;
    uint8_t *codes8 = nullptr;
    float *scales = nullptr;
    unsigned long long *d_counter = nullptr;
    float *colerr = nullptr;  // PACE_STATS_ERR: [B, H, d_v, 2]
    double *d_err = nullptr;  // PACE_STATS_ERR: [H, 2] per-head sums
    void *step_kv = nullptr;       // PACE_STEP_BUFFER: [B * H][period - 1][d_k + d_v] in_dtype
    float *step_ab = nullptr;      // PACE_STEP_BUFFER: [B * H][period - 1][2]
    int32_t *step_fill = nullptr;  // PACE_STEP_BUFFER: [B * H]
    float *adapt = nullptr;        // PACE_ADAPTIVE: [B * H][2] = (A, R)
    uint8_t *win_codes = nullptr;  // PACE_FP8_WINDOW: [B * H][S][d_k + d_v]
    float *win_f = nullptr;        // PACE_FP8_WINDOW: [B * H][S][3]
    int32_t *win_meta = nullptr;   // PACE_FP8_WINDOW: count [B * H], then head [B * H]
    float *win_lam = nullptr;      // PACE_FP8_WINDOW: [B * H]
    size_t bytes4 = 0, bytes8 = 0, bytes_scales = 0, bytes_step = 0;
    uint64_t periods = 0, tokens = 0;

    pace::PoolView view() const {
        pace::PoolView p;
        p.codes4 = codes4;
        p.codes8 = codes8;
        p.scales = scales;
        p.head_map = d_map;
        p.colerr = colerr;
        p.B = cfg.batch;
        p.H = cfg.heads;
        p.dk = cfg.d_k;
        p.dv = cfg.d_v;
        p.n4 = n4;
        p.n8 = n8;
        return p;
    }
    pace::StepView step_view(const uint8_t *active) const {
        pace::StepView v;
        v.kv = step_kv;
        v.ab = step_ab;
        v.fill = step_fill;
        v.active = active;
        v.slots = cfg.period - 1;
        v.period = cfg.period;
        v.adapt = adapt;
        v.tau = adapt ? cfg.adapt_tau : 0.f;
        return v;
    }
    bool stepped() const { return (cfg.flags & PACE_STEP_BUFFER) != 0; }
    bool windowed() const { return (cfg.flags & PACE_FP8_WINDOW) != 0; }
    pace::WindowView window_view(const uint8_t *active) const {
        pace::WindowView w;
        const size_t states = (size_t)cfg.batch * cfg.heads;
        w.codes = win_codes;
        w.f = win_f;
        w.count = win_meta;
        w.head = win_meta + states;
        w.lam = win_lam;
        w.active = active;
        w.S = cfg.fp8_window;
        return w;
    }
};

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return PACE_OK;
}

int hip_fail(hipError_t e, const char *what) {
    // clear the runtime's sticky last-error so that the caller's next HIP
    // launch (ours or another library's) does not report this failure again
    (void)hipGetLastError();
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
        return fail(PACE_ENOMEM, "%s: %s", what, hipGetErrorString(e));
    return fail(PACE_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_shape(int32_t batch, int32_t heads, int32_t d_k, int32_t d_v) {
    if (batch < 1 || heads < 1) return fail(PACE_EINVAL, "batch and heads must be >= 1");
    if (d_k < 1 || d_v < 1) return fail(PACE_EINVAL, "d_k and d_v must be >= 1");
    if ((int64_t)batch * heads > (int64_t)1 << 30)
        return fail(PACE_EINVAL, "batch * heads too large");
    if (d_k != 64 && d_k != 128) return fail(PACE_EUNSUPPORTED, "d_k must be 64 or 128");
    if (d_v % 16 != 0 || d_v > 256) return fail(PACE_EUNSUPPORTED, "d_v must be a multiple of 16 up to 256");
    return PACE_OK;
}

int check_dtype(int32_t dt) {
    if (dt != PACE_DTYPE_F32 && dt != PACE_DTYPE_BF16)
        return fail(PACE_EINVAL, "in_dtype must be PACE_DTYPE_F32 or PACE_DTYPE_BF16");
    return PACE_OK;
}

int check_tokens(int32_t n_tok, int32_t in_dtype, const void *q, const void *k, const void *v,
                 const float *alpha, const float *beta) {
    if (!q || !k || !v || !alpha || !beta) return fail(PACE_EINVAL, "null input pointer");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return fail(PACE_EINVAL, "q, k, v must be 16-byte aligned");
    if (!aligned(alpha, 4) || !aligned(beta, 4))
        return fail(PACE_EINVAL, "alpha, beta must be 4-byte aligned");
    (void)n_tok;
    (void)in_dtype;
    return PACE_OK;
}

}  // namespace

PACE_API int pace_abi_version(void) { return PACE_ABI_VERSION; }

PACE_API const char *pace_last_error(void) { return g_err.c_str(); }

PACE_API int pace_state_alloc(const pace_config *cfg, int init_kind, const void *init,
                              void *stream, pace_state **out) {
    if (!cfg || !out) return fail(PACE_EINVAL, "cfg and out must not be NULL");
    int rc = check_shape(cfg->batch, cfg->heads, cfg->d_k, cfg->d_v);
    if (rc) return rc;
    if (cfg->period < 1 || cfg->period > 64) return fail(PACE_EUNSUPPORTED, "period must be 1..64");
    if ((rc = check_dtype(cfg->in_dtype))) return rc;
    if (cfg->flags & ~(PACE_STATS_ERR | PACE_STEP_BUFFER | PACE_ADAPTIVE | PACE_FP8_WINDOW))
        return fail(PACE_EINVAL, "unknown flags 0x%x", cfg->flags);
    if (cfg->flags & PACE_FP8_WINDOW) {
        if (cfg->flags & (PACE_STEP_BUFFER | PACE_ADAPTIVE))
            return fail(PACE_EINVAL, "PACE_FP8_WINDOW excludes PACE_STEP_BUFFER and PACE_ADAPTIVE");
        if (cfg->fp8_window < 1 || cfg->fp8_window > 64)
            return fail(PACE_EINVAL, "fp8_window must be 1..64");
    }
    if (cfg->flags & PACE_ADAPTIVE) {
        if (!(cfg->flags & PACE_STEP_BUFFER)) return fail(PACE_EINVAL, "PACE_ADAPTIVE needs PACE_STEP_BUFFER");
        if (!(cfg->adapt_tau > 0.f) || !(cfg->adapt_tau < 3.0e38f))
            return fail(PACE_EINVAL, "adapt_tau must be finite and > 0");
    }
    if ((cfg->flags & PACE_STATS_ERR) && cfg->heads > PACE_STATS_MAX_HEADS)
        return fail(PACE_EINVAL, "PACE_STATS_ERR takes at most %d heads", PACE_STATS_MAX_HEADS);
    if (!cfg->head_bits) return fail(PACE_EINVAL, "head_bits must not be NULL");
    for (int h = 0; h < cfg->heads; ++h)
        if (cfg->head_bits[h] != 4 && cfg->head_bits[h] != 8)
            return fail(PACE_EINVAL, "head_bits[%d] = %d; must be 4 or 8", h, cfg->head_bits[h]);
    if (init_kind == PACE_INIT_ZERO) {
        if (init) return fail(PACE_EINVAL, "PACE_INIT_ZERO takes init = NULL");
    } else if (init_kind == PACE_INIT_F32) {
        if (!init || !aligned(init, 16)) return fail(PACE_EINVAL, "PACE_INIT_F32 needs a 16-byte aligned device pointer");
    } else if (init_kind == PACE_INIT_RAW) {
        if (!init) return fail(PACE_EINVAL, "PACE_INIT_RAW needs a device pointer");
    } else {
        return fail(PACE_EINVAL, "unknown init_kind %d", init_kind);
    }

    pace_state *st = new (std::nothrow) pace_state();
    if (!st) return fail(PACE_ENOMEM, "host allocation failed");
    st->cfg = *cfg;
    st->bits.assign(cfg->head_bits, cfg->head_bits + cfg->heads);
    st->cfg.head_bits = st->bits.data();
    st->map.resize(cfg->heads);
    std::vector<int32_t> h8, h4;
    for (int h = 0; h < cfg->heads; ++h) {
        int b = st->bits[h];
        int slot = b == 4 ? st->n4++ : st->n8++;
        st->map[h] = slot | (b << 16);
        (b == 4 ? h4 : h8).push_back(h);
    }
    // device copy: [H] head map, then the head of each 8-bit slot, then of each 4-bit slot
    st->map.insert(st->map.end(), h8.begin(), h8.end());
    st->map.insert(st->map.end(), h4.begin(), h4.end());
    const size_t tiles_b = (size_t)cfg->batch;
    st->bytes4 = tiles_b * st->n4 * pace::tile_code_bytes(cfg->d_k, cfg->d_v, 4);
    st->bytes8 = tiles_b * st->n8 * pace::tile_code_bytes(cfg->d_k, cfg->d_v, 8);
    st->bytes_scales = tiles_b * cfg->heads * cfg->d_v * sizeof(float);

    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    auto cleanup = [&](int code, const char *what, hipError_t err) {
        if (st->codes4) (void)hipFree(st->codes4);
        if (st->codes8) (void)hipFree(st->codes8);
        if (st->scales) (void)hipFree(st->scales);
        if (st->d_map) (void)hipFree(st->d_map);
        if (st->d_counter) (void)hipFree(st->d_counter);
        if (st->colerr) (void)hipFree(st->colerr);
        if (st->d_err) (void)hipFree(st->d_err);
        if (st->step_kv) (void)hipFree(st->step_kv);
        if (st->step_ab) (void)hipFree(st->step_ab);
        if (st->step_fill) (void)hipFree(st->step_fill);
        if (st->adapt) (void)hipFree(st->adapt);
        if (st->win_codes) (void)hipFree(st->win_codes);
        if (st->win_f) (void)hipFree(st->win_f);
        if (st->win_meta) (void)hipFree(st->win_meta);
        if (st->win_lam) (void)hipFree(st->win_lam);
        delete st;
        (void)code;
        return hip_fail(err, what);
    };
    if ((e = hipGetDevice(&st->device)) != hipSuccess) return cleanup(0, "hipGetDevice", e);
    if (st->bytes4 && (e = hipMalloc((void **)&st->codes4, st->bytes4)) != hipSuccess)
        return cleanup(0, "hipMalloc(codes4)", e);
    if (st->bytes8 && (e = hipMalloc((void **)&st->codes8, st->bytes8)) != hipSuccess)
        return cleanup(0, "hipMalloc(codes8)", e);
    if ((e = hipMalloc((void **)&st->scales, st->bytes_scales)) != hipSuccess)
        return cleanup(0, "hipMalloc(scales)", e);
    if ((e = hipMalloc((void **)&st->d_map, sizeof(int32_t) * st->map.size())) != hipSuccess)
        return cleanup(0, "hipMalloc(head map)", e);
    if ((e = hipMalloc((void **)&st->d_counter, sizeof(unsigned long long))) != hipSuccess)
        return cleanup(0, "hipMalloc(counter)", e);
    const size_t bytes_err = (size_t)cfg->batch * cfg->heads * cfg->d_v * 2 * sizeof(float);
    if (cfg->flags & PACE_STATS_ERR) {
        if ((e = hipMalloc((void **)&st->colerr, bytes_err)) != hipSuccess)
            return cleanup(0, "hipMalloc(error statistics)", e);
        if ((e = hipMalloc((void **)&st->d_err, 2 * sizeof(double) * cfg->heads)) != hipSuccess)
            return cleanup(0, "hipMalloc(error sums)", e);
        if (init_kind != PACE_INIT_F32 && (e = hipMemsetAsync(st->colerr, 0, bytes_err, s)) != hipSuccess)
            return cleanup(0, "zero error statistics", e);
    }
    if (cfg->flags & PACE_STEP_BUFFER) {
        const size_t states = (size_t)cfg->batch * cfg->heads, slots = (size_t)cfg->period - 1;
        const size_t elem = cfg->in_dtype == PACE_DTYPE_BF16 ? 2 : 4;
        const size_t b_kv = states * slots * (cfg->d_k + cfg->d_v) * elem, b_ab = states * slots * 8;
        st->bytes_step = b_kv + b_ab + states * 4;
        if (slots && (e = hipMalloc(&st->step_kv, b_kv)) != hipSuccess)
            return cleanup(0, "hipMalloc(step buffer)", e);
        if (slots && (e = hipMalloc((void **)&st->step_ab, b_ab)) != hipSuccess)
            return cleanup(0, "hipMalloc(step buffer gates)", e);
        if ((e = hipMalloc((void **)&st->step_fill, states * 4)) != hipSuccess)
            return cleanup(0, "hipMalloc(step fill)", e);
        if ((e = hipMemsetAsync(st->step_fill, 0, states * 4, s)) != hipSuccess)
            return cleanup(0, "zero step fill", e);
        if ((cfg->flags & PACE_ADAPTIVE) && (e = hipMalloc((void **)&st->adapt, states * 8)) != hipSuccess)
            return cleanup(0, "hipMalloc(adaptive period)", e);
        st->bytes_step += st->adapt ? states * 8 : 0;
    }
    if ((e = hipMemcpyAsync(st->d_map, st->map.data(), sizeof(int32_t) * st->map.size(),
                            hipMemcpyHostToDevice, s)) != hipSuccess)
        return cleanup(0, "copy head map", e);

    if (init_kind == PACE_INIT_ZERO) {
        if (st->bytes4 && (e = hipMemsetAsync(st->codes4, 0, st->bytes4, s)) != hipSuccess)
            return cleanup(0, "zero codes4", e);
        if (st->bytes8 && (e = hipMemsetAsync(st->codes8, 0, st->bytes8, s)) != hipSuccess)
            return cleanup(0, "zero codes8", e);
        if ((e = hipMemsetAsync(st->scales, 0, st->bytes_scales, s)) != hipSuccess)
            return cleanup(0, "zero scales", e);
    } else if (init_kind == PACE_INIT_F32) {
        if ((e = pace::launch_encode_f32(st->view(), (const float *)init, s)) != hipSuccess)
            return cleanup(0, "encode kernel", e);
    } else {
        const uint8_t *src = (const uint8_t *)init;
        if (st->bytes4 && (e = hipMemcpyAsync(st->codes4, src, st->bytes4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
            return cleanup(0, "raw copy codes4", e);
        src += st->bytes4;
        if (st->bytes8 && (e = hipMemcpyAsync(st->codes8, src, st->bytes8, hipMemcpyDeviceToDevice, s)) != hipSuccess)
            return cleanup(0, "raw copy codes8", e);
        src += st->bytes8;
        if ((e = hipMemcpyAsync(st->scales, src, st->bytes_scales, hipMemcpyDeviceToDevice, s)) != hipSuccess)
            return cleanup(0, "raw copy scales", e);
    }
    if (cfg->flags & PACE_FP8_WINDOW) {
        const size_t states = (size_t)cfg->batch * cfg->heads, S = (size_t)cfg->fp8_window;
        const size_t b_codes = states * S * (cfg->d_k + cfg->d_v), b_f = states * S * 12;
        st->bytes_step = b_codes + b_f + states * 12;
        if ((e = hipMalloc((void **)&st->win_codes, b_codes)) != hipSuccess)
            return cleanup(0, "hipMalloc(fp8 window)", e);
        if ((e = hipMalloc((void **)&st->win_f, b_f)) != hipSuccess)
            return cleanup(0, "hipMalloc(fp8 window scales)", e);
        if ((e = hipMalloc((void **)&st->win_meta, states * 8)) != hipSuccess)
            return cleanup(0, "hipMalloc(fp8 window counts)", e);
        if ((e = hipMalloc((void **)&st->win_lam, states * 4)) != hipSuccess)
            return cleanup(0, "hipMalloc(fp8 window decay)", e);
        if ((e = hipMemsetAsync(st->win_meta, 0, states * 8, s)) != hipSuccess)
            return cleanup(0, "zero fp8 window counts", e);
        std::vector<float> ones(states, 1.f);
        if ((e = hipMemcpyAsync(st->win_lam, ones.data(), states * 4, hipMemcpyHostToDevice, s)) != hipSuccess ||
            (e = hipStreamSynchronize(s)) != hipSuccess)
            return cleanup(0, "init fp8 window decay", e);
    }
    if (st->adapt && (e = pace::launch_adapt_init(st->view(), st->adapt, s)) != hipSuccess)
        return cleanup(0, "adaptive period init", e);
    // the host copy of the head map must outlive the async copy: wait for it
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return cleanup(0, "initialisation", e);
    *out = st;
    return ok();
}

PACE_API int pace_state_free(pace_state *st) {
    if (!st) return ok();
    hipError_t e = hipDeviceSynchronize();
    if (st->codes4) (void)hipFree(st->codes4);
    if (st->codes8) (void)hipFree(st->codes8);
    if (st->scales) (void)hipFree(st->scales);
    if (st->d_map) (void)hipFree(st->d_map);
    if (st->d_counter) (void)hipFree(st->d_counter);
    if (st->colerr) (void)hipFree(st->colerr);
    if (st->d_err) (void)hipFree(st->d_err);
    if (st->step_kv) (void)hipFree(st->step_kv);
    if (st->step_ab) (void)hipFree(st->step_ab);
    if (st->step_fill) (void)hipFree(st->step_fill);
    if (st->adapt) (void)hipFree(st->adapt);
    if (st->win_codes) (void)hipFree(st->win_codes);
    if (st->win_f) (void)hipFree(st->win_f);
    if (st->win_meta) (void)hipFree(st->win_meta);
    if (st->win_lam) (void)hipFree(st->win_lam);
    delete st;
    if (e != hipSuccess) return hip_fail(e, "pace_state_free");
    return ok();
}

PACE_API int pace_state_config(const pace_state *st, pace_config *out) {
    if (!st || !out) return fail(PACE_EINVAL, "null argument");
    *out = st->cfg;
    return ok();
}

PACE_API int pace_raw_bytes(const pace_state *st, uint64_t *out) {
    if (!st || !out) return fail(PACE_EINVAL, "null argument");
    *out = st->bytes4 + st->bytes8 + st->bytes_scales;
    return ok();
}

PACE_API int pace_decode_period(pace_state *st, int32_t n_tok, const void *q, const void *k,
                                const void *v, const float *alpha, const float *beta,
                                float *out, void *stream) {
    if (!st) return fail(PACE_EINVAL, "null state handle");
    if (st->stepped() || st->windowed())
        return fail(PACE_EINVAL, "a per-step handle decodes with pace_decode_step");
    if (n_tok < 1 || n_tok > st->cfg.period)
        return fail(PACE_EINVAL, "n_tok = %d outside 1..period (%d)", n_tok, st->cfg.period);
    int rc = check_tokens(n_tok, st->cfg.in_dtype, q, k, v, alpha, beta);
    if (rc) return rc;
    if (!out || !aligned(out, 16)) return fail(PACE_EINVAL, "out must be a 16-byte aligned device pointer");
    hipStream_t s = (hipStream_t)stream;
    const int bf16 = st->cfg.in_dtype == PACE_DTYPE_BF16;
    hipError_t e;
    if (pace::mfma_supported(st->cfg.d_k, st->cfg.d_v, n_tok, bf16,
                             (long long)st->cfg.batch * st->cfg.heads))
        e = pace::launch_decode_mfma(st->view(), st->d_map + st->cfg.heads,
                                     st->d_map + st->cfg.heads + st->n8, n_tok, q, k, v, alpha,
                                     beta, out, s);
    else
        e = pace::launch_decode_v0(st->view(), n_tok, q, k, v, alpha, beta, out, bf16, s);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    st->periods += 1;
    st->tokens += (uint64_t)n_tok;
    return ok();
}

PACE_API int pace_prefill_encode(pace_state *st, int32_t n_tok, const void *q, const void *k,
                                 const void *v, const float *alpha, const float *beta,
                                 float *out, void *stream) {
    if (!st) return fail(PACE_EINVAL, "null state handle");
    if (st->stepped() || st->windowed())
        return fail(PACE_EINVAL, "a per-step handle decodes with pace_decode_step");
    if (n_tok < 1) return fail(PACE_EINVAL, "n_tok must be >= 1");
    int rc = check_tokens(n_tok, st->cfg.in_dtype, q, k, v, alpha, beta);
    if (rc) return rc;
    if (out && !aligned(out, 16)) return fail(PACE_EINVAL, "out must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const int bf16 = st->cfg.in_dtype == PACE_DTYPE_BF16;
    hipError_t e;
    if (pace::prefill_mfma_supported(st->cfg.d_k, st->cfg.d_v, bf16,
                                     (long long)st->cfg.batch * st->cfg.heads))
        e = pace::launch_prefill_mfma(st->view(), n_tok, q, k, v, alpha, beta, out, s);
    else
        e = pace::launch_decode_v0(st->view(), n_tok, q, k, v, alpha, beta, out, bf16, s);
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    st->periods += 1;
    st->tokens += (uint64_t)n_tok;
    return ok();
}

PACE_API int pace_decode_step(pace_state *st, const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta, const uint8_t *active,
                              float *out, void *stream) {
    if (!st) return fail(PACE_EINVAL, "null state handle");
    if (!st->stepped() && !st->windowed())
        return fail(PACE_EINVAL, "the handle was not allocated with PACE_STEP_BUFFER or PACE_FP8_WINDOW");
    int rc = check_tokens(1, st->cfg.in_dtype, q, k, v, alpha, beta);
    if (rc) return rc;
    if (!out || !aligned(out, 16)) return fail(PACE_EINVAL, "out must be a 16-byte aligned device pointer");
    hipStream_t s = (hipStream_t)stream;
    const int bf16 = st->cfg.in_dtype == PACE_DTYPE_BF16;
    if (st->windowed()) {
        hipError_t e;
        if (pace::window_mfma_supported(st->cfg.d_k, st->cfg.d_v, bf16, st->cfg.fp8_window))
            e = pace::launch_window_step_mfma(st->view(), st->window_view(active), q, k, v, alpha,
                                              beta, out, s);
        else
            e = pace::launch_window_step(st->view(), st->window_view(active), q, k, v, alpha,
                                         beta, out, bf16, s);
        if (e != hipSuccess) return hip_fail(e, "window step launch");
        st->tokens += 1;
        return ok();
    }
    const pace::StepView sv = st->step_view(active);
    hipError_t e;
    if (pace::mfma_step_supported(st->cfg.d_k, st->cfg.d_v, st->cfg.period, bf16,
                                  (long long)st->cfg.batch * st->cfg.heads))
        e = pace::launch_step_mfma(st->view(), sv, st->d_map + st->cfg.heads,
                                   st->d_map + st->cfg.heads + st->n8, q, k, v, alpha, beta, out, s);
    else
        e = pace::launch_step_v0(st->view(), sv, q, k, v, alpha, beta, out, bf16, s);
    if (e != hipSuccess) return hip_fail(e, "step launch");
    st->tokens += 1;
    return ok();
}

PACE_API int pace_flush_steps(pace_state *st, void *stream) {
    if (!st) return fail(PACE_EINVAL, "null state handle");
    if (st->windowed()) {
        hipError_t e = pace::launch_window_flush(st->view(), st->window_view(nullptr), (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "window flush launch");
        return ok();
    }
    if (!st->stepped()) return fail(PACE_EINVAL, "the handle was not allocated with PACE_STEP_BUFFER");
    hipError_t e = pace::launch_flush_v0(st->view(), st->step_view(nullptr),
                                         st->cfg.in_dtype == PACE_DTYPE_BF16, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "flush launch");
    return ok();
}

PACE_API int pace_read_state(const pace_state *st, int what, void *dst, float *scales_dst,
                             void *stream) {
    if (!st) return fail(PACE_EINVAL, "null state handle");
    if (!dst) return fail(PACE_EINVAL, "dst must not be NULL");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (what == PACE_READ_CODES) {
        if (!scales_dst) return fail(PACE_EINVAL, "PACE_READ_CODES needs scales_dst");
        e = pace::launch_read(st->view(), 0, dst, scales_dst, s);
    } else if (what == PACE_READ_DEQUANT) {
        e = pace::launch_read(st->view(), 1, dst, scales_dst, s);
    } else if (what == PACE_READ_RAW) {
        if (scales_dst) return fail(PACE_EINVAL, "PACE_READ_RAW takes scales_dst = NULL");
        uint8_t *d = (uint8_t *)dst;
        e = hipSuccess;
        if (st->bytes4) e = hipMemcpyAsync(d, st->codes4, st->bytes4, hipMemcpyDeviceToDevice, s);
        d += st->bytes4;
        if (e == hipSuccess && st->bytes8)
            e = hipMemcpyAsync(d, st->codes8, st->bytes8, hipMemcpyDeviceToDevice, s);
        d += st->bytes8;
        if (e == hipSuccess)
            e = hipMemcpyAsync(d, st->scales, st->bytes_scales, hipMemcpyDeviceToDevice, s);
    } else if (what == PACE_READ_STEP && st->windowed()) {
        const size_t states = (size_t)st->cfg.batch * st->cfg.heads;
        e = hipMemcpyAsync(dst, st->win_meta, states * 4, hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess && scales_dst)
            e = pace::launch_window_meta(st->window_view(nullptr), scales_dst, states, s);
    } else if (what == PACE_READ_WINDOW) {
        if (!st->windowed()) return fail(PACE_EINVAL, "PACE_READ_WINDOW needs a PACE_FP8_WINDOW handle");
        const size_t states = (size_t)st->cfg.batch * st->cfg.heads, S = (size_t)st->cfg.fp8_window;
        e = hipMemcpyAsync(dst, st->win_codes, states * S * (st->cfg.d_k + st->cfg.d_v),
                           hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess && scales_dst)
            e = hipMemcpyAsync(scales_dst, st->win_f, states * S * 12, hipMemcpyDeviceToDevice, s);
    } else if (what == PACE_READ_STEP) {
        if (!st->stepped()) return fail(PACE_EINVAL, "PACE_READ_STEP needs a per-step handle");
        const size_t states = (size_t)st->cfg.batch * st->cfg.heads;
        e = hipMemcpyAsync(dst, st->step_fill, states * 4, hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess && scales_dst)
            e = st->adapt ? hipMemcpyAsync(scales_dst, st->adapt, states * 8, hipMemcpyDeviceToDevice, s)
                          : hipMemsetAsync(scales_dst, 0, states * 8, s);
    } else {
        return fail(PACE_EINVAL, "unknown read kind %d", what);
    }
    if (e != hipSuccess) return hip_fail(e, "read_state");
    return ok();
}

namespace {

// Storage accounting plus the device reductions of pace_quant_stats, with the
// zero-column counter and the per-head error sums in `counter` / `sums`
// (device memory, sums holding 2 doubles per head).  Host memory is a fixed
// array: nothing is allocated here.
int quant_stats(const pace_state *st, pace_stats *out, hipStream_t s, unsigned long long *counter,
                double *sums, const char *what) {
    const pace_config &c = st->cfg;
    pace_stats r = {};
    r.bytes_codes4 = st->bytes4;
    r.bytes_codes8 = st->bytes8;
    r.bytes_scales = st->bytes_scales;
    r.bytes_total = st->bytes4 + st->bytes8 + st->bytes_scales;
    r.bytes_fp16_equiv = (uint64_t)c.batch * c.heads * c.d_k * c.d_v * 2;
    r.bytes_int8_equiv = (uint64_t)c.batch * c.heads * c.d_k * c.d_v + st->bytes_scales;
    r.heads4 = st->n4;
    r.heads8 = st->n8;
    r.periods = st->periods;
    r.tokens = st->tokens;
    unsigned long long zeros = 0;
    double err[2 * PACE_STATS_MAX_HEADS];
    hipError_t e = hipMemsetAsync(counter, 0, sizeof zeros, s);
    if (e == hipSuccess) e = pace::launch_count_zero_scales(st->view(), counter, s);
    if (e == hipSuccess) e = hipMemcpyAsync(&zeros, counter, sizeof zeros, hipMemcpyDeviceToHost, s);
    if (st->colerr) {
        if (e == hipSuccess) e = pace::launch_reduce_colerr(st->view(), sums, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(err, sums, sizeof(double) * 2 * c.heads, hipMemcpyDeviceToHost, s);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, what);
    r.zero_columns = zeros;
    r.bytes_step_buffer = st->bytes_step;
    if (st->colerr) {
        r.err_tracked = 1;
        for (int h = 0; h < c.heads; ++h) {
            r.err_sq[h] = err[2 * h];
            r.ref_sq[h] = err[2 * h + 1];
        }
    }
    *out = r;
    return ok();
}

}  // namespace

PACE_API int pace_quant_stats(const pace_state *st, pace_stats *out, void *stream) {
    if (!st || !out) return fail(PACE_EINVAL, "null argument");
    return quant_stats(st, out, (hipStream_t)stream, st->d_counter, st->d_err, "quant_stats");
}

PACE_API int pace_quant_stats_static(const pace_state *st, pace_stats *out, void *stream) {
    if (!st || !out) return fail(PACE_EINVAL, "null argument");
    static_assert(pace::STATS_SCRATCH_HEADS == PACE_STATS_MAX_HEADS, "scratch holds every tracked head");
    if (st->colerr && st->cfg.heads > pace::STATS_SCRATCH_HEADS)
        return fail(PACE_EINVAL, "pace_quant_stats_static sums errors of at most %d heads (handle has %d)",
                    pace::STATS_SCRATCH_HEADS, st->cfg.heads);
    unsigned long long *scratch = nullptr;
    hipError_t e = pace::stats_scratch(st->device, &scratch);
    if (e != hipSuccess) return hip_fail(e, "quant_stats_static scratch");
    return quant_stats(st, out, (hipStream_t)stream, scratch, (double *)(scratch + 1),
                       "quant_stats_static");
}

PACE_API int pace_stream_copy(void *dst, const void *src, uint64_t bytes, void *stream) {
    if (!dst || !src) return fail(PACE_EINVAL, "null pointer");
    if (!aligned(dst, 16) || !aligned(src, 16)) return fail(PACE_EINVAL, "dst and src must be 16-byte aligned");
    if (bytes % 16) return fail(PACE_EINVAL, "bytes must be a multiple of 16");
    hipError_t e = pace::launch_stream_copy(dst, src, (size_t)bytes, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "stream copy launch");
    return ok();
}

PACE_API int pace_prefill_f32(int32_t batch, int32_t heads, int32_t d_k, int32_t d_v,
                              int32_t n_tok, int32_t in_dtype, const void *q, const void *k,
                              const void *v, const float *alpha, const float *beta,
                              float *state, float *out, void *stream) {
    int rc = check_shape(batch, heads, d_k, d_v);
    if (rc) return rc;
    if ((rc = check_dtype(in_dtype))) return rc;
    if (n_tok < 1) return fail(PACE_EINVAL, "n_tok must be >= 1");
    if ((rc = check_tokens(n_tok, in_dtype, q, k, v, alpha, beta))) return rc;
    if (!state || !aligned(state, 16)) return fail(PACE_EINVAL, "state must be a 16-byte aligned device pointer");
    if (out && !aligned(out, 16)) return fail(PACE_EINVAL, "out must be 16-byte aligned");
    hipError_t e = pace::launch_prefill_v0(batch, heads, d_k, d_v, n_tok,
                                           in_dtype == PACE_DTYPE_BF16, q, k, v, alpha, beta,
                                           state, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return ok();
}
