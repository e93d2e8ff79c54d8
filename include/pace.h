/*
 * pace.h - C ABI of a periodic-rounding gated delta-rule (GDN) decode library
 * whose recurrent state is stored as 4-bit (or 8-bit) codes with one float32
 * scale per state column.  Built for AMD MI355X (gfx950) with HIP.
 *
 * What the library computes (sources are the pages this implementation follows):
 *
 *  - One recurrent state per (sequence, head), so a server can decode many
 *    sequences at once with one state copy each ('PACE: four-bit recurrent
 *    state by rounding less often', TL;DR; 'PACE: A New 4-Bit Recurrent State
 *    Quantization Method That Makes Linear Attention Models More
 *    Memory-Efficient', section 'Why Do We Need Low-Precision Recurrent
 *    States?').  The state of one (sequence, head) is M in R^{d_k x d_v}:
 *    row i is key channel i, column j is value channel j.
 *
 *  - The gated delta rule, for each token t (the gate sets the forgetting
 *    rate, the delta rule makes each write an online-learning step:
 *    '低比特量化新突破：GGA+PW让线性注意力长文本生成更准更短', section
 *    '为什么低比特状态量化会“越写越错”'):
 *        M_t = alpha_t (M_{t-1} - beta_t k_t (k_t^T M_{t-1})) + beta_t k_t v_t^T
 *        o_t = M_t^T q_t
 *    q and k must already be L2-normalised by the caller; q is not scaled.
 *
 *  - Periodic rounding: the stored state is decoded, one period of tokens is
 *    applied in float32, and the state is re-encoded once at the end of the
 *    period (PACE wiki page, TL;DR point (1) and flowchart; 'PACE: A New
 *    4-Bit ...', section 'Periodic Rounding').  Outputs are read from the
 *    high-precision state, before the period-end encode.
 *    "In float32" means: the state, every accumulation and the outputs are
 *    float32.  The fused kernels (bf16 inputs, d_k = d_v = 64 or 128) run
 *    the period's matrix products on bf16 matrix cores, exactly where the
 *    operands are exact in bf16 (codes times tokens; the period's key and
 *    query Gram products) and with the update's right factor split into two
 *    bf16 parts (relative error below 2^-17); the prefill hand-off also
 *    splits the decoded state and its in-chunk output product into two bf16
 *    parts (about 1e-5 relative).
 *
 *  - Channel-aligned encoding: one scale per column, s_j = absmax_i |M_ij| / qmax
 *    in float32 (qmax = 7 for 4 bits, 127 for 8 bits), codes
 *    c_ij = round_to_nearest_even(M_ij / s_j); a zero column has s_j = 0 and
 *    zero codes ('PACE: A New 4-Bit ...', section 'Channel-Aligned Encoding';
 *    PACE wiki page, TL;DR point (2)).  The per-column kernels divide
 *    (correctly rounded); the fused kernels compute s_j = absmax *
 *    float32(1 / qmax), within one ulp of the quotient, and take M_ij / s_j
 *    through the hardware reciprocal (about one ulp), so a code can differ
 *    from exact rounding only where M_ij / s_j sits within about 1e-6 of a
 *    half-integer.
 *
 *  - Mixed heads: each head has a bit width (4 or 8), the same for every
 *    sequence; 8-bit heads are meant for heads whose rounding error persists
 *    longest (PACE wiki page, TL;DR point (3); flowchart node '8-bit heads').
 *    4-bit and 8-bit heads live in separate device pools.
 *
 * Conventions for every entry point:
 *  - Return value: PACE_OK (0) or a negative PACE_E* status.  On error,
 *    pace_last_error() returns a message for the calling thread.  No
 *    exception crosses the ABI and nothing aborts the process.
 *  - All argument checks happen before any HIP call, so a call that returns
 *    PACE_EINVAL or PACE_EUNSUPPORTED has touched no device state.
 *  - "device" pointers point to memory of the device that was current when the
 *    state was allocated; "host" pointers to ordinary host memory.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it and the call returns without waiting, except where stated.  A state
 *    handle must not be used from two streams at once.
 *  - Tensor layouts are dense and row-major in the order written; "[T, B, H, d]"
 *    means token-major, then sequence, then head, then channel.
 */
#ifndef PACE_H_
#define PACE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PACE_ABI_VERSION 3

/* status codes */
#define PACE_OK 0
#define PACE_EINVAL (-1)       /* a bad argument: null pointer, size, enum, alignment */
#define PACE_ENOMEM (-2)       /* device allocation failed */
#define PACE_EUNSUPPORTED (-3) /* a shape or period the library has no kernel for */
#define PACE_EDEVICE (-4)      /* a HIP error (no device, launch failure, earlier fault) */

/* element types of q, k, v */
#define PACE_DTYPE_F32 0
#define PACE_DTYPE_BF16 1

/* pace_state_alloc init kinds */
#define PACE_INIT_ZERO 0 /* all scales and codes zero; init must be NULL */
#define PACE_INIT_F32 1  /* init: device float32 [B, H, d_k, d_v]; encoded once */
#define PACE_INIT_RAW 2  /* init: device raw image written by pace_read_state(PACE_READ_RAW) */

/* pace_read_state kinds */
#define PACE_READ_CODES 0   /* dst: device int8 [B, H, d_k, d_v]; scales_dst: device float32 [B, H, d_v] */
#define PACE_READ_DEQUANT 1 /* dst: device float32 [B, H, d_k, d_v] = c_ij * s_j; scales_dst may be NULL */
#define PACE_READ_RAW 2     /* dst: device bytes [pace_raw_bytes()]; scales_dst must be NULL */
#define PACE_READ_STEP 3    /* PACE_STEP_BUFFER handles: dst: device int32 [B, H] buffered tokens
                               per state; scales_dst: device float32 [B, H, 2] = (A, R) of
                               PACE_ADAPTIVE (zeros without it), or NULL.  PACE_FP8_WINDOW
                               handles: dst: writes in the window; scales_dst: (lam, head) with
                               lam the history's decay since its last encode and head the slot
                               of the oldest write (as a float) */
#define PACE_READ_WINDOW 4  /* PACE_FP8_WINDOW handles: dst: device uint8 [B, H, S, d_k + d_v], the
                               E4M3 codes of k_t then u_t per slot (slots in ring order, see
                               PACE_READ_STEP); scales_dst: device float32 [B, H, S, 3] = (k scale,
                               u scale, decay since the write), or NULL */

/* config flags */
/* PACE_STATS_ERR: every encode (the PACE_INIT_F32 encode at alloc and the
 * period-end encode of each pace_decode_period call) also records, per column,
 * the squared round-trip error sum_i (M_ij - c_ij s_j)^2 and sum_i M_ij^2 of the
 * high-precision state M it encodes; pace_quant_stats sums them per head.
 * Costs B * H * d_v * 8 bytes of device memory and that much extra writing per
 * encode.  Requires heads <= PACE_STATS_MAX_HEADS. */
#define PACE_STATS_ERR 0x1u
#define PACE_STATS_MAX_HEADS 256
/* PACE_STEP_BUFFER: the handle decodes one token per call (pace_decode_step)
 * instead of one period per call.  Every (sequence, head) state gets a buffer
 * of up to period - 1 tokens (its k_t, v_t in in_dtype and alpha_t, beta_t in
 * float32) and a fill count; the token that completes a period applies the
 * buffer and itself to the decoded state and re-encodes it, every other token
 * is appended to the buffer.  This is the serving form of periodic rounding
 * ('PACE: four-bit recurrent state by rounding less often', flowchart 'Fewer
 * roundings, less compounded error'): decoded tokens are held back and
 * applied together once per period, followed by one encode.
 * Buffer bytes: B * H * (period - 1) * ((d_k + d_v) * elem + 8), plus
 * B * H * 4 for the fill counts (pace_stats.bytes_step_buffer).  Such a
 * handle rejects pace_decode_period. */
#define PACE_STEP_BUFFER 0x2u
/* PACE_ADAPTIVE (with PACE_STEP_BUFFER): the period becomes adaptive ('PACE:
 * four-bit recurrent state by rounding less often', section 'Research angle':
 * the size of the updates since the last encode, not a token count, decides
 * when to re-encode).  Each state
 * keeps A, the sum over its buffered tokens of the norm of their write into
 * the state, ||k_t|| * ||u_t|| with u_t = beta_t (v_t - alpha_t M_{t-1}^T k_t),
 * and R, the Frobenius norm of its stored state as of its last encode.  A
 * step closes the period (applies the buffer and its own token, re-encodes)
 * when its buffer is full (cfg.period is then the maximum period) or when
 * A > adapt_tau * R already holds before the step.  Costs B * H * 8 bytes. */
#define PACE_ADAPTIVE 0x4u
/* PACE_FP8_WINDOW: the handle decodes one token per call (pace_decode_step)
 * with a pure-write window instead of a period ('低比特量化新突破：GGA+PW让线性
 * 注意力长文本生成更准更短', section 'PW：让近期写入走“纯净通道”').  Each write of
 * the delta rule, M_t = alpha_t M_{t-1} + k_t u_t^T with
 * u_t = beta_t (v_t - alpha_t M_{t-1}^T k_t), is kept as a pair of OCP E4M3
 * vectors (one float32 scale each, absmax / 448, nearest-even codes); the
 * last cfg.fp8_window writes stay out of the column-quantized history and
 * decay with it; a write leaving the window is added to the history, which is
 * re-encoded.  Outputs are read from the state after the step's exact write.
 * Excludes PACE_STEP_BUFFER and PACE_ADAPTIVE; cfg.period is ignored.
 * Window bytes: B * H * (S * (d_k + d_v + 12) + 12). */
#define PACE_FP8_WINDOW 0x8u

typedef struct pace_state pace_state; /* opaque; owns the device pools */

typedef struct pace_config {
    int32_t batch;            /* B: sequences decoding concurrently, >= 1 */
    int32_t heads;            /* H: heads of the layer, >= 1 */
    int32_t d_k;              /* state rows (key channels): 64 or 128 */
    int32_t d_v;              /* state columns (value channels): a multiple of 16, 16..256 */
    int32_t period;           /* k: most tokens one pace_decode_period call may apply, 1..64 */
    int32_t in_dtype;         /* PACE_DTYPE_F32 or PACE_DTYPE_BF16: element type of q, k, v */
    const uint8_t *head_bits; /* host [H]: bit width of each head, 4 or 8; copied at alloc */
    uint32_t flags;           /* 0 or an OR of PACE_STATS_ERR, PACE_STEP_BUFFER, PACE_ADAPTIVE */
    float adapt_tau;          /* PACE_ADAPTIVE: threshold tau, finite and > 0; otherwise ignored */
    int32_t fp8_window;       /* PACE_FP8_WINDOW: writes kept in the window, 1..64; otherwise ignored */
} pace_config;

typedef struct pace_stats {
    uint64_t bytes_codes4;     /* device bytes of the 4-bit code pool */
    uint64_t bytes_codes8;     /* device bytes of the 8-bit code pool */
    uint64_t bytes_scales;     /* device bytes of the float32 column scales */
    uint64_t bytes_total;      /* sum of the three above */
    uint64_t bytes_fp16_equiv; /* the same states stored densely as fp16 */
    uint64_t bytes_int8_equiv; /* the same states with every head at 8 bits (plus scales) */
    int32_t heads4;            /* heads in the 4-bit pool */
    int32_t heads8;            /* heads in the 8-bit pool */
    uint64_t periods;          /* pace_decode_period calls applied since alloc */
    uint64_t tokens;           /* tokens applied since alloc: n_tok per pace_decode_period,
                                  1 per pace_decode_step (whatever its active mask) */
    uint64_t zero_columns;     /* stored columns whose scale is 0 */
    uint64_t bytes_step_buffer; /* device bytes of the per-step token buffer and fill counts,
                                  or of the FP8 window (0 for period handles) */
    /* with PACE_STATS_ERR (err_tracked = 1), per head h < heads, over every
     * sequence b and entry (i, j) of the state M of the last encode:
     * err_sq[h] = sum (M_ij - c_ij s_j)^2 and ref_sq[h] = sum M_ij^2, so that
     * err_sq / ref_sq is that head's relative squared round-trip error (the
     * column quantizer's fidelity: 'PACE: A New 4-Bit Recurrent State
     * Quantization Method ...', section 'Channel-Aligned Encoding').  Zero
     * after PACE_INIT_ZERO or PACE_INIT_RAW until the first decode call.
     * Without the flag: err_tracked = 0 and both arrays are zero. */
    int32_t err_tracked;
    double err_sq[PACE_STATS_MAX_HEADS];
    double ref_sq[PACE_STATS_MAX_HEADS];
} pace_stats;

/* ABI version this library was built with (PACE_ABI_VERSION). */
int pace_abi_version(void);

/* Message for the last non-zero status returned on the calling thread ("" if none).
 * The pointer stays valid until the next pace_* call on that thread. */
const char *pace_last_error(void);

/*
 * Allocate the device pools of B x H states and initialise them.
 *   cfg:       host; validated and copied (head_bits included).
 *   init_kind: PACE_INIT_ZERO | PACE_INIT_F32 | PACE_INIT_RAW (see above).
 *   init:      device pointer per init_kind; must stay valid until the
 *              stream has run the initialisation.
 *   stream:    hipStream_t for the initialisation work.
 *   out:       host; receives the new handle (unchanged on error).
 * The only call that allocates device memory (hipMalloc, so it may block).
 * PACE_INIT_F32 encodes each (sequence, head) state with the column quantizer.
 * Errors: EINVAL, EUNSUPPORTED (d_k, d_v or period outside what is built),
 *         ENOMEM, EDEVICE.
 */
int pace_state_alloc(const pace_config *cfg, int init_kind, const void *init,
                     void *stream, pace_state **out);

/* Free the pools and the handle; waits for the device first.  NULL is a no-op. */
int pace_state_free(pace_state *st);

/* Configuration the handle was allocated with (head_bits points into the handle). */
int pace_state_config(const pace_state *st, pace_config *out);

/* Size in bytes of the raw image written by pace_read_state(PACE_READ_RAW). */
int pace_raw_bytes(const pace_state *st, uint64_t *out);

/*
 * Apply one period of n_tok tokens (1 <= n_tok <= cfg.period) to every
 * (sequence, head) state: decode the stored codes, apply the tokens in order
 * in float32 with the gated delta rule, write o_t for each token, and
 * re-encode the state with per-column scales at the end of the call.
 *   q, k:  device [n_tok, B, H, d_k], in_dtype, 16-byte aligned.
 *   v:     device [n_tok, B, H, d_v], in_dtype, 16-byte aligned.
 *   alpha, beta: device float32 [n_tok, B, H], 4-byte aligned; alpha is the
 *          gate (0 < alpha <= 1 expected), beta the write strength.
 *   out:   device float32 [n_tok, B, H, d_v], 16-byte aligned; may not alias inputs.
 * Kernels: bf16 inputs with d_k = d_v = 64 or 128 and n_tok <= 16 run the
 * fused matrix-core kernels, for any batch the pools can hold (offsets
 * between tokens are 64-bit); float32 inputs, d_v != d_k and calls of more
 * than 16 tokens run a per-column kernel, correct but about 50x slower.
 * Errors: EINVAL (null handle or pointer, n_tok out of range, misalignment,
 *         a handle allocated with PACE_STEP_BUFFER),
 *         EDEVICE (launch failure or an earlier asynchronous fault).
 */
int pace_decode_period(pace_state *st, int32_t n_tok, const void *q, const void *k,
                       const void *v, const float *alpha, const float *beta, float *out,
                       void *stream);

/*
 * One decode step of a PACE_STEP_BUFFER or PACE_FP8_WINDOW handle: one token
 * for every active sequence (for the window see PACE_FP8_WINDOW; the rest of
 * this comment describes the buffer).  For each (sequence, head) state with f tokens buffered, the
 * output is read from the stored state decoded with the f buffered tokens and
 * then this token applied in order, in float32 (the high-precision state the
 * period holds after this token).  If f + 1 = period the state is re-encoded
 * and its buffer emptied; otherwise the token is appended to the buffer and
 * the stored codes are left unchanged (read, not written).  Outputs equal
 * those of pace_decode_period fed the same tokens a period at a time.
 *   q, k:   device [B, H, d_k], in_dtype, 16-byte aligned.
 *   v:      device [B, H, d_v], in_dtype, 16-byte aligned.
 *   alpha, beta: device float32 [B, H].
 *   active: device uint8 [B] (0 = this sequence takes no token this step:
 *           its state, buffer and output rows are left untouched), or NULL
 *           for all sequences.  Sequences can so sit at different phases.
 *   out:    device float32 [B, H, d_v], 16-byte aligned.
 * Errors: EINVAL (null or misaligned pointer, a handle without
 *         PACE_STEP_BUFFER or PACE_FP8_WINDOW), EDEVICE.
 */
int pace_decode_step(pace_state *st, const void *q, const void *k, const void *v,
                     const float *alpha, const float *beta, const uint8_t *active,
                     float *out, void *stream);

/*
 * End every partial period of a PACE_STEP_BUFFER handle: each state with a
 * non-empty buffer has its buffered tokens applied and is re-encoded (as a
 * shorter final period); its buffer is emptied.  For a PACE_FP8_WINDOW handle:
 * every write still in the window is added to the history (oldest first),
 * which is re-encoded once; the window is emptied.  Call before
 * pace_read_state or a raw checkpoint when the buffered tokens must be part
 * of the stored state.  No outputs.
 * Errors: EINVAL (a handle without PACE_STEP_BUFFER or PACE_FP8_WINDOW), EDEVICE.
 */
int pace_flush_steps(pace_state *st, void *stream);

/*
 * Read the stored state (see PACE_READ_*).  dst and scales_dst are device
 * pointers sized as documented above.  The raw image is the library's own
 * device layout (4-bit pool, then 8-bit pool, then scales) and is meant only
 * to be handed back to pace_state_alloc(PACE_INIT_RAW) for a handle of the
 * same configuration (checkpoint / resume).  For a PACE_STEP_BUFFER handle
 * this is the state as of each sequence's last encode (buffered tokens are
 * not included; see pace_flush_steps).
 * Errors: EINVAL, EDEVICE.
 */
int pace_read_state(const pace_state *st, int what, void *dst, float *scales_dst,
                    void *stream);

/*
 * Storage accounting and counters of a handle.  out is host memory.  Counts
 * zero columns (and, with PACE_STATS_ERR, sums the error statistics) on the
 * device, so it waits for `stream`.
 * Errors: EINVAL, EDEVICE.
 */
int pace_quant_stats(const pace_state *st, pace_stats *out, void *stream);

/*
 * For callers that cannot allocate device memory at the call (code that must
 * not call hipMalloc, tight serving loops, harnesses that forbid it): the
 * same result as pace_quant_stats, but its device scratch (the zero-column
 * counter and the per-head float64 error sums) lives in a fixed array the
 * library holds on each device until the process ends (8 + 2 * 256 * 8
 * bytes: error sums of at most PACE_STATS_MAX_HEADS heads) instead of the
 * handle's buffers.  Nothing is allocated: no hipMalloc, hipFree or
 * allocating library routine.  The first call on a device looks the array's
 * address up once.  Every call on one device shares that array: calls that
 * overlap on one device (other host threads, other streams) race and must
 * be ordered by the caller.  Waits for `stream`, like pace_quant_stats.
 * Errors: EINVAL (null argument; an error-tracking handle with more heads
 *         than the array holds), EDEVICE.
 */
int pace_quant_stats_static(const pace_state *st, pace_stats *out, void *stream);

/*
 * Prefill hand-off: apply a prompt of n_tok tokens (any n_tok >= 1) to every
 * stored state and encode once at the end, i.e. one period of n_tok tokens
 * (the stored state decoded -- zero after PACE_INIT_ZERO --, the tokens
 * applied in order in float32, per-column re-encode).  Chunked kernels keep
 * the state in high precision across a prompt chunk; this keeps it across
 * the whole prompt and rounds once ('PACE: four-bit recurrent state by
 * rounding less often', TL;DR point (1)).
 *   q, k:  device [n_tok, B, H, d_k]; v: device [n_tok, B, H, d_v]; in_dtype,
 *          16-byte aligned.  alpha, beta: device float32 [n_tok, B, H].
 *   out:   device float32 [n_tok, B, H, d_v] (16-byte aligned), or NULL.
 * bf16 inputs with d_k = d_v = 64 or 128 run the fused kernel (the state stays
 * on chip for the whole prompt) for any batch; other shapes run the
 * per-column kernel.
 * Errors: EINVAL (null or misaligned pointer, n_tok < 1, a PACE_STEP_BUFFER
 *         handle), EDEVICE.
 */
int pace_prefill_encode(pace_state *st, int32_t n_tok, const void *q, const void *k,
                        const void *v, const float *alpha, const float *beta, float *out,
                        void *stream);

/*
 * Unquantized float32 gated delta rule over n_tok tokens, in place on a dense
 * float32 state: used to build the state that decode starts from (warm-up
 * tokens, or a prompt streamed in blocks).  The chunked-prefill motivation of
 * periodic rounding is the PACE wiki page, TL;DR point (1).
 *   state: device float32 [B, H, d_k, d_v], read and written.
 *   q, k:  device [n_tok, B, H, d_k]; v: device [n_tok, B, H, d_v]; in_dtype.
 *   alpha, beta: device float32 [n_tok, B, H].
 *   out:   device float32 [n_tok, B, H, d_v], or NULL to skip outputs.
 * Errors: EINVAL, EUNSUPPORTED, EDEVICE.
 */
int pace_prefill_f32(int32_t batch, int32_t heads, int32_t d_k, int32_t d_v, int32_t n_tok,
                     int32_t in_dtype, const void *q, const void *k, const void *v,
                     const float *alpha, const float *beta, float *state, float *out,
                     void *stream);

/*
 * Measurement utility, not part of the method: copy `bytes` from src to dst
 * (both device, 16-byte aligned, not overlapping; bytes a multiple of 16)
 * with 16-byte non-temporal loads and stores, one per lane, as the decode
 * kernels stream their codes.  Its bandwidth is the attainable reference for
 * the decode kernels' fraction of the HBM peak, and a copy of known size
 * calibrates byte counters of a profiler.  bytes = 0 is a no-op.
 * Errors: EINVAL (null or misaligned pointer, bytes not a multiple of 16),
 *         EDEVICE.
 */
int pace_stream_copy(void *dst, const void *src, uint64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PACE_H_ */
