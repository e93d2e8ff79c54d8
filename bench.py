#!/usr/bin/env python3
"""Benchmark of PACE-style periodic-rounding GDN decode on one MI355X.

One step = one decode period over the whole batch: every (sequence, head)
state is decoded from its 4/8-bit codes, the period's k tokens are applied in
float32 with the gated delta rule (outputs written for every token), and the
state is re-encoded with per-column scales.  Default workload: 4096 sequences,
16 heads (12 at 4 bits, 4 at 8 bits), d_k = d_v = 128, period 8, bf16 q/k/v,
8 outlier value channels; 128 steps = 1024 decode steps.

Inputs are synthetic and seeded (linear_attn_decode_pace_amd.inputs); a ring
of distinct periods is resident in HBM before timing.  The initial state comes
from 32 unquantized warm-up tokens run by the library's prefill kernel.

Prints one JSON line: token-steps/s (sequences x tokens per second), the
decode kernel's achieved HBM bandwidth against MI355X's 8 TB/s with per-launch
minimum, median and maximum, the attainable bandwidth of a streaming
device-to-device copy timed after the decode region, and the float64 CPU
oracle timed over the whole batch on the host's cores (one process per core).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from linear_attn_decode_pace_amd import inputs  # noqa: E402

PEAK_HBM_GBS = 8000.0
PROMPT_HEAD = 64
# sources (with every header they include) of each timed kernel: the fused
# decode for 1..8 tokens per call, the 16-token chunk kernel for 9..16, the
# prefill and the FP8-window step.  A stored traffic figure counts only while
# the hash of its kernel's sources matches.
KERNEL_SOURCES = ["linear_attn_decode_pace_amd/csrc/decode_mfma.hip",
                  "linear_attn_decode_pace_amd/csrc/mfma_common.h",
                  "linear_attn_decode_pace_amd/csrc/pace_mfma.h",
                  "linear_attn_decode_pace_amd/csrc/pace_step.h",
                  "linear_attn_decode_pace_amd/csrc/pace_layout.h"]
PREFILL_SOURCES = ["linear_attn_decode_pace_amd/csrc/prefill_mfma.hip",
                   "linear_attn_decode_pace_amd/csrc/pace_prefill.h",
                   "linear_attn_decode_pace_amd/csrc/mfma_common.h",
                   "linear_attn_decode_pace_amd/csrc/pace_mfma.h",
                   "linear_attn_decode_pace_amd/csrc/pace_step.h",
                   "linear_attn_decode_pace_amd/csrc/pace_layout.h"]
KERNEL_SOURCES_16 = ["linear_attn_decode_pace_amd/csrc/decode_mfma16.hip",
                     "linear_attn_decode_pace_amd/csrc/chunk16.h",
                     "linear_attn_decode_pace_amd/csrc/mfma_common.h",
                     "linear_attn_decode_pace_amd/csrc/pace_mfma.h",
                     "linear_attn_decode_pace_amd/csrc/pace_step.h",
                     "linear_attn_decode_pace_amd/csrc/pace_layout.h"]
# the FP8-window step kernel
WINDOW_SOURCES = ["linear_attn_decode_pace_amd/csrc/window_mfma.hip",
                  "linear_attn_decode_pace_amd/csrc/e4m3.h",
                  "linear_attn_decode_pace_amd/csrc/pace_window.h",
                  "linear_attn_decode_pace_amd/csrc/mfma_common.h",
                  "linear_attn_decode_pace_amd/csrc/pace_mfma.h",
                  "linear_attn_decode_pace_amd/csrc/pace_step.h",
                  "linear_attn_decode_pace_amd/csrc/pace_layout.h"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(w: inputs.Workload, n_tok: int, head_bits) -> int:
    """Bytes one decode call must move at minimum: every stored code and scale
    read and written once, q/k/v/alpha/beta read once, outputs written once
    (float32)."""
    e_in = 2 if w.dtype == inputs.DT_BF16 else 4
    state = 0
    for b in head_bits:
        state += w.dk * w.dv * int(b) // 8 + 4 * w.dv
    per_seq_tok = w.H * ((w.dk * 2 + w.dv) * e_in + 8 + 4 * w.dv)
    return w.B * (2 * state + n_tok * per_seq_tok)


def algorithmic_bytes_step(w: inputs.Workload, head_bits, k_eff=None) -> float:
    """Mean bytes of one per-step decode call over a period of k = w.period
    calls: the stored state is read by every call and written by the last;
    call f reads the f buffered tokens (k_t, v_t, alpha_t, beta_t) and every
    call but the last appends its own; each call reads its q/k/v/alpha/beta and
    writes its float32 outputs.  An adaptive period passes its measured mean
    length as k_eff (the model then treats every period as that long)."""
    e_in = 2 if w.dtype == inputs.DT_BF16 else 4
    k = w.period if k_eff is None else k_eff
    state = sum(w.dk * w.dv * int(b) // 8 + 4 * w.dv for b in head_bits)
    buf_tok = w.H * ((w.dk + w.dv) * e_in + 8)
    io_tok = w.H * ((w.dk * 2 + w.dv) * e_in + 8 + 4 * w.dv)
    per_period = (k + 1) * state + (k * (k - 1) / 2 + (k - 1)) * buf_tok + k * io_tok
    return w.B * per_period / k


def step_bytes_exact(w: inputs.Workload, head_bits, fill_before, closed) -> float:
    """Bytes of one per-step decode call from the states' buffer fills before
    the call and whether the call closed their period: every state reads its
    codes and scales, its buffered tokens and the call's q/k/v/alpha/beta and
    writes its float32 outputs; a state that closes its period writes its
    codes and scales, the others append the token to the buffer.  fill_before
    and closed are [B, H] tensors."""
    import torch
    e_in = 2 if w.dtype == inputs.DT_BF16 else 4
    state_h = torch.tensor([w.dk * w.dv * int(b) // 8 + 4 * w.dv for b in head_bits],
                           dtype=torch.float64, device=fill_before.device)
    buf_tok = (w.dk + w.dv) * e_in + 8
    io_tok = (w.dk * 2 + w.dv) * e_in + 8 + 4 * w.dv
    closed = closed.to(torch.float64)
    total = (w.B * state_h.sum() + fill_before.to(torch.float64).sum() * buf_tok
             + w.B * w.H * io_tok + (closed * state_h[None, :]).sum()
             + (1.0 - closed).sum() * buf_tok)
    return float(total.item())


def kernel_sha(period: int = 8, prefill: bool = False, window: bool = False) -> str:
    h = hashlib.sha256()
    srcs = (PREFILL_SOURCES if prefill else WINDOW_SOURCES if window
            else KERNEL_SOURCES_16 if period > 8 else KERNEL_SOURCES)
    for p in srcs:
        fp = os.path.join(ROOT, p)
        if os.path.exists(fp):
            with open(fp, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def _gen_block(args):
    w, seed, seg, t0, t1 = args
    return inputs.tokens(w, seed, seg, t0, t1)


def generate(w, seed, jobs, workers):
    if workers <= 1 or len(jobs) == 1:
        return [_gen_block((w, seed) + j) for j in jobs]
    with cf.ProcessPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(_gen_block, [(w, seed) + j for j in jobs]))


def traffic_from_profile(name: str, sha: str, n_launch_bytes: int):
    """HBM bytes per launch from a committed counter profile, if it was taken
    on these kernel sources (profiles/traffic_<name>.json)."""
    fp = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(fp):
        return None
    with open(fp) as f:
        t = json.load(f)
    if t.get("kernel_sha") != sha:
        return None
    return t.get("bytes_per_launch")


# What the decode path computes in: 4/8-bit codes with float32 column scales,
# bf16 tokens, float32 state, accumulators and outputs; matrix products on bf16
# MFMA with exact operands (codes, tokens) or two bf16 parts (the update's W,
# relative error below 2^-17); scale = absmax * float32(1 / qmax), quotients
# through the hardware reciprocal.
ARITHMETIC_DTYPE = "f32+bf16"
ARITHMETIC = ("float32 state/accumulators/outputs; bf16 MFMA on exact code and token operands; "
              "update W in two bf16 parts (rel. err < 2^-17); 4/8-bit codes, float32 scales")


def copy_calibration(nbytes: int, reps: int = 10) -> dict:
    """Attainable device bandwidth, timed after the timed region (so it
    cannot warm anything up for it): the library's streaming copy (16-byte
    non-temporal loads and stores, the decode kernels' pattern) and torch's
    device-to-device copy of the same buffers, best of `reps` each; GB/s
    count read + write bytes."""
    import torch

    from linear_attn_decode_pace_amd import pace

    nbytes -= nbytes % 16
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)

    def best(fn):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return 2 * nbytes / (min(ts) * 1e-3) / 1e9

    stream_gbs = best(lambda: pace.pace_stream_copy(dst, src, nbytes))
    torch_gbs = best(lambda: dst.copy_(src))
    del src, dst
    return {"stream_copy_gbs": stream_gbs, "torch_copy_gbs": torch_gbs, "bytes": nbytes,
            "unit": "GB/s", "frac_of_peak": stream_gbs / PEAK_HBM_GBS,
            "note": "read + write bytes; best of %d; timed after the timed region" % reps}


def _cpu_model() -> str:
    try:
        return next((l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                     if l.startswith("model name")), platform.processor())
    except OSError:
        return platform.processor()


def _oracle_shard(args):
    """One worker of the CPU baseline: the float64 oracle over sequences
    [b0, b1), all heads.  Its warm-up state and initial encode are untimed;
    the timed periods start when every worker has reached the barrier."""
    (dk, dv, H, head_bits, warm, periods, barrier, results) = args
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import gdn
    from oracle import pace as opace
    from oracle import quant

    with threadpool_limits(limits=1):
        n = warm[0].shape[1]
        bits = np.tile(np.asarray(head_bits), n // H).astype(np.int64)
        M0 = gdn.from_zero(dk, dv, *warm)
        codes, scales = quant.encode(M0, bits)
        del M0
        barrier.wait()
        t0 = time.perf_counter()
        for a in periods:
            _, codes, scales, _ = opace.period(codes, scales, bits, *a)
        results.put(time.perf_counter() - t0)


def cpu_baseline(w, warm_tok, periods_tok, head_bits, workers):
    """Time the float64 oracle over the whole batch (all sequences and heads)
    for the given periods, the batch split across `workers` processes with
    one BLAS thread each (fresh interpreters: none inherits the parent's GPU
    context).  The value is batch x tokens over the slowest worker's time."""
    import multiprocessing as mp

    import numpy as np

    def f64(tok, name, b0, b1):
        a = getattr(tok, name)[:, b0:b1]
        if name in ("q", "k", "v") and tok.dtype == inputs.DT_BF16:
            a = inputs.bf16_to_f32(a)
        a = a.astype(np.float64)
        return a.reshape((a.shape[0], (b1 - b0) * w.H) + a.shape[3:])

    def arrays(tok, b0, b1):
        return [f64(tok, x, b0, b1) for x in ("q", "k", "v", "alpha", "beta")]

    ctx = mp.get_context("spawn")
    workers = max(1, min(workers, w.B))
    barrier, results = ctx.Barrier(workers, timeout=1800), ctx.Queue()
    cuts = np.linspace(0, w.B, workers + 1).astype(int)
    procs = []
    for i in range(workers):
        b0, b1 = int(cuts[i]), int(cuts[i + 1])
        args = (w.dk, w.dv, w.H, list(map(int, head_bits)), arrays(warm_tok, b0, b1),
                [arrays(t, b0, b1) for t in periods_tok], barrier, results)
        p = ctx.Process(target=_oracle_shard, args=(args,))
        p.start()
        procs.append(p)
    import queue as _queue
    times = []
    try:
        while len(times) < len(procs):
            try:
                times.append(results.get(timeout=2.0))
            except _queue.Empty:
                dead = [p.exitcode for p in procs if p.exitcode not in (None, 0)]
                if dead:
                    raise RuntimeError(f"CPU baseline worker exited with {dead[0]}")
    finally:
        for p in procs:
            if p.exitcode is None and len(times) < len(procs):
                p.terminate()
            p.join()
    dt = max(times)
    n_tok = sum(t.T for t in periods_tok)
    return {"value": w.B * n_tok / dt, "unit": "token-steps/s", "cores": workers, "kind": "oracle",
            "sample": f"all {w.B} sequences x {w.H} heads, {len(periods_tok)} period(s) of "
                      f"{periods_tok[0].T} tokens ({n_tok} decode steps), float64 numpy oracle, "
                      f"{workers} processes x 1 BLAS thread, {dt:.1f} s for the slowest shard "
                      f"({_cpu_model()}); warm-up and initial encode untimed",
            "seconds": dt}


def window_bytes(w: inputs.Workload, head_bits, S: int) -> int:
    """Bytes of one FP8-window step with a full window: the stored history read
    and written (a write leaves the window every step), the S pairs of E4M3
    vectors and their scales read, one pair written, the token read and the
    float32 outputs written."""
    e_in = 2 if w.dtype == inputs.DT_BF16 else 4
    state = sum(w.dk * w.dv * int(b) // 8 + 4 * w.dv for b in head_bits)
    win = w.H * (S * (w.dk + w.dv + 12) + (w.dk + w.dv + 12))
    io = w.H * ((w.dk * 2 + w.dv) * e_in + 8 + 4 * w.dv)
    return w.B * (2 * state + win + io)


def prefill_bytes(w: inputs.Workload, n_tok: int, head_bits) -> int:
    """Bytes of one prefill call at minimum: the prompt's q/k/v/alpha/beta read
    once, its float32 outputs written once, every code and scale read and
    written once."""
    e_in = 2 if w.dtype == inputs.DT_BF16 else 4
    state = sum(w.dk * w.dv * int(b) // 8 + 4 * w.dv for b in head_bits)
    per_tok = w.H * ((w.dk * 2 + w.dv) * e_in + 8 + 4 * w.dv)
    return w.B * (2 * state + n_tok * per_tok)


def device_prompt(tok, T: int):
    """The generated prompt tokens `tok` (D of them) repeated on the device to
    a prompt of T tokens [T, B, H, d]."""
    import torch

    from linear_attn_decode_pace_amd import runtime

    small = runtime.DeviceTokens(tok)
    D = small.T
    big = runtime.DeviceTokens.__new__(runtime.DeviceTokens)
    for name in ("q", "k", "v", "alpha", "beta"):
        x = getattr(small, name)
        y = torch.empty((T,) + tuple(x.shape[1:]), dtype=x.dtype, device="cuda")
        for t0 in range(0, T, D):
            y[t0:t0 + D].copy_(x[:min(D, T - t0)])
        setattr(big, name, y)
    big.T = T
    return big


def bench_prefill(args) -> int:
    """Time pace_prefill_encode over whole prompts (the hand-off workload)."""
    import torch

    from linear_attn_decode_pace_amd import pace, runtime

    if args.gpus != 1:
        print("bench.py runs on one GPU only", file=sys.stderr)
        return 2
    w = inputs.WORKLOADS[args.workload]
    T = w.prompt
    if not T:
        raise SystemExit(f"{w.name} has no prompt; use --workload prefill-b512")
    torch.cuda.set_device(0)
    head_bits = inputs.head_bits(w, args.seed)
    D = min(T, args.prompt_distinct)
    t = time.time()
    blocks = generate(w, args.seed, [(inputs.SEG_PROMPT, t0, min(D, t0 + 64)) for t0 in range(0, D, 64)],
                      args.workers)
    log(f"generated {D} distinct prompt tokens in {time.time() - t:.1f} s")
    # device prompt [T, B, H, d]: the D generated tokens repeated to length T
    big = device_prompt(inputs.concat(blocks), T)
    out = runtime.out_buffer(w, T)
    st = runtime.State(w, head_bits, pace.PACE_INIT_ZERO)
    torch.cuda.synchronize()
    log(f"prompt resident: {big.nbytes / 1e9:.1f} GB inputs, {out.numel() * 4 / 1e9:.1f} GB outputs")
    for _ in range(max(1, args.warmup)):
        st.prefill(big, out)
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record()
        st.prefill(big, out)
        ev[i][1].record()
    torch.cuda.synchronize()
    per_launch = [a.elapsed_time(b) for a, b in ev]
    ms = sum(per_launch) / K
    nbytes = prefill_bytes(w, T, head_bits)
    sha = kernel_sha(prefill=True)
    achieved = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "prefill prompt tokens/s into the quantized state (seqs x prompt tokens)",
        "value": w.B * T / (ms * 1e-3), "unit": "token-steps/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": ARITHMETIC_DTYPE, "data": "synthetic",
        "config": {"workload": w.name, "mode": "prefill", "batch": w.B, "heads": w.H,
                   "d_k": w.dk, "d_v": w.dv, "prompt_tokens": T, "distinct_prompt_tokens": D,
                   "heads_int8": int((head_bits == 8).sum()), "inputs": w.dtype},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic_from_profile(f"{w.name}_prefill", sha, nbytes),
                     "algorithmic_bytes_per_launch": nbytes, "launch_ms": ms,
                     "launch_ms_min": min(per_launch), "launch_ms_median": sorted(per_launch)[K // 2],
                     "launch_ms_max": max(per_launch), "kernel_sha": sha},
        "cpu_baseline": None,
    }
    st.free()
    res["copy_calibration"] = copy_calibration(args.copy_bytes) if args.copy_bytes else None
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=inputs.HEADLINE.name, choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--mode", default="period", choices=("period", "step", "prefill", "window"),
                    help="period: one call per period of k tokens; step: one call per token "
                         "(PACE_STEP_BUFFER handle), every sequence active; prefill: one "
                         "pace_prefill_encode call per prompt (the workload's prompt length); "
                         "window: one call per token with the FP8 write window")
    ap.add_argument("--fp8-window", type=int, default=8, help="window mode: writes kept in FP8")
    ap.add_argument("--prompt-distinct", type=int, default=256,
                    help="prefill mode: distinct prompt tokens generated on the host; the "
                         "device prompt repeats them to the full length")
    ap.add_argument("--adapt-tau", type=float, default=0.0,
                    help="step mode: adaptive period with this threshold (the workload's period "
                         "is the maximum)")
    ap.add_argument("--period", type=int, default=None, help="override the workload's period")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--ring", type=int, default=4, help="distinct input periods resident in HBM")
    ap.add_argument("--cpu-periods", type=int, default=2,
                    help="periods of the whole batch the CPU oracle baseline is timed on")
    ap.add_argument("--cpu-workers", type=int, default=min(16, len(os.sched_getaffinity(0))),
                    help="processes of the CPU baseline (one BLAS thread each)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workers", type=int, default=min(16, len(os.sched_getaffinity(0))))
    ap.add_argument("--copy-bytes", type=int, default=2 << 30,
                    help="bytes of the device-to-device copy timed after the decode region "
                         "(attainable-bandwidth reference; 0 skips it)")
    args = ap.parse_args()

    if args.mode == "prefill":
        return bench_prefill(args)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): every (sequence, head) "
              "state is independent, so this layer needs no collective; the single-GPU figure "
              "is the per-GPU figure.", file=sys.stderr)
        return 2

    import torch

    from linear_attn_decode_pace_amd import pace, runtime

    w = inputs.WORKLOADS[args.workload]
    if args.period:
        w = w.replace(period=args.period)
    C = w.period
    torch.cuda.set_device(0)
    head_bits = inputs.head_bits(w, args.seed)

    t = time.time()
    ring_n = max(1, args.ring)
    # starting state: the workload's warm-up tokens from zero, or for a prompt
    # workload the hand-off of its whole prompt (the first `prompt_distinct`
    # generated prompt tokens repeated to the prompt's length on the device)
    # through pace_prefill_encode
    if w.prompt:
        D = min(w.prompt, args.prompt_distinct)
        warm_jobs = [(inputs.SEG_PROMPT, t0, min(D, t0 + 64)) for t0 in range(0, D, 64)]
    else:
        warm_jobs = [(inputs.SEG_WARMUP, 0, w.warmup)]
    jobs = warm_jobs + [(inputs.SEG_DECODE, p * C, (p + 1) * C) for p in range(ring_n)]
    toks = generate(w, args.seed, jobs, args.workers)
    warm_tok, ring_tok = inputs.concat(toks[:len(warm_jobs)]), toks[len(warm_jobs):]
    log(f"generated inputs in {time.time() - t:.1f} s")

    step_mode = args.mode in ("step", "window")
    window_mode = args.mode == "window"
    adaptive = step_mode and args.adapt_tau > 0
    flags = (pace.PACE_STEP_BUFFER if step_mode and not window_mode else 0) | \
        (pace.PACE_ADAPTIVE if adaptive else 0) | (pace.PACE_FP8_WINDOW if window_mode else 0)
    kw = dict(flags=flags, adapt_tau=args.adapt_tau if adaptive else 0.0,
              fp8_window=args.fp8_window if window_mode else 0)
    if w.prompt:
        h0 = runtime.State(w, head_bits, pace.PACE_INIT_ZERO)
        big = device_prompt(warm_tok, w.prompt)
        h0.prefill(big)
        del big
        raw = h0.read_raw()
        h0.free()
        st = runtime.State(w, head_bits, pace.PACE_INIT_RAW, raw, **kw)
        del raw
        start_state = (f"hand-off of a {w.prompt}-token prompt ({D} distinct generated tokens "
                       f"repeated) through pace_prefill_encode")
        # the CPU oracle starts from a short prompt prefix instead: the cost of
        # a decode period does not depend on the state's values
        cpu_warm = warm_tok.slice(0, min(D, PROMPT_HEAD))
    else:
        M0 = torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
        runtime.prefill(w, runtime.DeviceTokens(warm_tok), M0)
        st = runtime.State(w, head_bits, pace.PACE_INIT_F32, M0, **kw)
        del M0
        start_state = f"{w.warmup} warm-up tokens from zero"
        cpu_warm = warm_tok
    ring = [runtime.DeviceTokens(tk) for tk in ring_tok]
    if step_mode:   # one token per call: the ring's periods cut into tokens
        ring = [r.slice(t, t + 1) for r in ring for t in range(C)]
        ring_n = len(ring)
    out = runtime.out_buffer(w, 1 if step_mode else C)
    call = st.step if step_mode else st.decode
    torch.cuda.synchronize()
    log(f"state and {ring_n} input periods resident ({sum(r.nbytes for r in ring) / 1e9:.2f} GB)")

    for i in range(args.warmup):
        call(ring[i % ring_n], out)
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(K):
        ev[i][0].record()
        call(ring[(args.warmup + i) % ring_n], out)
        ev[i][1].record()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    per_launch = [a.elapsed_time(b) for a, b in ev]
    launch_ms = sum(per_launch) / K
    log(f"timed {K} steps: {total_ms:.3f} ms on the device, {t_wall * 1e3:.1f} ms wall")
    log("per-launch ms: " + " ".join(f"{x:.4f}" for x in per_launch))

    k_eff = None
    adapt_bytes = None
    if adaptive:
        # realised mean period and exact bytes per call: replay as many steps
        # untimed, reading every state's buffer fill before and after each
        # call (a fill back to 0 closed the period)
        closes, total = 0, 0.0
        fill, _ = st.read_step()
        for i in range(K):
            call(ring[(args.warmup + K + i) % ring_n], out)
            after, _ = st.read_step()
            closed = after == 0
            closes += int(closed.sum().item())
            total += step_bytes_exact(w, head_bits, fill, closed)
            fill = after
        k_eff = K * w.B * w.H / max(1, closes)
        adapt_bytes = total / K
        log(f"adaptive period: mean period {k_eff:.2f} tokens over {K} steps, "
            f"{adapt_bytes / 1e6:.1f} MB per call")
    if window_mode:
        nbytes = window_bytes(w, head_bits, args.fp8_window)
    elif adaptive:
        nbytes = adapt_bytes
    elif step_mode:
        nbytes = algorithmic_bytes_step(w, head_bits, k_eff)
    else:
        nbytes = algorithmic_bytes(w, C, head_bits)
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    sha = kernel_sha(1 if step_mode else C, window=window_mode)
    tokens_per_call = 1 if step_mode else C
    value = w.B * tokens_per_call * K / (total_ms * 1e-3)
    res = {
        "metric": "decode token-steps/s per GDN layer (seqs x tokens) + achieved HBM GB/s vs peak",
        "value": value,
        "unit": "token-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": total_ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ARITHMETIC_DTYPE,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "d_k": w.dk, "d_v": w.dv,
                   "period": C, "heads_int8": int((head_bits == 8).sum()),
                   "inputs": w.dtype, "outlier_channels": w.n_outliers,
                   "mode": args.mode, "decode_steps": K * tokens_per_call,
                   "adapt_tau": args.adapt_tau if adaptive else None,
                   "fp8_window": args.fp8_window if window_mode else None,
                   "mean_period": k_eff,
                   "input_ring_calls": ring_n, "arithmetic": ARITHMETIC,
                   "start_state": start_state},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": None if step_mode else traffic_from_profile(w.name, sha, nbytes),
                     "algorithmic_bytes_per_launch": nbytes, "launch_ms": launch_ms,
                     "launch_ms_min": min(per_launch),
                     "launch_ms_median": sorted(per_launch)[K // 2],
                     "launch_ms_max": max(per_launch),
                     "kernel_sha": sha},
    }
    st.free()
    del ring, out
    res["copy_calibration"] = copy_calibration(args.copy_bytes) if args.copy_bytes else None
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, cpu_warm, ring_tok[:max(1, args.cpu_periods)], head_bits,
                          args.cpu_workers)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
