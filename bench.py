"""Benchmark of the Falcon chunked forward pass on one MI355X.

Default workload: Falcon-1, the layer shape of the pages' 124-130M models
(batch 8, 12 heads, head dim 64, T = 2048, bf16 q/k/v, fp32 state, chunk 64),
synthetic N(0,1) inputs.  One step = one falcon_chunk_fwd call over one batch
(gates, outputs o, final S and x_prev included).  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--variant V]

Timing: three rotating input sets (more bytes than the 256 MB MALL), W untimed
calls, then K timed calls bracketed by torch.cuda.synchronize() and by one pair of
HIP events on the stream they are launched on: the wall time gives the
throughput, the event time over K each call's average device time, used for the
roofline.  Before the warmup steps, about --settle-ms (300) of untimed calls let
the GPU's clocks settle.  A second, untimed pass brackets each call by events of its own for the
p10 / p50 / p90 of the durations (per-call events cost the stream a few
microseconds each, so they stay out of the timed loop), and a third reuses one
input set (the warm figure).  Paths
(--path): "onepass" calls without a workspace (the one-pass kernel where it is
built, else the fused kernel); "split" passes a workspace (allocated once
outside the timed region): the prep kernel over all systems, then the state
scan (for Falcon-3A windows at head dim 64: the banded-weight kernels, the
chunks' state increments, their scan and the outputs).  "auto" (default) takes the faster one measured per shape class: split
for Falcon-3 windows and head dim 128, one-pass otherwise, and for long
sequences too few to fill the device (B*H*dv/16 <= 128 scan workgroups, T >=
16384, one pair per step) the segment-parallel form with 8 segments.
--segments P runs the segment-parallel form with P segments.

--backward times falcon_chunk_bwd instead: the gradients of every input from
the forward's per-chunk states, which are computed once outside the timed
region.  Falcon-1 / 1A / 2 / 2A at head dim 64 run the chunk-parallel kernels;
windows (--variant F3 / F3A --window B_w) and other head dims the recurrent
form.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

class TimingEvent:
    """A HIP event used only for timing, created with hipEventDisableSystemFence:
    recording it skips the system-scope fence (cache writeback and invalidation)
    that a default event performs, which HIP documents as the form for timing
    measurements.  The elapsed times are read after a device synchronisation, so
    nothing relies on the fence.  Recorded on the stream the kernels run on."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._ct = ctypes
        self.handle = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.handle), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = TimingEvent._hip.hipEventRecord(self.handle, self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        ms = self._ct.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if TimingEvent._hip is not None and self.handle:
            TimingEvent._hip.hipEventDestroy(self.handle)


def settle(call, sets, ms):
    """Untimed, before the warmup steps: calls for about `ms` milliseconds, so the
    GPU's clocks reach their steady state (20 warmup calls of the 130M-layer
    forward are about 1 ms, after which the same loop still ran 15 % slower than
    after 2000).  Synchronises every 64 calls to keep the queue short."""
    import torch
    t_end = time.perf_counter() + ms / 1e3
    i = 0
    while time.perf_counter() < t_end:
        call(sets[i % len(sets)])
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def with_settle(line, args):
    """The settle phase's length, stated in the line's roofline object."""
    line["roofline"]["settle_ms"] = args.settle_ms
    return line


def time_loop(call, sets, K, stream):
    """The timed region: K calls, input sets rotating, bracketed by device
    synchronisations and by one pair of timing events on the launch stream, with
    nothing else in the loop.  Returns (wall seconds, event seconds); the event
    time over K is each launch's average duration."""
    import torch
    start, end = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        call(sets[i % len(sets)])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / 1e3


def per_call_ms(call, sets, K, stream, rotate=True):
    """Outside the timed region: each of K calls bracketed by events of its own,
    the distribution of launch durations (ms, sorted).  Recording two events per
    call costs the stream a few microseconds per call, so these run apart from
    the timed loop.  rotate=False reuses one input set (the warm figure)."""
    import torch
    ev = [(TimingEvent(), TimingEvent()) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record(stream)
        call(sets[i % len(sets)] if rotate else sets[0])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)


METRIC = "tokens/sec, Falcon-1 chunked fwd (H=12,d=64,T=2048) + % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA


def alg_bytes(w, variant):
    """Algorithmic HBM bytes of one call: q, k, v, o in the input dtype, the fp32
    gates (beta is per channel for F2/F2A), the final S and x_prev."""
    e = 2 if w.dtype == "bf16" else 4
    per_th = (2 * w.dk + 2 * w.dv) * e + 8 + (4 * w.dv - 4 if variant in ("F2", "F2A") else 0)
    per_seq = w.dv * w.dk * 4 + w.dk * 4
    return w.batch * w.heads * (w.seqlen * per_th + per_seq)


def ref_flops(w, variant, window=1):
    """Fixed reference flop count of the chunked form at the configured chunk C.

    Falcon-3 with a window: per WY system of C/Bw steps and C virtual rows, since
    every pair's residual enters the triangular system.  Falcon-3A keeps the
    per-chunk count of the additive write: with no residual, the window average
    folds into banded weights on a score matrix of C rows (the chunked formulas'
    F3A form), so a window adds no products; the kernels' virtual rows are an
    implementation choice and are not counted."""
    C, dk, dv = w.chunk, w.dk, w.dv
    if variant == "F3" and window > 1:
        cs, m = C // window, C
        per_sub = (2 * m * m * (2 * dk + dv) + m ** 3 / 3 + 4 * m * dk * dv + 2 * cs * m * (dk + dv)
                   + 2 * cs * dk * dv)
        return w.batch * w.heads * (-(-w.seqlen // cs)) * per_sub
    per_chunk = {
        "F1": 2 * C * C * (3 * dk + 2 * dv) + 6 * C * dk * dv + C ** 3 / 3,
        "F1A": 2 * C * C * (dk + dv) + 4 * C * dk * dv,
        "F2": 4 * C * C * dk + 6 * C * dk * dv + 2 * C * C * dv + C * C * dv,
        "F2A": 2 * C * C * (dk + dv) + 4 * C * dk * dv,
        "F3": 2 * C * C * (3 * dk + 2 * dv) + 6 * C * dk * dv + C ** 3 / 3,
        "F3A": 2 * C * C * (dk + dv) + 4 * C * dk * dv,
    }[variant]
    nch = -(-w.seqlen // C)
    return w.batch * w.heads * nch * per_chunk


DECODE = dict(batch=256, heads=16, d=128)   # the long-context workload's decode step


def bench_decode(args):
    """One falcon_recurrent_step over batch 256 x 16 heads x 128x128 fp32 states
    (bf16 q/k/v/o): HBM-bound, the state is read and written once."""
    import torch
    import workloads as W
    from recurrent_sequence_models_amd import recurrent_step
    B, H, d = DECODE["batch"], DECODE["heads"], DECODE["d"]
    dev = torch.device("cuda:0")
    bw = args.window if args.variant in ("F3", "F3A") else 1
    sets = []
    for i in range(3):
        inp = W.make_decode_inputs(B, H, d, d, args.variant, seed=505 + i, window=bw, dtype="bf16")
        dd = {n: torch.from_numpy(a).to(dev) for n, a in inp.items()}
        for n in ("q", "k", "v"):
            dd[n] = dd[n].to(torch.bfloat16).contiguous()
        sets.append(dd)
    stream = torch.cuda.current_stream()

    def call(dd):
        recurrent_step(args.variant, dd["q"], dd["k"], dd["v"], dd["beta"], dd["log_lambda"], dd,
                       window=bw, stream=stream)

    settle(call, sets, args.settle_ms)
    for i in range(args.warmup):
        call(sets[i % 3])
    torch.cuda.synchronize()
    K = args.steps
    wall, ev_s = time_loop(call, sets, K, stream)
    kern_s = ev_s / K
    per_ms = per_call_ms(call, sets, K, stream)
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    per_state = 2 * d * d * 4 + 2 * d * 4 + (2 * d + 2 * d) * 2 + 8 + (2 * (bw - 1) * 2 * d * 4 if bw > 1 else 0)
    nbytes = B * H * per_state
    ach = nbytes / kern_s / 1e9
    return {
        "metric": "decode steps/sec (batch 256 x 16 heads x 128x128 fp32 states)",
        "value": round(B / (wall / K), 1), "unit": "sequences/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"Falcon-{args.variant[1:]} recurrent step, B{B} H{H} d{d}, fp32 state, bf16 q/k/v/o",
                   "variant": args.variant, "window": bw},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"decode {args.variant} b{B} h{H} d{d} w{bw}", DECODE_SOURCES),
                     "kernel": "step_kernel",
                     "kernel_us": {"mean": round(kern_s * 1e6, 2), "per_call_mean": round(sum(per_ms) / K * 1e3, 2),
                                   "p10": round(per_ms[K // 10] * 1e3, 2), "p50": round(per_ms[K // 2] * 1e3, 2),
                                   "p90": round(per_ms[(9 * K) // 10] * 1e3, 2)}, "alg_bytes": nbytes},
    }


MFMA_FP32_PEAK_TFS = 157.3    # MI355X dense fp32 MFMA
VALU_FP32_PEAK_TFS = 157.3    # MI355X fp32 vector ALUs


def bwd_flops(w, variant):
    """Algorithmic flops of one backward call, per chunk of C steps: the chunked
    products of the adjoint (a triangular C x C product counts half).  With
    u = 2 C d^2 (C = d): F1 and F2 = 15 u (prep 3, scan 2, per-chunk adjoint 10);
    F1A and F2A = 6.5 u (prep 1, adjoint 5.5)."""
    C, d = w.chunk, w.dk
    u = 2 * C * d * d
    # F2: the products of F1 with F = eta (.) E in place of diag(eta) E (its per-channel
    # diagonal-block substitutions are not counted); F2A: F1A on beta (.) v
    per_chunk = {"F1": 15 * u, "F1A": 6.5 * u, "F2": 15 * u, "F2A": 6.5 * u}[variant]
    return w.batch * w.heads * (-(-w.seqlen // C)) * per_chunk


def bwd_rows_path(w, variant, window):
    """True where the backward runs in the recurrent form (windows of more than
    one pair, head dims other than 64); the chunk-parallel kernels elsewhere."""
    return (variant in ("F3", "F3A") and window > 1) or w.dk != 64


def bwd_rows_flops(w, variant, window):
    """Algorithmic flops of the recurrent-form backward: per step and sequence,
    one forward step, (1 + 4 B_w) d^2, and its adjoint, (7 + 10 B_w) d^2 (B_w = 1
    outside Falcon-3 / 3A).  They run on the vector ALUs in fp32."""
    bw = window if variant in ("F3", "F3A") else 1
    return w.batch * w.heads * w.seqlen * (8 + 14 * bw) * w.dk * w.dv


def bwd_bytes(w, variant="F1"):
    """Algorithmic HBM bytes of one backward call: q, k, v, do in the input
    dtype, beta and g, the per-chunk states, the fp32 gradients of q, k, v,
    beta and g, and the final-state gradient and initial-state gradients
    (F2A: beta and its gradient per value channel)."""
    e = 2 if w.dtype == "bf16" else 4
    nch = -(-w.seqlen // w.chunk)
    nb = w.dv if variant in ("F2", "F2A") else 1
    per_th = 4 * w.dk * e + 4 * nb + 4 + 3 * w.dk * 4 + 4 * nb + 4
    per_seq = nch * w.dv * w.dk * 4 + 2 * w.dv * w.dk * 4 + w.dk * 4
    return w.batch * w.heads * (w.seqlen * per_th + per_seq)


def host_cores():
    """Cores this process may run on (the oracle itself uses one)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline_bwd(w, variant, window=1, budget_s=20.0):
    """Time the oracle's backward (as it stands) on a prefix of the same workload,
    on one host core; scaled to tokens/s of the full batch."""
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    import oracle
    import workloads as W
    inp = W.make_inputs(w, variant, seed=w.seed, window=window)
    cot = W.make_cotangents(w, w.seed + 1)
    t_probe = 16
    t0 = time.perf_counter()
    oracle.recurrent_backward(variant, **{n: a[:, :t_probe] for n, a in inp.items()}, do=cot["do"][:, :t_probe],
                              dS_T=cot["dS_T"], window=window)
    per_step = (time.perf_counter() - t0) / t_probe
    T_s = int(max(t_probe, min(w.seqlen, budget_s / max(per_step, 1e-9))))
    t0 = time.perf_counter()
    oracle.recurrent_backward(variant, **{n: a[:, :T_s] for n, a in inp.items()}, do=cot["do"][:, :T_s],
                              dS_T=cot["dS_T"], window=window)
    dt = time.perf_counter() - t0
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    return {"value": w.batch * T_s / dt, "unit": "tokens/s", "cores": 1, "host_cores": host_cores(),
            "kind": "oracle",
            "sample": f"fp64 NumPy reverse-time adjoint (with its forward) over all {w.batch * w.heads} "
                      f"sequences of the workload, first {T_s} of {w.seqlen} steps ({dt:.1f} s on 1 of "
                      f"{host_cores()} host cores)"}


def bench_backward(args):
    """K timed falcon_chunk_bwd calls over three rotating input sets (inputs,
    cotangents and the forward's per-chunk states resident in HBM)."""
    import torch
    import workloads as W
    from recurrent_sequence_models_amd import chunk_bwd, chunk_fwd
    from recurrent_sequence_models_amd.falcon import bwd_workspace_bytes
    w = W.WORKLOADS[args.workload]
    variant = args.variant
    win = args.window if variant in ("F3", "F3A") else 1
    rows = bwd_rows_path(w, variant, win)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    sets = []
    for i in range(3):
        inp = W.make_inputs(w, variant, seed=w.seed + i, window=win)
        cot = W.make_cotangents(w, w.seed + 10 + i)
        d = {n: torch.from_numpy(a).to(dev) for n, a in inp.items()}
        for n in ("q", "k", "v"):
            d[n] = d[n].to(tdt).contiguous()
        d["do"] = torch.from_numpy(cot["do"]).to(dev).to(tdt).contiguous()
        d["dS_T"] = torch.from_numpy(cot["dS_T"]).to(dev)
        _, _, d["cs"] = chunk_fwd(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], chunk=w.chunk,
                                  window=win, final=False, chunk_states=True)
        d["out"] = dict(dq=torch.empty(w.batch, w.seqlen, w.heads, w.dk, device=dev),
                        dk=torch.empty(w.batch, w.seqlen, w.heads, w.dk, device=dev),
                        dv=torch.empty(w.batch, w.seqlen, w.heads, w.dv, device=dev),
                        dbeta=torch.empty(*d["beta"].shape, device=dev),
                        dg=torch.empty(w.batch, w.seqlen, w.heads, device=dev))
        d["d_init"] = dict(S=torch.empty(w.batch, w.heads, w.dv, w.dk, device=dev),
                           x_prev=torch.empty(w.batch, w.heads, w.dk, device=dev))
        if win > 1:
            d["d_init"]["win_x"] = torch.empty(w.batch, w.heads, win - 1, w.dk, device=dev)
            d["d_init"]["win_v"] = torch.empty(w.batch, w.heads, win - 1, w.dv, device=dev)
        sets.append(d)
    ws_bytes = bwd_workspace_bytes(variant, w.dtype, w.batch, w.seqlen, w.heads, w.dk, w.dv, w.chunk, window=win)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def call(d):
        chunk_bwd(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], d["do"], d["cs"], dS_T=d["dS_T"],
                  chunk=w.chunk, window=win, d_init=d["d_init"], out=d["out"], workspace=ws, stream=stream)

    settle(call, sets, args.settle_ms)
    for i in range(args.warmup):
        call(sets[i % 3])
    torch.cuda.synchronize()
    K = args.steps
    wall, ev_s = time_loop(call, sets, K, stream)
    avg_s = ev_s / K
    kern_ms = per_call_ms(call, sets, K, stream)
    flops = bwd_rows_flops(w, variant, win) if rows else bwd_flops(w, variant)
    nbytes = bwd_bytes(w, variant)
    tfs = flops / avg_s / 1e12
    gbs = nbytes / avg_s / 1e9
    # bf16 inputs run the chunk-parallel products on bf16 MFMA, fp32 inputs on fp32
    # MFMA; the recurrent form runs on the fp32 vector ALUs.  The roofline is
    # whichever of that peak and HBM bounds the call
    bf = w.dtype == "bf16"
    mpeak = VALU_FP32_PEAK_TFS if rows else MFMA_BF16_PEAK_TFS if bf else MFMA_FP32_PEAK_TFS
    if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (mpeak * 1e12):
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "alu" if rows else "mfma", "achieved": round(tfs, 2), "peak": mpeak, "unit": "TFLOP/s",
                "frac": round(tfs / mpeak, 4)}
    line = {
        "metric": f"tokens/sec, Falcon-{variant[1:]} {'recurrent-form' if rows else 'chunked'} backward "
                  f"(H={w.heads},d={w.dk},T={w.seqlen}{f',B_w={win}' if win > 1 else ''}) + % roofline",
        "value": round(w.batch * w.seqlen / (wall / K), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf else "f32", "data": "synthetic",
        "config": {"workload": f"Falcon-{variant[1:]} backward, {w.name}: B{w.batch} H{w.heads} "
                               f"T{w.seqlen} d{w.dk} chunk {w.chunk}{f' window {win}' if win > 1 else ''}, "
                               f"{w.dtype} q/k/v/do, fp32 gradients",
                   "variant": variant, "batch": w.batch, "heads": w.heads, "seq_len": w.seqlen,
                   "head_dim": w.dk, "chunk": w.chunk, "window": win},
        "roofline": {**roof, "traffic": None,
                     "kernel": "bwd_rows + bwd_rows_finish" if rows else "bwd_prep + bwd_scan + bwd_chunk",
                     "kernel_us": {"mean": round(avg_s * 1e6, 2), "per_call_mean": round(sum(kern_ms) / K * 1e3, 2),
                                   "p10": round(kern_ms[K // 10] * 1e3, 2),
                                   "p50": round(kern_ms[K // 2] * 1e3, 2),
                                   "p90": round(kern_ms[(9 * K) // 10] * 1e3, 2)},
                     "alg_flops": flops, "alg_bytes": nbytes,
                     "mfma_frac": None if rows else round(tfs / mpeak, 4), "mfma_peak": None if rows else mpeak,
                     "measured_busy": None if rows else measured_busy(f"backward {variant} {w.name}", BWD_SOURCES),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "workspace_bytes": ws_bytes},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_bwd(w, variant, win)
    return line


KERNEL_SOURCES = ("split_impl.h", "falcon_fwd_split.hip", "falcon_fwd_split_win.hip", "falcon_fwd_pipe.hip",
                  "chunk_common.h", "mfma_frag.h", "falcon_kernels.h")


DECODE_SOURCES = ("falcon_step.hip", "falcon_kernels.h", "mfma_frag.h")
BWD_SOURCES = ("falcon_bwd.hip", "falcon_kernels.h", "mfma_frag.h", "lane_ops.h")
# the segment-parallel forward also runs the boundary and combine kernels
SEG_SOURCES = KERNEL_SOURCES + ("falcon_segment.hip",)
# Falcon-3A windows at d = 64, chunk 64: the banded-weight kernels
BAND_SOURCES = ("falcon_fwd_band.hip", "chunk_common.h", "mfma_frag.h", "falcon_kernels.h")


def band_path(w, variant, window, path):
    """True where the two-kernel request runs the banded-weight kernels."""
    return path == "split" and variant == "F3A" and window > 1 and w.dk == 64 and w.dv == 64 and w.chunk == 64


def measured_traffic(key, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed counter record, or None when the
    kernel code changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))[key]
    except (OSError, KeyError, ValueError):
        return None
    return round(rec["bytes_per_launch"]) if code_digest(sources) == rec["source_sha256"] else None


def measured_busy(key, sources=KERNEL_SOURCES):
    """Unit busy fractions from the committed SQ-counter record (rocprofv3, the
    dominant kernel), or None when the kernel code changed since they were taken:
    mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES), the share
    of the MFMA pipes' cycles in use while the kernel held its compute units, and
    valu_issue = SQ_INSTS_VALU / SQ_BUSY_CU_CYCLES (MFMA included; a compute unit
    issues at most one wave64 VALU instruction per cycle)."""
    path = os.path.join(ROOT, "profiles", "sq_counters.json")
    try:
        rec = json.load(open(path))[key]
    except (OSError, KeyError, ValueError):
        return None
    if code_digest(sources) != rec["source_sha256"]:
        return None
    return {"kernel": rec["kernel"], "mfma_busy": round(rec["mfma_busy"], 4), "valu_issue": round(rec["valu_issue"], 4)}


def code_digest(sources):
    """sha256 over the kernel sources with comments and blank lines removed, so
    that a comment edit keeps the counter record while any code change drops it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "recurrent_sequence_models_amd", "csrc", f)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            line = re.sub(r"//.*$", "", line).rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def cpu_baseline(w, variant, window=1, budget_s=20.0):
    """Time the fp64 oracle (as it stands) on a prefix of the same workload, on
    one host core; scaled to tokens/s of the full batch."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    import oracle
    import workloads as W
    inp = W.make_inputs(w, variant, seed=w.seed)
    # calibrate on a short prefix, then run a prefix sized for the time budget
    t_probe = 32
    t0 = time.perf_counter()
    oracle.recurrent(variant, **{n: a[:, :t_probe] for n, a in inp.items()}, window=window)
    per_step = (time.perf_counter() - t0) / t_probe
    T_s = int(max(t_probe, min(w.seqlen, budget_s / max(per_step, 1e-9))))
    t0 = time.perf_counter()
    oracle.recurrent(variant, **{n: a[:, :T_s] for n, a in inp.items()}, window=window)
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {"value": w.batch * T_s / dt, "unit": "tokens/s", "cores": 1, "host_cores": host_cores(),
            "kind": "oracle",
            "sample": f"fp64 NumPy step loop over all {w.batch * w.heads} sequences of the workload, "
                      f"first {T_s} of {w.seqlen} steps ({dt:.1f} s on 1 of {host_cores()} host cores)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed calls before the warmup steps, in ms of wall time (clock settling)")
    ap.add_argument("--workload", default="layer130m")
    ap.add_argument("--variant", default="F1")
    ap.add_argument("--window", type=int, default=4, help="Falcon-3/3A window (pairs)")
    ap.add_argument("--decode", action="store_true", help="time the single-token step instead")
    ap.add_argument("--backward", action="store_true", help="time the chunked backward pass instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=("auto", "onepass", "split"), default="auto",
                    help="forward path: one-pass (no workspace), split (workspace), or auto")
    ap.add_argument("--segments", type=int, default=0,
                    help="cut every sequence into this many segments run at once (segment-parallel form)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every (b, h) sequence is independent: more GPUs would each run their own share)",
              file=sys.stderr)
        sys.exit(2)

    if args.decode:
        print(json.dumps(with_settle(bench_decode(args), args)), flush=True)
        return
    if args.backward:
        print(json.dumps(with_settle(bench_backward(args), args)), flush=True)
        return

    import torch
    import workloads as W
    from recurrent_sequence_models_amd import ForwardCall, chunk_fwd_segmented, new_state
    from recurrent_sequence_models_amd.falcon import segmented_workspace_bytes, workspace_bytes

    w = W.WORKLOADS[args.workload]
    variant = args.variant
    window = args.window if variant in ("F3", "F3A") else 1
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    # three rotating input sets, each with its own outputs and final state
    sets = []
    for i in range(3):
        inp = W.make_inputs(w, variant, seed=w.seed + i)
        d = {n: torch.from_numpy(a).to(dev) for n, a in inp.items()}
        for n in ("q", "k", "v"):
            d[n] = d[n].to(tdt).contiguous()
        d["o"] = torch.empty(w.batch, w.seqlen, w.heads, w.dv, dtype=tdt, device=dev)
        d["final"] = new_state(w.batch, w.heads, w.dk, w.dv, window=window, device=dev)
        sets.append(d)
    del inp
    stream = torch.cuda.current_stream()
    split_bytes = workspace_bytes(variant, w.dtype, w.batch, w.seqlen, w.heads, w.dk, w.dv, w.chunk, window)
    want = args.path if args.path != "auto" else ("split" if (window > 1 or w.dk >= 128) else "onepass")
    ws_bytes = split_bytes if want == "split" else 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else False
    path = "split" if ws_bytes else "onepass"
    if (args.path == "auto" and args.segments == 0 and window == 1 and variant != "F2"
            and w.batch * w.heads * (w.dv // 16) <= 128 and w.seqlen >= 16384 and w.seqlen % 16 == 0):
        args.segments = 8

    if args.segments > 0:
        ws_bytes = segmented_workspace_bytes(variant, w.dtype, w.batch, w.seqlen, w.heads, w.dk, w.dv, args.segments,
                                             w.chunk, window)
        if ws_bytes == 0:
            print(f"the segmented form is not built for {variant} {w.name} with {args.segments} segments",
                  file=sys.stderr)
            sys.exit(2)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        path = f"segmented x{args.segments}"

    # each input set's forward, validated once (ForwardCall): a step is then one C call
    if args.segments == 0:
        for d in sets:
            d["fwd"] = ForwardCall(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], chunk=w.chunk,
                                   window=window, final=d["final"], out=d["o"], stream=stream, workspace=ws)

    def call(d):
        if args.segments > 0:
            chunk_fwd_segmented(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], args.segments,
                                chunk=w.chunk, window=window, final=d["final"], out=d["o"], stream=stream,
                                workspace=ws)
            return
        d["fwd"]()

    settle(call, sets, args.settle_ms)
    for i in range(args.warmup):
        call(sets[i % 3])
    torch.cuda.synchronize()

    K = args.steps
    wall, ev_s = time_loop(call, sets, K, stream)
    avg_kernel_s = ev_s / K
    ms_per_step = wall / K * 1e3
    tokens = w.batch * w.seqlen
    # outside the timed region: each call's duration (p10 / p50 / p90), and the warm
    # figure, one input set reused (104 MB stays in the 256 MB MALL)
    kern_ms = per_call_ms(call, sets, K, stream)
    warm_ms = per_call_ms(call, sets, K, stream, rotate=False)
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    nbytes = alg_bytes(w, variant) + (w.batch * w.heads * (window - 1) * (w.dk + w.dv) * 4 if window > 1 else 0)
    flops = ref_flops(w, variant, window)
    achieved = nbytes / avg_kernel_s / 1e9
    mfma_tfs = flops / avg_kernel_s / 1e12
    bound = "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFS * 1e12) else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(mfma_tfs, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(mfma_tfs / MFMA_BF16_PEAK_TFS, 4)}
    key = f"{path} {variant} {w.name}" + (f" w{window}" if window > 1 else "")
    band = band_path(w, variant, window, path)
    sources = SEG_SOURCES if path.startswith("segmented") else BAND_SOURCES if band else KERNEL_SOURCES
    roof["traffic"] = measured_traffic(key, sources)
    roof["measured_busy"] = measured_busy(key, sources)
    roof["kernel"] = ("seg_boundary + chunk_prep + 2 x chunk_scan (map form) + seg_combine + chunk_scan"
                      if path.startswith("segmented") else
                      "band_state + band_scan + band_out" if band else
                      "chunk_prep + chunk_scan" if path == "split" else
                      "chunk_scan (one-pass)" if (w.dtype == "bf16" and w.dk <= 64 and w.chunk <= 64) else
                      "chunk_fwd_pipe" if w.dk <= 64 else "chunk_fwd_rows")
    roof["path"] = path
    roof["workspace_bytes"] = ws_bytes
    # mean: the timed region's event pair over K; the rest from each call's own events
    roof["kernel_us"] = {"mean": round(avg_kernel_s * 1e6, 2), "per_call_mean": round(sum(kern_ms) / K * 1e3, 2),
                         "p10": round(kern_ms[K // 10] * 1e3, 2),
                         "p50": round(kern_ms[K // 2] * 1e3, 2), "p90": round(kern_ms[(9 * K) // 10] * 1e3, 2)}
    roof["kernel_us_warm"] = {"mean": round(sum(warm_ms) / K * 1e3, 2), "p50": round(warm_ms[K // 2] * 1e3, 2)}
    roof["alg_bytes"] = nbytes
    roof["ref_flops"] = flops
    roof["mfma_frac"] = round(mfma_tfs / MFMA_BF16_PEAK_TFS, 4)

    line = {
        "metric": METRIC,
        "value": round(tokens / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"Falcon-{variant[1:]} chunked forward, {w.name}: B{w.batch} H{w.heads} "
                               f"T{w.seqlen} d{w.dk} chunk {w.chunk}" + (f" window {window}" if window > 1 else "")
                               + f", {w.dtype} q/k/v/o, fp32 state",
                   "variant": variant, "batch": w.batch, "heads": w.heads, "seq_len": w.seqlen,
                   "head_dim": w.dk, "chunk": w.chunk, "window": window, "segments": max(args.segments, 1)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, variant, window)
    print(json.dumps(with_settle(line, args)), flush=True)


if __name__ == "__main__":
    main()
