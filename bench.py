#!/usr/bin/env python3
"""Benchmark of the MI355X SSD layer (chunked forward + recurrent decode).

One step = one full forward (all four stages) of the Mamba-2 2.7B-shaped SSD
layer -- batch 8, seqlen 4096, 80 heads, headdim 64, state 128, 1 group,
chunk 256, bf16 X/B/C with fp32 a, returning the final state -- over one
batch of seeded synthetic inputs already resident in HBM.  Distinct input
batches are cycled so that the timed loop's working set exceeds the 256 MB
Infinity Cache.

Before each timed leg's W warm-up steps the GPU runs CLOCK_SETTLE_MS of
the library's streaming kernel on a scratch array (clock_settle_ms in the
line): after the host-side input generation its clocks need ~25 ms of
sustained work to come back up, which would otherwise land in the K timed
steps.

Prints ONE JSON line.  Besides the contract fields it carries:
  roofline      the dominant kernel (the fused pass) against the HBM peak:
                algorithmic bytes per launch over that kernel's own average
                launch duration, measured with HIP events on the launch
                stream (the pass alone through its stage entry point when the
                step has several launches, the step itself when it is that
                one launch); `traffic` is the counter-measured HBM bytes of a
                launch from the committed rocprofv3 summary when that was
                taken on the current kernel source;
  mfma          MFMA flops of the step against the bf16 dense peak, counted
                at the caller's chunk (the survey's algorithmic count:
                causal halves of the chunk's C B^T and masked product, chunk
                state and state-to-output) and at the 64-step blocks the
                kernels execute;
  passes        the step's launches timed one by one the same way;
  cpu_baseline  the fp64 CPU oracle on the same workload (host cores);
  secondary     the rest of the metric's workloads: the 130M-shaped layer
                (bf16, and fp32 through the VALU kernel),
                the state-64 seqlen sweep at all six lengths (512 .. 512K),
                the decode step's HBM bandwidth (and the in-place stream
                ceiling of the same state array), and the backward of the
                130M-shaped layer.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector


def fwd_algo_bytes_per_token(sh):
    """Minimum HBM bytes per token: X in, Y out, B and C, a (fp32)."""
    es = 2 if sh.dtype == "bf16" else 4
    return sh.nheads * sh.headdim * 2 * es + 2 * sh.ngroups * sh.dstate * es + 4 * sh.nheads


def fwd_algo_bytes(sh):
    """Minimum HBM bytes of one forward: every token's bytes, plus the final
    state (fp32) when the workload returns it."""
    fin = sh.batch * sh.nheads * sh.headdim * sh.dstate * 4 if sh.final_state else 0
    return sh.batch * sh.seqlen * fwd_algo_bytes_per_token(sh) + fin


KERNEL_BLOCK = 64   # the fused kernels' block length (the output does not depend on it)


def fwd_algo_flops_per_token(sh, block=KERNEL_BLOCK):
    """MFMA flops per token of the blocked form with blocks of `block` steps:
    causal half of C B^T once per group, causal half of (L o S) X per head,
    block state and state-to-output per head.  With block = the caller's
    chunk this is the survey's algorithmic count."""
    Q, N, P, H, G = block, sh.dstate, sh.headdim, sh.nheads, sh.ngroups
    return (Q + 1) * (N * G + P * H) + 4 * N * P * H


def stored_traffic(profile):
    """HBM bytes per launch of the fused-pass kernel from a committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary (calibrated on a plain copy), or None when
    that summary was taken on a different kernel source."""
    prof = os.path.join(ROOT, "profiles", profile)
    try:
        sha = fused_kernel_sha()
        fields = dict(l.split(":", 1) for l in open(prof) if l.startswith(("traffic_bytes", "kernel_source")))
    except (OSError, ValueError):
        return None
    if fields.get("kernel_source_sha256_16", "").strip() != sha:
        return None
    return int(fields["traffic_bytes_per_launch"])


def fused_kernel_sha():
    """First 16 hex digits of the SHA-256 of the fused-pass kernel's sources."""
    import hashlib
    h = hashlib.sha256()
    for f in ("kernels_fwd.hip", "mfma_util.hpp"):
        h.update(open(os.path.join(ROOT, "ssd_chunked_scan_chunk_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def upload(d):
    import torch
    dt = d["shape"].dtype
    out = {}
    for k in ("X", "B", "C"):
        arr = d[k]
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16)).view(torch.bfloat16) \
            if dt == "bf16" else torch.from_numpy(arr)
        out[k] = t.to("cuda")
    out["a"] = torch.from_numpy(d["a"]).to("cuda")
    return out


CLOCK_SETTLE_MS = 100.0
_settle_buf = None


def settle_clocks(ms=CLOCK_SETTLE_MS):
    """Keep the GPU busy for `ms` milliseconds with the library's streaming
    kernel on a 256 MB scratch array (not a step of any workload).  After the
    seconds of host-side input generation the GPU's clocks take ~25 ms of
    sustained work to come back up: the 2.7B-shaped forward reads 0.27-0.29 ms
    in its first 20 steps after a 5-step warm-up and 0.226 ms from ~100 steps
    on.  Every timed leg calls this right before its warm-up steps, so the K
    timed steps measure the kernels at their running clocks."""
    import torch
    import ssd_chunked_scan_chunk_amd as ssd
    global _settle_buf
    if _settle_buf is None:
        _settle_buf = torch.zeros(64 << 20, dtype=torch.float32, device="cuda")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    done = 0.0
    while done < ms:
        e0.record()
        for _ in range(20):
            ssd.stream_rmw(_settle_buf, 1.0, 1, True)
        e1.record()
        e1.synchronize()
        done += e0.elapsed_time(e1)


def warm(fn, min_steps, min_ms=30.0):
    """Untimed calls of fn: at least min_steps, and at least min_ms of GPU
    time (the secondary legs, whose steps range from 20 us to 2 ms)."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    done, i = 0.0, 0
    while i < min_steps or done < min_ms:
        e0.record()
        for _ in range(max(1, min_steps)):
            fn(i)
            i += 1
        e1.record()
        e1.synchronize()
        done += e0.elapsed_time(e1)


def time_events(fn, steps):
    """Seconds for `steps` calls of fn, between HIP events on the current
    stream.  One untimed call is queued ahead of the first event, so that a
    host-side pause at the first launch after the synchronisation lands
    outside the timed region; the garbage collector is held off meanwhile
    (not run first: a collection idles the GPU long enough for its clocks to
    drop before the timed calls)."""
    import gc
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    gc.disable()
    try:
        torch.cuda.synchronize()
        fn(steps)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
    finally:
        gc.enable()
    return e0.elapsed_time(e1) / 1e3  # seconds


def bench_forward(sh, steps, warmup, nbatch, seed0=0, warm_ms=0.0):
    """Time `steps` forwards cycling over `nbatch` seeded batches.
    Returns (seconds per step, seconds per launch of the full-pass kernel,
    plan, per-pass milliseconds)."""
    import torch
    import ssd_chunked_scan_chunk_amd as ssd
    import ssd_inputs as si
    batches = [upload(si.make_fwd(sh, seed=seed0 + i)) for i in range(nbatch)]
    Ys = [torch.empty_like(b["X"]) for b in batches]
    fin = torch.empty((sh.batch, sh.nheads, sh.headdim, sh.dstate), dtype=torch.float32, device="cuda")
    X0 = batches[0]["X"]
    plan = ssd.fwd_plan(X0, batches[0]["B"], sh.chunk, with_units=True)
    nws = ssd.workspace_bytes(X0, batches[0]["B"], sh.chunk)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def step(i):
        g = batches[i % nbatch]
        ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], sh.chunk, Y=Ys[i % nbatch],
                           final_state=fin if sh.final_state else None, workspace=ws)

    settle_clocks()
    warm(step, warmup, warm_ms)
    t_step = time_events(step, steps) / steps

    # The step's launches one by one, in the configuration the step uses.
    # With one segment the step is the full pass itself (one launch).  With
    # several: the state-only pass over the segments, the segment scan, and
    # the full pass (the dominant kernel) fed entering states (their values
    # do not change the work).
    algo, seg_chunks, nseg, units = plan
    passes = {}
    t_kernel = None
    if algo == ssd.SSD_ALGO_MFMA and nseg == 1:
        t_kernel = t_step
        passes["full_pass_ms"] = t_step * 1e3
    elif algo == ssd.SSD_ALGO_MFMA:
        Bz, H, P, N = sh.batch, sh.nheads, sh.headdim, sh.dstate
        Sin = torch.zeros((Bz, nseg, H, P, N), dtype=torch.float32, device="cuda")

        def full(i):
            g = batches[i % nbatch]
            ssd.chunk_scan(g["X"], g["a"], g["B"], g["C"], sh.chunk, states_in=Sin,
                           seg_chunks=seg_chunks, Y=Ys[i % nbatch], wg_units=units)

        for i in range(warmup):
            full(i)
        t_kernel = time_events(full, steps) / steps
        passes["full_pass_ms"] = t_kernel * 1e3
        dS = torch.empty((Bz, nseg, H, P, N), dtype=torch.float32, device="cuda")
        lam_u = torch.zeros((Bz, H, nseg), dtype=torch.float32, device="cuda")

        def state(i):
            g = batches[i % nbatch]
            ssd.chunk_state(g["X"], g["a"], g["B"], sh.chunk, seg_chunks=seg_chunks, out=dS)

        def scan(i):
            ssd.state_passing(dS, lam_u, sh.chunk, sh.seqlen, out=Sin, return_final_state=False,
                              seg_chunks=seg_chunks)

        for fn, key in ((state, "state_pass_ms"), (scan, "segment_scan_ms")):
            for i in range(warmup):
                fn(i)
            passes[key] = time_events(fn, steps) / steps * 1e3
        del dS, lam_u, Sin
    del batches, Ys
    torch.cuda.empty_cache()
    return t_step, t_kernel, plan, passes


def n_batches(sh):
    """Distinct input batches to cycle: more than 2x the Infinity Cache."""
    return max(1, int(np.ceil(2 * 256e6 / fwd_algo_bytes(sh))))


def measure_forward(sh, steps, warmup, warm_ms=0.0):
    """One forward workload: step time, tokens/s, plan, passes, and the
    HBM / MFMA fractions of the step and of its full pass."""
    t_step, t_kernel, plan, passes = bench_forward(sh, steps, warmup, n_batches(sh), warm_ms=warm_ms)
    tok = sh.batch * sh.seqlen
    nbytes = fwd_algo_bytes(sh)
    fq = tok * fwd_algo_flops_per_token(sh, sh.chunk)
    f64 = tok * fwd_algo_flops_per_token(sh)
    return {"tokens_per_s": tok / t_step, "ms_per_step": t_step * 1e3,
            "plan": {"algo": plan[0], "seg_chunks": plan[1], "nseg": plan[2], "wg_units": plan[3]},
            "hbm_frac": nbytes / t_step / 1e9 / HBM_PEAK_GBS,
            "full_pass_hbm_frac": nbytes / t_kernel / 1e9 / HBM_PEAK_GBS if t_kernel else None,
            "mfma_frac": fq / t_step / 1e12 / BF16_PEAK_TFLOPS,
            "mfma_frac_blocks64": f64 / t_step / 1e12 / BF16_PEAK_TFLOPS,
            "algo_bytes": nbytes, "algo_flops": fq, "algo_flops_blocks64": f64,
            "passes": passes, "_t_kernel": t_kernel, "_t_step": t_step}


def bench_decode(steps, warmup):
    import torch
    import ssd_chunked_scan_chunk_amd as ssd
    import ssd_inputs as si
    sh = si.DECODE_CONFIG
    T = 16  # distinct per-step inputs, cycled (same bytes per step as fresh ones)
    d = si.make_decode(sh, seed=0, steps=T)
    state = torch.from_numpy(d["state"]).cuda()
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16)).view(torch.bfloat16).cuda()
    x, B, C = bf(d["x"]), bf(d["B"]), bf(d["C"])
    a = torch.from_numpy(d["a"]).cuda()
    y = torch.empty_like(x[0])

    def step(i):
        t = i % T
        ssd.step(state, x[t], a[t], B[t], C[t], y=y)

    Bz, H, P, N, G = sh.batch, sh.nheads, sh.headdim, sh.dstate, sh.ngroups
    nbytes = 2 * Bz * H * P * N * 4 + 2 * Bz * H * P * 2 + 2 * Bz * G * N * 2 + Bz * H * 4
    # The practical ceiling first (it also brings the GPU out of the idle
    # spell of the input generation): the library's plain in-place
    # read-modify-write of the same state array (scale 1, so the state keeps
    # its values), for each of its launch shapes.
    ceiling = {}
    settle_clocks()
    for per_thread in (1, 2, 4, 8):
        for nt in (False, True):
            def fn(i, v=per_thread, n=nt):
                ssd.stream_rmw(state, 1.0, v, n)
            for i in range(warmup):
                fn(i)
            tr = time_events(fn, steps) / steps
            ceiling["v%d%s" % (per_thread, "_nt" if nt else "")] = 2 * state.numel() * 4 / tr / 1e9
    # then the decode steps: a longer warm-up, and the timed steps in chunks
    # of 20 (their spread shows whether clocks were still settling)
    for i in range(max(warmup, 50)):
        step(i)
    chunks = [time_events(step, 20) / 20 for _ in range(max(1, steps // 20))]
    t = float(np.median(chunks))
    del state, x, B, C, a, y
    torch.cuda.empty_cache()
    ceiling["_chunks_us"] = [round(c * 1e6, 1) for c in chunks]
    return t, nbytes, ceiling


def decode_record(td, nbytes, ceiling):
    chunks = ceiling.pop("_chunks_us")
    best = max(ceiling.values())
    return {"workload": "batch 256, 80 heads, headdim 64, dstate 128, fp32 state in place",
            "us_per_step": td * 1e6, "GB_per_s": nbytes / td / 1e9,
            "hbm_frac": nbytes / td / 1e9 / HBM_PEAK_GBS, "tokens_per_s": 256 / td,
            "bytes_per_step": nbytes, "us_per_step_by_20_step_chunk": chunks,
            "stream_ceiling": {"GB_per_s": best, "hbm_frac": best / HBM_PEAK_GBS,
                               "decode_frac_of_ceiling": nbytes / td / 1e9 / best,
                               "kernel": "ssd_stream_rmw: in-place fp32 x *= 1 over the same state array",
                               "by_launch_shape_GB_per_s": ceiling}}


def bwd_algo_flops_per_token(sh, block=KERNEL_BLOCK):
    """MFMA flops per token of the backward as the library evaluates it: the
    time-reversed forward for dX (same flops as the forward), the dC and dB
    passes (the forward with headdim and state exchanged, the state split into
    64-wide sub-heads), the per-chunk states of the forward and of the reversed
    problem, and the da stage (per chunk Q: the lower triangle of 32x32 tiles
    of C B^T per group and of dY X^T per head, plus C S_in^T and B R^T)."""
    import dataclasses
    P, N, H, G, Q = sh.headdim, sh.dstate, sh.nheads, sh.ngroups, sh.chunk
    ns = N // 64
    swapped = dataclasses.replace(sh, nheads=H * ns, headdim=N // ns, dstate=P, ngroups=H)
    nI = Q // 32
    tiles = nI * (nI + 1) // 2
    da = (G * tiles * 32 * 32 * 2 * N + H * (tiles * 32 * 32 * 2 * P + 2 * 2 * Q * P * N)) / Q
    states = 2 * 2 * N * P * H   # chunk states of the forward and of the reversed problem
    return fwd_algo_flops_per_token(sh, block) + 2 * fwd_algo_flops_per_token(swapped, block) + da + states


def bench_backward(sh, steps, warmup, nbatch, seed0=100):
    """Time `steps` backward calls (all of dX, da, dB, dC, dS0) cycling over
    `nbatch` seeded batches with their upstream gradients."""
    import torch
    import ssd_chunked_scan_chunk_amd as ssd
    import ssd_inputs as si
    batches = []
    for i in range(nbatch):
        g = upload(si.make_fwd(sh, seed=seed0 + i, with_initial_state=True))
        d = si.make_fwd(sh, seed=seed0 + i, with_initial_state=True)
        g["S0"] = torch.from_numpy(d["S0"]).cuda()
        u = si.make_upstream_grads(sh, seed=seed0 + i)
        g["dY"] = torch.from_numpy(np.ascontiguousarray(u["dY"], dtype=np.uint16)).view(torch.bfloat16).cuda()
        g["dSf"] = torch.from_numpy(u["dS_fin"]).cuda()
        batches.append(g)
    g0 = batches[0]
    ws = torch.empty(max(1, ssd.bwd_workspace_bytes(g0["X"], g0["B"], sh.chunk)), dtype=torch.uint8,
                     device="cuda")

    def step(i):
        g = batches[i % nbatch]
        ssd.chunk_scan_bwd(g["X"], g["a"], g["B"], g["C"], g["dY"], sh.chunk, initial_state=g["S0"],
                           dfinal_state=g["dSf"], return_dinitial_state=True, workspace=ws)

    settle_clocks()
    warm(step, warmup, 30.0)
    t = time_events(step, steps) / steps

    # the dominant kernel (da) alone through its stage entry point, fed chunk
    # states of the right shape (their values do not change the work)
    nc = (sh.seqlen + sh.chunk - 1) // sh.chunk
    st_shape = (sh.batch, nc, sh.nheads, sh.headdim, sh.dstate)
    Sin = 0.1 * torch.randn(st_shape, device="cuda")
    Adj = 0.1 * torch.randn(st_shape, device="cuda")
    da = torch.empty_like(g0["a"])
    wsda = torch.empty(ssd.bwd_da_workspace_bytes(g0["X"], g0["B"], sh.chunk), dtype=torch.uint8, device="cuda")

    def da_step(i):
        g = batches[i % nbatch]
        ssd.bwd_da(g["X"], g["a"], g["B"], g["C"], g["dY"], sh.chunk, Sin, Adj, da=da, workspace=wsda)

    for i in range(warmup):
        da_step(i)
    t_da = time_events(da_step, steps) / steps
    del batches, ws, Sin, Adj, da, wsda
    torch.cuda.empty_cache()
    return t, t_da


def bwd_da_work(sh):
    """(MFMA flops, algorithmic HBM bytes) of one call of the da stage (the
    C B^T tile kernel and the da kernel): per chunk and group the
    lower-triangle 32x32 tiles of C B^T (K = N), per chunk and head those of
    dY X^T (K = P) plus C S_in^T and B R^T; X, dY, B, C, a and the two fp32
    chunk-state arrays in, da out."""
    P, N, H, G, Q = sh.headdim, sh.dstate, sh.nheads, sh.ngroups, sh.chunk
    nc = (sh.seqlen + Q - 1) // Q
    nI = Q // 32
    tiles = nI * (nI + 1) // 2
    flops = sh.batch * nc * (G * tiles * 32 * 32 * 2 * N + H * (tiles * 32 * 32 * 2 * P + 2 * 2 * Q * P * N))
    tok = sh.batch * sh.seqlen
    nbytes = tok * (2 * H * P * 2 + 2 * G * N * 2 + 2 * H * 4) + 2 * sh.batch * nc * H * P * N * 4
    return flops, nbytes


def cpu_baseline(sh):
    """The fp64 oracle (never tuned) on a bounded sample of the same workload,
    on the host cores: the first batch rows of the seeded batch, all heads,
    full length (heads and batch rows are independent, so this is the same
    per-token work), repeated until about 10 CPU-seconds are timed."""
    import oracle
    import ssd_inputs as si
    d = si.make_fwd(sh, seed=0)
    rows = max(1, min(sh.batch, 2))
    w = {k: si.widen(d[k][:rows], sh.dtype) for k in ("X", "B", "C")}
    a = d["a"][:rows].astype(np.float64)
    del d
    threads = min(16, os.cpu_count() or 1)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.fwd(w["X"], a, w["B"], w["C"], nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt * threads >= 10.0 or dt >= 30.0:
            break
    tokens = rows * sh.seqlen * reps
    # one thread on one batch row and a quarter of the heads
    hq = max(1, sh.nheads // 4)
    t1 = time.perf_counter()
    oracle.fwd(w["X"][:1, :, :hq], a[:1, :, :hq], w["B"][:1], w["C"][:1], nthreads=1)
    dt1 = time.perf_counter() - t1
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of the %d batch rows (%d heads, %d steps each), %d time(s), through the "
                      "sequential fp64 recurrence with (batch, head) slices spread over %d threads; "
                      "%.2f s wall" % (rows, sh.batch, sh.nheads, sh.seqlen, reps, threads, dt),
            "single_thread_value": sh.seqlen * hq / sh.nheads / dt1,
            "single_thread_sample": "one batch row, %d of %d heads, one thread (tokens/s scaled to all "
                                    "heads)" % (hq, sh.nheads),
            "cpu_model": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps before the timed ones; the default covers the ~25 ms the GPU clocks take to come up under this workload")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--workload", default="m2_2p7b",
                    help="forward workload of the headline: m2_2p7b (default), m2_130m, or "
                         "sweep<seqlen> (for profiling one workload alone)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time the decode step (batch 256, 80 heads; for profiling)")
    ap.add_argument("--bwd-only", action="store_true",
                    help="only time the backward of the 130M-shaped layer (for profiling)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 512 MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: there is no multi-GPU path (the layer would "
              "shard over (batch, head) with no exchange); run it with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE per dispatch of
        # this kernel, divided by 512 MiB, calibrates the HBM byte counters
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": 512 << 20, "copies": 5}))
        return
    import ssd_inputs as si
    import ssd_chunked_scan_chunk_amd as ssd  # noqa: F401  (fails loudly if libssd.so is missing)

    if args.decode_only:
        td, nbytes, ceil = bench_decode(args.steps, args.warmup)
        print(json.dumps({"decode_step": decode_record(td, nbytes, ceil)}))
        return
    s130 = si.FWD_CONFIGS["m2_130m"]
    if args.bwd_only:
        tokens = s130.batch * s130.seqlen
        tb, tda = bench_backward(s130, args.steps, args.warmup, 2)
        fl = tokens * bwd_algo_flops_per_token(s130)
        dfl, dby = bwd_da_work(s130)
        print(json.dumps({"backward_m2_130m": {"ms_per_step": tb * 1e3, "tokens_per_s": tokens / tb,
                                               "mfma_frac": fl / tb / 1e12 / BF16_PEAK_TFLOPS,
                                               "da_kernel_us": tda * 1e6,
                                               "da_mfma_frac": dfl / tda / 1e12 / BF16_PEAK_TFLOPS,
                                               "da_hbm_frac": dby / tda / 1e9 / HBM_PEAK_GBS}}))
        return

    wl = args.workload
    sh = si.sweep_shape(int(wl[5:])) if wl.startswith("sweep") else si.FWD_CONFIGS[wl]
    m = measure_forward(sh, args.steps, args.warmup)
    t_kernel = m.pop("_t_kernel")
    m.pop("_t_step")
    tokens = sh.batch * sh.seqlen
    algo_bytes = m["algo_bytes"]
    achieved = algo_bytes / t_kernel / 1e9 if t_kernel else None
    names = {"m2_2p7b": "m2_2p7b SSD layer fwd + final state: batch 8, seqlen 4096, 80 heads, headdim 64, "
                        "dstate 128, 1 group, chunk 256",
             "m2_130m": "m2_130m SSD layer fwd: batch 4, seqlen 2048, 24 heads, headdim 64, dstate 128, "
                        "1 group, chunk 256"}
    workload = names.get(wl, "state-64 sweep fwd: batch 1, seqlen %d, 32 heads, headdim 64, dstate 64, "
                             "1 group, chunk 256" % sh.seqlen)
    profile = {"m2_2p7b": "k_fwd_m2_2p7b_hbm_traffic.md",
               "m2_130m": "k_fwd_m2_130m_hbm_traffic.md"}.get(wl, "")
    out = {
        "metric": "SSD fwd tokens/s + MFMA% of bf16 peak at N=64/128; decode GB/s % of HBM peak",
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_ms": CLOCK_SETTLE_MS,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) X/B/C, a = dt*A per the workload's dt recipe; %d batch(es) cycled)"
                % n_batches(sh),
        "config": {"workload": workload, "plan": m["plan"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
                     "traffic": stored_traffic(profile) if profile else None,
                     "kernel": "k_fwd (fused pass)", "kernel_ms": t_kernel * 1e3 if t_kernel else None,
                     "algo_bytes_per_launch": algo_bytes},
        "passes": m["passes"],
        "mfma": {"achieved": m["algo_flops"] / (m["ms_per_step"] * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": m["mfma_frac"],
                 "flops_per_step": m["algo_flops"], "count": "algorithmic, at the caller's chunk",
                 "frac_blocks64": m["mfma_frac_blocks64"], "flops_per_step_blocks64": m["algo_flops_blocks64"]},
        "hbm_frac_step": m["hbm_frac"],
    }

    if not args.no_secondary:
        sec = {}
        if wl != "m2_130m":
            r = measure_forward(s130, args.steps, args.warmup, warm_ms=30.0)
            r.pop("_t_kernel"), r.pop("_t_step")
            sec["m2_130m"] = r
        for L in si.SWEEP_SEQLENS:
            shp = si.sweep_shape(L)
            r = measure_forward(shp, max(5, args.steps // (1 + L // 65536)), 2, warm_ms=30.0)
            r.pop("_t_kernel"), r.pop("_t_step")
            sec["sweep_n64_L%d" % L] = r
        # the fp32 path (the VALU kernel, exact segment sums, fp32 throughout)
        # on the 130M-shaped layer
        import dataclasses
        s130f = dataclasses.replace(s130, dtype=si.F32)
        r = measure_forward(s130f, max(5, args.steps // 5), 2, warm_ms=30.0)
        sec["m2_130m_fp32"] = {
            "workload": "the 130M-shaped layer with fp32 X, B, C (VALU kernel)",
            "ms_per_step": r["ms_per_step"], "tokens_per_s": r["tokens_per_s"], "plan": r["plan"],
            "hbm_frac": r["hbm_frac"], "algo_bytes": r["algo_bytes"],
            "valu_fp32": {"flops_per_step": r["algo_flops"],
                          "achieved": r["algo_flops"] / (r["ms_per_step"] * 1e-3) / 1e12,
                          "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": r["algo_flops"] / (r["ms_per_step"] * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS,
                          "count": "the chunked form's flops at the caller's chunk"}}
        td, nbytes, ceil = bench_decode(max(100, args.steps), 5)
        sec["decode_step"] = decode_record(td, nbytes, ceil)
        tokens130 = s130.batch * s130.seqlen
        tb, tda = bench_backward(s130, max(10, args.steps // 2), 3, 2)
        fl = tokens130 * bwd_algo_flops_per_token(s130)
        dfl, dby = bwd_da_work(s130)
        fwd130 = sec["m2_130m"]["ms_per_step"] if "m2_130m" in sec else m["ms_per_step"]
        sec["backward_m2_130m"] = {
            "workload": "gradients dX, da, dB, dC, d(initial state) of the 130M-shaped layer "
                        "for upstream dY and d(final state)",
            "ms_per_step": tb * 1e3, "tokens_per_s": tokens130 / tb, "bwd_over_fwd": tb * 1e3 / fwd130,
            "mfma_frac": fl / tb / 1e12 / BF16_PEAK_TFLOPS, "algo_flops_per_step": fl,
            # its dominant kernel, timed alone with HIP events
            "dominant_kernel": {"kernel": "k_bwd_da (with k_cb_tiles: the da stage)", "us": tda * 1e6,
                                "mfma": {"achieved": dfl / tda / 1e12, "peak": BF16_PEAK_TFLOPS,
                                         "unit": "TFLOP/s", "frac": dfl / tda / 1e12 / BF16_PEAK_TFLOPS},
                                "hbm": {"achieved": dby / tda / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": dby / tda / 1e9 / HBM_PEAK_GBS},
                                "algo_flops_per_launch": dfl, "algo_bytes_per_launch": dby}}
        out["secondary"] = sec

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(sh)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
