#!/usr/bin/env python3
"""Benchmark of the MI355X SSD layer (chunked forward + recurrent decode).

One step = one full forward (all four stages) of the Mamba-2 130M-shaped SSD
layer -- batch 4, seqlen 2048, 24 heads, headdim 64, state 128, 1 group,
chunk 256, bf16 X/B/C with fp32 a -- over one batch of seeded synthetic
inputs already resident in HBM.  Several distinct input batches are cycled so
that the working set of the timed loop (> 256 MB) does not sit in the 256 MB
Infinity Cache.

Prints ONE JSON line.  Besides the contract fields it carries:
  roofline      the dominant kernel (the MFMA full pass) against the HBM peak,
                from algorithmic bytes and that kernel's own launch duration,
                measured with HIP events on the launch stream (the pass is
                launched alone through the stage entry point, in the same
                segment configuration the step uses);
  passes        the step's three launches timed one by one the same way;
  mfma          MFMA flops of the step (the 64-step blocking the kernels run)
                against the bf16 dense peak;
  cpu_baseline  the fp64 CPU oracle on the same workload (host cores);
  secondary     the other workloads of the metric: the 2.7B-shaped layer,
                the state-64 sweep at seqlen 32K, the decode step's HBM
                bandwidth, and the backward of the 130M-shaped layer.
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


def fwd_algo_bytes_per_token(sh):
    """Minimum HBM bytes per token: X in, Y out, B and C, a (fp32)."""
    es = 2 if sh.dtype == "bf16" else 4
    return sh.nheads * sh.headdim * 2 * es + 2 * sh.ngroups * sh.dstate * es + 4 * sh.nheads


KERNEL_BLOCK = 64   # the fused kernels' block length (the output does not depend on it)


def fwd_algo_flops_per_token(sh, block=KERNEL_BLOCK):
    """MFMA flops per token of the blocked form with blocks of `block` steps:
    causal half of C B^T once per group, causal half of (L o S) X per head,
    block state and state-to-output per head."""
    Q, N, P, H, G = block, sh.dstate, sh.headdim, sh.nheads, sh.ngroups
    return (Q + 1) * (N * G + P * H) + 4 * N * P * H


def stored_traffic():
    """HBM bytes per launch of the full-pass kernel from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary (calibrated on a plain copy), or
    None when that summary was taken on a different kernel source."""
    import hashlib
    src = os.path.join(ROOT, "ssd_chunked_scan_chunk_amd", "csrc", "kernels_mfma.hip")
    prof = os.path.join(ROOT, "profiles", "k_mfma_seg_full_m2_130m_hbm_traffic.md")
    try:
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        fields = dict(l.split(":", 1) for l in open(prof) if l.startswith(("traffic_bytes", "kernel_source")))
    except OSError:
        return None
    if fields.get("kernel_source_sha256_16", "").strip() != sha:
        return None
    return int(fields["traffic_bytes_per_launch"])


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


def time_events(fn, steps):
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3  # seconds


def bench_forward(sh, steps, warmup, nbatch, seed0=0):
    """Time `steps` forwards cycling over `nbatch` seeded batches.
    Returns (seconds per step, seconds per launch of the full-pass kernel, plan)."""
    import torch
    import ssd_chunked_scan_chunk_amd as ssd
    import ssd_inputs as si
    batches = [upload(si.make_fwd(sh, seed=seed0 + i)) for i in range(nbatch)]
    Ys = [torch.empty_like(b["X"]) for b in batches]
    fin = torch.empty((sh.batch, sh.nheads, sh.headdim, sh.dstate), dtype=torch.float32, device="cuda")
    X0 = batches[0]["X"]
    plan = ssd.fwd_plan(X0, batches[0]["B"], sh.chunk)
    nws = ssd.workspace_bytes(X0, batches[0]["B"], sh.chunk)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def step(i):
        g = batches[i % nbatch]
        ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], sh.chunk, Y=Ys[i % nbatch],
                           final_state=fin if sh.final_state else None, workspace=ws)

    for i in range(warmup):
        step(i)
    t_step = time_events(step, steps) / steps

    # the step's launches one by one, in the configuration the step uses: the
    # state-only pass over the segments, the segment scan, and the full pass
    # (the dominant kernel) fed entering states (their values do not change
    # the work)
    algo, seg_chunks, nseg = plan
    passes = {}
    if algo == ssd.SSD_ALGO_MFMA:
        Bz, H, P, N = sh.batch, sh.nheads, sh.headdim, sh.dstate
        Sin = torch.zeros((Bz, nseg, H, P, N), dtype=torch.float32, device="cuda")

        def full(i):
            g = batches[i % nbatch]
            ssd.chunk_scan(g["X"], g["a"], g["B"], g["C"], sh.chunk, states_in=Sin,
                           seg_chunks=seg_chunks, Y=Ys[i % nbatch])

        for i in range(warmup):
            full(i)
        passes["full_pass_ms"] = time_events(full, steps) / steps * 1e3
        if nseg > 1:
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
            del dS, lam_u
        del Sin
    t_kernel = passes.get("full_pass_ms", 0.0) / 1e3 or None
    del batches, Ys
    torch.cuda.empty_cache()
    return t_step, t_kernel, plan, passes


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

    for i in range(warmup):
        step(i)
    t = time_events(step, steps) / steps
    Bz, H, P, N, G = sh.batch, sh.nheads, sh.headdim, sh.dstate, sh.ngroups
    nbytes = 2 * Bz * H * P * N * 4 + 2 * Bz * H * P * 2 + 2 * Bz * G * N * 2 + Bz * H * 4
    del state, x, B, C, a, y
    torch.cuda.empty_cache()
    return t, nbytes


def bwd_algo_flops_per_token(sh, block=KERNEL_BLOCK):
    """MFMA flops per token of the backward as the library evaluates it: the
    time-reversed forward for dX (same flops as the forward), the dC and dB
    passes (the forward with headdim and state exchanged, the state split into
    64-wide sub-heads), the per-chunk states of the forward and of the reversed
    problem, and the da kernel (per chunk Q: the lower triangle of 32x32 tiles
    of dY X^T and C B^T per head, plus C S_in^T and B R^T)."""
    import dataclasses
    P, N, H, Q = sh.headdim, sh.dstate, sh.nheads, sh.chunk
    ns = N // 64
    swapped = dataclasses.replace(sh, nheads=H * ns, headdim=N // ns, dstate=P, ngroups=H)
    nI = Q // 32
    da = H * ((nI * (nI + 1) // 2) * 32 * 32 * 2 * (P + N) + 2 * 2 * Q * P * N) / Q
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

    for i in range(warmup):
        step(i)
    t = time_events(step, steps) / steps

    # the dominant kernel (da) alone through its stage entry point, fed chunk
    # states of the right shape (their values do not change the work)
    nc = (sh.seqlen + sh.chunk - 1) // sh.chunk
    st_shape = (sh.batch, nc, sh.nheads, sh.headdim, sh.dstate)
    Sin = 0.1 * torch.randn(st_shape, device="cuda")
    Adj = 0.1 * torch.randn(st_shape, device="cuda")
    da = torch.empty_like(g0["a"])

    def da_step(i):
        g = batches[i % nbatch]
        ssd.bwd_da(g["X"], g["a"], g["B"], g["C"], g["dY"], sh.chunk, Sin, Adj, da=da)

    for i in range(warmup):
        da_step(i)
    t_da = time_events(da_step, steps) / steps
    del batches, ws, Sin, Adj, da
    torch.cuda.empty_cache()
    return t, t_da


def bwd_da_work(sh):
    """(MFMA flops, algorithmic HBM bytes) of one da-kernel launch: per chunk
    and head the lower-triangle 32x32 tiles of dY X^T (K = P) and C B^T (K = N)
    plus C S_in^T and B R^T; X, dY, B, C, a and the two fp32 chunk-state
    arrays in, da out."""
    P, N, H, G, Q = sh.headdim, sh.dstate, sh.nheads, sh.ngroups, sh.chunk
    nc = (sh.seqlen + Q - 1) // Q
    nI = Q // 32
    flops = sh.batch * nc * H * ((nI * (nI + 1) // 2) * 32 * 32 * 2 * (P + N) + 2 * 2 * Q * P * N)
    tok = sh.batch * sh.seqlen
    nbytes = tok * (2 * H * P * 2 + 2 * G * N * 2 + 2 * H * 4) + 2 * sh.batch * nc * H * P * N * 4
    return flops, nbytes


def cpu_baseline(sh):
    """The fp64 oracle (never tuned) on the same workload, on the host cores."""
    import oracle
    import ssd_inputs as si
    d = si.make_fwd(sh, seed=0)
    w = {k: si.widen(d[k], sh.dtype) for k in ("X", "B", "C")}
    a = d["a"].astype(np.float64)
    threads = os.cpu_count() or 1
    reps, t0 = 0, time.perf_counter()
    while True:   # repeat the batch until ~10 CPU-seconds of work are timed
        oracle.fwd(w["X"], a, w["B"], w["C"], nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt * threads >= 10.0 or dt >= 30.0:
            break
    tokens = sh.batch * sh.seqlen * reps
    # one thread on one batch row (a bounded sample of the same work)
    t1 = time.perf_counter()
    oracle.fwd(w["X"][:1], a[:1], w["B"][:1], w["C"][:1], nthreads=1)
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
            "sample": "the full %dx%d-token batch (%d heads), %d times, through the sequential "
                      "fp64 recurrence with (batch, head) slices spread over %d threads; %.2f s wall"
                      % (sh.batch, sh.seqlen, sh.nheads, reps, threads, dt),
            "single_thread_value": sh.seqlen / dt1, "single_thread_sample": "one batch row, one thread",
            "cpu_model": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
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

    sh = si.FWD_CONFIGS["m2_130m"]
    tokens = sh.batch * sh.seqlen
    if args.decode_only:
        td, nbytes = bench_decode(args.steps, args.warmup)
        print(json.dumps({"decode_step": {"us_per_step": td * 1e6, "GB_per_s": nbytes / td / 1e9,
                                          "hbm_frac": nbytes / td / 1e9 / HBM_PEAK_GBS,
                                          "bytes_per_step": nbytes}}))
        return
    if args.bwd_only:
        tb, tda = bench_backward(sh, args.steps, args.warmup, 2)
        fl = tokens * bwd_algo_flops_per_token(sh)
        dfl, dby = bwd_da_work(sh)
        print(json.dumps({"backward_m2_130m": {"ms_per_step": tb * 1e3, "tokens_per_s": tokens / tb,
                                               "mfma_frac": fl / tb / 1e12 / BF16_PEAK_TFLOPS,
                                               "da_kernel_us": tda * 1e6,
                                               "da_mfma_frac": dfl / tda / 1e12 / BF16_PEAK_TFLOPS,
                                               "da_hbm_frac": dby / tda / 1e9 / HBM_PEAK_GBS}}))
        return
    per_batch = tokens * fwd_algo_bytes_per_token(sh)
    nbatch = max(2, int(np.ceil(2 * 256e6 / per_batch)))   # > 2x the Infinity Cache
    t_step, t_kernel, plan, passes = bench_forward(sh, args.steps, args.warmup, nbatch)

    algo_bytes = tokens * fwd_algo_bytes_per_token(sh)
    algo_flops = tokens * fwd_algo_flops_per_token(sh)
    achieved = algo_bytes / t_kernel / 1e9 if t_kernel else None
    out = {
        "metric": "SSD fwd tokens/s + MFMA% of bf16 peak at N=64/128; decode GB/s % of HBM peak",
        "value": tokens / t_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) X/B/C, a = dt*A with Mamba-2 dt recipe; %d batches cycled)" % nbatch,
        "config": {"workload": "m2_130m SSD layer fwd: batch 4, seqlen 2048, 24 heads, headdim 64, "
                               "dstate 128, 1 group, chunk 256",
                   "plan": {"algo": plan[0], "seg_chunks": plan[1], "nseg": plan[2]}},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": (achieved / HBM_PEAK_GBS) if achieved else None, "traffic": stored_traffic(),
                     "kernel": "k_mfma_seg full pass", "kernel_ms": t_kernel * 1e3 if t_kernel else None,
                     "algo_bytes_per_launch": algo_bytes},
        "passes": passes,
        "mfma": {"achieved": algo_flops / t_step / 1e12, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": algo_flops / t_step / 1e12 / BF16_PEAK_TFLOPS,
                 "algo_flops_per_step": algo_flops},
    }

    if not args.no_secondary:
        sec = {}
        for name, shp in (("m2_2p7b", si.FWD_CONFIGS["m2_2p7b"]), ("sweep_n64_L32768", si.sweep_shape(32768))):
            tok = shp.batch * shp.seqlen
            nb = max(1, int(np.ceil(2 * 256e6 / (tok * fwd_algo_bytes_per_token(shp)))))
            ts, tk, pl, ps = bench_forward(shp, max(5, args.steps // 5), 2, nb)
            fl = tok * fwd_algo_flops_per_token(shp)
            sec[name] = {"tokens_per_s": tok / ts, "ms_per_step": ts * 1e3,
                         "hbm_frac": tok * fwd_algo_bytes_per_token(shp) / ts / 1e9 / HBM_PEAK_GBS,
                         "mfma_frac": fl / ts / 1e12 / BF16_PEAK_TFLOPS, "plan": list(pl),
                         "full_pass_hbm_frac": (tok * fwd_algo_bytes_per_token(shp) / tk / 1e9 / HBM_PEAK_GBS
                                                if tk else None), "passes": ps}
        td, nbytes = bench_decode(max(20, args.steps), 5)
        sec["decode_step"] = {"workload": "batch 256, 80 heads, headdim 64, dstate 128, fp32 state in place",
                              "us_per_step": td * 1e6, "GB_per_s": nbytes / td / 1e9,
                              "hbm_frac": nbytes / td / 1e9 / HBM_PEAK_GBS, "tokens_per_s": 256 / td}
        tb, tda = bench_backward(sh, max(10, args.steps // 2), 3, 2)
        fl = tokens * bwd_algo_flops_per_token(sh)
        dfl, dby = bwd_da_work(sh)
        sec["backward_m2_130m"] = {
            "workload": "gradients dX, da, dB, dC, d(initial state) of the 130M-shaped layer "
                        "for upstream dY and d(final state)",
            "ms_per_step": tb * 1e3, "tokens_per_s": tokens / tb, "bwd_over_fwd": tb / t_step,
            "mfma_frac": fl / tb / 1e12 / BF16_PEAK_TFLOPS, "algo_flops_per_step": fl,
            # its dominant kernel, timed alone with HIP events
            "dominant_kernel": {"kernel": "k_bwd_da", "us": tda * 1e6,
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
