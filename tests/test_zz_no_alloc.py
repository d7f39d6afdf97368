"""The allocation-free forward entry point (ssd_chunk_scan_fwd_noalloc)
against ssd_chunk_scan_fwd, through the C ABI, on two calls in a row -- the
second with a smaller input -- both of which use the library's per-GPU
device array for the segment states."""
import numpy as np
import pytest
import torch

import ssd_chunked_scan_chunk_amd as ssd
import ssd_inputs as si
from gpu_util import host_f64, log, upload_fwd
from parity import TOL, state_err, y_err

pytestmark = pytest.mark.gpu


def run_pair(sh, seed, seg):
    d = si.make_fwd(sh, seed=seed, with_initial_state=True)
    g = upload_fwd(d)
    plan = ssd.fwd_plan(g["X"], g["B"], sh.chunk, seg_chunks=seg)
    Yr, Sr = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], sh.chunk, initial_state=g["S0"],
                                return_final_state=True, seg_chunks=seg)
    Y = torch.full_like(g["X"], float("nan"))
    S = torch.full_like(Sr, float("nan"))
    ssd.chunk_scan_fwd_noalloc(g["X"], g["a"], g["B"], g["C"], sh.chunk, initial_state=g["S0"], Y=Y,
                               final_state=S, seg_chunks=seg)
    torch.cuda.synchronize()
    return plan, Y, S, Yr, Sr


def test_noalloc_two_calls_second_smaller():
    # first call: several segments (the fixed device array holds their states);
    # second call: a smaller input that leaves stale states of the first in the
    # array, which must not be read
    cases = [(si.FwdShape(3, 2000, 12, 64, 128, 2, 256, si.BF16), 41, 1),
             (si.FwdShape(2, 700, 6, 64, 64, 1, 128, si.BF16), 42, 2)]
    for sh, seed, seg in cases:
        log("noalloc %s seg=%d" % (sh, seg))
        plan, Y, S, Yr, Sr = run_pair(sh, seed, seg)
        assert plan[2] > 1, plan                       # the scratch is really used
        ey, es = y_err(host_f64(Y), host_f64(Yr)), state_err(host_f64(S), host_f64(Sr))
        log("   plan %s  vs allocating entry point: Y %.3e  S %.3e" % (plan, ey, es))
        # same plan, same kernels: the results agree to the bit, so certainly
        # to the bf16 tolerance
        assert ey <= TOL["bf16"] and es <= TOL["bf16"]
        assert torch.equal(Y, Yr) and torch.equal(S, Sr)


def test_noalloc_rejects_a_pinned_plan_beyond_the_array():
    # 64 x 24 heads x 16 segments of 32 KiB states = 768 MiB > 64 MiB: rejected
    # on the host (nothing enqueued, Y untouched); the automatic plan fits
    sh = si.FwdShape(64, 4096, 24, 64, 128, 1, 256, si.BF16)
    X = torch.zeros((sh.batch, sh.seqlen, sh.nheads, sh.headdim), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((sh.batch, sh.seqlen, sh.nheads), dtype=torch.float32, device="cuda")
    B = torch.zeros((sh.batch, sh.seqlen, 1, sh.dstate), dtype=torch.bfloat16, device="cuda")
    Y = torch.full_like(X, 7.0)
    with pytest.raises(ssd.SSDError, match="SSD_ERR_WORKSPACE"):
        ssd.chunk_scan_fwd_noalloc(X, a, B, B.clone(), sh.chunk, Y=Y, seg_chunks=1)
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())
