"""GPU parity at the full benchmark sizes, in the launch configuration that
bench.py times (the library's own plan), on sampled (batch, head) slices.

Heads are independent: the oracle run on a few heads alone (their X and a,
with their group's B and C) gives exactly those slices' outputs and final
states, so full-length slices are checked without running the oracle over
the whole layer.  Tolerance as everywhere for bf16 inputs: slice-normwise
relative error <= 2e-2."""
import numpy as np
import pytest
import torch

import oracle
import ssd_chunked_scan_chunk_amd as ssd
import ssd_inputs as si
from gpu_util import log, oracle_threads, upload_fwd
from parity import TOL, chunk_rel_err, elementwise_diag, state_err, y_err

pytestmark = pytest.mark.gpu


def check_sampled(sh, seed, picks):
    """picks: {batch index: [heads]}; all picked heads of one call share a group."""
    log("full-size %s seed=%d" % (sh, seed))
    d = si.make_fwd(sh, seed=seed)
    g = upload_fwd(d)
    plan = ssd.fwd_plan(g["X"], g["B"], sh.chunk)
    Y, S = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], sh.chunk, return_final_state=True)
    torch.cuda.synchronize()
    log("   plan %s" % (plan,))
    H, G = sh.nheads, sh.ngroups
    worst = 0.0
    for b, heads in picks.items():
        for grp in sorted({h * G // H for h in heads}):
            hs = [h for h in heads if h * G // H == grp]
            X = si.widen(d["X"][b:b + 1, :, hs], sh.dtype)
            a = d["a"][b:b + 1, :, hs].astype(np.float64)
            B = si.widen(d["B"][b:b + 1, :, grp:grp + 1], sh.dtype)
            C = si.widen(d["C"][b:b + 1, :, grp:grp + 1], sh.dtype)
            Yr, Sr = oracle.fwd(X, a, B, C, nthreads=min(len(hs), oracle_threads()))
            idx = torch.tensor(hs, device="cuda")
            Yg = Y[b:b + 1].index_select(2, idx).to(torch.float64).cpu().numpy()
            Sg = S[b:b + 1].index_select(1, idx).to(torch.float64).cpu().numpy()
            ey, es = y_err(Yg, Yr), state_err(Sg, Sr)
            # each chunk normalised by its own magnitude (bounded like the
            # slice metric), and the elementwise relative error over entries
            # >= 1e-3 of the slice maximum (logged only: unbounded near zero)
            ec = chunk_rel_err(Yg, Yr, sh.chunk)
            ee = elementwise_diag(Yg, Yr, (0, 2))
            log("   b=%d heads=%s err Y=%.3e S=%.3e per-chunk Y=%.3e elementwise(>=1e-3 max)=%.3e"
                % (b, hs, ey, es, ec, ee))
            assert np.isfinite(Yg).all()
            assert ey <= TOL[sh.dtype] and es <= TOL[sh.dtype], (b, hs, ey, es)
            assert ec <= TOL[sh.dtype], (b, hs, ec)
            worst = max(worst, ey, es, ec)
    return worst


def test_m2_2p7b_sampled():
    # batch 8, seqlen 4096, 80 heads, P=64, N=128: first and last head sets
    # (the last partly filled), a middle one, first and last batch rows
    sh = si.FWD_CONFIGS["m2_2p7b"]
    check_sampled(sh, 0, {0: [0, 1, 2, 40, 78, 79], 7: [3, 41, 77, 79], 4: [23, 57]})


def test_sweep_n64_512k_sampled():
    # the longest N=64 sweep point: batch 1, seqlen 524288, 32 heads, P=N=64
    sh = si.sweep_shape(524288)
    check_sampled(sh, 0, {0: [0, 17, 31]})


@pytest.mark.parametrize("L", [32768, 131072])
def test_sweep_n64_long_sampled(L):
    # the remaining N=64 sweep points (their segment plans differ from the
    # shorter ones checked in full): first, a middle and the last head
    check_sampled(si.sweep_shape(L), 0, {0: [0, 15, 31]})
