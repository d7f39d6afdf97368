"""GPU parity of the full forward against the fp64 oracle.

Every case runs the HIP path through the C ABI (ssd_chunk_scan_fwd) and
compares with oracle.fwd on the same seeded inputs, in the slice-normwise
relative error (1e-5 for fp32 inputs, 2e-2 for bf16 inputs)."""
import numpy as np
import pytest
import torch

import oracle
import ssd_chunked_scan_chunk_amd as ssd
import ssd_inputs as si
from gpu_util import host_f64, log, oracle_threads, upload_fwd, widen_fwd
from parity import TOL, state_err, y_err

pytestmark = pytest.mark.gpu


def run_case(shape, seed=0, algo=ssd.SSD_ALGO_AUTO, seg_chunks=0, with_s0=False, tag=""):
    log("case %s %s algo=%d seg=%d s0=%s" % (tag, shape, algo, seg_chunks, with_s0))
    d = si.make_fwd(shape, seed=seed, with_initial_state=with_s0)
    g = upload_fwd(d)
    Y, S = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], shape.chunk,
                              initial_state=g.get("S0"), return_final_state=True,
                              algo=algo, seg_chunks=seg_chunks)
    torch.cuda.synchronize()
    w = widen_fwd(d)
    Yr, Sr = oracle.fwd(w["X"], w["a"], w["B"], w["C"], S0=w.get("S0"), nthreads=oracle_threads())
    ey, es = y_err(host_f64(Y), Yr), state_err(host_f64(S), Sr)
    log("   err Y=%.3e S=%.3e" % (ey, es))
    tol = TOL[shape.dtype]
    assert ey <= tol and es <= tol, (ey, es)
    return ey, es


def test_tiny_f32_workload():
    # batch 1, seqlen 256, 2 heads, P=N=16, chunk 64, fp32: the VALU path
    ey, es = run_case(si.FWD_CONFIGS["tiny_f32"], tag="tiny_f32")
    assert ey <= 1e-5


@pytest.mark.parametrize("Q,P,N", [(256, 64, 128), (256, 64, 64), (128, 64, 128), (64, 64, 64),
                                   (128, 32, 64), (128, 32, 128), (64, 32, 128)])
def test_mfma_shapes_ragged(Q, P, N):
    # several tiles plus a ragged tail; one workgroup walks all chunks
    L = 3 * Q + 37
    run_case(si.FwdShape(2, L, 3, P, N, 1, Q, si.BF16), seed=Q + P + N, algo=ssd.SSD_ALGO_MFMA,
             tag="mfma")


@pytest.mark.parametrize("H,P,N", [(7, 64, 128), (13, 32, 64), (5, 64, 64)])
def test_partial_head_sets(H, P, N):
    # heads split over several workgroups, the last one only partly filled
    run_case(si.FwdShape(2, 2 * 256 + 70, H, P, N, 1, 256, si.BF16), seed=H, algo=ssd.SSD_ALGO_MFMA,
             tag="heads")


@pytest.mark.parametrize("seg", [1, 2, 3])
def test_mfma_segmented_with_initial_state(seg):
    # segments of 1..3 chunks: state-only pass + segment scan + full pass
    run_case(si.FwdShape(2, 7 * 256 + 100, 4, 64, 128, 1, 256, si.BF16), seed=seg,
             algo=ssd.SSD_ALGO_MFMA, seg_chunks=seg, with_s0=True, tag="seg")


def test_segmented_many_workgroups():
    # 16 segments x 16 batches x 16 head sets: several rounds of workgroups per
    # launch, and a wide segment scan
    run_case(si.FwdShape(16, 1024, 48, 64, 128, 1, 64, si.BF16), seed=5, algo=ssd.SSD_ALGO_MFMA,
             seg_chunks=1, with_s0=True, tag="3-launch")


@pytest.mark.parametrize("H,P,N,G,Q,seg", [(8, 64, 128, 2, 128, 2), (12, 32, 128, 3, 64, 3),
                                             (7, 32, 64, 1, 256, 1)])
def test_segmented_groups_and_narrow_heads(H, P, N, G, Q, seg):
    # segmented plans with several B/C groups and with 32-wide heads (six heads
    # per workgroup, split between the copy waves' stage-1 work), ragged tail
    # and an initial state
    run_case(si.FwdShape(2, 4 * Q + 37, H, P, N, G, Q, si.BF16), seed=H + G, algo=ssd.SSD_ALGO_MFMA,
             seg_chunks=seg, with_s0=True, tag="seg-groups")


def test_groups_and_valu_bf16():
    # G=2 groups (heads 0-1 read group 0, 2-3 group 1), on both paths
    sh = si.FwdShape(1, 300, 4, 64, 64, 2, 64, si.BF16)
    run_case(sh, algo=ssd.SSD_ALGO_MFMA, tag="G2 mfma")
    run_case(sh, algo=ssd.SSD_ALGO_VALU, tag="G2 valu")
    run_case(si.FwdShape(1, 70, 2, 16, 16, 1, 32, si.BF16), tag="bf16 16x16 valu")


def test_chunk_size_invariance():
    # the same inputs through chunk 64, 128, 256 agree with each other
    d = si.make_fwd(si.FwdShape(1, 1000, 4, 64, 128, 1, 64, si.BF16), seed=5)
    g = upload_fwd(d)
    ys = []
    for Q in (64, 128, 256):
        Y, S = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], Q, return_final_state=True)
        ys.append((host_f64(Y), host_f64(S)))
    torch.cuda.synchronize()
    for Y, S in ys[1:]:
        assert y_err(Y, ys[0][0]) < 2e-2 and state_err(S, ys[0][1]) < 1e-2


def test_m2_130m_full():
    # batch 4, seqlen 2048, 24 heads, P=64, N=128, chunk 256 (full-size, all slices)
    run_case(si.FWD_CONFIGS["m2_130m"], tag="m2_130m")


@pytest.mark.parametrize("L", [512, 2048, 8192])
def test_sweep_n64_full(L):
    run_case(si.sweep_shape(L), tag="sweep")


def test_empty_and_degenerate():
    dev = "cuda"
    # seqlen 0: the final state is the initial state
    X = torch.zeros((2, 0, 3, 64), dtype=torch.bfloat16, device=dev)
    a = torch.zeros((2, 0, 3), dtype=torch.float32, device=dev)
    B = torch.zeros((2, 0, 1, 64), dtype=torch.bfloat16, device=dev)
    S0 = torch.randn((2, 3, 64, 64), device=dev)
    Y, S = ssd.chunk_scan_fwd(X, a, B, B.clone(), 256, initial_state=S0, return_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    _, S = ssd.chunk_scan_fwd(X, a, B, B.clone(), 256, return_final_state=True)
    assert not S.any()
    # batch 0 is a no-op
    ssd.chunk_scan_fwd(torch.zeros((0, 5, 3, 64), dtype=torch.bfloat16, device=dev),
                       torch.zeros((0, 5, 3), device=dev),
                       torch.zeros((0, 5, 1, 64), dtype=torch.bfloat16, device=dev),
                       torch.zeros((0, 5, 1, 64), dtype=torch.bfloat16, device=dev), 64)
    # single step and a sequence shorter than one chunk
    run_case(si.FwdShape(1, 1, 2, 64, 128, 1, 256, si.BF16), tag="L1")
    run_case(si.FwdShape(1, 5, 2, 16, 16, 1, 64, si.F32), tag="L5 f32")


def test_strong_decay_no_nan():
    # a = -1e4 everywhere: decays underflow to 0, masked entries must not turn into NaN
    d = si.make_fwd(si.FwdShape(1, 600, 2, 64, 128, 1, 256, si.BF16), seed=2)
    d["a"][:] = -1e4
    g = upload_fwd(d)
    Y, S = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], 256, return_final_state=True)
    torch.cuda.synchronize()
    w = widen_fwd(d)
    Yr, Sr = oracle.fwd(w["X"], w["a"], w["B"], w["C"])
    assert torch.isfinite(Y.float()).all()
    assert y_err(host_f64(Y), Yr) < 2e-2 and state_err(host_f64(S), Sr) < 2e-2


@pytest.mark.parametrize("seg", [0, 1])
def test_decay_regimes_per_head(seg):
    # One head per decay regime of the 64-step blocks (log2-decay per 16-step
    # quarter ~1.2, 69, 28, 138, growth, mixed per half, recipe, rare deep
    # drops), so the output and state scales are re-based at block starts and
    # at quarter boundaries, and the direct form runs for some blocks.
    sh = si.FwdShape(2, 64 * 12 + 17, 8, 64, 128, 1, 256, si.BF16)
    d = si.make_fwd(sh, seed=11)
    a = d["a"]
    rng = np.random.default_rng(5)
    a[:, :, 0] = -0.05
    a[:, :, 1] = -3.0
    a[:, :, 2] = -1.2
    a[:, :, 3] = -6.0
    a[:, :, 4] = 0.05
    halves = rng.choice(np.array([-0.01, -0.6, -1.2, -2.5, -3.5], dtype=np.float32),
                        size=(sh.batch, sh.seqlen // 32 + 1))
    a[:, :, 5] = np.repeat(halves, 32, axis=1)[:, :sh.seqlen]
    a[:, :, 7] = -0.02
    a[:, ::50, 7] = -100.0
    g = upload_fwd(d)
    Y, S = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], sh.chunk, return_final_state=True,
                              algo=ssd.SSD_ALGO_MFMA, seg_chunks=seg)
    torch.cuda.synchronize()
    w = widen_fwd(d)
    Yr, Sr = oracle.fwd(w["X"], w["a"], w["B"], w["C"], nthreads=oracle_threads())
    ey, es = y_err(host_f64(Y), Yr), state_err(host_f64(S), Sr)
    log("   decay regimes seg=%d err Y=%.3e S=%.3e" % (seg, ey, es))
    assert torch.isfinite(Y.float()).all()
    assert ey <= TOL[si.BF16] and es <= TOL[si.BF16], (ey, es)


def test_deep_rebase_keeps_the_state():
    # Per 64-step block of head 0, log2-decays per 16-step quarter of 100, 45,
    # then 15 near-free steps and one step of 178, then a mild quarter.  The
    # second quarter leaves the state's scale at its floor (2^-95 of the
    # output scale) and the third re-bases it by about 184 octaves: a factor
    # of 2^-184 would round to zero in fp32, yet the state still carries most
    # of the outputs of that quarter's first 15 steps.
    sh = si.FwdShape(1, 64 * 4 + 9, 2, 64, 128, 1, 256, si.BF16)
    d = si.make_fwd(sh, seed=13)
    ln2 = np.log(2.0)
    blk = np.concatenate([np.full(16, -100.0 / 16), np.full(16, -45.0 / 16),
                          np.full(15, -0.01), [-178.0 + 0.15], np.full(16, -0.3)]) * ln2
    d["a"][0, :, 0] = np.tile(blk, 5)[:sh.seqlen].astype(np.float32)
    g = upload_fwd(d)
    Y, S = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], sh.chunk, return_final_state=True,
                              algo=ssd.SSD_ALGO_MFMA)
    torch.cuda.synchronize()
    w = widen_fwd(d)
    Yr, Sr = oracle.fwd(w["X"], w["a"], w["B"], w["C"], nthreads=oracle_threads())
    ey, es = y_err(host_f64(Y), Yr), state_err(host_f64(S), Sr)
    log("   deep re-base err Y=%.3e S=%.3e" % (ey, es))
    assert ey <= TOL[si.BF16] and es <= TOL[si.BF16], (ey, es)


def test_nan_stays_in_its_slice():
    # a NaN in X[b=1, t=200, h=2] reaches only slice (1, 2).  Within that slice
    # it may also reach the steps of its own 32-step block of the chunk before
    # t=200 (the masked zeros of the blocked product meet it as 0 * NaN), but
    # never an earlier block.
    d = si.make_fwd(si.FwdShape(2, 512, 3, 64, 64, 1, 128, si.BF16), seed=3)
    g = upload_fwd(d)
    g["X"][1, 200, 2, 5] = float("nan")
    Y, S = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], 128, return_final_state=True)
    torch.cuda.synchronize()
    bad = torch.isnan(Y.float())
    assert bad[1, 200:, 2].any()
    assert not bad[1, :192, 2].any()
    bad[1, :, 2] = False
    assert not bad.any(), "NaN leaked into another (batch, head) slice"
    badS = torch.isnan(S)
    badS[1, 2] = False
    assert not badS.any()


def test_deterministic():
    d = si.make_fwd(si.FwdShape(2, 1500, 4, 64, 128, 1, 256, si.BF16), seed=4)
    g = upload_fwd(d)
    Y1, S1 = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], 256, return_final_state=True, seg_chunks=2)
    Y2, S2 = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], 256, return_final_state=True, seg_chunks=2)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(S1, S2)


@pytest.mark.parametrize("Q,P,N,G,seg", [(256, 64, 128, 1, 1), (128, 64, 64, 2, 0), (64, 32, 128, 1, 2),
                                         (128, 32, 64, 3, 1)])
def test_fwd_exact_decay_free(Q, P, N, G, seg):
    # zero decay and entries in {-1, 0, 1}: the scores, the states (below 256
    # here) and every fp32 sum are exact small integers, so Y must equal the
    # exact result rounded once to bf16 and the final state must be exact --
    # a check of every mask, tile, scale and index of the MFMA path
    H = 6 if G == 3 else 4
    sh = si.FwdShape(2, 3 * Q + 37, H, P, N, G, Q, si.BF16)
    log("exact fwd %s seg=%d" % (sh, seg))
    d = si.make_integer_grads_case(sh, seed=41 + Q + P)
    g = upload_fwd(d)
    Y, S = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], Q, initial_state=g["S0"],
                              return_final_state=True, algo=ssd.SSD_ALGO_MFMA, seg_chunks=seg)
    torch.cuda.synchronize()
    w = widen_fwd(d)
    Yr, Sr = oracle.fwd(w["X"], w["a"], w["B"], w["C"], S0=w["S0"])
    assert np.abs(Sr).max() < 256
    Yr_bf16 = si.widen(si.f32_to_bf16_bits(Yr.astype(np.float32)), si.BF16)
    log("   max |Y| %.0f, max |S| %.0f" % (np.abs(Yr).max(), np.abs(Sr).max()))
    assert np.array_equal(host_f64(Y), Yr_bf16)
    assert np.array_equal(host_f64(S), Sr)


def test_fwd_workspace_contents_ignored():
    # segmented plan (its workspace holds segment states; slot 0 is neither
    # written nor read): a workspace of NaN bytes gives the same Y and state
    sh = si.FwdShape(2, 4 * 256 + 37, 6, 64, 128, 1, 256, si.BF16)
    d = si.make_fwd(sh, seed=91, with_initial_state=True)
    g = upload_fwd(d)
    n = ssd.workspace_bytes(g["X"], g["B"], sh.chunk, seg_chunks=1)
    assert n > 0
    outs = []
    for fill in (0, 0xFF):
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
        outs.append(ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], sh.chunk, initial_state=g["S0"],
                                       return_final_state=True, seg_chunks=1, workspace=ws))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.isfinite(outs[1][0].float()).all()
