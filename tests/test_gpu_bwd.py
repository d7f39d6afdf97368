"""GPU parity of the backward against the fp64 adjoint of the recurrence.

Every case runs ssd_chunk_scan_bwd through the C ABI and compares dX, da, dB,
dC and the initial-state gradient with oracle.bwd on the same seeded inputs
and upstream gradients, in the slice-normwise relative error (2e-2 for bf16
inputs with fp32 accumulation; the outputs dX, dB, dC are bf16)."""
import numpy as np
import pytest
import torch

import oracle
import ssd_chunked_scan_chunk_amd as ssd
import ssd_inputs as si
from gpu_util import dev_tensor, host_f64, log, upload_fwd, widen_fwd
from parity import TOL, slice_rel_err, state_err, y_err

pytestmark = pytest.mark.gpu


def bwd_case(shape, seed=0, with_s0=True, with_dsf=True, want_ds0=True, tag=""):
    log("bwd case %s %s s0=%s dsf=%s" % (tag, shape, with_s0, with_dsf))
    d = si.make_fwd(shape, seed=seed, with_initial_state=with_s0)
    u = si.make_upstream_grads(shape, seed=seed)
    g = upload_fwd(d)
    dY = dev_tensor(u["dY"], shape.dtype)
    dSf = dev_tensor(u["dS_fin"], si.F32) if with_dsf else None
    out = ssd.chunk_scan_bwd(g["X"], g["a"], g["B"], g["C"], dY, shape.chunk,
                             initial_state=g.get("S0"), dfinal_state=dSf,
                             return_dinitial_state=want_ds0)
    torch.cuda.synchronize()
    w = widen_fwd(d)
    ref = oracle.bwd(w["X"], w["a"], w["B"], w["C"], si.widen(u["dY"], shape.dtype),
                     S0=w.get("S0"), dS_fin=u["dS_fin"].astype(np.float64) if with_dsf else None)
    errs = {"dX": y_err(host_f64(out["dX"]), ref["dX"]),
            "da": slice_rel_err(host_f64(out["da"]), ref["da"], (0, 2)),
            "dB": slice_rel_err(host_f64(out["dB"]), ref["dB"], (0, 2)),
            "dC": slice_rel_err(host_f64(out["dC"]), ref["dC"], (0, 2))}
    if want_ds0:
        errs["dS0"] = state_err(host_f64(out["dinitial_state"]), ref["dS0"])
    log("   " + " ".join("%s=%.3e" % kv for kv in errs.items()))
    tol = TOL[shape.dtype]
    assert all(v <= tol for v in errs.values()), errs
    return out


@pytest.mark.parametrize("Q,P,N,H,G", [(256, 64, 128, 4, 1), (128, 64, 64, 4, 2), (64, 64, 128, 6, 3),
                                       (128, 32, 64, 3, 1), (64, 32, 128, 2, 2)])
def test_bwd_shapes_ragged(Q, P, N, H, G):
    # several chunks plus a ragged tail, grouped B/C, initial state and dS_fin
    bwd_case(si.FwdShape(2, 3 * Q + 37, H, P, N, G, Q, si.BF16), seed=Q + P + N + G, tag="shapes")


@pytest.mark.parametrize("Q,P,N,H,G", [(256, 64, 128, 4, 1), (128, 64, 64, 4, 2), (64, 64, 128, 6, 3),
                                       (128, 32, 64, 3, 1)])
def test_bwd_shapes_whole_chunks(Q, P, N, H, G):
    # a whole number of chunks: the reversed problem needs no padding and the
    # headdim-64 plans read (and write) it in place, with the reversed step 0
    # taking no decay; headdim 32 still copies it out
    bwd_case(si.FwdShape(2, 3 * Q, H, P, N, G, Q, si.BF16), seed=Q + P + N + G + 1, tag="whole-chunks")


def test_bwd_without_states():
    # no initial state and no final-state gradient; L a whole number of chunks
    bwd_case(si.FwdShape(2, 512, 4, 64, 128, 1, 128, si.BF16), seed=5, with_s0=False,
             with_dsf=False, tag="no-states")


def test_bwd_single_short_chunk():
    bwd_case(si.FwdShape(3, 45, 2, 64, 64, 1, 256, si.BF16), seed=6, tag="short")


def test_bwd_weak_decay_long():
    # the 130M value recipe (slow decays: the states carry far) over 8 chunks
    bwd_case(si.FwdShape(1, 2048, 4, 64, 128, 1, 256, si.BF16, dt_recipe="mamba2_dt"), seed=7,
             tag="weak-decay")


def test_bwd_empty_sequence():
    sh = si.FwdShape(2, 0, 4, 64, 128, 1, 256, si.BF16)
    X = torch.empty((2, 0, 4, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((2, 0, 1, 128), dtype=torch.bfloat16, device="cuda")
    a = torch.empty((2, 0, 4), dtype=torch.float32, device="cuda")
    dSf = torch.randn((2, 4, 64, 128), device="cuda")
    out = ssd.chunk_scan_bwd(X, a, B, B.clone(), X.clone(), sh.chunk, dfinal_state=dSf,
                             return_dinitial_state=True)
    torch.cuda.synchronize()
    assert torch.equal(out["dinitial_state"], dSf)


def test_bwd_deterministic():
    sh = si.FwdShape(2, 600, 4, 64, 128, 1, 256, si.BF16)
    d = si.make_fwd(sh, seed=8, with_initial_state=True)
    u = si.make_upstream_grads(sh, seed=8)
    g = upload_fwd(d)
    dY = dev_tensor(u["dY"], sh.dtype)
    dSf = dev_tensor(u["dS_fin"], si.F32)
    r1 = ssd.chunk_scan_bwd(g["X"], g["a"], g["B"], g["C"], dY, 256, g["S0"], dSf, True)
    r2 = ssd.chunk_scan_bwd(g["X"], g["a"], g["B"], g["C"], dY, 256, g["S0"], dSf, True)
    torch.cuda.synchronize()
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k


def test_bwd_m2_130m_shape():
    # the Mamba-2 130M layer shape at batch 2 (the oracle's adjoint at full batch takes longer)
    sh = si.FWD_CONFIGS["m2_130m"]
    bwd_case(si.FwdShape(2, sh.seqlen, sh.nheads, sh.headdim, sh.dstate, sh.ngroups, sh.chunk,
                         sh.dtype, dt_recipe=sh.dt_recipe), seed=9, tag="m2-130m")


def test_bwd_m2_2p7b_row():
    # one batch row of the Mamba-2 2.7B layer shape (80 heads sharing one
    # group, 16 chunks), all gradients against the full oracle adjoint
    sh = si.FWD_CONFIGS["m2_2p7b"]
    bwd_case(si.FwdShape(1, sh.seqlen, sh.nheads, sh.headdim, sh.dstate, sh.ngroups, sh.chunk,
                         sh.dtype), seed=11, tag="m2-2p7b-row")


def test_bwd_long_many_chunks():
    # 64 chunks of 64 steps with a ragged tail: the reversed sequence's padding,
    # the chunk-state scans over many units and the per-chunk adjoint slots
    bwd_case(si.FwdShape(1, 64 * 64 - 21, 3, 64, 64, 1, 64, si.BF16, dt_recipe="mamba2_dt"),
             seed=12, tag="many-chunks")


def _chunk_states_and_adjoints(w, dY, dSf, Q):
    """fp64 states entering each chunk and the adjoint dl/dS at the first step
    of each next chunk (dS_fin for the last), by the recurrence and its adjoint
    written out step by step (small shapes only)."""
    X, a, B, C, S0 = w["X"], w["a"], w["B"], w["C"], w.get("S0")
    Bz, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    nc = (L + Q - 1) // Q
    Sin = np.zeros((Bz, nc, H, P, N))
    Adj = np.zeros((Bz, nc, H, P, N))
    for b in range(Bz):
        for h in range(H):
            g = h * G // H
            s = S0[b, h].copy() if S0 is not None else np.zeros((P, N))
            for t in range(L):
                if t % Q == 0:
                    Sin[b, t // Q, h] = s
                s = np.exp(a[b, t, h]) * s + np.outer(X[b, t, h], B[b, t, g])
            gst = dSf[b, h].copy()
            for t in range(L - 1, -1, -1):
                gst = np.outer(dY[b, t, h], C[b, t, g]) + (np.exp(a[b, t + 1, h]) * gst if t + 1 < L else gst)
                if t % Q == 0 and t > 0:
                    Adj[b, t // Q - 1, h] = gst
            Adj[b, nc - 1, h] = dSf[b, h]
    return Sin, Adj


@pytest.mark.parametrize("Q,P,N", [(64, 64, 128), (128, 32, 64)])
def test_bwd_da_stage(Q, P, N):
    # the da kernel on its own, fed exact chunk states, against the oracle's da
    sh = si.FwdShape(2, 2 * Q + 29, 3, P, N, 1, Q, si.BF16)
    log("da stage %s" % (sh,))
    d = si.make_fwd(sh, seed=21, with_initial_state=True)
    u = si.make_upstream_grads(sh, seed=21)
    w = widen_fwd(d)
    dY = si.widen(u["dY"], sh.dtype)
    dSf = u["dS_fin"].astype(np.float64)
    Sin, Adj = _chunk_states_and_adjoints(w, dY, dSf, Q)
    g = upload_fwd(d)
    da = ssd.bwd_da(g["X"], g["a"], g["B"], g["C"], dev_tensor(u["dY"], sh.dtype), Q,
                    torch.from_numpy(Sin.astype(np.float32)).cuda(),
                    torch.from_numpy(Adj.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    ref = oracle.bwd(w["X"], w["a"], w["B"], w["C"], dY, S0=w["S0"], dS_fin=dSf)
    e = slice_rel_err(host_f64(da), ref["da"], (0, 2))
    log("   err da=%.3e" % e)
    assert e <= TOL[sh.dtype], e


def _integer_case(sh, seed):
    d = si.make_integer_grads_case(sh, seed=seed)
    w = widen_fwd(d)
    dY = si.widen(d["dY"], sh.dtype)
    dSf = d["dS_fin"].astype(np.float64)
    ref = oracle.bwd(w["X"], w["a"], w["B"], w["C"], dY, S0=w["S0"], dS_fin=dSf)
    return d, w, dY, dSf, ref


@pytest.mark.parametrize("Q,P,N", [(64, 64, 128), (128, 32, 64)])
def test_bwd_da_stage_exact(Q, P, N):
    # zero decay and entries in {-1, 0, 1}: every product and sum in the da
    # kernel is an exact small integer (the states stay below 256 in magnitude,
    # so their bf16 operands are exact too), so da must equal the oracle's
    # exactly -- a check of every mask, tile and index of the kernel
    sh = si.FwdShape(2, 2 * Q + 29, 3, P, N, 1, Q, si.BF16)
    log("exact da stage %s" % (sh,))
    d, w, dY, dSf, ref = _integer_case(sh, 31)
    Sin, Adj = _chunk_states_and_adjoints(w, dY, dSf, Q)
    assert np.abs(Sin).max() < 256 and np.abs(Adj).max() < 256
    g = upload_fwd(d)
    da = ssd.bwd_da(g["X"], g["a"], g["B"], g["C"], dev_tensor(d["dY"], sh.dtype), Q,
                    torch.from_numpy(Sin.astype(np.float32)).cuda(),
                    torch.from_numpy(Adj.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    got = host_f64(da)
    log("   max |da| %.0f, max abs error %.3g" % (np.abs(ref["da"]).max(), np.abs(got - ref["da"]).max()))
    assert np.array_equal(got, ref["da"])


@pytest.mark.parametrize("G", [2, 4])
def test_bwd_exact_decay_free(G):
    # the whole backward on the same kind of inputs.  Its states and adjoints
    # stay below 256, so every bf16 operand inside is exact and every sum an
    # exact integer: da and the initial-state gradient must be exact, dX, dB
    # and dC the exact values rounded once to bf16 (dB and dC sum the heads'
    # fp32 contributions before that rounding)
    sh = si.FwdShape(2, 3 * 64 + 17, 4, 64, 128, G, 64, si.BF16)
    log("exact backward %s" % (sh,))
    d, w, dY, dSf, ref = _integer_case(sh, 33)
    g = upload_fwd(d)
    out = ssd.chunk_scan_bwd(g["X"], g["a"], g["B"], g["C"], dev_tensor(d["dY"], sh.dtype), sh.chunk,
                             initial_state=g["S0"], dfinal_state=dev_tensor(d["dS_fin"], si.F32),
                             return_dinitial_state=True)
    torch.cuda.synchronize()
    bf = lambda v: si.widen(si.f32_to_bf16_bits(v.astype(np.float32)), si.BF16)
    log("   max |da| %.0f, max |dX| %.0f" % (np.abs(ref["da"]).max(), np.abs(ref["dX"]).max()))
    assert np.array_equal(host_f64(out["da"]), ref["da"])
    assert np.array_equal(host_f64(out["dinitial_state"]), ref["dS0"])
    assert np.array_equal(host_f64(out["dX"]), bf(ref["dX"]))
    for k in ("dB", "dC"):
        assert np.array_equal(host_f64(out[k]), bf(ref[k])), k


@pytest.mark.parametrize("with_s0,with_dsf", [(True, False), (False, True)])
def test_bwd_one_group_per_head(with_s0, with_dsf):
    # G = H: each head reads its own B and C (the exchanged-dimension passes
    # then read B / C per head); initial state and final-state gradient each
    # present without the other
    bwd_case(si.FwdShape(2, 2 * 128 + 45, 4, 64, 128, 4, 128, si.BF16), seed=13 + with_s0,
             with_s0=with_s0, with_dsf=with_dsf, tag="G=H")


@pytest.mark.parametrize("shape", [si.FWD_CONFIGS["tiny_f32"],
                                   si.FwdShape(2, 3 * 64 + 37, 4, 32, 32, 2, 64, si.F32),
                                   si.FwdShape(1, 2 * 128 + 5, 2, 16, 64, 1, 128, si.F32)],
                         ids=["tiny_f32", "ragged_G2", "Q128"])
def test_bwd_f32(shape):
    # the fp32 backward (VALU kernels throughout) at the fp32 tolerance
    bwd_case(shape, seed=61, tag="f32")


@pytest.mark.parametrize("L,dtype", [(1, si.BF16), (1, si.F32), (65, si.BF16), (65, si.F32)])
def test_bwd_one_step_tails(L, dtype):
    # a single step, and a last chunk of one step: the reversed sequence is
    # then almost all padding
    P, N = (64, 64) if dtype == si.BF16 else (16, 32)
    bwd_case(si.FwdShape(2, L, 3, P, N, 1, 64, dtype), seed=70 + L, tag="tail")


@pytest.mark.parametrize("dtype", [si.BF16, si.F32])
def test_bwd_workspace_contents_ignored(dtype):
    # a workspace full of NaN bytes gives bit-for-bit the gradients of a zeroed
    # one: no pass reads a workspace region it has not written
    P, N = (64, 128) if dtype == si.BF16 else (16, 32)
    sh = si.FwdShape(2, 2 * 64 + 19, 3, P, N, 1, 64, dtype)
    d = si.make_fwd(sh, seed=81, with_initial_state=True)
    u = si.make_upstream_grads(sh, seed=81)
    g = upload_fwd(d)
    dY = dev_tensor(u["dY"], dtype)
    dSf = dev_tensor(u["dS_fin"], si.F32)
    n = ssd.bwd_workspace_bytes(g["X"], g["B"], sh.chunk)
    outs = []
    for fill in (0, 0xFF):
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
        outs.append(ssd.chunk_scan_bwd(g["X"], g["a"], g["B"], g["C"], dY, sh.chunk, g["S0"], dSf, True,
                                       workspace=ws))
    torch.cuda.synchronize()
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k]), k
        assert torch.isfinite(outs[1][k].float()).all(), k
