"""GPU parity of the recurrent decode step (ssd_step) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import ssd_chunked_scan_chunk_amd as ssd
import ssd_inputs as si
from gpu_util import dev_tensor, host_f64, log, upload_fwd, widen_fwd
from parity import slice_rel_err, y_err

pytestmark = pytest.mark.gpu


def upload_decode(d):
    dt = d["shape"].dtype
    return {"state": dev_tensor(d["state"], si.F32), "x": dev_tensor(d["x"], dt),
            "a": dev_tensor(d["a"], si.F32), "B": dev_tensor(d["B"], dt), "C": dev_tensor(d["C"], dt)}


def run_steps(shape, steps, sample_b, seed=0):
    d = si.make_decode(shape, seed=seed, steps=steps)
    g = upload_decode(d)
    T = steps
    ys = []
    for t in range(T):
        y = ssd.step(g["state"], g["x"][t], g["a"][t], g["B"][t], g["C"][t])
        ys.append(y[sample_b].clone())
    torch.cuda.synchronize()
    dt = shape.dtype
    st = d["state"][sample_b].astype(np.float64)
    worst = 0.0
    for t in range(T):
        st, yr = oracle.step(st, si.widen(d["x"][t][sample_b], dt), d["a"][t][sample_b],
                             si.widen(d["B"][t][sample_b], dt), si.widen(d["C"][t][sample_b], dt))
        worst = max(worst, slice_rel_err(host_f64(ys[t]), yr, (0, 1)))
    es = slice_rel_err(host_f64(g["state"][sample_b]), st, (0, 1))
    return worst, es


@pytest.mark.parametrize("P,N,dtype", [(64, 128, si.BF16), (64, 64, si.BF16), (64, 128, si.F32),
                                       (24, 40, si.BF16)])
def test_step_small(P, N, dtype):
    log("step small %d %d %s" % (P, N, dtype))
    sh = si.StepShape(3, 8, P, N, 2 if N == 128 else 1, dtype, 40)
    ey, es = run_steps(sh, 40, np.arange(3))
    tol = 1e-5 if dtype == si.F32 else 2e-2
    assert ey < tol and es < 1e-5, (ey, es)


def test_decode_workload_1024_steps():
    # batch 256, 80 heads, P=64, N=128, 1024 consecutive in-place steps;
    # every step's y and the final state checked on sampled batch rows
    log("decode workload 1024 steps")
    sample = np.array([0, 97, 255])
    ey, es = run_steps(si.DECODE_CONFIG, 1024, sample)
    log("   err y=%.3e state=%.3e" % (ey, es))
    assert ey < 2e-2 and es < 1e-5


def test_decode_equals_forward():
    # L steps from the zero state reproduce the chunked forward
    log("decode == forward")
    sh = si.FwdShape(2, 300, 4, 64, 128, 1, 128, si.BF16)
    d = si.make_fwd(sh, seed=9)
    g = upload_fwd(d)
    Yf, Sf = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], sh.chunk, return_final_state=True)
    state = torch.zeros((2, 4, 64, 128), device="cuda")
    ys = []
    for t in range(sh.seqlen):
        ys.append(ssd.step(state, g["X"][:, t].contiguous(), g["a"][:, t].contiguous(),
                           g["B"][:, t].contiguous(), g["C"][:, t].contiguous()))
    Ys = torch.stack(ys, dim=1)
    torch.cuda.synchronize()
    w = widen_fwd(d)
    Yr, Sr = oracle.fwd(w["X"], w["a"], w["B"], w["C"])
    assert y_err(host_f64(Ys), Yr) < 2e-2
    assert slice_rel_err(host_f64(state), Sr, (0, 1)) < 1e-5
    assert y_err(host_f64(Ys), host_f64(Yf)) < 2e-2
    assert slice_rel_err(host_f64(state), host_f64(Sf), (0, 1)) < 2e-2


def test_step_deterministic_and_resumable():
    log("decode determinism")
    d = si.make_decode(si.StepShape(4, 8, 64, 128, 1, si.BF16, 20), seed=3, steps=20)
    g1 = upload_decode(d)
    g2 = upload_decode(d)
    snap = None
    for t in range(20):
        y1 = ssd.step(g1["state"], g1["x"][t], g1["a"][t], g1["B"][t], g1["C"][t])
        y2 = ssd.step(g2["state"], g2["x"][t], g2["a"][t], g2["B"][t], g2["C"][t])
        if t == 9:
            snap = g1["state"].clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(g1["state"], g2["state"])
    # resume from the snapshot taken after step 9: bitwise the same continuation
    st = snap
    for t in range(10, 20):
        y3 = ssd.step(st, g1["x"][t], g1["a"][t], g1["B"][t], g1["C"][t])
    torch.cuda.synchronize()
    assert torch.equal(st, g1["state"]) and torch.equal(y3, y1)


def test_decode_exact_decay_free():
    # a = 0 and ternary x, B, C with an integer state: every step's update is an
    # exact small-integer fp32 sum, so the state is exact and y is the exact
    # value rounded once to bf16
    import ssd_inputs as si
    rng = np.random.default_rng(51)
    Bz, H, P, N, G, T = 3, 4, 64, 128, 2, 20
    tern = lambda *sz: rng.integers(-1, 2, size=sz).astype(np.float32)
    st = rng.integers(-3, 4, size=(Bz, H, P, N)).astype(np.float32)
    state = torch.from_numpy(st).cuda()
    ref = st.astype(np.float64)
    for t in range(T):
        x, B, C = tern(Bz, H, P), tern(Bz, G, N), tern(Bz, G, N)
        a = np.zeros((Bz, H), np.float32)
        bf = lambda v: torch.from_numpy(si.f32_to_bf16_bits(v)).view(torch.bfloat16).cuda()
        y = ssd.step(state, bf(x), torch.from_numpy(a).cuda(), bf(B), bf(C))
        ref, yr = oracle.step(ref, x.astype(np.float64), a.astype(np.float64), B.astype(np.float64),
                              C.astype(np.float64))
        torch.cuda.synchronize()
        yr_bf16 = si.widen(si.f32_to_bf16_bits(yr.astype(np.float32)), si.BF16)
        assert np.array_equal(y.float().cpu().numpy().astype(np.float64), yr_bf16), t
    assert np.array_equal(state.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("dtype,seg", [(si.BF16, 0), (si.BF16, 1), (si.F32, 0)])
def test_prefill_then_decode_handoff(dtype, seg):
    # constant-memory inference: a chunked forward over the first L1 steps
    # (ragged last chunk; seg=1 forces one chunk per segment, so the final
    # state comes out of the segmented plan) hands its final state to ssd_step,
    # which continues in place for L2 steps; outputs and the state after L1+L2
    # steps must match the oracle run over the whole sequence
    Bz, H, P, N, G, Q, L1, L2 = 3, 8, 64, 128, 2, 256, 700, 40
    log("prefill->decode %s seg=%d" % (dtype, seg))
    sh = si.FwdShape(Bz, L1 + L2, H, P, N, G, Q, dtype)
    d = si.make_fwd(sh, seed=23)
    g = upload_fwd(d)
    Yp, state = ssd.chunk_scan_fwd(g["X"][:, :L1].contiguous(), g["a"][:, :L1].contiguous(),
                                   g["B"][:, :L1].contiguous(), g["C"][:, :L1].contiguous(), Q,
                                   return_final_state=True, seg_chunks=seg)
    ys = []
    for t in range(L1, L1 + L2):
        ys.append(ssd.step(state, g["X"][:, t].contiguous(), g["a"][:, t].contiguous(),
                           g["B"][:, t].contiguous(), g["C"][:, t].contiguous()))
    Yd = torch.stack(ys, dim=1)
    torch.cuda.synchronize()
    w = widen_fwd(d)
    Yr, Sr = oracle.fwd(w["X"], w["a"], w["B"], w["C"])
    tol = 1e-5 if dtype == si.F32 else 2e-2
    ep, ed = y_err(host_f64(Yp), Yr[:, :L1]), y_err(host_f64(Yd), Yr[:, L1:])
    es = slice_rel_err(host_f64(state), Sr, (0, 1))
    log("   err prefill Y=%.3e decode y=%.3e state=%.3e" % (ep, ed, es))
    assert ep < tol and ed < tol and es < tol, (ep, ed, es)


@pytest.mark.parametrize("n,per_thread,nt", [(4, 8, True), (4 * 1000 + 4, 1, False), (1 << 20, 8, True),
                                             (1 << 20, 2, False), (3 * 256 * 4 * 4 + 12, 4, True)])
def test_stream_rmw_exact(n, per_thread, nt):
    # the ceiling kernel multiplies every element exactly once (ragged tails
    # included) and touches nothing past n
    g = torch.Generator().manual_seed(n)
    base = torch.randn(n + 64, generator=g, dtype=torch.float32)
    t = base.cuda()
    ssd.stream_rmw(t[:n], 0.75, per_thread, nt)
    torch.cuda.synchronize()
    got = t.cpu()
    assert torch.equal(got[:n], base[:n] * 0.75)
    assert torch.equal(got[n:], base[n:])

