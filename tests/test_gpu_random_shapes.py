"""Seeded random shapes through the forward and the backward (bf16, MFMA
path) against the fp64 oracle: a spread of batch sizes, sequence lengths
(ragged, shorter than a chunk, a single step), head counts not divisible by
the heads per workgroup, group counts, head dims, state sizes and chunks, with
and without the initial state and the final-state gradient."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import ssd_chunked_scan_chunk_amd as ssd
import ssd_inputs as si
from gpu_util import dev_tensor, host_f64, log, oracle_threads, upload_fwd, widen_fwd
from parity import TOL, slice_rel_err, state_err, y_err

pytestmark = pytest.mark.gpu


def _shapes(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        G = int(rng.choice([1, 2, 3]))
        H = G * int(rng.integers(1, 5))
        P = int(rng.choice([32, 64]))
        N = int(rng.choice([64, 128]))
        Q = int(rng.choice([64, 128, 256]))
        kind = rng.choice(3, p=[0.15, 0.35, 0.5])
        L = 1 if kind == 0 else int(rng.integers(2, Q)) if kind == 1 else int(rng.integers(Q, 4 * Q))
        Bz = int(rng.integers(1, 4))
        out.append((si.FwdShape(Bz, L, H, P, N, G, Q, si.BF16), bool(rng.integers(0, 2)),
                    bool(rng.integers(0, 2)), 100 + k))
    return out


@pytest.mark.parametrize("shape,with_s0,with_dsf,seed", _shapes(),
                         ids=lambda v: str(v) if not isinstance(v, si.FwdShape) else
                         "B%dL%dH%dP%dN%dG%dQ%d" % (v.batch, v.seqlen, v.nheads, v.headdim, v.dstate,
                                                    v.ngroups, v.chunk))
def test_random_shape_fwd_bwd(shape, with_s0, with_dsf, seed):
    log("random %s s0=%s dsf=%s" % (shape, with_s0, with_dsf))
    d = si.make_fwd(shape, seed=seed, with_initial_state=with_s0)
    u = si.make_upstream_grads(shape, seed=seed)
    g = upload_fwd(d)
    w = widen_fwd(d)
    tol = TOL[shape.dtype]
    Y, S = ssd.chunk_scan_fwd(g["X"], g["a"], g["B"], g["C"], shape.chunk, initial_state=g.get("S0"),
                              return_final_state=True)
    dSf = dev_tensor(u["dS_fin"], si.F32) if with_dsf else None
    gr = ssd.chunk_scan_bwd(g["X"], g["a"], g["B"], g["C"], dev_tensor(u["dY"], shape.dtype), shape.chunk,
                            initial_state=g.get("S0"), dfinal_state=dSf, return_dinitial_state=True)
    torch.cuda.synchronize()
    Yr, Sr = oracle.fwd(w["X"], w["a"], w["B"], w["C"], S0=w.get("S0"), nthreads=oracle_threads())
    ref = oracle.bwd(w["X"], w["a"], w["B"], w["C"], si.widen(u["dY"], shape.dtype), S0=w.get("S0"),
                     dS_fin=u["dS_fin"].astype(np.float64) if with_dsf else None)
    errs = {"Y": y_err(host_f64(Y), Yr), "S": state_err(host_f64(S), Sr),
            "dX": y_err(host_f64(gr["dX"]), ref["dX"]),
            "da": slice_rel_err(host_f64(gr["da"]), ref["da"], (0, 2)),
            "dB": slice_rel_err(host_f64(gr["dB"]), ref["dB"], (0, 2)),
            "dC": slice_rel_err(host_f64(gr["dC"]), ref["dC"], (0, 2)),
            "dS0": state_err(host_f64(gr["dinitial_state"]), ref["dS0"])}
    log("   " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    assert all(v <= tol for v in errs.values()), errs


def _weak_decay_shapes(n=8, seed=99):
    # the same spread with Mamba-2's dt recipe: weak decay, long memory, large states
    return [(dataclasses.replace(sh, dt_recipe="mamba2_dt"), s0, dsf, sd) for (sh, s0, dsf, sd) in _shapes(n, seed)]


@pytest.mark.parametrize("shape,with_s0,with_dsf,seed", _weak_decay_shapes(),
                         ids=lambda v: str(v) if not isinstance(v, si.FwdShape) else
                         "B%dL%dH%dP%dN%dG%dQ%d" % (v.batch, v.seqlen, v.nheads, v.headdim, v.dstate,
                                                    v.ngroups, v.chunk))
def test_random_shape_fwd_bwd_weak_decay(shape, with_s0, with_dsf, seed):
    test_random_shape_fwd_bwd(shape, with_s0, with_dsf, seed)


def _f32_shapes(n=8, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        G = int(rng.choice([1, 2]))
        H = G * int(rng.integers(1, 4))
        P = int(rng.choice([8, 16, 32]))
        N = int(rng.choice([16, 32, 64]))
        Q = int(rng.choice([32, 64, 128]))
        L = int(rng.integers(1, 3 * Q))
        Bz = int(rng.integers(1, 3))
        out.append((si.FwdShape(Bz, L, H, P, N, G, Q, si.F32), bool(rng.integers(0, 2)),
                    bool(rng.integers(0, 2)), 900 + k))
    return out


@pytest.mark.parametrize("shape,with_s0,with_dsf,seed", _f32_shapes(),
                         ids=lambda v: str(v) if not isinstance(v, si.FwdShape) else
                         "B%dL%dH%dP%dN%dG%dQ%d" % (v.batch, v.seqlen, v.nheads, v.headdim, v.dstate,
                                                    v.ngroups, v.chunk))
def test_random_shape_fwd_bwd_f32(shape, with_s0, with_dsf, seed):
    # the same on fp32 inputs (VALU kernels) at the fp32 tolerance
    test_random_shape_fwd_bwd(shape, with_s0, with_dsf, seed)


@pytest.mark.parametrize("shape,with_s0,with_dsf,seed", [
    (si.FwdShape(2, 1, 12, 64, 128, 3, 256, si.BF16), True, False, 120),
    (si.FwdShape(3, 1, 9, 64, 64, 3, 256, si.BF16), True, False, 132),
    (si.FwdShape(2, 1, 2, 64, 128, 1, 256, si.BF16), True, True, 156),
], ids=["G3x4", "G3x3", "G1x2_dsf"])
def test_one_step_group_cancellation(shape, with_s0, with_dsf, seed):
    # regression: at one step the group sums of dB and dC are a sum over heads
    # of x.dy times one row, which can nearly cancel (x.dy of -2.01, -7.61 and
    # 10.15 in one of these groups): the heads' contributions are summed in
    # fp32 before rounding, and each head's own score and state terms must keep
    # more than bf16's 8 bits, or their rounding dominates the cancelled sum
    test_random_shape_fwd_bwd(shape, with_s0, with_dsf, seed)
