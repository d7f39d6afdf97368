"""Per-stage GPU parity: each stage entry point against the matching
intermediate of the oracle's fp64 chunked form (cs, chunk totals, chunk
states, entering states, intra-chunk output, full output)."""
import numpy as np
import pytest
import torch

import oracle
import ssd_chunked_scan_chunk_amd as ssd
import ssd_inputs as si
from gpu_util import dev_tensor, host_f64, log, upload_fwd, widen_fwd
from parity import slice_rel_err, y_err

pytestmark = pytest.mark.gpu

SHAPE = si.FwdShape(2, 5 * 128 + 77, 3, 64, 128, 1, 128, si.BF16)


@pytest.fixture(scope="module")
def case():
    d = si.make_fwd(SHAPE, seed=21)
    w = widen_fwd(d)
    ref = oracle.chunked_fwd(w["X"], w["a"], w["B"], w["C"], SHAPE.chunk)
    return d, upload_fwd(d), ref


def test_stage1_cumsum(case):
    d, g, ref = case
    log("stage1 cumsum")
    cs, lam = ssd.chunk_cumsum(g["a"], SHAPE.chunk)
    torch.cuda.synchronize()
    cs, lam = host_f64(cs), host_f64(lam)
    # fp32 wavefront scan of up to Q terms: error bounded by ~log2(Q) roundings of |partial sums|
    bound = 8 * np.finfo(np.float32).eps * np.abs(ref["cs"]).max() * np.log2(SHAPE.chunk)
    assert np.abs(cs - ref["cs"]).max() <= bound
    assert np.abs(lam - ref["lam"]).max() <= bound
    # the entries past the ragged end are zero, the chunk total is the last entry
    Lc = SHAPE.seqlen % SHAPE.chunk
    assert not cs[:, :, -1, Lc:].any()


def test_stage3_chunk_state(case):
    d, g, ref = case
    log("stage3 chunk_state")
    dS = host_f64(ssd.chunk_state(g["X"], g["a"], g["B"], SHAPE.chunk))
    torch.cuda.synchronize()
    assert slice_rel_err(dS, ref["dS"], (0, 1, 2)) < 2e-2


def test_stage4_state_passing(case):
    d, g, ref = case
    log("stage4 state_passing")
    dS = torch.from_numpy(ref["dS"].astype(np.float32)).cuda()
    lam = torch.from_numpy(ref["lam"].astype(np.float32)).cuda()
    Sin, fin = ssd.state_passing(dS, lam, SHAPE.chunk, SHAPE.seqlen)
    torch.cuda.synchronize()
    # fp32 arithmetic on fp32-rounded inputs: well inside 1e-5
    assert slice_rel_err(host_f64(Sin), ref["S_in"], (0, 1, 2)) < 1e-5
    assert slice_rel_err(host_f64(fin), ref["S_fin"], (0, 1)) < 1e-5
    # in place
    Sin2, _ = ssd.state_passing(dS, lam, SHAPE.chunk, SHAPE.seqlen, out=dS)
    torch.cuda.synchronize()
    assert torch.equal(Sin2, Sin)


def test_stage2_intra_chunk_only(case):
    d, g, ref = case
    log("stage2 chunk_scan zero states")
    Y = ssd.chunk_scan(g["X"], g["a"], g["B"], g["C"], SHAPE.chunk)
    torch.cuda.synchronize()
    assert y_err(host_f64(Y), ref["Ydiag"]) < 2e-2


def test_stage5_with_states(case):
    d, g, ref = case
    log("stage2+5 chunk_scan with states")
    Sin = torch.from_numpy(ref["S_in"].astype(np.float32)).cuda()
    Y = ssd.chunk_scan(g["X"], g["a"], g["B"], g["C"], SHAPE.chunk, states_in=Sin)
    torch.cuda.synchronize()
    assert y_err(host_f64(Y), ref["Y"]) < 2e-2


def test_stages_compose_to_forward(case):
    d, g, ref = case
    log("stages compose")
    dS = ssd.chunk_state(g["X"], g["a"], g["B"], SHAPE.chunk)
    _, lam = ssd.chunk_cumsum(g["a"], SHAPE.chunk)
    Sin, fin = ssd.state_passing(dS, lam, SHAPE.chunk, SHAPE.seqlen)
    Y = ssd.chunk_scan(g["X"], g["a"], g["B"], g["C"], SHAPE.chunk, states_in=Sin)
    torch.cuda.synchronize()
    assert y_err(host_f64(Y), ref["Y"]) < 2e-2
    assert slice_rel_err(host_f64(fin), ref["S_fin"], (0, 1)) < 2e-2


@pytest.mark.parametrize("k", [2, 4])
def test_stages_in_units_of_several_chunks(case, k):
    """Stages 3-5 on units of k chunks (the full forward's segments; the last
    unit is shorter): unit states from the oracle's chunk states, and the
    composed output."""
    d, g, ref = case
    log("stages in units of %d chunks" % k)
    nc = ref["dS"].shape[1]
    nu = (nc + k - 1) // k
    dS = ssd.chunk_state(g["X"], g["a"], g["B"], SHAPE.chunk, seg_chunks=k)
    assert dS.shape[1] == nu
    # the unit state is the chunk states combined by the chunk decays (fp64)
    lam_c = ref["lam"]                              # [b][h][c]
    want = np.zeros_like(ref["dS"][:, :nu])
    for u in range(nu):
        for c in range(u * k, min(nc, (u + 1) * k)):
            dec = np.exp(lam_c[:, :, c])[:, :, None, None]
            want[:, u] = want[:, u] * dec + ref["dS"][:, c]
    torch.cuda.synchronize()
    assert slice_rel_err(host_f64(dS), want, (0, 1, 2)) < 2e-2
    # unit totals, summed from the per-chunk ones; the scan and the output
    _, lam = ssd.chunk_cumsum(g["a"], SHAPE.chunk)
    pad = nu * k - nc
    lam_u = torch.nn.functional.pad(lam, (0, pad)).view(lam.shape[0], lam.shape[1], nu, k).sum(-1).contiguous()
    Sin, fin = ssd.state_passing(dS, lam_u, SHAPE.chunk, SHAPE.seqlen, seg_chunks=k)
    Y = ssd.chunk_scan(g["X"], g["a"], g["B"], g["C"], SHAPE.chunk, states_in=Sin, seg_chunks=k)
    torch.cuda.synchronize()
    assert slice_rel_err(host_f64(Sin), ref["S_in"][:, ::k], (0, 1, 2)) < 2e-2
    assert y_err(host_f64(Y), ref["Y"]) < 2e-2
    assert slice_rel_err(host_f64(fin), ref["S_fin"], (0, 1)) < 2e-2
