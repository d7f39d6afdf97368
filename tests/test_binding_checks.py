"""The torch binding checks every tensor against the call's sizes before the
C ABI sees a pointer: a wrong shape or dtype raises ValueError naming the
tensor.  CPU tensors suffice (shape and dtype are checked before the device),
so nothing here launches a kernel."""
import pytest
import torch

import ssd_chunked_scan_chunk_amd as ssd

Bz, L, H, P, G, N = 2, 40, 4, 64, 1, 128


def fwd_inputs(dtype=torch.bfloat16):
    X = torch.zeros((Bz, L, H, P), dtype=dtype)
    a = torch.zeros((Bz, L, H), dtype=torch.float32)
    B = torch.zeros((Bz, L, G, N), dtype=dtype)
    C = torch.zeros((Bz, L, G, N), dtype=dtype)
    return X, a, B, C


def state(*lead):
    return torch.zeros(lead + (P, N), dtype=torch.float32)


@pytest.mark.parametrize("which,bad,match", [
    ("a", torch.zeros((Bz, L - 1, H)), "a has shape"),
    ("a", torch.zeros((Bz, L, H), dtype=torch.bfloat16), "a has dtype"),
    ("B", torch.zeros((Bz + 1, L, G, N), dtype=torch.bfloat16), "B has shape"),
    ("B", torch.zeros((Bz, L, G, N), dtype=torch.float32), "B has dtype"),
    ("C", torch.zeros((Bz, L, G, N - 8), dtype=torch.bfloat16), "C has shape"),
    ("C", torch.zeros((Bz, L, G, N), dtype=torch.float16), "C has dtype"),
])
def test_fwd_inputs_checked(which, bad, match):
    X, a, B, C = fwd_inputs()
    args = {"X": X, "a": a, "B": B, "C": C}
    args[which] = bad
    with pytest.raises(ValueError, match=match):
        ssd.chunk_scan_fwd(args["X"], args["a"], args["B"], args["C"], 64)


@pytest.mark.parametrize("kw,bad,match", [
    ("initial_state", state(Bz, H - 1), "initial_state has shape"),
    ("initial_state", state(Bz, H).double(), "initial_state has dtype"),
    ("Y", torch.zeros((Bz, L, H, P - 32), dtype=torch.bfloat16), "Y has shape"),
    ("Y", torch.zeros((Bz, L, H, P), dtype=torch.float32), "Y has dtype"),
    ("final_state", state(Bz, H)[:, :, :, :64].contiguous(), "final_state has shape"),
])
def test_fwd_outputs_checked(kw, bad, match):
    X, a, B, C = fwd_inputs()
    with pytest.raises(ValueError, match=match):
        ssd.chunk_scan_fwd(X, a, B, C, 64, **{kw: bad})


def test_fwd_workspace_size_checked():
    X, a, B, C = fwd_inputs()
    X, a, B, C = (torch.cat([t] * 5, dim=1) for t in (X, a, B, C))   # 200 steps: four chunks
    need = ssd.workspace_bytes(X, B, 64, seg_chunks=1)
    assert need > 0
    ws = torch.zeros(need - 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="workspace holds"):
        ssd.chunk_scan_fwd(X, a, B, C, 64, seg_chunks=1, workspace=ws)


def test_fwd_rank_checked():
    X, a, B, C = fwd_inputs()
    with pytest.raises(ValueError, match="4-D"):
        ssd.chunk_scan_fwd(X[0], a, B, C, 64)


@pytest.mark.parametrize("kw,bad,match", [
    ("dY", torch.zeros((Bz, L, H, P), dtype=torch.float32), "dY has dtype"),
    ("dY", torch.zeros((Bz, L + 1, H, P), dtype=torch.bfloat16), "dY has shape"),
    ("dfinal_state", state(Bz, H + 1), "dfinal_state has shape"),
])
def test_bwd_checked(kw, bad, match):
    X, a, B, C = fwd_inputs()
    args = {"dY": torch.zeros_like(X), "dfinal_state": None}
    args[kw] = bad
    with pytest.raises(ValueError, match=match):
        ssd.chunk_scan_bwd(X, a, B, C, args["dY"], 64, dfinal_state=args["dfinal_state"])


def test_bwd_da_states_checked():
    X, a, B, C = fwd_inputs()
    nc = (L + 63) // 64
    good = state(Bz, nc, H)
    with pytest.raises(ValueError, match="adjoint_in has shape"):
        ssd.bwd_da(X, a, B, C, torch.zeros_like(X), 64, good, state(Bz, nc + 1, H))
    with pytest.raises(ValueError, match="da has dtype"):
        ssd.bwd_da(X, a, B, C, torch.zeros_like(X), 64, good, good, da=torch.zeros_like(a).double())


@pytest.mark.parametrize("which,bad,match", [
    ("a", torch.zeros((3, H + 1)), "a has shape"),
    ("B", torch.zeros((3, G, N), dtype=torch.float32), "B has dtype"),
    ("C", torch.zeros((3, G, N + 8), dtype=torch.bfloat16), "C has shape"),
    ("x", torch.zeros((3, H, P - 1), dtype=torch.bfloat16), "x has shape"),
    ("y", torch.zeros((3, H, P), dtype=torch.float32), "y has dtype"),
    ("state", state(3, H).half(), "state has dtype"),
])
def test_step_checked(which, bad, match):
    args = {"state": state(3, H), "x": torch.zeros((3, H, P), dtype=torch.bfloat16),
            "a": torch.zeros((3, H)), "B": torch.zeros((3, G, N), dtype=torch.bfloat16),
            "C": torch.zeros((3, G, N), dtype=torch.bfloat16), "y": None}
    args[which] = bad
    with pytest.raises(ValueError, match=match):
        ssd.step(args["state"], args["x"], args["a"], args["B"], args["C"], y=args["y"])


def test_stage_entry_points_checked():
    X, a, B, C = fwd_inputs()
    with pytest.raises(ValueError, match="out has shape"):
        ssd.chunk_state(X, a, B, 64, seg_chunks=1, out=state(Bz, 2, H))      # 40 steps: one unit
    with pytest.raises(ValueError, match="states_in has shape"):
        ssd.chunk_scan(X, a, B, C, 64, states_in=state(Bz, 3, H))
    dS = state(Bz, 1, H)
    with pytest.raises(ValueError, match="units"):
        ssd.state_passing(dS, torch.zeros((Bz, H, 1)), 16, L)             # 40 steps of 16: three units
    with pytest.raises(ValueError, match="lam has shape"):
        ssd.state_passing(dS, torch.zeros((Bz, H, 2)), 64, L)
    with pytest.raises(ValueError, match="a has dtype"):
        ssd.chunk_cumsum(torch.zeros((Bz, L, H), dtype=torch.float64), 64)
