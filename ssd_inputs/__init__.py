"""Seeded synthetic inputs for the SSD layer.

This module is shared by the tests, the benchmark and the smoke check.  It
holds only input generation (random draws, dtype rounding, the named
workloads); none of the layer's arithmetic lives here, and it imports neither
the oracle nor the HIP library.

Value recipe (the pages describe the layer's inputs only as input-dependent,
time-varying SSM parameters -- Mamba digest, lryc.cn page, section "Selective
State Space Models"; wiki review, "Core concepts" -- so the distributions are
synthetic stand-ins):

* X, B, C ~ N(0, 1), drawn in float32, stored as float32 or rounded to
  bfloat16 (round to nearest even) for bf16 workloads.
* Per-head rate A_h = -exp(u_h), u_h ~ U(0, ln 16), fixed for the head.
* Step size dt = softplus(z - 2), z ~ N(0, 1) i.i.d. per (batch, step, head)
  ("standard" recipe), or the "mamba2_dt" recipe: a per-head bias chosen so
  that softplus(bias_h) = dt0_h with dt0_h log-uniform in [1e-3, 0.1], then
  dt = clamp(softplus(z + bias_h), 1e-3, 0.1).
* a = dt * A_h, computed in float64 and stored float32.
* Decode state cache ~ N(0, 0.1^2) in float32.

The generator is numpy's PCG64 (``default_rng(seed)``); draws happen in a fixed
order (A, dt noise, X, B, C, then the state cache).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32, BF16 = "f32", "bf16"


# ---------------------------------------------------------------------------
# bfloat16 helpers (host side, numpy): storage is uint16 bit patterns.
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even; returns uint16 bit patterns.
    NaN stays NaN (quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    r = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(u) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def widen(arr, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored input (float32 or bf16 bits)."""
    if dtype == BF16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == BF16 else np.ascontiguousarray(x32, np.float32)


def _softplus(z):
    return np.logaddexp(0.0, z)


# ---------------------------------------------------------------------------
# The named workloads.
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class FwdShape:
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str
    dt_recipe: str = "standard"
    final_state: bool = True     # whether the workload returns the final state


FWD_CONFIGS = {
    # tiny fp32 case that the oracle finishes instantly
    "tiny_f32": FwdShape(1, 256, 2, 16, 16, 1, 64, F32),
    # Mamba-2 130M-shaped layer
    "m2_130m": FwdShape(4, 2048, 24, 64, 128, 1, 256, BF16, dt_recipe="mamba2_dt", final_state=False),
    # Mamba-2 2.7B-shaped layer, returns the final state
    "m2_2p7b": FwdShape(8, 4096, 80, 64, 128, 1, 256, BF16),
}
# seqlen sweep at state size 64
SWEEP_SEQLENS = (512, 2048, 8192, 32768, 131072, 524288)


def sweep_shape(seqlen: int) -> FwdShape:
    return FwdShape(1, seqlen, 32, 64, 64, 1, 256, BF16, final_state=False)


@dataclasses.dataclass(frozen=True)
class StepShape:
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    dtype: str
    steps: int


DECODE_CONFIG = StepShape(256, 80, 64, 128, 1, BF16, 1024)


def _a(rng, Bz, L, H, recipe):
    A = -np.exp(rng.uniform(0.0, np.log(16.0), size=H))
    z = rng.standard_normal((Bz, L, H))
    if recipe == "standard":
        dt = _softplus(z - 2.0)
    elif recipe == "mamba2_dt":
        dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(0.1), size=H))
        bias = np.log(np.expm1(dt0))
        dt = np.clip(_softplus(z + bias), 1e-3, 0.1)
    else:
        raise ValueError(recipe)
    return (dt * A).astype(np.float32)


def make_fwd(shape: FwdShape, seed: int = 0, with_initial_state: bool = False):
    """Draw one forward batch.  Returns a dict with X, a, B, C (+ S0), where
    X/B/C are float32 arrays or uint16 bf16 bit patterns per ``shape.dtype``
    and a (and S0) are float32."""
    rng = np.random.default_rng(seed)
    Bz, L, H, P = shape.batch, shape.seqlen, shape.nheads, shape.headdim
    G, N = shape.ngroups, shape.dstate
    a = _a(rng, Bz, L, H, shape.dt_recipe)
    X = _store(rng.standard_normal((Bz, L, H, P), dtype=np.float32), shape.dtype)
    B = _store(rng.standard_normal((Bz, L, G, N), dtype=np.float32), shape.dtype)
    C = _store(rng.standard_normal((Bz, L, G, N), dtype=np.float32), shape.dtype)
    out = {"X": X, "a": a, "B": B, "C": C, "shape": shape}
    if with_initial_state:
        out["S0"] = (0.1 * rng.standard_normal((Bz, H, P, N), dtype=np.float32)).astype(np.float32)
    return out


def make_upstream_grads(shape: FwdShape, seed: int = 0):
    """Upstream gradients for a backward test: dY ~ N(0, 1) in the shape's
    dtype (like Y) and dS_fin ~ N(0, 0.1^2) float32 [Bz,H,P,N], drawn in that
    order from their own stream (seed offset so they differ from the inputs)."""
    rng = np.random.default_rng(seed + 0x5EED)
    Bz, L, H, P = shape.batch, shape.seqlen, shape.nheads, shape.headdim
    dY = _store(rng.standard_normal((Bz, L, H, P), dtype=np.float32), shape.dtype)
    dSf = (0.1 * rng.standard_normal((Bz, H, P, shape.dstate), dtype=np.float32)).astype(np.float32)
    return {"dY": dY, "dS_fin": dSf}


def make_integer_grads_case(shape: FwdShape, seed: int = 0):
    """Decay-free integer inputs for exactness checks: a = 0, X, B, C, dY with
    entries in {-1, 0, 1} (exact in bf16), S0 and dS_fin with integer entries
    in [-2, 2].  Every product and partial sum the layer and its gradients form
    is then a small integer."""
    rng = np.random.default_rng(seed)
    Bz, L, H, P = shape.batch, shape.seqlen, shape.nheads, shape.headdim
    G, N = shape.ngroups, shape.dstate
    tern = lambda *sz: rng.integers(-1, 2, size=sz).astype(np.float32)
    out = {"X": _store(tern(Bz, L, H, P), shape.dtype), "a": np.zeros((Bz, L, H), np.float32),
           "B": _store(tern(Bz, L, G, N), shape.dtype), "C": _store(tern(Bz, L, G, N), shape.dtype),
           "shape": shape}
    out["S0"] = rng.integers(-2, 3, size=(Bz, H, P, N)).astype(np.float32)
    out["dY"] = _store(tern(Bz, L, H, P), shape.dtype)
    out["dS_fin"] = rng.integers(-2, 3, size=(Bz, H, P, N)).astype(np.float32)
    return out


def make_decode(shape: StepShape, seed: int = 0, steps: Optional[int] = None):
    """Draw a decode run: state cache [Bz,H,P,N] f32 and per-step inputs
    x [T,Bz,H,P], a [T,Bz,H], B/C [T,Bz,G,N]."""
    rng = np.random.default_rng(seed)
    T = shape.steps if steps is None else steps
    Bz, H, P, N, G = shape.batch, shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    # a drawn as a [Bz, T, H] sequence, then laid out step-major
    a = _a(rng, Bz, T, H, "standard").transpose(1, 0, 2).copy()
    x = _store(rng.standard_normal((T, Bz, H, P), dtype=np.float32), shape.dtype)
    B = _store(rng.standard_normal((T, Bz, G, N), dtype=np.float32), shape.dtype)
    C = _store(rng.standard_normal((T, Bz, G, N), dtype=np.float32), shape.dtype)
    state = (0.1 * rng.standard_normal((Bz, H, P, N), dtype=np.float32)).astype(np.float32)
    return {"state": state, "x": x, "a": a, "B": B, "C": C, "shape": shape}


def custom_fwd(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
               seed=0, dt_recipe="standard", with_initial_state=False):
    """Any shape with the standard value recipe (used for ragged/edge cases)."""
    return make_fwd(FwdShape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                             dtype, dt_recipe), seed=seed,
                    with_initial_state=with_initial_state)
