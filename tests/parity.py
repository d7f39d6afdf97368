"""Error metrics and golden-fixture reader shared by the tests."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Tolerances: max relative error 1e-5 for fp32 inputs and 2e-2 for bf16
# inputs with fp32 accumulation, in the slice-normwise sense below.
TOL = {"f32": 1e-5, "bf16": 2e-2}


def slice_rel_err(got, ref, slice_axes):
    """max over slices of  max|got - ref| / max|ref|  (computed in fp64).

    ``slice_axes`` are the axes that index a slice (e.g. batch and head); the
    remaining axes are reduced inside each slice.  Elementwise relative error
    is meaningless near zero, so each (batch, head) slice is normalised by its
    own largest reference magnitude."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    other = tuple(i for i in range(ref.ndim) if i not in slice_axes)
    num = np.abs(got - ref).max(axis=other)
    den = np.abs(ref).max(axis=other)
    den = np.where(den == 0, 1.0, den)
    if np.isnan(got).any():
        return float("inf")
    return float((num / den).max())


def elementwise_diag(got, ref, slice_axes, floor=1e-3):
    """Diagnostic: max |got - ref| / |ref| over the entries whose |ref| is at
    least ``floor`` times their slice's largest |ref| (elementwise relative
    error is unbounded near zero, so it is logged, not bounded)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    other = tuple(i for i in range(ref.ndim) if i not in slice_axes)
    smax = np.abs(ref).max(axis=other, keepdims=True)
    keep = np.abs(ref) >= floor * smax
    if not keep.any():
        return 0.0
    return float((np.abs(got - ref)[keep] / np.abs(ref)[keep]).max())


def chunk_rel_err(got, ref, chunk):
    """Y [Bz, L, H, P]: max over (batch, head, chunk of ``chunk`` steps) of
    max|got - ref| / max|ref| inside that chunk -- the slice-normwise error
    with each chunk normalised by its own magnitude (a tighter check than one
    normalisation over a whole long sequence)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    Bz, L, H, P = ref.shape
    nc = (L + chunk - 1) // chunk
    pad = nc * chunk - L
    if pad:
        z = np.zeros((Bz, pad, H, P))
        got, ref = np.concatenate([got, z], 1), np.concatenate([ref, z], 1)
    d = np.abs(got - ref).reshape(Bz, nc, chunk, H, P).max(axis=(2, 4))
    m = np.abs(ref).reshape(Bz, nc, chunk, H, P).max(axis=(2, 4))
    if np.isnan(got).any():
        return float("inf")
    return float((d / np.where(m == 0, 1.0, m)).max())


def y_err(got, ref):
    """Y is [Bz, L, H, P]: slices are (batch, head)."""
    return slice_rel_err(got, ref, (0, 2))


def state_err(got, ref):
    """States are [Bz, H, P, N]: slices are (batch, head)."""
    return slice_rel_err(got, ref, (0, 1))


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = np.array([float(t) for t in v.split()])
    return out
