"""fp64 CPU oracle for the SSD layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``ssd_chunked_scan_chunk_amd``) and never imports it.

Two independent formulations live here:

* ``fwd`` / ``step`` / ``chunked_fwd`` / ``bwd``: the C oracle in
  ``ssd_oracle.c`` (sequential recurrence, one recurrent step, the fp64
  chunked four-stage form with every intermediate, and the gradients through
  the recurrence's adjoint), called through ctypes.
* ``quadratic``: numpy brute force of the dual "structured masked attention"
  form ``Y = (L o C B^T) X`` (wiki review of "Transformers are SSMs", section
  "Core concepts": SMA generalises linear attention with a data-dependent
  mask; CiteArk page, section "what this means": 1-semiseparable SSMs are
  exactly structured masked attention).  Tiny inputs only.

Every public function takes float64 numpy arrays in the layouts documented in
``ssd_oracle.c`` and returns float64 arrays.  Parity status: every function is
pinned by ``tests/test_oracle.py`` (closed forms, special cases, brute force
and the hand-derived fixtures under ``tests/golden/``); nothing here is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
# SSD_ORACLE_LIB names another build of ssd_oracle.c (a sanitizer build)
_LIB_PATH = os.environ.get("SSD_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc -O2 (no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups")]


def _load():
    global _lib
    if _lib is None:
        if not os.environ.get("SSD_ORACLE_LIB") and (not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_fwd.argtypes = [ctypes.POINTER(_Dims), dp, dp, dp, dp, dp, dp, dp,
                                   ctypes.c_int]
        lib.oracle_step.argtypes = [ctypes.POINTER(_Dims), dp, dp, dp, dp, dp, dp]
        lib.oracle_chunked_fwd.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int64] + [dp] * 13
        lib.oracle_bwd.argtypes = [ctypes.POINTER(_Dims)] + [dp] * 12
        for f in (lib.oracle_fwd, lib.oracle_step, lib.oracle_chunked_fwd, lib.oracle_bwd):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(arr):
    if arr is None:
        return None
    assert arr.dtype == np.float64 and arr.flags.c_contiguous
    return arr.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _dims(X, B):
    Bz, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    return _Dims(Bz, L, H, P, N, G)


def fwd(X, a, B, C, S0=None, nthreads: int = 1):
    """Sequential fp64 recurrence.  Returns (Y, S_fin).

    X [Bz,L,H,P], a [Bz,L,H], B/C [Bz,L,G,N], S0 [Bz,H,P,N] or None.
    """
    X, a, B, C, S0 = map(_f64, (X, a, B, C, S0))
    Bz, L, H, P = X.shape
    N = B.shape[3]
    Y = np.empty((Bz, L, H, P))
    S_fin = np.empty((Bz, H, P, N))
    d = _dims(X, B)
    rc = _load().oracle_fwd(ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(C),
                            _ptr(S0), _ptr(Y), _ptr(S_fin), int(nthreads))
    if rc:
        raise ValueError("oracle_fwd rejected its arguments (code %d)" % rc)
    return Y, S_fin


def step(state, x, a, B, C):
    """One recurrent step, returns (new_state, y); the input state is not modified.

    state [Bz,H,P,N], x [Bz,H,P], a [Bz,H], B/C [Bz,G,N].
    """
    state = np.array(state, dtype=np.float64, order="C", copy=True)
    x, a, B, C = map(_f64, (x, a, B, C))
    Bz, H, P, N = state.shape
    G = B.shape[1]
    y = np.empty((Bz, H, P))
    d = _Dims(Bz, 1, H, P, N, G)
    rc = _load().oracle_step(ctypes.byref(d), _ptr(state), _ptr(x), _ptr(a), _ptr(B),
                             _ptr(C), _ptr(y))
    if rc:
        raise ValueError("oracle_step rejected its arguments (code %d)" % rc)
    return state, y


def chunked_fwd(X, a, B, C, chunk: int, S0=None):
    """fp64 chunked four-stage form.  Returns a dict of every intermediate:
    cs [Bz,H,nc,Q], lam [Bz,H,nc], dS / S_in [Bz,nc,H,P,N],
    Ydiag / Yoff / Y [Bz,L,H,P], S_fin [Bz,H,P,N]."""
    X, a, B, C, S0 = map(_f64, (X, a, B, C, S0))
    Bz, L, H, P = X.shape
    N = B.shape[3]
    Q = int(chunk)
    nc = (L + Q - 1) // Q
    out = {
        "cs": np.empty((Bz, H, nc, Q)), "lam": np.empty((Bz, H, nc)),
        "dS": np.empty((Bz, nc, H, P, N)), "S_in": np.empty((Bz, nc, H, P, N)),
        "Ydiag": np.empty((Bz, L, H, P)), "Yoff": np.empty((Bz, L, H, P)),
        "Y": np.empty((Bz, L, H, P)), "S_fin": np.empty((Bz, H, P, N)),
    }
    d = _dims(X, B)
    rc = _load().oracle_chunked_fwd(
        ctypes.byref(d), Q, _ptr(X), _ptr(a), _ptr(B), _ptr(C), _ptr(S0),
        _ptr(out["cs"]), _ptr(out["lam"]), _ptr(out["dS"]), _ptr(out["S_in"]),
        _ptr(out["Ydiag"]), _ptr(out["Yoff"]), _ptr(out["Y"]), _ptr(out["S_fin"]))
    if rc:
        raise ValueError("oracle_chunked_fwd rejected its arguments (code %d)" % rc)
    return out


def bwd(X, a, B, C, dY, S0=None, dS_fin=None):
    """Gradients of l = sum(dY * Y) + sum(dS_fin * S_fin) through the fp64
    recurrence, by its adjoint (reverse-mode chain rule, see ssd_oracle.c).

    Returns a dict with dX [Bz,L,H,P], da [Bz,L,H], dB / dC [Bz,L,G,N] (summed
    over each group's heads) and dS0 [Bz,H,P,N]."""
    X, a, B, C, dY, S0, dS_fin = map(_f64, (X, a, B, C, dY, S0, dS_fin))
    Bz, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    out = {"dX": np.empty((Bz, L, H, P)), "da": np.empty((Bz, L, H)),
           "dB": np.empty((Bz, L, G, N)), "dC": np.empty((Bz, L, G, N)),
           "dS0": np.empty((Bz, H, P, N))}
    d = _dims(X, B)
    rc = _load().oracle_bwd(ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(C), _ptr(S0),
                            _ptr(dY), _ptr(dS_fin), _ptr(out["dX"]), _ptr(out["da"]),
                            _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dS0"]))
    if rc:
        raise ValueError("oracle_bwd rejected its arguments (code %d)" % rc)
    return out


def decay_mask(a_seq):
    """The 1-semiseparable mask of one (b, h) sequence, fp64, by direct sums:
    Lmask[t, s] = exp(a[s+1] + ... + a[t]) for t >= s, else 0."""
    a_seq = np.asarray(a_seq, dtype=np.float64)
    L = a_seq.shape[0]
    M = np.zeros((L, L))
    for t in range(L):
        seg = 0.0
        M[t, t] = 1.0
        for s in range(t - 1, -1, -1):
            seg += a_seq[s + 1]
            M[t, s] = np.exp(seg)
    return M


def quadratic(X, a, B, C):
    """Brute-force dual form: per (b, h), Y = (Lmask o (C B^T)) X, fp64.

    Returns Y [Bz,L,H,P].  O(L^2) memory per slice: tiny inputs only."""
    X, a, B, C = map(_f64, (X, a, B, C))
    Bz, L, H, P = X.shape
    G = B.shape[2]
    Y = np.empty((Bz, L, H, P))
    for b in range(Bz):
        for h in range(H):
            g = h * G // H
            M = decay_mask(a[b, :, h]) * (C[b, :, g, :] @ B[b, :, g, :].T)
            Y[b, :, h, :] = M @ X[b, :, h, :]
    return Y
