"""MI355X (gfx950) SSD layer: chunked forward, its backward, and the recurrent
decode step.

A thin torch binding over libssd.so's C ABI (include/ssd.h).  This module
only marshals arguments -- checks devices/dtypes/contiguity, allocates
outputs and workspace with torch, and passes raw device pointers plus the
current HIP stream.  Every step of the computation runs in the library's HIP
kernels; there is no fallback of any kind, and every function raises if the
library is not built.

Layouts (contiguous): X, Y [batch, seqlen, nheads, headdim]; a [batch, seqlen,
nheads] float32; B, C [batch, seqlen, ngroups, dstate]; states [batch, nheads,
headdim, dstate] float32.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (SSD_ALGO_AUTO, SSD_ALGO_MFMA, SSD_ALGO_VALU, SSD_BF16, SSD_F32,
                   SSDError)

__all__ = ["chunk_scan_fwd", "chunk_scan_bwd", "bwd_workspace_bytes", "bwd_da", "step", "chunk_cumsum", "chunk_state", "state_passing",
           "chunk_scan", "fwd_plan", "workspace_bytes", "SSDError", "SSD_ALGO_AUTO",
           "SSD_ALGO_MFMA", "SSD_ALGO_VALU", "library_path"]


def library_path() -> str:
    return _lib.LIB_PATH


def _L():
    return _lib.load()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise TypeError("X/B/C must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _desc(X, B, chunk, algo, seg_chunks):
    Bz, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    return _lib.fwd_desc(Bz, L, H, P, N, G, int(chunk), _dtype_code(X), int(algo), int(seg_chunks))


def fwd_plan(X, B, chunk, algo=SSD_ALGO_AUTO, seg_chunks=0):
    """(algo, seg_chunks, nseg) the library would use for these shapes."""
    d = _desc(X, B, chunk, algo, seg_chunks)
    a = ctypes.c_int32()
    k = ctypes.c_int64()
    n = ctypes.c_int64()
    _lib.check(_L().ssd_fwd_plan(ctypes.byref(d), ctypes.byref(a), ctypes.byref(k), ctypes.byref(n)))
    return a.value, k.value, n.value


def workspace_bytes(X, B, chunk, algo=SSD_ALGO_AUTO, seg_chunks=0) -> int:
    d = _desc(X, B, chunk, algo, seg_chunks)
    n = ctypes.c_size_t()
    _lib.check(_L().ssd_fwd_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def chunk_scan_fwd(X, a, B, C, chunk, initial_state=None, return_final_state=False,
                   algo=SSD_ALGO_AUTO, seg_chunks=0, Y=None, final_state=None, workspace=None):
    """Full SSD forward.  Returns (Y, final_state or None)."""
    d = _desc(X, B, chunk, algo, seg_chunks)
    dev = X.device
    if Y is None:
        Y = torch.empty_like(X)
    if final_state is None and return_final_state:
        final_state = torch.empty((X.shape[0], X.shape[2], X.shape[3], B.shape[3]),
                                  dtype=torch.float32, device=dev)
    nws = ctypes.c_size_t()
    _lib.check(_L().ssd_fwd_workspace_bytes(ctypes.byref(d), ctypes.byref(nws)))
    if workspace is None and nws.value > 0:
        workspace = torch.empty(nws.value, dtype=torch.uint8, device=dev)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(_L().ssd_chunk_scan_fwd(
        ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(C), _ptr(initial_state), _ptr(Y),
        _ptr(final_state), _ptr(workspace), wsz, _stream(dev)))
    return Y, final_state


def bwd_workspace_bytes(X, B, chunk) -> int:
    d = _desc(X, B, chunk, SSD_ALGO_AUTO, 0)
    n = ctypes.c_size_t()
    _lib.check(_L().ssd_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def chunk_scan_bwd(X, a, B, C, dY, chunk, initial_state=None, dfinal_state=None,
                   return_dinitial_state=False, workspace=None):
    """Gradients of the full forward for upstream dY (and dfinal_state).

    Returns a dict with dX, dB, dC (X's dtype), da (float32) and dinitial_state
    (float32, or None unless requested)."""
    d = _desc(X, B, chunk, SSD_ALGO_AUTO, 0)
    dev = X.device
    dX = torch.empty_like(X)
    dB = torch.empty_like(B)
    dC = torch.empty_like(C)
    da = torch.empty_like(a)
    dS0 = None
    if return_dinitial_state:
        dS0 = torch.empty((X.shape[0], X.shape[2], X.shape[3], B.shape[3]), dtype=torch.float32,
                          device=dev)
    nws = ctypes.c_size_t()
    _lib.check(_L().ssd_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(nws)))
    if workspace is None and nws.value > 0:
        workspace = torch.empty(nws.value, dtype=torch.uint8, device=dev)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(_L().ssd_chunk_scan_bwd(
        ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(C), _ptr(initial_state), _ptr(dY),
        _ptr(dfinal_state), _ptr(dX), _ptr(da), _ptr(dB), _ptr(dC), _ptr(dS0), _ptr(workspace),
        wsz, _stream(dev)))
    return {"dX": dX, "da": da, "dB": dB, "dC": dC, "dinitial_state": dS0}


def bwd_da(X, a, B, C, dY, chunk, states_in, adjoint_in, da=None):
    """The backward's da stage alone, from the states entering each chunk and
    the adjoint dl/dS at the first step of each next chunk (dS_fin for the
    last), both [Bz, nchunks, H, P, N] float32."""
    d = _desc(X, B, chunk, SSD_ALGO_AUTO, 0)
    if da is None:
        da = torch.empty_like(a)
    _lib.check(_L().ssd_bwd_da(ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(C), _ptr(dY),
                               _ptr(states_in), _ptr(adjoint_in), _ptr(da), _stream(X.device)))
    return da


def step(state, x, a, B, C, y=None):
    """One recurrent decode step; ``state`` is updated in place.  Returns y.

    state [Bz,H,P,N] f32, x [Bz,H,P], a [Bz,H] f32, B/C [Bz,G,N]."""
    Bz, H, P, N = state.shape
    G = B.shape[1]
    if y is None:
        y = torch.empty_like(x)
    d = _lib.StepDesc(Bz, H, P, N, G, _dtype_code(x), 0)
    _lib.check(_L().ssd_step(ctypes.byref(d), _ptr(state), _ptr(x), _ptr(a), _ptr(B), _ptr(C),
                             _ptr(y), _stream(state.device)))
    return y


# ---- stage entry points ------------------------------------------------------
def chunk_cumsum(a, chunk):
    """Stage 1: (cs [Bz,H,nc,Q], lam [Bz,H,nc]) from a [Bz,L,H]."""
    Bz, L, H = a.shape
    Q = int(chunk)
    nc = (L + Q - 1) // Q
    d = _lib.fwd_desc(Bz, L, H, 4, 4, 1, Q, SSD_F32)
    cs = torch.empty((Bz, H, nc, Q), dtype=torch.float32, device=a.device)
    lam = torch.empty((Bz, H, nc), dtype=torch.float32, device=a.device)
    _lib.check(_L().ssd_chunk_cumsum(ctypes.byref(d), _ptr(a), _ptr(cs), _ptr(lam), _stream(a.device)))
    return cs, lam


def chunk_state(X, a, B, chunk, seg_chunks=1, out=None):
    """Stage 3: states built inside each unit of `seg_chunks` chunks from a
    zero state, dS [Bz,U,H,P,N] f32 (U = number of units)."""
    Bz, L, H, P = X.shape
    N = B.shape[3]
    nc = (L + int(chunk) - 1) // int(chunk)
    k = max(1, int(seg_chunks))
    d = _desc(X, B, chunk, SSD_ALGO_MFMA, k)
    if out is None:
        out = torch.empty((Bz, (nc + k - 1) // k, H, P, N), dtype=torch.float32, device=X.device)
    _lib.check(_L().ssd_chunk_state(ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(out),
                                    _stream(X.device)))
    return out


def state_passing(dstates, lam, chunk, seqlen, initial_state=None, return_final_state=True,
                  out=None, seg_chunks=1):
    """Stage 4: states entering each unit of `seg_chunks` chunks [Bz,U,H,P,N]
    (+ final state); lam [Bz,H,U] holds each unit's total log-decay."""
    Bz, nu, H, P, N = dstates.shape
    d = _lib.fwd_desc(Bz, seqlen, H, P, N, 1, int(chunk), SSD_F32)
    d.seg_chunks = max(1, int(seg_chunks))
    if out is None:
        out = torch.empty_like(dstates)
    fin = torch.empty((Bz, H, P, N), dtype=torch.float32, device=dstates.device) if return_final_state else None
    _lib.check(_L().ssd_state_passing(ctypes.byref(d), _ptr(dstates), _ptr(lam), _ptr(initial_state),
                                      _ptr(out), _ptr(fin), _stream(dstates.device)))
    return out, fin


def chunk_scan(X, a, B, C, chunk, states_in=None, seg_chunks=1, Y=None):
    """Stages 2 + 5: Y from the inputs and the states entering each unit of
    `seg_chunks` chunks ([Bz,U,H,P,N]; None = zero)."""
    d = _desc(X, B, chunk, SSD_ALGO_MFMA, max(1, int(seg_chunks)))
    if Y is None:
        Y = torch.empty_like(X)
    _lib.check(_L().ssd_chunk_scan(ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(C),
                                   _ptr(states_in), _ptr(Y), _stream(X.device)))
    return Y
