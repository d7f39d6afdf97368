"""MI355X (gfx950) SSD layer: chunked forward, its backward, and the recurrent
decode step.

A thin torch binding over libssd.so's C ABI (include/ssd.h).  This module
only marshals arguments -- checks every tensor's shape, dtype, device and
contiguity against the call's sizes (raising ValueError before anything is
launched), allocates outputs and workspace with torch, and passes raw device
pointers plus the current HIP stream.  Every step of the computation runs in the library's HIP
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

__all__ = ["chunk_scan_fwd", "chunk_scan_fwd_noalloc", "chunk_scan_bwd", "bwd_workspace_bytes", "bwd_da_workspace_bytes", "bwd_da", "step", "stream_rmw", "chunk_cumsum", "chunk_state", "state_passing",
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


def _check(name, t, shape, dtype, device):
    """Raise ValueError unless tensor ``t`` (None is accepted: optional) has
    exactly ``shape``, ``dtype`` (None: any) and lives on ``device``; shape
    and dtype are checked first so that a mismatch is reported as such."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s (the device of X)" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_bytes(name, t, nbytes, device):
    """A workspace: any dtype, contiguous, on ``device``, at least ``nbytes``."""
    if t is None:
        return
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes, %d needed" % (name, t.numel() * t.element_size(), nbytes))


def _fwd_sizes(X, B):
    """(Bz, L, H, P, G, N) from X [Bz,L,H,P] and B [Bz,L,G,N] (checked)."""
    if not isinstance(X, torch.Tensor) or X.dim() != 4:
        raise ValueError("X must be a 4-D tensor [batch, seqlen, nheads, headdim]")
    _dtype_code(X)
    if not isinstance(B, torch.Tensor) or B.dim() != 4:
        raise ValueError("B must be a 4-D tensor [batch, seqlen, ngroups, dstate]")
    Bz, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    _check("B", B, (Bz, L, G, N), X.dtype, X.device)
    return Bz, L, H, P, G, N


def _check_fwd_inputs(X, a, B, C):
    Bz, L, H, P, G, N = _fwd_sizes(X, B)
    _check("a", a, (Bz, L, H), torch.float32, X.device)
    _check("C", C, (Bz, L, G, N), X.dtype, X.device)
    if a is None or C is None:
        raise ValueError("a and C are required")
    return Bz, L, H, P, G, N


def _units(L, chunk, seg_chunks):
    nc = (int(L) + int(chunk) - 1) // int(chunk)
    k = max(1, int(seg_chunks))
    return (nc + k - 1) // k


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _desc(X, B, chunk, algo, seg_chunks, wg_units=0):
    Bz, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    return _lib.fwd_desc(Bz, L, H, P, N, G, int(chunk), _dtype_code(X), int(algo), int(seg_chunks),
                         int(wg_units))


def fwd_plan(X, B, chunk, algo=SSD_ALGO_AUTO, seg_chunks=0, wg_units=0, with_units=False):
    """(algo, seg_chunks, nseg) the library would use for these shapes, plus
    the fused pass's units per workgroup when ``with_units``."""
    d = _desc(X, B, chunk, algo, seg_chunks, wg_units)
    a = ctypes.c_int32()
    k = ctypes.c_int64()
    n = ctypes.c_int64()
    u = ctypes.c_int32()
    _lib.check(_L().ssd_fwd_plan(ctypes.byref(d), ctypes.byref(a), ctypes.byref(k), ctypes.byref(n),
                                 ctypes.byref(u)))
    return (a.value, k.value, n.value, u.value) if with_units else (a.value, k.value, n.value)


def workspace_bytes(X, B, chunk, algo=SSD_ALGO_AUTO, seg_chunks=0, wg_units=0) -> int:
    d = _desc(X, B, chunk, algo, seg_chunks, wg_units)
    n = ctypes.c_size_t()
    _lib.check(_L().ssd_fwd_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def chunk_scan_fwd(X, a, B, C, chunk, initial_state=None, return_final_state=False,
                   algo=SSD_ALGO_AUTO, seg_chunks=0, Y=None, final_state=None, workspace=None,
                   wg_units=0):
    """Full SSD forward.  Returns (Y, final_state or None)."""
    Bz, L, H, P, G, N = _check_fwd_inputs(X, a, B, C)
    dev = X.device
    _check("initial_state", initial_state, (Bz, H, P, N), torch.float32, dev)
    _check("Y", Y, X.shape, X.dtype, dev)
    _check("final_state", final_state, (Bz, H, P, N), torch.float32, dev)
    d = _desc(X, B, chunk, algo, seg_chunks, wg_units)
    if Y is None:
        Y = torch.empty_like(X)
    if final_state is None and return_final_state:
        final_state = torch.empty((X.shape[0], X.shape[2], X.shape[3], B.shape[3]),
                                  dtype=torch.float32, device=dev)
    nws = ctypes.c_size_t()
    _lib.check(_L().ssd_fwd_workspace_bytes(ctypes.byref(d), ctypes.byref(nws)))
    _check_bytes("workspace", workspace, nws.value, dev)
    if workspace is None and nws.value > 0:
        workspace = torch.empty(nws.value, dtype=torch.uint8, device=dev)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(_L().ssd_chunk_scan_fwd(
        ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(C), _ptr(initial_state), _ptr(Y),
        _ptr(final_state), _ptr(workspace), wsz, _stream(dev)))
    return Y, final_state


def chunk_scan_fwd_noalloc(X, a, B, C, chunk, initial_state=None, Y=None, final_state=None,
                           algo=SSD_ALGO_AUTO, seg_chunks=0, wg_units=0):
    """The forward through the C ABI's allocation-free entry point: the
    library's own per-GPU device array holds the segment states, so the call
    allocates nothing when Y (and final_state, if wanted) are passed in.
    Returns (Y, final_state or None)."""
    Bz, L, H, P, G, N = _check_fwd_inputs(X, a, B, C)
    dev = X.device
    _check("initial_state", initial_state, (Bz, H, P, N), torch.float32, dev)
    _check("Y", Y, X.shape, X.dtype, dev)
    _check("final_state", final_state, (Bz, H, P, N), torch.float32, dev)
    d = _desc(X, B, chunk, algo, seg_chunks, wg_units)
    if Y is None:
        Y = torch.empty_like(X)
    _lib.check(_L().ssd_chunk_scan_fwd_noalloc(
        ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(C), _ptr(initial_state), _ptr(Y),
        _ptr(final_state), _stream(dev)))
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
    Bz, L, H, P, G, N = _check_fwd_inputs(X, a, B, C)
    dev = X.device
    _check("dY", dY, X.shape, X.dtype, dev)
    if dY is None:
        raise ValueError("dY is required")
    _check("initial_state", initial_state, (Bz, H, P, N), torch.float32, dev)
    _check("dfinal_state", dfinal_state, (Bz, H, P, N), torch.float32, dev)
    d = _desc(X, B, chunk, SSD_ALGO_AUTO, 0)
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
    _check_bytes("workspace", workspace, nws.value, dev)
    if workspace is None and nws.value > 0:
        workspace = torch.empty(nws.value, dtype=torch.uint8, device=dev)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(_L().ssd_chunk_scan_bwd(
        ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(C), _ptr(initial_state), _ptr(dY),
        _ptr(dfinal_state), _ptr(dX), _ptr(da), _ptr(dB), _ptr(dC), _ptr(dS0), _ptr(workspace),
        wsz, _stream(dev)))
    return {"dX": dX, "da": da, "dB": dB, "dC": dC, "dinitial_state": dS0}


def bwd_da_workspace_bytes(X, B, chunk) -> int:
    d = _desc(X, B, chunk, SSD_ALGO_AUTO, 0)
    n = ctypes.c_size_t()
    _lib.check(_L().ssd_bwd_da_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def bwd_da(X, a, B, C, dY, chunk, states_in, adjoint_in, da=None, workspace=None):
    """The backward's da stage alone, from the states entering each chunk and
    the adjoint dl/dS at the first step of each next chunk (dS_fin for the
    last), both [Bz, nchunks, H, P, N] float32.  The workspace (uint8, at
    least bwd_da_workspace_bytes) is allocated when not given."""
    Bz, L, H, P, G, N = _check_fwd_inputs(X, a, B, C)
    dev = X.device
    _check("dY", dY, X.shape, X.dtype, dev)
    nc = _units(L, chunk, 1)
    for nm, t in (("states_in", states_in), ("adjoint_in", adjoint_in)):
        if t is None:
            raise ValueError("%s is required" % nm)
        _check(nm, t, (Bz, nc, H, P, N), torch.float32, dev)
    _check("da", da, (Bz, L, H), torch.float32, dev)
    d = _desc(X, B, chunk, SSD_ALGO_AUTO, 0)
    if da is None:
        da = torch.empty_like(a)
    nws = ctypes.c_size_t()
    _lib.check(_L().ssd_bwd_da_workspace_bytes(ctypes.byref(d), ctypes.byref(nws)))
    _check_bytes("workspace", workspace, nws.value, dev)
    if workspace is None and nws.value > 0:
        workspace = torch.empty(nws.value, dtype=torch.uint8, device=dev)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(_L().ssd_bwd_da(ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(C), _ptr(dY),
                               _ptr(states_in), _ptr(adjoint_in), _ptr(da), _ptr(workspace), wsz,
                               _stream(X.device)))
    return da


def step(state, x, a, B, C, y=None):
    """One recurrent decode step; ``state`` is updated in place.  Returns y.

    state [Bz,H,P,N] f32, x [Bz,H,P], a [Bz,H] f32, B/C [Bz,G,N]."""
    if not isinstance(state, torch.Tensor) or state.dim() != 4:
        raise ValueError("state must be a 4-D tensor [batch, nheads, headdim, dstate]")
    if not isinstance(B, torch.Tensor) or B.dim() != 3:
        raise ValueError("B must be a 3-D tensor [batch, ngroups, dstate]")
    Bz, H, P, N = state.shape
    G = B.shape[1]
    dev = state.device
    _check("state", state, (Bz, H, P, N), torch.float32, dev)
    if not isinstance(x, torch.Tensor):
        raise ValueError("x is required")
    _dtype_code(x)
    _check("x", x, (Bz, H, P), x.dtype, dev)
    _check("a", a, (Bz, H), torch.float32, dev)
    _check("B", B, (Bz, G, N), x.dtype, dev)
    _check("C", C, (Bz, G, N), x.dtype, dev)
    _check("y", y, (Bz, H, P), x.dtype, dev)
    if a is None or C is None:
        raise ValueError("a and C are required")
    if y is None:
        y = torch.empty_like(x)
    d = _lib.StepDesc(Bz, H, P, N, G, _dtype_code(x), 0)
    _lib.check(_L().ssd_step(ctypes.byref(d), _ptr(state), _ptr(x), _ptr(a), _ptr(B), _ptr(C),
                             _ptr(y), _stream(state.device)))
    return y


def stream_rmw(t, scale, per_thread=8, nontemporal=True):
    """In-place ``t *= scale`` over a contiguous fp32 device tensor through the
    library's streaming kernel: the HBM ceiling the decode step is measured
    against.  Returns t."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError("t must be a contiguous float32 tensor")
    if t.numel() % 4 != 0:
        raise ValueError("t.numel() must be a multiple of 4")
    _lib.check(_L().ssd_stream_rmw(_ptr(t), t.numel(), float(scale), int(per_thread), int(bool(nontemporal)),
                                   _stream(t.device)))
    return t


# ---- stage entry points ------------------------------------------------------
def chunk_cumsum(a, chunk):
    """Stage 1: (cs [Bz,H,nc,Q], lam [Bz,H,nc]) from a [Bz,L,H]."""
    if not isinstance(a, torch.Tensor) or a.dim() != 3:
        raise ValueError("a must be a 3-D tensor [batch, seqlen, nheads]")
    Bz, L, H = a.shape
    _check("a", a, (Bz, L, H), torch.float32, a.device)
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
    Bz, L, H, P, G, N = _fwd_sizes(X, B)
    _check("a", a, (Bz, L, H), torch.float32, X.device)
    if a is None:
        raise ValueError("a is required")
    k = max(1, int(seg_chunks))
    U = _units(L, chunk, k)
    _check("out", out, (Bz, U, H, P, N), torch.float32, X.device)
    d = _desc(X, B, chunk, SSD_ALGO_MFMA, k)
    if out is None:
        out = torch.empty((Bz, U, H, P, N), dtype=torch.float32, device=X.device)
    _lib.check(_L().ssd_chunk_state(ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(out),
                                    _stream(X.device)))
    return out


def state_passing(dstates, lam, chunk, seqlen, initial_state=None, return_final_state=True,
                  out=None, seg_chunks=1):
    """Stage 4: states entering each unit of `seg_chunks` chunks [Bz,U,H,P,N]
    (+ final state); lam [Bz,H,U] holds each unit's total log-decay."""
    if not isinstance(dstates, torch.Tensor) or dstates.dim() != 5:
        raise ValueError("dstates must be a 5-D tensor [batch, units, nheads, headdim, dstate]")
    Bz, nu, H, P, N = dstates.shape
    dev = dstates.device
    want = _units(seqlen, chunk, seg_chunks)
    if nu != want:
        raise ValueError("dstates has %d units; seqlen %d in units of %d chunks of %d needs %d"
                         % (nu, seqlen, max(1, int(seg_chunks)), int(chunk), want))
    _check("dstates", dstates, (Bz, nu, H, P, N), torch.float32, dev)
    _check("lam", lam, (Bz, H, nu), torch.float32, dev)
    if lam is None:
        raise ValueError("lam is required")
    _check("initial_state", initial_state, (Bz, H, P, N), torch.float32, dev)
    _check("out", out, (Bz, nu, H, P, N), torch.float32, dev)
    d = _lib.fwd_desc(Bz, seqlen, H, P, N, 1, int(chunk), SSD_F32)
    d.seg_chunks = max(1, int(seg_chunks))
    if out is None:
        out = torch.empty_like(dstates)
    fin = torch.empty((Bz, H, P, N), dtype=torch.float32, device=dstates.device) if return_final_state else None
    _lib.check(_L().ssd_state_passing(ctypes.byref(d), _ptr(dstates), _ptr(lam), _ptr(initial_state),
                                      _ptr(out), _ptr(fin), _stream(dstates.device)))
    return out, fin


def chunk_scan(X, a, B, C, chunk, states_in=None, seg_chunks=1, Y=None, wg_units=0):
    """Stages 2 + 5: Y from the inputs and the states entering each unit of
    `seg_chunks` chunks ([Bz,U,H,P,N]; None = zero)."""
    Bz, L, H, P, G, N = _check_fwd_inputs(X, a, B, C)
    U = _units(L, chunk, seg_chunks)
    _check("states_in", states_in, (Bz, U, H, P, N), torch.float32, X.device)
    _check("Y", Y, X.shape, X.dtype, X.device)
    d = _desc(X, B, chunk, SSD_ALGO_MFMA, max(1, int(seg_chunks)), wg_units)
    if Y is None:
        Y = torch.empty_like(X)
    _lib.check(_L().ssd_chunk_scan(ctypes.byref(d), _ptr(X), _ptr(a), _ptr(B), _ptr(C),
                                   _ptr(states_in), _ptr(Y), _stream(X.device)))
    return Y
