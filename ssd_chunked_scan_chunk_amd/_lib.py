"""ctypes view of libssd.so: the C ABI declared in include/ssd.h.

This module needs neither torch nor a GPU: it only opens the shared library
and declares argument types.  Import torch *before* calling ``load()`` in a
process that will launch kernels, so that libssd resolves the HIP runtime that
torch already loaded (both link libamdhip64.so.7) instead of a second copy.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SSD_LIB names another build of the same C ABI (the tests use it to run the
# host-side validation under the sanitizers)
LIB_PATH = os.environ.get("SSD_LIB") or os.path.join(HERE, "libssd.so")

SSD_OK, SSD_ERR_NULL, SSD_ERR_SHAPE, SSD_ERR_DTYPE, SSD_ERR_ALIGN = 0, 1, 2, 3, 4
SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP, SSD_ERR_ALIAS = 5, 6, 7, 8
STATUS_NAMES = {
    0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_DTYPE",
    4: "SSD_ERR_ALIGN", 5: "SSD_ERR_UNSUPPORTED", 6: "SSD_ERR_WORKSPACE",
    7: "SSD_ERR_HIP", 8: "SSD_ERR_ALIAS",
}
SSD_F32, SSD_BF16 = 0, 1
SSD_ALGO_AUTO, SSD_ALGO_VALU, SSD_ALGO_MFMA = 0, 1, 2

# every symbol include/ssd.h declares
EXPORTS = (
    "ssd_fwd_workspace_bytes", "ssd_fwd_plan", "ssd_chunk_scan_fwd", "ssd_step",
    "ssd_chunk_cumsum", "ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan",
    "ssd_status_str", "ssd_last_error", "ssd_version", "ssd_bwd_workspace_bytes",
    "ssd_chunk_scan_bwd", "ssd_bwd_da_workspace_bytes", "ssd_bwd_da", "ssd_chunk_scan_fwd_noalloc",
    "ssd_stream_rmw",
)
SSD_NOALLOC_SCRATCH_BYTES = 64 << 20


class FwdDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("algo", ctypes.c_int32), ("seg_chunks", ctypes.c_int64),
                ("wg_units", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class StepDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("ngroups", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class SSDError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), detail))


_lib = None


def load(path: str = LIB_PATH):
    """Open libssd.so and declare its prototypes.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "libssd.so is not built (%s); run `python -m ssd_chunked_scan_chunk_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pd = ctypes.POINTER(FwdDesc)
    lib.ssd_fwd_workspace_bytes.argtypes = [pd, ctypes.POINTER(sz)]
    lib.ssd_fwd_plan.argtypes = [pd, ctypes.POINTER(i32), ctypes.POINTER(i64), ctypes.POINTER(i64),
                                 ctypes.POINTER(i32)]
    lib.ssd_chunk_scan_fwd.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_chunk_scan_fwd_noalloc.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_step.argtypes = [ctypes.POINTER(StepDesc), vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_chunk_cumsum.argtypes = [pd, vp, vp, vp, vp]
    lib.ssd_chunk_state.argtypes = [pd, vp, vp, vp, vp, vp]
    lib.ssd_state_passing.argtypes = [pd, vp, vp, vp, vp, vp, vp]
    lib.ssd_chunk_scan.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_bwd_workspace_bytes.argtypes = [pd, ctypes.POINTER(sz)]
    lib.ssd_chunk_scan_bwd.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_bwd_da_workspace_bytes.argtypes = [pd, ctypes.POINTER(sz)]
    lib.ssd_bwd_da.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_stream_rmw.argtypes = [vp, ctypes.c_int64, ctypes.c_float, i32, i32, vp]
    for f in ("ssd_fwd_workspace_bytes", "ssd_fwd_plan", "ssd_chunk_scan_fwd", "ssd_chunk_scan_fwd_noalloc",
              "ssd_step",
              "ssd_chunk_cumsum", "ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan",
              "ssd_bwd_workspace_bytes", "ssd_chunk_scan_bwd", "ssd_bwd_da_workspace_bytes", "ssd_bwd_da",
              "ssd_stream_rmw"):
        getattr(lib, f).restype = ctypes.c_int
    lib.ssd_status_str.argtypes = [ctypes.c_int]
    lib.ssd_status_str.restype = ctypes.c_char_p
    lib.ssd_last_error.argtypes = []
    lib.ssd_last_error.restype = ctypes.c_char_p
    lib.ssd_version.argtypes = []
    lib.ssd_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def check(status: int):
    if status != SSD_OK:
        raise SSDError(status, load().ssd_last_error().decode())


def fwd_desc(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
             algo=SSD_ALGO_AUTO, seg_chunks=0, wg_units=0) -> FwdDesc:
    return FwdDesc(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, algo,
                   seg_chunks, wg_units, 0)
