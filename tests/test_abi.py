"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects bad arguments on the CPU before any HIP call (so these
run without a GPU and never launch a kernel: every call here fails
validation or is host-only)."""
import ctypes
import os
import re

import pytest

from ssd_chunked_scan_chunk_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_symbols():
    hdr = open(os.path.join(ROOT, "include", "ssd.h")).read()
    return sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", hdr)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert lib.ssd_version() >= 100


def test_status_strings(lib):
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.ssd_status_str(code).decode().startswith(name)
    assert b"unknown" in lib.ssd_status_str(99)


FAKE = ctypes.c_void_p(1 << 20)          # 16-byte aligned, never dereferenced
FAKE2 = ctypes.c_void_p(1 << 30)


def desc(**kw):
    base = dict(batch=2, seqlen=512, nheads=4, headdim=64, dstate=128, ngroups=1, chunk=256,
                dtype=_lib.SSD_BF16)
    base.update(kw)
    return _lib.fwd_desc(**base)


def fwd(lib, d, X=FAKE, a=FAKE, B=FAKE, C=FAKE, S0=None, Y=FAKE2, fin=None, ws=None, wsz=0):
    return lib.ssd_chunk_scan_fwd(ctypes.byref(d), X, a, B, C, S0, Y, fin, ws, wsz, None)


@pytest.mark.parametrize("kw,code", [
    (dict(nheads=6, ngroups=4), _lib.SSD_ERR_SHAPE),
    (dict(chunk=0), _lib.SSD_ERR_SHAPE),
    (dict(batch=-1), _lib.SSD_ERR_SHAPE),
    (dict(seqlen=-5), _lib.SSD_ERR_SHAPE),
    (dict(headdim=0), _lib.SSD_ERR_SHAPE),
    (dict(dtype=7), _lib.SSD_ERR_DTYPE),
    (dict(chunk=300), _lib.SSD_ERR_UNSUPPORTED),
    (dict(headdim=128, dstate=256), _lib.SSD_ERR_UNSUPPORTED),
])
def test_fwd_rejects_bad_shapes(lib, kw, code):
    assert fwd(lib, desc(**kw)) == code
    assert lib.ssd_last_error() != b""


def test_fwd_rejects_nulls_alignment_alias_workspace(lib):
    d = desc()
    assert fwd(lib, d, X=None) == _lib.SSD_ERR_NULL
    assert fwd(lib, d, Y=None) == _lib.SSD_ERR_NULL
    assert fwd(lib, d, X=ctypes.c_void_p((1 << 20) + 2)) == _lib.SSD_ERR_ALIGN
    # Y overlapping X
    assert fwd(lib, d, Y=FAKE) == _lib.SSD_ERR_ALIAS
    # a plan with several segments needs a workspace
    d2 = desc(batch=1, seqlen=16384, nheads=2, headdim=64, dstate=64)
    n = ctypes.c_size_t()
    assert lib.ssd_fwd_workspace_bytes(ctypes.byref(d2), ctypes.byref(n)) == 0
    assert n.value > 0
    assert fwd(lib, d2) == _lib.SSD_ERR_WORKSPACE
    assert fwd(lib, d2, ws=ctypes.c_void_p(1 << 34), wsz=n.value - 1) == _lib.SSD_ERR_WORKSPACE
    # forcing the MFMA path on fp32 or an uncompiled shape
    assert fwd(lib, desc(dtype=_lib.SSD_F32, algo=_lib.SSD_ALGO_MFMA)) == _lib.SSD_ERR_UNSUPPORTED
    assert fwd(lib, desc(headdim=48, algo=_lib.SSD_ALGO_MFMA)) == _lib.SSD_ERR_UNSUPPORTED


def plan(lib, d, units=False):
    a, k, n, u = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    assert lib.ssd_fwd_plan(ctypes.byref(d), ctypes.byref(a), ctypes.byref(k), ctypes.byref(n),
                            ctypes.byref(u)) == 0
    return (a.value, k.value, n.value, u.value) if units else (a.value, k.value, n.value)


def test_plans(lib):
    # fp32 -> VALU; bf16 compiled shapes -> MFMA with a balanced segment plan
    assert plan(lib, desc(dtype=_lib.SSD_F32))[0] == _lib.SSD_ALGO_VALU
    assert plan(lib, desc(headdim=16, dstate=16))[0] == _lib.SSD_ALGO_VALU
    a, k, n = plan(lib, desc(batch=64, seqlen=4096, nheads=80))
    assert (a, k, n) == (_lib.SSD_ALGO_MFMA, 16, 1)      # 1280 head quads fill the GPU
    a, k, n = plan(lib, desc(batch=8, seqlen=4096, nheads=80))
    assert a == _lib.SSD_ALGO_MFMA and k * n >= 16 and k * (n - 1) < 16
    a, k, n = plan(lib, desc(batch=1, seqlen=524288, nheads=32, dstate=64))
    assert a == _lib.SSD_ALGO_MFMA and n > 1 and k * n >= 2048
    a, k, n = plan(lib, desc(seg_chunks=3, seqlen=256 * 10))
    assert (k, n) == (3, 4)
    # the 2.7B-shaped layer: 8 x 80 x 2 = 1280 units in 256 workgroups of five, one segment
    assert plan(lib, desc(batch=8, seqlen=4096, nheads=80), units=True) == (_lib.SSD_ALGO_MFMA, 16, 1, 5)
    # long sequences: segments of at most 16K steps
    assert plan(lib, desc(batch=1, seqlen=524288, nheads=32, dstate=64))[1] * 256 <= 16384
    # a forced split is honoured; others are rejected on the host
    assert plan(lib, desc(wg_units=4), units=True)[3] == 4
    assert plan(lib, desc(wg_units=6, seg_chunks=1), units=True)[1:] == (1, 2, 6)
    for bad in (1, 3, 7):
        assert fwd(lib, desc(wg_units=bad)) == _lib.SSD_ERR_UNSUPPORTED
    assert plan(lib, desc(dtype=_lib.SSD_F32), units=True)[3] == 0
    # workspace is zero for a single segment
    n0 = ctypes.c_size_t(123)
    assert lib.ssd_fwd_workspace_bytes(ctypes.byref(desc(batch=64, seqlen=4096, nheads=80)), ctypes.byref(n0)) == 0
    assert n0.value == 0


def test_step_validation(lib):
    def st(**kw):
        base = dict(batch=4, nheads=8, headdim=64, dstate=128, ngroups=1, dtype=_lib.SSD_BF16, reserved=0)
        base.update(kw)
        return _lib.StepDesc(**base)
    F = [ctypes.c_void_p(1 << k) for k in (20, 24, 26, 28, 30, 32)]
    call = lambda d, *p: lib.ssd_step(ctypes.byref(d), *p, None)
    assert call(st(nheads=6, ngroups=4), *F) == _lib.SSD_ERR_SHAPE
    assert call(st(dtype=9), *F) == _lib.SSD_ERR_DTYPE
    assert call(st(reserved=1), *F) == _lib.SSD_ERR_SHAPE
    # 2^20 (b, h) slices of 64 x 128: 2^31 threads of 4 state elements is fine,
    # 2^22 slices would need 2^33 threads in one launch
    assert call(st(batch=1 << 14, nheads=64), None, *F[1:]) == _lib.SSD_ERR_NULL
    assert call(st(batch=1 << 16, nheads=64), *F) == _lib.SSD_ERR_UNSUPPORTED
    assert call(st(), None, *F[1:]) == _lib.SSD_ERR_NULL
    assert call(st(), ctypes.c_void_p((1 << 20) + 4), *F[1:]) == _lib.SSD_ERR_ALIGN
    assert call(st(), F[0], F[1], F[2], F[3], F[4], F[0]) == _lib.SSD_ERR_ALIAS


def test_stream_rmw_validation(lib):
    call = lambda *a: lib.ssd_stream_rmw(*a, None)
    p = ctypes.c_void_p(1 << 20)
    assert call(p, 6, 1.0, 8, 1) == _lib.SSD_ERR_SHAPE            # n not a multiple of 4
    assert call(p, -4, 1.0, 8, 1) == _lib.SSD_ERR_SHAPE
    assert call(p, 64, 1.0, 3, 1) == _lib.SSD_ERR_UNSUPPORTED     # per_thread not in {1,2,4,8}
    assert call(p, 64, 1.0, 8, 2) == _lib.SSD_ERR_SHAPE           # nontemporal not 0/1
    assert call(None, 64, 1.0, 8, 1) == _lib.SSD_ERR_NULL
    assert call(ctypes.c_void_p((1 << 20) + 4), 64, 1.0, 8, 1) == _lib.SSD_ERR_ALIGN
    assert call(None, 0, 1.0, 8, 1) == _lib.SSD_OK                # empty: nothing to do
    assert call(p, 4 << 32, 1.0, 1, 1) == _lib.SSD_ERR_UNSUPPORTED  # 2^32 float4: too many threads


def test_stage_validation(lib):
    d = desc(dtype=_lib.SSD_F32)
    # stage kernels 2/3/5 are the bf16 MFMA building blocks
    assert lib.ssd_chunk_state(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE2, None) == _lib.SSD_ERR_UNSUPPORTED
    assert lib.ssd_chunk_scan(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE2, None) == _lib.SSD_ERR_UNSUPPORTED
    assert lib.ssd_chunk_cumsum(ctypes.byref(desc(chunk=512)), FAKE, FAKE2, FAKE2, None) == _lib.SSD_ERR_UNSUPPORTED
    assert lib.ssd_chunk_cumsum(ctypes.byref(desc()), None, FAKE2, FAKE2, None) == _lib.SSD_ERR_NULL
    assert lib.ssd_state_passing(ctypes.byref(desc()), FAKE, FAKE, None, None, None, None) == _lib.SSD_ERR_NULL


def bwd(lib, d, X=FAKE, a=FAKE, B=FAKE, C=FAKE, S0=None, dY=FAKE, dSf=None, dX=FAKE2, da=None,
        dB=None, dC=None, dS0=None, ws=None, wsz=0):
    da = da if da is not None else ctypes.c_void_p((1 << 30) + (1 << 26))
    dB = dB if dB is not None else ctypes.c_void_p((1 << 30) + (2 << 26))
    dC = dC if dC is not None else ctypes.c_void_p((1 << 30) + (3 << 26))
    return lib.ssd_chunk_scan_bwd(ctypes.byref(d), X, a, B, C, S0, dY, dSf, dX, da, dB, dC, dS0,
                                  ws, wsz, None)


def test_bwd_validation(lib):
    n = ctypes.c_size_t()
    d = desc()
    assert lib.ssd_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    # per-chunk forward and adjoint states at least
    assert n.value >= 2 * 2 * 2 * 4 * 64 * 128 * 4
    # the MFMA path forced on fp32, the VALU path forced on bf16, shapes without
    # kernels are rejected on the host; fp32 itself is planned (VALU kernels)
    nf = ctypes.c_size_t()
    assert lib.ssd_bwd_workspace_bytes(ctypes.byref(desc(dtype=_lib.SSD_F32)), ctypes.byref(nf)) == 0
    for kw in (dict(dtype=_lib.SSD_F32, algo=_lib.SSD_ALGO_MFMA), dict(algo=_lib.SSD_ALGO_VALU),
               dict(headdim=48), dict(chunk=32), dict(dstate=32), dict(dtype=_lib.SSD_F32, chunk=512),
               dict(dtype=_lib.SSD_F32, headdim=3, nheads=3)):
        assert lib.ssd_bwd_workspace_bytes(ctypes.byref(desc(**kw)), ctypes.byref(n)) == _lib.SSD_ERR_UNSUPPORTED
        assert bwd(lib, desc(**kw)) == _lib.SSD_ERR_UNSUPPORTED
    assert bwd(lib, desc(nheads=6, ngroups=4)) == _lib.SSD_ERR_SHAPE
    assert bwd(lib, d, dY=None) == _lib.SSD_ERR_NULL
    assert bwd(lib, d, dX=ctypes.c_void_p((1 << 30) + 8)) == _lib.SSD_ERR_ALIGN
    # a workspace is required, and outputs may not overlap inputs, each other or it
    assert bwd(lib, d) == _lib.SSD_ERR_WORKSPACE
    ws = ctypes.c_void_p(1 << 36)
    assert lib.ssd_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    assert bwd(lib, d, ws=ws, wsz=n.value - 1) == _lib.SSD_ERR_WORKSPACE
    lib.ssd_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(n))
    assert bwd(lib, d, dX=FAKE, ws=ws, wsz=n.value) == _lib.SSD_ERR_ALIAS
    assert bwd(lib, d, dB=FAKE2, ws=ws, wsz=n.value) == _lib.SSD_ERR_ALIAS
    assert bwd(lib, d, dC=ws, ws=ws, wsz=n.value) == _lib.SSD_ERR_ALIAS
    # an empty batch is a no-op that needs nothing
    assert lib.ssd_bwd_workspace_bytes(ctypes.byref(desc(batch=0)), ctypes.byref(n)) == 0 and n.value == 0
    assert bwd(lib, desc(batch=0), X=None, dY=None) == 0


def test_bwd_da_stage_validation(lib):
    n = ctypes.c_size_t()
    assert lib.ssd_bwd_da_workspace_bytes(ctypes.byref(desc()), ctypes.byref(n)) == 0
    assert n.value == 2 * 2 * 1 * 36 * 32 * 32 * 4    # batch x chunks x groups x 8*9/2 tiles of 32x32 fp32
    WS = ctypes.c_void_p(1 << 38)
    call = lambda d, *p, ws=WS, wsz=n.value: lib.ssd_bwd_da(ctypes.byref(d), *p, ws, wsz, None)
    F = [ctypes.c_void_p(1 << k) for k in (20, 24, 26, 28, 30, 32, 34)]
    out = ctypes.c_void_p(1 << 36)
    assert call(desc(dtype=_lib.SSD_F32), *F, out) == _lib.SSD_ERR_UNSUPPORTED
    assert call(desc(chunk=32), *F, out) == _lib.SSD_ERR_UNSUPPORTED
    assert call(desc(), None, *F[1:], out) == _lib.SSD_ERR_NULL
    assert call(desc(), *F, None) == _lib.SSD_ERR_NULL
    assert call(desc(), *F[:5], ctypes.c_void_p((1 << 32) + 8), F[6], out) == _lib.SSD_ERR_ALIGN
    assert call(desc(), *F, F[6]) == _lib.SSD_ERR_ALIAS
    # the workspace: missing, too small, misaligned, overlapping an input or da
    assert call(desc(), *F, out, ws=None) == _lib.SSD_ERR_WORKSPACE
    assert call(desc(), *F, out, wsz=n.value - 1) == _lib.SSD_ERR_WORKSPACE
    assert call(desc(), *F, out, ws=ctypes.c_void_p((1 << 38) + 8)) == _lib.SSD_ERR_ALIGN
    assert call(desc(), *F, out, ws=F[3]) == _lib.SSD_ERR_ALIAS
    assert call(desc(), *F, out, ws=out) == _lib.SSD_ERR_ALIAS
    assert call(desc(batch=0), None, None, None, None, None, None, None, None, ws=None, wsz=0) == 0
    assert lib.ssd_bwd_da_workspace_bytes(ctypes.byref(desc(dtype=_lib.SSD_F32)),
                                          ctypes.byref(n)) == _lib.SSD_ERR_UNSUPPORTED
    # other chunk lengths and groups: T = chunk/32 row tiles give T(T+1)/2 tiles per (batch, chunk, group);
    # a ragged last chunk counts whole
    for kw, tiles, chunks, groups in ((dict(chunk=64, seqlen=300), 3, 5, 1),
                                      (dict(chunk=128, ngroups=2, seqlen=512), 10, 4, 2),
                                      (dict(batch=3, seqlen=257), 36, 2, 1)):
        assert lib.ssd_bwd_da_workspace_bytes(ctypes.byref(desc(**kw)), ctypes.byref(n)) == 0
        assert n.value == kw.get("batch", 2) * chunks * groups * tiles * 32 * 32 * 4, (kw, n.value)
    # the whole backward's workspace holds the same tiles among its regions
    nb = ctypes.c_size_t()
    assert lib.ssd_bwd_workspace_bytes(ctypes.byref(desc()), ctypes.byref(nb)) == 0
    assert nb.value >= 2 * 2 * 1 * 36 * 32 * 32 * 4
