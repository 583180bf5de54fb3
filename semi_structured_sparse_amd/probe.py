"""Measurement helpers (libnmprobe.so): the streaming-read and matrix-pipe ceilings of the
machine at hand, for reporting beside the nominal peaks.  Not part of the method and not
exported by libnmsparse; only the benchmark and its tests use them."""
from __future__ import annotations

import ctypes
import os

from . import NM_OK, NMError, _ptr, _stream

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnmprobe.so")
_PLIB = None


def plib() -> ctypes.CDLL:
    global _PLIB
    if _PLIB is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with semi_structured_sparse_amd.build.build()")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        _i64, _int, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.nm_probe_sink_bytes.restype = _i64
        L.nm_probe_sink_bytes.argtypes = []
        L.nm_probe_read.restype = _int
        L.nm_probe_read.argtypes = [_vp, _i64, _vp, _int, _vp]
        L.nm_probe_mfma_flops.restype = _i64
        L.nm_probe_mfma_flops.argtypes = [_i64]
        L.nm_probe_mfma.restype = _int
        L.nm_probe_mfma.argtypes = [_i64, _vp, _vp]
        _PLIB = L
    return _PLIB


def _check(st, where):
    if st != NM_OK:
        raise NMError(st, where)


def nm_probe_sink_bytes() -> int:
    return int(plib().nm_probe_sink_bytes())


def nm_probe_read(buf, nbytes, sink, stream=None, *, mode=0, check=True):
    st = plib().nm_probe_read(_ptr(buf), nbytes, _ptr(sink), mode, _stream(stream))
    if check:
        _check(st, "nm_probe_read")
    return st


def nm_probe_mfma_flops(iters) -> int:
    return int(plib().nm_probe_mfma_flops(iters))


def nm_probe_mfma(iters, sink, stream=None, *, check=True):
    st = plib().nm_probe_mfma(iters, _ptr(sink), _stream(stream))
    if check:
        _check(st, "nm_probe_mfma")
    return st
