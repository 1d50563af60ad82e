"""Binding of libkvc_probe.so: a plain streaming-read probe of HBM bandwidth.

Not part of the decode path.  ``stream_read`` launches the probe kernel once
on torch's current stream; the benchmark times it with HIP events.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc_probe.so")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkvc_probe.so is not built (%s); run "
                              "`python -m kv_cached_decode_kvc_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.kvc_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        L.kvc_probe_stream_read.restype = ctypes.c_int
        _lib = L
    return _lib


def stream_read(src: torch.Tensor, nontemporal: bool, workgroups: int, sink: torch.Tensor):
    """Read all of ``src`` (a contiguous device tensor) once."""
    assert src.is_cuda and src.is_contiguous() and sink.is_cuda
    st = lib().kvc_probe_stream_read(
        ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(), int(nontemporal),
        int(workgroups), ctypes.c_void_p(sink.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise RuntimeError("kvc_probe_stream_read failed: %d" % st)
