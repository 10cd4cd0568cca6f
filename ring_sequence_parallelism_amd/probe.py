"""ctypes binding of librba_probe.so (include/rba_probe.h): the dense bf16
MFMA loop and the plain HBM copy the benchmark times to measure the chip's
sustained ceilings.  Argument marshalling only; torch supplies device
memory and the current stream."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .rba import RbaError, _ptr, _stream

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librba_probe.so")
EXPORTS = ("rba_probe_mfma_bf16", "rba_probe_copy")

_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"probe library not built: {path} is missing "
                           "(run `python -m ring_sequence_parallelism_amd.build`)")
    lib = ctypes.CDLL(path)
    I32, I64, P = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.rba_probe_mfma_bf16.argtypes = [I32, I32, P, ctypes.POINTER(ctypes.c_double), P]
    lib.rba_probe_copy.argtypes = [P, P, I64, I32, P]
    for fn in EXPORTS:
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def rba_probe_mfma_bf16(workgroups: int, iters: int, out: torch.Tensor, stream=None) -> float:
    """Launches the MFMA loop; returns the flops of the launch."""
    fl = ctypes.c_double(0.0)
    rc = load().rba_probe_mfma_bf16(int(workgroups), int(iters), _ptr(out), ctypes.byref(fl), _stream(stream))
    if rc < 0:
        raise RbaError("rba_probe_mfma_bf16", rc, "invalid arguments or launch failure")
    return fl.value


def rba_probe_copy(src: torch.Tensor, dst: torch.Tensor, nbytes: int, workgroups: int, stream=None) -> None:
    rc = load().rba_probe_copy(_ptr(src), _ptr(dst), int(nbytes), int(workgroups), _stream(stream))
    if rc < 0:
        raise RbaError("rba_probe_copy", rc, "invalid arguments or launch failure")
