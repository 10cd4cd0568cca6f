"""Python binding of the ring block-attention C ABI (include/rba.h).

Argument marshalling only: every function forwards to the entry point of the
same name in librba.so, passing device pointers of torch tensors and the
current torch stream.  Nothing here computes any part of the attention.
Loading fails loudly when the library has not been built.

torch must be imported before the library is loaded so that the library
binds to the HIP runtime torch already mapped (the loader matches the
runtime's soname); :func:`load` verifies that exactly one HIP runtime is
mapped into the process.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

RBA_OK, RBA_STEP_EMPTY = 0, 1
RBA_ERR_INVALID, RBA_ERR_UNSUPPORTED, RBA_ERR_ALIGNMENT, RBA_ERR_HIP = -1, -2, -3, -4
RBA_BF16, RBA_F32 = 0, 1
RBA_MASK_NONE, RBA_MASK_CAUSAL, RBA_MASK_DOC_CAUSAL = 0, 1, 2
RBA_MAX_SEGS = 16

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librba.so")

EXPORTS = ("rba_fwd_step", "rba_fwd_step_acc", "rba_merge", "rba_bwd_preprocess", "rba_bwd_step", "rba_bwd_step_acc",
           "rba_plan_step", "rba_step_full_tiles", "rba_merge_layout", "rba_fwd_step_ws", "rba_fwd_workspace_size",
           "rba_fwd_step_noalloc", "rba_last_error", "rba_version")


class RbaError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


class rba_segs(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32),
                ("start", ctypes.c_int64 * RBA_MAX_SEGS),
                ("len", ctypes.c_int64 * RBA_MAX_SEGS),
                ("stride", ctypes.c_int64 * RBA_MAX_SEGS)]


class rba_attn(ctypes.Structure):
    _fields_ = [("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int), ("mask", ctypes.c_int),
                ("cu_seqlens_dev", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
                ("n_docs", ctypes.c_int32)]


def make_segs(segments: Sequence[Tuple[int, ...]]) -> rba_segs:
    """[(start, length) or (start, length, stride), ...] in row order -> rba_segs
    (stride 1 when omitted)."""
    s = rba_segs()
    if len(segments) > RBA_MAX_SEGS:
        raise ValueError(f"at most {RBA_MAX_SEGS} segments")
    s.n = len(segments)
    for i, seg in enumerate(segments):
        s.start[i] = int(seg[0])
        s.len[i] = int(seg[1])
        s.stride[i] = int(seg[2]) if len(seg) > 2 else 1
    return s


_lib = None


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({l.split()[-1] for l in f if "libamdhip64" in l})
    except OSError:
        return []


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load librba.so once; raises if it is missing or a second HIP runtime got mapped."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("RBA_LIB", LIB_PATH)
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run `python -m ring_sequence_parallelism_amd.build`)")
    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes mapped into the process: {runtimes}")
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    A, S = ctypes.POINTER(rba_attn), ctypes.POINTER(rba_segs)
    lib.rba_fwd_step.argtypes = [A, P, I64, S, P, P, I64, S, P, P, P]
    lib.rba_fwd_step_acc.argtypes = [A, P, I64, S, P, P, I64, S, P, P, P, I32, P]
    lib.rba_merge.argtypes = [I64, I32, I32, P, P, P, P, P, I32, P]
    lib.rba_bwd_preprocess.argtypes = [I64, I32, I32, I32, I32, P, P, P, P]
    lib.rba_bwd_step.argtypes = [A, P, I64, S, P, P, I64, S, P, P, P, P, P, P, P]
    lib.rba_bwd_step_acc.argtypes = [A, P, I64, S, P, P, I64, S, P, P, P, P, P, P, P]
    lib.rba_plan_step.argtypes = [A, I64, S, I64, S, ctypes.POINTER(I64)]
    lib.rba_step_full_tiles.argtypes = [A, I64, S, I64, S, ctypes.POINTER(I32), ctypes.POINTER(I32)]
    lib.rba_merge_layout.argtypes = [I32, ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32)]
    lib.rba_fwd_step_ws.argtypes = [A, P, I64, S, P, P, I64, S, P, P, I32, P, I32, P, I64, P]
    lib.rba_fwd_workspace_size.argtypes = [A, I64, S, I64, S, ctypes.POINTER(I64)]
    lib.rba_fwd_step_noalloc.argtypes = [A, P, I64, S, P, P, I64, S, P, P, I32, P, I32, P]
    for fn in ("rba_fwd_step", "rba_fwd_step_acc", "rba_merge", "rba_bwd_preprocess", "rba_bwd_step", "rba_bwd_step_acc",
               "rba_plan_step", "rba_step_full_tiles", "rba_merge_layout", "rba_fwd_step_ws", "rba_fwd_workspace_size",
               "rba_fwd_step_noalloc"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.rba_last_error.restype = ctypes.c_char_p
    lib.rba_last_error.argtypes = []
    lib.rba_version.restype = ctypes.c_char_p
    lib.rba_version.argtypes = []
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, rc: int) -> int:
    if rc < 0:
        raise RbaError(fn, rc, load().rba_last_error().decode())
    return rc


def attn_params(hq: int, hkv: int, d: int, scale: float, dtype: int, mask: int,
                cu_seqlens_dev: Optional[torch.Tensor] = None, cu_seqlens_host=None) -> rba_attn:
    """Build an rba_attn.  Both cu_seqlens arrays are kept alive on the struct."""
    a = rba_attn()
    a.hq, a.hkv, a.d, a.scale, a.dtype, a.mask = hq, hkv, d, scale, dtype, mask
    a.cu_seqlens_dev = None if cu_seqlens_dev is None else cu_seqlens_dev.data_ptr()
    a._cu_dev_keepalive = cu_seqlens_dev   # the struct holds a raw pointer into it
    a.n_docs = 0
    if cu_seqlens_host is not None:
        import numpy as np
        host = np.ascontiguousarray(cu_seqlens_host, dtype=np.int32)
        a._cu_keepalive = host
        a.cu_seqlens_host = host.ctypes.data
        a.n_docs = len(host) - 1
    elif cu_seqlens_dev is not None:
        a.n_docs = cu_seqlens_dev.numel() - 1
    return a


def rba_fwd_step(a: rba_attn, q, q_segs: rba_segs, k, v, kv_segs: rba_segs,
                 o_part, lse_part, stream=None) -> int:
    return _check("rba_fwd_step", load().rba_fwd_step(
        ctypes.byref(a), _ptr(q), q.shape[0], ctypes.byref(q_segs), _ptr(k), _ptr(v), k.shape[0],
        ctypes.byref(kv_segs), _ptr(o_part), _ptr(lse_part), _stream(stream)))


def rba_fwd_step_acc(a: rba_attn, q, q_segs: rba_segs, k, v, kv_segs: rba_segs, o_acc, lse_acc,
                     o_final=None, final_dtype: int = RBA_BF16, stream=None) -> int:
    return _check("rba_fwd_step_acc", load().rba_fwd_step_acc(
        ctypes.byref(a), _ptr(q), q.shape[0], ctypes.byref(q_segs), _ptr(k), _ptr(v), k.shape[0],
        ctypes.byref(kv_segs), _ptr(o_acc), _ptr(lse_acc), _ptr(o_final), final_dtype, _stream(stream)))


def rba_fwd_step_ws(a: rba_attn, q, q_segs: rba_segs, k, v, kv_segs: rba_segs, o, lse, accumulate: bool,
                    o_final=None, final_dtype: int = RBA_BF16, workspace=None, stream=None) -> int:
    """workspace: a device tensor (its byte size is passed) or None."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _check("rba_fwd_step_ws", load().rba_fwd_step_ws(
        ctypes.byref(a), _ptr(q), q.shape[0], ctypes.byref(q_segs), _ptr(k), _ptr(v), k.shape[0],
        ctypes.byref(kv_segs), _ptr(o), _ptr(lse), 1 if accumulate else 0, _ptr(o_final), final_dtype,
        _ptr(workspace), ws_bytes, _stream(stream)))


def rba_fwd_step_noalloc(a: rba_attn, q, q_segs: rba_segs, k, v, kv_segs: rba_segs, o, lse, accumulate: bool,
                         o_final=None, final_dtype: int = RBA_BF16, stream=None) -> int:
    """rba_fwd_step_ws with the library's per-device workspace array."""
    return _check("rba_fwd_step_noalloc", load().rba_fwd_step_noalloc(
        ctypes.byref(a), _ptr(q), q.shape[0], ctypes.byref(q_segs), _ptr(k), _ptr(v), k.shape[0],
        ctypes.byref(kv_segs), _ptr(o), _ptr(lse), 1 if accumulate else 0, _ptr(o_final), final_dtype,
        _stream(stream)))


def rba_fwd_workspace_size(a: rba_attn, sq: int, q_segs: rba_segs, sk: int, kv_segs: rba_segs) -> int:
    """Workspace bytes rba_fwd_step_ws would use for the step (0: no split)."""
    n = ctypes.c_int64(0)
    _check("rba_fwd_workspace_size", load().rba_fwd_workspace_size(
        ctypes.byref(a), sq, ctypes.byref(q_segs), sk, ctypes.byref(kv_segs), ctypes.byref(n)))
    return n.value


def rba_merge(o_acc, lse_acc, o_part=None, lse_part=None, o_final=None, final_dtype: int = RBA_BF16,
              stream=None) -> int:
    sq, hq, d = o_acc.shape
    return _check("rba_merge", load().rba_merge(
        sq, hq, d, _ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part), _ptr(o_final),
        final_dtype, _stream(stream)))


def _dtype_of(t) -> int:
    if t.dtype == torch.bfloat16:
        return RBA_BF16
    if t.dtype == torch.float32:
        return RBA_F32
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def rba_bwd_preprocess(o, d_o, delta, stream=None) -> int:
    sq, hq, d = o.shape
    return _check("rba_bwd_preprocess", load().rba_bwd_preprocess(
        sq, hq, d, _dtype_of(o), _dtype_of(d_o), _ptr(o), _ptr(d_o), _ptr(delta), _stream(stream)))


def rba_bwd_step(a: rba_attn, q, q_segs: rba_segs, k, v, kv_segs: rba_segs, d_o, lse, delta,
                 dq_acc, dk_step, dv_step, stream=None) -> int:
    return _check("rba_bwd_step", load().rba_bwd_step(
        ctypes.byref(a), _ptr(q), q.shape[0], ctypes.byref(q_segs), _ptr(k), _ptr(v), k.shape[0],
        ctypes.byref(kv_segs), _ptr(d_o), _ptr(lse), _ptr(delta), _ptr(dq_acc), _ptr(dk_step),
        _ptr(dv_step), _stream(stream)))


def rba_bwd_step_acc(a: rba_attn, q, q_segs: rba_segs, k, v, kv_segs: rba_segs, d_o, lse, delta,
                     dq_acc, dk_acc, dv_acc, stream=None) -> int:
    return _check("rba_bwd_step_acc", load().rba_bwd_step_acc(
        ctypes.byref(a), _ptr(q), q.shape[0], ctypes.byref(q_segs), _ptr(k), _ptr(v), k.shape[0],
        ctypes.byref(kv_segs), _ptr(d_o), _ptr(lse), _ptr(delta), _ptr(dq_acc), _ptr(dk_acc),
        _ptr(dv_acc), _stream(stream)))


def rba_plan_step(a: rba_attn, sq: int, q_segs: rba_segs, sk: int, kv_segs: rba_segs) -> Tuple[int, int]:
    """(status, pairs per query head) — host only, no device needed."""
    pairs = ctypes.c_int64(0)
    rc = _check("rba_plan_step", load().rba_plan_step(
        ctypes.byref(a), sq, ctypes.byref(q_segs), sk, ctypes.byref(kv_segs), ctypes.byref(pairs)))
    return rc, pairs.value


def rba_step_full_tiles(a: rba_attn, sq: int, q_segs: rba_segs, sk: int, kv_segs: rba_segs) -> Tuple[int, int]:
    """(forward full, backward full) launch choices of a step — host only, no device needed."""
    f, b = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("rba_step_full_tiles", load().rba_step_full_tiles(
        ctypes.byref(a), sq, ctypes.byref(q_segs), sk, ctypes.byref(kv_segs), ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def rba_merge_layout(d: int) -> Tuple[int, int, int, int]:
    """(status, lanes per pair, vectors per lane, threads per workgroup) of
    rba_merge's thread map for head dimension d — host only.  The status is
    returned, not raised, so that rejected d can be checked."""
    lpp, vpl, tpw = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    rc = load().rba_merge_layout(int(d), ctypes.byref(lpp), ctypes.byref(vpl), ctypes.byref(tpw))
    return rc, lpp.value, vpl.value, tpw.value


def rba_version() -> str:
    return load().rba_version().decode()


def rba_last_error() -> str:
    return load().rba_last_error().decode()
