"""ctypes binding of libcpattn (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
only turns torch tensors into device pointers, host metadata into int32 arrays,
and status codes into exceptions.  PyTorch provides device memory and the
current HIP stream.  If the library is not built the calls raise: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p
from typing import Optional, Tuple

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpattn.so")

# Status codes (include/cpattn.h).
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
BF16, FP32 = 0, 1

# Every symbol include/cpattn.h declares.
EXPORTED = ("cpattn_workspace_size", "cpattn_fwd_chunk", "cpattn_merge", "cpattn_status_string",
            "cpattn_last_error", "cpattn_plan_build")


class CpattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"cpattn status {status}: {message}")
        self.status = status


class PlanEntry(ctypes.Structure):
    _fields_ = [(name, c_int32) for name in
                ("row0", "nrows", "k_start", "k_len", "delta", "cost", "seq", "tblock")]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_entries", c_int32), ("n_tiles", c_int32), ("tokens_per_tile", c_int32),
                ("heads_per_tile", c_int32), ("head_groups", c_int32), ("block_n", c_int32),
                ("visible_pairs", c_int64), ("key_blocks", c_int64), ("plan_bytes", c_size_t)]


PLAN_DTYPE = np.dtype([(name, np.int32) for name, _ in PlanEntry._fields_])

_lib = None
_I32P = POINTER(c_int32)


def load(path: str = LIB_PATH):
    """Load libcpattn.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m context_ring_attention_amd.build`")
    lib = ctypes.CDLL(path)
    lib.cpattn_workspace_size.restype = c_size_t
    lib.cpattn_workspace_size.argtypes = [c_int32, _I32P, c_int32, c_int32, c_int32]
    lib.cpattn_fwd_chunk.restype = c_int
    lib.cpattn_fwd_chunk.argtypes = [c_void_p, c_void_p, c_void_p, _I32P, _I32P, _I32P, _I32P,
                                     c_int32, c_int32, c_int32, c_int32, c_int, c_int32,
                                     c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.cpattn_merge.restype = c_int
    lib.cpattn_merge.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_int32,
                                 c_void_p]
    lib.cpattn_status_string.restype = c_char_p
    lib.cpattn_status_string.argtypes = [c_int]
    lib.cpattn_last_error.restype = c_char_p
    lib.cpattn_last_error.argtypes = []
    lib.cpattn_plan_build.restype = c_int
    lib.cpattn_plan_build.argtypes = [_I32P, _I32P, _I32P, _I32P, c_int32, c_int32, c_int32,
                                      c_int32, c_int, c_int32, c_void_p, c_size_t,
                                      POINTER(PlanInfo)]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != OK:
        lib = load()
        msg = lib.cpattn_last_error().decode() or lib.cpattn_status_string(status).decode()
        raise CpattnError(status, msg)


def _host_i32(a, n: Optional[int] = None, name: str = "array"):
    """Host int32 copy of metadata (numpy, list or CPU tensor); None stays None."""
    if a is None:
        return None, None
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    arr = np.ascontiguousarray(np.asarray(a), dtype=np.int32)
    if n is not None and arr.shape != (n,):
        raise ValueError(f"{name} must have shape ({n},), got {arr.shape}")
    return arr, arr.ctypes.data_as(_I32P)


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def cpattn_workspace_size(nseq: int, cu_seqlens_q, hq: int, hkv: int, d: int) -> int:
    arr, ptr = _host_i32(cu_seqlens_q, nseq + 1, "cu_seqlens_q")
    return int(load().cpattn_workspace_size(nseq, ptr, hq, hkv, d))


def cpattn_plan_build(cu_seqlens_q, cu_seqlens_k, q_pos_offset=None, k_pos_offset=None, *,
                      hq: int, hkv: int, d: int, dtype: int = BF16, causal: bool = True):
    """Host-only plan: (entries as a numpy structured array, info dict)."""
    cq, pq = _host_i32(cu_seqlens_q, None, "cu_seqlens_q")
    nseq = len(cq) - 1
    ck, pk = _host_i32(cu_seqlens_k, nseq + 1, "cu_seqlens_k")
    qo, pqo = _host_i32(q_pos_offset, nseq, "q_pos_offset")
    ko, pko = _host_i32(k_pos_offset, nseq, "k_pos_offset")
    lib = load()
    info = PlanInfo()
    _check(lib.cpattn_plan_build(pq, pk, pqo, pko, nseq, hq, hkv, d, dtype, int(causal), None, 0,
                                 ctypes.byref(info)))
    entries = np.zeros(info.n_entries, dtype=PLAN_DTYPE)
    _check(lib.cpattn_plan_build(pq, pk, pqo, pko, nseq, hq, hkv, d, dtype, int(causal),
                                 c_void_p(entries.ctypes.data), entries.nbytes, ctypes.byref(info)))
    return entries, {name: getattr(info, name) for name, _ in PlanInfo._fields_}


def cpattn_fwd_chunk(q, k, v, cu_seqlens_q, cu_seqlens_k, q_pos_offset=None, k_pos_offset=None,
                     causal: bool = True, out=None, lse=None, workspace=None,
                     stream=None) -> Tuple["object", "object"]:
    """One KV chunk -> (O [Tq, Hq, D] fp32, LSE [Hq, Tq] fp32), asynchronously on the stream.

    q [Tq, Hq, D], k/v [Tk, Hkv, D]: contiguous CUDA tensors, bfloat16 or float32.
    cu_seqlens_*, *_pos_offset: host metadata (numpy / list / CPU tensor), int32.
    """
    import torch
    lib = load()
    cq, pq = _host_i32(cu_seqlens_q, None, "cu_seqlens_q")
    nseq = len(cq) - 1
    ck, pk = _host_i32(cu_seqlens_k, nseq + 1, "cu_seqlens_k")
    qo, pqo = _host_i32(q_pos_offset, nseq, "q_pos_offset")
    ko, pko = _host_i32(k_pos_offset, nseq, "k_pos_offset")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [T, H, D]")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    tq, hq, d = q.shape
    tk, hkv, dk = k.shape
    if v.shape != k.shape or dk != d:
        raise ValueError("k and v must be [Tk, Hkv, D] with Q's D")
    if int(cq[-1]) != tq or int(ck[-1]) != tk:
        raise ValueError("cu_seqlens must end at the row counts of q and k")
    if out is None:
        out = torch.empty((tq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    if out.shape != (tq, hq, d) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [Tq, Hq, D] tensor")
    if lse.shape != (hq, tq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [Hq, Tq] tensor")
    need = lib.cpattn_workspace_size(nseq, pq, hq, hkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib.cpattn_fwd_chunk(c_void_p(q.data_ptr()), c_void_p(k.data_ptr()),
                                c_void_p(v.data_ptr()), pq, pk, pqo, pko, nseq, hq, hkv, d, dt,
                                int(causal), c_void_p(out.data_ptr()), c_void_p(lse.data_ptr()),
                                c_void_p(workspace.data_ptr()), workspace.numel(),
                                _stream_handle(stream)))
    return out, lse


def cpattn_merge(o_a, lse_a, o_b, lse_b, stream=None) -> None:
    """In place: (o_a, lse_a) <- merge((o_a, lse_a), (o_b, lse_b)).  fp32 CUDA tensors."""
    import torch
    lib = load()
    if o_a.dim() != 3 or o_a.shape != o_b.shape:
        raise ValueError("o_a and o_b must both be [T, H, D]")
    t, hq, d = o_a.shape
    for name, x, shp in (("o_a", o_a, (t, hq, d)), ("o_b", o_b, (t, hq, d)),
                         ("lse_a", lse_a, (hq, t)), ("lse_b", lse_b, (hq, t))):
        if (not x.is_cuda or x.dtype != torch.float32 or not x.is_contiguous()
                or tuple(x.shape) != shp):
            raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of shape {shp}")
    _check(lib.cpattn_merge(c_void_p(o_a.data_ptr()), c_void_p(lse_a.data_ptr()),
                            c_void_p(o_b.data_ptr()), c_void_p(lse_b.data_ptr()), t, hq, d,
                            _stream_handle(stream)))
