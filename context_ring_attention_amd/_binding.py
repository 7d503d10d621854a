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
from typing import Optional, Sequence, Tuple

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpattn.so")

# Status codes (include/cpattn.h).
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
BF16, FP32 = 0, 1

# Every symbol include/cpattn.h declares.
EXPORTED = ("cpattn_workspace_size", "cpattn_workspace_size_chunks", "cpattn_fwd_chunk",
            "cpattn_fwd_chunk_accum", "cpattn_fwd_chunks", "cpattn_bwd_chunk", "cpattn_bwd_chunks",
            "cpattn_bwd_workspace_size", "cpattn_bwd_workspace_size_chunks", "cpattn_merge",
            "cpattn_status_string",
            "cpattn_last_error", "cpattn_plan_build", "cpattn_plan_build_chunks",
            "cpattn_key_plan_build", "cpattn_dcp_schedule", "cpattn_fwd_chunks_noalloc",
            "cpattn_plan_build_device")
MAX_CHUNKS = 16  # CPATTN_MAX_CHUNKS


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
                ("visible_pairs", c_int64), ("key_blocks", c_int64), ("plan_bytes", c_size_t),
                ("n_chunks", c_int32), ("reserved", c_int32)]


PLAN_DTYPE = np.dtype([(name, np.int32) for name, _ in PlanEntry._fields_])
KEY_TILE_DTYPE = np.dtype([(name, np.int32) for name in
                           ("row0", "nrows", "q_start", "q_len", "delta", "cost", "chunk", "reserved")])


class KeyPlanInfo(ctypes.Structure):
    _fields_ = [(name, c_int32) for name in ("n_tiles", "keys_per_tile", "query_block", "reserved")]

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
    lib.cpattn_workspace_size_chunks.restype = c_size_t
    lib.cpattn_workspace_size_chunks.argtypes = [c_int32, _I32P, c_int32, c_int32, c_int32, c_int32]
    for name in ("cpattn_fwd_chunk", "cpattn_fwd_chunk_accum"):
        fn = getattr(lib, name)
        fn.restype = c_int
        fn.argtypes = [c_void_p, c_void_p, c_void_p, _I32P, _I32P, _I32P, _I32P, c_int32, c_int32,
                       c_int32, c_int32, c_int, c_int32, c_void_p, c_void_p, c_void_p, c_size_t,
                       c_void_p]
    lib.cpattn_fwd_chunks.restype = c_int
    lib.cpattn_fwd_chunks.argtypes = [c_void_p, POINTER(c_void_p), POINTER(c_void_p), c_int32,
                                      _I32P, _I32P, _I32P, _I32P, c_int32, c_int32, c_int32,
                                      c_int32, c_int, c_int32, c_int32, c_void_p, c_void_p,
                                      c_void_p, c_size_t, c_void_p]
    lib.cpattn_fwd_chunks_noalloc.restype = c_int
    lib.cpattn_fwd_chunks_noalloc.argtypes = [c_void_p, POINTER(c_void_p), POINTER(c_void_p), c_int32,
                                              _I32P, _I32P, _I32P, _I32P, c_int32, c_int32, c_int32,
                                              c_int32, c_int, c_int32, c_int32, c_void_p, c_void_p,
                                              c_void_p]
    lib.cpattn_bwd_chunk.restype = c_int
    lib.cpattn_bwd_chunk.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     _I32P, _I32P, _I32P, _I32P, c_int32, c_int32, c_int32,
                                     c_int32, c_int, c_int32, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]
    lib.cpattn_bwd_chunks.restype = c_int
    lib.cpattn_bwd_chunks.argtypes = [c_void_p, POINTER(c_void_p), POINTER(c_void_p), c_int32,
                                      c_void_p, c_void_p, c_void_p, _I32P, _I32P, _I32P, _I32P,
                                      c_int32, c_int32, c_int32, c_int32, c_int, c_int32, c_void_p,
                                      POINTER(c_void_p), POINTER(c_void_p), c_void_p, c_size_t,
                                      c_void_p]
    lib.cpattn_bwd_workspace_size.restype = c_size_t
    lib.cpattn_bwd_workspace_size.argtypes = [c_int32, _I32P, _I32P, c_int32, c_int32, c_int32]
    lib.cpattn_bwd_workspace_size_chunks.restype = c_size_t
    lib.cpattn_bwd_workspace_size_chunks.argtypes = [c_int32, _I32P, _I32P, c_int32, c_int32,
                                                     c_int32, c_int32]
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
    lib.cpattn_plan_build_chunks.restype = c_int
    lib.cpattn_plan_build_chunks.argtypes = [_I32P, _I32P, _I32P, _I32P, c_int32, c_int32, c_int32,
                                             c_int32, c_int32, c_int, c_int32, c_void_p, c_size_t,
                                             POINTER(PlanInfo)]
    lib.cpattn_key_plan_build.restype = c_int
    lib.cpattn_key_plan_build.argtypes = [_I32P, _I32P, _I32P, _I32P, c_int32, c_int32, c_int32,
                                          c_int32, c_int32, c_int32, c_void_p, c_size_t,
                                          POINTER(KeyPlanInfo)]
    lib.cpattn_plan_build_device.restype = c_int
    lib.cpattn_plan_build_device.argtypes = [_I32P, _I32P, _I32P, _I32P, c_int32, c_int32, c_int32,
                                             c_int32, c_int32, c_int, c_int32, c_void_p, c_size_t,
                                             c_void_p]
    lib.cpattn_dcp_schedule.restype = c_int
    lib.cpattn_dcp_schedule.argtypes = [_I32P, c_int32, c_int32, c_int32, _I32P, _I32P, _I32P, _I32P,
                                        _I32P]
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


def _chunk_meta(cu_seqlens_ks: Sequence, k_pos_offsets: Optional[Sequence], nseq: int):
    """Host [nchunks][nseq + 1] cu_seqlens and [nchunks][nseq] offsets (or None), int32."""
    nchunks = len(cu_seqlens_ks)
    ck = np.stack([_host_i32(c, nseq + 1, "cu_seqlens_k")[0] for c in cu_seqlens_ks]) \
        if nchunks else np.zeros((0, nseq + 1), np.int32)
    ck = np.ascontiguousarray(ck, np.int32)
    if k_pos_offsets is None or all(o is None for o in k_pos_offsets):
        return ck, None
    ko = np.stack([np.zeros(nseq, np.int32) if o is None else _host_i32(o, nseq, "k_pos_offset")[0]
                   for o in k_pos_offsets])
    return ck, np.ascontiguousarray(ko, np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_I32P)


def cpattn_plan_build_chunks(cu_seqlens_q, cu_seqlens_ks: Sequence, q_pos_offset=None,
                             k_pos_offsets: Optional[Sequence] = None, *, hq: int, hkv: int, d: int,
                             dtype: int = BF16, causal: bool = True):
    """Host-only plan over several chunks: (entries [n_tiles * nchunks], info dict)."""
    cq, pq = _host_i32(cu_seqlens_q, None, "cu_seqlens_q")
    nseq = len(cq) - 1
    qo, pqo = _host_i32(q_pos_offset, nseq, "q_pos_offset")
    ck, ko = _chunk_meta(cu_seqlens_ks, k_pos_offsets, nseq)
    lib = load()
    info = PlanInfo()
    nch = len(cu_seqlens_ks)
    _check(lib.cpattn_plan_build_chunks(pq, _ptr(ck), pqo, _ptr(ko), nch, nseq, hq, hkv, d, dtype,
                                        int(causal), None, 0, ctypes.byref(info)))
    entries = np.zeros(info.n_entries, dtype=PLAN_DTYPE)
    _check(lib.cpattn_plan_build_chunks(pq, _ptr(ck), pqo, _ptr(ko), nch, nseq, hq, hkv, d, dtype,
                                        int(causal), c_void_p(entries.ctypes.data), entries.nbytes,
                                        ctypes.byref(info)))
    return entries, {name: getattr(info, name) for name, _ in PlanInfo._fields_}


def cpattn_plan_build_device(cu_seqlens_q, cu_seqlens_ks: Sequence, q_pos_offset=None,
                             k_pos_offsets: Optional[Sequence] = None, *, hq: int, hkv: int, d: int,
                             dtype: int = BF16, causal: bool = True, stream=None):
    """The forward's plan built by the device planner, as a numpy array like
    cpattn_plan_build_chunks's entries (synchronises the stream)."""
    import torch
    cq, pq = _host_i32(cu_seqlens_q, None, "cu_seqlens_q")
    nseq = len(cq) - 1
    qo, pqo = _host_i32(q_pos_offset, nseq, "q_pos_offset")
    ck, ko = _chunk_meta(cu_seqlens_ks, k_pos_offsets, nseq)
    lib = load()
    nch = len(cu_seqlens_ks)
    info = PlanInfo()
    _check(lib.cpattn_plan_build_chunks(pq, _ptr(ck), pqo, _ptr(ko), nch, nseq, hq, hkv, d, dtype,
                                        int(causal), None, 0, ctypes.byref(info)))
    buf = torch.zeros(max(info.plan_bytes, 32), dtype=torch.uint8, device="cuda")
    _check(lib.cpattn_plan_build_device(pq, _ptr(ck), pqo, _ptr(ko), nch, nseq, hq, hkv, d, dtype,
                                        int(causal), c_void_p(buf.data_ptr()), buf.numel(),
                                        _stream_handle(stream)))
    torch.cuda.synchronize()
    return buf[:info.plan_bytes].cpu().numpy().view(PLAN_DTYPE)


def cpattn_plan_build(cu_seqlens_q, cu_seqlens_k, q_pos_offset=None, k_pos_offset=None, *,
                      hq: int, hkv: int, d: int, dtype: int = BF16, causal: bool = True):
    """Host-only plan of one chunk: (entries as a numpy structured array, info dict)."""
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


def cpattn_key_plan_build(cu_seqlens_q, cu_seqlens_ks: Sequence, q_pos_offset=None,
                          k_pos_offsets: Optional[Sequence] = None, *, hq: int, hkv: int, d: int,
                          causal: bool = True):
    """Host-only key-stationary plan of the backward over the chunks: (tiles, info dict)."""
    cq, pq = _host_i32(cu_seqlens_q, None, "cu_seqlens_q")
    nseq = len(cq) - 1
    qo, pqo = _host_i32(q_pos_offset, nseq, "q_pos_offset")
    ck, ko = _chunk_meta(cu_seqlens_ks, k_pos_offsets, nseq)
    lib = load()
    info = KeyPlanInfo()
    nch = len(cu_seqlens_ks)
    _check(lib.cpattn_key_plan_build(pq, _ptr(ck), pqo, _ptr(ko), nch, nseq, hq, hkv, d,
                                     int(causal), None, 0, ctypes.byref(info)))
    tiles = np.zeros(info.n_tiles, dtype=KEY_TILE_DTYPE)
    _check(lib.cpattn_key_plan_build(pq, _ptr(ck), pqo, _ptr(ko), nch, nseq, hq, hkv, d,
                                     int(causal), c_void_p(tiles.ctypes.data), tiles.nbytes,
                                     ctypes.byref(info)))
    return tiles, {name: getattr(info, name) for name, _ in KeyPlanInfo._fields_}


def cpattn_dcp_schedule(lengths, world: int, max_seqlen_per_rank: int) -> dict:
    """Dynamic CP schedule of a mini-batch (host only): per-sample cp_size, micro_batch,
    group_rank (first rank of its CP group) and slot (position in the group's pack) as int32
    arrays, and n_micro_batches."""
    n = len(lengths)
    arr, ptr = _host_i32(lengths, n, "lengths")
    outs = {k: np.zeros(max(n, 1), dtype=np.int32) for k in ("cp_size", "micro_batch", "group_rank", "slot")}
    nmb = np.zeros(1, dtype=np.int32)
    p = lambda a: a.ctypes.data_as(_I32P)
    _check(load().cpattn_dcp_schedule(ptr, n, int(world), int(max_seqlen_per_rank), p(outs["cp_size"]),
                                      p(outs["micro_batch"]), p(outs["group_rank"]), p(outs["slot"]),
                                      p(nmb)))
    res = {k: v[:n] for k, v in outs.items()}
    res["n_micro_batches"] = int(nmb[0])
    return res


def cpattn_workspace_size_chunks(nseq: int, cu_seqlens_q, hq: int, hkv: int, d: int,
                                 nchunks: int) -> int:
    arr, ptr = _host_i32(cu_seqlens_q, nseq + 1, "cu_seqlens_q")
    return int(load().cpattn_workspace_size_chunks(nseq, ptr, hq, hkv, d, nchunks))


def _check_tensor(name, t):
    if t.dim() != 3:
        raise ValueError(f"{name} must be [T, H, D]")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA tensor")


def _on_device(name, t, device):
    """A caller-supplied output or workspace must live on q's GPU: the kernels write through
    its pointer, and a host pointer handed to a kernel faults the GPU."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a CUDA tensor on {device} (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(workspace, need: int, device):
    """The caller's workspace (checked) or a fresh one; returns (tensor, bytes)."""
    import torch
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    _on_device("workspace", workspace, device)
    return workspace, workspace.numel() * workspace.element_size()


def _outputs(q, out, lse):
    import torch
    tq, hq, d = q.shape
    if out is None:
        out = torch.empty((tq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _on_device("out", out, q.device)
    _on_device("lse", lse, q.device)
    if out.shape != (tq, hq, d) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [Tq, Hq, D] tensor")
    if lse.shape != (hq, tq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [Hq, Tq] tensor")
    return out, lse


def _fwd_one(fn_name, q, k, v, cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, causal,
             out, lse, workspace, stream):
    import torch
    lib = load()
    cq, pq = _host_i32(cu_seqlens_q, None, "cu_seqlens_q")
    nseq = len(cq) - 1
    ck, pk = _host_i32(cu_seqlens_k, nseq + 1, "cu_seqlens_k")
    qo, pqo = _host_i32(q_pos_offset, nseq, "q_pos_offset")
    ko, pko = _host_i32(k_pos_offset, nseq, "k_pos_offset")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    tq, hq, d = q.shape
    tk, hkv, dk = k.shape
    if v.shape != k.shape or dk != d:
        raise ValueError("k and v must be [Tk, Hkv, D] with Q's D")
    if int(cq[-1]) != tq or int(ck[-1]) != tk:
        raise ValueError("cu_seqlens must end at the row counts of q and k")
    for name, t in (("k", k), ("v", v)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device {q.device}")
    out, lse = _outputs(q, out, lse)
    need = lib.cpattn_workspace_size(nseq, pq, hq, hkv, d)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    _check(getattr(lib, fn_name)(c_void_p(q.data_ptr()), c_void_p(k.data_ptr()),
                                 c_void_p(v.data_ptr()), pq, pk, pqo, pko, nseq, hq, hkv, d, dt,
                                 int(causal), c_void_p(out.data_ptr()), c_void_p(lse.data_ptr()),
                                 c_void_p(workspace.data_ptr()), ws_bytes,
                                 _stream_handle(stream)))
    return out, lse


def cpattn_fwd_chunk(q, k, v, cu_seqlens_q, cu_seqlens_k, q_pos_offset=None, k_pos_offset=None,
                     causal: bool = True, out=None, lse=None, workspace=None,
                     stream=None) -> Tuple["object", "object"]:
    """One KV chunk -> (O [Tq, Hq, D] fp32, LSE [Hq, Tq] fp32), asynchronously on the stream.

    q [Tq, Hq, D], k/v [Tk, Hkv, D]: contiguous CUDA tensors, bfloat16 or float32.
    cu_seqlens_*, *_pos_offset: host metadata (numpy / list / CPU tensor), int32.
    """
    return _fwd_one("cpattn_fwd_chunk", q, k, v, cu_seqlens_q, cu_seqlens_k, q_pos_offset,
                    k_pos_offset, causal, out, lse, workspace, stream)


def cpattn_fwd_chunk_accum(q, k, v, cu_seqlens_q, cu_seqlens_k, q_pos_offset=None,
                           k_pos_offset=None, causal: bool = True, out=None, lse=None,
                           workspace=None, stream=None) -> Tuple["object", "object"]:
    """(out, lse) <- merge((out, lse), partial of this chunk); out/lse are required."""
    if out is None or lse is None:
        raise ValueError("cpattn_fwd_chunk_accum folds into existing out and lse tensors")
    return _fwd_one("cpattn_fwd_chunk_accum", q, k, v, cu_seqlens_q, cu_seqlens_k, q_pos_offset,
                    k_pos_offset, causal, out, lse, workspace, stream)


def _chunks_args(q, ks, vs, cu_seqlens_q, cu_seqlens_ks, q_pos_offset, k_pos_offsets, accumulate,
                 out, lse):
    """Checked host metadata and tensors of a multi-chunk forward call."""
    nch = len(ks)
    if nch != len(vs) or nch != len(cu_seqlens_ks):
        raise ValueError("ks, vs and cu_seqlens_ks must have one entry per chunk")
    if k_pos_offsets is not None and len(k_pos_offsets) != nch:
        raise ValueError("k_pos_offsets must have one entry per chunk")
    cq, pq = _host_i32(cu_seqlens_q, None, "cu_seqlens_q")
    nseq = len(cq) - 1
    qo, pqo = _host_i32(q_pos_offset, nseq, "q_pos_offset")
    ck, ko = _chunk_meta(cu_seqlens_ks, k_pos_offsets, nseq)
    _check_tensor("q", q)
    dt = _dtype_code(q)
    tq, hq, d = q.shape
    if int(cq[-1]) != tq:
        raise ValueError("cu_seqlens_q must end at the row count of q")
    hkv = None
    for c in range(nch):
        _check_tensor(f"ks[{c}]", ks[c])
        _check_tensor(f"vs[{c}]", vs[c])
        if ks[c].dtype != q.dtype or vs[c].dtype != q.dtype:
            raise TypeError("q and every chunk's k, v must share one dtype")
        if vs[c].shape != ks[c].shape or ks[c].shape[2] != d:
            raise ValueError("k and v must be [Tk, Hkv, D] with Q's D")
        if hkv is not None and ks[c].shape[1] != hkv:
            raise ValueError("every chunk must have the same kv head count")
        hkv = ks[c].shape[1]
        if int(ck[c, -1]) != ks[c].shape[0]:
            raise ValueError(f"cu_seqlens_ks[{c}] must end at chunk {c}'s row count")
        if ks[c].device != q.device or vs[c].device != q.device:
            raise ValueError(f"chunk {c}'s k and v must be on q's device {q.device}")
    if hkv is None:
        raise ValueError("need at least one chunk")
    if accumulate and (out is None or lse is None):
        raise ValueError("accumulate=True folds into existing out and lse tensors")
    out, lse = _outputs(q, out, lse)
    kp = (c_void_p * max(nch, 1))(*[t.data_ptr() for t in ks])
    vp = (c_void_p * max(nch, 1))(*[t.data_ptr() for t in vs])
    return dict(nch=nch, nseq=nseq, pq=pq, pqo=pqo, ck=ck, ko=ko, dt=dt, hq=hq, hkv=hkv, d=d,
                out=out, lse=lse, kp=kp, vp=vp, keep=(cq, qo))


def cpattn_fwd_chunks(q, ks: Sequence, vs: Sequence, cu_seqlens_q, cu_seqlens_ks: Sequence,
                      q_pos_offset=None, k_pos_offsets: Optional[Sequence] = None,
                      causal: bool = True, accumulate: bool = False, out=None, lse=None,
                      workspace=None, stream=None) -> Tuple["object", "object"]:
    """All KV chunks in one launch -> (O, LSE) over the union of their keys.

    ks[c], vs[c]: chunk c's [Tk_c, Hkv, D] CUDA tensors; cu_seqlens_ks[c], k_pos_offsets[c]: its
    host metadata.  accumulate=True folds the result into the given out/lse.
    """
    lib = load()
    a = _chunks_args(q, ks, vs, cu_seqlens_q, cu_seqlens_ks, q_pos_offset, k_pos_offsets,
                     accumulate, out, lse)
    need = lib.cpattn_workspace_size_chunks(a["nseq"], a["pq"], a["hq"], a["hkv"], a["d"], a["nch"])
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    _check(lib.cpattn_fwd_chunks(c_void_p(q.data_ptr()), a["kp"], a["vp"], a["nch"], a["pq"],
                                 _ptr(a["ck"]), a["pqo"], _ptr(a["ko"]), a["nseq"], a["hq"],
                                 a["hkv"], a["d"], a["dt"], int(causal), int(accumulate),
                                 c_void_p(a["out"].data_ptr()), c_void_p(a["lse"].data_ptr()),
                                 c_void_p(workspace.data_ptr()), ws_bytes, _stream_handle(stream)))
    return a["out"], a["lse"]


def cpattn_fwd_chunks_noalloc(q, ks: Sequence, vs: Sequence, cu_seqlens_q,
                              cu_seqlens_ks: Sequence, q_pos_offset=None,
                              k_pos_offsets: Optional[Sequence] = None, causal: bool = True,
                              accumulate: bool = False, out=None, lse=None,
                              stream=None) -> Tuple["object", "object"]:
    """cpattn_fwd_chunks with the work plan in the library's static device scratch (no
    workspace, no device allocation by the library; pass out and lse to allocate nothing at
    all).  Calls that overlap on one GPU race on that scratch."""
    lib = load()
    a = _chunks_args(q, ks, vs, cu_seqlens_q, cu_seqlens_ks, q_pos_offset, k_pos_offsets,
                     accumulate, out, lse)
    _check(lib.cpattn_fwd_chunks_noalloc(c_void_p(q.data_ptr()), a["kp"], a["vp"], a["nch"],
                                         a["pq"], _ptr(a["ck"]), a["pqo"], _ptr(a["ko"]),
                                         a["nseq"], a["hq"], a["hkv"], a["d"], a["dt"], int(causal),
                                         int(accumulate), c_void_p(a["out"].data_ptr()),
                                         c_void_p(a["lse"].data_ptr()), _stream_handle(stream)))
    return a["out"], a["lse"]


def cpattn_bwd_workspace_size(nseq: int, cu_seqlens_q, cu_seqlens_k, hq: int, hkv: int,
                              d: int) -> int:
    cq, pq = _host_i32(cu_seqlens_q, nseq + 1, "cu_seqlens_q")
    ck, pk = _host_i32(cu_seqlens_k, nseq + 1, "cu_seqlens_k")
    return int(load().cpattn_bwd_workspace_size(nseq, pq, pk, hq, hkv, d))


def cpattn_bwd_chunk(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, q_pos_offset=None,
                     k_pos_offset=None, causal: bool = True, dq=None, dk=None, dv=None,
                     workspace=None, stream=None):
    """Backward of one KV chunk: ADDS this chunk's contributions to dq, dk, dv (fp32 CUDA
    tensors, zero-filled when not given) and returns (dq, dk, dv).

    q, do [Tq, Hq, D] and k, v [Tk, Hkv, D]: bfloat16; o [Tq, Hq, D] and lse [Hq, Tq]: the
    share's final forward output (float32).
    """
    import torch
    lib = load()
    cq, pq = _host_i32(cu_seqlens_q, None, "cu_seqlens_q")
    nseq = len(cq) - 1
    ck, pk = _host_i32(cu_seqlens_k, nseq + 1, "cu_seqlens_k")
    qo, pqo = _host_i32(q_pos_offset, nseq, "q_pos_offset")
    ko, pko = _host_i32(k_pos_offset, nseq, "k_pos_offset")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_tensor(name, t)
    if not lse.is_cuda or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous CUDA tensor")
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("do", do)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype")
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    if v.shape != k.shape or k.shape[2] != d or tuple(do.shape) != (tq, hq, d):
        raise ValueError("k, v must be [Tk, Hkv, D] and do [Tq, Hq, D]")
    if o.dtype != torch.float32 or tuple(o.shape) != (tq, hq, d):
        raise ValueError("o must be float32 [Tq, Hq, D]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (hq, tq):
        raise ValueError("lse must be float32 [Hq, Tq]")
    if int(cq[-1]) != tq or int(ck[-1]) != tk:
        raise ValueError("cu_seqlens must end at the row counts of q and k")
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.zeros((tq, hq, d), **f32) if dq is None else dq
    dk = torch.zeros((tk, hkv, d), **f32) if dk is None else dk
    dv = torch.zeros((tk, hkv, d), **f32) if dv is None else dv
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do), ("lse", lse)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device {q.device}")
    for name, t, shp in (("dq", dq, (tq, hq, d)), ("dk", dk, (tk, hkv, d)), ("dv", dv, (tk, hkv, d))):
        _on_device(name, t, q.device)
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shp:
            raise ValueError(f"{name} must be a contiguous float32 tensor of shape {shp}")
    need = lib.cpattn_bwd_workspace_size(nseq, pq, pk, hq, hkv, d)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    _check(lib.cpattn_bwd_chunk(c_void_p(q.data_ptr()), c_void_p(k.data_ptr()),
                                c_void_p(v.data_ptr()), c_void_p(o.data_ptr()),
                                c_void_p(do.data_ptr()), c_void_p(lse.data_ptr()), pq, pk, pqo, pko,
                                nseq, hq, hkv, d, dt, int(causal), c_void_p(dq.data_ptr()),
                                c_void_p(dk.data_ptr()), c_void_p(dv.data_ptr()),
                                c_void_p(workspace.data_ptr()), ws_bytes,
                                _stream_handle(stream)))
    return dq, dk, dv


def cpattn_bwd_workspace_size_chunks(nseq: int, cu_seqlens_q, cu_seqlens_ks: Sequence, hq: int,
                                     hkv: int, d: int) -> int:
    cq, pq = _host_i32(cu_seqlens_q, nseq + 1, "cu_seqlens_q")
    ck, _ = _chunk_meta(cu_seqlens_ks, None, nseq)
    return int(load().cpattn_bwd_workspace_size_chunks(nseq, pq, _ptr(ck), len(cu_seqlens_ks), hq,
                                                        hkv, d))


def cpattn_bwd_chunks(q, ks: Sequence, vs: Sequence, o, lse, do, cu_seqlens_q,
                      cu_seqlens_ks: Sequence, q_pos_offset=None,
                      k_pos_offsets: Optional[Sequence] = None, causal: bool = True, dq=None,
                      dks: Optional[Sequence] = None, dvs: Optional[Sequence] = None,
                      workspace=None, stream=None):
    """Backward of all chunks in one pass: ADDS to dq and to each chunk's dk, dv (fp32 CUDA
    tensors, zero-filled when not given); returns (dq, dks, dvs)."""
    import torch
    lib = load()
    nch = len(ks)
    if nch != len(vs) or nch != len(cu_seqlens_ks):
        raise ValueError("ks, vs and cu_seqlens_ks must have one entry per chunk")
    cq, pq = _host_i32(cu_seqlens_q, None, "cu_seqlens_q")
    nseq = len(cq) - 1
    qo, pqo = _host_i32(q_pos_offset, nseq, "q_pos_offset")
    ck, ko = _chunk_meta(cu_seqlens_ks, k_pos_offsets, nseq)
    for name, t in (("q", q), ("o", o), ("do", do)):
        _check_tensor(name, t)
    dt = _dtype_code(q)
    tq, hq, d = q.shape
    if do.dtype != q.dtype or tuple(do.shape) != (tq, hq, d):
        raise ValueError("do must match q")
    if o.dtype != torch.float32 or tuple(o.shape) != (tq, hq, d):
        raise ValueError("o must be float32 [Tq, Hq, D]")
    if (not lse.is_cuda or not lse.is_contiguous() or lse.dtype != torch.float32
            or tuple(lse.shape) != (hq, tq)):
        raise ValueError("lse must be a contiguous float32 CUDA tensor [Hq, Tq]")
    if int(cq[-1]) != tq:
        raise ValueError("cu_seqlens_q must end at the row count of q")
    hkv = None
    for c in range(nch):
        _check_tensor(f"ks[{c}]", ks[c]); _check_tensor(f"vs[{c}]", vs[c])
        if ks[c].dtype != q.dtype or vs[c].dtype != q.dtype or vs[c].shape != ks[c].shape:
            raise ValueError("every chunk's k, v must be [Tk, Hkv, D] in q's dtype")
        if hkv is not None and ks[c].shape[1] != hkv:
            raise ValueError("every chunk must have the same kv head count")
        hkv = ks[c].shape[1]
        if int(ck[c, -1]) != ks[c].shape[0]:
            raise ValueError(f"cu_seqlens_ks[{c}] must end at chunk {c}'s row count")
    if hkv is None:
        raise ValueError("need at least one chunk")
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.zeros((tq, hq, d), **f32) if dq is None else dq
    dks = [torch.zeros(t.shape, **f32) for t in ks] if dks is None else list(dks)
    dvs = [torch.zeros(t.shape, **f32) for t in vs] if dvs is None else list(dvs)
    for name, t in (("o", o), ("do", do), ("lse", lse)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device {q.device}")
    if len(dks) != nch or len(dvs) != nch:
        raise ValueError("dks and dvs must have one entry per chunk")
    _on_device("dq", dq, q.device)
    if dq.dtype != torch.float32 or not dq.is_contiguous() or tuple(dq.shape) != (tq, hq, d):
        raise ValueError("dq must be a contiguous float32 tensor like q")
    for c in range(nch):
        if ks[c].device != q.device or vs[c].device != q.device:
            raise ValueError(f"chunk {c}'s k and v must be on q's device {q.device}")
        for name, t in (("dks", dks[c]), ("dvs", dvs[c])):
            _on_device(f"{name}[{c}]", t, q.device)
            if t.dtype != torch.float32 or not t.is_contiguous() or t.shape != ks[c].shape:
                raise ValueError(f"{name}[{c}] must be a contiguous float32 tensor like ks[{c}]")
    need = lib.cpattn_bwd_workspace_size_chunks(nseq, pq, _ptr(ck), nch, hq, hkv, d)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    arr = lambda ts: (c_void_p * max(nch, 1))(*[t.data_ptr() for t in ts])
    _check(lib.cpattn_bwd_chunks(c_void_p(q.data_ptr()), arr(ks), arr(vs), nch,
                                 c_void_p(o.data_ptr()), c_void_p(do.data_ptr()),
                                 c_void_p(lse.data_ptr()), pq, _ptr(ck), pqo, _ptr(ko), nseq, hq,
                                 hkv, d, dt, int(causal), c_void_p(dq.data_ptr()), arr(dks),
                                 arr(dvs), c_void_p(workspace.data_ptr()), ws_bytes,
                                 _stream_handle(stream)))
    return dq, dks, dvs


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
                or tuple(x.shape) != shp or x.device != o_a.device):
            raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of shape {shp} "
                             f"on {o_a.device}")
    _check(lib.cpattn_merge(c_void_p(o_a.data_ptr()), c_void_p(lse_a.data_ptr()),
                            c_void_p(o_b.data_ptr()), c_void_p(lse_b.data_ptr()), t, hq, d,
                            _stream_handle(stream)))
