"""Python binding of the unified-max split-KV decode-attention library (gfx950).

The binding only marshals arguments: torch tensors give the device pointers
and the current HIP stream, every step of the computation runs in the HIP
kernels of ``libfd_attn.so`` (declared in ``include/fd_attn.h``).  The
function names are those of the C ABI.  If the shared library is missing the
import of the first function raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
import numpy as np
from typing import Optional, Sequence

__all__ = ["fd_attn_decode", "fd_attn_decode_static", "fd_attn_plan", "FD_PLAN_SHAPE",
           "FD_PLAN_FUSED", "FD_PLAN_SPLIT", "FD_PLAN_SHARES", "prepare_decode", "DecodeCall", "fd_attn_prefill", "fd_attn_score_stats", "fd_attn_choose_band",
           "fd_attn_workspace_size", "fd_flat_gemm", "fd_flat_gemm_plan",
           "fd_flat_gemm_workspace_size", "fd_flat_gemm_pack_weights", "fd_flat_gemm_packed_bytes",
           "make_gemm_desc",
           "fd_attn_status_string", "FdAttnError", "make_desc", "make_prefill_desc",
           "library_path", "FD_F32", "FD_BF16", "FD_FP8_E4M3FN"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfd_attn.so")

FD_F32, FD_BF16, FD_FP8_E4M3FN = 0, 1, 2
_DTYPE_CODE = {"f32": FD_F32, "bf16": FD_BF16, "e4m3fn": FD_FP8_E4M3FN}


class FdAttnError(RuntimeError):
    """A nonzero status from the C ABI."""

    def __init__(self, status: int, msg: str):
        super().__init__("fd_attn status %d: %s" % (status, msg))
        self.status = status


class FdAttnDesc(ctypes.Structure):
    """Mirror of fd_attn_desc_t."""
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("scale", ctypes.c_float),
                ("q_dtype", ctypes.c_int), ("kv_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("stage_events", ctypes.c_void_p),
                ("plan", ctypes.c_int32)]


# fd_attn_desc_t.plan bits (include/fd_attn.h)
FD_PLAN_FUSED, FD_PLAN_SPLIT, FD_PLAN_SHARES = 0x10, 0x20, 0x40


def FD_PLAN_SHAPE(k: int) -> int:
    return k + 1


class FdPrefillDesc(ctypes.Structure):
    """Mirror of fd_prefill_desc_t."""
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q_len", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("stage_events", ctypes.c_void_p), ("kv_dtype", ctypes.c_int),
                ("page_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class FdGemmDesc(ctypes.Structure):
    """Mirror of fd_gemm_desc_t."""
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("a_dtype", ctypes.c_int), ("w_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("variant", ctypes.c_int32), ("ksplit", ctypes.c_int32),
                ("w_layout", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stage_events", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libfd_attn.so is not built; run python split_kv_asynchronous_amd/build.py "
                              "(hipcc --offload-arch=gfx950)")
        lib = ctypes.CDLL(_LIB_PATH)
        D = ctypes.POINTER(FdAttnDesc)
        lib.fd_attn_workspace_size.argtypes = [D]
        lib.fd_attn_workspace_size.restype = ctypes.c_size_t
        lib.fd_attn_decode.argtypes = [D, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
        lib.fd_attn_decode.restype = ctypes.c_int
        lib.fd_attn_decode_static.argtypes = lib.fd_attn_decode.argtypes
        lib.fd_attn_decode_static.restype = ctypes.c_int
        lib.fd_attn_prefill.argtypes = [ctypes.POINTER(FdPrefillDesc), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.fd_attn_prefill.restype = ctypes.c_int
        lib.fd_attn_score_stats.argtypes = [D, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_float, ctypes.c_float,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]
        lib.fd_attn_score_stats.restype = ctypes.c_int
        lib.fd_attn_choose_band.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                            ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]
        lib.fd_attn_choose_band.restype = ctypes.c_int
        G = ctypes.POINTER(FdGemmDesc)
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.fd_flat_gemm_plan.argtypes = [G, i32p, i32p, i32p, i32p]
        lib.fd_flat_gemm_plan.restype = ctypes.c_int
        lib.fd_flat_gemm_workspace_size.argtypes = [G]
        lib.fd_flat_gemm_workspace_size.restype = ctypes.c_size_t
        lib.fd_flat_gemm.argtypes = [G, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
        lib.fd_flat_gemm.restype = ctypes.c_int
        lib.fd_flat_gemm_packed_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
        lib.fd_flat_gemm_packed_bytes.restype = ctypes.c_size_t
        lib.fd_flat_gemm_pack_weights.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p]
        lib.fd_flat_gemm_pack_weights.restype = ctypes.c_int
        lib.fd_attn_plan.argtypes = [D, i32p, i32p, i32p, i32p, i32p]
        lib.fd_attn_plan.restype = ctypes.c_int
        lib.fd_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]
        lib.fd_probe_read.restype = ctypes.c_int
        lib.fd_attn_status_string.argtypes = [ctypes.c_int]
        lib.fd_attn_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def fd_attn_status_string(status: int) -> str:
    return _load().fd_attn_status_string(int(status)).decode()


def make_desc(*, batch: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int,
              chunk_size: int, page_size: int = 0, max_blocks_per_seq: int = 0,
              num_pages: int = 0, scale: Optional[float] = None, q_dtype: str = "bf16",
              kv_dtype: str = "bf16", out_dtype: str = "f32", head_dim: int = 128,
              k_scale_ptr: int = 0, v_scale_ptr: int = 0, workspace_ptr: int = 0,
              workspace_bytes: int = 0, stage_events_ptr: int = 0, plan: int = 0) -> FdAttnDesc:
    return FdAttnDesc(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, chunk_size,
                      page_size, max_blocks_per_seq, num_pages,
                      -1.0 if scale is None else float(scale), _DTYPE_CODE[q_dtype],
                      _DTYPE_CODE[kv_dtype], _DTYPE_CODE[out_dtype], k_scale_ptr or None,
                      v_scale_ptr or None, workspace_ptr or None, workspace_bytes,
                      stage_events_ptr or None, int(plan))


def fd_attn_plan(desc: FdAttnDesc) -> dict:
    """The plan the library runs for this descriptor (fd_attn_plan): chunk
    size, kernel family, kernel shape, whether the merge is fused, and the
    number of balanced shares (0: fixed chunks)."""
    vals = [ctypes.c_int32() for _ in range(5)]
    rc = _load().fd_attn_plan(ctypes.byref(desc), *[ctypes.byref(v) for v in vals])
    if rc != 0:
        raise FdAttnError(rc, fd_attn_status_string(rc))
    return dict(zip(("chunk_size", "family", "shape", "fused", "shares"), (v.value for v in vals)))


def fd_attn_workspace_size(desc: FdAttnDesc) -> int:
    return int(_load().fd_attn_workspace_size(ctypes.byref(desc)))


def _torch_code(t) -> str:
    import torch
    return {torch.float32: "f32", torch.bfloat16: "bf16", torch.float8_e4m3fn: "e4m3fn",
            torch.int16: "bf16", torch.uint16: "bf16", torch.uint8: "e4m3fn"}[t.dtype]


class DecodeCall:
    """A validated fd_attn_decode call with its descriptor and pointers
    marshalled once (prepare_decode); calling it enqueues the call again on
    the same tensors, optionally with another band or stream.  It holds
    references to every tensor it points at."""

    def __init__(self, desc, ptrs, keep, phi, a, b, stream):
        self.desc, self._ptrs, self._keep = desc, ptrs, keep
        self.phi, self.a, self.b, self.stream = float(phi), float(a), float(b), stream
        self.out, self.fallback_flags, self.workspace = keep[-3], keep[-2], keep[-1]
        self._fn = _load().fd_attn_decode

    def __call__(self, phi=None, a=None, b=None, stream=None, stage_events=None):
        import torch
        desc = self.desc
        ev_arr = None
        if stage_events is not None:
            ev_arr = _event_array(stage_events)
            desc.stage_events = ctypes.cast(ev_arr, ctypes.c_void_p)
        else:
            desc.stage_events = None
        if stream is None:
            stream = self.stream
        if stream is None:
            stream = torch.cuda.current_stream(self.out.device).cuda_stream
        q, k, v, lens, table, out, flags = self._ptrs
        rc = self._fn(ctypes.byref(desc), q, k, v, lens, table,
                      self.phi if phi is None else float(phi), self.a if a is None else float(a),
                      self.b if b is None else float(b), out, flags, stream)
        desc.stage_events = None
        if rc != 0:
            raise FdAttnError(rc, fd_attn_status_string(rc))
        return self.out, self.fallback_flags


def _marshal_decode(q, k_cache, v_cache, seq_lens, block_table, out, fallback_flags, *,
                    chunk_size, max_seq_len, num_kv_heads, page_size, scale, k_scale, v_scale,
                    q_dtype, kv_dtype, out_dtype, plan=0):
    """Checks the tensors of a decode call; returns (descriptor without a
    workspace, pointers, tensors to keep alive).  Allocates only a missing
    out or fallback_flags."""
    import torch
    dev = q.device
    B, Hq, D = q.shape
    qd = q_dtype or _torch_code(q)
    kd = kv_dtype or _torch_code(k_cache)
    if num_kv_heads is None:
        num_kv_heads = k_cache.shape[1]
    for t in (q, k_cache, v_cache, seq_lens):
        if t.device != dev or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous and on the same device")
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    max_blocks = num_pages = 0
    if page_size:
        if block_table is None or block_table.dtype != torch.int32 or not block_table.is_contiguous():
            raise ValueError("paged caches need a contiguous int32 block_table")
        max_blocks = block_table.shape[1]
        num_pages = k_cache.shape[0]
    ks = vs = 0
    if kd == "e4m3fn":
        if k_scale is None or v_scale is None:
            raise ValueError("fp8 caches need k_scale and v_scale")
        if not (k_scale.is_contiguous() and v_scale.is_contiguous()):
            raise ValueError("k_scale and v_scale must be contiguous")
        ks, vs = k_scale.data_ptr(), v_scale.data_ptr()
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16,
                          device=dev)
    if fallback_flags is None:
        fallback_flags = torch.empty((B, Hq), dtype=torch.uint8, device=dev)
    desc = make_desc(batch=B, num_q_heads=Hq, num_kv_heads=num_kv_heads, max_seq_len=max_seq_len,
                     chunk_size=chunk_size, page_size=page_size, max_blocks_per_seq=max_blocks,
                     num_pages=num_pages, scale=scale, q_dtype=qd, kv_dtype=kd,
                     out_dtype=out_dtype, head_dim=D, k_scale_ptr=ks, v_scale_ptr=vs, plan=plan)
    table = block_table if page_size else None
    ptrs = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
            table.data_ptr() if table is not None else None, out.data_ptr(),
            fallback_flags.data_ptr())
    keep = (q, k_cache, v_cache, seq_lens, table, k_scale, v_scale, out, fallback_flags)
    return desc, ptrs, keep


def prepare_decode(q, k_cache, v_cache, seq_lens, block_table, phi: float, a: float, b: float,
                   out=None, fallback_flags=None, *, chunk_size: int, max_seq_len: int,
                   num_kv_heads: Optional[int] = None, page_size: int = 0,
                   scale: Optional[float] = None, k_scale=None, v_scale=None, workspace=None,
                   q_dtype: Optional[str] = None, kv_dtype: Optional[str] = None,
                   out_dtype: str = "f32", stream=None, plan: int = 0) -> DecodeCall:
    """Checks and marshals the arguments of fd_attn_decode (same meaning)
    once; returns a DecodeCall that enqueues the call each time it is called.
    ``plan``: fd_attn_desc_t.plan (0: the library's table)."""
    import torch
    desc, ptrs, keep = _marshal_decode(q, k_cache, v_cache, seq_lens, block_table, out, fallback_flags,
                                       chunk_size=chunk_size, max_seq_len=max_seq_len,
                                       num_kv_heads=num_kv_heads, page_size=page_size, scale=scale,
                                       k_scale=k_scale, v_scale=v_scale, q_dtype=q_dtype,
                                       kv_dtype=kv_dtype, out_dtype=out_dtype, plan=plan)
    need = fd_attn_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    desc.workspace = workspace.data_ptr()
    desc.workspace_bytes = workspace.numel() * workspace.element_size()
    return DecodeCall(desc, ptrs, keep + (workspace,), phi, a, b, stream)


def fd_attn_decode_static(q, k_cache, v_cache, seq_lens, block_table, phi: float, a: float,
                          b: float, out, fallback_flags, *, chunk_size: int, max_seq_len: int,
                          num_kv_heads: Optional[int] = None, page_size: int = 0,
                          scale: Optional[float] = None, k_scale=None, v_scale=None,
                          q_dtype: Optional[str] = None, kv_dtype: Optional[str] = None,
                          out_dtype: Optional[str] = None, stream=None, plan: int = 0):
    """fd_attn_decode_static of include/fd_attn.h: one decode call whose
    workspace is the library's static device array, so nothing is allocated
    here or in the library; ``out`` and ``fallback_flags`` are required.
    Arguments otherwise as fd_attn_decode.  Returns (out, fallback_flags)."""
    import torch
    if out is None or fallback_flags is None:
        raise ValueError("fd_attn_decode_static allocates nothing: pass out and fallback_flags")
    if out_dtype is None:
        out_dtype = "f32" if out.dtype == torch.float32 else "bf16"
    desc, ptrs, _ = _marshal_decode(q, k_cache, v_cache, seq_lens, block_table, out, fallback_flags,
                                    chunk_size=chunk_size, max_seq_len=max_seq_len,
                                    num_kv_heads=num_kv_heads, page_size=page_size, scale=scale,
                                    k_scale=k_scale, v_scale=v_scale, q_dtype=q_dtype,
                                    kv_dtype=kv_dtype, out_dtype=out_dtype, plan=plan)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    qp, kp, vp, lp, tp, op, fp = ptrs
    rc = _load().fd_attn_decode_static(ctypes.byref(desc), qp, kp, vp, lp, tp, float(phi), float(a),
                                       float(b), op, fp, stream)
    if rc != 0:
        raise FdAttnError(rc, fd_attn_status_string(rc))
    return out, fallback_flags


def fd_attn_decode(q, k_cache, v_cache, seq_lens, block_table, phi: float, a: float, b: float,
                   out=None, fallback_flags=None, *, chunk_size: int, max_seq_len: int,
                   num_kv_heads: Optional[int] = None, page_size: int = 0,
                   scale: Optional[float] = None, k_scale=None, v_scale=None, workspace=None,
                   q_dtype: Optional[str] = None, kv_dtype: Optional[str] = None,
                   out_dtype: str = "f32", stream=None, stage_events: Optional[Sequence] = None,
                   plan: int = 0):
    """One decode-attention call on device tensors; returns (out, fallback_flags).

    Tensors must live on the same GPU.  Layouts as in include/fd_attn.h:
    q [B][Hq][128]; contiguous caches [B][Hkv][max_seq_len][128] or paged
    caches [pages][Hkv][page_size][128]; seq_lens int32 [B]; block_table
    int32 [B][max_blocks] (paged) or None.  bf16 data may be passed as
    torch.bfloat16 or as 16-bit integer bit patterns, E4M3FN as
    torch.float8_e4m3fn or uint8 codes.  ``workspace`` is a uint8 device
    tensor of at least fd_attn_workspace_size() bytes (allocated here if None).
    For repeated calls on the same tensors, prepare_decode marshals once.
    """
    call = prepare_decode(q, k_cache, v_cache, seq_lens, block_table, phi, a, b, out,
                          fallback_flags, chunk_size=chunk_size, max_seq_len=max_seq_len,
                          num_kv_heads=num_kv_heads, page_size=page_size, scale=scale,
                          k_scale=k_scale, v_scale=v_scale, workspace=workspace, q_dtype=q_dtype,
                          kv_dtype=kv_dtype, out_dtype=out_dtype, stream=stream, plan=plan)
    return call(stage_events=stage_events)


def make_prefill_desc(*, batch: int, num_q_heads: int, num_kv_heads: int, q_len: int,
                      max_seq_len: int, scale: Optional[float] = None, dtype: str = "bf16",
                      out_dtype: str = "f32", head_dim: int = 128,
                      stage_events_ptr: int = 0, kv_dtype: str = "bf16", page_size: int = 0,
                      max_blocks_per_seq: int = 0, num_pages: int = 0, block_table_ptr: int = 0,
                      k_scale_ptr: int = 0, v_scale_ptr: int = 0) -> FdPrefillDesc:
    return FdPrefillDesc(batch, num_q_heads, num_kv_heads, head_dim, q_len, max_seq_len,
                         -1.0 if scale is None else float(scale), _DTYPE_CODE[dtype],
                         _DTYPE_CODE[out_dtype], stage_events_ptr or None, _DTYPE_CODE[kv_dtype],
                         page_size, max_blocks_per_seq, num_pages, block_table_ptr or None,
                         k_scale_ptr or None, v_scale_ptr or None)


def _event_array(stage_events):
    handles = [e.cuda_event if hasattr(e, "cuda_event") else int(e) for e in stage_events]
    if len(handles) != 2 or not all(handles):
        raise ValueError("stage_events: 2 created HIP events -- kernel start/stop "
                         "(record a torch event once to create it)")
    return (ctypes.c_void_p * 2)(*handles)


def fd_attn_prefill(q, k, v, kv_lens, phi: float, a: float, b: float, out=None,
                    fallback_flags=None, *, num_kv_heads: Optional[int] = None,
                    scale: Optional[float] = None, out_dtype: str = "f32", stream=None,
                    stage_events: Optional[Sequence] = None, block_table=None, page_size: int = 0,
                    max_seq_len: Optional[int] = None, k_scale=None, v_scale=None):
    """Causal prefill attention of a query block per sequence; returns (out, fallback_flags).

    Layouts as in include/fd_prefill.h: q [B][Hq][q_len][128] bf16; k, v
    contiguous [B][Hkv][max_seq_len][128] or, with page_size > 0, paged
    [pages][Hkv][page_size][128] with block_table int32 [B][max_blocks] and
    max_seq_len given; bf16 or E4M3FN (with k_scale, v_scale fp32 [Hkv]);
    kv_lens int32 [B] (keys per sequence, the query block included: query j
    sits at position kv_lens[b] - q_len + j).  bf16 data may be
    torch.bfloat16 or 16-bit integer bit patterns, E4M3FN
    torch.float8_e4m3fn or uint8 codes.
    """
    import torch
    dev = q.device
    B, Hq, Lq, D = q.shape
    for t in (q, k, v, kv_lens):
        if t.device != dev or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous and on the same device")
    if _torch_code(q) != "bf16":
        raise ValueError("q must be bf16")
    kvd = _torch_code(k)
    if kvd not in ("bf16", "e4m3fn") or _torch_code(v) != kvd:
        raise ValueError("k and v must both be bf16 or both E4M3FN")
    if kv_lens.dtype != torch.int32:
        raise ValueError("kv_lens must be int32")
    if k.dim() != 4 or v.shape != k.shape:
        raise ValueError("k and v must be [B][Hkv][max_seq_len][128] or [pages][Hkv][page_size][128]")
    if num_kv_heads is None:
        num_kv_heads = k.shape[1]
    max_blocks = num_pages = 0
    table_ptr = 0
    if page_size:
        if block_table is None or block_table.dtype != torch.int32 or not block_table.is_contiguous():
            raise ValueError("paged caches need a contiguous int32 block_table")
        if max_seq_len is None:
            raise ValueError("paged caches need max_seq_len")
        max_blocks, num_pages, table_ptr = block_table.shape[1], k.shape[0], block_table.data_ptr()
    else:
        max_seq_len = k.shape[2]
    ks = vs = 0
    if kvd == "e4m3fn":
        if k_scale is None or v_scale is None or not (k_scale.is_contiguous() and v_scale.is_contiguous()):
            raise ValueError("E4M3FN caches need contiguous k_scale and v_scale")
        ks, vs = k_scale.data_ptr(), v_scale.data_ptr()
    if out is None:
        out = torch.empty((B, Hq, Lq, D),
                          dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device=dev)
    if fallback_flags is None:
        fallback_flags = torch.empty((B, Hq, Lq), dtype=torch.uint8, device=dev)
    desc = make_prefill_desc(batch=B, num_q_heads=Hq, num_kv_heads=num_kv_heads, q_len=Lq,
                             max_seq_len=max_seq_len, scale=scale, out_dtype=out_dtype,
                             head_dim=D, kv_dtype=kvd, page_size=page_size,
                             max_blocks_per_seq=max_blocks, num_pages=num_pages,
                             block_table_ptr=table_ptr, k_scale_ptr=ks, v_scale_ptr=vs)
    ev_arr = None
    if stage_events is not None:
        ev_arr = _event_array(stage_events)
        desc.stage_events = ctypes.cast(ev_arr, ctypes.c_void_p)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = _load().fd_attn_prefill(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 kv_lens.data_ptr(), float(phi), float(a), float(b),
                                 out.data_ptr(), fallback_flags.data_ptr(), stream)
    if rc != 0:
        raise FdAttnError(rc, fd_attn_status_string(rc))
    return out, fallback_flags


def fd_attn_score_stats(q, k_cache, seq_lens, block_table=None, *, max_seq_len: int,
                        chunk_size: int = 512, num_kv_heads: Optional[int] = None,
                        page_size: int = 0, scale: Optional[float] = None, k_scale=None,
                        hist_lo: float = -16.0, hist_hi: float = 16.0, nbins: int = 0,
                        q_dtype: Optional[str] = None, kv_dtype: Optional[str] = None,
                        stream=None):
    """Per-row score extremes (and optionally a histogram) of decode inputs.

    Same tensors and layouts as fd_attn_decode (V is not read).  Returns
    (row_max [B][Hq] f32, row_min [B][Hq] f32, hist uint32 [nbins + 2] as an
    int32 tensor of the same bits, or None).
    """
    import torch
    dev = q.device
    B, Hq, D = q.shape
    qd = q_dtype or _torch_code(q)
    kd = kv_dtype or _torch_code(k_cache)
    if num_kv_heads is None:
        num_kv_heads = k_cache.shape[1]
    for t in (q, k_cache, seq_lens):
        if t.device != dev or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous and on the same device")
    max_blocks = num_pages = 0
    if page_size:
        max_blocks = block_table.shape[1]
        num_pages = k_cache.shape[0]
    ks = 0
    if kd == "e4m3fn":
        if k_scale is None:
            raise ValueError("fp8 caches need k_scale")
        k_scale = k_scale.contiguous()
        ks = k_scale.data_ptr()
    desc = make_desc(batch=B, num_q_heads=Hq, num_kv_heads=num_kv_heads, max_seq_len=max_seq_len,
                     chunk_size=chunk_size, page_size=page_size, max_blocks_per_seq=max_blocks,
                     num_pages=num_pages, scale=scale, q_dtype=qd, kv_dtype=kd, head_dim=D,
                     k_scale_ptr=ks)
    row_max = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    row_min = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    hist = torch.empty(nbins + 2, dtype=torch.int32, device=dev) if nbins > 0 else None
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = _load().fd_attn_score_stats(ctypes.byref(desc), q.data_ptr(), k_cache.data_ptr(),
                                     seq_lens.data_ptr(),
                                     block_table.data_ptr() if page_size else None,
                                     float(hist_lo), float(hist_hi), int(nbins),
                                     row_max.data_ptr(), row_min.data_ptr(),
                                     hist.data_ptr() if hist is not None else None, stream)
    if rc != 0:
        raise FdAttnError(rc, fd_attn_status_string(rc))
    return row_max, row_min, hist


def fd_attn_choose_band(row_max, row_min, max_flag_fraction: float = 0.0, a_share: float = 0.5,
                        max_width: float = 64.0, pad: float = 1e-3):
    """Host band choice (include/fd_calib.h) from per-row extremes (array-likes
    or CPU/GPU tensors).  Returns (phi, a, b, flagged_rows)."""
    import numpy as np
    def host(x):
        if hasattr(x, "detach"):
            x = x.detach().float().cpu().numpy()
        return np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    mx, mn = host(row_max), host(row_min)
    if mx.shape != mn.shape:
        raise ValueError("row_max and row_min differ in size")
    phi, a, b = ctypes.c_float(), ctypes.c_float(), ctypes.c_float()
    flagged = ctypes.c_int64()
    rc = _load().fd_attn_choose_band(mx.ctypes.data, mn.ctypes.data, mx.size,
                                     float(max_flag_fraction), float(a_share), float(max_width),
                                     float(pad), ctypes.byref(phi), ctypes.byref(a),
                                     ctypes.byref(b), ctypes.byref(flagged))
    if rc != 0:
        raise FdAttnError(rc, fd_attn_status_string(rc))
    return phi.value, a.value, b.value, flagged.value


_W_LAYOUT = {"rows": 0, "packed": 1}


def make_gemm_desc(*, m: int, n: int, k: int, out_dtype: str = "f32", variant: int = 0,
                   ksplit: int = 0, w_layout: str = "rows") -> FdGemmDesc:
    return FdGemmDesc(m, n, k, FD_BF16, FD_BF16, _DTYPE_CODE[out_dtype], variant, ksplit,
                      _W_LAYOUT[w_layout], None, 0, None)


def fd_flat_gemm_packed_bytes(n: int, k: int) -> int:
    return int(_load().fd_flat_gemm_packed_bytes(n, k))


def fd_flat_gemm_pack_weights(w, out=None, stream=None):
    """Packs w ([N][K] bf16, device) into the fragment-major layout of
    include/fd_gemm.h; returns a flat bf16 tensor of fd_flat_gemm_packed_bytes."""
    import torch
    if w.dim() != 2 or not w.is_contiguous() or _torch_code(w) != "bf16":
        raise ValueError("w must be a contiguous [N][K] bf16 tensor")
    N, K = w.shape
    nbytes = fd_flat_gemm_packed_bytes(N, K)
    if nbytes == 0:
        raise FdAttnError(-2, fd_attn_status_string(-2))
    if out is None:
        out = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=w.device)
    if stream is None:
        stream = torch.cuda.current_stream(w.device).cuda_stream
    rc = _load().fd_flat_gemm_pack_weights(N, K, w.data_ptr(), out.data_ptr(), stream)
    if rc != 0:
        raise FdAttnError(rc, fd_attn_status_string(rc))
    return out


def fd_flat_gemm_plan(m: int, n: int, k: int, *, variant: int = 0, ksplit: int = 0,
                      out_dtype: str = "f32", w_layout: str = "rows") -> dict:
    """The configuration fd_flat_gemm runs for this shape (include/fd_gemm.h)."""
    desc = make_gemm_desc(m=m, n=n, k=k, out_dtype=out_dtype, variant=variant, ksplit=ksplit,
                          w_layout=w_layout)
    v, s, per, wg = (ctypes.c_int32() for _ in range(4))
    rc = _load().fd_flat_gemm_plan(ctypes.byref(desc), ctypes.byref(v), ctypes.byref(s),
                                   ctypes.byref(per), ctypes.byref(wg))
    if rc != 0:
        raise FdAttnError(rc, fd_attn_status_string(rc))
    return {"variant": v.value, "ksplit": s.value, "steps_per_slice": per.value,
            "workgroups": wg.value}


def fd_flat_gemm_workspace_size(m: int, n: int, k: int, *, variant: int = 0, ksplit: int = 0,
                                out_dtype: str = "f32", w_layout: str = "rows") -> int:
    desc = make_gemm_desc(m=m, n=n, k=k, out_dtype=out_dtype, variant=variant, ksplit=ksplit,
                          w_layout=w_layout)
    return int(_load().fd_flat_gemm_workspace_size(ctypes.byref(desc)))


def fd_flat_gemm(a, w, out=None, *, out_dtype: str = "f32", variant: int = 0, ksplit: int = 0,
                 workspace=None, stream=None, stage_events: Optional[Sequence] = None,
                 n: Optional[int] = None):
    """C = A . W^T on device tensors (include/fd_gemm.h); returns C.

    a [M][K] and w [N][K] are bf16 (torch.bfloat16 or 16-bit bit patterns);
    w may instead be the flat output of fd_flat_gemm_pack_weights, with the
    row count given as ``n``.  C is [M][N] float32 or bfloat16.
    ``workspace`` is a uint8 device tensor of at least
    fd_flat_gemm_workspace_size() bytes (allocated here if None).
    """
    import torch
    dev = a.device
    packed = n is not None
    if a.dim() != 2:
        raise ValueError("a must be [M][K]")
    M, K = a.shape
    if packed:
        if w.dim() != 1 or w.numel() * w.element_size() < fd_flat_gemm_packed_bytes(n, K):
            raise ValueError("packed w must be the flat output of fd_flat_gemm_pack_weights")
        N = n
    else:
        if w.dim() != 2 or a.shape[1] != w.shape[1]:
            raise ValueError("a must be [M][K] and w [N][K]")
        N = w.shape[0]
    for t in (a, w):
        if t.device != dev or not t.is_contiguous() or _torch_code(t) != "bf16":
            raise ValueError("a and w must be contiguous bf16 tensors on the same device")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16,
                          device=dev)
    desc = make_gemm_desc(m=M, n=N, k=K, out_dtype=out_dtype, variant=variant, ksplit=ksplit,
                          w_layout="packed" if packed else "rows")
    need = int(_load().fd_flat_gemm_workspace_size(ctypes.byref(desc)))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        desc.workspace = workspace.data_ptr()
        desc.workspace_bytes = workspace.numel() * workspace.element_size()
    ev_arr = None
    if stage_events is not None:
        ev_arr = _event_array(stage_events)
        desc.stage_events = ctypes.cast(ev_arr, ctypes.c_void_p)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = _load().fd_flat_gemm(ctypes.byref(desc), a.data_ptr(), w.data_ptr(), out.data_ptr(),
                              stream)
    if rc != 0:
        raise FdAttnError(rc, fd_attn_status_string(rc))
    return out


# numpy layout of fd_probe_unit_t (include/fd_probe.h)
PROBE_UNIT = np.dtype([("offset", "<u8"), ("bytes", "<u4"), ("reserved", "<u4")])


def fd_probe_read(k, v, units, shape: int = 0, pages=None, page_bytes: int = 0, sink=None, stream=None):
    """Streams the units (a device uint8 tensor of PROBE_UNIT records) of k
    and v -- byte ranges, or with `pages` (a device int64 tensor of page byte
    offsets) whole pages -- through a decode kernel's DMA ring shape and
    computes nothing (include/fd_probe.h): a read-bandwidth measurement."""
    import torch
    if units.dtype != torch.uint8 or units.numel() % PROBE_UNIT.itemsize or not units.is_contiguous():
        raise ValueError("units must be a contiguous uint8 tensor of PROBE_UNIT records")
    if pages is not None and (pages.dtype != torch.int64 or not pages.is_contiguous()):
        raise ValueError("pages must be a contiguous int64 tensor of byte offsets")
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device=k.device)
    if stream is None:
        stream = torch.cuda.current_stream(k.device).cuda_stream
    rc = _load().fd_probe_read(k.data_ptr(), v.data_ptr(), units.data_ptr(),
                               units.numel() // PROBE_UNIT.itemsize,
                               None if pages is None else pages.data_ptr(), page_bytes, shape,
                               sink.data_ptr(), stream)
    if rc != 0:
        raise FdAttnError(rc, fd_attn_status_string(rc))


def default_scale(head_dim: int = 128) -> float:
    return 1.0 / math.sqrt(head_dim)
