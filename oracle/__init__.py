"""TEST INFRASTRUCTURE: float64 CPU oracle for unified-max split-KV decode attention.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library neither imports nor links it, and the two share
no source.  The arithmetic lives in ``fd_oracle.c`` (plain C, float64, one
OpenMP loop over rows); this module only marshals numpy arrays.

The flat GEMM of the decode linear layers (``flat_gemm``) is numpy float64
arithmetic in this module.

Functions follow the FlashDecoding++ theory page: ``decode_exact`` is the plain
max-subtracted softmax attention plus the safe-band test (section 3, first
formula and the fallback rule); ``decode_unified`` walks the method's steps --
per-chunk sums against the preset constant phi, online-softmax recompute of a
chunk whose scores leave the band, plain-sum merge (section 3, second formula
and the fallback rule; the split-KV figure of section 1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libfd_oracle.so")

_DT = {"f32": 0, "bf16": 1, "e4m3fn": 2}
_NP_DT = {"f32": np.float32, "bf16": np.uint16, "e4m3fn": np.uint8}


def build(force: bool = False) -> str:
    """Compile fd_oracle.c with gcc (float64, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                        "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("scale", ctypes.c_double)]


class _Inputs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P, I = ctypes.POINTER(_Problem), ctypes.POINTER(_Inputs)
        lib.orc_decode_exact.argtypes = [P, I, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p]
        lib.orc_decode_exact.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_set_threads.restype = None
        lib.orc_decode_unified.argtypes = [P, I, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.orc_decode_unified.restype = ctypes.c_int
        lib.orc_scores.argtypes = [P, I, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.orc_scores.restype = ctypes.c_int
        lib.orc_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.orc_decode_bf16.restype = ctypes.c_double
        lib.orc_decode_e4m3fn.argtypes = [ctypes.c_uint8]
        lib.orc_decode_e4m3fn.restype = ctypes.c_double
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _marshal(q, k_cache, v_cache, seq_lens, block_table, num_kv_heads, max_seq_len, page_size,
             q_dtype, kv_dtype, scale, k_scale, v_scale):
    q = np.ascontiguousarray(q, dtype=_NP_DT[q_dtype])
    k_cache = np.ascontiguousarray(k_cache, dtype=_NP_DT[kv_dtype])
    v_cache = np.ascontiguousarray(v_cache, dtype=_NP_DT[kv_dtype])
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, Hq, D = q.shape
    if Hq % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if seq_lens.shape != (B,):
        raise ValueError("seq_lens must have shape [batch]")
    if page_size:
        if block_table is None:
            raise ValueError("paged cache needs a block table")
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        if block_table.ndim != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be [batch][max_blocks]")
        if block_table.shape[1] * page_size < min(max_seq_len, int(seq_lens.max(initial=0))):
            raise ValueError("block_table too narrow for the sequence lengths")
        if k_cache.shape[1:] != (num_kv_heads, page_size, D):
            raise ValueError("paged cache must be [pages][Hkv][page_size][D]")
        max_blocks = block_table.shape[1]
    else:
        block_table = None
        if k_cache.shape != (B, num_kv_heads, max_seq_len, D):
            raise ValueError("contiguous cache must be [B][Hkv][max_seq_len][D]")
        max_blocks = 0
    if kv_dtype == "e4m3fn":
        k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
        v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
        if k_scale.shape != (num_kv_heads,) or v_scale.shape != (num_kv_heads,):
            raise ValueError("k_scale/v_scale must be [num_kv_heads]")
    else:
        k_scale = v_scale = None
    prob = _Problem(B, Hq, num_kv_heads, D, max_seq_len, page_size, max_blocks,
                    _DT[q_dtype], _DT[kv_dtype], float(scale))
    keep = (q, k_cache, v_cache, seq_lens, block_table, k_scale, v_scale)
    ins = _Inputs(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(block_table),
                  _ptr(k_scale), _ptr(v_scale))
    return prob, ins, keep


def _rows(rows, B, Hq):
    if rows is None:
        return None, B * Hq
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    if rows.size and (rows.min() < 0 or rows.max() >= B * Hq):
        raise ValueError("row id out of range")
    return rows, rows.size


def set_threads(n: int) -> None:
    """Caps the oracle's OpenMP threads at n for the calls that follow (n < 1:
    the default, every core)."""
    _load().orc_set_threads(int(n))


def decode_exact(q, k_cache, v_cache, seq_lens, block_table=None, *, num_kv_heads, max_seq_len,
                 page_size=0, q_dtype="bf16", kv_dtype="bf16", scale, phi, a, b, k_scale=None,
                 v_scale=None, rows=None, with_threads=False):
    """Exact softmax decode attention + band flags, float64.

    Returns (out [nrows][D] float64, flags [nrows] uint8, margin [nrows] float64);
    rows are ids b * Hq + h (default: all, in order).  margin is the smallest
    distance of any valid score to a band edge.  With with_threads=True the
    number of OpenMP threads used is appended.
    """
    prob, ins, keep = _marshal(q, k_cache, v_cache, seq_lens, block_table, num_kv_heads,
                               max_seq_len, page_size, q_dtype, kv_dtype, scale, k_scale, v_scale)
    B, Hq, D = keep[0].shape
    rows, n = _rows(rows, B, Hq)
    out = np.zeros((n, D), dtype=np.float64)
    flags = np.zeros(n, dtype=np.uint8)
    margin = np.zeros(n, dtype=np.float64)
    th = _load().orc_decode_exact(ctypes.byref(prob), ctypes.byref(ins), phi, a, b, n, _ptr(rows),
                                  _ptr(out), _ptr(flags), _ptr(margin))
    return (out, flags, margin, th) if with_threads else (out, flags, margin)


def decode_unified(q, k_cache, v_cache, seq_lens, block_table=None, *, num_kv_heads, max_seq_len,
                   page_size=0, q_dtype="bf16", kv_dtype="bf16", scale, phi, a, b, chunk_size,
                   k_scale=None, v_scale=None, rows=None):
    """The method's steps in float64 (unified-max chunk partials, band test,
    online-softmax recompute of flagged chunks, merge).

    Returns (out [nrows][D] float64, flags [nrows] uint8, recomputed chunks [nrows] int32).
    """
    prob, ins, keep = _marshal(q, k_cache, v_cache, seq_lens, block_table, num_kv_heads,
                               max_seq_len, page_size, q_dtype, kv_dtype, scale, k_scale, v_scale)
    B, Hq, D = keep[0].shape
    rows, n = _rows(rows, B, Hq)
    out = np.zeros((n, D), dtype=np.float64)
    flags = np.zeros(n, dtype=np.uint8)
    rec = np.zeros(n, dtype=np.int32)
    rc = _load().orc_decode_unified(ctypes.byref(prob), ctypes.byref(ins), int(chunk_size), phi, a,
                                    b, n, _ptr(rows), _ptr(out), _ptr(flags), _ptr(rec))
    if rc < 0:
        raise ValueError("chunk_size must be positive")
    return out, flags, rec


def scores(q, k_cache, v_cache, seq_lens, block_table=None, *, num_kv_heads, max_seq_len,
           page_size=0, q_dtype="bf16", kv_dtype="bf16", scale, batch_index, head,
           k_scale=None, v_scale=None, **_ignored):
    """float64 scores s_t = scale * q . k_t of one row, t < seq_lens[b]."""
    prob, ins, keep = _marshal(q, k_cache, v_cache, seq_lens, block_table, num_kv_heads,
                               max_seq_len, page_size, q_dtype, kv_dtype, scale, k_scale, v_scale)
    L = int(np.clip(keep[3][batch_index], 0, max_seq_len))
    s = np.zeros(max(L, 1), dtype=np.float64)
    n = _load().orc_scores(ctypes.byref(prob), ctypes.byref(ins), int(batch_index), int(head),
                           _ptr(s))
    return s[:n]


def decode_e4m3fn(codes) -> np.ndarray:
    """E4M3FN codes -> float64 values, through the oracle's own decoder."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([lib.orc_decode_e4m3fn(int(x)) for x in c], dtype=np.float64)


def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 values, through the oracle's own decoder."""
    lib = _load()
    c = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.orc_decode_bf16(int(x)) for x in c], dtype=np.float64)


# ---------------------------------------------------------------------------
# prefill: a block of q_len queries per sequence, causal against its keys
# ---------------------------------------------------------------------------

class _PrefillProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("scale", ctypes.c_double)]


class _PrefillInputs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("kv_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


def _load_prefill():
    lib = _load()
    if not getattr(lib, "_prefill_ready", False):
        P, I = ctypes.POINTER(_PrefillProblem), ctypes.POINTER(_PrefillInputs)
        lib.orc_prefill_exact.argtypes = [P, I, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
        lib.orc_prefill_exact.restype = ctypes.c_int
        lib.orc_prefill_unified.argtypes = [P, I, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                            ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.orc_prefill_unified.restype = ctypes.c_int
        lib._prefill_ready = True
    return lib


def _marshal_prefill(q, k, v, kv_lens, num_kv_heads, q_dtype, kv_dtype, scale, block_table=None,
                     page_size=0, max_seq_len=None, k_scale=None, v_scale=None):
    q = np.ascontiguousarray(q, dtype=_NP_DT[q_dtype])
    k = np.ascontiguousarray(k, dtype=_NP_DT[kv_dtype])
    v = np.ascontiguousarray(v, dtype=_NP_DT[kv_dtype])
    kv_lens = np.ascontiguousarray(kv_lens, dtype=np.int32)
    if q_dtype == "e4m3fn":
        raise ValueError("prefill queries are f32 or bf16")
    B, Hq, Lq, D = q.shape
    if Hq % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if k.ndim != 4 or k.shape[1] != num_kv_heads or k.shape[3] != D or v.shape != k.shape:
        raise ValueError("k and v must be [B][Hkv][max_seq_len][D] or [pages][Hkv][page_size][D]")
    if kv_lens.shape != (B,):
        raise ValueError("kv_lens must have shape [batch]")
    max_blocks = 0
    if page_size:
        if block_table is None or k.shape[2] != page_size:
            raise ValueError("paged K/V need a block table and [pages][Hkv][page_size][D] caches")
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        max_blocks = block_table.shape[1]
        if max_seq_len is None or max_blocks * page_size < max_seq_len:
            raise ValueError("paged K/V need max_seq_len <= max_blocks * page_size")
    else:
        if k.shape[0] != B:
            raise ValueError("contiguous K/V are [B][Hkv][max_seq_len][D]")
        max_seq_len = k.shape[2]
        block_table = None
    if kv_dtype == "e4m3fn":
        if k_scale is None or v_scale is None:
            raise ValueError("E4M3FN caches need k_scale and v_scale")
        k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
        v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
    else:
        k_scale = v_scale = None
    prob = _PrefillProblem(B, Hq, num_kv_heads, D, int(max_seq_len), Lq, _DT[q_dtype], _DT[kv_dtype],
                           int(page_size), int(max_blocks), float(scale))
    keep = (q, k, v, kv_lens, block_table, k_scale, v_scale)
    ins = _PrefillInputs(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_lens),
                         None if block_table is None else _ptr(block_table),
                         None if k_scale is None else _ptr(k_scale),
                         None if v_scale is None else _ptr(v_scale))
    return prob, ins, keep


def _prefill_rows(rows, total):
    if rows is None:
        return None, total
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    if rows.size and (rows.min() < 0 or rows.max() >= total):
        raise ValueError("row id out of range")
    return rows, rows.size


def prefill_exact(q, k, v, kv_lens, *, num_kv_heads, q_dtype="bf16", kv_dtype="bf16", scale,
                  phi, a, b, rows=None, with_threads=False, block_table=None, page_size=0,
                  max_seq_len=None, k_scale=None, v_scale=None):
    """Exact causal softmax attention of a query block + band flags, float64.

    q [B][Hq][Lq][D]; k, v contiguous [B][Hkv][max_seq_len][D] or, with
    page_size > 0, paged [pages][Hkv][page_size][D] with block_table
    [B][max_blocks] (max_seq_len then given); E4M3FN K/V codes are multiplied
    by k_scale / v_scale [Hkv].  Query j of sequence b sits at position
    kv_lens[b] - Lq + j and sees keys 0..position (none if negative).  Rows
    are ids (b * Hq + h) * Lq + j (default: all, in order).  Returns
    (out [nrows][D], flags [nrows] uint8, margin [nrows]); margin is the
    smallest distance of a visible score to a band edge.
    """
    prob, ins, keep = _marshal_prefill(q, k, v, kv_lens, num_kv_heads, q_dtype, kv_dtype, scale,
                                       block_table, page_size, max_seq_len, k_scale, v_scale)
    B, Hq, Lq, D = keep[0].shape
    rows, n = _prefill_rows(rows, B * Hq * Lq)
    out = np.zeros((n, D), dtype=np.float64)
    flags = np.zeros(n, dtype=np.uint8)
    margin = np.zeros(n, dtype=np.float64)
    th = _load_prefill().orc_prefill_exact(ctypes.byref(prob), ctypes.byref(ins), phi, a, b, n,
                                           _ptr(rows), _ptr(out), _ptr(flags), _ptr(margin))
    return (out, flags, margin, th) if with_threads else (out, flags, margin)


def prefill_unified(q, k, v, kv_lens, *, num_kv_heads, q_dtype="bf16", kv_dtype="bf16", scale,
                    phi, a, b, tile, rows=None, block_table=None, page_size=0, max_seq_len=None,
                    k_scale=None, v_scale=None):
    """The method's steps for a causal query block, float64: key tiles of `tile`
    tokens reduced against phi, online-softmax redo of a tile with a visible
    out-of-band score, merge.  Cache layouts as prefill_exact.  Returns (out,
    flags, redone tiles [nrows] int32)."""
    prob, ins, keep = _marshal_prefill(q, k, v, kv_lens, num_kv_heads, q_dtype, kv_dtype, scale,
                                       block_table, page_size, max_seq_len, k_scale, v_scale)
    B, Hq, Lq, D = keep[0].shape
    rows, n = _prefill_rows(rows, B * Hq * Lq)
    out = np.zeros((n, D), dtype=np.float64)
    flags = np.zeros(n, dtype=np.uint8)
    red = np.zeros(n, dtype=np.int32)
    rc = _load_prefill().orc_prefill_unified(ctypes.byref(prob), ctypes.byref(ins), int(tile), phi,
                                             a, b, n, _ptr(rows), _ptr(out), _ptr(flags), _ptr(red))
    if rc < 0:
        raise ValueError("tile must be positive")
    return out, flags, red


# ---------------------------------------------------------------------------
# calibration: score extremes and histogram, band choice
# ---------------------------------------------------------------------------

def _load_calib():
    lib = _load()
    if not getattr(lib, "_calib_ready", False):
        P, I = ctypes.POINTER(_Problem), ctypes.POINTER(_Inputs)
        lib.orc_score_stats.argtypes = [P, I, ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.orc_score_stats.restype = ctypes.c_int
        lib.orc_rows_in_band.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_double, ctypes.c_double, ctypes.c_double]
        lib.orc_rows_in_band.restype = ctypes.c_int64
        lib.orc_min_band_width.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int64]
        lib.orc_min_band_width.restype = ctypes.c_double
        lib._calib_ready = True
    return lib


def score_stats(q, k_cache, v_cache, seq_lens, block_table=None, *, num_kv_heads, max_seq_len,
                page_size=0, q_dtype="bf16", kv_dtype="bf16", scale, k_scale=None, v_scale=None,
                hist_lo=-16.0, hist_hi=16.0, nbins=0, with_threads=False, **_ignored):
    """Per-row largest and smallest valid score (float64; empty rows -inf / +inf)
    and, if nbins > 0, the histogram counts [below, bin 0 .. nbins-1, at or above]
    of every valid score over [hist_lo, hist_hi)."""
    prob, ins, keep = _marshal(q, k_cache, v_cache, seq_lens, block_table, num_kv_heads,
                               max_seq_len, page_size, q_dtype, kv_dtype, scale, k_scale, v_scale)
    B, Hq, _ = keep[0].shape
    mx = np.zeros(B * Hq, dtype=np.float64)
    mn = np.zeros(B * Hq, dtype=np.float64)
    counts = np.zeros(max(nbins, 0) + 2, dtype=np.int64)
    th = _load_calib().orc_score_stats(ctypes.byref(prob), ctypes.byref(ins), float(hist_lo),
                                       float(hist_hi), int(nbins), _ptr(mx), _ptr(mn), _ptr(counts))
    res = (mx, mn, counts if nbins > 0 else None)
    return res + (th,) if with_threads else res


def rows_in_band(row_max, row_min, phi, a, b) -> int:
    """Non-empty rows whose extremes lie inside [phi - a, phi + b] (float64)."""
    mx = np.ascontiguousarray(row_max, dtype=np.float64)
    mn = np.ascontiguousarray(row_min, dtype=np.float64)
    return int(_load_calib().orc_rows_in_band(_ptr(mx), _ptr(mn), mx.size, float(phi), float(a),
                                              float(b)))


def min_band_width(row_max, row_min, allowed) -> float:
    """Smallest band width a + b for which all but `allowed` non-empty rows fit
    (float64, exact over the given extremes; 0 if no row needs to fit)."""
    mx = np.ascontiguousarray(row_max, dtype=np.float64)
    mn = np.ascontiguousarray(row_min, dtype=np.float64)
    return float(_load_calib().orc_min_band_width(_ptr(mx), _ptr(mn), mx.size, int(allowed)))


# ---------------------------------------------------------------------------
# flat GEMM of the decode linear layers
# ---------------------------------------------------------------------------

def flat_gemm(a, w, *, a_dtype="bf16", w_dtype="bf16"):
    """C = A . W^T in float64 (FlashDecoding++ theory page, section 2 item 2 and
    section 4: the linear layers of decoding multiply a flat activation matrix
    A [M][K], M small, by the weights W [N][K]).

    The operands are decoded from their storage format by the oracle's own
    decoders (bf16: upper half of a binary32; f32 as stored); the product is
    numpy's float64 matrix multiply.  Returns C [M][N] float64.
    """
    def dec(x, dt):
        x = np.ascontiguousarray(x)
        if dt == "f32":
            return x.astype(np.float64)
        if dt == "bf16":
            return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        raise ValueError("flat GEMM operands are f32 or bf16")
    A = dec(a, a_dtype)
    W = dec(w, w_dtype)
    if A.ndim != 2 or W.ndim != 2 or A.shape[1] != W.shape[1]:
        raise ValueError("A must be [M][K] and W [N][K]")
    return A @ W.T


def flat_gemm_abs(a, w, *, a_dtype="bf16", w_dtype="bf16"):
    """|A| . |W|^T in float64: the scale of the rounding error bound of an
    fp32 accumulation of C = A . W^T."""
    return flat_gemm(np.abs(_as_f32(a, a_dtype)), np.abs(_as_f32(w, w_dtype)), a_dtype="f32",
                     w_dtype="f32")


def _as_f32(x, dt):
    x = np.ascontiguousarray(x)
    if dt == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x.astype(np.float32)
