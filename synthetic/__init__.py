"""Seeded synthetic inputs for unified-max split-KV decode attention.

The pages measure no public benchmark; these generators stand in for the
workloads they describe: a single decode query per (batch, head) against a
long, optionally ragged and optionally paged KV cache (FlashDecoding++ theory
page, section 1; export-strategy page, section 2).

This module draws numbers and stores them in the caller-visible storage
formats (fp32, bf16 bit patterns, OCP E4M3FN codes).  It holds none of the
attention arithmetic: no scores, exponentials, band tests or merges.  Both the
float64 oracle and the GPU library consume what it returns.

Recipe:
  * every value ~ N(0, 1), drawn as float32 from numpy's PCG64 stream keyed by
    (seed, tensor id, batch, kv head), so any subset of rows can be drawn
    alone and is identical to the same rows of a full draw;
  * bf16 storage: float32 rounded to nearest-even on the upper 16 bits;
  * E4M3FN storage: per-KV-head scale = max|x| / 448 over that head's draws,
    code = nearest-even E4M3FN of x / scale (saturating at +-448);
  * ragged lengths ~ U{lo..hi} inclusive; paged caches place tokens in
    16-token pages whose physical ids are a seeded permutation of the pool,
    assigned in (batch, token) order, unused table slots = -1;
  * limit cases: one sequence of up to 2^23 tokens drawn in parallel blocks
    of rows (make_long_sequence), and a large batch whose sequences share the
    pages of a small paged problem (share_pages).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

__all__ = ["Problem", "CONFIGS", "make_config", "make_problem", "make_long_sequence",
           "share_pages", "PrefillProblem", "PREFILL_CONFIGS", "make_prefill",
           "make_prefill_config", "bf16_round", "bf16_to_f32", "e4m3fn_encode", "e4m3fn_values"]

HEAD_DIM = 128
SEED_BASE = 0x5EED0000

# stream ids (second word of the numpy seed sequence)
_S_Q, _S_K, _S_V, _S_LENS, _S_PERM, _S_PAIRS = 1, 2, 3, 4, 5, 6

# The five workloads.  Field names match the arguments of the library and of
# the oracle.  "lens" is ("fixed", L) or ("uniform", lo, hi).
CONFIGS = {
    1: dict(workload="mha1x1-L4096-f32", batch=1, num_q_heads=1, num_kv_heads=1,
            lens=("fixed", 4096), max_seq_len=4096, q_dtype="f32", kv_dtype="f32",
            page_size=0, chunk_size=1024, phi=3.0, a=20.0, b=8.0),
    2: dict(workload="mha8x32-L8192-bf16", batch=8, num_q_heads=32, num_kv_heads=32,
            lens=("fixed", 8192), max_seq_len=8192, q_dtype="bf16", kv_dtype="bf16",
            page_size=0, chunk_size=512, phi=4.0, a=20.0, b=6.0),
    3: dict(workload="gqa32x64/8-L1k..32k-bf16", batch=32, num_q_heads=64, num_kv_heads=8,
            lens=("uniform", 1024, 32768), max_seq_len=32768, q_dtype="bf16", kv_dtype="bf16",
            page_size=0, chunk_size=1024, phi=4.0, a=20.0, b=6.0),
    4: dict(workload="mha1x32-L131072-bf16-1pct-fallback", batch=1, num_q_heads=32,
            num_kv_heads=32, lens=("fixed", 131072), max_seq_len=131072, q_dtype="bf16",
            kv_dtype="bf16", page_size=0, chunk_size=1024, phi=4.0, a=20.0, b=6.0,
            perturb_fraction=0.01, perturb_factor=8.0),
    5: dict(workload="paged16-gqa64x32/8-L512..16k-fp8e4m3", batch=64, num_q_heads=32,
            num_kv_heads=8, lens=("uniform", 512, 16384), max_seq_len=16384, q_dtype="bf16",
            kv_dtype="e4m3fn", page_size=16, chunk_size=512, phi=4.0, a=16.0, b=6.0),
}

_PLAN_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "tests", "golden", "config4_perturbation.txt")


@dataclasses.dataclass
class Problem:
    """One decode-attention call's inputs, in storage format (host arrays)."""
    q: np.ndarray                 # [B][Hq][D]; float32 or uint16 (bf16 bits)
    k_cache: np.ndarray           # contiguous [B][Hkv][Lmax][D] or paged [pages][Hkv][P][D]
    v_cache: np.ndarray
    seq_lens: np.ndarray          # int32 [B]
    block_table: Optional[np.ndarray]  # int32 [B][max_blocks] or None
    num_kv_heads: int
    max_seq_len: int
    page_size: int
    q_dtype: str                  # "f32" | "bf16"
    kv_dtype: str                 # "f32" | "bf16" | "e4m3fn"
    scale: float
    phi: float
    a: float
    b: float
    chunk_size: int
    k_scale: Optional[np.ndarray] = None   # float32 [Hkv] (E4M3FN only)
    v_scale: Optional[np.ndarray] = None
    workload: str = "custom"
    perturbed: Optional[np.ndarray] = None  # int32 [n][3] (head, chunk, token), batch 0

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[1]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]

    def kv_bytes(self) -> int:
        """Bytes of valid K and V elements (each read once by the method)."""
        elt = {"f32": 4, "bf16": 2, "e4m3fn": 1}[self.kv_dtype]
        return int(np.clip(self.seq_lens, 0, self.max_seq_len).astype(np.int64).sum()) \
            * self.num_kv_heads * self.head_dim * 2 * elt

    def args(self) -> dict:
        """Keyword arguments shared by the oracle and the library binding."""
        return dict(q=self.q, k_cache=self.k_cache, v_cache=self.v_cache,
                    seq_lens=self.seq_lens, block_table=self.block_table,
                    num_kv_heads=self.num_kv_heads, max_seq_len=self.max_seq_len,
                    page_size=self.page_size, q_dtype=self.q_dtype,
                    kv_dtype=self.kv_dtype, scale=self.scale, phi=self.phi,
                    a=self.a, b=self.b, k_scale=self.k_scale, v_scale=self.v_scale)


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))))
            >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def e4m3fn_values() -> np.ndarray:
    """The 127 finite non-negative OCP E4M3FN values, codes 0x00..0x7E, ascending.

    Used only for encoding: exponent bias 7, 3 mantissa bits, codes with
    exponent field 0 are subnormal (m * 2^-9), 0x7F is NaN, no infinities.
    """
    vals = np.empty(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_VALS = e4m3fn_values()
_E4M3_MID = (_E4M3_VALS[:-1] + _E4M3_VALS[1:]) / 2.0   # rounding thresholds


def e4m3fn_encode(y: np.ndarray) -> np.ndarray:
    """float -> E4M3FN codes (uint8): nearest, ties to even code, saturating at 448."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.minimum(np.abs(y), 448.0)
    idx = np.searchsorted(_E4M3_MID, mag, side="left")      # first midpoint >= mag
    # exactly on a midpoint: searchsorted(left) picked the lower code; ties go to the even one
    on_mid = (idx < _E4M3_MID.size) & (mag == _E4M3_MID[np.minimum(idx, _E4M3_MID.size - 1)])
    idx = np.where(on_mid & (idx % 2 == 1), idx + 1, idx)
    code = idx.astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << np.uint8(7)
    return code | sign


# ----------------------------------------------------------------------------
# drawing
# ----------------------------------------------------------------------------

def _rng(seed: int, stream: int, *keys: int) -> np.random.Generator:
    return np.random.default_rng([seed & 0xFFFFFFFF, stream, *[int(k) for k in keys]])


def _draw_kv_rows(seed: int, stream: int, b: int, kvh: int, n: int, d: int) -> np.ndarray:
    return _rng(seed, stream, b, kvh).standard_normal((n, d), dtype=np.float32)


def _draw_lens(spec, batch: int, seed: int) -> np.ndarray:
    if spec[0] == "fixed":
        return np.full(batch, spec[1], dtype=np.int32)
    lo, hi = spec[1], spec[2]
    return _rng(seed, _S_LENS).integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_problem(*, batch: int, num_q_heads: int, num_kv_heads: int, seq_lens,
                 q_dtype: str = "bf16", kv_dtype: str = "bf16", page_size: int = 0,
                 chunk_size: int = 512, phi: float = 4.0, a: float = 20.0, b: float = 6.0,
                 max_seq_len: Optional[int] = None, scale: Optional[float] = None,
                 head_dim: int = HEAD_DIM, seed: int = SEED_BASE, workload: str = "custom",
                 value_sigma: float = 1.0, extra_pages: int = 0) -> Problem:
    """Draw one problem.  seq_lens: int or sequence of ints (may include 0)."""
    if np.isscalar(seq_lens):
        seq_lens = np.full(batch, int(seq_lens), dtype=np.int32)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (batch,)
    if max_seq_len is None:
        max_seq_len = max(1, int(seq_lens.max(initial=0)))
    if page_size:
        max_seq_len = -(-max_seq_len // page_size) * page_size
    assert num_q_heads % num_kv_heads == 0
    D = head_dim
    if scale is None:
        scale = 1.0 / math.sqrt(D)

    # query
    qf = _rng(seed, _S_Q).standard_normal((batch, num_q_heads, D), dtype=np.float32) * value_sigma
    q = qf if q_dtype == "f32" else bf16_round(qf)

    # K/V draws per (batch, kv head), only valid tokens
    lens = np.clip(seq_lens, 0, max_seq_len)
    jobs = [(b_, h) for b_ in range(batch) for h in range(num_kv_heads)]

    def draw(job, stream):
        b_, h = job
        return _draw_kv_rows(seed, stream, b_, h, int(lens[b_]), D) * np.float32(value_sigma)

    with ThreadPoolExecutor(_threads()) as ex:
        kf = list(ex.map(lambda j: draw(j, _S_K), jobs))
        vf = list(ex.map(lambda j: draw(j, _S_V), jobs))

    k_scale = v_scale = None
    if kv_dtype == "e4m3fn":
        k_scale = np.zeros(num_kv_heads, dtype=np.float32)
        v_scale = np.zeros(num_kv_heads, dtype=np.float32)
        for h in range(num_kv_heads):
            mk = max([float(np.abs(kf[i]).max(initial=0.0)) for i, j in enumerate(jobs) if j[1] == h])
            mv = max([float(np.abs(vf[i]).max(initial=0.0)) for i, j in enumerate(jobs) if j[1] == h])
            k_scale[h] = np.float32(mk / 448.0) if mk > 0 else np.float32(1.0)
            v_scale[h] = np.float32(mv / 448.0) if mv > 0 else np.float32(1.0)

    def store(i, arrs, sc):
        x = arrs[i]
        if kv_dtype == "f32":
            return x
        if kv_dtype == "bf16":
            return bf16_round(x)
        return e4m3fn_encode(x / sc[jobs[i][1]])

    with ThreadPoolExecutor(_threads()) as ex:
        ks = list(ex.map(lambda i: store(i, kf, k_scale), range(len(jobs))))
        vs = list(ex.map(lambda i: store(i, vf, v_scale), range(len(jobs))))
    del kf, vf

    sdt = {"f32": np.float32, "bf16": np.uint16, "e4m3fn": np.uint8}[kv_dtype]
    block_table = None
    if page_size == 0:
        k_cache = np.zeros((batch, num_kv_heads, max_seq_len, D), dtype=sdt)
        v_cache = np.zeros_like(k_cache)
        for i, (b_, h) in enumerate(jobs):
            n = int(lens[b_])
            k_cache[b_, h, :n] = ks[i]
            v_cache[b_, h, :n] = vs[i]
    else:
        P = page_size
        max_blocks = max_seq_len // P
        pages_per_seq = [-(-int(n) // P) for n in lens]
        pool = int(sum(pages_per_seq)) + int(extra_pages)
        perm = _rng(seed, _S_PERM).permutation(pool).astype(np.int32)
        block_table = np.full((batch, max(1, max_blocks)), -1, dtype=np.int32)
        k_cache = np.zeros((max(1, pool), num_kv_heads, P, D), dtype=sdt)
        v_cache = np.zeros_like(k_cache)
        nxt = 0
        for b_ in range(batch):
            for blk in range(pages_per_seq[b_]):
                block_table[b_, blk] = perm[nxt]
                nxt += 1
        for i, (b_, h) in enumerate(jobs):
            n = int(lens[b_])
            for blk in range(pages_per_seq[b_]):
                t0, t1 = blk * P, min(n, (blk + 1) * P)
                pg = block_table[b_, blk]
                k_cache[pg, h, :t1 - t0] = ks[i][t0:t1]
                v_cache[pg, h, :t1 - t0] = vs[i][t0:t1]
    return Problem(q=q, k_cache=k_cache, v_cache=v_cache, seq_lens=seq_lens,
                   block_table=block_table, num_kv_heads=num_kv_heads,
                   max_seq_len=max_seq_len, page_size=page_size, q_dtype=q_dtype,
                   kv_dtype=kv_dtype, scale=float(scale), phi=float(phi), a=float(a),
                   b=float(b), chunk_size=chunk_size, k_scale=k_scale, v_scale=v_scale,
                   workload=workload)


def perturbation_pairs(num_heads: int, num_chunks: int, fraction: float, seed: int) -> np.ndarray:
    """(head, chunk) pairs, round(fraction * H * C) of them, uniform without replacement."""
    n = int(round(fraction * num_heads * num_chunks))
    flat = _rng(seed, _S_PAIRS).choice(num_heads * num_chunks, size=n, replace=False)
    flat.sort()
    return np.stack([flat // num_chunks, flat % num_chunks], axis=1).astype(np.int32)


def load_perturbation_plan(path: str = _PLAN_FILE) -> np.ndarray:
    """Rows (head, chunk, token) of the stored config-4 plan (batch 0)."""
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.asarray(rows, dtype=np.int32).reshape(-1, 3)


def apply_key_scaling(prob: Problem, plan: np.ndarray, factor: float) -> None:
    """Multiply the listed keys (batch 0) by `factor` in place (exact for a power of two)."""
    for h, _c, t in plan:
        row = prob.k_cache[0, h, t]
        if prob.kv_dtype == "bf16":
            prob.k_cache[0, h, t] = bf16_round(bf16_to_f32(row) * np.float32(factor))
        elif prob.kv_dtype == "f32":
            prob.k_cache[0, h, t] = row * np.float32(factor)
        else:
            raise ValueError("key scaling is defined for f32/bf16 caches")
    prob.perturbed = np.asarray(plan, dtype=np.int32)


_S_LONG_K, _S_LONG_V = 10, 11


def make_long_sequence(length: int, *, num_q_heads: int, num_kv_heads: int = 1,
                       chunk_size: int = 0, phi: float = 4.0, a: float = 20.0, b: float = 6.0,
                       seed: int = SEED_BASE + 0x40, block: int = 1 << 20) -> Problem:
    """One sequence of `length` tokens, contiguous bf16 cache, N(0, 1) values.

    K/V rows of each KV head are drawn in blocks of `block` tokens, block i
    from its own stream keyed by (seed, tensor id, kv head, i), so the blocks
    are drawn (and rounded to bf16) in parallel straight into the cache."""
    D = HEAD_DIM
    q = bf16_round(_rng(seed, _S_Q).standard_normal((1, num_q_heads, D), dtype=np.float32))
    k_cache = np.empty((1, num_kv_heads, length, D), dtype=np.uint16)
    v_cache = np.empty_like(k_cache)
    pieces = [(cache, stream, h, i) for cache, stream in ((k_cache, _S_LONG_K), (v_cache, _S_LONG_V))
              for h in range(num_kv_heads) for i in range(-(-length // block))]

    def fill(piece):
        cache, stream, h, i = piece
        t0, t1 = i * block, min(length, (i + 1) * block)
        cache[0, h, t0:t1] = bf16_round(
            _rng(seed, stream, h, i).standard_normal((t1 - t0, D), dtype=np.float32))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, pieces))
    return Problem(q=q, k_cache=k_cache, v_cache=v_cache,
                   seq_lens=np.array([length], dtype=np.int32), block_table=None,
                   num_kv_heads=num_kv_heads, max_seq_len=length, page_size=0, q_dtype="bf16",
                   kv_dtype="bf16", scale=1.0 / math.sqrt(D), phi=phi, a=a, b=b,
                   chunk_size=chunk_size, workload="long-sequence")


def share_pages(prob: Problem, batch: int, *, chunk_size: Optional[int] = None,
                seed: Optional[int] = None) -> Problem:
    """A larger batch over the page pool of a paged problem: sequence b reads
    the pages of sequence b % prob.batch (pages shared between sequences, as a
    common prefix is), with its own queries drawn for the new batch.  The
    cache stays small while the batch, and with it every per-row and per-chunk
    index of a call, grows."""
    assert prob.page_size and prob.block_table is not None
    seed = SEED_BASE + 0x51 if seed is None else seed
    src = np.arange(batch) % prob.batch
    qf = _rng(seed, _S_Q).standard_normal((batch, prob.num_q_heads, prob.head_dim),
                                          dtype=np.float32)
    q = qf if prob.q_dtype == "f32" else bf16_round(qf)
    return dataclasses.replace(
        prob, q=q, seq_lens=np.ascontiguousarray(prob.seq_lens[src]),
        block_table=np.ascontiguousarray(prob.block_table[src]),
        chunk_size=prob.chunk_size if chunk_size is None else chunk_size,
        workload="shared-pages", perturbed=None)


def make_config(cfg: int, *, batch: Optional[int] = None, length: Optional[int] = None,
                lens: Optional[tuple] = None, seed: Optional[int] = None,
                perturb: bool = True) -> Problem:
    """The numbered workload, optionally shrunk (batch, fixed length or length range)."""
    c = dict(CONFIGS[cfg])
    seed = SEED_BASE + cfg if seed is None else seed
    B = batch or c["batch"]
    spec = c["lens"]
    if length is not None:
        spec = ("fixed", length)
    elif lens is not None:
        spec = ("uniform", lens[0], lens[1])
    seq = _draw_lens(spec, B, seed)
    max_len = c["max_seq_len"] if (batch is None and length is None and lens is None) else int(
        spec[1] if spec[0] == "fixed" else spec[2])
    prob = make_problem(batch=B, num_q_heads=c["num_q_heads"], num_kv_heads=c["num_kv_heads"],
                        seq_lens=seq, q_dtype=c["q_dtype"], kv_dtype=c["kv_dtype"],
                        page_size=c["page_size"], chunk_size=c["chunk_size"], phi=c["phi"],
                        a=c["a"], b=c["b"], max_seq_len=max_len, seed=seed,
                        workload=c["workload"])
    if cfg == 4 and perturb and batch is None and length is None:
        apply_key_scaling(prob, load_perturbation_plan(), c["perturb_factor"])
    return prob


# ----------------------------------------------------------------------------
# prefill: a causal block of query tokens per sequence
# ----------------------------------------------------------------------------

_S_PQ, _S_PK, _S_PV = 7, 8, 9

# Prefill workloads.  "lens" as above gives kv_lens; q_len queries sit at the
# end of each sequence (q_len == kv_len: a whole prompt; q_len < kv_len: a new
# block appended to a cached prefix).
PREFILL_CONFIGS = {
    1: dict(workload="prefill-gqa2x4/1-Lq300-kv300..517-bf16", batch=2, num_q_heads=4,
            num_kv_heads=1, q_len=300, lens=("uniform", 300, 517), max_seq_len=517,
            phi=4.0, a=20.0, b=6.0),
    2: dict(workload="prefill-gqa2x32/8-L8192-causal-bf16", batch=2, num_q_heads=32,
            num_kv_heads=8, q_len=8192, lens=("fixed", 8192), max_seq_len=8192,
            phi=4.0, a=20.0, b=6.0),
}


@dataclasses.dataclass
class PrefillProblem:
    """One prefill call's inputs (storage formats, host arrays)."""
    q: np.ndarray                 # [B][Hq][Lq][D]; bf16 bit patterns or float32
    k: np.ndarray                 # contiguous [B][Hkv][max_seq_len][D] or paged [pages][Hkv][P][D]
    v: np.ndarray
    kv_lens: np.ndarray           # int32 [B]
    num_kv_heads: int
    dtype: str                    # queries: "bf16" | "f32"
    scale: float
    phi: float
    a: float
    b: float
    workload: str = "custom"
    kv_dtype: Optional[str] = None         # cache format ("bf16" | "f32" | "e4m3fn"); None: as dtype
    page_size: int = 0
    block_table: Optional[np.ndarray] = None   # int32 [B][max_blocks] (paged)
    paged_max_seq_len: int = 0                 # max_seq_len of a paged cache
    k_scale: Optional[np.ndarray] = None       # float32 [Hkv] (E4M3FN)
    v_scale: Optional[np.ndarray] = None

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[1]

    @property
    def q_len(self) -> int:
        return self.q.shape[2]

    @property
    def head_dim(self) -> int:
        return self.q.shape[3]

    @property
    def max_seq_len(self) -> int:
        return self.paged_max_seq_len if self.page_size else self.k.shape[2]

    def visible_pairs(self) -> int:
        """(query, key) pairs that are attended, summed over heads."""
        kv = np.clip(self.kv_lens.astype(np.int64), 0, self.max_seq_len)
        pos = kv[:, None] - self.q_len + np.arange(self.q_len)[None, :]
        return int(np.clip(pos + 1, 0, None).sum()) * self.num_q_heads

    def args(self) -> dict:
        """Keyword arguments shared by the oracle and the library binding."""
        a = dict(q=self.q, k=self.k, v=self.v, kv_lens=self.kv_lens,
                 num_kv_heads=self.num_kv_heads, q_dtype=self.dtype, kv_dtype=self.cache_dtype,
                 scale=self.scale, phi=self.phi, a=self.a, b=self.b)
        if self.page_size:
            a.update(block_table=self.block_table, page_size=self.page_size,
                     max_seq_len=self.max_seq_len)
        if self.cache_dtype == "e4m3fn":
            a.update(k_scale=self.k_scale, v_scale=self.v_scale)
        return a


def make_prefill(*, batch: int, num_q_heads: int, num_kv_heads: int, q_len: int, kv_lens,
                 dtype: str = "bf16", phi: float = 4.0, a: float = 20.0, b: float = 6.0,
                 max_seq_len: Optional[int] = None, scale: Optional[float] = None,
                 head_dim: int = HEAD_DIM, seed: int = SEED_BASE + 100,
                 workload: str = "custom", value_sigma: float = 1.0, kv_dtype: Optional[str] = None,
                 page_size: int = 0, extra_pages: int = 0) -> PrefillProblem:
    """Draw one prefill problem: N(0, value_sigma^2) queries, keys and values;
    keys/values drawn for the first kv_lens[b] positions, zero beyond.  The
    cache is stored as kv_dtype (default: dtype; E4M3FN with a per-KV-head
    scale max|x| / 448 as in make_problem), contiguous or in pages of
    page_size tokens with a seeded page permutation (unused slots zero).  The
    float32 draws are the same for every format and layout."""
    if np.isscalar(kv_lens):
        kv_lens = np.full(batch, int(kv_lens), dtype=np.int32)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    assert kv_lens.shape == (batch,)
    assert num_q_heads % num_kv_heads == 0
    kvd = kv_dtype or dtype
    if max_seq_len is None:
        max_seq_len = max(1, int(kv_lens.max(initial=0)))
    if page_size:
        max_seq_len = -(-max_seq_len // page_size) * page_size
    D = head_dim
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lens = np.clip(kv_lens, 0, max_seq_len)
    sdt = np.float32 if dtype == "f32" else np.uint16

    def conv(x):
        return x if dtype == "f32" else bf16_round(x)

    q = np.zeros((batch, num_q_heads, q_len, D), dtype=sdt)
    kf = np.zeros((batch, num_kv_heads, max_seq_len, D), dtype=np.float32)
    vf = np.zeros_like(kf)
    sig = np.float32(value_sigma)

    def fill_q(job):
        b_, h = job
        q[b_, h] = conv(_rng(seed, _S_PQ, b_, h).standard_normal((q_len, D), dtype=np.float32) * sig)

    def fill_kv(job):
        b_, h = job
        n = int(lens[b_])
        kf[b_, h, :n] = _draw_kv_rows(seed, _S_PK, b_, h, n, D) * sig
        vf[b_, h, :n] = _draw_kv_rows(seed, _S_PV, b_, h, n, D) * sig

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill_q, [(b_, h) for b_ in range(batch) for h in range(num_q_heads)]))
        list(ex.map(fill_kv, [(b_, h) for b_ in range(batch) for h in range(num_kv_heads)]))

    k_scale = v_scale = None
    if kvd == "e4m3fn":
        mk = np.abs(kf).max(axis=(0, 2, 3))
        mv = np.abs(vf).max(axis=(0, 2, 3))
        k_scale = np.where(mk > 0, mk / 448.0, 1.0).astype(np.float32)
        v_scale = np.where(mv > 0, mv / 448.0, 1.0).astype(np.float32)
        k = e4m3fn_encode(kf / k_scale[None, :, None, None])
        v = e4m3fn_encode(vf / v_scale[None, :, None, None])
    elif kvd == "bf16":
        k, v = bf16_round(kf), bf16_round(vf)
    else:
        k, v = kf, vf
    del kf, vf

    block_table = None
    if page_size:
        P = page_size
        pages_per_seq = [-(-int(n) // P) for n in lens]
        pool = int(sum(pages_per_seq)) + int(extra_pages)
        perm = _rng(seed, _S_PERM).permutation(pool).astype(np.int32)
        block_table = np.full((batch, max(1, max_seq_len // P)), -1, dtype=np.int32)
        kp = np.zeros((max(1, pool), num_kv_heads, P, D), dtype=k.dtype)
        vp = np.zeros_like(kp)
        nxt = 0
        for b_ in range(batch):
            for blk in range(pages_per_seq[b_]):
                pg = perm[nxt]
                nxt += 1
                block_table[b_, blk] = pg
                t0, t1 = blk * P, min(int(lens[b_]), (blk + 1) * P)
                kp[pg, :, :t1 - t0] = k[b_, :, t0:t1]
                vp[pg, :, :t1 - t0] = v[b_, :, t0:t1]
        k, v = kp, vp
    return PrefillProblem(q=q, k=k, v=v, kv_lens=kv_lens, num_kv_heads=num_kv_heads, dtype=dtype,
                          scale=float(scale), phi=float(phi), a=float(a), b=float(b),
                          workload=workload, kv_dtype=kv_dtype, page_size=page_size,
                          block_table=block_table, paged_max_seq_len=max_seq_len if page_size else 0,
                          k_scale=k_scale, v_scale=v_scale)


def make_prefill_config(cfg: int, *, batch: Optional[int] = None, q_len: Optional[int] = None,
                        seed: Optional[int] = None) -> PrefillProblem:
    """The numbered prefill workload, optionally shrunk (batch, query block length)."""
    c = dict(PREFILL_CONFIGS[cfg])
    seed = SEED_BASE + 100 + cfg if seed is None else seed
    B = batch or c["batch"]
    Lq = q_len or c["q_len"]
    kv = _draw_lens(c["lens"], B, seed)
    if q_len is not None:
        kv = np.maximum(kv - c["q_len"] + Lq, 0).astype(np.int32)
    return make_prefill(batch=B, num_q_heads=c["num_q_heads"], num_kv_heads=c["num_kv_heads"],
                        q_len=Lq, kv_lens=kv, phi=c["phi"], a=c["a"], b=c["b"],
                        max_seq_len=max(int(kv.max(initial=1)), 1), seed=seed,
                        workload=c["workload"])


# ----------------------------------------------------------------------------
# flat GEMM of the decode linear layers
# ----------------------------------------------------------------------------

_S_GA, _S_GW = 10, 11

# Linear layers of one decoder block of a 7B-class model (hidden 4096, FFN
# 11008; the theory page's section 4 lists them: Q/K/V generation, the O
# projection and the two FFN layers, with K and N fixed by the weights and M
# the tokens of the decode step).  Shapes are (N, K); W is [N][K].
LINEAR_LAYERS_7B = [("qkv", 3 * 4096, 4096), ("o", 4096, 4096), ("gate_up", 2 * 11008, 4096),
                    ("down", 4096, 11008)]

GEMM_CONFIGS = {
    1: dict(workload="flatgemm-small-M5-N200-K96", m=5, layers=[("w", 200, 96)]),
    2: dict(workload="flatgemm-7b-block-M16-bf16", m=16, layers=LINEAR_LAYERS_7B),
}


def make_gemm(m: int, n: int, k: int, *, seed: int = SEED_BASE + 200, layer: int = 0,
              dtype: str = "bf16"):
    """Activations A [m][k] and weights W [n][k], N(0, 1), in storage format."""
    a = _rng(seed, _S_GA, layer).standard_normal((m, k), dtype=np.float32)
    w = _rng(seed, _S_GW, layer).standard_normal((n, k), dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(a), bf16_round(w)
    return a, w
