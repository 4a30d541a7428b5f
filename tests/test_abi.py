"""The C-ABI library: it loads, exports every function include/fd_attn.h
declares, sizes workspaces and rejects invalid calls before touching the GPU.
No test here launches a kernel."""
import ctypes
import os
import re

import pytest

import split_kv_asynchronous_amd as fd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(fd_(?:attn|flat_gemm|probe)\w*)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert names == ["fd_attn_choose_band", "fd_attn_decode", "fd_attn_decode_static", "fd_attn_plan",
                     "fd_attn_prefill",
                     "fd_attn_score_stats", "fd_attn_status_string", "fd_attn_workspace_size",
                     "fd_flat_gemm", "fd_flat_gemm_pack_weights", "fd_flat_gemm_packed_bytes",
                     "fd_flat_gemm_plan", "fd_flat_gemm_workspace_size", "fd_probe_read"]
    lib = ctypes.CDLL(fd.library_path())
    for n in names:
        assert hasattr(lib, n), n


def _desc(**kw):
    base = dict(batch=32, num_q_heads=64, num_kv_heads=8, max_seq_len=32768, chunk_size=1024)
    base.update(kw)
    return fd.make_desc(**base)


def test_workspace_size_formula():
    d = _desc()
    rows, maxch = 32 * 64, 32
    slots = rows * maxch
    n = fd.fd_attn_workspace_size(d)
    # header, per-(row, chunk) o/l/m/flag, per-row epoch-tagged counter
    assert n >= 256 + slots * (128 * 4 + 4 + 4 + 1) + rows * 8
    assert n < 256 + slots * (128 * 4 + 4 + 4 + 1) + rows * 8 + 5 * 256
    assert n % 256 == 0
    assert fd.fd_attn_workspace_size(_desc(head_dim=64)) == 0
    assert fd.fd_attn_workspace_size(_desc(chunk_size=48)) == 0


def test_status_strings():
    for code in range(-7, 1):
        assert fd.fd_attn_status_string(code) not in ("", "unknown status")
    assert fd.fd_attn_status_string(5) == "unknown status"


FAKE = 0x10000  # never dereferenced: every case below fails validation first


def _call(desc, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, bt=None, phi=4.0, a=20.0, b=6.0, out=FAKE,
          flags=FAKE):
    lib = fd._load()
    return lib.fd_attn_decode(ctypes.byref(desc), q, k, v, lens, bt, phi, a, b, out, flags, None)


def _valid_desc(**kw):
    d = _desc(**kw)
    d.workspace = 0x100000
    d.workspace_bytes = 1 << 40
    return d


@pytest.mark.parametrize("kw,code", [
    (dict(num_q_heads=63), -2), (dict(head_dim=64), -2), (dict(chunk_size=16), -2),
    (dict(chunk_size=100), -2), (dict(max_seq_len=0), -2), (dict(batch=0), -2),
    (dict(max_seq_len=(1 << 23) + 1), -2),
    (dict(page_size=24, max_blocks_per_seq=2048, num_pages=10), -2),
    (dict(page_size=16, max_blocks_per_seq=10, num_pages=10), -2),
    (dict(page_size=64, chunk_size=32, max_blocks_per_seq=1024, num_pages=10), -2),
])
def test_bad_shapes(kw, code):
    assert _call(_valid_desc(**kw)) == code


def test_bad_pointers_dtypes_alignment_band_workspace():
    assert _call(_valid_desc(), q=None) == -1
    assert _call(_valid_desc(page_size=16, max_blocks_per_seq=2048, num_pages=5)) == -1
    assert _call(_valid_desc(kv_dtype="e4m3fn")) == -1          # no scales
    d = _valid_desc()
    d.q_dtype = 2
    assert _call(d) == -3
    d = _valid_desc()
    d.out_dtype = 7
    assert _call(d) == -3
    assert _call(_valid_desc(), k=FAKE + 4) == -4
    assert _call(_valid_desc(), phi=float("nan")) == -5
    assert _call(_valid_desc(), a=-1.0) == -5
    assert _call(_valid_desc(), b=65.0) == -5
    assert _call(_valid_desc(), b=float("inf")) == -5
    d = _valid_desc()
    d.workspace_bytes = 1000
    assert _call(d) == -6
    d = _valid_desc()
    d.workspace = 0x100010
    assert _call(d) == -6
    d = _valid_desc()
    d.scale = float("inf")
    assert _call(d) == -2


def _pcall(desc, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, phi=4.0, a=20.0, b=6.0, out=FAKE, flags=FAKE):
    lib = fd._load()
    return lib.fd_attn_prefill(ctypes.byref(desc), q, k, v, lens, phi, a, b, out, flags, None)


def _pdesc(**kw):
    base = dict(batch=2, num_q_heads=32, num_kv_heads=8, q_len=8192, max_seq_len=8192)
    base.update(kw)
    return fd.make_prefill_desc(**base)


def test_prefill_descriptor_layout_matches_the_header():
    src = open(os.path.join(ROOT, "include", "fd_prefill.h")).read()
    body = src[src.index("typedef struct {"):src.index("} fd_prefill_desc_t;")]
    fields = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+);", body, flags=re.M)
    assert fields == [f for f, _ in fd.FdPrefillDesc._fields_]


@pytest.mark.parametrize("kw,code", [
    (dict(num_q_heads=30), -2), (dict(head_dim=64), -2), (dict(q_len=0), -2),
    (dict(q_len=(1 << 23) + 1), -2), (dict(max_seq_len=0), -2), (dict(batch=0), -2),
    (dict(batch=65536), -2), (dict(max_seq_len=(1 << 23) + 1), -2),
    (dict(dtype="f32"), -3), (dict(dtype="e4m3fn"), -3), (dict(out_dtype="e4m3fn"), -3),
    (dict(kv_dtype="f32"), -3),
    (dict(page_size=12, max_blocks_per_seq=1000, num_pages=5, block_table_ptr=FAKE), -2),
    (dict(page_size=512, max_blocks_per_seq=16, num_pages=5, block_table_ptr=FAKE), -2),
    (dict(page_size=16, max_blocks_per_seq=511, num_pages=5, block_table_ptr=FAKE), -2),
    (dict(page_size=16, max_blocks_per_seq=512, num_pages=0, block_table_ptr=FAKE), -2),
    (dict(page_size=16, max_blocks_per_seq=512, num_pages=5), -1),
    (dict(kv_dtype="e4m3fn"), -1), (dict(kv_dtype="e4m3fn", k_scale_ptr=FAKE), -1),
])
def test_prefill_bad_shapes_and_dtypes(kw, code):
    assert _pcall(_pdesc(**kw)) == code


def test_prefill_bad_pointers_alignment_band():
    assert _pcall(_pdesc(), q=None) == -1
    assert _pcall(_pdesc(), lens=None) == -1
    assert _pcall(_pdesc(), flags=None) == -1
    assert _pcall(_pdesc(), v=FAKE + 2) == -4
    assert _pcall(_pdesc(), out=FAKE + 8) == -4
    assert _pcall(_pdesc(), phi=float("inf")) == -5
    assert _pcall(_pdesc(), a=65.0) == -5
    assert _pcall(_pdesc(), b=-0.5) == -5
    d = _pdesc()
    d.scale = float("nan")
    assert _pcall(d) == -2
    assert fd._load().fd_attn_prefill(None, FAKE, FAKE, FAKE, FAKE, 4.0, 20.0, 6.0, FAKE, FAKE,
                                      None) == -1


def _scall(desc, q=FAKE, k=FAKE, lens=FAKE, bt=None, lo=-16.0, hi=16.0, nbins=64, mx=FAKE, mn=FAKE,
           hist=FAKE):
    return fd._load().fd_attn_score_stats(ctypes.byref(desc), q, k, lens, bt, lo, hi, nbins, mx, mn,
                                          hist, None)


def test_score_stats_validation():
    d = _desc()
    assert _scall(d, q=None) == -1
    assert _scall(d, mx=None) == -1
    assert _scall(_desc(page_size=16, max_blocks_per_seq=2048, num_pages=5)) == -1
    assert _scall(_desc(kv_dtype="e4m3fn")) == -1               # no k_scale
    assert _scall(_desc(head_dim=64)) == -2
    assert _scall(d, nbins=8193) == -2
    assert _scall(d, nbins=-1) == -2
    assert _scall(d, lo=1.0, hi=1.0) == -2
    assert _scall(d, lo=float("nan")) == -2
    assert _scall(d, k=FAKE + 8) == -4
    bad = _desc()
    bad.q_dtype = 2
    assert _scall(bad) == -3


def _gcall(desc, a=FAKE, w=FAKE, c=FAKE):
    return fd._load().fd_flat_gemm(ctypes.byref(desc), a, w, c, None)


def test_flat_gemm_plan_and_workspace():
    # every variant and split gives slices that cover K exactly, none empty
    for m, n, k in [(1, 16, 32), (5, 200, 96), (16, 4096, 4096), (16, 22016, 4096),
                    (64, 4096, 11008), (100, 48, 256)]:
        for v in range(0, 15):
            for ks in (0, 1, 3):
                if ks > k // 32:
                    continue
                if v in (13, 14) and (k % 128 or (v == 13 and m > 48)):
                    # DMA variants: whole 4-step stages; variant 13's rings leave
                    # no room for a slice of 64 rows of A
                    with pytest.raises(fd.FdAttnError):
                        fd.fd_flat_gemm_plan(m, n, k, variant=v, ksplit=ks)
                    continue
                p = fd.fd_flat_gemm_plan(m, n, k, variant=v, ksplit=ks)
                steps = k // 32
                assert 1 <= p["ksplit"] <= steps
                assert (p["ksplit"] - 1) * p["steps_per_slice"] < steps <= p["ksplit"] * p["steps_per_slice"]
                if v:
                    assert p["variant"] == v
                ws = fd.fd_flat_gemm_workspace_size(m, n, k, variant=v, ksplit=ks)
                assert ws == (p["ksplit"] * m * n * 4 if p["ksplit"] > 1 else 0)


@pytest.mark.parametrize("kw,code", [
    (dict(m=0), -2), (dict(m=4097), -2), (dict(n=0), -2), (dict(k=48), -2), (dict(k=0), -2),
    (dict(variant=15), -2), (dict(variant=-1), -2), (dict(ksplit=5, k=128), -2),
])
def test_flat_gemm_shape_errors(kw, code):
    base = dict(m=16, n=4096, k=4096)
    base.update(kw)
    d = fd.make_gemm_desc(**base)
    assert _gcall(d) == code
    assert fd._load().fd_flat_gemm_plan(ctypes.byref(d), None, None, None, None) == code
    assert fd._load().fd_flat_gemm_workspace_size(ctypes.byref(d)) == 0


def test_flat_gemm_pointer_dtype_and_workspace_errors():
    d = fd.make_gemm_desc(m=16, n=4096, k=4096)
    assert _gcall(d, a=None) == -1
    assert _gcall(d, c=None) == -1
    assert fd._load().fd_flat_gemm(None, FAKE, FAKE, FAKE, None) == -1
    assert _gcall(d, w=FAKE + 8) == -4
    assert _gcall(d, c=FAKE + 4) == -4
    bad = fd.make_gemm_desc(m=16, n=4096, k=4096)
    bad.a_dtype = 0
    assert _gcall(bad) == -3
    bad = fd.make_gemm_desc(m=16, n=4096, k=4096, out_dtype="e4m3fn")
    assert _gcall(bad) == -3
    # K split over workgroups needs a workspace: missing, unaligned, too small
    d = fd.make_gemm_desc(m=16, n=4096, k=4096, ksplit=4)
    assert _gcall(d) == -6
    d.workspace, d.workspace_bytes = FAKE + 16, 1 << 30
    assert _gcall(d) == -6
    d.workspace, d.workspace_bytes = FAKE, 4 * 16 * 4096 * 4 - 1
    assert _gcall(d) == -6


def test_flat_gemm_packed_weights_host_checks():
    assert fd.fd_flat_gemm_packed_bytes(200, 96) == 208 * 96 * 2
    assert fd.fd_flat_gemm_packed_bytes(16, 32) == 16 * 32 * 2
    assert fd.fd_flat_gemm_packed_bytes(0, 32) == 0
    assert fd.fd_flat_gemm_packed_bytes(16, 48) == 0
    lib = fd._load()
    assert lib.fd_flat_gemm_pack_weights(16, 32, None, FAKE, None) == -1
    assert lib.fd_flat_gemm_pack_weights(16, 40, FAKE, FAKE, None) == -2
    assert lib.fd_flat_gemm_pack_weights(16, 32, FAKE + 8, FAKE, None) == -4
    # packed weights take the direct variants only; unknown layouts are refused
    p = fd.fd_flat_gemm_plan(16, 12288, 4096, w_layout="packed")
    assert 5 <= p["variant"] <= 12
    for v in (1, 4, 13, 14):
        d = fd.make_gemm_desc(m=16, n=4096, k=4096, variant=v, w_layout="packed")
        assert _gcall(d) == -2
    d = fd.make_gemm_desc(m=16, n=4096, k=4096)
    d.w_layout = 2
    assert _gcall(d) == -3


def test_flat_gemm_table_covers_the_7b_layers():
    # every M of the measured ranges picks a valid plan for both weight layouts,
    # packed weights always a direct variant, and K slices that tile K
    for n, k in [(12288, 4096), (4096, 4096), (22016, 4096), (4096, 11008)]:
        for m in range(1, 65):
            for layout in ("rows", "packed"):
                p = fd.fd_flat_gemm_plan(m, n, k, w_layout=layout)
                steps = k // 32
                assert 1 <= p["ksplit"] <= steps
                assert (p["ksplit"] - 1) * p["steps_per_slice"] < steps <= p["ksplit"] * p["steps_per_slice"]
                if layout == "packed":
                    assert 5 <= p["variant"] <= 12


# The plan table (measured on MI355X; the rows of fd_host.h): per kernel
# family, paging and max_seq_len range, the chunk size for chunk_size = 0, the
# kernel shape at that chunk, and the largest chunk size whose calls merge in
# the launch (0: none; grids of one round of workgroups, and calls whose chunk
# covers max_seq_len, always do).
FAMILY_KW = {0: dict(), 1: dict(kv_dtype="e4m3fn"), 2: dict(num_kv_heads=64)}
PLAN_ROWS = [
    # family, paged, max_seq_len probes, chunk, shape, largest chunk merged in
    # the launch, balanced shares for chunk_size 0 (shape + 1; 0: fixed chunks)
    (0, 0, (1, 2048), 2048, 0, 0, 0), (0, 0, (2049, 8192), 4096, 1, 512, 0),
    (0, 0, (8193, 32768), 2048, 0, 1024, 1), (0, 0, (32769, 1 << 18), 1024, 0, 0, 0),
    (0, 1, (16, 2048), 2048, 0, 0, 0), (0, 1, (2064, 8192), 4096, 1, 1024, 0),
    (0, 1, (8208, 32768), 2048, 0, 2048, 0), (0, 1, (32784, 1 << 18), 2048, 0, 0, 0),
    (1, 0, (1, 2048), 1024, 0, 1024, 0), (1, 0, (2049, 16384), 1024, 0, 1024, 1),
    (1, 0, (16385, 1 << 18), 2048, 0, 0, 1),
    (1, 1, (16, 2048), 1024, 0, 1024, 0), (1, 1, (2064, 16384), 1024, 0, 1024, 1),
    (1, 1, (16400, 1 << 18), 2048, 0, 0, 1),
    (2, 0, (1, 2048), 1024, 0, 0, 0), (2, 0, (2049, 8192), 2048, 0, 0, 0),
    (2, 0, (8193, 1 << 18), 1024, 0, 0, 0),
    (2, 1, (16, 2048), 1024, 0, 0, 0), (2, 1, (2064, 8192), 2048, 0, 0, 0),
    (2, 1, (8208, 1 << 18), 1024, 0, 0, 0),
]


@pytest.mark.parametrize("fam,paged,lens,chunk,shape,fused_chunk,shares", PLAN_ROWS)
def test_plan_table(fam, paged, lens, chunk, shape, fused_chunk, shares):
    for L in lens:
        kw = dict(FAMILY_KW[fam], max_seq_len=L, chunk_size=0, batch=256)
        if paged:
            kw.update(page_size=16, max_blocks_per_seq=-(-L // 16), num_pages=5)
        d = _desc(**kw)
        got = fd.fd_attn_plan(d)
        c = max(chunk, 16 if paged else 0)
        blocks = 8 if fam != 2 else 64
        if shares:
            # shape k's persistent grid: 2, 1 or 3 workgroups per compute unit
            assert got == dict(chunk_size=0, family=fam, shape=shares - 1, fused=1,
                               shares=256 * (2, 1, 3)[shares - 1]), (kw, got)
            assert fd.fd_attn_workspace_size(d) != fd.fd_attn_workspace_size(_desc(**dict(kw, chunk_size=chunk)))
        else:
            big = -(-L // c) * 256 * blocks > 512
            fused = c <= fused_chunk or not big or c >= L      # a chunk covering max_seq_len: one-chunk rows
            assert got == dict(chunk_size=c, family=fam, shape=shape, fused=int(fused), shares=0), (kw, got)
            # the workspace follows the plan's chunk
            assert fd.fd_attn_workspace_size(d) == fd.fd_attn_workspace_size(_desc(**dict(kw, chunk_size=chunk)))
        # an explicit chunk size other than the table's runs shape 0, and
        # merges in the launch up to the row's largest such chunk
        for other in (256, 512, 2048, 4096):
            if other == chunk or other % (16 if paged else 32):
                continue
            p = fd.fd_attn_plan(_desc(**dict(kw, chunk_size=other)))
            big = -(-L // other) * 256 * blocks > 512
            fused = other <= fused_chunk or not big or other >= L
            assert p["shape"] == 0 and p["fused"] == int(fused), (kw, other, p)


def test_plan_small_grids_merge_in_the_launch_and_forced_plans():
    small = _desc(batch=1, num_q_heads=8, num_kv_heads=1, max_seq_len=4096, chunk_size=1024)
    assert fd.fd_attn_plan(small)["fused"] == 1
    big = _desc(kv_dtype="e4m3fn", max_seq_len=16384, chunk_size=512)
    assert fd.fd_attn_plan(big) == dict(chunk_size=512, family=1, shape=0, fused=1, shares=0)
    big = _desc(kv_dtype="e4m3fn", max_seq_len=16384, chunk_size=2048)
    assert fd.fd_attn_plan(big) == dict(chunk_size=2048, family=1, shape=0, fused=0, shares=0)
    forced = _desc(kv_dtype="e4m3fn", max_seq_len=16384, chunk_size=512,
                   plan=fd.FD_PLAN_SHAPE(2) | fd.FD_PLAN_FUSED)
    assert fd.fd_attn_plan(forced) == dict(chunk_size=512, family=1, shape=2, fused=1, shares=0)
    split = _desc(batch=1, num_q_heads=8, num_kv_heads=1, max_seq_len=4096, chunk_size=1024,
                  plan=fd.FD_PLAN_SPLIT)
    assert fd.fd_attn_plan(split)["fused"] == 0
    # a shape the family does not have, both placements, unknown bits: rejected
    for bad in (fd.FD_PLAN_SHAPE(3), fd.FD_PLAN_FUSED | fd.FD_PLAN_SPLIT, 0x80):
        d = _desc(plan=bad)
        assert fd.fd_attn_workspace_size(d) == 0
        with pytest.raises(fd.FdAttnError):
            fd.fd_attn_plan(d)
        assert _call(_valid_desc(plan=bad)) == -2
    assert _call(_valid_desc(num_kv_heads=64, plan=fd.FD_PLAN_SHAPE(1))) == -2   # vector: one shape


def test_serving_batches_run_balanced_shares():
    # serving batches run balanced shares in shape 2 (3 workgroups per
    # compute unit): whole chunks, for a chunk size that is a multiple of 64
    # (merged by a second launch unless a chunk covers max_seq_len), from
    # 8192 (bf16) / 16384 (E4M3FN) row groups; for chunk_size 0, from 16384
    # row groups in both families: whole chunks covering every row when rows
    # are at most 2K tokens, pieces beyond.  Fewer row groups, a chunk size
    # off the 64 grid or a forced plan: fixed chunks
    for kw, whole_needed in ((dict(), 8192), (dict(kv_dtype="e4m3fn", num_q_heads=32), 16384)):
        for batch in sorted({whole_needed // 8 - 1, whole_needed // 8, 16384 // 8 - 1, 16384 // 8}):
            base = dict(kw, batch=batch, max_seq_len=2048, chunk_size=0)
            got = fd.fd_attn_plan(_desc(**base))
            whole = fd.fd_attn_plan(_desc(**dict(base, chunk_size=512)))
            one = fd.fd_attn_plan(_desc(**dict(base, chunk_size=2048)))
            if batch * 8 >= 16384:
                # rows of up to 2K tokens: whole-chunk shares, one chunk per row
                assert got == dict(chunk_size=2048, family=got["family"], shape=2, fused=1, shares=768), (base, got)
                long_rows = fd.fd_attn_plan(_desc(**dict(base, max_seq_len=4096)))
                assert long_rows["shares"] > 0 and long_rows["chunk_size"] == 0 and long_rows["fused"] == 1
            else:
                assert got["shares"] == 0 and got["chunk_size"] > 0, (base, got)
            if batch * 8 >= whole_needed:
                assert whole == dict(chunk_size=512, family=whole["family"], shape=2, fused=0, shares=768)
                assert one["shares"] == 768 and one["fused"] == 1
            else:
                assert whole["shares"] == 0 and one["shares"] == 0, (base, whole, one)
            assert fd.fd_attn_plan(_desc(**dict(base, chunk_size=96)))["shares"] == 0
            assert fd.fd_attn_plan(_desc(**dict(base, plan=fd.FD_PLAN_SPLIT)))["shares"] == 0
    # one query per KV head: never
    assert fd.fd_attn_plan(_desc(batch=4096, num_kv_heads=64, max_seq_len=2048, chunk_size=0))["shares"] == 0


def test_balanced_share_plans():
    # FD_PLAN_SHARES: a persistent grid of as many workgroups per compute unit
    # (256) as the shape's ring lets be resident.  chunk_size 0: pieces cut at
    # the shares' edges (reported chunk size 0), merged in the launch; the
    # workspace holds one partial per (segment, row group) piece -- at most
    # (shares + pool grains) * heads_per_block + rows.  A chunk size (a
    # multiple of 64): whole chunks, the fixed-chunk workspace, either merge
    # placement.
    for kw in (dict(), dict(kv_dtype="e4m3fn"), dict(page_size=16, max_blocks_per_seq=2048, num_pages=9)):
        fam = 1 if kw.get("kv_dtype") else 0
        for shape, per_cu in ((0, 2), (1, 1), (2, 3)):
            plan = fd.FD_PLAN_SHARES | fd.FD_PLAN_SHAPE(shape)
            d = _desc(**dict(kw, max_seq_len=32768, chunk_size=0, plan=plan))
            got = fd.fd_attn_plan(d)
            assert got == dict(chunk_size=0, family=fam, shape=shape, fused=1, shares=256 * per_cu), (kw, got)
            rows = 32 * 64
            # pool grains of the largest call: 64-token quanta, a quarter
            # pooled in grains of 16 quanta (calls of at least 4 quanta per share)
            W, nmax = 256 * per_cu, 512 * 32 * 8
            grains = -(-(nmax // 4) // 16) if nmax >= 4 * W else 0
            slots = (W + grains) * 8 + rows
            assert slots * (128 * 4 + 9) <= fd.fd_attn_workspace_size(d) <= slots * (128 * 4 + 9) + 8 * rows + 2048
            for place, fused in ((0, 1), (fd.FD_PLAN_FUSED, 1), (fd.FD_PLAN_SPLIT, 0)):
                d = _desc(**dict(kw, max_seq_len=32768, chunk_size=1024, plan=plan | place))
                assert fd.fd_attn_plan(d) == dict(chunk_size=1024, family=fam, shape=shape, fused=fused,
                                                  shares=256 * per_cu)
                assert fd.fd_attn_workspace_size(d) == fd.fd_attn_workspace_size(
                    _desc(**dict(kw, max_seq_len=32768, chunk_size=1024)))
    # no shares for the one-query-per-KV-head kernel, nor pieces with a merge
    # launch, nor whole chunks of a size that is not a multiple of 64
    for bad in (_valid_desc(num_kv_heads=64, plan=fd.FD_PLAN_SHARES),
                _valid_desc(chunk_size=0, plan=fd.FD_PLAN_SHARES | fd.FD_PLAN_SPLIT),
                _valid_desc(chunk_size=96, plan=fd.FD_PLAN_SHARES)):
        assert fd.fd_attn_workspace_size(bad) == 0
        assert _call(bad) == -2


def test_static_workspace_variant_checks_before_the_gpu():
    # the allocation-free entry point validates exactly as fd_attn_decode does
    # and refuses a call whose workspace exceeds its static array
    lib = fd._load()

    def scall(d, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, table=None, phi=4.0, a=20.0, b=6.0, out=FAKE, flags=FAKE)
        a.update(kw)
        return lib.fd_attn_decode_static(ctypes.byref(d), a["q"], a["k"], a["v"], a["lens"], a["table"],
                                         a["phi"], a["a"], a["b"], a["out"], a["flags"], None)
    assert scall(_valid_desc(), q=None) == -1
    assert scall(_valid_desc(), k=FAKE + 4) == -4
    assert scall(_valid_desc(), b=65.0) == -5
    assert scall(_valid_desc(head_dim=64)) == -2
    big = _valid_desc(batch=64, num_q_heads=64, num_kv_heads=8, max_seq_len=1 << 20, chunk_size=1024)
    assert fd.fd_attn_workspace_size(big) > (64 << 20)
    assert scall(big) == -6


def test_read_probe_host_checks():
    # the read probe (include/fd_probe.h) rejects its arguments before any
    # launch: NULL buffers or sink, units NULL with units to read, a negative
    # count, a ring shape other than 0..2, with a page list a page size that
    # is not a multiple of 1 KiB in [1 KiB, 1 MiB], unaligned buffers; no
    # units: OK, nothing enqueued
    lib = ctypes.CDLL(fd.library_path())
    lib.fd_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p]
    k, v, u, pg, sink = 0x10000, 0x20000, 0x30000, 0x50000, 0x40000

    def call(k=k, v=v, u=u, n=1, pages=None, page_bytes=0, shape=0, sink=sink):
        return lib.fd_probe_read(k, v, u, n, pages, page_bytes, shape, sink, None)
    assert call(k=None) == -1 and call(v=None) == -1 and call(sink=None) == -1 and call(u=None) == -1
    assert call(u=None, n=0) == 0
    assert call(n=-1) == -2
    for bad in (-1, 3, 4):
        assert call(shape=bad) == -2
    for bad in (0, 512, 1536, 2 << 20):
        assert call(pages=pg, page_bytes=bad) == -2
    assert call(pages=pg, page_bytes=2048, n=0) == 0
    assert call(k=k + 8) == -4 and call(v=v + 4, shape=2) == -4
    assert fd.PROBE_UNIT.itemsize == 16


def test_small_calls_plan_smaller_chunks_and_no_shares():
    # chunk_size 0 on a call with few rows: the table's chunk (measured on
    # full batches) is halved, down to 256 tokens and to no more than 32
    # chunks per row (256 for one query per KV head), until the call has 256
    # units (2048 for the E4M3FN family, 1024 for one query per KV head;
    # counted at max_seq_len);
    # balanced shares need 128 quanta of 64 tokens per share.  Full batches
    # keep the table's pick.
    def plan(**kw):
        return fd.fd_attn_plan(_desc(**dict(kw, chunk_size=0)))

    def units(p, kw):
        g = kw["num_q_heads"] // kw["num_kv_heads"]
        gb = kw["num_q_heads"] if p["family"] == 2 else kw["num_q_heads"] // max(
            k for k in range(1, min(g, 16) + 1) if g % k == 0)
        return -(-kw["max_seq_len"] // p["chunk_size"]) * gb * kw["batch"]

    small = [dict(batch=1, num_q_heads=1, num_kv_heads=1, max_seq_len=4096, q_dtype="f32", kv_dtype="f32"),
             dict(batch=1, num_q_heads=1, num_kv_heads=1, max_seq_len=131072),
             dict(batch=1, num_q_heads=32, num_kv_heads=8, max_seq_len=8192),
             dict(batch=1, num_q_heads=64, num_kv_heads=8, max_seq_len=32768),
             dict(batch=2, num_q_heads=32, num_kv_heads=8, max_seq_len=16384, kv_dtype="e4m3fn"),
             dict(batch=1, num_q_heads=32, num_kv_heads=8, max_seq_len=16384, kv_dtype="e4m3fn", page_size=16,
                  max_blocks_per_seq=1024, num_pages=1024)]
    want = [256, 512, 256, 1024, 512, 512]
    for kw, c in zip(small, want):
        p = plan(**kw)
        assert p["shares"] == 0 and p["chunk_size"] == c, (kw, p)
        # the largest chunk (at least 256, and no more than 32 chunks per
        # row in the grouped families, 256 for one query per KV head) that
        # gives the family's units
        target = (256, 2048, 1024)[p["family"]]
        per_row = 256 if p["family"] == 2 else 32
        assert c == 256 or c * per_row < 2 * kw["max_seq_len"] or \
            units(p, kw) >= target > units(dict(p, chunk_size=2 * c), kw), (kw, p)
        assert -(-kw["max_seq_len"] // c) <= per_row or c == 256, (kw, p)
        assert p["fused"] == 1       # a grid of at most 512 units merges in the launch
        assert fd.fd_attn_workspace_size(_desc(**dict(kw, chunk_size=0))) == \
            fd.fd_attn_workspace_size(_desc(**dict(kw, chunk_size=c)))
    # full batches: the table's pick, balanced shares where the table takes them
    assert plan(batch=32, num_q_heads=64, num_kv_heads=8, max_seq_len=32768)["shares"] == 512
    assert plan(batch=64, num_q_heads=32, num_kv_heads=8, max_seq_len=16384, kv_dtype="e4m3fn", page_size=16,
                max_blocks_per_seq=1024, num_pages=40000)["shares"] == 512
    assert plan(batch=8, num_q_heads=32, num_kv_heads=32, max_seq_len=8192)["chunk_size"] == 2048
    assert plan(batch=1, num_q_heads=32, num_kv_heads=32, max_seq_len=131072)["chunk_size"] == 1024
    # one query per KV head: 1024 units, but at most 256 chunks per row
    assert plan(batch=8, num_q_heads=32, num_kv_heads=32, max_seq_len=2048)["chunk_size"] == 512
    assert plan(batch=1, num_q_heads=32, num_kv_heads=32, max_seq_len=32768)["chunk_size"] == 1024
    assert plan(batch=1, num_q_heads=1, num_kv_heads=1, max_seq_len=131072)["chunk_size"] == 512
    assert plan(batch=1, num_q_heads=1, num_kv_heads=1, max_seq_len=1 << 20)["chunk_size"] == 4096
    # at most 256 chunks per row: rows this long double the table's chunk
    assert plan(batch=4, num_q_heads=64, num_kv_heads=8, max_seq_len=1 << 20)["chunk_size"] == 4096
    assert plan(batch=64, num_q_heads=32, num_kv_heads=32, max_seq_len=1 << 23)["chunk_size"] == 32768
    # an explicit chunk size is kept as given
    assert fd.fd_attn_plan(_desc(batch=1, num_q_heads=1, num_kv_heads=1, max_seq_len=4096,
                                 chunk_size=2048))["chunk_size"] == 2048


def test_automatic_plans_are_valid_on_random_calls():
    # chunk_size 0 over random shapes: every plan is one the call accepts --
    # a chunk of at least 256 tokens (a multiple of the page size) and at
    # most 256 chunks per row, or balanced shares (grouped families only;
    # pieces, or whole chunks covering every row) -- and a fixed-chunk plan
    # sizes the same workspace as the call with that chunk stated
    import numpy as np
    rng = np.random.default_rng(2024)
    for _ in range(400):
        hkv = int(rng.choice([1, 2, 4, 8, 32]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        kv = str(rng.choice(["bf16", "e4m3fn", "f32"]))
        page = int(rng.choice([0, 0, 16, 32, 256]))
        L = int(rng.choice([1, 17, 300, 2048, 5000, 32768, 200000, 1 << 23]))
        kw = dict(batch=int(rng.choice([1, 3, 16, 200, 2048, 20000])), num_q_heads=g * hkv, num_kv_heads=hkv,
                  max_seq_len=L, kv_dtype=kv, q_dtype="f32" if kv == "f32" else "bf16")
        if page:
            kw.update(page_size=page, max_blocks_per_seq=-(-L // page), num_pages=4)
        d = _desc(**dict(kw, chunk_size=0))
        p = fd.fd_attn_plan(d)
        if p["shares"]:
            # pieces, or (serving batches of short rows) whole chunks covering every row
            c = p["chunk_size"]
            assert p["family"] in (0, 1) and p["fused"] == 1, (kw, p)
            assert c == 0 or (c >= L and c % 64 == 0 and c % max(page, 1) == 0), (kw, p)
            continue
        c = p["chunk_size"]
        assert c >= 256 and c % 32 == 0 and c % max(page, 1) == 0, (kw, p)
        assert -(-L // c) <= 256 or c == 256, (kw, p)
        assert fd.fd_attn_workspace_size(d) == fd.fd_attn_workspace_size(_desc(**dict(kw, chunk_size=c))), (kw, p)
