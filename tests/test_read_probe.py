"""The read probe (include/fd_probe.h) and the bench's unit lists for it.

CPU: the unit list of a grouped-query call covers every (sequence, head
block) slice exactly once, in the chunk kernel's order (full chunks first),
and holds the call's K bytes; on a paged cache its pages are the block
table's, in order.  GPU: the probe runs through the C ABI over ragged units
(empty ones, ones that end inside a group, the last one ending at the
buffer's end), contiguous and paged, with every ring shape."""
import os
import sys

import numpy as np
import pytest

import split_kv_asynchronous_amd as fd
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

LENS = [0, 1, 16, 17, 3 * 256 - 7, 5]


@pytest.mark.parametrize("hq,hkv,chunk,kv_dtype,page",
                         [(64, 8, 1024, "bf16", 0), (32, 8, 512, "e4m3fn", 0), (40, 2, 256, "bf16", 0),
                          (32, 8, 512, "e4m3fn", 16), (64, 8, 256, "bf16", 32)])
def test_probe_units_cover_the_call_once(hq, hkv, chunk, kv_dtype, page):
    lens = np.array([L * chunk // 256 if L > 16 else L for L in LENS], dtype=np.int32)
    prob = synthetic.make_problem(batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, seq_lens=lens,
                                  kv_dtype=kv_dtype, page_size=page, chunk_size=chunk, seed=3)
    units, pages, page_bytes = bench.probe_units(prob, chunk)
    G = hq // hkv
    GB = bench.heads_per_block(G)
    nhb = hq // GB
    row = 128 * (2 if kv_dtype == "bf16" else 1)
    assert int(units["bytes"].sum()) == int(lens.sum()) * nhb * row
    assert len(units) == sum(-(-int(L) // chunk) if L else 1 for L in lens) * nhb
    # full chunks first, then the partial last chunks
    full = units["bytes"] == chunk * row
    assert full.all() or not np.any(full[np.argmin(full):])
    # per (sequence, KV head): the units of its head blocks tile [0, L) once each
    if not page:
        assert pages is None and page_bytes == 0
        S = prob.max_seq_len
        slice_of = units["offset"] // (S * row)
        assert np.all(units["offset"] + units["bytes"] <= (slice_of + 1) * S * row)
        for b, L in enumerate(lens.tolist()):
            for kvh in range(hkv):
                sel = slice_of == b * hkv + kvh
                got = sorted(zip((units["offset"][sel] % (S * row)).tolist(), units["bytes"][sel].tolist()))
                want = []
                for c in range(-(-L // chunk) if L else 1):
                    want += [(c * chunk * row, (min(L, (c + 1) * chunk) - c * chunk) * row)] * (G // GB)
                assert got == sorted(want), (b, kvh)
    else:
        assert page_bytes == page * row
        # unit u's pages: its chunk's block-table entries, as pieces of its KV head
        seen = {}
        for u in range(len(units)):
            n = -(-int(units["bytes"][u]) // page_bytes)
            pieces = pages[units["offset"][u]:units["offset"][u] + n]
            blk, kvh = np.divmod(pieces // page_bytes, hkv)
            assert np.all(pieces % page_bytes == 0) and len(set(kvh.tolist())) <= 1
            for p in blk.tolist():
                seen[(p, int(kvh[0]))] = seen.get((p, int(kvh[0])), 0) + 1
        # every used page of every sequence, once per head block of each KV head
        want = {}
        for b, L in enumerate(lens.tolist()):
            for p in prob.block_table[b, :-(-L // page)].tolist():
                for h in range(hkv):
                    want[(p, h)] = want.get((p, h), 0) + G // GB
        assert seen == want


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [0, 1, 2])
@pytest.mark.parametrize("paged", [False, True])
def test_probe_reads_ragged_units(shape, paged):
    import torch
    nbytes = 1 << 20
    k = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    v = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    units = np.zeros(7, dtype=fd.PROBE_UNIT)
    units["bytes"] = [0, 16, 4096, 4100, 12288 * 3 + 48, 77777, 12304]
    pages, page_bytes = None, 0
    if paged:
        # 2 KiB pages scattered over the buffers, each unit's pages listed in turn
        page_bytes = 2048
        rng = np.random.default_rng(5)
        need = [-(-int(b) // page_bytes) for b in units["bytes"]]
        assert max(need) <= 64
        units["offset"] = np.concatenate([[0], np.cumsum(need)[:-1]])
        pages = rng.integers(0, nbytes // page_bytes, size=sum(need)).astype(np.int64) * page_bytes
        assert np.all(pages + page_bytes <= nbytes)
        pages = torch.from_numpy(pages).cuda()
    else:
        units["offset"] = [0, 4096, 65536, 65536, 300016, 500000 - 500000 % 16, nbytes - 12304]
        assert np.all(units["offset"] % 16 == 0) and np.all(units["offset"] + units["bytes"] <= nbytes)
    dev = torch.from_numpy(units.view(np.uint8).copy()).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    print("probe: shape %d, paged %s, %d units" % (shape, paged, len(units)), flush=True)
    for _ in range(3):
        fd.fd_probe_read(k, v, dev, shape, pages, page_bytes, sink)
    torch.cuda.synchronize()
    # an empty list enqueues nothing
    fd.fd_probe_read(k, v, dev[:0], shape, pages, page_bytes, sink)
    torch.cuda.synchronize()
