"""The read probe (include/fd_probe.h) and the bench's unit list for it.

CPU: the unit list of a contiguous grouped-query call covers every
(sequence, head block) slice exactly once, in the chunk kernel's order (full
chunks first), and holds the call's K bytes.  GPU: the probe runs through the
C ABI over ragged units (empty ones, ones that end inside a 4 KiB group, the
last one ending at the buffer's end) with both ring depths."""
import os
import sys

import numpy as np
import pytest

import split_kv_asynchronous_amd as fd
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("hq,hkv,chunk", [(64, 8, 1024), (32, 8, 512), (40, 2, 256)])
def test_probe_units_cover_the_call_once(hq, hkv, chunk):
    lens = np.array([0, 1, chunk, chunk + 1, 3 * chunk - 7, 5], dtype=np.int32)
    prob = synthetic.make_problem(batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, seq_lens=lens,
                                  kv_dtype="bf16", chunk_size=chunk, seed=3)
    units = bench.probe_units(prob, chunk)
    G = hq // hkv
    GB = bench.heads_per_block(G)
    nhb = hq // GB
    row = 256
    # every unit lies inside its KV head's slice of its sequence
    S = prob.max_seq_len
    slice_of = units["offset"] // (S * row)
    assert np.all((units["offset"] + units["bytes"]) <= (slice_of + 1) * S * row)
    # per (sequence, KV head) slice: the units of its head blocks tile [0, L) once each
    for b, L in enumerate(lens.tolist()):
        for kvh in range(hkv):
            sel = slice_of == b * hkv + kvh
            got = sorted(zip((units["offset"][sel] % (S * row)).tolist(), units["bytes"][sel].tolist()))
            per_block = G // GB   # head blocks reading this KV head
            want = []
            for c in range(-(-L // chunk) if L else 1):
                want += [(c * chunk * row, (min(L, (c + 1) * chunk) - c * chunk) * row)] * per_block
            assert got == sorted(want), (b, kvh)
    # full chunks first, then the partial last chunks
    full = units["bytes"] == chunk * row
    assert not np.any(full[np.argmin(full):]) or full.all()
    assert int(units["bytes"].sum()) == int(lens.sum()) * nhb * row
    assert len(units) == sum(-(-int(L) // chunk) if L else 1 for L in lens) * nhb


@pytest.mark.gpu
@pytest.mark.parametrize("stages", [2, 3])
def test_probe_reads_ragged_units(stages):
    import torch
    nbytes = 1 << 20
    k = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    v = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    units = np.zeros(7, dtype=fd.PROBE_UNIT)
    units["offset"] = [0, 4096, 65536, 65536, 300016, 500000 - 500000 % 16, nbytes - 12304]
    units["bytes"] = [0, 16, 4096, 4100, 12288 * 3 + 48, 77777, 12304]
    assert np.all(units["offset"] % 16 == 0) and np.all(units["offset"] + units["bytes"] <= nbytes)
    dev = torch.from_numpy(units.view(np.uint8).copy()).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    print("probe: stages %d, %d units" % (stages, len(units)), flush=True)
    for _ in range(3):
        fd.fd_probe_read(k, v, dev, stages, sink)
    torch.cuda.synchronize()
    # an empty list enqueues nothing
    fd.fd_probe_read(k, v, dev[:0], stages, sink)
    torch.cuda.synchronize()
