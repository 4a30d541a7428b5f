"""GPU: the allocation-free decode entry point (fd_attn_decode_static) against
fd_attn_decode, through the C ABI.

Both run the same kernels; only the workspace differs (the library's static
device array against a caller-allocated one), so the outputs and flags must
be identical bit for bit -- within the parity bar a fortiori.  Two calls in a
row share the static array, the second with a smaller problem, and a problem
whose workspace would exceed the array is refused before anything is
enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import split_kv_asynchronous_amd as fd
import synthetic
from gpu_helpers import DeviceProblem, compare

pytestmark = pytest.mark.gpu

STATIC_BYTES = 64 << 20      # FD_ATTN_STATIC_WORKSPACE_BYTES in include/fd_attn.h

CASES = [
    # (first, second): the second call smaller than the first
    (dict(batch=8, num_q_heads=32, num_kv_heads=8, seq_lens=[4000, 9000, 1, 0, 12000, 7000, 300, 16000],
          kv_dtype="bf16", page_size=0, chunk_size=512, seed=801),
     dict(batch=2, num_q_heads=16, num_kv_heads=4, seq_lens=[700, 1500], kv_dtype="bf16", page_size=0,
          chunk_size=256, seed=802)),
    (dict(batch=6, num_q_heads=32, num_kv_heads=8, seq_lens=[5000, 16384, 512, 9000, 3, 12000],
          kv_dtype="e4m3fn", page_size=16, chunk_size=512, seed=803),
     dict(batch=3, num_q_heads=8, num_kv_heads=2, seq_lens=[900, 0, 2100], kv_dtype="e4m3fn", page_size=16,
          chunk_size=128, seed=804)),
    (dict(batch=4, num_q_heads=32, num_kv_heads=32, seq_lens=[8192, 6000, 100, 8000], kv_dtype="bf16",
          page_size=0, chunk_size=512, seed=805),
     dict(batch=1, num_q_heads=8, num_kv_heads=8, seq_lens=[3000], kv_dtype="bf16", page_size=0,
          chunk_size=1024, seed=806)),
]


def _static_call(dp, phi=None, a=None, b=None, plan=0):
    p = dp.prob
    return fd.fd_attn_decode_static(
        dp.q, dp.k, dp.v, dp.seq_lens, dp.block_table, p.phi if phi is None else phi,
        p.a if a is None else a, p.b if b is None else b, dp.out, dp.flags, chunk_size=p.chunk_size,
        max_seq_len=p.max_seq_len, num_kv_heads=p.num_kv_heads, page_size=p.page_size, scale=p.scale,
        k_scale=dp.k_scale, v_scale=dp.v_scale, q_dtype=p.q_dtype, kv_dtype=p.kv_dtype, plan=plan)


@pytest.mark.parametrize("first,second", CASES, ids=["gqa-bf16", "paged-e4m3fn", "mha-bf16"])
def test_static_workspace_equals_caller_workspace(first, second):
    for i, kw in enumerate((first, second)):
        # a narrow band on the second call, so that chunks are recomputed
        band = dict(phi=1.0, a=3.0, b=1.5) if i else {}
        prob = synthetic.make_problem(**kw, **band)
        print("case no-alloc call %d: %s" % (i, {k: v for k, v in kw.items() if k != "seq_lens"}), flush=True)
        dp = DeviceProblem(prob)
        assert fd.fd_attn_workspace_size(dp.desc()) <= STATIC_BYTES
        dp.run()
        ref_out, ref_flags = dp.out.clone(), dp.flags.clone()
        dp.out.fill_(float("nan"))
        dp.flags.fill_(7)
        _static_call(dp)
        torch.cuda.synchronize()
        assert torch.equal(dp.out, ref_out), "output differs from fd_attn_decode"
        assert torch.equal(dp.flags, ref_flags), "flags differ from fd_attn_decode"
        if not i:
            out, flags = dp.results()
            compare(prob, out, flags)


SHARE_CALLS = [
    # balanced shares in pieces (a quarter of the work in claimed grains,
    # narrow band: pieces recomputed), then whole 512-token chunks of a
    # smaller paged E4M3FN call, then the first call again on what the
    # second left in the array
    dict(batch=4, num_q_heads=16, num_kv_heads=2, seq_lens=[40000, 30000, 50000, 2000], kv_dtype="bf16",
         page_size=0, chunk_size=0, seed=808, phi=1.0, a=3.0, b=1.5),
    dict(batch=4, num_q_heads=8, num_kv_heads=2, seq_lens=[5000, 700, 0, 3000], kv_dtype="e4m3fn",
         page_size=16, chunk_size=512, seed=809),
]


def test_static_workspace_runs_balanced_shares():
    plan = fd.FD_PLAN_SHARES | fd.FD_PLAN_SHAPE(0)
    dps = [DeviceProblem(synthetic.make_problem(**kw), plan=plan) for kw in SHARE_CALLS]
    for i in (0, 1, 0):
        dp = dps[i]
        got = fd.fd_attn_plan(dp.desc())
        print("case no-alloc shares call %d: plan %s" % (i, got), flush=True)
        assert got["shares"] > 0 and fd.fd_attn_workspace_size(dp.desc()) <= STATIC_BYTES
        dp.run()
        ref_out, ref_flags, ref_rec = dp.out.clone(), dp.flags.clone(), dp.recomputed()
        if i == 0:
            assert ref_rec > 0 and bool(ref_flags.any())
        dp.out.fill_(float("nan"))
        dp.flags.fill_(7)
        _static_call(dp, plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(dp.out, ref_out), "output differs from fd_attn_decode"
        assert torch.equal(dp.flags, ref_flags), "flags differ from fd_attn_decode"


def test_static_entry_replayed_from_a_captured_graph():
    # the callers it is for include code under graph capture: a captured
    # static call (balanced shares, chunks recomputed) replayed with eager
    # static calls of another, smaller problem between the replays, which
    # rewrite the array the captured call uses
    plan = fd.FD_PLAN_SHARES | fd.FD_PLAN_SHAPE(0)
    dps = [DeviceProblem(synthetic.make_problem(**kw), plan=plan) for kw in SHARE_CALLS]
    refs = []
    for dp in dps:
        dp.run()
        refs.append((dp.out.clone(), dp.flags.clone()))
        _static_call(dp, plan=plan)        # eager static calls first (the array's address is looked up)
        torch.cuda.synchronize()
        assert torch.equal(dp.out, refs[-1][0]) and torch.equal(dp.flags, refs[-1][1])
    a, b = dps
    print("case no-alloc graph replay", flush=True)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=stream):
        _static_call(a, plan=plan)
    torch.cuda.synchronize()
    for i in range(5):
        a.out.fill_(float("nan"))
        a.flags.fill_(7)
        if i % 2:
            b.out.fill_(float("nan"))
            _static_call(b, plan=plan)
            torch.cuda.synchronize()
            assert torch.equal(b.out, refs[1][0]) and torch.equal(b.flags, refs[1][1])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(a.out, refs[0][0]), "replay %d: output differs from fd_attn_decode" % i
        assert torch.equal(a.flags, refs[0][1]), "replay %d: flags differ" % i


def test_static_workspace_refuses_oversized_calls():
    prob = synthetic.make_problem(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[100, 50], chunk_size=32,
                                  seed=807)
    dp = DeviceProblem(prob)
    # the same tensors, described as a problem whose partials exceed the array
    big = fd.make_desc(batch=2, num_q_heads=8, num_kv_heads=2, max_seq_len=1 << 23, chunk_size=32)
    assert fd.fd_attn_workspace_size(big) > STATIC_BYTES
    dp.out.fill_(float("nan"))
    lib = fd._load()
    rc = lib.fd_attn_decode_static(ctypes.byref(big), dp.q.data_ptr(), dp.k.data_ptr(), dp.v.data_ptr(),
                                   dp.seq_lens.data_ptr(), None, 4.0, 20.0, 6.0, dp.out.data_ptr(),
                                   dp.flags.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == -6
    torch.cuda.synchronize()
    assert torch.isnan(dp.out).all(), "a refused call wrote its output"
    # and a call that fits still works afterwards
    _static_call(dp)
    out, flags = dp.results()
    compare(prob, out, flags)
