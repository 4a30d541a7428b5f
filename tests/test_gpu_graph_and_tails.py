"""GPU: decode replayed from a captured graph, and caches whose unused slots
hold NaN, through the C ABI.

Replay (a serving loop replays one captured decode step per token): the
captured call keeps the epoch it was captured with, so every replay must
still start its counters from zero.  Each replay's output and flags must be
bit-equal to the eager call's, and the workspace's recomputed-pair count must
equal the eager call's count after every replay, with eager calls on the same
workspace (new epochs) and poisoned outputs between the replays.

Unused slots: a paged cache's last page of a sequence has slots past the
sequence's end, a contiguous cache has capacity past it, and a pool may hold
pages no sequence uses.  Their contents are not part of the call (the oracle
never reads them), so filling all of them with NaN (E4M3FN 0x7F, bf16 0x7FC0,
fp32 NaN) must not change any result.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import DeviceProblem, compare

pytestmark = pytest.mark.gpu

REPLAY_CASES = [
    # id, group, kv dtype, page size, lens, chunk, merge placement -- the merge
    # inside the chunk launch and in a second launch, grouped and
    # single-query kernels, small grids and grids of many rounds
    ("fused-gqa-bf16", 4, "bf16", 0, [700, 1500], 256, "fused"),
    ("fused-gqa-e4m3fn-paged", 8, "e4m3fn", 16, [2000, 900], 128, "fused"),
    ("fused-large-gqa-bf16", 8, "bf16", 0, [20000, 9000, 15000, 30000], 256, "fused"),
    ("split-gqa-bf16", 4, "bf16", 0, [8192, 6000, 8192, 5000], 256, "split"),
    ("split-mha-bf16", 1, "bf16", 0, [3000] * 4, 64, "split"),
    ("split-gqa-e4m3fn-paged", 4, "e4m3fn", 16, [4096, 3000, 2500, 4000], 128, "split"),
    # balanced shares with pool grains claimed from the workspace's counter:
    # pieces cut at segment edges (chunk 0) and whole chunks
    ("shares-pieces-gqa-bf16", 8, "bf16", 0, [20000, 9000, 15000, 30000], 0, "shares"),
    ("shares-gqa-bf16", 8, "bf16", 0, [20000, 9000, 15000, 30000], 256, "shares"),
    ("shares-gqa-e4m3fn-paged", 4, "e4m3fn", 16, [30000, 20000, 25000, 12000], 256, "shares"),
]


@pytest.mark.parametrize("name,g,kv,page,lens,chunk,place", REPLAY_CASES, ids=[c[0] for c in REPLAY_CASES])
def test_decode_replayed_from_a_captured_graph(name, g, kv, page, lens, chunk, place):
    import split_kv_asynchronous_amd as fd
    hkv = 2 if g > 1 else 8
    # a narrow band, so that chunks leave it and are recomputed
    prob = synthetic.make_problem(batch=len(lens), num_q_heads=g * hkv, num_kv_heads=hkv, seq_lens=lens,
                                  kv_dtype=kv, page_size=page, chunk_size=chunk, phi=1.0, a=3.0, b=1.5,
                                  seed=600 + g)
    print("case replay %s" % name, flush=True)
    dp = DeviceProblem(prob, plan={"fused": fd.FD_PLAN_FUSED, "split": fd.FD_PLAN_SPLIT,
                                   "shares": fd.FD_PLAN_SHARES}[place])
    plan = fd.fd_attn_plan(dp.desc())
    assert plan["fused"] == (place != "split") and (plan["shares"] > 0) == (place == "shares")
    dp.run()
    out0, flags0 = dp.results()
    count0 = dp.recomputed()
    ref_out, ref_flags, margin = oracle.decode_exact(**prob.args())
    sure = margin >= 1e-3
    np.testing.assert_array_equal(flags0[sure], ref_flags[sure])
    compare(prob, out0, np.where(sure, flags0, ref_flags), ref=(ref_out, ref_flags))
    assert count0 > 0, "the band should send some chunks to the recompute"
    eager_out, eager_flags = dp.out.clone(), dp.flags.clone()

    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=stream):
        dp.run()
    torch.cuda.synchronize()
    for i in range(5):
        dp.out.fill_(float("nan"))
        dp.flags.fill_(7)
        if i % 2:
            dp.run()                       # an eager call (a fresh epoch) on the same workspace
            torch.cuda.synchronize()
            assert torch.equal(dp.out, eager_out) and dp.recomputed() == count0
            dp.out.fill_(float("nan"))
            dp.flags.fill_(7)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dp.out, eager_out), "replay %d: output differs from the eager call" % i
        assert torch.equal(dp.flags, eager_flags), "replay %d: flags differ" % i
        assert dp.recomputed() == count0, "replay %d: count %d, eager %d" % (i, dp.recomputed(), count0)
    print("%s: %d recomputed pairs on every replay" % (name, count0))


def _poison_unused(prob):
    """Fill every cache slot that no valid token uses with NaN, in place."""
    nan = {"bf16": np.uint16(0x7FC0), "e4m3fn": np.uint8(0x7F), "f32": np.float32(np.nan)}[prob.kv_dtype]
    lens = np.clip(prob.seq_lens, 0, prob.max_seq_len)
    if prob.page_size == 0:
        for b, L in enumerate(lens):
            prob.k_cache[b, :, L:] = nan
            prob.v_cache[b, :, L:] = nan
        return int((prob.max_seq_len - lens).sum())
    P = prob.page_size
    used = np.zeros((prob.k_cache.shape[0], P), dtype=bool)
    for b, L in enumerate(lens):
        for blk in range(-(-int(L) // P)):
            used[prob.block_table[b, blk], :min(P, int(L) - blk * P)] = True
    for c in (prob.k_cache, prob.v_cache):
        view = c.transpose(0, 2, 1, 3)          # [pages][P][Hkv][D]
        view[~used] = nan
    return int((~used).sum())


TAIL_CASES = [
    # group, kv dtype, page size, lens, chunk, extra pages, max_seq_len
    (1, "bf16", 0, [1000, 37, 0, 513], 128, 0, 1100),
    (4, "bf16", 0, [700, 95, 1], 64, 0, 800),
    (4, "bf16", 16, [17, 500, 1023, 0], 128, 3, None),
    (8, "e4m3fn", 16, [1000, 1, 257, 30], 256, 2, None),
    (4, "e4m3fn", 0, [333, 64, 7], 64, 0, 400),
    (16, "bf16", 64, [300, 129], 64, 1, None),
    (1, "f32", 32, [333, 64, 5], 64, 1, None),
    (2, "bf16", 32, [1000, 77], 32, 0, None),
]


@pytest.mark.parametrize("g,kv,page,lens,chunk,extra,cap", TAIL_CASES)
def test_unused_cache_slots_hold_nan(g, kv, page, lens, chunk, extra, cap):
    hkv = 2
    prob = synthetic.make_problem(batch=len(lens), num_q_heads=g * hkv, num_kv_heads=hkv, seq_lens=lens,
                                  kv_dtype=kv, q_dtype="f32" if kv == "f32" else "bf16", page_size=page,
                                  chunk_size=chunk, extra_pages=extra, max_seq_len=cap, seed=700 + g)
    poisoned = _poison_unused(prob)
    print("case nan tails g=%d kv=%s page=%d lens=%s: %d slots poisoned" % (g, kv, page, lens, poisoned),
          flush=True)
    assert poisoned > 0
    dp = DeviceProblem(prob)
    dp.run()
    out, flags = dp.results()
    assert np.isfinite(out).all(), "a NaN from an unused slot reached the output"
    compare(prob, out, flags)
