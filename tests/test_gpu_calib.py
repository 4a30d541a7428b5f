"""GPU parity of the score-statistics pass (fd_attn_score_stats) against the
float64 calibration oracle, and the calibration loop end to end.

Bar: extremes within fp32 score rounding of the oracle's (2e-5 * (1 + max|s|));
empty rows exactly -inf / +inf; the histogram's total exactly the number of
valid scores, and every bin within the number of scores that lie within 1e-4
of one of its edges (the GPU bins fp32 scores, the oracle float64 ones).
End to end: a band chosen to keep every row raises no flag in the decode
call, and a band chosen to flag some rows flags exactly the rows the
chooser counted.
"""
import numpy as np
import pytest
import torch

import oracle
import split_kv_asynchronous_amd as fd
import synthetic
from gpu_device import DeviceProblem
from gpu_helpers import compare

pytestmark = pytest.mark.gpu


def _gpu_stats(dp, lo, hi, nbins):
    p = dp.prob
    mx, mn, hist = fd.fd_attn_score_stats(dp.q, dp.k, dp.seq_lens, dp.block_table,
                                          max_seq_len=p.max_seq_len, chunk_size=p.chunk_size,
                                          num_kv_heads=p.num_kv_heads, page_size=p.page_size,
                                          scale=p.scale, k_scale=dp.k_scale, hist_lo=lo,
                                          hist_hi=hi, nbins=nbins, q_dtype=p.q_dtype,
                                          kv_dtype=p.kv_dtype)
    torch.cuda.synchronize()
    h = None if hist is None else hist.cpu().numpy().view(np.uint32).astype(np.int64)
    return mx.cpu().numpy().ravel(), mn.cpu().numpy().ravel(), h


def _check(prob, gmx, gmn, ghist, lo, hi, nbins, per_score=True):
    mx, mn, counts = oracle.score_stats(**prob.args(), hist_lo=lo, hist_hi=hi, nbins=nbins)
    empty = mx == -np.inf
    assert np.all(gmx[empty] == -np.inf) and np.all(gmn[empty] == np.inf)
    live = ~empty
    tol = 2e-5 * (1.0 + max(np.abs(mx[live]).max(initial=0), np.abs(mn[live]).max(initial=0)))
    np.testing.assert_allclose(gmx[live], mx[live], rtol=0, atol=tol)
    np.testing.assert_allclose(gmn[live], mn[live], rtol=0, atol=tol)
    if ghist is None:
        return
    assert ghist.sum() == counts.sum()
    if not per_score:
        return
    edges = lo + (hi - lo) * np.arange(nbins + 1) / nbins
    near = np.zeros(nbins + 2, dtype=np.int64)     # scores within 1e-4 of a slot's edges
    for b in range(prob.batch):
        for h in range(prob.num_q_heads):
            s = oracle.scores(**prob.args(), batch_index=b, head=h)
            if s.size == 0:
                continue
            idx = np.searchsorted(edges, s, side="right")   # slot of each score
            d = np.abs(s[:, None] - edges[None, :]).min(axis=1)
            for sl, dd in zip(idx, d):
                if dd < 1e-4:
                    near[max(sl - 1, 0):min(sl + 2, nbins + 2)] += 1
    assert np.all(np.abs(ghist - counts) <= near), (ghist - counts, near)


CASES = [
    (1, dict(length=1500)),                  # fp32 MHA
    (2, dict(batch=2, length=3000)),         # bf16 MHA
    (3, dict(batch=3, lens=(1, 5000))),      # bf16 GQA (group 8)
    (5, dict(batch=4, lens=(1, 3000))),      # fp8 paged GQA
]


@pytest.mark.parametrize("cfg,kw", CASES, ids=["cfg%d" % c for c, _ in CASES])
def test_stats_small(cfg, kw):
    prob = synthetic.make_config(cfg, **kw)
    print("case stats cfg%d %s" % (cfg, kw), flush=True)
    dp = DeviceProblem(prob)
    lo, hi, nb = -6.0, 6.0, 240
    gmx, gmn, gh = _gpu_stats(dp, lo, hi, nb)
    _check(prob, gmx, gmn, gh, lo, hi, nb)


def test_stats_group16_and_empty_rows():
    prob = synthetic.make_problem(batch=3, num_q_heads=32, num_kv_heads=2, seq_lens=[700, 0, 2100],
                                  seed=41)
    print("case stats group 16", flush=True)
    dp = DeviceProblem(prob)
    gmx, gmn, gh = _gpu_stats(dp, -5.0, 5.0, 100)
    _check(prob, gmx, gmn, gh, -5.0, 5.0, 100)
    gmx2, gmn2, gh2 = _gpu_stats(dp, 0.0, 0.0, 0)          # no histogram
    assert gh2 is None and np.array_equal(gmx2, gmx) and np.array_equal(gmn2, gmn)


@pytest.mark.parametrize("kv", ["bf16", "e4m3fn"])
@pytest.mark.parametrize("page_size,nbins", [(16, 200), (64, 8000), (0, 300)])
def test_stats_grouped_layouts(kv, page_size, nbins):
    # grouped bf16 queries over paged and contiguous caches, ragged lengths
    # across chunk, page and 16-token boundaries (17, 2049: a group's second
    # half past the end); 8000 bins take the two-stage ring
    prob = synthetic.make_problem(batch=3, num_q_heads=16, num_kv_heads=2, kv_dtype=kv,
                                  seq_lens=[2049, 17, 4133], page_size=page_size, seed=43)
    print("case stats %s page %d nbins %d" % (kv, page_size, nbins), flush=True)
    dp = DeviceProblem(prob)
    gmx, gmn, gh = _gpu_stats(dp, -6.0, 6.0, nbins)
    _check(prob, gmx, gmn, gh, -6.0, 6.0, nbins)


def test_stats_full_gqa32k():
    prob = synthetic.make_config(3)
    print("case stats full cfg3", flush=True)
    dp = DeviceProblem(prob)
    gmx, gmn, gh = _gpu_stats(dp, -8.0, 8.0, 4096)
    _check(prob, gmx, gmn, gh, -8.0, 8.0, 4096, per_score=False)


def test_calibrated_band_end_to_end():
    prob = synthetic.make_config(3, batch=4, lens=(100, 5000))
    print("case calibration end to end", flush=True)
    dp = DeviceProblem(prob)
    gmx, gmn, _ = _gpu_stats(dp, 0.0, 0.0, 0)
    # a band that keeps every row: no flag, exact result
    phi, a, b, flagged = fd.fd_attn_choose_band(gmx, gmn, 0.0, 0.7, 40.0, 1e-3)
    assert flagged == 0
    dp.run(phi=phi, a=a, b=b)
    out, flags = dp.results()
    assert flags.sum() == 0
    compare(prob, out, flags, ref=oracle.decode_exact(**dict(prob.args(), phi=phi, a=a, b=b))[:2])
    # a band that flags about a quarter of the rows: the decode call flags
    # exactly the rows the chooser counted (when no row sits near an edge)
    phi, a, b, flagged = fd.fd_attn_choose_band(gmx, gmn, 0.25, 0.5, 40.0, 1e-3)
    m = int((gmx >= gmn).sum())
    assert 0 < flagged <= m // 4
    dp.run(phi=phi, a=a, b=b)
    out, flags = dp.results()
    lo_e, hi_e = phi - a, phi + b
    omx, omn, _ = oracle.score_stats(**prob.args())
    live = omx >= omn
    clear = ~live | (np.minimum(np.abs(omx - hi_e), np.abs(omn - lo_e)) > 1e-4)
    if clear.all():
        assert int(flags.sum()) == flagged
    ref = oracle.decode_exact(**dict(prob.args(), phi=phi, a=a, b=b))
    np.testing.assert_array_equal(flags[clear], ref[1][clear])
    out_ok = np.abs(out - ref[0]).max() <= 2e-3 * np.abs(ref[0]).max()
    assert out_ok
    print("band [%.3f, %.3f] phi %.3f flags %d of %d rows" % (lo_e, hi_e, phi, flagged, m))
