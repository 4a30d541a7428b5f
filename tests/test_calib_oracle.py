"""Pins for the float64 calibration oracle (score extremes, histogram, band width).

FlashDecoding++ theory page, section 3: phi is set beforehand from the
observed score distribution and rows that leave the band fall back.  The
oracle reports every row's score extremes and a histogram of all scores, and
the smallest band width that keeps all but a given number of rows in band.
Each function is pinned by something other than its own code: scores
recomputed here from torch-decoded operands, numpy's histogram, direct
boolean counts, and exhaustive search over row subsets.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synthetic


def _scores(p):
    """float64 scores per row from torch-decoded operands (contiguous or paged)."""
    def dec(a, dt):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dt == "f32":
            return t.double().numpy()
        if dt == "bf16":
            return t.view(torch.int16).view(torch.bfloat16).double().numpy()
        return t.view(torch.float8_e4m3fn).double().numpy()
    q = dec(p.q, p.q_dtype)
    k = dec(p.k_cache, p.kv_dtype)
    if p.kv_dtype == "e4m3fn":
        k = k * p.k_scale.astype(np.float64)[None, :, None, None]
    g = p.num_q_heads // p.num_kv_heads
    out = []
    for b in range(p.batch):
        L = int(np.clip(p.seq_lens[b], 0, p.max_seq_len))
        for h in range(p.num_q_heads):
            kvh = h // g
            if p.page_size:
                rows = [k[p.block_table[b, t // p.page_size], kvh, t % p.page_size] for t in range(L)]
                kk = np.array(rows).reshape(L, -1)
            else:
                kk = k[b, kvh, :L]
            out.append(p.scale * kk @ q[b, h])
    return out


@pytest.mark.parametrize("kw", [
    dict(batch=3, num_q_heads=4, num_kv_heads=2, seq_lens=[40, 0, 77], head_dim=16, seed=31),
    dict(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[33, 64], head_dim=32, kv_dtype="e4m3fn",
         page_size=16, seed=32),
])
def test_extremes_and_histogram(kw):
    p = synthetic.make_problem(**kw)
    lo, hi, nb = -3.0, 2.5, 11
    mx, mn, counts = oracle.score_stats(**p.args(), hist_lo=lo, hist_hi=hi, nbins=nb)
    scores = _scores(p)
    for r, s in enumerate(scores):
        if s.size:
            np.testing.assert_allclose([mx[r], mn[r]], [s.max(), s.min()], rtol=1e-13, atol=1e-14)
        else:
            assert mx[r] == -np.inf and mn[r] == np.inf
    allv = np.concatenate(scores)
    inside, _ = np.histogram(allv[(allv >= lo) & (allv < hi)], bins=nb, range=(lo, hi))
    np.testing.assert_array_equal(counts[1:-1], inside)
    assert counts[0] == (allv < lo).sum() and counts[-1] == (allv >= hi).sum()
    assert counts.sum() == allv.size


def test_rows_in_band_counts_directly():
    rng = np.random.default_rng(7)
    mx = rng.uniform(0, 5, 200)
    mn = mx - rng.uniform(0, 6, 200)
    mx[:5], mn[:5] = -np.inf, np.inf                 # empty rows never count
    for phi, a, b in [(1.0, 4.0, 2.0), (2.5, 1.0, 3.0), (0.0, 10.0, 10.0)]:
        want = int(((phi - a <= mn) & (mx <= phi + b) & (mx >= mn)).sum())
        assert oracle.rows_in_band(mx, mn, phi, a, b) == want


@pytest.mark.parametrize("seed", range(6))
def test_min_band_width_matches_exhaustive_search(seed):
    rng = np.random.default_rng(100 + seed)
    n = 8
    mx = rng.normal(3, 1.5, n)
    mn = mx - rng.uniform(0.5, 4, n)
    if seed % 2:
        mx[2], mn[2] = -np.inf, np.inf               # an empty row
    live = [r for r in range(n) if mx[r] >= mn[r]]
    for allowed in range(0, len(live) + 1):
        need = len(live) - allowed
        if need <= 0:
            assert oracle.min_band_width(mx, mn, allowed) == 0.0
            continue
        best = min(max(mx[list(c)]) - min(mn[list(c)]) for c in itertools.combinations(live, need))
        assert oracle.min_band_width(mx, mn, allowed) == pytest.approx(best, abs=1e-12)


def test_min_band_width_closed_forms():
    # identical rows: the width is their own spread; nested rows: the outer one's
    assert oracle.min_band_width([2.0, 2.0, 2.0], [-1.0, -1.0, -1.0], 0) == 3.0
    assert oracle.min_band_width([5.0, 3.0], [-5.0, -1.0], 0) == 10.0
    assert oracle.min_band_width([5.0, 3.0], [-5.0, -1.0], 1) == 4.0
    # rows [1, 5], [0, 3], [2, 4]: the best pair spans 4, and a band of that
    # width placed on it keeps both rows
    mx, mn = np.array([5.0, 3.0, 4.0]), np.array([1.0, 0.0, 2.0])
    w = oracle.min_band_width(mx, mn, 1)
    assert w == 4.0 and oracle.rows_in_band(mx, mn, 2.0, 2.0, 2.0) == 2
