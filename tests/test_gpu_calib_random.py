"""GPU parity of the score-statistics pass on seeded random shapes, through the
C ABI: the decode shapes of the random decode sweep (formats, query groups,
paging, ragged and empty sequences), each with its own histogram range and bin
count (none, one bin, or many).  Bar as in the other statistics tests: extremes
within fp32 score rounding of the float64 oracle, empty rows exactly -inf /
+inf, the histogram total exact, and -- where the case is small enough to list
every score -- every bin within the number of scores lying within 1e-4 of one
of its edges.
"""
import numpy as np
import pytest

import synthetic
from gpu_device import DeviceProblem
from test_gpu_calib import _check, _gpu_stats
from test_gpu_random_shapes import NCASES, draw_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("i", range(NCASES))
def test_stats_random_shape(i):
    kw = draw_case(i)
    rng = np.random.default_rng(0x5EED6000 + i)
    nbins = int(rng.choice([0, 1, 64, 4096]))
    lo = float(rng.uniform(-8.0, -0.5))
    hi = float(lo + rng.uniform(0.5, 12.0))
    print("case stats %d: nbins %d range [%.3f, %.3f) %s" % (
        i, nbins, lo, hi, {k: (v.tolist() if isinstance(v, np.ndarray) else v)
                           for k, v in kw.items()}), flush=True)
    prob = synthetic.make_problem(**kw)
    dp = DeviceProblem(prob)
    gmx, gmn, ghist = _gpu_stats(dp, lo, hi, nbins)
    nscores = int(np.clip(prob.seq_lens, 0, prob.max_seq_len).sum()) * prob.num_q_heads
    _check(prob, gmx, gmn, ghist, lo, hi, nbins, per_score=nscores <= 200_000)
