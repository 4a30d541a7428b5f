"""The synthetic workloads: determinism, and the fallback flags they are built to give.

Configs 1, 2, 3 and 5 draw N(0, 1) queries and keys, so every score sits many
standard deviations inside the safe band and no row is flagged.  Config 4
scales one key in 1% of its (head, chunk) pairs by 8, which pushes that score
past phi + b; exactly the heads holding such a pair are flagged, and exactly
those chunks are recomputed (FlashDecoding++ theory page, section 3).  Every
workload keeps each score at least 1e-3 away from both band edges, so the
flag decision does not depend on the precision the scores are computed in.
"""
import numpy as np
import pytest

import oracle
import synthetic

MARGIN = 1e-3


def test_draws_are_deterministic_and_subset_stable():
    a = synthetic.make_config(3, batch=3, lens=(100, 900))
    b = synthetic.make_config(3, batch=3, lens=(100, 900))
    for x, y in [(a.q, b.q), (a.k_cache, b.k_cache), (a.v_cache, b.v_cache),
                 (a.seq_lens, b.seq_lens)]:
        np.testing.assert_array_equal(x, y)
    # the rows of (batch 1, kv head 2) do not depend on what else is drawn
    c = synthetic.make_problem(batch=3, num_q_heads=64, num_kv_heads=8, seq_lens=a.seq_lens,
                               max_seq_len=900, seed=synthetic.SEED_BASE + 3)
    np.testing.assert_array_equal(c.k_cache[1, 2], a.k_cache[1, 2])


def test_paged_layout_is_a_permutation_of_the_pool():
    p = synthetic.make_config(5, batch=6, lens=(1, 200))
    used = p.block_table[p.block_table >= 0]
    assert len(used) == len(np.unique(used)) == p.k_cache.shape[0]
    need = -(-p.seq_lens // 16)
    assert np.array_equal((p.block_table >= 0).sum(axis=1), need)


@pytest.mark.parametrize("cfg,kw", [(1, {}), (2, dict(batch=2, length=3000)),
                                    (3, dict(batch=3, lens=(1024, 6000))),
                                    (5, dict(batch=4, lens=(512, 3000)))])
def test_unperturbed_workloads_stay_inside_the_band(cfg, kw):
    p = synthetic.make_config(cfg, **kw)
    out, flags, margin = oracle.decode_exact(**p.args())
    assert flags.sum() == 0
    assert margin.min() >= MARGIN
    assert np.isfinite(out).all()


@pytest.mark.slow
def test_config4_plan_and_expected_flags():
    c = synthetic.CONFIGS[4]
    C, L = c["chunk_size"], c["max_seq_len"]
    plain = synthetic.make_config(4, perturb=False)
    plan = synthetic.load_perturbation_plan()
    pairs = synthetic.perturbation_pairs(c["num_q_heads"], L // C, 0.01, synthetic.SEED_BASE + 4)
    assert len(plan) == round(0.01 * 32 * (L // C)) == 41
    np.testing.assert_array_equal(plan[:, :2], pairs)
    # each listed key is its chunk's largest score
    for h, ch, t in plan:
        s = oracle.scores(**plain.args(), batch_index=0, head=int(h))
        assert ch * C <= t < (ch + 1) * C and t == ch * C + np.argmax(s[ch * C:(ch + 1) * C])
    del plain
    p = synthetic.make_config(4)
    out, flags, margin = oracle.decode_exact(**p.args())
    heads = set(int(h) for h in plan[:, 0])
    assert set(np.nonzero(flags)[0].tolist()) == heads
    assert margin.min() >= MARGIN
    for h, ch, t in plan:
        s = oracle.scores(**p.args(), batch_index=0, head=int(h))
        assert s[t] >= p.phi + p.b + MARGIN
    u, uf, rec = oracle.decode_unified(**p.args(), chunk_size=C)
    np.testing.assert_array_equal(uf, flags)
    assert rec.sum() == 41
    for h in range(32):
        assert rec[h] == np.count_nonzero(plan[:, 0] == h)
    np.testing.assert_allclose(u, out, rtol=0, atol=1e-12 * np.abs(out).max())
