"""Pins for the float64 prefill oracle (causal query block), independent of its code.

The prefill form of the method (FlashDecoding++ theory page, section 3: the
unified maximum is used in prefill as well as decode; section 1: prefill takes
all prompt tokens in one pass) scores a block of queries against the keys of
their own sequence up to their own position.  Each test fixes a result by
something other than the oracle: 50-digit decimal brute force, scipy's softmax
over a causal mask built by numpy, closed forms, invariants of causal softmax
attention, and the already-pinned decode oracle (a block of one query is a
decode step).
"""
import decimal

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synthetic


def _small(batch=1, hq=1, hkv=1, lq=5, kv=5, dtype="f32", d=4, seed=1, **kw):
    return synthetic.make_prefill(batch=batch, num_q_heads=hq, num_kv_heads=hkv, q_len=lq,
                                  kv_lens=kv, dtype=dtype, head_dim=d, seed=seed, **kw)


def _f64(arr, dtype):
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype == "f32":
        return t.double().numpy()
    return t.view(torch.int16).view(torch.bfloat16).double().numpy()


def _row(p, b, h, j):
    return (b * p.num_q_heads + h) * p.q_len + j


def _decimal_attention(qv, K, V, scale):
    ctx = decimal.Context(prec=50)
    Dm = decimal.Decimal
    sc = Dm(float(scale))
    s = [ctx.multiply(sc, sum((ctx.multiply(Dm(float(a)), Dm(float(b))) for a, b in zip(qv, k)),
                              Dm(0))) for k in K]
    e = [ctx.exp(x) for x in s]
    z = sum(e, Dm(0))
    return [float(sum((ctx.multiply(w, Dm(float(v[d]))) for w, v in zip(e, V)), Dm(0)) / z)
            for d in range(len(V[0]))]


@pytest.mark.parametrize("dtype,seed", [("f32", 11), ("bf16", 12)])
def test_brute_force_tiny(dtype, seed):
    # two sequences: a whole prompt (Lq == kv) and a block after a cached prefix
    p = _small(batch=2, hq=2, hkv=1, lq=4, kv=[4, 7], dtype=dtype, seed=seed, value_sigma=1.6)
    out, flags, _ = oracle.prefill_exact(**p.args())
    q, k, v = _f64(p.q, dtype), _f64(p.k, dtype), _f64(p.v, dtype)
    for b in range(2):
        for h in range(2):
            for j in range(4):
                pos = int(p.kv_lens[b]) - 4 + j
                ref = _decimal_attention(q[b, h, j], k[b, 0, :pos + 1], v[b, 0, :pos + 1], p.scale)
                np.testing.assert_allclose(out[_row(p, b, h, j)], ref, rtol=1e-13, atol=1e-15)


def test_matches_scipy_softmax_over_a_tril_mask():
    p = _small(batch=1, hq=3, hkv=3, lq=40, kv=40, d=16, seed=13)
    out, _, _ = oracle.prefill_exact(**p.args())
    q, k, v = _f64(p.q, "f32"), _f64(p.k, "f32"), _f64(p.v, "f32")
    mask = np.tril(np.ones((40, 40), dtype=bool))
    for h in range(3):
        s = p.scale * q[0, h] @ k[0, h].T
        w = scipy.special.softmax(np.where(mask, s, -np.inf), axis=1)
        np.testing.assert_allclose(out[h * 40:(h + 1) * 40], w @ v[0, h], rtol=1e-12, atol=1e-14)


def test_single_query_block_is_a_decode_step():
    # Lq = 1: the query sits at the last position and sees every key
    p = _small(batch=3, hq=4, hkv=2, lq=1, kv=[9, 1, 33], dtype="bf16", d=32, seed=14)
    out, flags, margin = oracle.prefill_exact(**p.args())
    ref, rflags, rmargin = oracle.decode_exact(
        p.q[:, :, 0, :], p.k, p.v, p.kv_lens, num_kv_heads=2, max_seq_len=p.max_seq_len,
        q_dtype="bf16", kv_dtype="bf16", scale=p.scale, phi=p.phi, a=p.a, b=p.b)
    np.testing.assert_array_equal(out, ref)
    np.testing.assert_array_equal(flags, rflags)
    np.testing.assert_array_equal(margin, rmargin)


def test_first_position_returns_its_value():
    p = _small(batch=1, hq=2, hkv=1, lq=6, kv=6, d=8, value_sigma=3.0, seed=15)
    out, _, _ = oracle.prefill_exact(**p.args())
    for h in range(2):
        np.testing.assert_array_equal(out[_row(p, 0, h, 0)], p.v[0, 0, 0].astype(np.float64))


def test_zero_queries_give_running_means_of_values():
    p = _small(batch=1, hq=1, hkv=1, lq=25, kv=60, d=8, seed=16)
    p.q[:] = 0
    out, _, _ = oracle.prefill_exact(**p.args())
    v = p.v[0, 0].astype(np.float64)
    means = np.cumsum(v, axis=0) / np.arange(1, 61)[:, None]
    np.testing.assert_allclose(out, means[35:60], rtol=1e-13, atol=1e-15)


def test_future_keys_do_not_matter_and_past_keys_do():
    p = _small(batch=1, hq=1, hkv=1, lq=12, kv=12, d=8, seed=17)
    base, _, _ = oracle.prefill_exact(**p.args())
    p.k[0, 0, 7] *= -3.0
    p.v[0, 0, 7] += 1.0
    moved, _, _ = oracle.prefill_exact(**p.args())
    np.testing.assert_array_equal(moved[:7], base[:7])          # positions 0..6 cannot see key 7
    assert np.all(np.abs(moved[7:] - base[7:]).max(axis=1) > 1e-6)


def test_gqa_equals_mha_with_repeated_kv():
    p = _small(batch=2, hq=6, hkv=2, lq=9, kv=[9, 20], dtype="bf16", d=16, seed=18)
    out, flags, _ = oracle.prefill_exact(**p.args())
    rep = synthetic.PrefillProblem(q=p.q, k=np.repeat(p.k, 3, axis=1), v=np.repeat(p.v, 3, axis=1),
                                   kv_lens=p.kv_lens, num_kv_heads=6, dtype="bf16", scale=p.scale,
                                   phi=p.phi, a=p.a, b=p.b)
    out2, flags2, _ = oracle.prefill_exact(**rep.args())
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(flags, flags2)


def test_identical_values_are_returned_whatever_the_scores():
    p = _small(batch=1, hq=2, hkv=1, lq=30, kv=50, dtype="bf16", d=16, value_sigma=4.0, seed=19)
    row = synthetic.bf16_round(np.linspace(-2, 2, 16).astype(np.float32))
    p.v[0, 0, :50] = row
    out, _, _ = oracle.prefill_exact(**p.args())
    np.testing.assert_allclose(out, np.broadcast_to(_f64(row, "bf16"), out.shape), rtol=1e-13)


def test_short_sequences_leave_early_queries_empty():
    # kv_len < Lq: queries at negative positions see nothing; kv_len 0: every row empty
    p = _small(batch=2, hq=1, hkv=1, lq=10, kv=[4, 0], d=8, seed=20, max_seq_len=4)
    out, flags, margin = oracle.prefill_exact(**p.args())
    assert np.all(out[:6] == 0) and np.all(flags[:6] == 0) and np.all(np.isinf(margin[:6]))
    np.testing.assert_array_equal(out[6], p.v[0, 0, 0].astype(np.float64))
    assert np.all(out[10:] == 0) and np.all(flags[10:] == 0)


@pytest.mark.parametrize("at", [0, 20, 31])
def test_flags_see_only_visible_scores(at):
    # one huge key at position `at`: flagged exactly for the queries that see it
    p = _small(batch=1, hq=1, hkv=1, lq=32, kv=32, d=4, seed=21, phi=0.0, a=30.0, b=30.0)
    p.q[0, 0] = np.abs(p.q[0, 0]) + 0.5
    p.k[0, 0, at] = 400.0
    out, flags, margin = oracle.prefill_exact(**p.args())
    np.testing.assert_array_equal(flags, (np.arange(32) >= at).astype(np.uint8))
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("tile", [1, 7, 16, 64, 1000])
def test_unified_steps_equal_exact_and_ignore_tiling(tile):
    p = synthetic.make_prefill_config(1, q_len=37)
    rows = np.arange(0, p.batch * p.num_q_heads * p.q_len, 5)
    ex, fe, margin = oracle.prefill_exact(**p.args(), rows=rows)
    un, fu, red = oracle.prefill_unified(**p.args(), tile=tile, rows=rows)
    assert margin.min() > 1e-3 and not fe.any()
    np.testing.assert_array_equal(fu, fe)
    assert not red.any()
    np.testing.assert_allclose(un, ex, rtol=1e-12, atol=1e-13)


def test_out_of_band_tiles_are_redone_and_still_exact():
    # scores far above and far below the band: without the redo the first
    # overflows exp(s - phi) and the second underflows it to zero
    p = _small(batch=1, hq=2, hkv=2, lq=48, kv=64, d=8, seed=22, phi=0.0, a=5.0, b=5.0)
    p.q[0, 0] = 1.0
    p.k[0, 0, :] = 0.0
    p.k[0, 0, 40, :] = 300.0                  # head 0: s = 300 * 8 / sqrt(8) for key 40
    p.q[0, 1] = -1.0
    p.k[0, 1, :] = 300.0                      # head 1: every score far below the band
    ex, fe, _ = oracle.prefill_exact(**p.args())
    for tile in (3, 16, 64):
        un, fu, red = oracle.prefill_unified(**p.args(), tile=tile)
        np.testing.assert_array_equal(fu, fe)
        assert np.all(np.isfinite(un))
        np.testing.assert_allclose(un, ex, rtol=1e-12, atol=1e-13)
        # head 0: queries at positions >= 40 flagged (one tile redone); head 1: all rows
        pos = 16 + np.arange(48)
        np.testing.assert_array_equal(fu[:48], (pos >= 40).astype(np.uint8))
        assert np.all(red[:48][pos >= 40] == 1) and not red[:48][pos < 40].any()
        assert np.all(fu[48:] == 1)
        np.testing.assert_array_equal(red[48:], (pos + 1 + tile - 1) // tile)


@pytest.mark.parametrize("kv_dtype", ["bf16", "e4m3fn"])
def test_paged_cache_equals_contiguous_bit_for_bit(kv_dtype):
    # the same draws stored in permuted 16-token pages (decode's paged layout)
    kw = dict(batch=3, hq=4, hkv=2, lq=37, kv=[37, 100, 20], d=32, seed=31, dtype="bf16",
              kv_dtype=kv_dtype)
    flat = _small(**kw)
    paged = _small(page_size=16, extra_pages=3, **kw)
    assert paged.block_table is not None and paged.k.shape[2] == 16
    a = oracle.prefill_exact(**flat.args())
    b = oracle.prefill_exact(**paged.args())
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_e4m3fn_cache_equals_its_dequantised_values():
    # codes times per-KV-head scales: with power-of-two scales the products are
    # exact in float32, so an fp32 cache holding them gives the same bits
    p = _small(batch=2, hq=4, hkv=2, lq=30, kv=[30, 45], d=16, seed=32, dtype="bf16", kv_dtype="e4m3fn")
    p.k_scale = np.array([2.0 ** -6, 2.0 ** -5], dtype=np.float32)
    p.v_scale = np.array([2.0 ** -7, 2.0 ** -4], dtype=np.float32)
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()   # torch's decoder
    kf = (dec(p.k) * p.k_scale[None, :, None, None]).astype(np.float32)
    vf = (dec(p.v) * p.v_scale[None, :, None, None]).astype(np.float32)
    args = p.args()
    got = oracle.prefill_exact(**args)
    args.update(k=kf, v=vf, kv_dtype="f32", k_scale=None, v_scale=None)
    ref = oracle.prefill_exact(**args)
    for x, y in zip(got, ref):
        np.testing.assert_array_equal(x, y)
    # and against torch's E4M3FN decoder with the generator's own scales
    q = _small(batch=1, hq=2, hkv=1, lq=8, kv=8, d=16, seed=33, dtype="bf16", kv_dtype="e4m3fn")
    kd = torch.from_numpy(q.k).view(torch.float8_e4m3fn).double().numpy() * float(q.k_scale[0])
    vd = torch.from_numpy(q.v).view(torch.float8_e4m3fn).double().numpy() * float(q.v_scale[0])
    out, _, _ = oracle.prefill_exact(**q.args())
    qq = _f64(q.q, "bf16")
    mask = np.tril(np.ones((8, 8), dtype=bool))
    for h in range(2):
        s = q.scale * qq[0, h] @ kd[0, 0].T
        w = scipy.special.softmax(np.where(mask, s, -np.inf), axis=1)
        np.testing.assert_allclose(out[h * 8:(h + 1) * 8], w @ vd[0, 0], rtol=1e-12, atol=1e-14)


def test_single_query_block_on_a_paged_e4m3fn_cache_is_a_decode_step():
    p = _small(batch=3, hq=4, hkv=2, lq=1, kv=[40, 1, 97], dtype="bf16", d=32, seed=34, kv_dtype="e4m3fn",
               page_size=16, extra_pages=2)
    out, flags, margin = oracle.prefill_exact(**p.args())
    ref, rflags, rmargin = oracle.decode_exact(
        p.q[:, :, 0, :], p.k, p.v, p.kv_lens, p.block_table, num_kv_heads=2, max_seq_len=p.max_seq_len,
        page_size=16, q_dtype="bf16", kv_dtype="e4m3fn", scale=p.scale, phi=p.phi, a=p.a, b=p.b,
        k_scale=p.k_scale, v_scale=p.v_scale)
    np.testing.assert_array_equal(out, ref)
    np.testing.assert_array_equal(flags, rflags)
    np.testing.assert_array_equal(margin, rmargin)


def test_unified_steps_on_paged_e4m3fn_cache_equal_exact():
    p = _small(batch=2, hq=4, hkv=2, lq=50, kv=[50, 80], d=32, seed=35, dtype="bf16", kv_dtype="e4m3fn",
               page_size=16, phi=1.0, a=2.0, b=1.5)
    exact, eflags, _ = oracle.prefill_exact(**p.args())
    args = p.args()
    uni, uflags, redone = oracle.prefill_unified(**args, tile=32)
    assert redone.sum() > 0
    np.testing.assert_array_equal(uflags, eflags)
    np.testing.assert_allclose(uni, exact, rtol=1e-12, atol=1e-13)
