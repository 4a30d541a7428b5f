"""Pins for the float64 oracle, independent of the oracle's own code.

Each test fixes a result by something other than the oracle: a high-precision
direct evaluation, a closed form, an invariant of softmax attention, or a
library routine (scipy's softmax/expit, torch's bf16 and float8_e4m3fn
decoders).  Together they are chosen so that a dropped term, a wrong sign, a
wrong head or page index, or a transposed operand in the oracle fails at
least one of them.

Sources: FlashDecoding++ theory page, section 3 (the max-subtracted softmax,
the unified-max softmax and the out-of-band fallback); sparse-3D inference
page, section 2.2 (rows of attention weights sum to one, so identical value
rows give that row back whatever the scores are, given at least one valid
token).
"""
import decimal
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synthetic

D_SMALL = 3


def _small(batch=1, hq=1, hkv=1, lens=5, kv="f32", q="f32", d=D_SMALL, page=0, seed=1, **kw):
    return synthetic.make_problem(batch=batch, num_q_heads=hq, num_kv_heads=hkv, seq_lens=lens,
                                  q_dtype=q, kv_dtype=kv, page_size=page, head_dim=d, seed=seed,
                                  **kw)


def _decoded(arr, dtype):
    """Independent decode through torch (library)."""
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype == "f32":
        return t.double().numpy()
    if dtype == "bf16":
        return t.view(torch.int16).view(torch.bfloat16).double().numpy()
    return t.view(torch.float8_e4m3fn).double().numpy()


def _dense_kv(p):
    """float64 K, V as [B][Hkv][Lmax][D] from any layout, decoded by torch."""
    k = _decoded(p.k_cache, p.kv_dtype)
    v = _decoded(p.v_cache, p.kv_dtype)
    if p.kv_dtype == "e4m3fn":
        k = k * p.k_scale.astype(np.float64)[None, :, None, None]
        v = v * p.v_scale.astype(np.float64)[None, :, None, None]
    if p.page_size:
        B, P = p.batch, p.page_size
        kd = np.zeros((B, p.num_kv_heads, p.max_seq_len, p.head_dim))
        vd = np.zeros_like(kd)
        for b in range(B):
            for t in range(int(p.seq_lens[b])):
                pg = p.block_table[b, t // P]
                kd[b, :, t] = k[pg, :, t % P]
                vd[b, :, t] = v[pg, :, t % P]
        return kd, vd
    return k, v


# --------------------------------------------------------------------------
# brute force in 50-digit decimal arithmetic, no max subtraction
# --------------------------------------------------------------------------

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


@pytest.mark.parametrize("kv,q,seed", [("f32", "f32", 3), ("bf16", "bf16", 4),
                                        ("e4m3fn", "bf16", 5), ("bf16", "f32", 6)])
def test_brute_force_tiny(kv, q, seed):
    p = _small(batch=2, hq=2, hkv=1, lens=[4, 6], kv=kv, q=q, seed=seed, value_sigma=1.7)
    out, flags, _ = oracle.decode_exact(**p.args())
    qd = _decoded(p.q, q)
    kd, vd = _dense_kv(p)
    for b in range(2):
        for h in range(2):
            L = int(p.seq_lens[b])
            ref = _decimal_attention(qd[b, h], kd[b, 0, :L], vd[b, 0, :L], p.scale)
            np.testing.assert_allclose(out[b * 2 + h], ref, rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_single_token_returns_its_value():
    p = _small(lens=1, d=8, value_sigma=3.0)
    out, flags, _ = oracle.decode_exact(**p.args())
    np.testing.assert_array_equal(out[0], p.v_cache[0, 0, 0].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    p = _small(lens=37, d=8)
    p.q[:] = 0
    out, _, _ = oracle.decode_exact(**p.args())
    np.testing.assert_allclose(out[0], p.v_cache[0, 0, :37].astype(np.float64).mean(axis=0),
                               rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("x", [-7.5, -1.0, 0.3, 2.0, 9.0])
def test_two_tokens_logistic_weights(x):
    # q = (x, 0), k0 = (1, 0), k1 = (0, 0): s0 = scale*x, s1 = 0, w0 = expit(s0)
    p = _small(lens=2, d=2, scale=0.5)
    p.q[0, 0] = [x, 0.0]
    p.k_cache[0, 0, :2] = [[1.0, 0.0], [0.0, 0.0]]
    p.v_cache[0, 0, :2] = [[2.0, -1.0], [-3.0, 5.0]]
    out, _, _ = oracle.decode_exact(**p.args())
    w0 = scipy.special.expit(0.5 * float(p.q[0, 0, 0]))   # x as stored in float32
    ref = w0 * np.array([2.0, -1.0]) + (1 - w0) * np.array([-3.0, 5.0])
    np.testing.assert_allclose(out[0], ref, rtol=1e-14, atol=1e-15)


def test_identical_values_are_returned_whatever_the_scores():
    # attention weights of a row sum to one, so equal value rows come back unchanged
    p = _small(batch=2, hq=4, hkv=2, lens=[300, 1], kv="bf16", q="bf16", d=16, value_sigma=2.0)
    row = synthetic.bf16_round(np.linspace(-3, 3, 16).astype(np.float32))
    p.v_cache[:, :, :] = row
    out, _, _ = oracle.decode_exact(**p.args())
    ref = synthetic.bf16_to_f32(row).astype(np.float64)
    for r in range(out.shape[0]):
        np.testing.assert_allclose(out[r], ref, rtol=1e-14, atol=1e-15)


def test_one_hot_values_expose_scipy_softmax():
    # v_t = e_t turns the output into the weight vector itself
    L, D = 20, 32
    p = _small(lens=L, d=D, value_sigma=2.5)
    p.v_cache[0, 0] = 0
    p.v_cache[0, 0, :L, :L] = np.eye(L, dtype=np.float32)
    out, _, _ = oracle.decode_exact(**p.args())
    s = p.scale * (p.k_cache[0, 0, :L].astype(np.float64) @ p.q[0, 0].astype(np.float64))
    w = scipy.special.softmax(s)
    np.testing.assert_allclose(out[0, :L], w, rtol=1e-13, atol=1e-16)
    assert abs(out[0].sum() - 1.0) < 1e-14
    assert np.all(out[0, L:] == 0)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_token_permutation_invariance():
    p = _small(lens=257, d=16, kv="bf16", q="bf16", seed=9)
    out, _, _ = oracle.decode_exact(**p.args())
    perm = np.random.default_rng(0).permutation(257)
    p.k_cache[0, 0, :257] = p.k_cache[0, 0, perm]
    p.v_cache[0, 0, :257] = p.v_cache[0, 0, perm]
    out2, _, _ = oracle.decode_exact(**p.args())
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-16)


def test_gqa_equals_mha_with_repeated_kv():
    p = _small(batch=2, hq=6, hkv=2, lens=[33, 70], kv="bf16", q="bf16", d=16, seed=11)
    out, flags, _ = oracle.decode_exact(**p.args())
    m = _small(batch=2, hq=6, hkv=6, lens=[33, 70], kv="bf16", q="bf16", d=16, seed=11)
    m.q[:] = p.q
    m.k_cache = np.repeat(p.k_cache, 3, axis=1)     # q head h reads kv head h // 3
    m.v_cache = np.repeat(p.v_cache, 3, axis=1)
    out_m, flags_m, _ = oracle.decode_exact(**m.args())
    np.testing.assert_array_equal(out, out_m)
    # and the mapping is not h % Hkv: swapping the kv heads changes heads 0..2
    p.k_cache = p.k_cache[:, ::-1].copy()
    out_s, _, _ = oracle.decode_exact(**p.args())
    assert not np.allclose(out_s[:3], out[:3])


def test_paged_equals_contiguous_bitwise():
    lens = [1, 16, 17, 100]
    pg = _small(batch=4, hq=4, hkv=2, lens=lens, kv="e4m3fn", q="bf16", d=32, page=16, seed=12,
                max_seq_len=112, extra_pages=5)
    out_p, fl_p, _ = oracle.decode_exact(**pg.args())
    # same stored bits re-laid as a contiguous cache
    ct = _small(batch=4, hq=4, hkv=2, lens=lens, kv="e4m3fn", q="bf16", d=32, seed=12,
                max_seq_len=112)
    ct.q[:] = pg.q
    ct.k_scale, ct.v_scale = pg.k_scale, pg.v_scale
    ct.k_cache[:] = 0
    ct.v_cache[:] = 0
    for b, L in enumerate(lens):
        for t in range(L):
            page = pg.block_table[b, t // 16]
            ct.k_cache[b, :, t] = pg.k_cache[page, :, t % 16]
            ct.v_cache[b, :, t] = pg.v_cache[page, :, t % 16]
    out_c, fl_c, _ = oracle.decode_exact(**ct.args())
    np.testing.assert_array_equal(out_p, out_c)
    np.testing.assert_array_equal(fl_p, fl_c)


def test_fp8_scales_apply_to_keys_and_values():
    # power-of-two scales make the dequantised cache exact in float32
    p = _small(batch=1, hq=2, hkv=2, lens=50, kv="e4m3fn", q="bf16", d=16, seed=13)
    p.k_scale = np.array([0.25, 2.0], dtype=np.float32)
    p.v_scale = np.array([4.0, 0.125], dtype=np.float32)
    out, _, _ = oracle.decode_exact(**p.args())
    f = _small(batch=1, hq=2, hkv=2, lens=50, kv="f32", q="bf16", d=16, seed=13)
    f.q[:] = p.q
    f.k_cache = (_decoded(p.k_cache, "e4m3fn") * p.k_scale[None, :, None, None]).astype(np.float32)
    f.v_cache = (_decoded(p.v_cache, "e4m3fn") * p.v_scale[None, :, None, None]).astype(np.float32)
    out_f, _, _ = oracle.decode_exact(**f.args())
    np.testing.assert_allclose(out, out_f, rtol=1e-14, atol=1e-16)


def test_scale_argument_multiplies_scores():
    p = _small(lens=40, d=16, seed=14, scale=0.37)
    out, _, _ = oracle.decode_exact(**p.args())
    s = 0.37 * (p.k_cache[0, 0, :40].astype(np.float64) @ p.q[0, 0].astype(np.float64))
    ref = scipy.special.softmax(s) @ p.v_cache[0, 0, :40].astype(np.float64)
    np.testing.assert_allclose(out[0], ref, rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# safe band
# --------------------------------------------------------------------------

def _band_problem(score_values, L=None, phi=4.0, a=20.0, b=6.0):
    """D = 1, q = 1, scale = 1: score_t equals k_t exactly."""
    n = len(score_values)
    p = _small(lens=n if L is None else L, d=1, scale=1.0, phi=phi, a=a, b=b, max_seq_len=n)
    p.q[:] = 1.0
    p.k_cache[0, 0, :n, 0] = np.asarray(score_values, dtype=np.float32)
    p.v_cache[0, 0, :n, 0] = np.arange(n, dtype=np.float32)
    return p


@pytest.mark.parametrize("s,flag", [(10.0, 0), (-16.0, 0), (10.0 + 2 ** -19, 1),
                                    (-16.0 - 2 ** -19, 1), (0.0, 0), (float("nan"), 1),
                                    (float("inf"), 1), (-float("inf"), 1)])
def test_band_is_closed_and_nan_is_outside(s, flag):
    p = _band_problem([0.5, s, -1.0])
    _, flags, _ = oracle.decode_exact(**p.args())
    assert flags[0] == flag


def test_tokens_past_the_length_are_not_tested():
    p = _band_problem([0.5, 1.0, 1e6, float("nan")], L=2)
    out, flags, margin = oracle.decode_exact(**p.args())
    assert flags[0] == 0
    w = scipy.special.softmax([0.5, 1.0])
    np.testing.assert_allclose(out[0, 0], w[1], rtol=1e-14)
    assert margin[0] == pytest.approx(9.0)


def test_nan_score_poisons_the_row():
    p = _band_problem([0.5, float("nan"), 1.0])
    out, flags, _ = oracle.decode_exact(**p.args())
    assert flags[0] == 1 and np.isnan(out[0]).all()


def test_empty_and_clamped_lengths():
    p = _small(batch=3, hq=2, hkv=1, lens=[0, -5, 7], d=4, max_seq_len=6)
    out, flags, margin = oracle.decode_exact(**p.args())
    assert np.all(out[:4] == 0) and np.all(flags[:4] == 0) and np.all(np.isinf(margin[:4]))
    # length 7 > capacity 6 is clamped to 6
    q = p.q[2, 0].astype(np.float64)
    s = p.scale * (p.k_cache[2, 0, :6].astype(np.float64) @ q)
    ref = scipy.special.softmax(s) @ p.v_cache[2, 0, :6].astype(np.float64)
    np.testing.assert_allclose(out[4], ref, rtol=1e-13)


# --------------------------------------------------------------------------
# the method's steps in float64 agree with the plain definition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 16, 64, 1000, 5000])
def test_unified_max_equals_exact_and_ignores_chunking(chunk):
    p = _small(batch=2, hq=4, hkv=2, lens=[1000, 333], kv="bf16", q="bf16", d=32, seed=21)
    out, flags, _ = oracle.decode_exact(**p.args())
    assert flags.sum() == 0
    for phi in (p.phi, 0.0, 9.0):    # any preset constant with every score in the band
        p.phi = phi
        u, uf, rec = oracle.decode_unified(**p.args(), chunk_size=chunk)
        np.testing.assert_allclose(u, out, rtol=1e-13, atol=1e-15 * np.abs(out).max())
        assert rec.sum() == 0 and uf.sum() == 0


def test_flagged_chunks_are_recomputed_and_still_exact():
    p = _small(batch=1, hq=2, hkv=1, lens=4096, kv="bf16", q="bf16", d=32, seed=22)
    # scale three keys by 8 (chunks 0, 1 and 3 of 1024) and head 0's query by 3
    for t in (5, 1500, 3100):
        p.k_cache[0, 0, t] = synthetic.bf16_round(synthetic.bf16_to_f32(p.k_cache[0, 0, t]) * 8)
    p.q[0, 0] = synthetic.bf16_round(synthetic.bf16_to_f32(p.q[0, 0]) * 3)
    out, flags, _ = oracle.decode_exact(**p.args())
    u, uf, rec = oracle.decode_unified(**p.args(), chunk_size=1024)
    np.testing.assert_array_equal(uf, flags)
    for h in range(2):
        s = oracle.scores(**p.args(), batch_index=0, head=h)
        bad = np.nonzero((s < p.phi - p.a) | (s > p.phi + p.b))[0]
        assert rec[h] == len({t // 1024 for t in bad})
        assert flags[h] == (len(bad) > 0)
    assert flags[0] == 1
    np.testing.assert_allclose(u, out, rtol=1e-12, atol=1e-14 * np.abs(out).max())


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

def test_e4m3fn_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(mine[ok], ref[ok])
    # anchors of the OCP 8-bit float definition
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9 and mine[0x07] == 7 * 2.0 ** -9
    assert mine[0x38] == 1.0 and np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    assert np.count_nonzero(np.isnan(mine)) == 2
    # every finite code is exact in bf16
    fin = mine[ok]
    assert np.array_equal(torch.from_numpy(fin).to(torch.bfloat16).double().numpy(), fin)


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(3).integers(0, 1 << 16, size=4000).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]           # skip inf/nan patterns
    mine = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(mine, ref)


def test_generator_e4m3fn_encoder_matches_torch():
    x = np.random.default_rng(5).standard_normal(20000) * 100
    x = np.concatenate([x, [0.0, 448.0, 460.0, -1000.0, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625]])
    mine = synthetic.e4m3fn_encode(x)
    ref = torch.from_numpy(np.clip(x, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(mine, ref.view(torch.uint8).numpy())
