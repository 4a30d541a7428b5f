"""GPU parity of causal prefill (fd_attn_prefill) against the float64 oracle.

Bar: flags bit-exact; max|gpu - oracle| <= 2e-3 * max|oracle| over the
compared rows (the tolerance stated for bf16 operands, global over the
output as for decode), and every element within the bound the kernel's
arithmetic allows.  The kernel splits each weight into a bf16 high part and a
bf16 remainder (together a relative error <= u = 2^-18), multiplies the
values by both parts and divides by the sum of the fp32 weights, so

    |out' - out| = |sum_t w_t d_t v_t| / sum_t w_t <= u * max|v|   (|d_t| <= u)

(the test allows 2u * max|v| = 2^-17 * max|v| for this part)

plus fp32 accumulation of the weighted values and of the weight sum over n
keys in any order, <= 2 * gamma_n * max|v| with gamma_n = n 2^-24 / (1 - n 2^-24).
Inputs keep every visible score at least 1e-3 from both band edges (checked
on the oracle's margins), so the flag decision does not depend on precision.
Cases span several query tiles (128 queries) and key stages (32 keys), ragged
tails, blocks appended to a cached prefix, sequences shorter than the block
(empty early rows), empty sequences, and both fallback directions.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_device import DevicePrefill

pytestmark = pytest.mark.gpu

TOL = 2e-3   # max|err| relative to max|out|, bf16 operands


def _vmax(prob):
    """max |v| over the cache as stored (bf16 values, or E4M3FN codes times
    v_scale), ignoring NaN in slots that no key uses."""
    if not prob.v.size:
        return 0.0
    if prob.cache_dtype == "e4m3fn":
        codes = torch.from_numpy(np.ascontiguousarray(prob.v)).view(torch.float8_e4m3fn).double().abs()
        per_head = torch.nan_to_num(codes, nan=0.0).amax(dim=(0, 2, 3)).numpy()
        return float((per_head * prob.v_scale.astype(np.float64)).max())
    return float(np.nanmax(np.abs(synthetic.bf16_to_f32(prob.v))))


def _bound(prob):
    """Elementwise error bound of the kernel's arithmetic (see the top of the file)."""
    vmax = _vmax(prob)
    n = max(int(np.max(prob.kv_lens, initial=0)), 1)
    gamma = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    return (2.0 ** -17 + 2 * gamma) * vmax


def _check(prob, dp, rows=None):
    out, flags = dp.results()
    ref, ref_flags, margin = oracle.prefill_exact(**prob.args(), rows=rows)
    if rows is not None:
        out, flags = out[rows], flags[rows]
    assert margin.min() >= 1e-3, "input puts a score within 1e-3 of a band edge"
    np.testing.assert_array_equal(flags, ref_flags)
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = float(np.abs(out - ref).max())
    assert err <= TOL * scale, "max|err| %.3e > %.0e * max|out| (%.3e)" % (err, TOL, scale)
    bound = _bound(prob)
    assert err <= bound, "max|err| %.3e > arithmetic bound %.3e" % (err, bound)
    return err / scale, ref_flags


CASES = {
    "whole-and-prefixed": dict(batch=2, num_q_heads=4, num_kv_heads=1, q_len=300, kv_lens=[300, 517]),
    "one-partial-tile": dict(batch=1, num_q_heads=2, num_kv_heads=2, q_len=37, kv_lens=[37]),
    "short-and-empty": dict(batch=3, num_q_heads=8, num_kv_heads=2, q_len=129, kv_lens=[129, 100, 0]),
    "single-query": dict(batch=1, num_q_heads=8, num_kv_heads=1, q_len=1, kv_lens=[700]),
    "exact-tiles-long-prefix": dict(batch=2, num_q_heads=16, num_kv_heads=2, q_len=256,
                                    kv_lens=[1000, 256]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_small(name):
    kw = CASES[name]
    print("case prefill %s %s" % (name, kw), flush=True)
    prob = synthetic.make_prefill(**kw, seed=synthetic.SEED_BASE + 300 + sorted(CASES).index(name))
    dp = DevicePrefill(prob)
    dp.run()
    rel, ref_flags = _check(prob, dp)
    assert not ref_flags.any()
    print("rel err %.3e" % rel)


def test_prefill_config_small():
    prob = synthetic.make_prefill_config(1)
    print("case prefill config1 kv=%s" % prob.kv_lens.tolist(), flush=True)
    dp = DevicePrefill(prob)
    dp.run()
    rel, _ = _check(prob, dp)
    print("rel err %.3e" % rel)


def test_prefill_bf16_output_is_the_rounded_f32_output():
    prob = synthetic.make_prefill(**CASES["whole-and-prefixed"], seed=77)
    print("case prefill bf16 out", flush=True)
    a = DevicePrefill(prob, out_dtype="f32")
    b = DevicePrefill(prob, out_dtype="bf16")
    a.run()
    b.run()
    torch.cuda.synchronize()
    assert torch.equal(a.out.to(torch.bfloat16), b.out)
    assert torch.equal(a.flags, b.flags)


def test_prefill_fallback_overflow_mid_row():
    # keys at positions 200 and 333 scaled by 8 (exact in bf16): the rows that
    # see them score far above phi + b and switch to online softmax after
    # several in-band stages
    prob = synthetic.make_prefill(batch=1, num_q_heads=4, num_kv_heads=1, q_len=400,
                                  kv_lens=[400], seed=91)
    for t in (200, 333):
        prob.k[0, 0, t] = synthetic.bf16_round(synthetic.bf16_to_f32(prob.k[0, 0, t]) * 8)
    print("case prefill overflow", flush=True)
    dp = DevicePrefill(prob)
    dp.run()
    rel, ref_flags = _check(prob, dp)
    flags = ref_flags.reshape(4, 400)
    assert flags[:, :200].sum() == 0 and flags.sum() > 0
    print("rel err %.3e, %d rows flagged" % (rel, int(ref_flags.sum())))


def test_prefill_fallback_underflow_everywhere():
    # band [10, 36]: every score lies below it, so exp(s - phi) alone would
    # underflow; every row with a key is flagged and computed online from the
    # first stage
    prob = synthetic.make_prefill(batch=2, num_q_heads=4, num_kv_heads=2, q_len=150,
                                  kv_lens=[150, 90], phi=30.0, a=20.0, b=6.0, seed=92)
    print("case prefill underflow", flush=True)
    dp = DevicePrefill(prob)
    dp.run()
    rel, ref_flags = _check(prob, dp)
    pos = np.concatenate([np.tile(np.arange(150), 4), np.tile(np.arange(150) - 60, 4)])
    np.testing.assert_array_equal(ref_flags, (pos >= 0).astype(np.uint8))
    print("rel err %.3e" % rel)


def test_prefill_fallback_in_one_head_only():
    prob = synthetic.make_prefill(batch=1, num_q_heads=8, num_kv_heads=2, q_len=256,
                                  kv_lens=[256], seed=93)
    prob.q[0, 5] = synthetic.bf16_round(synthetic.bf16_to_f32(prob.q[0, 5]) * 4)
    print("case prefill one head", flush=True)
    dp = DevicePrefill(prob)
    dp.run()
    rel, ref_flags = _check(prob, dp)
    flags = ref_flags.reshape(8, 256)
    assert flags[5].any() and flags[np.arange(8) != 5].sum() == 0
    print("rel err %.3e" % rel)


def test_prefill_full_config():
    prob = synthetic.make_prefill_config(2)
    B, Hq, Lq = prob.batch, prob.num_q_heads, prob.q_len
    print("case prefill full config2 %s" % prob.workload, flush=True)
    dp = DevicePrefill(prob)
    dp.run()
    # every visible score inside the band with margin (fp32 scores, per head),
    # so the expected flags are all zero
    q = dp.q.float()
    k = dp.k.float()
    mask = torch.ones(Lq, Lq, dtype=torch.bool, device="cuda").tril()
    lo, hi = prob.phi - prob.a, prob.phi + prob.b
    smin, smax = float("inf"), -float("inf")
    for b in range(B):
        for h in range(Hq):
            kt = k[b, h // (Hq // prob.num_kv_heads)].t().contiguous()
            s = torch.matmul(q[b, h], kt) * prob.scale
            vis = s[mask]
            smin = min(smin, float(vis.min()))
            smax = max(smax, float(vis.max()))
    assert smin >= lo + 1e-3 and smax <= hi - 1e-3
    torch.cuda.synchronize()
    assert int(dp.flags.sum()) == 0
    # every row of two whole heads (one per sequence, different KV heads),
    # and sampled rows of three more -- every query tile boundary region and
    # both ends -- against the oracle
    rng = np.random.default_rng(5)
    js = np.unique(np.concatenate([[0, 1, 127, 128, 129, Lq // 2, Lq - 2, Lq - 1],
                                   rng.integers(0, Lq, 40)]))
    bh = [(0, 3), (0, 31), (1, 7)]
    rows = [(b * Hq + h) * Lq + j for b, h in bh for j in js]
    for b, h in [(0, 0), (1, 16)]:
        rows.extend((b * Hq + h) * Lq + np.arange(Lq))
    rows = np.array(rows, dtype=np.int32)
    rel, _ = _check(prob, dp, rows=rows)
    # the stated bar also on the long rows alone (their outputs are small)
    out, _ = dp.results()
    tail = np.array([(b * Hq + h) * Lq + j for b, h in [(0, 0), (1, 16)] for j in range(Lq - 512, Lq)],
                    dtype=np.int32)
    ref_tail, _, _ = oracle.prefill_exact(**prob.args(), rows=tail)
    err_tail = float(np.abs(out[tail] - ref_tail).max())
    assert err_tail <= TOL * float(np.abs(ref_tail).max()), "last 512 rows: max|err| %.3e" % err_tail
    out1 = dp.out.clone()
    dp.run()
    torch.cuda.synchronize()
    assert torch.equal(out1, dp.out)
    print("full config2: rel err %.3e on %d sampled rows, scores in [%.3f, %.3f]"
          % (rel, len(rows), smin, smax))


FORMAT_CASES = [
    # kv dtype, page size, case
    ("bf16", 16, "whole-and-prefixed"), ("bf16", 32, "short-and-empty"),
    ("e4m3fn", 0, "whole-and-prefixed"), ("e4m3fn", 0, "single-query"),
    ("e4m3fn", 16, "exact-tiles-long-prefix"), ("e4m3fn", 64, "one-partial-tile"),
    ("bf16", 256, "exact-tiles-long-prefix"),
]


@pytest.mark.parametrize("kv,page,name", FORMAT_CASES)
def test_prefill_cache_formats(kv, page, name):
    # E4M3FN caches (per-KV-head scales) and paged caches (permuted pages,
    # spare pages in the pool), the decode call's formats
    kw = CASES[name]
    print("case prefill %s kv=%s page=%d" % (name, kv, page), flush=True)
    prob = synthetic.make_prefill(**kw, kv_dtype=kv, page_size=page, extra_pages=2 if page else 0,
                                  seed=synthetic.SEED_BASE + 320 + sorted(CASES).index(name))
    dp = DevicePrefill(prob)
    dp.run()
    rel, ref_flags = _check(prob, dp)
    assert not ref_flags.any()
    print("rel err %.3e" % rel)


@pytest.mark.parametrize("kv", ["bf16", "e4m3fn"])
def test_prefill_paged_equals_contiguous_bitwise(kv):
    kw = dict(batch=3, num_q_heads=8, num_kv_heads=2, q_len=200, kv_lens=[200, 517, 64], kv_dtype=kv,
              seed=94, phi=1.0, a=2.5, b=2.0)
    print("case prefill paged = contiguous kv=%s" % kv, flush=True)
    flat = DevicePrefill(synthetic.make_prefill(**kw))
    paged = DevicePrefill(synthetic.make_prefill(**kw, page_size=16, extra_pages=5))
    flat.run()
    paged.run()
    torch.cuda.synchronize()
    assert torch.equal(flat.out, paged.out) and torch.equal(flat.flags, paged.flags)
    assert int(flat.flags.sum()) > 0     # the narrow band sends rows to the online path


@pytest.mark.parametrize("kv,page", [("bf16", 16), ("e4m3fn", 16), ("e4m3fn", 0), ("bf16", 0)])
def test_prefill_unused_cache_slots_hold_nan(kv, page):
    prob = synthetic.make_prefill(batch=3, num_q_heads=4, num_kv_heads=2, q_len=70, kv_lens=[70, 133, 20],
                                  kv_dtype=kv, page_size=page, extra_pages=3 if page else 0,
                                  max_seq_len=None if page else 180, seed=95)
    nan = np.uint16(0x7FC0) if kv == "bf16" else np.uint8(0x7F)
    lens = prob.kv_lens
    if page:
        used = np.zeros((prob.k.shape[0], page), dtype=bool)
        for b, L in enumerate(lens):
            for blk in range(-(-int(L) // page)):
                used[prob.block_table[b, blk], :min(page, int(L) - blk * page)] = True
        for c in (prob.k, prob.v):
            c.transpose(0, 2, 1, 3)[~used] = nan
    else:
        for b, L in enumerate(lens):
            prob.k[b, :, L:] = nan
            prob.v[b, :, L:] = nan
    print("case prefill nan tails kv=%s page=%d" % (kv, page), flush=True)
    dp = DevicePrefill(prob)
    dp.run()
    out, _ = dp.results()
    assert np.isfinite(out).all()
    _check(prob, dp)
