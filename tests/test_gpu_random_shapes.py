"""GPU parity on seeded random decode shapes, through the C ABI.

Each case draws a batch, a query-head group over 1-4 KV heads, ragged lengths
(some sequences empty), a chunk size, a cache layout (contiguous, possibly with
spare capacity, or paged with 16-64-token pages), query and cache formats, and
either a wide band (no score leaves it) or a narrow one (many chunks are
recomputed with online softmax).  Bar as in the other parity tests: max|err|
<= tol * max|oracle| over every row, flags bit-exact on every row whose scores
all lie at least 1e-3 from both band edges (a row with a score closer than that
may take either path; its output is the exact softmax either way).
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_helpers import DeviceProblem, compare

pytestmark = pytest.mark.gpu

NCASES = 32


def draw_case(i):
    """Shape and band of case i (a pure function of i)."""
    rng = np.random.default_rng(0x5EED2000 + i)
    kv = ["f32", "bf16", "e4m3fn"][rng.integers(3)]
    q = "f32" if kv == "f32" else ("f32" if rng.random() < 0.25 else "bf16")
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 16]))
    batch = int(rng.integers(1, 7))
    lmax = int(rng.choice([40, 300, 1500, 5000]))
    lens = rng.integers(0, lmax + 1, size=batch)
    lens[rng.random(batch) < 0.15] = 0
    page = int(rng.choice([0, 0, 16, 32, 64]))
    chunks = [c for c in (32, 64, 96, 128, 256, 512, 1024) if page == 0 or c % page == 0]
    chunk = int(rng.choice(chunks))
    cap = int(max(lens.max(), 1))
    if page == 0 and rng.random() < 0.5:
        cap += int(rng.integers(1, 200))            # spare capacity past the longest sequence
    if rng.random() < 0.5:
        phi, a, b = float(rng.uniform(2.0, 5.0)), 20.0, 6.0
    else:
        phi, a, b = float(rng.uniform(-0.5, 1.5)), float(rng.uniform(1.5, 4.0)), float(rng.uniform(1.0, 3.0))
    return dict(batch=batch, num_q_heads=g * hkv, num_kv_heads=hkv, seq_lens=lens.astype(np.int32),
                q_dtype=q, kv_dtype=kv, page_size=page, chunk_size=chunk, max_seq_len=cap,
                phi=phi, a=a, b=b, seed=0x5EED3000 + i)


@pytest.mark.parametrize("i", range(NCASES))
def test_random_shape(i):
    kw = draw_case(i)
    print("case %d: %s" % (i, {k: (v.tolist() if isinstance(v, np.ndarray) else v)
                               for k, v in kw.items()}), flush=True)
    prob = synthetic.make_problem(**kw)
    ref_out, ref_flags, margin = oracle.decode_exact(**prob.args())
    dp = DeviceProblem(prob)
    dp.run()
    out, flags = dp.results()
    sure = margin >= 1e-3
    np.testing.assert_array_equal(flags[sure], ref_flags[sure])
    compare(prob, out, np.where(sure, flags, ref_flags), ref=(ref_out, ref_flags))
    # a second call on the same workspace gives the same bits
    dp.run()
    out2, flags2 = dp.results()
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(flags2, flags)


@pytest.mark.parametrize("i", range(NCASES))
def test_random_shape_balanced_shares(i):
    # the same random cases through balanced shares, where the family has
    # them (grouped bf16 queries over a bf16 or E4M3FN cache): pieces cut at
    # the segments' edges (chunk_size 0) and, for a chunk size on the 64-token
    # grid, whole chunks
    import split_kv_asynchronous_amd as fd
    kw = draw_case(i)
    g = kw["num_q_heads"] // kw["num_kv_heads"]
    if g == 1 or kw["q_dtype"] != "bf16" or kw["kv_dtype"] == "f32":
        pytest.skip("no balanced shares for this family")
    prob = synthetic.make_problem(**kw)
    ref_out, ref_flags, margin = oracle.decode_exact(**prob.args())
    sure = margin >= 1e-3
    chunk = prob.chunk_size
    for c in (0, chunk) if chunk % 64 == 0 else (0,):
        prob.chunk_size = c
        print("case %d shares chunk %d" % (i, c), flush=True)
        dp = DeviceProblem(prob, plan=fd.FD_PLAN_SHARES)
        assert fd.fd_attn_plan(dp.desc())["shares"] > 0
        dp.run()
        out, flags = dp.results()
        np.testing.assert_array_equal(flags[sure], ref_flags[sure])
        compare(prob, out, np.where(sure, flags, ref_flags), ref=(ref_out, ref_flags))
    prob.chunk_size = chunk


@pytest.mark.parametrize("i", range(NCASES))
def test_random_shape_library_plan(i):
    # the same random cases under the library's own plan (chunk_size 0): the
    # plan table refined by the call's size (smaller chunks for small calls,
    # balanced shares only with enough work per share)
    import split_kv_asynchronous_amd as fd
    kw = dict(draw_case(i), chunk_size=0)
    prob = synthetic.make_problem(**kw)
    ref_out, ref_flags, margin = oracle.decode_exact(**prob.args())
    sure = margin >= 1e-3
    dp = DeviceProblem(prob)
    plan = fd.fd_attn_plan(dp.desc())
    print("case %d library plan %s" % (i, plan), flush=True)
    assert plan["shares"] > 0 or plan["chunk_size"] >= 256
    dp.run()
    out, flags = dp.results()
    np.testing.assert_array_equal(flags[sure], ref_flags[sure])
    compare(prob, out, np.where(sure, flags, ref_flags), ref=(ref_out, ref_flags))
