"""GPU parity of causal prefill on seeded random shapes, through the C ABI.

Each case draws a batch, a query-head group over 1-2 KV heads, a query block
length, per-sequence key lengths (a cached prefix before the block, a sequence
shorter than the block, or an empty one), either a wide band (no visible
score leaves it) or a narrow one (rows switch to online softmax part-way), and
a cache format (bf16 or E4M3FN) and layout (contiguous or pages of 16-128).
Bar as in the other prefill tests: max|gpu - oracle| <= 2e-3 * max|oracle|,
and every output element within the bound the kernel's arithmetic allows
(weights carried as a bf16 pair to a relative 2^-18, fp32 accumulation);
flags bit-exact on every row whose visible scores all lie at least 1e-3 from
both band edges (a row with a score closer than that may take either path).
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_device import DevicePrefill
from test_gpu_prefill import TOL, _bound

pytestmark = pytest.mark.gpu

NCASES = 24


def draw_case(i):
    """Shape and band of case i (a pure function of i)."""
    rng = np.random.default_rng(0x5EED4000 + i)
    hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 2, 4, 8]))
    batch = int(rng.integers(1, 4))
    q_len = int(rng.integers(1, 401))
    kv = q_len + rng.integers(-q_len // 2, 301, size=batch)
    kv[rng.random(batch) < 0.15] = 0
    kv = np.maximum(kv, 0).astype(np.int32)
    if rng.random() < 0.5:
        phi, a, b = float(rng.uniform(2.0, 5.0)), 20.0, 6.0
    else:
        phi, a, b = float(rng.uniform(-0.5, 1.5)), float(rng.uniform(1.5, 4.0)), float(rng.uniform(1.0, 3.0))
    # cache format and layout from a stream of their own (the shapes above
    # stay what they were without them)
    fmt = np.random.default_rng(0x5EED4100 + i)
    kv_dtype = str(fmt.choice(["bf16", "e4m3fn"]))
    page = int(fmt.choice([0, 0, 16, 32, 128]))
    return dict(batch=batch, num_q_heads=g * hkv, num_kv_heads=hkv, q_len=q_len, kv_lens=kv,
                phi=phi, a=a, b=b, seed=0x5EED5000 + i, kv_dtype=kv_dtype, page_size=page,
                extra_pages=int(fmt.integers(0, 4)) if page else 0)


@pytest.mark.parametrize("i", range(NCASES))
def test_prefill_random_shape(i):
    kw = draw_case(i)
    print("case prefill %d: %s" % (i, {k: (v.tolist() if isinstance(v, np.ndarray) else v)
                                       for k, v in kw.items()}), flush=True)
    prob = synthetic.make_prefill(**kw)
    ref, ref_flags, margin = oracle.prefill_exact(**prob.args())
    dp = DevicePrefill(prob)
    dp.run()
    out, flags = dp.results()
    sure = margin >= 1e-3
    np.testing.assert_array_equal(flags[sure], ref_flags[sure])
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = float(np.abs(out - ref).max())
    assert err <= TOL * scale, "max|err| %.3e > %.0e * max|out| (%.3e)" % (err, TOL, scale)
    bound = _bound(prob)
    assert err <= bound, "max|err| %.3e > arithmetic bound %.3e" % (err, bound)
