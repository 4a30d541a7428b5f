"""GPU parity at the size limits the C ABI accepts (include/fd_attn.h,
include/fd_gemm.h), against the float64 oracle on sampled outputs.

Each case sits at or near a limit where a 32-bit index would wrap:
  * the longest sequence (2^23 tokens, one KV head: a 4 GiB K/V slice whose
    last row starts 2^31 - 256 bytes into its buffer);
  * a batch of 2048 sequences x 32 heads x 512 chunks whose per-chunk
    partials reach float index 2^32 - 1 (17 GB of workspace), the sequences
    sharing the pages of a small pool so the cache stays small;
  * the largest batch (65535 sequences, ragged and empty, paged);
  * the flat GEMM at its largest M x N (an output of 2^32 elements) and its
    longest K (2^20).
Bars as in the other parity tests: flags bit-exact, max|err| <= 2e-3 x
max|out| (bf16/E4M3FN caches); GEMM entries within the fp32 summation bound.
"""
import numpy as np
import pytest
import torch

import oracle
import split_kv_asynchronous_amd as fd
import synthetic
from gpu_device import to_device
from gpu_helpers import DeviceProblem, compare

pytestmark = pytest.mark.gpu


def _sample_rows(n, seed, extra=()):
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in rng.choice(n, size=min(n, 96), replace=False))
    rows.update(r for r in (0, 1, n // 2, n - 2, n - 1, *extra) if 0 <= r < n)
    return np.array(sorted(rows), dtype=np.int32)


def _check_decode(prob, rows):
    dp = DeviceProblem(prob)
    print("workspace %.2f GB" % (dp.workspace.numel() / 1e9), flush=True)
    dp.run()
    out, flags = dp.results()
    assert np.isfinite(out).all()
    assert flags.sum() == 0 and dp.recomputed() == 0
    rel, _, _ = compare(prob, out, flags, rows=rows)
    print("sampled %d rows, rel err %.3e" % (rows.size, rel), flush=True)
    del dp
    torch.cuda.empty_cache()


def test_longest_sequence():
    print("case longest sequence: 2^23 tokens, group 8, bf16, library chunk", flush=True)
    prob = synthetic.make_long_sequence(1 << 23, num_q_heads=8, num_kv_heads=1, chunk_size=0)
    _check_decode(prob, np.arange(8, dtype=np.int32))


@pytest.mark.parametrize("kv", ["bf16", "e4m3fn"])
def test_partials_past_32bit_index(kv):
    print("case shared pages: batch 2048 x 32/8 heads, 16384 tokens, chunk 32, %s" % kv,
          flush=True)
    base = synthetic.make_problem(batch=4, num_q_heads=32, num_kv_heads=8, seq_lens=16384,
                                  kv_dtype=kv, page_size=16, chunk_size=32,
                                  a=16.0 if kv == "e4m3fn" else 20.0,
                                  seed=synthetic.SEED_BASE + 0x41)
    prob = synthetic.share_pages(base, 2048, seed=synthetic.SEED_BASE + 0x42)
    n = prob.batch * prob.num_q_heads
    # partial slot (b * 512 + c) * 32 + h holds floats 128 slot .. +127: from
    # b = 1024 on past index 2^31, the last row's up to 2^32 - 1
    _check_decode(prob, _sample_rows(n, 7, extra=(1024 * 32, 1024 * 32 + 31, n - 32)))


@pytest.mark.parametrize("g,kv", [(1, "bf16"), (8, "bf16"), (4, "e4m3fn")])
def test_largest_batch(g, kv):
    print("case batch 65535, group %d, %s, paged" % (g, kv), flush=True)
    # 61 ragged sequences (some empty) shared round-robin by the whole batch
    lens = np.random.default_rng(11).integers(0, 100, size=61, endpoint=True)
    lens[[3, 40]] = 0
    base = synthetic.make_problem(batch=61, num_q_heads=g, num_kv_heads=1, seq_lens=lens,
                                  kv_dtype=kv, page_size=16, chunk_size=32,
                                  seed=synthetic.SEED_BASE + 0x43 + g)
    prob = synthetic.share_pages(base, 65535, seed=synthetic.SEED_BASE + 0x45 + g)
    n = prob.batch * prob.num_q_heads
    _check_decode(prob, _sample_rows(n, 13, extra=range(n - 64, n)))


def _gemm_bound(a, w, k):
    u = 2.0 ** -24
    return 2 * k * u / (1 - k * u) * oracle.flat_gemm_abs(a, w) + 1e-30


@pytest.mark.parametrize("m,n,k", [(4096, 1 << 20, 32), (3, 16, 1 << 20), (4096, 64, 512)])
def test_gemm_limits(m, n, k):
    print("case gemm limits m=%d n=%d k=%d" % (m, n, k), flush=True)
    a, w = synthetic.make_gemm(m, n, k, seed=synthetic.SEED_BASE + 0x44)
    A, W = to_device(a, "bf16"), to_device(w, "bf16")
    c = fd.fd_flat_gemm(A, W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([rng.choice(m, size=min(m, 24), replace=False), [0, m - 1]]))
    cols = np.unique(np.concatenate([rng.choice(n, size=min(n, 1024), replace=False), [0, n - 1]]))
    got = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
    got = got.float().cpu().numpy().astype(np.float64)
    ref = oracle.flat_gemm(a[rows], w[cols])
    err = np.abs(got - ref)
    bound = _gemm_bound(a[rows], w[cols], k)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), (rows[worst[0]], cols[worst[1]], err[worst], bound[worst])
    del c
    torch.cuda.empty_cache()
