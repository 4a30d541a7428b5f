"""Decode calls running concurrently on separate streams (include/fd_attn.h:
calls may overlap on different streams when each has its own workspace and
outputs).

Four calls of different kernel families and plans -- grouped bf16 merged in
the chunk launch, paged E4M3FN with a narrow band (rows recompute chunks),
one query per KV head with a merge launch, and balanced shares -- each on a
stream of its own (default priority), enqueued in turn several times with no
synchronisation between them.  Every call's output, flags and recomputed-pair
count must be bit-identical to the same call run alone on one stream."""
import numpy as np
import pytest
import torch

import synthetic
from gpu_device import DeviceProblem

pytestmark = pytest.mark.gpu


def _problems():
    rng = np.random.default_rng(0x5EED7000)
    yield dict(batch=8, num_q_heads=64, num_kv_heads=8, seq_lens=rng.integers(1024, 8193, size=8),
               chunk_size=512, seed=71)
    yield dict(batch=16, num_q_heads=32, num_kv_heads=8, seq_lens=rng.integers(512, 4097, size=16),
               kv_dtype="e4m3fn", page_size=16, chunk_size=256, seed=72, a=3.0, b=2.0, phi=1.0)
    yield dict(batch=4, num_q_heads=32, num_kv_heads=32, seq_lens=rng.integers(2048, 8193, size=4),
               chunk_size=512, seed=73)
    yield dict(batch=32, num_q_heads=64, num_kv_heads=8, seq_lens=rng.integers(1024, 16385, size=32),
               chunk_size=0, seed=74)


def _state(dp):
    out, flags = dp.results()
    return out.copy(), flags.copy(), dp.recomputed()


def test_calls_on_separate_streams_match_their_serial_results():
    dps = [DeviceProblem(synthetic.make_problem(**kw)) for kw in _problems()]
    print("concurrency: %d calls, plans %s" % (len(dps), [d.desc().chunk_size for d in dps]), flush=True)
    # each call alone, on the current stream
    want = []
    for dp in dps:
        dp.run()
        want.append(_state(dp))
    assert any(w[2] > 0 for w in want), "the narrow-band call recomputes chunks"
    # all of them together: one stream each, enqueued in turn, five rounds
    streams = [torch.cuda.Stream() for _ in dps]
    torch.cuda.synchronize()
    for _ in range(5):
        for dp, s in zip(dps, streams):
            with torch.cuda.stream(s):
                dp.out.fill_(float("nan"))     # on the call's own stream, before it
            dp.run(stream=s.cuda_stream)
    torch.cuda.synchronize()
    for i, (dp, (out, flags, rec)) in enumerate(zip(dps, want)):
        got_out, got_flags, got_rec = _state(dp)
        np.testing.assert_array_equal(got_out, out, err_msg="call %d" % i)
        np.testing.assert_array_equal(got_flags, flags, err_msg="call %d" % i)
        assert got_rec == rec, (i, got_rec, rec)
