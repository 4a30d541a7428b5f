"""GPU parity: the HIP library against the float64 oracle, through the C ABI.

Bar: flags bit-exact; max|gpu - oracle| <= tol * max|oracle| with tol = 2e-3
for bf16/fp8 caches and 1e-5 for fp32 caches (float64 oracle, fp32 GPU
accumulation).  Inputs keep every score at least 1e-3 from both band edges
(checked by the oracle), so the flag decision does not depend on precision.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import DeviceProblem, compare

pytestmark = pytest.mark.gpu

SMALL = [
    # (config, shrink) -- several chunks, ragged tails, every code path
    (1, dict(length=1000)),
    (2, dict(batch=2, length=3000)),
    (3, dict(batch=3, lens=(1, 5000))),
    (4, dict(length=9000)),
    (5, dict(batch=5, lens=(1, 3000))),
]


@pytest.mark.parametrize("cfg,kw", SMALL, ids=["cfg%d" % c for c, _ in SMALL])
def test_small_configs(cfg, kw):
    prob = synthetic.make_config(cfg, **kw)
    print("case cfg%d %s lens=%s" % (cfg, kw, prob.seq_lens.tolist()), flush=True)
    dp = DeviceProblem(prob)
    dp.run()
    out, flags = dp.results()
    rel, _, _ = compare(prob, out, flags)
    print("rel err %.3e" % rel)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_configs(cfg):
    print("case full cfg%d" % cfg, flush=True)
    prob = synthetic.make_config(cfg)
    dp = DeviceProblem(prob)
    dp.run()
    out, flags = dp.results()
    rel, ref_out, ref_flags = compare(prob, out, flags)
    if cfg == 4:
        heads = sorted(set(int(h) for h in prob.perturbed[:, 0]))
        assert np.nonzero(flags)[0].tolist() == heads
        assert dp.recomputed() == len(prob.perturbed) == 41
    else:
        assert flags.sum() == 0 and dp.recomputed() == 0
    # a second call gives the same bits
    out1 = dp.out.clone()
    dp.run()
    torch.cuda.synchronize()
    assert torch.equal(out1, dp.out)
    print("cfg%d rel err %.3e flagged %d" % (cfg, rel, int(flags.sum())))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_configs_library_plan(cfg):
    # the same workloads with chunk_size 0, as the bench times them beside
    # the stated chunk: the library's own plan (balanced shares on some)
    import split_kv_asynchronous_amd as fd
    prob = synthetic.make_config(cfg)
    prob.chunk_size = 0
    dp = DeviceProblem(prob)
    plan = fd.fd_attn_plan(dp.desc())
    print("case full cfg%d library plan %s" % (cfg, plan), flush=True)
    dp.run()
    out, flags = dp.results()
    rel, _, _ = compare(prob, out, flags)
    if cfg == 4:
        # one recomputed pair per chunk that holds a perturbed key
        heads = sorted(set(int(h) for h in prob.perturbed[:, 0]))
        assert np.nonzero(flags)[0].tolist() == heads
        assert 0 < dp.recomputed() <= len(prob.perturbed)
    else:
        assert flags.sum() == 0 and dp.recomputed() == 0
    out1 = dp.out.clone()
    dp.run()
    torch.cuda.synchronize()
    assert torch.equal(out1, dp.out)
    print("cfg%d library plan rel err %.3e" % (cfg, rel))


GQA_CASES = [
    # group, kv dtype, page size, chunk, lens
    (2, "bf16", 0, 64, [1, 31, 32, 33, 200]),
    (4, "bf16", 16, 128, [17, 500, 1023]),
    (6, "bf16", 0, 96, [700, 95]),
    (8, "e4m3fn", 0, 256, [1000, 1, 257]),
    (16, "bf16", 32, 64, [300, 129]),
    (32, "e4m3fn", 64, 128, [640, 1]),
    (4, "f32", 0, 64, [333, 64]),
]


@pytest.mark.parametrize("g,kv,page,chunk,lens", GQA_CASES)
def test_group_sizes_layouts_dtypes(g, kv, page, chunk, lens):
    print("case g=%d kv=%s page=%d chunk=%d lens=%s" % (g, kv, page, chunk, lens), flush=True)
    hkv = 2
    prob = synthetic.make_problem(batch=len(lens), num_q_heads=g * hkv, num_kv_heads=hkv,
                                  seq_lens=lens, kv_dtype=kv, q_dtype="bf16", page_size=page,
                                  chunk_size=chunk, seed=100 + g)
    dp = DeviceProblem(prob)
    dp.run()
    compare(prob, *dp.results())


def test_fp32_query_with_bf16_cache_and_bf16_output():
    prob = synthetic.make_problem(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[900, 77],
                                  q_dtype="f32", kv_dtype="bf16", chunk_size=128, seed=7)
    dp = DeviceProblem(prob, out_dtype="bf16")
    dp.run()
    out, flags = dp.results()
    compare(prob, out, flags, tol=6e-3)   # bf16 output adds up to 2^-9 relative rounding


def test_zero_and_clamped_lengths():
    prob = synthetic.make_problem(batch=4, num_q_heads=8, num_kv_heads=2, seq_lens=[0, 5, 64, 300],
                                  chunk_size=64, max_seq_len=300, seed=8)
    prob.seq_lens = np.array([0, 5, 64, 999], dtype=np.int32)   # 999 is clamped to 300
    dp = DeviceProblem(prob)
    dp.run()
    out, flags = dp.results()
    assert np.all(out[:8] == 0) and np.all(flags[:8] == 0)
    compare(prob, out, flags)


@pytest.mark.parametrize("g,kv,page", [(1, "bf16", 0), (4, "bf16", 0), (4, "e4m3fn", 16),
                                       (1, "f32", 0)])
def test_empty_sequences_in_every_kernel(g, kv, page):
    # an empty sequence has no chunk, yet its rows must still be written (zeros)
    prob = synthetic.make_problem(batch=4, num_q_heads=2 * g, num_kv_heads=2,
                                  seq_lens=[0, 300, 0, 37], kv_dtype=kv, page_size=page,
                                  chunk_size=64, max_seq_len=320, seed=9 + g)
    print("case empty g=%d kv=%s page=%d" % (g, kv, page), flush=True)
    dp = DeviceProblem(prob)
    dp.out.fill_(float("nan"))
    dp.flags.fill_(7)
    dp.run()
    out, flags = dp.results()
    rows = out.reshape(prob.batch, prob.num_q_heads, -1)
    assert np.all(rows[0] == 0) and np.all(rows[2] == 0)
    compare(prob, out, flags)


def test_workspace_needs_no_initialisation():
    # The per-row-group counters carry the epoch of the call that wrote them, so
    # any workspace contents work, a workspace can move between problems, and
    # every call reports its own recomputed-chunk count.
    narrow = synthetic.make_problem(batch=3, num_q_heads=8, num_kv_heads=2,
                                    seq_lens=[2000, 700, 1500], chunk_size=256, seed=41,
                                    phi=1.0, a=3.0, b=1.5)
    wide = synthetic.make_problem(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[900, 2100],
                                  chunk_size=128, seed=42)
    ref_out, ref_flags, margin = oracle.decode_exact(**narrow.args())
    sure = margin >= 1e-3     # rows whose flag cannot depend on rounding
    dn, dw = DeviceProblem(narrow), DeviceProblem(wide)
    ws = dn.workspace if dn.workspace.numel() >= dw.workspace.numel() else dw.workspace
    dn.workspace = dw.workspace = ws
    gen = torch.Generator(device="cpu").manual_seed(5)
    fills = [lambda: ws.fill_(0xFF), lambda: ws.fill_(0),
             lambda: ws.copy_(torch.randint(0, 256, (ws.numel(),), generator=gen,
                                            dtype=torch.uint8).cuda())]
    counts = []
    for fill in fills:
        fill()
        for _ in range(2):
            dn.run()
            out, flags = dn.results()
            np.testing.assert_array_equal(flags[sure], ref_flags[sure])
            compare(narrow, out, np.where(sure, flags, ref_flags), ref=(ref_out, ref_flags))
            counts.append(dn.recomputed())
        dw.run()
        out, flags = dw.results()
        compare(wide, out, flags)
        assert dw.recomputed() == 0
    # the same (deterministic) count on every call, whatever the workspace held
    assert counts[0] > 0 and len(set(counts)) == 1, counts


@pytest.mark.parametrize("g,kv,page", [(1, "bf16", 0), (8, "bf16", 0), (4, "e4m3fn", 16),
                                       (1, "f32", 0), (1, "e4m3fn", 16)])
def test_out_of_band_rows_fall_back(g, kv, page):
    hkv = 2
    prob = synthetic.make_problem(batch=3, num_q_heads=g * hkv, num_kv_heads=hkv,
                                  seq_lens=[2000, 700, 1500], kv_dtype=kv, page_size=page,
                                  chunk_size=256, seed=30 + g, phi=1.0, a=3.0, b=1.5)
    print("case fallback g=%d kv=%s page=%d" % (g, kv, page), flush=True)
    # narrow band [-2, 2.5]: many scores leave it, so most rows are recomputed in part
    ref_out, ref_flags, margin = oracle.decode_exact(**prob.args())
    assert ref_flags.sum() > 0
    dp = DeviceProblem(prob)
    dp.run()
    out, flags = dp.results()
    # a row with a score within 1e-3 of an edge may take either path; its output
    # is the exact softmax either way, only its flag is left unchecked
    sure = margin >= 1e-3
    assert sure.any()
    np.testing.assert_array_equal(flags[sure], ref_flags[sure])
    compare(prob, out, np.where(sure, flags, ref_flags), ref=(ref_out, ref_flags))
    assert dp.recomputed() > 0


def test_nan_query_row_is_flagged_and_nan():
    prob = synthetic.make_problem(batch=2, num_q_heads=4, num_kv_heads=1, seq_lens=[300, 300],
                                  chunk_size=64, seed=9)
    prob.q[1, 2, 5] = 0x7FC0    # bf16 NaN
    dp = DeviceProblem(prob)
    dp.run()
    out, flags = dp.results()
    assert flags.tolist() == [0, 0, 0, 0, 0, 0, 1, 0]
    assert np.isnan(out[6]).all() and np.isfinite(np.delete(out, 6, axis=0)).all()
    compare(prob, out, flags)


def test_paged_equals_contiguous_bitwise():
    lens = [1, 16, 17, 999]
    pg = synthetic.make_problem(batch=4, num_q_heads=16, num_kv_heads=4, seq_lens=lens,
                                kv_dtype="bf16", page_size=16, chunk_size=64, seed=12,
                                max_seq_len=1008)
    ct = synthetic.make_problem(batch=4, num_q_heads=16, num_kv_heads=4, seq_lens=lens,
                                kv_dtype="bf16", chunk_size=64, seed=12, max_seq_len=1008)
    np.testing.assert_array_equal(ct.q, pg.q)
    outs = []
    for p in (pg, ct):
        dp = DeviceProblem(p)
        dp.run()
        outs.append(dp.results())
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_chunk_size_and_phi_do_not_change_the_result():
    base = synthetic.make_config(3, batch=2, lens=(3000, 9000))
    ref_out, ref_flags, _ = oracle.decode_exact(**base.args())
    for chunk in (32, 256, 2048, 0):          # 0: the library's pick
        for phi in (0.0, 4.0, 7.0):
            base.chunk_size = chunk
            dp = DeviceProblem(base)
            dp.run(phi=phi)
            compare(base, *dp.results(), ref=(ref_out, ref_flags))


@pytest.mark.parametrize("cfg", [2, 5])
def test_library_chunk_pick(cfg):
    # chunk_size 0 on the MHA vector kernel and the paged fp8 kernel
    prob = synthetic.make_config(cfg, batch=3, lens=(100, 4000))
    prob.chunk_size = 0
    print("case chunk pick cfg%d" % cfg, flush=True)
    dp = DeviceProblem(prob)
    dp.run()
    compare(prob, *dp.results())


def test_prepared_call_equals_direct_call():
    # a DecodeCall marshalled once gives the bits of a direct call, also with
    # the band changed per call (a band that flags every row, then the original)
    import split_kv_asynchronous_amd as fd
    prob = synthetic.make_config(5, batch=3, lens=(100, 4000))
    print("case prepared call", flush=True)
    dp = DeviceProblem(prob)
    direct = []
    for phi, b in ((prob.phi, prob.b), (-30.0, 0.0), (prob.phi, prob.b)):
        o, f = fd.fd_attn_decode(dp.q, dp.k, dp.v, dp.seq_lens, dp.block_table, phi, prob.a, b,
                                 chunk_size=prob.chunk_size, max_seq_len=prob.max_seq_len,
                                 num_kv_heads=prob.num_kv_heads, page_size=prob.page_size,
                                 scale=prob.scale, k_scale=dp.k_scale, v_scale=dp.v_scale)
        direct.append((o.clone(), f.clone()))
        dp.run(phi=phi, b=b)
        torch.cuda.synchronize()
        assert torch.equal(dp.out, direct[-1][0]) and torch.equal(dp.flags, direct[-1][1])
    valid = torch.from_numpy(prob.seq_lens > 0).cuda()
    assert torch.equal(direct[1][1].bool(), valid[:, None].expand(-1, prob.num_q_heads))
    assert not bool(direct[0][1].any())


SHAPE_CASES = [
    # group, kv dtype, page size, kernel shapes of the family
    (8, "bf16", 0, 3),
    (4, "bf16", 16, 3),
    (4, "e4m3fn", 16, 3),
    (8, "e4m3fn", 0, 3),
    (1, "bf16", 0, 1),
    (1, "e4m3fn", 32, 1),
]


@pytest.mark.parametrize("g,kv,page,nshapes", SHAPE_CASES)
def test_every_kernel_shape_and_merge_placement(g, kv, page, nshapes):
    # every shape of the family with the merge forced into the chunk launch
    # and into a second launch; a narrow band sends chunks to the recompute
    import split_kv_asynchronous_amd as fd
    prob = synthetic.make_problem(batch=3, num_q_heads=2 * g, num_kv_heads=2, seq_lens=[1000, 37, 2200],
                                  kv_dtype=kv, page_size=page, chunk_size=256, phi=1.0, a=3.0, b=1.5,
                                  seed=900 + g)
    ref_out, ref_flags, margin = oracle.decode_exact(**prob.args())
    sure = margin >= 1e-3
    for shape in range(nshapes):
        for place in (fd.FD_PLAN_FUSED, fd.FD_PLAN_SPLIT):
            plan = fd.FD_PLAN_SHAPE(shape) | place
            print("case g=%d kv=%s page=%d shape=%d %s" % (g, kv, page, shape,
                                                           "fused" if place == fd.FD_PLAN_FUSED else "split"),
                  flush=True)
            dp = DeviceProblem(prob, plan=plan)
            got = fd.fd_attn_plan(dp.desc())
            assert got["shape"] == shape and got["fused"] == (place == fd.FD_PLAN_FUSED)
            dp.run()
            out, flags = dp.results()
            np.testing.assert_array_equal(flags[sure], ref_flags[sure])
            compare(prob, out, np.where(sure, flags, ref_flags), ref=(ref_out, ref_flags))
            assert dp.recomputed() > 0


ONE_CHUNK_CASES = [
    # group, kv dtype, page size, kernel shape, output dtype
    (8, "bf16", 0, 0, "f32"), (8, "bf16", 16, 2, "bf16"), (4, "bf16", 0, 1, "f32"),
    (4, "e4m3fn", 16, 0, "f32"), (8, "e4m3fn", 0, 2, "bf16"), (16, "e4m3fn", 32, 1, "f32"),
    (1, "bf16", 0, 0, "f32"), (1, "e4m3fn", 16, 0, "bf16"), (1, "f32", 32, 0, "f32"),
]


@pytest.mark.parametrize("g,kv,page,shape,out_dtype", ONE_CHUNK_CASES)
def test_one_chunk_rows_written_by_the_chunk_kernel(g, kv, page, shape, out_dtype):
    # Every sequence fits in one chunk (some empty): with the merge in the
    # chunk launch the chunk kernel writes those rows itself, in the merge's
    # arithmetic, so outputs, flags and the recomputed count equal the
    # two-launch call's bit for bit; a narrow band sends some chunks to the
    # recompute.
    import split_kv_asynchronous_amd as fd
    lens = [0, 1, 17, 200, 511, 512, 300, 64] * 40
    prob = synthetic.make_problem(batch=len(lens), num_q_heads=2 * g, num_kv_heads=2, seq_lens=lens,
                                  kv_dtype=kv, q_dtype="f32" if kv == "f32" else "bf16", page_size=page,
                                  chunk_size=512, phi=1.0, a=3.0, b=1.5, seed=1200 + g)
    res = {}
    for place in (fd.FD_PLAN_FUSED, fd.FD_PLAN_SPLIT):
        print("case one-chunk g=%d kv=%s page=%d shape=%d out=%s place=%d" % (g, kv, page, shape, out_dtype, place),
              flush=True)
        dp = DeviceProblem(prob, out_dtype=out_dtype, plan=fd.FD_PLAN_SHAPE(shape) | place)
        dp.run()
        dp.run()                     # a second call on the same workspace (a new epoch)
        res[place] = (dp.out.clone(), dp.flags.clone(), dp.recomputed())
        if place == fd.FD_PLAN_FUSED and out_dtype == "f32":
            out, flags = dp.results()
            ref_out, ref_flags, margin = oracle.decode_exact(**prob.args())
            sure = margin >= 1e-3
            np.testing.assert_array_equal(flags[sure], ref_flags[sure])
            compare(prob, out, np.where(sure, flags, ref_flags), ref=(ref_out, ref_flags))
    fo, ff, fc = res[fd.FD_PLAN_FUSED]
    so, sf, sc = res[fd.FD_PLAN_SPLIT]
    assert torch.equal(fo, so) and torch.equal(ff, sf)
    assert fc == sc and fc > 0
    # the library's own plan: a chunk that covers max_seq_len merges in the
    # launch; against the two-launch call of the same kernel shape
    dp = DeviceProblem(prob, out_dtype=out_dtype)
    plan = fd.fd_attn_plan(dp.desc())
    assert plan["fused"] == 1
    dp.run()
    sp = DeviceProblem(prob, out_dtype=out_dtype, plan=fd.FD_PLAN_SHAPE(plan["shape"]) | fd.FD_PLAN_SPLIT)
    sp.run()
    assert torch.equal(dp.out, sp.out) and torch.equal(dp.flags, sp.flags)
    assert dp.recomputed() == sp.recomputed() == fc


TABLE_CASES = [
    # one call per row of the plan table (chunk_size = 0): group, kv dtype,
    # page size, sequence lengths, max_seq_len (selects the row)
    (8, "bf16", 0, [2000, 1], 2048), (8, "bf16", 0, [5000, 300], 8192),
    (8, "bf16", 0, [20000, 9000], 32768), (8, "bf16", 0, [35000, 777], 40000),
    (4, "bf16", 16, [2048, 100], 2048), (4, "bf16", 16, [6000, 31], 8192),
    (4, "bf16", 16, [30000, 0], 32768), (4, "bf16", 16, [34000, 2000], 36000),
    (4, "e4m3fn", 0, [1500, 2048], 2048), (4, "e4m3fn", 0, [16000, 9], 16384),
    (4, "e4m3fn", 0, [20000, 1], 24000),
    (8, "e4m3fn", 16, [777, 2048], 2048), (8, "e4m3fn", 16, [12000, 4000], 16384),
    (8, "e4m3fn", 16, [17000, 0], 20000),
    (1, "bf16", 0, [2048, 1000], 2048), (1, "bf16", 0, [8000, 3], 8192),
    (1, "bf16", 0, [9000, 12000], 12000),
    (1, "bf16", 16, [1024, 2000], 2048), (1, "bf16", 16, [7000, 0], 8192),
    (1, "f32", 16, [10000, 64], 10000),
]


@pytest.mark.parametrize("g,kv,page,lens,cap", TABLE_CASES)
def test_plan_table_rows(g, kv, page, lens, cap):
    import split_kv_asynchronous_amd as fd
    prob = synthetic.make_problem(batch=len(lens), num_q_heads=2 * g, num_kv_heads=2, seq_lens=lens,
                                  kv_dtype=kv, q_dtype="f32" if kv == "f32" else "bf16", page_size=page,
                                  chunk_size=0, max_seq_len=cap, seed=950 + g)
    dp = DeviceProblem(prob)
    plan = fd.fd_attn_plan(dp.desc())
    print("case table g=%d kv=%s page=%d cap=%d -> %s" % (g, kv, page, cap, plan), flush=True)
    dp.run()
    compare(prob, *dp.results())


@pytest.mark.parametrize("chunk,cap,fused,planned", [(0, 1024, 1, 1024), (0, 4096, 1, 0), (512, 1024, 0, 512),
                                                     (2048, 1024, 1, 2048)])
@pytest.mark.parametrize("kv", ["bf16", "e4m3fn"])
def test_serving_batch_runs_balanced_shares(kv, chunk, cap, fused, planned):
    # a serving batch (8192 sequences x 2 KV heads = 16384 row groups): the
    # library picks balanced shares -- for chunk_size 0 whole chunks covering
    # every row when max_seq_len is at most 2K, pieces beyond; whole chunks of
    # a stated size otherwise (merged by a second launch unless a chunk
    # covers max_seq_len)
    # (E4M3FN: 2048 sequences x 8 KV heads of 4 query heads, also 16384 row
    # groups; shares for its 4K rows take the table's shape 0)
    import split_kv_asynchronous_amd as fd
    if kv == "bf16":
        lens = np.random.default_rng(17).integers(0, 750, size=8192)
        prob = synthetic.make_problem(batch=8192, num_q_heads=8, num_kv_heads=2, seq_lens=lens, chunk_size=chunk,
                                      max_seq_len=cap, page_size=16, seed=1717)
    else:
        lens = np.random.default_rng(18).integers(0, 750, size=2048)
        prob = synthetic.make_problem(batch=2048, num_q_heads=32, num_kv_heads=8, seq_lens=lens, chunk_size=chunk,
                                      max_seq_len=cap, page_size=16, kv_dtype="e4m3fn", seed=1818)
    dp = DeviceProblem(prob)
    plan = fd.fd_attn_plan(dp.desc())
    print("case serving batch %s chunk %d cap %d -> %s" % (kv, chunk, cap, plan), flush=True)
    assert plan["shares"] > 0 and plan["fused"] == fused and plan["chunk_size"] == planned
    assert plan["shape"] == (0 if (kv, chunk, cap) == ("e4m3fn", 0, 4096) else 2)
    dp.run()
    compare(prob, *dp.results())


SHARE_CASES = [
    # id, group, kv dtype, page size, lens, kernel shape, output dtype, narrow band
    ("bf16-ragged", 8, "bf16", 0, [0, 1, 63, 64, 65, 1000, 5000, 20000], 0, "f32", False),
    ("bf16-paged-narrow", 4, "bf16", 16, [3000, 17, 0, 9000, 128], 0, "bf16", True),
    ("bf16-one-long-row", 8, "bf16", 0, [131072], 0, "f32", False),
    ("bf16-shape1-narrow", 8, "bf16", 0, [7000, 300, 12000], 1, "f32", True),
    ("bf16-shape2-paged", 16, "bf16", 32, [2500, 40, 6000, 1], 2, "bf16", False),
    ("e4m3fn-paged", 4, "e4m3fn", 16, [0, 5000, 700, 16384, 33], 0, "f32", False),
    ("e4m3fn-narrow", 8, "e4m3fn", 0, [9000, 64, 3000], 0, "f32", True),
    ("bf16-many-rows", 2, "bf16", 0, "many", 0, "f32", False),
    # calls of at least 4 quanta per share: a quarter of the quanta in claimed grains
    ("bf16-pool-narrow", 8, "bf16", 0, [40000, 30000, 50000, 2000], 0, "f32", True),
    ("e4m3fn-pool-paged", 4, "e4m3fn", 16, [30000, 5, 40000, 0, 25000], 0, "bf16", False),
    ("bf16-pool-shape2", 8, "bf16", 32, [60000, 45000, 70000], 2, "f32", False),
]


# units: pieces cut at the segments' edges (chunk_size 0), or whole chunks
# of 512 tokens merged in the launch or of 2048 tokens merged by a second launch
SHARE_UNITS = [(0, 0), (512, 0), (2048, 0x20)]


@pytest.mark.parametrize("chunk,place", SHARE_UNITS, ids=["pieces", "chunks512", "chunks2048-split"])
@pytest.mark.parametrize("name,g,kv,page,lens,shape,out_dtype,narrow", SHARE_CASES, ids=[c[0] for c in SHARE_CASES])
def test_balanced_shares(name, g, kv, page, lens, shape, out_dtype, narrow, chunk, place):
    # the persistent grid of equal shares and claimed grains: rows cut at
    # segment edges (a row group inside one segment is written directly, one
    # spread over many is merged from all its pieces) or whole chunks, empty
    # and short rows, more sequences than one 64-wide scan, and units
    # recomputed with online softmax
    import split_kv_asynchronous_amd as fd
    if lens == "many":
        lens = list(np.random.default_rng(5).integers(0, 300, size=700))
    hkv = 2
    band = dict(phi=1.0, a=3.0, b=1.5) if narrow else {}
    prob = synthetic.make_problem(batch=len(lens), num_q_heads=g * hkv, num_kv_heads=hkv, seq_lens=lens,
                                  kv_dtype=kv, page_size=page, chunk_size=chunk, seed=1300 + g, **band)
    print("case shares %s chunk %d place %d" % (name, chunk, place), flush=True)
    dp = DeviceProblem(prob, out_dtype=out_dtype, plan=fd.FD_PLAN_SHARES | fd.FD_PLAN_SHAPE(shape) | place)
    plan = fd.fd_attn_plan(dp.desc())
    assert plan["shares"] > 0 and plan["fused"] == (place == 0) and plan["shape"] == shape
    assert plan["chunk_size"] == chunk
    dp.run()
    out, flags = dp.results()
    ref_out, ref_flags, margin = oracle.decode_exact(**prob.args())
    sure = margin >= 1e-3
    np.testing.assert_array_equal(flags[sure], ref_flags[sure])
    tol = None if out_dtype == "f32" else 6e-3     # bf16 output adds up to 2^-9 relative rounding
    compare(prob, out, np.where(sure, flags, ref_flags), ref=(ref_out, ref_flags), tol=tol)
    if narrow:
        assert dp.recomputed() > 0
    # a second call on the same workspace (a new epoch) gives the same bits
    first = dp.out.clone(), dp.flags.clone()
    dp.out.fill_(float("nan"))
    dp.run()
    torch.cuda.synchronize()
    assert torch.equal(dp.out, first[0]) and torch.equal(dp.flags, first[1])
