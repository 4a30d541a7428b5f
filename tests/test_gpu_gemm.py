"""GPU parity of the flat GEMM (fd_flat_gemm, C = A . W^T of the decode linear
layers) against the float64 oracle.

Bar: every output within the rounding bound of an fp32 sum of exact bf16
products, 2 * gamma(K) * (|A| . |W|^T) with gamma(K) = K u / (1 - K u),
u = 2^-24 (the factor 2 leaves room for the matrix cores' internal
accumulation order); bf16 outputs add one bf16 rounding, 2^-8 of |C|.  Small
shapes run every kernel variant and several K splits, with ragged M and N
(tails of the 16-row and 16-column blocks, m-groups past 64 rows); the 7B
block layers run at full size with the library's own pick.
"""
import numpy as np
import pytest
import torch

import oracle
import split_kv_asynchronous_amd as fd
import synthetic
from gpu_device import to_device

pytestmark = pytest.mark.gpu


def _bound(a, w, k, out_dtype, ref):
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    b = 2 * gamma * oracle.flat_gemm_abs(a, w)
    if out_dtype == "bf16":
        b = b + 2.0 ** -8 * (np.abs(ref) + b)
    return b + 1e-30


def _run(a, w, out_dtype="f32", **kw):
    A, W = to_device(a, "bf16"), to_device(w, "bf16")
    c = fd.fd_flat_gemm(A, W, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return c.float().cpu().numpy().astype(np.float64)


def _check(m, n, k, out_dtype="f32", seed=300, **kw):
    a, w = synthetic.make_gemm(m, n, k, seed=seed)
    print("case gemm m=%d n=%d k=%d %s %s" % (m, n, k, out_dtype, kw), flush=True)
    got = _run(a, w, out_dtype, **kw)
    ref = oracle.flat_gemm(a, w)
    err = np.abs(got - ref)
    bound = _bound(a, w, k, out_dtype, ref)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), (worst, err[worst], bound[worst])
    return got


SMALL = [(1, 16, 32), (5, 200, 96), (16, 64, 256), (17, 130, 512), (33, 48, 1024),
         (64, 272, 320), (100, 40, 256)]


@pytest.mark.parametrize("variant", range(1, 15))
@pytest.mark.parametrize("m,n,k", SMALL, ids=["%dx%dx%d" % s for s in SMALL])
def test_variants_small(variant, m, n, k):
    if variant in (13, 14) and (k % 128 or (variant == 13 and min(m, 64) > 48)):
        pytest.skip("DMA variants take K in whole 128-wide stages and need LDS room for A")
    for ks in (1, 3, 0):
        if ks <= k // 32:
            _check(m, n, k, variant=variant, ksplit=ks)


@pytest.mark.parametrize("variant", [13, 14])
@pytest.mark.parametrize("m", [1, 16, 40])
def test_dma_variants_7b_shapes(variant, m):
    # full-size O projection and a 2-slice down projection through the DMA rings
    if variant == 13 and m > 48:
        pytest.skip("no LDS room")
    _check(m, 4096, 4096, variant=variant, seed=350 + m)
    _check(m, 1024, 11008, variant=variant, ksplit=2, seed=360 + m)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_small_config_default_plan(out_dtype):
    cfg = synthetic.GEMM_CONFIGS[1]
    (_, n, k), = cfg["layers"]
    _check(cfg["m"], n, k, out_dtype)


@pytest.mark.parametrize("layer", range(4))
def test_7b_block_layers_full(layer):
    cfg = synthetic.GEMM_CONFIGS[2]
    name, n, k = cfg["layers"][layer]
    print("layer", name, fd.fd_flat_gemm_plan(cfg["m"], n, k), flush=True)
    _check(cfg["m"], n, k, "bf16" if layer % 2 else "f32", seed=synthetic.SEED_BASE + 200 + layer)


@pytest.mark.parametrize("m", [1, 4, 32, 64])
def test_7b_m_range(m):
    # the O projection over the decode batch sizes the plan table covers
    _check(m, 4096, 4096, seed=310 + m)


def test_repeatable_and_workspace_reuse():
    a, w = synthetic.make_gemm(16, 1024, 2048, seed=320)
    A, W = to_device(a, "bf16"), to_device(w, "bf16")
    ws = torch.empty(fd.fd_flat_gemm_workspace_size(16, 1024, 2048, ksplit=8), dtype=torch.uint8,
                     device="cuda")
    c1 = fd.fd_flat_gemm(A, W, ksplit=8, workspace=ws).clone()
    c2 = fd.fd_flat_gemm(A, W, ksplit=8, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


def test_zero_weights_and_one_hot_rows():
    # exact cases: zero weights give exact zeros; a one-hot row of W copies a column of A
    a, _ = synthetic.make_gemm(7, 16, 128, seed=330)
    w = np.zeros((48, 128), dtype=np.uint16)
    got = _run(a, w, ksplit=2)
    assert np.all(got == 0.0)
    w[5, 17] = 0x3F80          # 1.0 in bf16
    w[40, 127] = 0xC000        # -2.0
    got = _run(a, w, variant=6, ksplit=1)
    A = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(got[:, 5], A[:, 17])
    np.testing.assert_array_equal(got[:, 40], -2.0 * A[:, 127])


def test_graph_replays_match_eager():
    # a captured decode step (split K: partial-sum and reduce kernels) replayed
    # several times, with eager work and synchronisations in between, gives the
    # eager result every time
    shapes = [(16, 1024, 2048, 4), (3, 272, 320, 1)]
    dev = []
    for i, (m, n, k, ks) in enumerate(shapes):
        a, w = synthetic.make_gemm(m, n, k, seed=340 + i)
        A, W = to_device(a, "bf16"), to_device(w, "bf16")
        ws = torch.empty(max(fd.fd_flat_gemm_workspace_size(m, n, k, ksplit=ks), 256),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty((m, n), dtype=torch.float32, device="cuda")
        dev.append((A, W, ws, out, ks))
    # and a packed-weight call (the decode step's layout)
    a, w = synthetic.make_gemm(16, 4096, 1024, seed=345)
    Wp = fd.fd_flat_gemm_pack_weights(to_device(w, "bf16"))
    wsp = torch.empty(max(fd.fd_flat_gemm_workspace_size(16, 4096, 1024, w_layout="packed"), 256),
                      dtype=torch.uint8, device="cuda")
    dev.append((to_device(a, "bf16"), Wp, wsp, torch.empty((16, 4096), dtype=torch.float32,
                                                            device="cuda"), 0))
    kw = [{}, {}, dict(n=4096)]
    eager = [fd.fd_flat_gemm(A, W, ksplit=ks, workspace=ws, **x).clone()
             for (A, W, ws, _, ks), x in zip(dev, kw)]
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for (A, W, ws, out, ks), x in zip(dev, kw):
                fd.fd_flat_gemm(A, W, out, ksplit=ks, workspace=ws, **x)
    torch.cuda.synchronize()
    for rep in range(4):
        for _, _, ws, out, _ in dev:
            out.fill_(float("nan"))
            ws.fill_(0x7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (_, _, _, out, _), e in zip(dev, eager):
            assert torch.equal(out, e), rep
        # eager work between replays
        fd.fd_flat_gemm(dev[0][0], dev[0][1], ksplit=2)
        torch.cuda.synchronize()


def _pack_reference(w):
    """The packed layout of include/fd_gemm.h, restated with numpy: block cb,
    step j, lane l holds row 16cb + l % 16, elements 32j + 8(l // 16) .. +7;
    rows past N are zero."""
    n, k = w.shape
    npad = -(-n // 16) * 16
    wp = np.zeros((npad, k), dtype=w.dtype)
    wp[:n] = w
    t = wp.reshape(npad // 16, 16, k // 32, 4, 8)          # [cb, r, j, g, e]
    return t.transpose(0, 2, 3, 1, 4).reshape(-1)          # [cb, j, l = 16g + r, e]


@pytest.mark.parametrize("n,k", [(16, 32), (200, 96), (130, 512), (4096, 256)])
def test_pack_weights_layout(n, k):
    _, w = synthetic.make_gemm(1, n, k, seed=370 + n)
    W = to_device(w, "bf16")
    got = fd.fd_flat_gemm_pack_weights(W)
    torch.cuda.synchronize()
    got = got.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, _pack_reference(w))


def _check_packed(m, n, k, out_dtype="f32", seed=380, **kw):
    a, w = synthetic.make_gemm(m, n, k, seed=seed)
    print("case packed gemm m=%d n=%d k=%d %s %s" % (m, n, k, out_dtype, kw), flush=True)
    A, W = to_device(a, "bf16"), to_device(w, "bf16")
    Wp = fd.fd_flat_gemm_pack_weights(W)
    c = fd.fd_flat_gemm(A, Wp, out_dtype=out_dtype, n=n, **kw)
    torch.cuda.synchronize()
    got = c.float().cpu().numpy().astype(np.float64)
    ref = oracle.flat_gemm(a, w)
    err = np.abs(got - ref)
    bound = _bound(a, w, k, out_dtype, ref)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), (worst, err[worst], bound[worst])


@pytest.mark.parametrize("variant", range(5, 13))
@pytest.mark.parametrize("m,n,k", SMALL, ids=["%dx%dx%d" % s for s in SMALL])
def test_packed_variants_small(variant, m, n, k):
    for ks in (1, 3, 0):
        if ks <= k // 32:
            _check_packed(m, n, k, variant=variant, ksplit=ks, seed=390 + m)


@pytest.mark.parametrize("layer", range(4))
def test_packed_7b_block_layers_full(layer):
    cfg = synthetic.GEMM_CONFIGS[2]
    name, n, k = cfg["layers"][layer]
    print("layer", name, fd.fd_flat_gemm_plan(cfg["m"], n, k, w_layout="packed"), flush=True)
    _check_packed(cfg["m"], n, k, "bf16" if layer % 2 else "f32",
                  seed=synthetic.SEED_BASE + 200 + layer)
