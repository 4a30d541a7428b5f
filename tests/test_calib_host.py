"""The band choice of the C ABI (fd_attn_choose_band, host code in the library)
against the float64 calibration oracle.  No GPU needed.

The chooser must return the narrowest band that keeps all but
floor(max_flag_fraction * m) of the m non-empty rows (exact over the given
extremes, up to float rounding of phi, a and b), a phi that keeps that many
rows, and the number of rows the returned band flags.  Several phi may be
optimal: the test checks the unique parts (width, kept count) and that the
phi it got is one of the optimal ones.
"""
import numpy as np
import pytest

import oracle
import split_kv_asynchronous_amd as fd


def _rows(seed, n=40, empty=3):
    rng = np.random.default_rng(seed)
    mx = rng.normal(3.0, 1.5, n).astype(np.float32)
    mn = (mx - rng.uniform(0.5, 6.0, n)).astype(np.float32)
    mx[:empty], mn[:empty] = -np.inf, np.inf
    return mx, mn


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("frac", [0.0, 0.1, 0.3, 0.5])
@pytest.mark.parametrize("share", [0.5, 0.8])
def test_narrowest_band_and_its_phi(seed, frac, share):
    mx, mn = _rows(seed)
    m = int((mx >= mn).sum())
    allowed = int(np.floor(frac * m))
    pad = 1e-3
    phi, a, b, flagged = fd.fd_attn_choose_band(mx, mn, frac, share, 64.0, pad)
    w_exact = oracle.min_band_width(mx.astype(np.float64), mn.astype(np.float64), allowed)
    # width: exact minimum, up to float rounding of a and b
    assert (a - pad) + (b - pad) == pytest.approx(w_exact, abs=1e-5 * max(1.0, w_exact))
    assert (a - pad) == pytest.approx(share * w_exact, abs=1e-5 * max(1.0, w_exact))
    # the reported count is the returned band's, and it is within the budget
    kept = oracle.rows_in_band(mx.astype(np.float64), mn.astype(np.float64), phi, a, b)
    assert flagged == m - kept
    assert flagged <= allowed
    # without the pad the chosen phi still keeps as many rows as any phi can
    a0, b0 = share * w_exact, (1 - share) * w_exact
    live = mx >= mn
    cands = np.concatenate([mx[live].astype(np.float64) - b0, mn[live].astype(np.float64) + a0])
    best = max(oracle.rows_in_band(mx, mn, c, a0 + 1e-9, b0 + 1e-9) for c in cands)
    got = oracle.rows_in_band(mx, mn, phi, a0 + 1e-5, b0 + 1e-5)
    assert got >= best and best >= m - allowed


def test_width_cap_reports_the_rows_it_cannot_keep():
    mx, mn = _rows(11)
    phi, a, b, flagged = fd.fd_attn_choose_band(mx, mn, 0.0, 0.5, 2.0, 0.0)
    assert a + b == pytest.approx(2.0, abs=1e-6)
    m = int((mx >= mn).sum())
    kept = oracle.rows_in_band(mx, mn, phi, a, b)
    assert flagged == m - kept and flagged > 0
    # the cap's phi keeps as many rows as any phi for that width
    live = mx >= mn
    cands = np.concatenate([mx[live].astype(np.float64) - 1.0, mn[live].astype(np.float64) + 1.0])
    assert kept == max(oracle.rows_in_band(mx, mn, c, 1.0, 1.0) for c in cands)


def test_empty_and_degenerate_inputs():
    inf = np.float32(np.inf)
    assert fd.fd_attn_choose_band([-inf, -inf], [inf, inf])[3] == 0
    assert fd.fd_attn_choose_band([], [])[3] == 0
    phi, a, b, flagged = fd.fd_attn_choose_band([2.0], [2.0], pad=0.5)
    assert flagged == 0 and phi == 2.0 and a == b == 0.5


@pytest.mark.parametrize("kw,code", [
    (dict(max_flag_fraction=-0.1), -5), (dict(max_flag_fraction=1.5), -5),
    (dict(a_share=1.2), -5), (dict(max_width=0.0), -5), (dict(max_width=float("inf")), -5),
    (dict(pad=-1.0), -5),
])
def test_argument_errors(kw, code):
    with pytest.raises(fd.FdAttnError) as e:
        fd.fd_attn_choose_band([1.0], [0.0], **kw)
    assert e.value.status == code


def test_null_pointers_are_rejected():
    import ctypes
    lib = fd._load()
    x = ctypes.c_float()
    n = ctypes.c_int64()
    assert lib.fd_attn_choose_band(None, None, 3, 0.0, 0.5, 10.0, 0.0, ctypes.byref(x),
                                   ctypes.byref(x), ctypes.byref(x), ctypes.byref(n)) == -1
    arr = (ctypes.c_float * 1)(1.0)
    assert lib.fd_attn_choose_band(arr, arr, 1, 0.0, 0.5, 10.0, 0.0, None, ctypes.byref(x),
                                   ctypes.byref(x), ctypes.byref(n)) == -1
