"""Pins for oracle.epilogue: a per-element pure-Python loop, p = 0 and p = 1,
linearity in the partials, N = 1."""

import numpy as np
import pytest

from oracle import epilogue, philox


def _per_element(partials, bias, residual, p, seed, offset, row0, col0, ld):
    rows, cols = partials[0].shape
    t = philox.keep_threshold(p)
    out = np.zeros((rows, cols))
    for i in range(rows):
        for j in range(cols):
            s = 0.0
            for x in partials:
                s += float(x[i, j])
            s += float(bias[j])
            e = (row0 + i) * ld + (col0 + j)
            w = int(philox.element_words(np.array([e], dtype=np.uint64), seed, offset)[0])
            d = s / (1.0 - p) if w >= t else 0.0
            out[i, j] = d + float(residual[i, j])
    return out


@pytest.mark.parametrize("n", [1, 2, 5])
def test_fused_epilogue_vs_per_element_loop(n):
    rng = np.random.default_rng(n)
    rows, cols = 5, 13
    parts = [rng.uniform(-1, 1, (rows, cols)) for _ in range(n)]
    bias = rng.uniform(-1, 1, cols)
    res = rng.uniform(-1, 1, (rows, cols))
    got, _ = epilogue.fused_reduce_epilogue(parts, bias, res, 0.3, 42, 7,
                                            row0=3, col0=5, mask_ld=40)
    ref = _per_element(parts, bias, res, 0.3, 42, 7, 3, 5, 40)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-14)


def test_p0_is_sum_bias_residual():
    rng = np.random.default_rng(1)
    parts = [rng.standard_normal((4, 8)) for _ in range(3)]
    bias = rng.standard_normal(8)
    res = rng.standard_normal((4, 8))
    got, keep = epilogue.fused_reduce_epilogue(parts, bias, res, 0.0, 0, 0)
    assert keep.all()
    np.testing.assert_allclose(got, parts[0] + parts[1] + parts[2] + bias + res,
                               rtol=1e-15, atol=1e-15)


def test_p1_is_residual():
    rng = np.random.default_rng(2)
    parts = [rng.standard_normal((4, 8)) for _ in range(2)]
    res = rng.standard_normal((4, 8))
    got, keep = epilogue.fused_reduce_epilogue(parts, np.ones(8), res, 1.0, 0, 0)
    assert not keep.any()
    np.testing.assert_array_equal(got, res)


def test_linear_in_partials_and_kept_scale():
    rng = np.random.default_rng(3)
    parts = [rng.standard_normal((6, 16)) for _ in range(2)]
    zero_b, zero_r = np.zeros(16), np.zeros((6, 16))
    y1, k1 = epilogue.fused_reduce_epilogue(parts, zero_b, zero_r, 0.25, 3, 4)
    y2, k2 = epilogue.fused_reduce_epilogue([2 * x for x in parts], zero_b, zero_r,
                                            0.25, 3, 4)
    assert np.array_equal(k1, k2)
    np.testing.assert_allclose(y2, 2 * y1, rtol=1e-15)
    s = parts[0] + parts[1]
    np.testing.assert_allclose(y1[k1], s[k1] / 0.75, rtol=1e-15)
    assert np.all(y1[~k1] == 0)


@pytest.mark.parametrize("n,rows,cols", [(1, 5, 7), (2, 6, 9), (4, 10, 16), (8, 8, 12), (3, 7, 5)])
@pytest.mark.parametrize("p", [0.0, 0.1, 1.0])
def test_fused_allreduce_is_epilogue_of_allreduce(n, rows, cols, p):
    """ReduceScatter -> epilogue on each rank's slice -> AllGather gives the
    whole-tensor epilogue of the AllReduce sum on every rank, bit for bit."""
    rng = np.random.default_rng(n * 100 + rows)
    parts = [rng.standard_normal((rows, cols)) for _ in range(n)]
    bias, res = rng.standard_normal(cols), rng.standard_normal((rows, cols))
    outs, keep = epilogue.fused_allreduce(parts, bias, res, p, 9, 2, col0=3, mask_ld=cols + 5)
    whole, wkeep = epilogue.fused_reduce_epilogue(parts, bias, res, p, 9, 2, row0=0, col0=3,
                                             mask_ld=cols + 5)
    assert np.array_equal(keep, wkeep)
    for o in outs:
        assert np.array_equal(o, whole)


# ---------------------------------------------------------------------------
# The float32 evaluation (fused_reduce_epilogue_fp32)
# ---------------------------------------------------------------------------
U32 = 2.0 ** -24            # unit roundoff of float32


def _gamma(m):
    return m * U32 / (1 - m * U32)


@pytest.mark.parametrize("n", [1, 2, 5, 8])
@pytest.mark.parametrize("p", [0.0, 0.1, 0.5])
def test_fp32_within_rounding_bound_of_fp64(n, p):
    """n - 1 additions, the bias, the scale (itself rounded once) and the
    residual: at most n + 3 roundings, so |fp32 - exact| <= gamma_(n+3) *
    (c (sum |P| + |b|) + |R|) element by element (the standard bound for a
    chain of rounded operations).  A dropped or doubled term, a wrong sign or
    a wrong scale breaks it by orders of magnitude."""
    rng = np.random.default_rng(100 + n)
    rows, cols = 7, 45
    f32 = lambda a: a.astype(np.float32).astype(np.float64)
    parts = [f32(rng.normal(0, 1, (rows, cols))) for _ in range(n)]
    bias = f32(rng.normal(0, 0.02, cols))
    res = f32(rng.normal(0, 1, (rows, cols)))
    got, keep = epilogue.fused_reduce_epilogue_fp32(parts, bias, res, p, 3, 1, 2, 5, 60)
    ref, keep64 = epilogue.fused_reduce_epilogue(parts, bias, res, p, 3, 1, 2, 5, 60)
    assert got.dtype == np.float32 and np.array_equal(keep, keep64)
    c = 1.0 / (1.0 - p)
    mag = c * (sum(np.abs(x) for x in parts) + np.abs(bias)[None, :]) + np.abs(res)
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= _gamma(n + 3) * mag)
    assert err.max() > 0            # the evaluation does round (not float64 in disguise)


def test_fp32_p1_is_the_residual_exactly():
    rng = np.random.default_rng(9)
    parts = [rng.normal(0, 1, (4, 9)).astype(np.float32) for _ in range(3)]
    res = rng.normal(0, 1, (4, 9)).astype(np.float32)
    got, keep = epilogue.fused_reduce_epilogue_fp32(parts, None, res, 1.0, 0, 0)
    assert not keep.any() and np.array_equal(got, res)


def test_fp32_sum_order():
    """2^25 + 1 is not a float32 (its neighbours are 4 apart), so the order of
    the partial sum shows: ((2^25 + 1) - 2^25) = 0, but ((2^25 - 2^25) + 1) = 1."""
    big = float(2 ** 25)
    a = [np.array([[big]]), np.array([[1.0]]), np.array([[-big]])]
    b = [np.array([[big]]), np.array([[-big]]), np.array([[1.0]])]
    assert epilogue.fused_reduce_epilogue_fp32(a, None, None, 0.0, 0, 0)[0][0, 0] == 0.0
    assert epilogue.fused_reduce_epilogue_fp32(b, None, None, 0.0, 0, 0)[0][0, 0] == 1.0
    # the float64 definition sees the exact sum in both orders
    assert epilogue.fused_reduce_epilogue(a, None, None, 0.0, 0, 0)[0][0, 0] == 1.0


def no_fma_case(p=0.1, seed=0, offset=0, cols=64):
    """A kept element e (the first of a row of `cols`) with s = 1.2345678 (as
    float32) and residual R = -fl32(s * c): rounding the product before the
    add gives exactly 0, a fused multiply-add gives the product's rounding
    error.  Returns (e, s, R, fused-multiply-add result)."""
    keep = philox.keep_mask(1, cols, p, seed, offset, 0, 0, cols)[0]
    e = int(np.argmax(keep))
    assert keep[e]
    s = np.float32(1.2345678)
    c = np.float32(1.0 / (1.0 - p))
    prod = np.float32(s * c)
    fma = float(s) * float(c) - float(prod)       # exact in float64 (24 x 24 bits)
    return e, s, -prod, fma


def test_fp32_no_fused_multiply_add():
    e, s, r, fma = no_fma_case()
    assert fma != 0.0                              # the case tells the two apart
    part = np.zeros((1, 64), dtype=np.float32)
    part[0, e] = s
    res = np.zeros((1, 64), dtype=np.float32)
    res[0, e] = r
    got, keep = epilogue.fused_reduce_epilogue_fp32([part], None, res, 0.1, 0, 0)
    assert keep[0, e] and got[0, e] == 0.0
