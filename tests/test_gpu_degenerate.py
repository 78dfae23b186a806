"""GPU checks of the degenerate shapes of every entry point, through the C ABI:
extents of zero rows or columns (the call returns without enqueueing work and
without error) and a zero-length contraction (every partial product is the
empty sum, exactly zero, so the AllGather and ReduceScatter results are zero
in every permute form and ring direction, and the fused epilogue sees a zero
partial).  The oracle of the last case is the float64 epilogue of a zero
partial."""

import numpy as np
import pytest
import torch

from oracle import epilogue as oep
import workloads as W
from gpu_util import np64, sync

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16


@pytest.fixture(scope="module")
def ctx():
    import collective_overlap_amd as cce
    c = cce.Context(0)
    yield c
    sync()
    c.close()


def _forms(cce):
    return {"stream": 0, "serial": cce.CCE_FLAG_SERIAL, "fused": cce.CCE_FLAG_FUSED_PERMUTE,
            "fused two-way": cce.CCE_FLAG_FUSED_PERMUTE | cce.CCE_FLAG_BIDIRECTIONAL,
            "stream two-way": cce.CCE_FLAG_BIDIRECTIONAL}


@pytest.mark.parametrize("form", ["stream", "serial", "fused", "fused two-way", "stream two-way"])
def test_zero_rows_and_columns_are_no_ops(ctx, form):
    """Outputs with no rows or no columns: every call returns without error
    and a sentinel tensor enqueued after it on the same stream is intact."""
    import collective_overlap_amd as cce
    flags = _forms(cce)[form]
    n, k = 4, 64
    print(f"[gpu] zero extents, {form}", flush=True)
    guard = torch.full((16,), 7.0, device=DEV)
    # AllGather: no rows per shard, then no output columns
    for m_s, N in ((0, 40), (24, 0)):
        x = [W.normal((m_s, k), 1.0, r, device=DEV) for r in range(n)]
        w = [W.normal((N, k), 0.05, 10 + r, device=DEV) for r in range(n)]
        out = [torch.empty((n * m_s, N), device=DEV, dtype=BF) for _ in range(n)]
        cce.cce_looped_allgather_einsum(ctx, "lhs_rows", x, w, out, flags=flags | cce.CCE_FLAG_GELU)
    # ReduceScatter and its fused epilogue: no rows per shard, then no columns
    for s, N in ((0, 40), (24, 0)):
        a = [W.normal((n * s, k), 1.0, 20 + r, device=DEV) for r in range(n)]
        b = [W.normal((N, k), 0.05, 30 + r, device=DEV) for r in range(n)]
        out = [torch.empty((s, N), device=DEV) for _ in range(n)]
        cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", a, b, out, flags=flags)
        res = [torch.empty((s, N), device=DEV, dtype=BF) for _ in range(n)]
        eout = [torch.empty((s, N), device=DEV, dtype=BF) for _ in range(n)]
        bias = torch.zeros((N,), device=DEV, dtype=BF)
        cce.cce_looped_einsum_reducescatter_epilogue(
            ctx, "slice_lhs_rows", a, b, bias, res, eout, 0.1, 1, 2,
            mask_row0=[r * s for r in range(n)], mask_col0=0, mask_ld=max(N, 1), flags=flags)
    ctx.check_signals()
    sync()
    assert bool((guard == 7.0).all())


def test_zero_extents_of_the_local_calls(ctx):
    import collective_overlap_amd as cce
    for M, N in ((0, 40), (24, 0), (0, 0)):
        a = [W.normal((M, 64), 1.0, 40 + g, device=DEV) for g in range(3)]
        b = [W.normal((N, 64), 0.05, 50 + g, device=DEV) for g in range(3)]
        c = [torch.empty((M, N), device=DEV) for _ in range(3)]
        cce.cce_grouped_gemm(ctx, a, b, c)
        p = [torch.empty((M, N), device=DEV) for _ in range(2)]
        out = torch.empty((M, N), device=DEV, dtype=BF)
        cce.cce_fused_reduce_epilogue(ctx, p, None, None, out, 0.1, 3, 4, mask_ld=max(N, 1))
    sync()


@pytest.mark.parametrize("form", ["stream", "serial", "fused", "fused two-way", "stream two-way"])
def test_zero_length_contraction_gives_zero_products(ctx, form):
    """K = 0: no k tile runs, every partial is the empty sum.  The AllGather
    writes GELU(0) = 0 into every slice, the ReduceScatter sums zeros, and the
    fused epilogue sees a zero partial (out = R + keep * b / (1 - p))."""
    import collective_overlap_amd as cce
    flags = _forms(cce)[form]
    n, m_s, N = 4, 40, 72
    print(f"[gpu] K = 0, {form}", flush=True)
    x = [W.normal((m_s, 0), 1.0, r, device=DEV) for r in range(n)]
    w = [W.normal((N, 0), 0.05, 10 + r, device=DEV) for r in range(n)]
    out = [torch.full((n * m_s, N), float("nan"), device=DEV, dtype=BF) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, "lhs_rows", x, w, out, flags=flags | cce.CCE_FLAG_GELU)
    a = [W.normal((n * m_s, 0), 1.0, 20 + r, device=DEV) for r in range(n)]
    rout = [torch.full((m_s, N), float("nan"), device=DEV) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", a, w, rout, flags=flags)
    bias = W.normal((N,), 0.02, 60, device=DEV, dtype=torch.float32)
    res = [W.normal((m_s, N), 1.0, 70 + r, device=DEV, dtype=torch.float32) for r in range(n)]
    eout = [torch.full((m_s, N), float("nan"), device=DEV) for _ in range(n)]
    row0 = [r * m_s for r in range(n)]
    cce.cce_looped_einsum_reducescatter_epilogue(
        ctx, "slice_lhs_rows", a, w, bias, res, eout, 0.1, 5, 6, mask_row0=row0, mask_col0=0,
        mask_ld=N, flags=flags)
    ctx.check_signals()
    sync()
    zero = np.zeros((m_s, N))
    for r in range(n):
        assert np.array_equal(np64(out[r]), np.zeros((n * m_s, N))), f"allgather rank {r}"
        assert np.array_equal(np64(rout[r]), zero), f"reducescatter rank {r}"
        want, _ = oep.fused_reduce_epilogue([zero], np64(bias), np64(res[r]), 0.1, 5, 6,
                                            row0=row0[r], col0=0, mask_ld=N)
        np.testing.assert_allclose(np64(eout[r]), want, rtol=1e-6, atol=1e-6,
                                   err_msg=f"epilogue rank {r}")


def test_zero_length_contraction_of_the_grouped_gemm(ctx):
    import collective_overlap_amd as cce
    a = [W.normal((300, 0), 1.0, 80 + g, device=DEV) for g in range(3)]
    b = [W.normal((264, 0), 0.05, 90 + g, device=DEV) for g in range(3)]
    for gelu, dt in ((False, torch.float32), (True, BF)):
        c = [torch.full((300, 264), float("nan"), device=DEV, dtype=dt) for _ in range(3)]
        cce.cce_grouped_gemm(ctx, a, b, c, gelu=gelu)
        sync()
        for g in range(3):
            assert np.array_equal(np64(c[g]), np.zeros((300, 264))), f"group {g} gelu {gelu}"
