"""GPU parity of the looped Einsum-ReduceScatter with the fused reduce
epilogue, through the C ABI: bit for bit the two-call path (ReduceScatter in
fp32, then the batched epilogue over the ranks), and within the bf16 / fp32
tolerance of the float64 oracle (monolithic ReduceScatter, then the epilogue
with its Philox keep mask)."""

import numpy as np
import pytest
import torch

from oracle import einsum as oe, epilogue as oep
import workloads as W
from gpu_util import np64, assert_bf16_close, assert_f32_close, sync

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def ctx():
    import collective_overlap_amd as cce
    c = cce.Context(0)
    yield c
    sync()
    c.close()


def _inputs(mode, n, dims, seed):
    s, k, c = dims
    if mode == "slice_lhs_rows":
        a = [W.normal((n * s, k), 1.0, seed + r, device=DEV, dtype=torch.bfloat16) for r in range(n)]
        b = [W.normal((c, k), 0.05, seed + 50 + r, device=DEV, dtype=torch.bfloat16) for r in range(n)]
        oshape = (s, c)
    else:
        a = [W.normal((c, k), 1.0, seed + r, device=DEV, dtype=torch.bfloat16) for r in range(n)]
        b = [W.normal((n * s, k), 0.05, seed + 50 + r, device=DEV, dtype=torch.bfloat16) for r in range(n)]
        oshape = (c, s)
    return a, b, oshape


FORMS = ["one-way stream", "one-way fused", "two-way stream", "two-way fused", "one-way serial",
         "one-way serial one-chain", "two-way stream one-chain"]
CASES = [
    # mode, (shard, K, other), n, out, p, bias, residual
    ("slice_lhs_rows", (72, 256, 264), 4, "bf16", 0.1, True, True),
    ("slice_lhs_rows", (73, 136, 96), 3, "f32", 0.3, True, False),     # ragged halves
    ("slice_rhs_cols", (96, 200, 40), 4, "bf16", 0.1, False, True),
    ("slice_rhs_cols", (104, 64, 33), 2, "f32", 1.0, True, True),      # drops everything
    ("slice_lhs_rows", (16, 64, 1024), 8, "bf16", 0.0, True, True),    # no dropout
]


def _flags(cce, form):
    f = 0
    if "fused" in form:
        f |= cce.CCE_FLAG_FUSED_PERMUTE
    if "two-way" in form:
        f |= cce.CCE_FLAG_BIDIRECTIONAL
    if "serial" in form:
        f |= cce.CCE_FLAG_SERIAL
    if "one-chain" in form:
        f |= cce.CCE_FLAG_ONE_CHAIN
    return f


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("form", FORMS)
def test_reducescatter_epilogue(ctx, case, form):
    import collective_overlap_amd as cce
    mode, dims, n, ot, p, has_b, has_r = case
    print(f"[gpu] reducescatter+epilogue {form} {case}", flush=True)
    odt = torch.bfloat16 if ot == "bf16" else torch.float32
    a, b, oshape = _inputs(mode, n, dims, seed=7 * n)
    rows, cols = oshape
    bias = W.normal((cols,), 0.02, 90, device=DEV, dtype=odt) if has_b else None
    res = [W.normal(oshape, 1.0, 100 + r, device=DEV, dtype=odt) for r in range(n)] if has_r else None
    row0 = [r * rows for r in range(n)]
    seed, off = 11, 3
    flags = _flags(cce, form)
    out = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter_epilogue(ctx, mode, a, b, bias, res, out, p, seed, off,
                                                 mask_row0=row0, mask_col0=0, mask_ld=cols,
                                                 flags=flags)
    # two calls: the ReduceScatter in fp32, then the batched epilogue
    s = [torch.full(oshape, float("nan"), device=DEV, dtype=torch.float32) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, s, flags=flags)
    two = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
    cce.cce_fused_reduce_epilogue_batched(ctx, [[x] for x in s], bias, res, two, p, seed, off,
                                          mask_row0=row0, mask_col0=0, mask_ld=cols)
    sync()
    it = torch.int16 if odt == torch.bfloat16 else torch.int32
    for r in range(n):
        assert torch.equal(out[r].view(it), two[r].view(it)), f"rank {r}: fused and two-call differ"
    ref = oe.einsum_reducescatter(mode, [np64(x) for x in a], [np64(x).T for x in b])
    for r in range(n):
        want, _ = oep.fused_reduce_epilogue([ref[r]], np64(bias) if has_b else None,
                                            np64(res[r]) if has_r else None, p, seed, off,
                                            row0[r], 0, cols)
        if ot == "bf16":
            assert_bf16_close(np64(out[r]), want, f"rank {r}")
        else:
            assert_f32_close(np64(out[r]), want, f"rank {r}")


def test_reducescatter_epilogue_rejects(ctx):
    import collective_overlap_amd as cce
    a = [torch.zeros((16, 64), device=DEV, dtype=torch.bfloat16)]
    b = [torch.zeros((32, 64), device=DEV, dtype=torch.bfloat16)]
    out = [torch.empty((16, 32), device=DEV, dtype=torch.bfloat16)]
    with pytest.raises(RuntimeError):      # one rank: no accumulators to fuse into
        cce.cce_looped_einsum_reducescatter_epilogue(ctx, "slice_lhs_rows", a, b, None, None,
                                                     out, 0.1)
