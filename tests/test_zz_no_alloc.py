"""GPU test of the allocation-free entry point
cce_looped_einsum_reducescatter_epilogue_noalloc, through the C ABI: its
outputs equal, bit for bit, those of cce_looped_einsum_reducescatter_epilogue
(the same kernels, with a caller workspace) on the same inputs, for two calls
in a row on one stream, the second with a smaller input (the static scratch
then still holds the first call's accumulators).  A call whose workspace would
exceed the static scratch is rejected before anything is enqueued."""

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def ctx():
    import collective_overlap_amd as cce
    c = cce.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


def _problem(n, shard, k, cols, seed):
    bf = torch.bfloat16
    a = [W.normal((n * shard, k), 1.0, seed + r, device=DEV, dtype=bf) for r in range(n)]
    b = [W.normal((cols, k), 0.05, seed + 50 + r, device=DEV, dtype=bf) for r in range(n)]
    bias = W.normal((cols,), 0.02, seed + 90, device=DEV, dtype=bf)
    res = [W.normal((shard, cols), 1.0, seed + 100 + r, device=DEV, dtype=bf) for r in range(n)]
    rows0 = [r * shard for r in range(n)]
    return a, b, bias, res, rows0


FORMS = {
    "one-way stream": 0,
    "one-way fused": "F",
    "two-way fused": "FB",
    "two-way stream": "B",
}


def _flags(cce, code):
    f = 0
    if code and "F" in code:
        f |= cce.CCE_FLAG_FUSED_PERMUTE
    if code and "B" in code:
        f |= cce.CCE_FLAG_BIDIRECTIONAL
    return f


@pytest.mark.parametrize("form", list(FORMS))
def test_noalloc_matches_workspace_entry_point(ctx, form):
    import collective_overlap_amd as cce
    flags = _flags(cce, FORMS[form])
    # (n, shard rows, K, cols): the second call is smaller than the first
    for call, (n, shard, k, cols) in enumerate([(4, 136, 256, 392), (3, 40, 128, 200)]):
        a, b, bias, res, rows0 = _problem(n, shard, k, cols, 1000 * (call + 1))
        ref = [torch.empty((shard, cols), device=DEV, dtype=torch.bfloat16) for _ in range(n)]
        got = [torch.full((shard, cols), float("nan"), device=DEV, dtype=torch.bfloat16)
               for _ in range(n)]
        cce.cce_looped_einsum_reducescatter_epilogue(
            ctx, "slice_lhs_rows", a, b, bias, res, ref, 0.1, 7, 3, mask_row0=rows0,
            mask_col0=0, mask_ld=cols, flags=flags)
        cce.cce_looped_einsum_reducescatter_epilogue_noalloc(
            ctx, "slice_lhs_rows", a, b, bias, res, got, 0.1, 7, 3, mask_row0=rows0,
            mask_col0=0, mask_ld=cols, flags=flags)
        torch.cuda.synchronize()
        for r in range(n):
            assert torch.equal(got[r].view(torch.int16), ref[r].view(torch.int16)), \
                f"{form}, call {call}, rank {r}"


def test_noalloc_rejects_workspace_beyond_scratch(ctx):
    import collective_overlap_amd as cce
    from collective_overlap_amd import _lib
    n, shard, k, cols = 8, 512, 8, 4096     # workspace 4 * 8 * 8 MiB > 64 MiB
    need = cce.cce_looped_einsum_reducescatter_workspace(n, "slice_lhs_rows", (shard, cols))
    assert need > _lib.CCE_NOALLOC_SCRATCH_BYTES
    a, b, bias, res, rows0 = _problem(n, shard, k, cols, 5000)
    out = [torch.zeros((shard, cols), device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    torch.cuda.synchronize()
    with pytest.raises(_lib.CceError) as e:
        cce.cce_looped_einsum_reducescatter_epilogue_noalloc(
            ctx, "slice_lhs_rows", a, b, bias, res, out, 0.1, mask_row0=rows0)
    assert e.value.status == _lib.CCE_EUNSUPPORTED
    torch.cuda.synchronize()
    assert all(int(torch.count_nonzero(o)) == 0 for o in out)   # nothing was enqueued
