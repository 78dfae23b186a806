"""GPU parity of the fine-grained overlap (CCE_FLAG_FINE_GRAINED: the
consumer of every output chunk of the looped Einsum-ReduceScatter -- the
align-and-sum of the two ring directions, or the fused reduce epilogue --
runs inside the launch that produces the chunk's last partials), through the
C ABI.  Outputs are compared bit for bit with the same call without the flag
(whose outputs the other GPU tests hold to the oracle), and one case per
entry point directly with the float64 oracle.  The give-up path of the
bounded wait is forced from the host (cce_debug_signal_giveup: the first
producers withhold their ready words), so every kernel still ends normally."""

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


def _inputs(mode, n, dims, seed, in_dt=torch.bfloat16):
    s, k, c = dims
    if mode == "slice_lhs_rows":
        a = [W.normal((n * s, k), 1.0, seed + r, device=DEV, dtype=in_dt) for r in range(n)]
        b = [W.normal((c, k), 0.05, seed + 50 + r, device=DEV, dtype=in_dt) for r in range(n)]
        return a, b, (s, c)
    a = [W.normal((c, k), 1.0, seed + r, device=DEV, dtype=in_dt) for r in range(n)]
    b = [W.normal((n * s, k), 0.05, seed + 50 + r, device=DEV, dtype=in_dt) for r in range(n)]
    return a, b, (c, s)


def _flags(cce, form):
    f = cce.CCE_FLAG_FUSED_PERMUTE if "fused" in form else 0
    if "two-way" in form:
        f |= cce.CCE_FLAG_BIDIRECTIONAL
    if "serial" in form:
        f |= cce.CCE_FLAG_SERIAL
    if "one-chain" in form:
        f |= cce.CCE_FLAG_ONE_CHAIN
    return f


def _ints(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


EPI_FORMS = ["two-way fused", "one-way fused", "one-way stream", "one-way serial",
             "one-way serial one-chain"]
EPI_CASES = [
    # mode, (shard, K, other), n, out, p, bias, residual
    ("slice_lhs_rows", (72, 256, 264), 4, "bf16", 0.1, True, True),     # pairs, ragged tiles
    ("slice_lhs_rows", (73, 136, 96), 3, "f32", 0.3, True, False),      # n odd, ragged halves
    ("slice_rhs_cols", (96, 200, 40), 4, "bf16", 0.1, False, True),
    ("slice_rhs_cols", (104, 64, 33), 2, "f32", 1.0, True, True),       # one iteration; drops all
    ("slice_lhs_rows", (16, 64, 1024), 8, "bf16", 0.0, True, True),     # no dropout
    ("slice_lhs_rows", (300, 512, 640), 6, "bf16", 0.1, True, True),    # several 256 x 256 tiles
]


@pytest.mark.parametrize("case", EPI_CASES)
@pytest.mark.parametrize("form", EPI_FORMS)
def test_epilogue_fine_equals_event_form(ctx, case, form):
    import collective_overlap_amd as cce
    mode, dims, n, ot, p, has_b, has_r = case
    print(f"[gpu] fine-grained epilogue {form} {case}", flush=True)
    odt = torch.bfloat16 if ot == "bf16" else torch.float32
    a, b, oshape = _inputs(mode, n, dims, seed=11 * n)
    rows, cols = oshape
    bias = W.normal((cols,), 0.02, 90, device=DEV, dtype=odt) if has_b else None
    res = [W.normal(oshape, 1.0, 100 + r, device=DEV, dtype=odt) for r in range(n)] if has_r else None
    row0 = [r * rows for r in range(n)]
    flags = _flags(cce, form)
    outs = {}
    for fine in (0, cce.CCE_FLAG_FINE_GRAINED):
        o = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
        cce.cce_looped_einsum_reducescatter_epilogue(ctx, mode, a, b, bias, res, o, p, 5, 2,
                                                     mask_row0=row0, mask_col0=0, mask_ld=cols,
                                                     flags=flags | fine)
        outs[fine] = o
    ctx.check_signals()
    for r in range(n):
        assert torch.equal(_ints(outs[0][r]), _ints(outs[cce.CCE_FLAG_FINE_GRAINED][r])), \
            f"rank {r}: fine-grained and event forms differ"


RS_CASES = [
    # mode, (shard, K, other), n, out dtype
    ("slice_lhs_rows", (72, 256, 264), 4, torch.float32),
    ("slice_lhs_rows", (73, 136, 96), 5, torch.bfloat16),
    ("slice_rhs_cols", (96, 200, 40), 2, torch.float32),
    ("slice_lhs_rows", (300, 512, 640), 8, torch.float32),
]


@pytest.mark.parametrize("case", RS_CASES)
def test_align_and_sum_fine_equals_event_form(ctx, case):
    """Two-way fused ReduceScatter without epilogue: the last launch writes
    out = cw + ccw itself (the align-and-sum launch goes)."""
    import collective_overlap_amd as cce
    mode, dims, n, odt = case
    print(f"[gpu] fine-grained align-and-sum {case}", flush=True)
    a, b, oshape = _inputs(mode, n, dims, seed=3 * n)
    flags = cce.CCE_FLAG_FUSED_PERMUTE | cce.CCE_FLAG_BIDIRECTIONAL
    outs = {}
    for fine in (0, cce.CCE_FLAG_FINE_GRAINED):
        o = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
        cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, o, flags=flags | fine)
        outs[fine] = o
    ctx.check_signals()
    for r in range(n):
        assert torch.equal(_ints(outs[0][r]), _ints(outs[cce.CCE_FLAG_FINE_GRAINED][r])), f"rank {r}"


@pytest.mark.parametrize("form", ["two-way fused", "one-way stream"])
def test_fine_against_oracle(ctx, form):
    import collective_overlap_amd as cce
    mode, (s, k, c), n, p = "slice_lhs_rows", (136, 384, 520), 4, 0.1
    a, b, oshape = _inputs(mode, n, (s, k, c), seed=77)
    bias = W.normal((c,), 0.02, 91, device=DEV, dtype=torch.bfloat16)
    res = [W.normal(oshape, 1.0, 110 + r, device=DEV, dtype=torch.bfloat16) for r in range(n)]
    row0 = [r * s for r in range(n)]
    out = [torch.full(oshape, float("nan"), device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter_epilogue(
        ctx, mode, a, b, bias, res, out, p, 9, 4, mask_row0=row0, mask_col0=0, mask_ld=c,
        flags=_flags(cce, form) | cce.CCE_FLAG_FINE_GRAINED)
    ctx.check_signals()
    ref = oe.einsum_reducescatter(mode, [np64(x) for x in a], [np64(x).T for x in b])
    for r in range(n):
        want, _ = oep.fused_reduce_epilogue([ref[r]], np64(bias), np64(res[r]), p, 9, 4,
                                            row0[r], 0, c)
        assert_bf16_close(np64(out[r]), want, f"rank {r}")


def test_fine_fp32_inputs(ctx):
    """fp32 operands take the fp32 MFMA kernel, which runs the same chunk
    protocol on its register path."""
    import collective_overlap_amd as cce
    mode, n = "slice_lhs_rows", 4
    a, b, oshape = _inputs(mode, n, (40, 64, 72), seed=21, in_dt=torch.float32)
    flags = cce.CCE_FLAG_FUSED_PERMUTE | cce.CCE_FLAG_BIDIRECTIONAL
    outs = {}
    for fine in (0, cce.CCE_FLAG_FINE_GRAINED):
        o = [torch.full(oshape, float("nan"), device=DEV) for _ in range(n)]
        cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, o, flags=flags | fine)
        outs[fine] = o
    ctx.check_signals()
    ref = oe.einsum_reducescatter(mode, [np64(x) for x in a], [np64(x).T for x in b])
    for r in range(n):
        assert torch.equal(_ints(outs[0][r]), _ints(outs[cce.CCE_FLAG_FINE_GRAINED][r]))
        assert_f32_close(np64(outs[cce.CCE_FLAG_FINE_GRAINED][r]), ref[r], f"rank {r}")


def test_forced_give_up_is_reported_and_leaves_the_next_call_exact(ctx):
    """The first producers withhold their ready words (host-armed hook): every
    waiting consumer gives up after a few polls and writes nothing, the
    context's check reports CCE_EHIP, and the next call is exact again."""
    import collective_overlap_amd as cce
    from collective_overlap_amd import _lib
    mode, n = "slice_lhs_rows", 4
    a, b, oshape = _inputs(mode, n, (72, 128, 264), seed=31)
    flags = cce.CCE_FLAG_FUSED_PERMUTE | cce.CCE_FLAG_BIDIRECTIONAL | cce.CCE_FLAG_FINE_GRAINED
    ref = [torch.full(oshape, float("nan"), device=DEV) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, ref, flags=flags & ~cce.CCE_FLAG_FINE_GRAINED)
    ctx.check_signals()
    sentinel = 12345.0
    out = [torch.full(oshape, sentinel, device=DEV) for _ in range(n)]
    cce.cce_debug_signal_giveup(4)
    cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, out, flags=flags)
    with pytest.raises(_lib.CceError) as e:
        ctx.check_signals()
    assert e.value.status == _lib.CCE_EHIP
    # every chunk has two producers in the last launch (n even): no consumer
    # wrote, so every output keeps the sentinel
    for r in range(n):
        assert bool((out[r] == sentinel).all()), f"rank {r}: a chunk was written after a give-up"
    ctx.check_signals()               # the word was cleared
    cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, out, flags=flags)
    ctx.check_signals()
    for r in range(n):
        assert torch.equal(_ints(out[r]), _ints(ref[r])), f"rank {r}"


def test_fine_noalloc_equals_workspace_call(ctx):
    """The allocation-free entry point holds the chunk signal words in its
    static scratch: the same bits as the workspace call."""
    import collective_overlap_amd as cce
    mode, n = "slice_lhs_rows", 4
    a, b, oshape = _inputs(mode, n, (72, 256, 264), seed=41)
    bias = W.normal((oshape[1],), 0.02, 92, device=DEV, dtype=torch.bfloat16)
    res = [W.normal(oshape, 1.0, 120 + r, device=DEV, dtype=torch.bfloat16) for r in range(n)]
    row0 = [r * oshape[0] for r in range(n)]
    flags = cce.CCE_FLAG_FUSED_PERMUTE | cce.CCE_FLAG_BIDIRECTIONAL | cce.CCE_FLAG_FINE_GRAINED
    x = [torch.empty(oshape, device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    y = [torch.empty(oshape, device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter_epilogue(ctx, mode, a, b, bias, res, x, 0.1, 1, 1,
                                                 mask_row0=row0, flags=flags)
    cce.cce_looped_einsum_reducescatter_epilogue_noalloc(ctx, mode, a, b, bias, res, y, 0.1, 1, 1,
                                                         mask_row0=row0, flags=flags)
    ctx.check_signals()
    for r in range(n):
        assert torch.equal(_ints(x[r]), _ints(y[r])), f"rank {r}"
