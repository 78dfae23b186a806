"""GPU parity of the fused reduce epilogue: keep masks bit-exact against the
oracle's Philox, values against the float64 oracle, and bit for bit against
the oracle's float32 evaluation in the library's fixed order (the sum in
partial order, + bias, x scale if kept, + residual, one rounding per step, no
fused multiply-add)."""

import numpy as np
import pytest
import torch

from oracle import epilogue as oep
from oracle import numerics
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


def assert_bits_fp32_order(out, parts, bias, res, p, seed, off, r0, c0, mld, what):
    """out (fp32 or bf16 tensor) equals the float32-order oracle bit for bit
    (bf16: that value rounded to nearest even once more)."""
    ref32, _ = oep.fused_reduce_epilogue_fp32(
        [np64(x) for x in parts], None if bias is None else np64(bias),
        None if res is None else np64(res), p, seed, off, r0, c0, mld)
    if out.dtype == torch.bfloat16:
        ref32 = numerics.bf16_round(ref32)
    got = out.float().cpu().numpy()
    bad = got.view(np.uint32) != np.ascontiguousarray(ref32).view(np.uint32)
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements differ from the float32-order "
                           f"oracle, first at {np.argwhere(bad)[0].tolist()}")


def _mk(shape, k, dtype, ld=None):
    rows, cols = shape
    x = W.normal((rows, ld or cols), 1.0, k, device=DEV, dtype=dtype)
    return x[:, :cols] if ld else x


CASES = [
    # rows, cols, ld, n, part, out, p, seed, offset, row0, col0, mask_ld
    (100, 264, None, 2, "f32", "f32", 0.1, 0, 0, 0, 0, None),
    (64, 256, None, 2, "f32", "f32", 0.1, 0, 0, 0, 0, None),
    (257, 512, None, 8, "bf16", "bf16", 0.1, 1234, 5, 0, 0, None),
    (33, 261, 272, 3, "bf16", "bf16", 0.3, 7, 9, 4, 8, 400),
    (40, 96, None, 1, "f32", "bf16", 0.1, 99, 0, 1024, 0, 96),
    (17, 88, None, 5, "f32", "f32", 0.5, 3, 2, 2, 3, 97),         # misaligned mask index
    (20, 64, None, 2, "bf16", "bf16", 0.0, 0, 0, 0, 0, None),
    (20, 64, None, 2, "f32", "f32", 1.0, 0, 0, 0, 0, None),
    (9, 8, None, 64, "f32", "f32", 0.2, 11, 1, 0, 0, None),
]


@pytest.mark.parametrize("case", CASES)
def test_fused_epilogue(ctx, case):
    import collective_overlap_amd as cce
    rows, cols, ld, n, pt, ot, p, seed, off, r0, c0, mld = case
    print(f"[gpu] epilogue {case}", flush=True)
    pdt = torch.float32 if pt == "f32" else torch.bfloat16
    odt = torch.float32 if ot == "f32" else torch.bfloat16
    parts = [_mk((rows, cols), 10 + k, pdt, ld) for k in range(n)]
    bias = W.normal((cols,), 0.02, 90, device=DEV, dtype=odt)
    res = _mk((rows, cols), 91, odt, ld)
    out_full = torch.full((rows, ld or cols), float("nan"), device=DEV, dtype=odt)
    out = out_full[:, :cols]
    mask = torch.full((rows, cols), 7, device=DEV, dtype=torch.uint8)
    cce.cce_fused_reduce_epilogue(ctx, parts, bias, res, out, p, seed, off, r0, c0, mld,
                                  mask_out=mask)
    sync()
    ref, keep = oep.fused_reduce_epilogue([np64(x) for x in parts], np64(bias), np64(res), p,
                                          seed, off, r0, c0, mld if mld else c0 + cols)
    assert np.array_equal(mask.cpu().numpy().astype(bool), keep), "keep mask differs"
    assert set(np.unique(mask.cpu().numpy())) <= {0, 1}
    if ot == "f32":
        assert_f32_close(np64(out), ref, "epilogue", tol=1e-6)
    else:
        assert_bf16_close(np64(out), ref, "epilogue")
    assert_bits_fp32_order(out, parts, bias, res, p, seed, off, r0, c0, mld if mld else c0 + cols,
                           "epilogue")
    if ld:
        assert torch.isnan(out_full[:, cols:].float()).all()    # padding untouched


def test_no_bias_no_residual(ctx):
    import collective_overlap_amd as cce
    parts = [_mk((32, 128), 1 + k, torch.float32) for k in range(2)]
    out = torch.empty((32, 128), device=DEV)
    cce.cce_fused_reduce_epilogue(ctx, parts, None, None, out, 0.25, 5, 6)
    sync()
    ref, _ = oep.fused_reduce_epilogue([np64(x) for x in parts], None, None, 0.25, 5, 6)
    assert_f32_close(np64(out), ref, "no bias/residual", tol=1e-6)


@pytest.mark.parametrize("kernel", ["vector", "general"])
def test_order_and_no_fused_multiply_add(ctx, kernel):
    """Hand-worked elements on which another order of the sum, or a fused
    multiply-add, gives a different result (the cases of the oracle's own
    float32 pins), through the library.  Asking for the mask output selects
    the general kernel."""
    import collective_overlap_amd as cce
    from test_oracle_epilogue import no_fma_case
    cols = 64
    mk = (lambda r: {"mask_out": torch.empty((r, cols), device=DEV, dtype=torch.uint8)}
          if kernel == "general" else {})
    big = float(2 ** 25)
    # p = 0, two partials and a bias: (2^25 + -2^25) + 1 = 1 in this order,
    # 2^25 + (-2^25 + 1) = 0 in the other (-2^25 + 1 rounds to -2^25)
    parts = [torch.zeros((2, cols), device=DEV) for _ in range(2)]
    parts[0][0, 0], parts[1][0, 0] = big, -big
    bias = torch.zeros((cols,), device=DEV)
    bias[0] = 1.0
    out = torch.full((2, cols), float("nan"), device=DEV)
    cce.cce_fused_reduce_epilogue(ctx, parts, bias, None, out, 0.0, 0, 0, **mk(2))
    sync()
    assert out[0, 0].item() == 1.0
    assert_bits_fp32_order(out, parts, bias, None, 0.0, 0, 0, 0, 0, cols, "bias order")
    # p = 0, three partials (the general kernel takes any call with more than
    # two): columns 0 and 1 hold the two orders of 2^25, 1, -2^25
    parts = [torch.zeros((2, cols), device=DEV) for _ in range(3)]
    for k, v in enumerate((big, 1.0, -big)):
        parts[k][0, 0] = v
    for k, v in enumerate((big, -big, 1.0)):
        parts[k][0, 1] = v
    out = torch.full((2, cols), float("nan"), device=DEV)
    cce.cce_fused_reduce_epilogue(ctx, parts, None, None, out, 0.0, 0, 0, **mk(2))
    sync()
    assert out[0, 0].item() == 0.0 and out[0, 1].item() == 1.0
    assert_bits_fp32_order(out, parts, None, None, 0.0, 0, 0, 0, 0, cols, "sum order")
    # p = 0.1: a kept element whose residual cancels the rounded product
    e, s_, r, fma = no_fma_case(cols=cols)
    part = torch.zeros((1, cols), device=DEV)
    part[0, e] = float(s_)
    res = torch.zeros((1, cols), device=DEV)
    res[0, e] = float(r)
    out = torch.full((1, cols), float("nan"), device=DEV)
    cce.cce_fused_reduce_epilogue(ctx, [part], None, res, out, 0.1, 0, 0, **mk(1))
    sync()
    assert out[0, e].item() == 0.0, f"got {out[0, e].item()!r}; a fused multiply-add gives {fma!r}"
    assert_bits_fp32_order(out, [part], None, res, 0.1, 0, 0, 0, 0, cols, "no fma")


def test_keep_rate_full_size_mask(ctx):
    """p = 0.1 over 8192 x 8192: keep count within 6 sigma of the binomial."""
    import collective_overlap_amd as cce
    rows = cols = 8192
    part = torch.zeros((rows, cols), device=DEV, dtype=torch.bfloat16)
    out = torch.empty_like(part)
    mask = torch.empty((rows, cols), device=DEV, dtype=torch.uint8)
    cce.cce_fused_reduce_epilogue(ctx, [part], None, None, out, 0.1, 0, 0, mask_out=mask)
    kept = int(mask.sum(dtype=torch.int64).item())
    n = rows * cols
    assert abs(kept - 0.9 * n) < 6 * (n * 0.09) ** 0.5
    # sampled rows against the oracle's mask
    from oracle import philox
    for r in (0, 1, 4095, 8191):
        want = philox.keep_mask(1, cols, 0.1, 0, 0, row0=r, col0=0, ld=cols)[0]
        assert np.array_equal(mask[r].cpu().numpy().astype(bool), want)


BATCHED = [
    # n_batch, n_partials, rows, cols, ld, part, out, p, seed, offset, mask_ld
    (3, 2, 45, 264, None, "bf16", "bf16", 0.1, 17, 3, 264),
    (8, 1, 16, 96, None, "f32", "bf16", 0.1, 0, 0, 96),
    (4, 3, 9, 61, 64, "f32", "f32", 0.4, 5, 1, 61),      # ragged columns, odd mask index
    (2, 32, 7, 40, None, "bf16", "f32", 0.2, 8, 0, 40),  # n_batch * n_partials == 64
]


@pytest.mark.parametrize("case", BATCHED)
def test_batched_equals_single_calls_and_oracle(ctx, case):
    """One batched launch gives, bit for bit, what n_batch single calls give,
    and each output matches the oracle (mask bit-exact) with its own row base."""
    import collective_overlap_amd as cce
    nb, n, rows, cols, ld, pt, ot, p, seed, off, mld = case
    print(f"[gpu] batched epilogue {case}", flush=True)
    pdt = torch.float32 if pt == "f32" else torch.bfloat16
    odt = torch.float32 if ot == "f32" else torch.bfloat16
    parts = [[_mk((rows, cols), 100 + 10 * b + k, pdt, ld) for k in range(n)] for b in range(nb)]
    bias = W.normal((cols,), 0.02, 90, device=DEV, dtype=odt)
    res = [_mk((rows, cols), 200 + b, odt, ld) for b in range(nb)]
    row0 = [b * rows for b in range(nb)]
    outs = [torch.full((rows, ld or cols), float("nan"), device=DEV, dtype=odt)[:, :cols]
            for _ in range(nb)]
    masks = [torch.full((rows, cols), 7, device=DEV, dtype=torch.uint8) for _ in range(nb)]
    cce.cce_fused_reduce_epilogue_batched(ctx, parts, bias, res, outs, p, seed, off,
                                          mask_row0=row0, mask_col0=0, mask_ld=mld,
                                          mask_outs=masks)
    single = [torch.empty((rows, ld or cols), device=DEV, dtype=odt)[:, :cols] for _ in range(nb)]
    for b in range(nb):
        cce.cce_fused_reduce_epilogue(ctx, parts[b], bias, res[b], single[b], p, seed, off,
                                      row0[b], 0, mld)
    sync()
    for b in range(nb):
        it = torch.int16 if odt == torch.bfloat16 else torch.int32
        assert torch.equal(outs[b].contiguous().view(it), single[b].contiguous().view(it))
        ref, keep = oep.fused_reduce_epilogue([np64(x) for x in parts[b]], np64(bias),
                                              np64(res[b]), p, seed, off, row0[b], 0, mld)
        assert np.array_equal(masks[b].cpu().numpy().astype(bool), keep), f"mask {b}"
        if ot == "f32":
            assert_f32_close(np64(outs[b]), ref, f"batched {b}", tol=1e-6)
        else:
            assert_bf16_close(np64(outs[b]), ref, f"batched {b}")
        assert_bits_fp32_order(outs[b], parts[b], bias, res[b], p, seed, off, row0[b], 0, mld,
                               f"batched {b}")


def test_batched_rejects_too_many_operands(ctx):
    import collective_overlap_amd as cce
    parts = [[torch.zeros((4, 8), device=DEV) for _ in range(33)] for _ in range(2)]
    outs = [torch.empty((4, 8), device=DEV) for _ in range(2)]
    with pytest.raises(RuntimeError):
        cce.cce_fused_reduce_epilogue_batched(ctx, parts, None, None, outs, 0.0)


ALLREDUCE = [
    # n, rows, cols, ld, part, out, p, seed, offset
    (8, 130, 512, None, "bf16", "bf16", 0.1, 3, 0),
    (4, 33, 261, 272, "f32", "bf16", 0.2, 1, 7),
    (2, 64, 96, None, "f32", "f32", 0.0, 0, 0),
    (1, 17, 40, None, "bf16", "f32", 0.5, 2, 1),
]


@pytest.mark.parametrize("case", ALLREDUCE)
def test_fused_allreduce(ctx, case):
    """Every rank's replica equals the oracle's step-by-step FusedAllReduce
    (ReduceScatter, epilogue per slice, AllGather), and, bit for bit, the
    single-output fused epilogue of the same partials."""
    import collective_overlap_amd as cce
    n, rows, cols, ld, pt, ot, p, seed, off = case
    print(f"[gpu] fused allreduce {case}", flush=True)
    pdt = torch.float32 if pt == "f32" else torch.bfloat16
    odt = torch.float32 if ot == "f32" else torch.bfloat16
    parts = [_mk((rows, cols), 300 + r, pdt, ld) for r in range(n)]
    bias = W.normal((cols,), 0.02, 90, device=DEV, dtype=odt)
    res = _mk((rows, cols), 91, odt, ld)
    outs = [torch.full((rows, ld or cols), float("nan"), device=DEV, dtype=odt)[:, :cols]
            for _ in range(n)]
    mask = torch.full((rows, cols), 7, device=DEV, dtype=torch.uint8)
    cce.cce_fused_allreduce_epilogue(ctx, parts, bias, res, outs, p, seed, off, mask_out=mask)
    single = torch.empty((rows, ld or cols), device=DEV, dtype=odt)[:, :cols]
    cce.cce_fused_reduce_epilogue(ctx, parts, bias, res, single, p, seed, off)
    sync()
    ref, keep = oep.fused_allreduce([np64(x) for x in parts], np64(bias), np64(res), p, seed, off)
    assert np.array_equal(mask.cpu().numpy().astype(bool), keep)
    it = torch.int16 if odt == torch.bfloat16 else torch.int32
    for r in range(n):
        assert torch.equal(outs[r].contiguous().view(it), single.contiguous().view(it)), f"rank {r}"
        if ot == "f32":
            assert_f32_close(np64(outs[r]), ref[r], f"rank {r}", tol=1e-6)
        else:
            assert_bf16_close(np64(outs[r]), ref[r], f"rank {r}")


VECTOR = [
    # rows, cols, n, part, out, p, bias, residual, row0, col0, mask_ld
    (64, 512, 1, "f32", "bf16", 0.1, True, True, 0, 0, None),
    (33, 264, 2, "f32", "f32", 0.3, True, False, 0, 0, None),
    (40, 1024, 8, "bf16", "bf16", 0.1, True, True, 0, 0, None),     # general kernel both ways
    (17, 96, 2, "bf16", "f32", 1.0, False, True, 0, 0, None),
    (17, 96, 2, "bf16", "bf16", 0.0, True, True, 0, 0, None),
    (9, 2056, 1, "bf16", "bf16", 0.5, True, True, 7, 4, 3000),
    (65600, 8, 1, "f32", "f32", 0.1, True, True, 0, 0, None),   # more rows than one grid row each
]


@pytest.mark.parametrize("case", VECTOR)
def test_vector_kernel_equals_general_kernel(ctx, case):
    """Calls without a mask output take the vector kernel (one or two
    partials, whole 8-column vectors, aligned mask index, at most 65535 rows);
    asking for the mask forces the general kernel.  Both give the same bits,
    and the oracle's values."""
    import collective_overlap_amd as cce
    rows, cols, n, pt, ot, p, has_b, has_r, r0, c0, mld = case
    print(f"[gpu] vector epilogue {case}", flush=True)
    pdt = torch.float32 if pt == "f32" else torch.bfloat16
    odt = torch.float32 if ot == "f32" else torch.bfloat16
    parts = [_mk((rows, cols), 400 + k, pdt) for k in range(n)]
    bias = W.normal((cols,), 0.02, 90, device=DEV, dtype=odt) if has_b else None
    res = _mk((rows, cols), 91, odt) if has_r else None
    fast = torch.full((rows, cols), float("nan"), device=DEV, dtype=odt)
    gen = torch.full((rows, cols), float("nan"), device=DEV, dtype=odt)
    mask = torch.empty((rows, cols), device=DEV, dtype=torch.uint8)
    cce.cce_fused_reduce_epilogue(ctx, parts, bias, res, fast, p, 3, 1, r0, c0, mld)
    cce.cce_fused_reduce_epilogue(ctx, parts, bias, res, gen, p, 3, 1, r0, c0, mld, mask_out=mask)
    sync()
    it = torch.int16 if odt == torch.bfloat16 else torch.int32
    assert torch.equal(fast.view(it), gen.view(it))
    ref, keep = oep.fused_reduce_epilogue([np64(x) for x in parts],
                                          np64(bias) if has_b else None,
                                          np64(res) if has_r else None, p, 3, 1, r0, c0,
                                          mld if mld else c0 + cols)
    assert np.array_equal(mask.cpu().numpy().astype(bool), keep)
    if ot == "f32":
        assert_f32_close(np64(fast), ref, "vector epilogue", tol=1e-6)
    else:
        assert_bf16_close(np64(fast), ref, "vector epilogue")
    assert_bits_fp32_order(fast, parts, bias, res, p, 3, 1, r0, c0, mld if mld else c0 + cols,
                           "vector epilogue")


def test_vector_kernel_replicas(ctx):
    """FusedAllReduce without a mask output (vector kernel, every replica
    stored) against the same call with one (general kernel)."""
    import collective_overlap_amd as cce
    n, rows, cols = 2, 96, 1024
    parts = [_mk((rows, cols), 500 + r, torch.bfloat16) for r in range(n)]
    bias = W.normal((cols,), 0.02, 90, device=DEV, dtype=torch.bfloat16)
    res = _mk((rows, cols), 91, torch.bfloat16)
    fast = [torch.full((rows, cols), float("nan"), device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    gen = [torch.full((rows, cols), float("nan"), device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    mask = torch.empty((rows, cols), device=DEV, dtype=torch.uint8)
    cce.cce_fused_allreduce_epilogue(ctx, parts, bias, res, fast, 0.1, 4, 2)
    cce.cce_fused_allreduce_epilogue(ctx, parts, bias, res, gen, 0.1, 4, 2, mask_out=mask)
    sync()
    for r in range(n):
        assert torch.equal(fast[r].view(torch.int16), gen[r].view(torch.int16)), f"replica {r}"
