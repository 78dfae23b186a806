"""Ordering of the looped calls against the caller's stream, and workspace
hygiene.

A call forks its copy stream from the caller's stream and joins it back
(every copy is ordered after the caller's earlier work and before its later
work).  The workspace holds receive buffers and accumulators that every call
writes before it reads them, so stale or poisoned bytes in it never reach a
result.  These tests delay the caller's stream with a bounded spin kernel
(torch.cuda._sleep) so that a missing fork would let the copies read inputs
that are not written yet, and they poison the workspace with all-ones bytes
(NaN in fp32 and bf16).  Inputs are integer probes, so every correct result
is exact and equal to the oracle's.  A call made to fail part-way (the
error-path hook) must return CCE_EHIP, leave nothing running that the
caller's stream does not wait for, and leave the context usable."""

import numpy as np
import pytest
import torch

from oracle import einsum as oe
import workloads as W
from gpu_util import np64, sync

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16
SLEEP = 50_000_000          # GPU cycles of the spin kernel, some tens of ms

# copy stream, DMA copies, serial, fused permute, two-way ring, both
FORMS = [0x0, 0x4, 0x1, 0x8, 0x10, 0x18]


@pytest.fixture(scope="module")
def ctx():
    import collective_overlap_amd as cce
    c = cce.Context(0)
    yield c
    sync()
    c.close()


def _probe(shape, k):
    return W.int_probe(shape, k, device=DEV, dtype=BF)


def _ag_case(n):
    # rhs_cols: looped B^T shards [c, k], local A [m, k] -> out [m, n c]
    m, k, c = 200, 264, 136
    looped = [_probe((c, k), 100 + r) for r in range(n)]
    local = [_probe((m, k), 200 + r) for r in range(n)]
    ref = oe.allgather_einsum("rhs_cols", [np64(t).T for t in looped], [np64(t) for t in local])
    out = [torch.full((m, n * c), float("nan"), device=DEV) for _ in range(n)]
    return looped, local, out, ref


def _rs_case(n):
    # slice_lhs_rows: A_r [n s, k], B^T_r [c, k] -> out_r [s, c]
    s, k, c = 136, 264, 200
    a = [_probe((n * s, k), 300 + r) for r in range(n)]
    b = [_probe((c, k), 400 + r) for r in range(n)]
    ref = oe.einsum_reducescatter("slice_lhs_rows", [np64(t) for t in a], [np64(t).T for t in b])
    out = [torch.full((s, c), float("nan"), device=DEV) for _ in range(n)]
    return a, b, out, ref


def _call(cce, ctx, kind, x, y, out, flags, stream=None, workspace=None):
    if kind == "ag":
        cce.cce_looped_allgather_einsum(ctx, "rhs_cols", x, y, out, workspace=workspace,
                                        flags=flags, stream=stream)
    else:
        cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", x, y, out,
                                            workspace=workspace, flags=flags, stream=stream)


@pytest.mark.parametrize("kind", ["ag", "rs"])
@pytest.mark.parametrize("flags", FORMS)
def test_inputs_written_behind_a_delay(ctx, kind, flags):
    """The inputs are written on the caller's stream behind a long spin; the
    call on that stream (not the current one) must see them, copies
    included, and a clone of the outputs queued after it must see the
    results."""
    import collective_overlap_amd as cce
    print(f"[gpu] ordering: inputs behind a delay, {kind} flags={flags:#x}", flush=True)
    n = 4
    x_src, y_src, out, ref = (_ag_case if kind == "ag" else _rs_case)(n)
    x = [torch.zeros_like(t) for t in x_src]
    y = [torch.zeros_like(t) for t in y_src]
    sync()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(SLEEP)
        for d, s in zip(x + y, x_src + y_src):
            d.copy_(s)
        _call(cce, ctx, kind, x, y, out, flags, stream=side)
        got = [o.clone() for o in out]
    side.synchronize()
    for r in range(n):
        assert np.array_equal(np64(got[r]), ref[r]), f"rank {r}"


@pytest.mark.parametrize("kind", ["ag", "rs"])
@pytest.mark.parametrize("flags", FORMS)
def test_poisoned_workspace(ctx, kind, flags):
    """A workspace full of NaN bytes, then reused dirty by a second call on
    other inputs: both results are exact."""
    import collective_overlap_amd as cce
    print(f"[gpu] ordering: poisoned workspace, {kind} flags={flags:#x}", flush=True)
    n = 5
    x, y, out, ref = (_ag_case if kind == "ag" else _rs_case)(n)
    if kind == "ag":
        need = cce.cce_looped_allgather_einsum_workspace(
            n, "rhs_cols", BF, torch.float32, tuple(x[0].shape), tuple(out[0].shape))
    else:
        need = cce.cce_looped_einsum_reducescatter_workspace(n, "slice_lhs_rows", tuple(out[0].shape))
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device=DEV)
    _call(cce, ctx, kind, x, y, out, flags, workspace=ws)
    sync()
    for r in range(n):
        assert np.array_equal(np64(out[r]), ref[r]), f"first call, rank {r}"
    # same workspace, left dirty by the first call; the inputs permuted
    x2, y2 = x[::-1], y[1:] + y[:1]
    if kind == "ag":
        ref2 = oe.allgather_einsum("rhs_cols", [np64(t).T for t in x2], [np64(t) for t in y2])
    else:
        ref2 = oe.einsum_reducescatter("slice_lhs_rows", [np64(t) for t in x2], [np64(t).T for t in y2])
    out2 = [torch.full_like(o, float("nan")) for o in out]
    _call(cce, ctx, kind, x2, y2, out2, flags, workspace=ws)
    sync()
    for r in range(n):
        assert np.array_equal(np64(out2[r]), ref2[r]), f"second call, rank {r}"


@pytest.mark.parametrize("kind", ["ag", "rs"])
@pytest.mark.parametrize("delay", [200_000, 2_000_000, 8_000_000])
def test_temporary_workspace_outlives_the_call(ctx, kind, delay):
    """A call on a side stream with a workspace the binding allocates: the
    workspace is released when the call returns, while the work is still
    queued.  Allocations on the current stream right after it, filled with
    NaN after a short delay, must not land in that workspace."""
    import collective_overlap_amd as cce
    print(f"[gpu] ordering: temporary workspace, {kind} delay={delay}", flush=True)
    n = 8
    x, y, out, ref = (_ag_case if kind == "ag" else _rs_case)(n)
    if kind == "ag":
        need = cce.cce_looped_allgather_einsum_workspace(
            n, "rhs_cols", BF, torch.float32, tuple(x[0].shape), tuple(out[0].shape))
    else:
        need = cce.cce_looped_einsum_reducescatter_workspace(n, "slice_lhs_rows", tuple(out[0].shape))
    sync()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(SLEEP // 10)
    _call(cce, ctx, kind, x, y, out, 0x0, stream=side)
    torch.cuda._sleep(delay)
    junk = [torch.empty(need, dtype=torch.uint8, device=DEV) for _ in range(4)]
    for j in junk:
        j.fill_(0xFF)
    side.synchronize()
    sync()
    for r in range(n):
        assert np.array_equal(np64(out[r]), ref[r]), f"rank {r}"


@pytest.mark.parametrize("kind", ["ag", "rs"])
@pytest.mark.parametrize("flags", FORMS)
def test_failed_call_joins_and_leaves_the_context_usable(ctx, kind, flags):
    """Every plan operation in turn is made to fail.  The call reports
    CCE_EHIP naming the operation; the caller's stream, synchronised, has
    nothing left pending; the workspace can be released; the next call on
    the same context gives the exact result."""
    import collective_overlap_amd as cce
    from collective_overlap_amd._lib import CceError
    print(f"[gpu] error path: {kind} flags={flags:#x}", flush=True)
    n = 3
    x, y, out, ref = (_ag_case if kind == "ag" else _rs_case)(n)
    failures = 0
    try:
        for k in range(1, 200):
            cce.cce_debug_fail_op(k)
            failed = False
            try:
                _call(cce, ctx, kind, x, y, out, flags)
            except CceError as e:
                assert e.status == 4, str(e)
                assert "injected failure" in str(e)
                failed = True
            torch.cuda.current_stream().synchronize()
            if not failed:
                break
            failures += 1
            good = [torch.full_like(o, float("nan")) for o in out]
            _call(cce, ctx, kind, x, y, good, flags)
            sync()
            for r in range(n):
                assert np.array_equal(np64(good[r]), ref[r]), f"after failure at op {k}, rank {r}"
    finally:
        cce.cce_debug_fail_op(0)
    assert failures >= 2


@pytest.mark.parametrize("kind", ["ag", "rs"])
@pytest.mark.parametrize("flags", [0x0, 0x10])
def test_caller_copy_stream(kind, flags):
    """The permute copies run on a stream the caller hands over
    (cce_ctx_set_copy_stream), with the caller's stream delayed behind a spin
    so a missing fork would read unwritten inputs; exact results, and exact
    again after the context's own copy stream is restored."""
    import collective_overlap_amd as cce
    print(f"[gpu] ordering: caller copy stream, {kind} flags={flags:#x}", flush=True)
    c = cce.Context(0)
    n = 4
    x_src, y_src, out, ref = (_ag_case if kind == "ag" else _rs_case)(n)
    x = [torch.zeros_like(t) for t in x_src]
    y = [torch.zeros_like(t) for t in y_src]
    copy_stream = torch.cuda.Stream()
    c.set_copy_stream(copy_stream)
    sync()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(SLEEP)
        for d, s in zip(x + y, x_src + y_src):
            d.copy_(s)
        _call(cce, c, kind, x, y, out, flags, stream=side)
        got = [o.clone() for o in out]
    side.synchronize()
    for r in range(n):
        assert np.array_equal(np64(got[r]), ref[r]), f"caller copy stream, rank {r}"
    c.set_copy_stream(None)
    for o in out:
        o.fill_(float("nan"))
    _call(cce, c, kind, x, y, out, flags)
    sync()
    for r in range(n):
        assert np.array_equal(np64(out[r]), ref[r]), f"own copy stream, rank {r}"
    c.close()
