"""The backward pass of a looped AllGather-Einsum through the same C ABI
(Wang et al. ASPLOS'23, Section 2.2: in the backward pass the weight
AllGather becomes a ReduceScatter that yields each device's partition of the
weight gradient).  Forward: Y_r = A_r @ concat_cols(B_s) (AllGather-Einsum,
case 1).  Backward: dB_s by the looped Einsum-ReduceScatter, dA_r by the
looped AllGather-Einsum with the contraction split (case 2).  Compared with
the oracle's gradients, which are pinned to torch autograd on the CPU."""

import numpy as np
import pytest
import torch

from oracle import einsum as oe
import workloads as W
from gpu_util import np64, assert_f32_close, sync

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def ctx():
    import collective_overlap_amd as cce
    c = cce.Context(0)
    yield c
    sync()
    c.close()


def _t(shape, k, probe):
    if probe:
        return W.int_probe(shape, k, device=DEV, dtype=torch.bfloat16)
    return W.normal(shape, 1.0, k, device=DEV, dtype=torch.bfloat16)


@pytest.mark.parametrize("n,probe", [(2, True), (4, True), (4, False), (3, False)])
@pytest.mark.parametrize("flags", [0, 0x8, 0x10])
def test_allgather_einsum_forward_and_backward(ctx, n, probe, flags):
    import collective_overlap_amd as cce
    M, K, ns = 200, 264, 136
    print(f"[gpu] backward duality n={n} probe={probe} flags={flags}", flush=True)
    Bt = [_t((ns, K), 10 + s, probe) for s in range(n)]        # B_s^T [n_s, K]
    A = [_t((M, K), 20 + r, probe) for r in range(n)]          # A_r [M, K]
    dY = [_t((M, n * ns), 30 + r, probe) for r in range(n)]    # dL/dY_r [M, n n_s]
    Y = [torch.empty((M, n * ns), device=DEV) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, "rhs_cols", Bt, A, Y, flags=flags)
    # dB_s [K, n_s] = sum_r (A_r^T dY_r)[:, s]: Einsum-ReduceScatter over
    # a_r = A_r^T [K, M] and b_r^T = dY_r^T [n n_s, M]
    At = [a.t().contiguous() for a in A]
    dYt = [d.t().contiguous() for d in dY]
    dB = [torch.empty((K, ns), device=DEV) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, "slice_rhs_cols", At, dYt, dB, flags=flags & 0x18)
    # dA_r [M, K] = dY_r @ concat_cols(B_s)^T: AllGather-Einsum, case 2, with
    # looped shards B_s stored [K, n_s] and local dY_r [M, n n_s]
    Bs = [b.t().contiguous() for b in Bt]
    dA = [torch.empty((M, K), device=DEV) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, "rhs_rows", Bs, dY, dA, flags=flags & 0x8)
    sync()
    looped = [np64(b).T for b in Bt]
    local = [np64(a) for a in A]
    ys = oe.allgather_einsum("rhs_cols", looped, local)
    d_looped, d_local = oe.allgather_einsum_backward("rhs_cols", looped, local,
                                                     [np64(d) for d in dY])
    for r in range(n):
        for got, ref, what in ((Y[r], ys[r], "Y"), (dB[r], d_looped[r], "dB"),
                               (dA[r], d_local[r], "dA")):
            if probe:
                assert np.array_equal(np64(got), ref), f"{what} rank {r}"
            else:
                assert_f32_close(np64(got), ref, f"{what} rank {r}")
