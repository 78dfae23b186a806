"""GPU parity of the looped AllGather-Einsum case 3 (Wang et al. ASPLOS'23,
Section 5.1: the looped LHS split on a batch dimension) against the CPU
oracle, through the C ABI, in every form (copy stream, serial, fused
permute, two-way ring); and of looped shards with padded rows (ld > cols),
whose receive buffers keep the caller's ld, in every form of case 1 and 3."""

import numpy as np
import pytest
import torch

from oracle import einsum as oe, numerics, ring
from gpu_util import np64, assert_bf16_close, assert_f32_close, sync
from test_gpu_parity import _t, _ag_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def ctx():
    import collective_overlap_amd as cce
    c = cce.Context(0)
    yield c
    sync()
    c.close()


def _case3_inputs(n, bs, dims, dtype, probe, seed, ld=None):
    """Stacked storage tensors and batched math-orientation oracle inputs."""
    m, k, c = dims
    looped = [_t((bs * m, k), seed + r, dtype, probe, ld) for r in range(n)]      # [b_s m, K]
    local = [_t((n * bs * c, k), seed + 100 + r, dtype, probe) for r in range(n)]  # B^T [n b_s N, K]
    o_looped = [np64(x).reshape(bs, m, k) for x in looped]
    o_local = [np64(x).reshape(n * bs, c, k).transpose(0, 2, 1) for x in local]    # [n b_s, K, N]
    return looped, local, (n * bs * m, c), o_looped, o_local


def _forms(cce):
    S, F, B = cce.CCE_FLAG_SERIAL, cce.CCE_FLAG_FUSED_PERMUTE, cce.CCE_FLAG_BIDIRECTIONAL
    return [0, S, F, B, B | S, B | F]


@pytest.mark.parametrize("dims", [(72, 136, 264), (256, 256, 256)])
@pytest.mark.parametrize("n,bs", [(1, 2), (2, 1), (2, 3), (3, 2), (4, 3)])
@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_case3_every_form(ctx, dims, n, bs, out_dt):
    """Every form equals the oracle's definition; each output element is one
    dot product, so all forms agree bit for bit."""
    import collective_overlap_amd as cce
    print(f"[gpu] case 3 n={n} b_s={bs} dims={dims} out={out_dt}", flush=True)
    odt = torch.bfloat16 if out_dt == "bf16" else torch.float32
    looped, local, oshape, ol, oc = _case3_inputs(n, bs, dims, torch.bfloat16, False, 60 + n)
    outs = []
    for flags in _forms(cce):
        out = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
        cce.cce_looped_allgather_einsum(ctx, "lhs_batch", looped, local, out, flags=flags)
        outs.append(out)
    sync()
    ref = oe.allgather_einsum("lhs_batch", ol, oc)
    for r in range(n):
        want = ref[r].reshape(oshape)
        if out_dt == "bf16":
            assert_bf16_close(np64(outs[0][r]), want, f"rank {r}")
        else:
            assert_f32_close(np64(outs[0][r]), want, f"rank {r}")
        for k in range(1, len(outs)):
            assert torch.equal(outs[0][r], outs[k][r]), f"form {k} rank {r}"


@pytest.mark.parametrize("n,bs", [(2, 2), (5, 3), (8, 4)])
def test_case3_integer_probe_and_gelu(ctx, n, bs):
    """Exact-integer inputs: bit-equal to the oracle's loop simulation, in
    the benchmark-like form (fused permute, two-way ring); GELU on the store."""
    import collective_overlap_amd as cce
    dims = (40, 64, 48)
    looped, local, oshape, ol, oc = _case3_inputs(n, bs, dims, torch.bfloat16, True, 5)
    out = [torch.empty(oshape, device=DEV) for _ in range(n)]
    flags = cce.CCE_FLAG_FUSED_PERMUTE | cce.CCE_FLAG_BIDIRECTIONAL
    cce.cce_looped_allgather_einsum(ctx, "lhs_batch", looped, local, out, flags=flags)
    g = [torch.empty(oshape, device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, "lhs_batch", looped, local, g, flags=cce.CCE_FLAG_GELU)
    sync()
    ref, sched, _ = ring.simulate_allgather_einsum("lhs_batch", ol, oc)
    for r in range(n):
        want = ref[r].reshape(oshape)
        assert np.array_equal(np64(out[r]), want), f"rank {r}"
        assert_bf16_close(np64(g[r]), numerics.gelu(want), f"gelu rank {r}")


def test_case3_rejects(ctx):
    import collective_overlap_amd as cce
    from collective_overlap_amd._lib import CceError
    n, bs, dims = 8, 5, (16, 64, 16)
    looped, local, oshape, _, _ = _case3_inputs(n, bs, dims, torch.bfloat16, False, 1)
    out = [torch.empty(oshape, device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, "lhs_batch", looped, local, out)   # 40 groups: fine
    with pytest.raises(CceError):      # two-way: 80 groups > CCE_MAX_RANKS
        cce.cce_looped_allgather_einsum(ctx, "lhs_batch", looped, local, out,
                                        flags=cce.CCE_FLAG_BIDIRECTIONAL)
    bad = [x[:-16] for x in local]     # local rows not n * b_s * out cols
    with pytest.raises(CceError):
        cce.cce_looped_allgather_einsum(ctx, "lhs_batch", looped, bad, out)
    sync()


# ---------------------------------------------------------------------------
# looped shards with padded rows
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["lhs_rows", "rhs_cols", "lhs_batch"])
@pytest.mark.parametrize("n", [2, 3, 4])
def test_padded_looped_shards_every_form(ctx, mode, n):
    """The looped shards have ld = K + 64: receive buffers take the same ld,
    so a launch that mixes a caller's shard with a received one (iteration 0
    of the two-way form) reads both right; all forms equal the oracle."""
    import collective_overlap_amd as cce
    print(f"[gpu] padded looped shards {mode} n={n}", flush=True)
    k = 136
    if mode == "lhs_batch":
        looped, local, oshape, ol, oc = _case3_inputs(n, 2, (40, k, 72), torch.bfloat16, True, 7,
                                                      ld=k + 64)
        ref = [x.reshape(oshape) for x in oe.allgather_einsum(mode, ol, oc)]
    else:
        dims = (72, k, 96)
        looped, local, oshape, ol, oc = _ag_inputs(mode, n, dims, torch.bfloat16, True, seed=9)
        # the same values with padded rows
        looped = [torch.cat([x, torch.zeros((x.shape[0], 64), device=DEV, dtype=x.dtype)], 1)[:, :k]
                  for x in looped]
        ref = oe.allgather_einsum(mode, ol, oc)
    assert looped[0].stride(0) == k + 64
    for flags in _forms(cce):
        out = [torch.full(oshape, float("nan"), device=DEV) for _ in range(n)]
        cce.cce_looped_allgather_einsum(ctx, mode, looped, local, out, flags=flags)
        sync()
        for r in range(n):
            assert np.array_equal(np64(out[r]), ref[r]), f"flags {flags} rank {r}"
