"""GPU parity of the bidirectional looped einsums (Wang et al. ASPLOS'23,
Section 5.4.2; CCE_FLAG_BIDIRECTIONAL) against the CPU oracle's two-way ring
simulation, through the C ABI.  The copy-stream, serial and fused-permute
forms must agree bit for bit; integer probes must match the oracle exactly."""

import numpy as np
import pytest
import torch

from oracle import numerics, ring
from gpu_util import np64, assert_bf16_close, assert_f32_close, sync
from test_gpu_parity import _ag_inputs, _rs_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def ctx():
    import collective_overlap_amd as cce
    c = cce.Context(0)
    yield c
    sync()
    c.close()


AG = [("lhs_rows", (136, 200, 264)), ("rhs_cols", (300, 136, 200))]
RS = [("slice_lhs_rows", (200, 264, 296)), ("slice_rhs_cols", (136, 264, 200)),
      ("slice_lhs_rows", (1, 64, 40))]


def _forms(cce):
    B = cce.CCE_FLAG_BIDIRECTIONAL
    return [B, B | cce.CCE_FLAG_SERIAL, B | cce.CCE_FLAG_FUSED_PERMUTE]


@pytest.mark.parametrize("mode,dims", AG)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_bidir_allgather(ctx, mode, dims, n, out_dt):
    """Every form equals the oracle, and (case 1: each element is one dot
    product) the one-way loop bit for bit."""
    import collective_overlap_amd as cce
    print(f"[gpu] bidir allgather {mode} n={n} out={out_dt}", flush=True)
    odt = torch.bfloat16 if out_dt == "bf16" else torch.float32
    looped, local, oshape, ol, oc = _ag_inputs(mode, n, dims, torch.bfloat16, False, seed=40 + n)
    outs = []
    for flags in [0] + _forms(cce):
        out = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
        cce.cce_looped_allgather_einsum(ctx, mode, looped, local, out, flags=flags)
        outs.append(out)
    sync()
    ref, _, _ = ring.simulate_allgather_einsum_bidir(mode, ol, oc)
    for r in range(n):
        if out_dt == "bf16":
            assert_bf16_close(np64(outs[1][r]), ref[r], f"rank {r}")
        else:
            assert_f32_close(np64(outs[1][r]), ref[r], f"rank {r}")
        for k in range(2, len(outs)):
            assert torch.equal(outs[1][r], outs[k][r]), f"form {k} rank {r}"
        assert torch.equal(outs[0][r], outs[1][r]), f"one-way vs two-way rank {r}"


@pytest.mark.parametrize("mode,dims", AG)
@pytest.mark.parametrize("n", [2, 5, 16])
def test_bidir_allgather_integer_probe_and_gelu(ctx, mode, dims, n):
    import collective_overlap_amd as cce
    looped, local, oshape, ol, oc = _ag_inputs(mode, n, dims, torch.bfloat16, True, seed=3)
    out = [torch.empty(oshape, device=DEV) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, mode, looped, local, out,
                                    flags=cce.CCE_FLAG_BIDIRECTIONAL | cce.CCE_FLAG_FUSED_PERMUTE)
    g = [torch.empty(oshape, device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, mode, looped, local, g,
                                    flags=cce.CCE_FLAG_BIDIRECTIONAL | cce.CCE_FLAG_GELU)
    sync()
    ref, _, _ = ring.simulate_allgather_einsum_bidir(mode, ol, oc)
    for r in range(n):
        assert np.array_equal(np64(out[r]), ref[r]), f"rank {r}"
        assert_bf16_close(np64(g[r]), numerics.gelu(ref[r]), f"gelu rank {r}")


@pytest.mark.parametrize("mode,dims", RS)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_bidir_reducescatter(ctx, mode, dims, n, out_dt):
    import collective_overlap_amd as cce
    print(f"[gpu] bidir reducescatter {mode} n={n} dims={dims} out={out_dt}", flush=True)
    odt = torch.bfloat16 if out_dt == "bf16" else torch.float32
    a, b, oshape, oa, ob = _rs_inputs(mode, n, dims, torch.bfloat16, False, seed=50 + n)
    outs = []
    for flags in _forms(cce):
        out = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
        cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, out, flags=flags)
        outs.append(out)
    sync()
    ref, _, _ = ring.simulate_einsum_reducescatter_bidir(mode, oa, ob)
    for r in range(n):
        if out_dt == "bf16":
            assert_bf16_close(np64(outs[0][r]), ref[r], f"rank {r}")
        else:
            assert_f32_close(np64(outs[0][r]), ref[r], f"rank {r}")
        for k in range(1, len(outs)):
            assert torch.equal(outs[0][r], outs[k][r]), f"form {k} rank {r}"


@pytest.mark.parametrize("mode,dims", RS[:2])
@pytest.mark.parametrize("n", [2, 4, 7, 16])
def test_bidir_reducescatter_integer_probe_bit_exact(ctx, mode, dims, n):
    import collective_overlap_amd as cce
    a, b, oshape, oa, ob = _rs_inputs(mode, n, dims, torch.bfloat16, True, seed=6)
    for flags in _forms(cce):
        out = [torch.empty(oshape, device=DEV) for _ in range(n)]
        cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, out, flags=flags)
        sync()
        ref, _, _ = ring.simulate_einsum_reducescatter_bidir(mode, oa, ob)
        for r in range(n):
            assert np.array_equal(np64(out[r]), ref[r]), f"flags {flags} rank {r}"


def test_bidir_rejects_case2(ctx):
    import collective_overlap_amd as cce
    from collective_overlap_amd._lib import CceError
    looped, local, oshape, _, _ = _ag_inputs("lhs_cols", 2, (64, 64, 64), torch.bfloat16, False)
    out = [torch.zeros(oshape, device=DEV) for _ in range(2)]
    with pytest.raises(CceError) as e:
        cce.cce_looped_allgather_einsum(ctx, "lhs_cols", looped, local, out,
                                        flags=cce.CCE_FLAG_BIDIRECTIONAL)
    assert e.value.status == 2
    assert all(torch.count_nonzero(o) == 0 for o in out)


def test_bidir_32_ranks_integer_probe(ctx):
    """The largest two-way ring (64 groups per launch), bit-exact."""
    import collective_overlap_amd as cce
    n = 32
    for flags in _forms(cce):
        looped, local, oshape, ol, oc = _ag_inputs("lhs_rows", n, (24, 64, 40), torch.bfloat16, True, 2)
        out = [torch.empty(oshape, device=DEV) for _ in range(n)]
        cce.cce_looped_allgather_einsum(ctx, "lhs_rows", looped, local, out, flags=flags)
        a, b, rshape, oa, ob = _rs_inputs("slice_rhs_cols", n, (8, 64, 24), torch.bfloat16, True, 3)
        rout = [torch.empty(rshape, device=DEV) for _ in range(n)]
        cce.cce_looped_einsum_reducescatter(ctx, "slice_rhs_cols", a, b, rout, flags=flags)
        sync()
        ref, _, _ = ring.simulate_allgather_einsum_bidir("lhs_rows", ol, oc)
        rref, _, _ = ring.simulate_einsum_reducescatter_bidir("slice_rhs_cols", oa, ob)
        for r in range(n):
            assert np.array_equal(np64(out[r]), ref[r]), f"flags {flags} allgather rank {r}"
            assert np.array_equal(np64(rout[r]), rref[r]), f"flags {flags} reducescatter rank {r}"
