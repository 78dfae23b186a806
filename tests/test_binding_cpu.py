"""CPU tests of the Python binding's own checks.  The C ABI takes one element
type per operand class and plain device pointers, so the binding is where a
tensor of another dtype, or one in host memory, is caught: it raises
ValueError before anything reaches the library (no GPU, no context needed)."""

import pytest
import torch

import collective_overlap_amd as cce


class _Ctx:
    """Stands in for a Context: the checks run before its handle is used."""
    device = 0
    handle = None


BF, F32 = torch.bfloat16, torch.float32


def _t(shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def test_reducescatter_epilogue_rejects_a_residual_or_bias_of_another_dtype():
    a, b = [_t((32, 64))] * 2, [_t((24, 64))] * 2
    out = [_t((16, 24), F32)] * 2
    with pytest.raises(ValueError, match="residuals"):
        cce.cce_looped_einsum_reducescatter_epilogue(_Ctx(), "slice_lhs_rows", a, b, None,
                                                     [_t((16, 24), BF)] * 2, out, 0.1)
    with pytest.raises(ValueError, match="bias"):
        cce.cce_looped_einsum_reducescatter_epilogue_noalloc(_Ctx(), "slice_lhs_rows", a, b,
                                                             _t((24,), BF), None, out, 0.1)


def test_factors_of_different_dtypes_are_rejected():
    with pytest.raises(ValueError, match="b must be"):
        cce.cce_grouped_gemm(_Ctx(), [_t((8, 16))], [_t((8, 16), F32)], [_t((8, 8), F32)])
    with pytest.raises(ValueError, match="b must be"):
        cce.cce_looped_einsum_reducescatter(_Ctx(), "slice_lhs_rows", [_t((32, 64))] * 2,
                                            [_t((24, 64), F32)] * 2, [_t((16, 24), F32)] * 2)
    with pytest.raises(ValueError, match="local operand"):
        cce.cce_looped_allgather_einsum(_Ctx(), "lhs_rows", [_t((16, 64))] * 2,
                                        [_t((24, 64), F32)] * 2, [_t((32, 24))] * 2)


def test_host_tensors_are_rejected_before_the_library_sees_them():
    """Host memory handed to a GPU kernel would fault the device: every entry
    point refuses tensors that are not on the context's GPU."""
    x = [_t((8, 16))]
    with pytest.raises(ValueError, match="cuda:0"):
        cce.cce_grouped_gemm(_Ctx(), x, x, [_t((8, 8), F32)])
    with pytest.raises(ValueError, match="cuda:0"):
        cce.cce_fused_reduce_epilogue(_Ctx(), [_t((8, 16), F32)], None, None, _t((8, 16), F32), 0.1)
    with pytest.raises(ValueError, match="cuda:0"):
        cce.cce_fused_reduce_epilogue_batched(_Ctx(), [[_t((8, 16), F32)]], None, None,
                                              [_t((8, 16), F32)], 0.1)
    with pytest.raises(ValueError, match="cuda:0"):
        cce.cce_fused_allreduce_epilogue(_Ctx(), [_t((8, 16), F32)] * 2, None, None,
                                         [_t((8, 16), F32)] * 2, 0.1)
    with pytest.raises(ValueError, match="cuda:0"):
        cce.cce_looped_allgather_einsum(_Ctx(), "lhs_rows", [_t((16, 64))] * 2,
                                        [_t((24, 64))] * 2, [_t((32, 24))] * 2)
    with pytest.raises(ValueError, match="cuda:0"):
        cce.cce_looped_einsum_reducescatter(_Ctx(), "slice_lhs_rows", [_t((32, 64))] * 2,
                                            [_t((24, 64))] * 2, [_t((16, 24), F32)] * 2)
    with pytest.raises(ValueError, match="cuda:0"):
        cce.cce_looped_einsum_reducescatter_epilogue(_Ctx(), "slice_lhs_rows", [_t((32, 64))] * 2,
                                                     [_t((24, 64))] * 2, None, None,
                                                     [_t((16, 24))] * 2, 0.1)
