"""Thin Python binding over the C ABI: torch tensors in, raw pointers out.

Every function here only marshals arguments (pointers, extents, leading
dimensions, the current stream) and calls the function of the same name in
libcce.so; all computation runs in the library's HIP kernels.  torch is used
for device memory and streams only.

Layout reminder (see include/cce.h): a product is A * B^T with A [M, K] and
B^T [N, K] both row-major; tensors must be 2-D with unit column stride.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (CCE_BF16, CCE_F32, CCE_FLAG_BIDIRECTIONAL, CCE_FLAG_COPY_DMA,
                   CCE_FLAG_FINE_GRAINED, CCE_FLAG_FUSED_PERMUTE, CCE_FLAG_GELU,
                   CCE_FLAG_ONE_CHAIN, CCE_FLAG_SERIAL,
                   AG_MODES, RS_MODES,
                   cce_mat, check, lib, ptr_array)

__all__ = [
    "Context", "cce_shard_schedule", "cce_looped_allgather_einsum",
    "cce_looped_allgather_einsum_workspace", "cce_looped_einsum_reducescatter",
    "cce_looped_einsum_reducescatter_workspace", "cce_looped_einsum_reducescatter_epilogue",
    "cce_looped_einsum_reducescatter_epilogue_noalloc", "cce_grouped_gemm",
    "cce_fused_reduce_epilogue", "cce_fused_reduce_epilogue_batched",
    "cce_fused_allreduce_epilogue", "cce_describe_plan", "cce_debug_fail_op",
    "cce_debug_signal_giveup", "cce_version",
    "CCE_FLAG_SERIAL", "CCE_FLAG_GELU", "CCE_FLAG_COPY_DMA", "CCE_FLAG_FUSED_PERMUTE",
    "CCE_FLAG_BIDIRECTIONAL", "CCE_FLAG_FINE_GRAINED", "CCE_FLAG_ONE_CHAIN",
    "AG_MODES", "RS_MODES",
]

_DT = {torch.float32: CCE_F32, torch.bfloat16: CCE_BF16}
_DT_NAME = {"f32": CCE_F32, "bf16": CCE_BF16, "fp32": CCE_F32}


def _dtype(x) -> int:
    if isinstance(x, torch.dtype):
        if x not in _DT:
            raise TypeError(f"unsupported dtype {x}")
        return _DT[x]
    if isinstance(x, str):
        return _DT_NAME[x]
    return int(x)


def _mat(t: torch.Tensor) -> cce_mat:
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("tensor must have unit column stride")
    if t.shape[1] == 0:
        ld = 0                                   # empty rows: no element is addressed
    elif t.shape[0] > 1:
        ld = t.stride(0)
    else:
        ld = max(t.shape[1], t.stride(0))
    return cce_mat(t.shape[0], t.shape[1], ld)


def _same(ts, what):
    m0 = _mat(ts[0])
    for t in ts[1:]:
        m = _mat(t)
        if (m.rows, m.cols, m.ld) != (m0.rows, m0.cols, m0.ld) or t.dtype != ts[0].dtype:
            raise ValueError(f"all {what} tensors must share shape, stride and dtype")
    return m0


def _dtype_is(ts, dtype, what):
    """Every tensor of `ts` (None entries skipped) has `dtype`: the C ABI takes
    one element type for these operands and reads them as that type."""
    for t in ts:
        if t is not None and t.dtype != dtype:
            raise ValueError(f"{what} must be {dtype} here, got {t.dtype}")


def _on_device(ctx, ts):
    """Every tensor of `ts` (None entries skipped) lives on the context's GPU:
    the library dereferences each pointer on that device."""
    dev = getattr(ctx, "device", None)
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or (dev is not None and t.device.index != dev):
            raise ValueError(f"every tensor must be on cuda:{dev}, got one on {t.device}")


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class Context:
    """Owns a cce_ctx (copy stream + event pool) on one device."""

    def __init__(self, device: int | torch.device = 0):
        if isinstance(device, torch.device):
            device = device.index or 0
        self.device = int(device)
        self._h = ctypes.c_void_p()
        check(lib().cce_ctx_create(self.device, ctypes.byref(self._h)), "cce_ctx_create")

    @property
    def handle(self):
        return self._h

    def set_profiling(self, enable: bool = True):
        """Bracket every kernel / permute step with timing events."""
        check(lib().cce_ctx_set_profiling(self._h, 1 if enable else 0), "cce_ctx_set_profiling")

    def read_profile(self, max_records: int = 65536) -> list[dict]:
        """Wait for the recorded events; return and clear the records."""
        recs = (_lib.cce_prof_record * max_records)()
        n = ctypes.c_int()
        check(lib().cce_ctx_read_profile(self._h, max_records, recs, ctypes.byref(n)),
              "cce_ctx_read_profile")
        kinds = {0: "gemm", 1: "copy", 2: "epilogue"}
        return [dict(kind=kinds.get(r.kind, str(r.kind)), iter=r.iter, ms=r.ms, flops=r.flops,
                     bytes=r.bytes) for r in recs[:n.value]]

    def set_copy_stream(self, stream=None):
        """Run the permute copies of this context's looped calls on `stream`
        (a torch.cuda.Stream or a hipStream_t handle); None restores the
        context's own copy stream.  The caller keeps the stream alive."""
        h = None if stream is None else (stream.cuda_stream if hasattr(stream, "cuda_stream")
                                         else int(stream))
        self._copy_stream = stream
        check(lib().cce_ctx_set_copy_stream(self._h, h), "cce_ctx_set_copy_stream")

    def check_signals(self, stream=None):
        """Wait for `stream` (default: the current one), then raise CceError
        (CCE_EHIP) if a fine-grained chunk consumer gave up waiting since the
        last check; clears the count."""
        check(lib().cce_ctx_check_signals(self._h, _stream(stream, self.device)),
              "cce_ctx_check_signals")

    def close(self):
        if self._h:
            lib().cce_ctx_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cce_version() -> str:
    return lib().cce_version().decode()


def cce_shard_schedule(n_ranks: int, kind: int) -> list[list]:
    """table[i][r]: shard ID rank r works on in iteration i (kind 0
    AllGather, 1 ReduceScatter); for the bidirectional kinds 2 / 3 a pair
    (clockwise shard, counter-clockwise shard or None)."""
    if kind in (2, 3):
        iters = (n_ranks + 1) // 2
        buf = (ctypes.c_int32 * (iters * n_ranks * 2))()
        check(lib().cce_shard_schedule(n_ranks, kind, buf), "cce_shard_schedule")
        cell = lambda v: None if v < 0 else v    # noqa: E731
        return [[(buf[(i * n_ranks + r) * 2], cell(buf[(i * n_ranks + r) * 2 + 1]))
                 for r in range(n_ranks)] for i in range(iters)]
    buf = (ctypes.c_int32 * (n_ranks * n_ranks))()
    check(lib().cce_shard_schedule(n_ranks, kind, buf), "cce_shard_schedule")
    return [[buf[i * n_ranks + r] for r in range(n_ranks)] for i in range(n_ranks)]


def cce_describe_plan(kind: int, n_ranks: int, mode: int, out_dtype=CCE_BF16, flags: int = 0) -> str:
    need = ctypes.c_size_t()
    check(lib().cce_describe_plan(kind, n_ranks, mode, _dtype(out_dtype), flags, None, 0,
                                  ctypes.byref(need)), "cce_describe_plan")
    buf = ctypes.create_string_buffer(need.value)
    check(lib().cce_describe_plan(kind, n_ranks, mode, _dtype(out_dtype), flags, buf, need.value,
                                  ctypes.byref(need)), "cce_describe_plan")
    return buf.value.decode()


def cce_debug_fail_op(index: int) -> None:
    """Error-path test hook: plan operation `index` (1-based) of the next
    looped call on this thread fails as a HIP error would; 0 disarms."""
    check(lib().cce_debug_fail_op(int(index)), "cce_debug_fail_op")


def cce_debug_signal_giveup(polls: int) -> None:
    """Test hook of the fine-grained overlap: in the next CCE_FLAG_FINE_GRAINED
    call on this thread the first producers withhold their ready words and
    every waiting consumer gives up after at most `polls` polls; 0 disarms."""
    check(lib().cce_debug_signal_giveup(int(polls)), "cce_debug_signal_giveup")


def cce_looped_allgather_einsum_workspace(n_ranks, mode, in_dtype, out_dtype, looped_shape,
                                          out_shape) -> int:
    """looped_shape/out_shape: (rows, cols[, ld])."""
    def m(s):
        return cce_mat(s[0], s[1], s[2] if len(s) > 2 else s[1])
    nb = ctypes.c_size_t()
    mode = AG_MODES[mode] if isinstance(mode, str) else mode
    check(lib().cce_looped_allgather_einsum_workspace(n_ranks, mode, _dtype(in_dtype),
                                                      _dtype(out_dtype), m(looped_shape),
                                                      m(out_shape), ctypes.byref(nb)),
          "cce_looped_allgather_einsum_workspace")
    return nb.value


def _torch_stream(stream, device):
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _workspace(need, device, workspace, stream=None):
    """The caller's workspace (the library checks its size), or a temporary
    one of need() bytes.  A temporary one is freed when the call returns,
    while the work that uses it may still be queued on `stream` (the copy
    stream joins back into it).  When that is not the current stream, the
    caching allocator is told, so that it does not hand the memory out again
    before `stream` has finished with it."""
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    nbytes = need()
    if nbytes == 0:
        return None, 0
    workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    s = _torch_stream(stream, device)
    if s != torch.cuda.current_stream(device):
        workspace.record_stream(s)
    return workspace, nbytes


def cce_looped_allgather_einsum(ctx: Context, mode, looped, local, out, workspace=None,
                                flags: int = 0, stream=None):
    """Looped AllGather-Einsum over n = len(looped) ranks; writes out[r]."""
    n = len(looped)
    mode = AG_MODES[mode] if isinstance(mode, str) else mode
    lm, cm, om = _same(looped, "looped"), _same(local, "local"), _same(out, "out")
    _dtype_is(local, looped[0].dtype, "the local operand")
    _on_device(ctx, [*looped, *local, *out, workspace])
    in_t, out_t = _dtype(looped[0].dtype), _dtype(out[0].dtype)
    def need():
        return cce_looped_allgather_einsum_workspace(n, mode, in_t, out_t,
                                                     (lm.rows, lm.cols, lm.ld),
                                                     (om.rows, om.cols, om.ld))
    ws, wsb = _workspace(need, out[0].device, workspace, stream)
    check(lib().cce_looped_allgather_einsum(
        ctx.handle, n, mode, in_t, out_t,
        ptr_array([t.data_ptr() for t in looped]), lm,
        ptr_array([t.data_ptr() for t in local]), cm,
        ptr_array([t.data_ptr() for t in out]), om,
        ws.data_ptr() if ws is not None else None, wsb, flags,
        _stream(stream, out[0].device)), "cce_looped_allgather_einsum")
    return out


def cce_looped_einsum_reducescatter_workspace(n_ranks, mode, out_shape) -> int:
    nb = ctypes.c_size_t()
    mode = RS_MODES[mode] if isinstance(mode, str) else mode
    s = out_shape
    check(lib().cce_looped_einsum_reducescatter_workspace(
        n_ranks, mode, CCE_F32, cce_mat(s[0], s[1], s[2] if len(s) > 2 else s[1]),
        ctypes.byref(nb)), "cce_looped_einsum_reducescatter_workspace")
    return nb.value


def cce_looped_einsum_reducescatter(ctx: Context, mode, a, b, out, workspace=None,
                                    flags: int = 0, stream=None):
    """Looped Einsum-ReduceScatter over n = len(a) ranks; writes out[r]."""
    n = len(a)
    mode = RS_MODES[mode] if isinstance(mode, str) else mode
    am, bm, om = _same(a, "a"), _same(b, "b"), _same(out, "out")
    _dtype_is(b, a[0].dtype, "b")
    _on_device(ctx, [*a, *b, *out, workspace])
    in_t, out_t = _dtype(a[0].dtype), _dtype(out[0].dtype)
    ws, wsb = _workspace(lambda: cce_looped_einsum_reducescatter_workspace(
        n, mode, (om.rows, om.cols, om.ld)), out[0].device, workspace, stream)
    check(lib().cce_looped_einsum_reducescatter(
        ctx.handle, n, mode, in_t, CCE_F32, out_t,
        ptr_array([t.data_ptr() for t in a]), am,
        ptr_array([t.data_ptr() for t in b]), bm,
        ptr_array([t.data_ptr() for t in out]), om,
        ws.data_ptr() if ws is not None else None, wsb, flags,
        _stream(stream, out[0].device)), "cce_looped_einsum_reducescatter")
    return out


def cce_looped_einsum_reducescatter_epilogue(ctx: Context, mode, a, b, bias, residuals, out,
                                             p_drop: float, seed: int = 0, offset: int = 0,
                                             mask_row0=None, mask_col0: int = 0,
                                             mask_ld: int | None = None, workspace=None,
                                             flags: int = 0, stream=None):
    """Looped Einsum-ReduceScatter over n = len(a) ranks with the fused reduce
    epilogue: out[r] = residuals[r] + keep * (S_r + bias) / (1 - p_drop), S_r
    the fp32 ReduceScatter result of rank r.  mask_row0: n row bases (default
    0 for every rank); residuals: list or None."""
    n = len(a)
    mode = RS_MODES[mode] if isinstance(mode, str) else mode
    am, bm, om = _same(a, "a"), _same(b, "b"), _same(out, "out")
    rm = _same(residuals, "residual") if residuals is not None else None
    # the ABI reads the bias and the residuals as the output's element type
    _dtype_is(b, a[0].dtype, "b")
    _dtype_is([bias, *(residuals or [])], out[0].dtype, "the bias and the residuals")
    _on_device(ctx, [*a, *b, bias, *(residuals or []), *out])
    if mask_ld is None:
        mask_ld = mask_col0 + om.cols
    rows0 = list(mask_row0) if mask_row0 is not None else [0] * n
    _on_device(ctx, [workspace])
    ws, wsb = _workspace(lambda: cce_looped_einsum_reducescatter_workspace(
        n, mode, (om.rows, om.cols, om.ld)), out[0].device, workspace, stream)
    check(lib().cce_looped_einsum_reducescatter_epilogue(
        ctx.handle, n, mode, _dtype(a[0].dtype), _dtype(out[0].dtype),
        ptr_array([t.data_ptr() for t in a]), am,
        ptr_array([t.data_ptr() for t in b]), bm,
        bias.data_ptr() if bias is not None else None,
        ptr_array([t.data_ptr() for t in residuals]) if residuals is not None else None,
        rm.ld if rm is not None else om.cols,
        float(p_drop), int(seed), int(offset), (ctypes.c_int64 * n)(*rows0), int(mask_col0),
        int(mask_ld), ptr_array([t.data_ptr() for t in out]), om,
        ws.data_ptr() if ws is not None else None, wsb, flags,
        _stream(stream, out[0].device)), "cce_looped_einsum_reducescatter_epilogue")
    return out


def cce_looped_einsum_reducescatter_epilogue_noalloc(ctx: Context, mode, a, b, bias, residuals,
                                                     out, p_drop: float, seed: int = 0,
                                                     offset: int = 0, mask_row0=None,
                                                     mask_col0: int = 0, mask_ld: int | None = None,
                                                     flags: int = 0, stream=None):
    """cce_looped_einsum_reducescatter_epilogue without a workspace: the
    library's static device scratch (CCE_NOALLOC_SCRATCH_BYTES per GPU) takes
    its place, and nothing is allocated.  Calls that overlap on one GPU race
    on that scratch."""
    n = len(a)
    mode = RS_MODES[mode] if isinstance(mode, str) else mode
    am, bm, om = _same(a, "a"), _same(b, "b"), _same(out, "out")
    rm = _same(residuals, "residual") if residuals is not None else None
    # the ABI reads the bias and the residuals as the output's element type
    _dtype_is(b, a[0].dtype, "b")
    _dtype_is([bias, *(residuals or [])], out[0].dtype, "the bias and the residuals")
    _on_device(ctx, [*a, *b, bias, *(residuals or []), *out])
    if mask_ld is None:
        mask_ld = mask_col0 + om.cols
    rows0 = list(mask_row0) if mask_row0 is not None else [0] * n
    check(lib().cce_looped_einsum_reducescatter_epilogue_noalloc(
        ctx.handle, n, mode, _dtype(a[0].dtype), _dtype(out[0].dtype),
        ptr_array([t.data_ptr() for t in a]), am,
        ptr_array([t.data_ptr() for t in b]), bm,
        bias.data_ptr() if bias is not None else None,
        ptr_array([t.data_ptr() for t in residuals]) if residuals is not None else None,
        rm.ld if rm is not None else om.cols,
        float(p_drop), int(seed), int(offset), (ctypes.c_int64 * n)(*rows0), int(mask_col0),
        int(mask_ld), ptr_array([t.data_ptr() for t in out]), om, flags,
        _stream(stream, out[0].device)), "cce_looped_einsum_reducescatter_epilogue_noalloc")
    return out


def cce_grouped_gemm(ctx: Context, a, b, c, gelu: bool = False, stream=None):
    """c[g] = a[g] @ b[g]^T for every g, one launch."""
    am, bm, cm = _same(a, "a"), _same(b, "b"), _same(c, "c")
    _dtype_is(b, a[0].dtype, "b")
    _on_device(ctx, [*a, *b, *c])
    check(lib().cce_grouped_gemm(
        ctx.handle, len(a), _dtype(a[0].dtype), _dtype(c[0].dtype),
        ptr_array([t.data_ptr() for t in a]), am,
        ptr_array([t.data_ptr() for t in b]), bm,
        ptr_array([t.data_ptr() for t in c]), cm,
        CCE_FLAG_GELU if gelu else 0, _stream(stream, c[0].device)), "cce_grouped_gemm")
    return c


def cce_fused_reduce_epilogue(ctx: Context, partials, bias, residual, out, p_drop: float,
                              seed: int = 0, offset: int = 0, mask_row0: int = 0,
                              mask_col0: int = 0, mask_ld: int | None = None, mask_out=None,
                              stream=None):
    """out = residual + keep * (sum(partials) + bias) / (1 - p_drop)."""
    pm = _same(partials, "partial")
    om = _mat(out)
    rm = _mat(residual) if residual is not None else None
    _on_device(ctx, [*partials, bias, residual, out, mask_out])
    if mask_ld is None:
        mask_ld = mask_col0 + pm.cols
    bias_t = _dtype(bias.dtype) if bias is not None else _dtype(out.dtype)
    res_t = _dtype(residual.dtype) if residual is not None else _dtype(out.dtype)
    check(lib().cce_fused_reduce_epilogue(
        ctx.handle, len(partials), _dtype(partials[0].dtype),
        ptr_array([t.data_ptr() for t in partials]), pm,
        bias.data_ptr() if bias is not None else None, bias_t,
        residual.data_ptr() if residual is not None else None, res_t,
        rm.ld if rm is not None else pm.cols,
        float(p_drop), int(seed), int(offset), int(mask_row0), int(mask_col0), int(mask_ld),
        out.data_ptr(), _dtype(out.dtype), om.ld,
        mask_out.data_ptr() if mask_out is not None else None, 0,
        _stream(stream, out.device)), "cce_fused_reduce_epilogue")
    return out


def cce_fused_reduce_epilogue_batched(ctx: Context, partials, bias, residuals, outs,
                                      p_drop: float, seed: int = 0, offset: int = 0,
                                      mask_row0=None, mask_col0: int = 0,
                                      mask_ld: int | None = None, mask_outs=None, stream=None):
    """outs[b] = residuals[b] + keep * (sum(partials[b]) + bias) / (1 - p_drop), one launch.
    partials: list of n_batch lists of equal length; residuals, mask_outs: lists or None;
    mask_row0: list of n_batch row bases (default 0 for every entry)."""
    nb = len(outs)
    if len(partials) != nb or len({len(p) for p in partials}) != 1:
        raise ValueError("partials must be n_batch lists of equal length")
    flat = [t for ps in partials for t in ps]
    pm = _same(flat, "partial")
    om = _same(outs, "out")
    _on_device(ctx, [*flat, bias, *(residuals or []), *outs, *(mask_outs or [])])
    rm = _same(residuals, "residual") if residuals is not None else None
    if mask_ld is None:
        mask_ld = mask_col0 + pm.cols
    rows0 = list(mask_row0) if mask_row0 is not None else [0] * nb
    bias_t = _dtype(bias.dtype) if bias is not None else _dtype(outs[0].dtype)
    res_t = _dtype(residuals[0].dtype) if residuals is not None else _dtype(outs[0].dtype)
    check(lib().cce_fused_reduce_epilogue_batched(
        ctx.handle, nb, len(partials[0]), _dtype(flat[0].dtype),
        ptr_array([t.data_ptr() for t in flat]), pm,
        bias.data_ptr() if bias is not None else None, bias_t,
        ptr_array([t.data_ptr() for t in residuals]) if residuals is not None else None, res_t,
        rm.ld if rm is not None else pm.cols,
        float(p_drop), int(seed), int(offset), (ctypes.c_int64 * nb)(*rows0), int(mask_col0),
        int(mask_ld), ptr_array([t.data_ptr() for t in outs]), _dtype(outs[0].dtype), om.ld,
        ptr_array([t.data_ptr() for t in mask_outs]) if mask_outs is not None else None, 0,
        _stream(stream, outs[0].device)), "cce_fused_reduce_epilogue_batched")
    return outs


def cce_fused_allreduce_epilogue(ctx: Context, partials, bias, residual, outs, p_drop: float,
                                 seed: int = 0, offset: int = 0, mask_row0: int = 0,
                                 mask_col0: int = 0, mask_ld: int | None = None, mask_out=None,
                                 stream=None):
    """FusedAllReduce: every outs[r] = residual + keep * (sum(partials) + bias) / (1 - p)."""
    pm = _same(partials, "partial")
    om = _same(outs, "out")
    if len(outs) != len(partials):
        raise ValueError("one output per rank")
    _on_device(ctx, [*partials, bias, residual, *outs, mask_out])
    rm = _mat(residual) if residual is not None else None
    if mask_ld is None:
        mask_ld = mask_col0 + pm.cols
    bias_t = _dtype(bias.dtype) if bias is not None else _dtype(outs[0].dtype)
    res_t = _dtype(residual.dtype) if residual is not None else _dtype(outs[0].dtype)
    check(lib().cce_fused_allreduce_epilogue(
        ctx.handle, len(partials), _dtype(partials[0].dtype),
        ptr_array([t.data_ptr() for t in partials]), pm,
        bias.data_ptr() if bias is not None else None, bias_t,
        residual.data_ptr() if residual is not None else None, res_t,
        rm.ld if rm is not None else pm.cols,
        float(p_drop), int(seed), int(offset), int(mask_row0), int(mask_col0), int(mask_ld),
        ptr_array([t.data_ptr() for t in outs]), _dtype(outs[0].dtype), om.ld,
        mask_out.data_ptr() if mask_out is not None else None, 0,
        _stream(stream, outs[0].device)), "cce_fused_allreduce_epilogue")
    return outs
