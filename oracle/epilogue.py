"""The fused reduce epilogue: sum of N partials, + bias, dropout, + residual.
TEST INFRASTRUCTURE ONLY (see the package header).

[CC] = CoCoNet, "Breaking the Computation and Communication Abstraction
Barrier in Distributed Machine Learning Workloads", ASPLOS'22.

Order of operations from the [CC] Figure 3 program (the Megatron
self-attention tail): the local MatMul partials are summed by AllReduce(+),
the bias is added with PyTorch broadcasting (bias [cols] repeated over rows),
dropout is applied, and the residual is added.  FusedAllReduce ([CC], fused
collective communication) performs exactly these operations while the summed
values are still in registers; the fusion changes where the values live, not
what is computed, so the plain definition below is the oracle.

Dropout is read as inverted dropout with p the drop probability: kept values
are multiplied by 1 / (1 - p), dropped ones become 0.  The keep decision
comes from oracle.philox.keep_mask.

Float64 throughout; the result is rounded to the output dtype only by the
caller's comparison.  `fused_reduce_epilogue_fp32` evaluates the same
definition in float32, one IEEE round-to-nearest-even operation per step in
a fixed order (the reading of the pages this library takes: the sum in
partial order, then the bias, the scale if kept, the residual; no fused
multiply-add), so that a kernel that keeps that order can be compared with it
bit for bit.

Parity pins (tests/test_oracle_epilogue.py): a per-element pure-Python loop on
small shapes, p = 0 (exactly sum + bias + residual), p = 1 (exactly the
residual), linearity in the partials, and the N = 1 case.  The float32
evaluation is pinned to the float64 one within the standard error bound of
n + 3 rounded operations, and by hand-worked cases in which the order of the
sum, or a fused multiply-add, would change the result.  The step-by-step
FusedAllReduce (ReduceScatter, epilogue per slice, AllGather) is pinned to the
whole-tensor epilogue of the AllReduce sum (the collective identity
AllReduce = ReduceScatter + AllGather, with the pointwise tail commuting with
the row split), bit for bit in float64, for ragged row splits as well.
"""

from __future__ import annotations

import numpy as np

from .philox import keep_mask


def fused_reduce_epilogue(partials, bias, residual, p: float, seed: int,
                          offset: int, row0: int = 0, col0: int = 0,
                          mask_ld: int | None = None):
    """out = residual + keep * (sum_k partials[k] + bias) * 1/(1-p).

    partials: list of [rows, cols] arrays; bias: [cols] or None;
    residual: [rows, cols] or None.  Returns (out float64, keep bool)."""
    parts = [np.asarray(x, dtype=np.float64) for x in partials]
    rows, cols = parts[0].shape
    s = parts[0].copy()
    for x in parts[1:]:
        s = s + x                                  # AllReduce(+)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)[None, :]
    keep = keep_mask(rows, cols, p, seed, offset, row0, col0,
                     mask_ld if mask_ld is not None else col0 + cols)
    if p > 0.0:
        scale = 1.0 / (1.0 - p) if p < 1.0 else 0.0
        d = np.where(keep, s * scale, 0.0)
    else:
        d = s
    if residual is not None:
        d = d + np.asarray(residual, dtype=np.float64)
    return d, keep


def fused_allreduce(partials, bias, residual, p: float, seed: int, offset: int,
                    col0: int = 0, mask_ld: int | None = None):
    """CoCoNet's FusedAllReduce across n ranks, step by step ([CC], fused
    collective communication): the AllReduce is split into a ReduceScatter
    and an AllGather, and the bias add, dropout and residual add run on each
    rank's reduced slice between the two.

    partials[r]: rank r's [rows, cols] partial.  Rank r reduces row block r
    (numpy's array_split of the rows into n nearly equal blocks: the
    collective's shard r) over all ranks in rank order, applies the epilogue
    with the block's global row base (so the mask is the one of the whole
    tensor), and the AllGather concatenates the blocks in rank order for
    every rank.  Returns (outputs: one float64 array per rank, keep mask)."""
    n = len(partials)
    parts = [np.asarray(x, dtype=np.float64) for x in partials]
    rows, cols = parts[0].shape
    bounds = np.cumsum([0] + [len(b) for b in np.array_split(np.arange(rows), n)])
    res = None if residual is None else np.asarray(residual, dtype=np.float64)
    blocks, keeps = [], []
    for r in range(n):                                     # ReduceScatter + epilogue
        lo, hi = bounds[r], bounds[r + 1]
        acc = parts[0][lo:hi].copy()
        for q in range(1, n):
            acc = acc + parts[q][lo:hi]
        out_r, keep_r = fused_reduce_epilogue(
            [acc], bias, None if res is None else res[lo:hi], p, seed, offset,
            row0=lo, col0=col0, mask_ld=mask_ld if mask_ld is not None else col0 + cols)
        blocks.append(out_r)
        keeps.append(keep_r)
    full = np.concatenate(blocks, axis=0)                  # AllGather
    return [full.copy() for _ in range(n)], np.concatenate(keeps, axis=0)


def fused_reduce_epilogue_fp32(partials, bias, residual, p: float, seed: int,
                               offset: int, row0: int = 0, col0: int = 0,
                               mask_ld: int | None = None):
    """The definition above evaluated in float32, step by step:

        s = ((P0 + P1) + ...) + P(n-1);  s = s + bias
        d = s * c if kept else 0  (c = 1/(1-p) rounded once to float32;
                                   p = 0: d = s; p >= 1: d = 0)
        out = d + residual

    every operation rounded to float32 (NumPy float32 arithmetic is IEEE
    round-to-nearest-even per operation).  Inputs must be exactly
    representable in float32 (fp32 or bf16 tensors).  Returns (out float32,
    keep bool); a bf16 output is this value rounded once more
    (oracle.numerics.bf16_round)."""
    f = np.float32
    parts = [np.asarray(x, dtype=np.float64) for x in partials]
    for x in parts:
        if not np.array_equal(x.astype(f).astype(np.float64), x, equal_nan=True):
            raise ValueError("partials must be exactly representable in float32")
    rows, cols = parts[0].shape
    s = parts[0].astype(f)
    for x in parts[1:]:
        s = (s + x.astype(f)).astype(f)
    if bias is not None:
        s = (s + np.asarray(bias, dtype=np.float64).astype(f)[None, :]).astype(f)
    keep = keep_mask(rows, cols, p, seed, offset, row0, col0,
                     mask_ld if mask_ld is not None else col0 + cols)
    if p <= 0.0:
        d = s
    elif p >= 1.0:
        d = np.zeros_like(s)
    else:
        c = f(1.0 / (1.0 - p))
        d = np.where(keep, (s * c).astype(f), f(0.0)).astype(f)
    if residual is not None:
        d = (d + np.asarray(residual, dtype=np.float64).astype(f)).astype(f)
    return d, keep
