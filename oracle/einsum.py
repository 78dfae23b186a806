"""Monolithic definitions of what the looped einsums compute.
TEST INFRASTRUCTURE ONLY (see the package header).

[OV] = Wang et al., "Overlap Communication with Dependent Computation via
Decomposition in Large Deep Learning Models", ASPLOS'23.

The decomposed loop is semantically equal to the original collective followed
by (or preceded by) the original einsum ([OV] Section 4), so the plain
definition is: gather the shards by partition ID, then one matmul; or one
matmul per rank, then reduce-scatter.  Orientation is mathematical: left
factor [m, k] times right factor [k, n], float64.

Parity pins (tests/test_oracle_einsum.py): a pure-Python triple loop on tiny
inputs, the N = 1 reduction to a plain matmul, bit-equality with the
brute-force loop simulation on exact-integer inputs, and the AllReduce =
ReduceScatter + AllGather identity.  The backward pass of the AllGather-Einsum
is pinned to torch autograd (float64, CPU) on the monolithic forward.
"""

from __future__ import annotations

import numpy as np

from .ring import allgather, reducescatter


def allgather_einsum(mode: str, looped: list[np.ndarray],
                     local: list[np.ndarray]) -> list[np.ndarray]:
    """Result of AllGather(looped shards) followed by the einsum with each
    rank's local operand ([OV] Section 5.1 cases 1 and 2).

      lhs_rows : Y_r = concat_rows(A_0..A_{N-1}) @ B_r      (case 1)
      rhs_cols : Y_r = A_r @ concat_cols(B_0..B_{N-1})      (case 1)
      lhs_cols : Y_r = concat_cols(A_0..A_{N-1}) @ B_r      (case 2)
      rhs_rows : Y_r = A_r @ concat_rows(B_0..B_{N-1})      (case 2)
      lhs_batch: Y_r = concat_batch(A_0..A_{N-1}) @ B_r     (case 3)
                 A_s [b_s, m, k], B_r [N b_s, k, n]: one matmul per batch
                 element, Y_r [N b_s, m, n]
    """
    if mode == "lhs_rows":
        full = allgather(looped, axis=0)
        return [full @ b for b in local]
    if mode == "rhs_cols":
        full = allgather(looped, axis=1)
        return [a @ full for a in local]
    if mode == "lhs_cols":
        full = allgather(looped, axis=1)
        return [full @ b for b in local]
    if mode == "rhs_rows":
        full = allgather(looped, axis=0)
        return [a @ full for a in local]
    if mode == "lhs_batch":
        full = allgather(looped, axis=0)            # [N b_s, m, k]
        return [np.matmul(full, b) for b in local]
    raise ValueError(mode)


def einsum_reducescatter(mode: str, a: list[np.ndarray],
                         b: list[np.ndarray]) -> list[np.ndarray]:
    """Result of each rank's full einsum followed by ReduceScatter along the
    result's partitioned non-contracting dim ([OV] Section 5.1).

      slice_lhs_rows : out_r = sum_q (A_q @ B_q)[rows of shard r]
      slice_rhs_cols : out_r = sum_q (A_q @ B_q)[cols of shard r]
    """
    fulls = [x @ y for x, y in zip(a, b)]
    axis = 0 if mode == "slice_lhs_rows" else 1
    if mode not in ("slice_lhs_rows", "slice_rhs_cols"):
        raise ValueError(mode)
    return reducescatter(fulls, axis=axis)


def local_matmuls(a: list[np.ndarray], b: list[np.ndarray]) -> list[np.ndarray]:
    """The per-rank MatMul of two tensors sliced on the contraction dim,
    which yields one local (rank-private) partial per rank (CoCoNet, Figure 3
    program: MatMul of the sliced input and sliced weight)."""
    return [x @ y for x, y in zip(a, b)]


def allgather_einsum_backward(mode: str, looped: list[np.ndarray],
                              local: list[np.ndarray], d_out: list[np.ndarray]):
    """Gradients of the case-1 AllGather-Einsum with respect to both operands.

    [OV] Section 2.2: the weights are AllGathered before each einsum in the
    forward pass, and in the backward pass that AllGather becomes a
    ReduceScatter producing each device's partition of the weight gradient.
    Written from the definitions (d_out[r] is dL/dY_r):

      rhs_cols, Y_r = A_r @ concat_cols(B_s):
        dB_s = sum_r (A_r^T @ dY_r)[:, cols of shard s]   (Einsum-ReduceScatter)
        dA_r = dY_r @ concat_cols(B_s)^T                 (AllGather-Einsum, K split)
      lhs_rows, Y_r = concat_rows(A_s) @ B_r:
        dA_s = sum_r (dY_r @ B_r^T)[rows of shard s]     (Einsum-ReduceScatter)
        dB_r = concat_rows(A_s)^T @ dY_r                 (AllGather-Einsum, K split)

    Returns (grads of the looped shards by shard ID, grads of the local
    operands by rank)."""
    if mode == "rhs_cols":
        full = allgather(looped, axis=1)
        d_looped = reducescatter([a.T @ dy for a, dy in zip(local, d_out)], axis=1)
        d_local = [dy @ full.T for dy in d_out]
        return d_looped, d_local
    if mode == "lhs_rows":
        full = allgather(looped, axis=0)
        d_looped = reducescatter([dy @ b.T for b, dy in zip(local, d_out)], axis=0)
        d_local = [full.T @ dy for dy in d_out]
        return d_looped, d_local
    raise ValueError(mode)
