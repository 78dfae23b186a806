"""Collective primitives and a brute-force N-rank simulation of the looped
CollectiveEinsum.  TEST INFRASTRUCTURE ONLY (see the package header).

[OV] = Wang et al., "Overlap Communication with Dependent Computation via
Decomposition in Large Deep Learning Models", ASPLOS'23.

Every rank is a Python list slot holding its own arrays; a CollectivePermute
is an explicit re-assignment of slots following the {source, destination}
pairs.  Nothing is computed from a closed-form shard formula: the shard that a
rank works on is whatever its buffers hold after the permutes ran, and the
starting slice of the ReduceScatter loop is found by pushing position markers
through the same permutes.

Parity pins (tests/test_oracle_ring.py): the 2-way worked examples of [OV]
Section 4 (Figures 4 and 5, golden fixtures), the ring pair list of [OV]
Section 5.1, the alignment rules stated there (AllGather at loop start,
ReduceScatter at loop end), agreement with the monolithic collectives for
N = 1..16 on exact-integer inputs, and AllReduce = ReduceScatter + AllGather
([OV] Section 2.1; CoCoNet's AllReduce split).
"""

from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# Collective primitives ([OV] Section 2.1)
# --------------------------------------------------------------------------

def ring_pairs(n: int) -> list[tuple[int, int]]:
    """{source, destination} pairs of the loop's CollectivePermute.

    [OV] Section 5.1 builds them as {0, N-1}, {1, 0}, {2, 1}, ..., {N-1, N-2}:
    every partition sends to the partition one below it, wrapping around.
    """
    return [(src, (src - 1) % n) for src in range(n)]


def collective_permute(bufs: list, pairs: list[tuple[int, int]]) -> list:
    """Point-to-point transfer between every listed {source, destination}
    pair ([OV] Section 2.1).  A destination that appears in no pair receives
    nothing (None)."""
    out = [None] * len(bufs)
    for src, dst in pairs:
        out[dst] = bufs[src]
    return out


def allgather(shards: list[np.ndarray], axis: int) -> np.ndarray:
    """Every partition receives every partition's data, concatenated in
    partition-ID order ([OV] Section 2.1)."""
    return np.concatenate(shards, axis=axis)


def reducescatter(fulls: list[np.ndarray], axis: int) -> list[np.ndarray]:
    """Partition r gets the elementwise sum, over all partitions, of the
    shard with ID r of their inputs ([OV] Section 2.1).  The shards are the
    N equal parts of each input along `axis`; the sum runs in rank order."""
    n = len(fulls)
    split = [np.split(f, n, axis=axis) for f in fulls]
    out = []
    for shard_id in range(n):
        acc = split[0][shard_id].copy()
        for q in range(1, n):
            acc = acc + split[q][shard_id]
        out.append(acc)
    return out


def allreduce(fulls: list[np.ndarray]) -> np.ndarray:
    """Elementwise sum over all partitions, replicated ([OV] Section 2.1)."""
    acc = fulls[0].copy()
    for f in fulls[1:]:
        acc = acc + f
    return acc


# --------------------------------------------------------------------------
# The looped AllGather-Einsum ([OV] Sections 4 and 5.1)
# --------------------------------------------------------------------------

AG_MODES = ("lhs_rows", "rhs_cols", "lhs_cols", "rhs_rows")
RS_MODES = ("slice_lhs_rows", "slice_rhs_cols")


def _ag_partial(mode: str, held: np.ndarray, local: np.ndarray, shard_id: int):
    """The per-iteration partial einsum of one rank.

    `held` is the looped shard the rank holds in this iteration, `local` the
    operand that never moves.  Orientation: the product is always
    (left factor) @ (right factor) with shapes [m, k] @ [k, n].
      case 1 ([OV] 5.1): the looped factor is split on a non-contracting dim;
        the einsum takes it as it is.
      case 2 ([OV] 5.1): the looped factor is split on the contracting dim;
        the local factor is DynamicSliced along its contracting dim with the
        size of the looped shard, at the looped shard's ID.
    """
    if mode == "rhs_cols":          # held = B_s [K, n_s], local = A_r [M, K]
        return local @ held
    if mode == "lhs_rows":          # held = A_s [m_s, K], local = B_r [K, N]
        return held @ local
    if mode == "lhs_cols":          # held = A_s [M, k_s], local = B_r [K, N]
        ks = held.shape[1]
        return held @ local[shard_id * ks:(shard_id + 1) * ks, :]
    if mode == "rhs_rows":          # held = B_s [k_s, N], local = A_r [M, K]
        ks = held.shape[0]
        return local[:, shard_id * ks:(shard_id + 1) * ks] @ held
    raise ValueError(mode)


def _ag_update(mode: str, out: np.ndarray, part: np.ndarray, shard_id: int):
    """Update of [OV] 5.1: DynamicUpdateSlice for case 1, Addition for case 2."""
    if mode == "rhs_cols":
        w = part.shape[1]
        out[:, shard_id * w:(shard_id + 1) * w] = part
    elif mode == "lhs_rows":
        h = part.shape[0]
        out[shard_id * h:(shard_id + 1) * h, :] = part
    else:
        out += part
    return out


def _ag_out_shape(mode: str, n: int, shard: np.ndarray, local: np.ndarray):
    if mode == "rhs_cols":
        return (local.shape[0], n * shard.shape[1])
    if mode == "lhs_rows":
        return (n * shard.shape[0], local.shape[1])
    if mode == "lhs_cols":
        return (shard.shape[0], local.shape[1])
    if mode == "rhs_rows":
        return (local.shape[0], shard.shape[1])
    raise ValueError(mode)


def simulate_allgather_einsum(mode: str, looped: list[np.ndarray],
                              local: list[np.ndarray]):
    """Run the looped AllGather-Einsum rank by rank with explicit buffers.

    looped[r] is partition r's own shard (shard ID r), local[r] its local
    operand.  Each of the N iterations starts the permute of the held shard
    ([OV] Section 4: a device sends the shard it holds while it computes on
    it), computes the partial einsum on the held shard, applies the update,
    and then takes the received shard.  The permute issued in the last
    iteration delivers nothing that is used; it is still simulated and logged.

    Returns (outputs, schedule, transfers):
      outputs[r]      -- rank r's result, float64;
      schedule[i][r]  -- the shard ID rank r computed on in iteration i;
      transfers[i]    -- list of (src, dst, shard_id) moved in iteration i.
    """
    n = len(looped)
    assert mode in AG_MODES and len(local) == n
    held = [(looped[r], r) for r in range(n)]       # aligned at loop start
    outs = [np.zeros(_ag_out_shape(mode, n, looped[0], local[r]))
            for r in range(n)]
    schedule, transfers = [], []
    pairs = ring_pairs(n)
    for _ in range(n):
        in_flight = collective_permute(held, pairs)            # Start
        transfers.append([(s, d, held[s][1]) for s, d in pairs])
        schedule.append([held[r][1] for r in range(n)])
        for r in range(n):
            buf, sid = held[r]
            part = _ag_partial(mode, buf, local[r], sid)
            outs[r] = _ag_update(mode, outs[r], part, sid)
        held = in_flight                                        # Done
    return outs, schedule, transfers


# --------------------------------------------------------------------------
# The looped Einsum-ReduceScatter ([OV] Sections 4 and 5.1)
# --------------------------------------------------------------------------

def reducescatter_start_ids(n: int) -> list[int]:
    """Shard ID each rank must start its accumulator with so that, after the
    accumulators have travelled through the loop's permutes, every rank ends
    with the shard of its own ID ([OV] Section 5.1: the ReduceScatter loop is
    aligned at loop end).

    Found mechanically: a marker placed at each rank is pushed through the
    N-1 permutes that follow the first accumulation; the rank a marker lands
    on is the shard ID its starting rank must compute first.
    """
    pairs = ring_pairs(n)
    markers = list(range(n))                 # markers[rank] = starting rank
    for _ in range(n - 1):
        markers = collective_permute(markers, pairs)
    start = [None] * n
    for landing_rank, starting_rank in enumerate(markers):
        start[starting_rank] = landing_rank
    return start


def _rs_partial(mode: str, a: np.ndarray, b: np.ndarray, n: int, shard_id: int):
    """DynamicSlice of the operand that owns the result's partitioned
    non-contracting dim, then the partial einsum ([OV] 5.1)."""
    if mode == "slice_lhs_rows":    # A_r [n*m_s, K], B_r [K, N]
        ms = a.shape[0] // n
        return a[shard_id * ms:(shard_id + 1) * ms, :] @ b
    if mode == "slice_rhs_cols":    # A_r [M, K], B_r [K, n*n_s]
        ns = b.shape[1] // n
        return a @ b[:, shard_id * ns:(shard_id + 1) * ns]
    raise ValueError(mode)


def simulate_einsum_reducescatter(mode: str, a: list[np.ndarray],
                                  b: list[np.ndarray]):
    """Run the looped Einsum-ReduceScatter rank by rank with explicit buffers.

    As in [OV] Section 4 (Figure 5): the accumulator starts at zero; each
    iteration starts sending the accumulator, computes the partial einsum on
    a slice whose ID is carried by the accumulator, and at its end adds the
    partial to the accumulator just received.

    Returns (outputs, schedule, transfers) as simulate_allgather_einsum,
    schedule[i][r] being the slice ID rank r computes in iteration i.
    """
    n = len(a)
    assert mode in RS_MODES and len(b) == n
    pairs = ring_pairs(n)
    ids = reducescatter_start_ids(n)
    shape = _rs_partial(mode, a[0], b[0], n, 0).shape
    acc = [np.zeros(shape) for _ in range(n)]
    # the label each accumulator carries: the zero accumulator that rank r
    # sends first is the one that will hold the shard rank r-1 computes.
    labels = collective_permute(ids, [(d, s) for s, d in pairs])
    schedule, transfers = [], []
    for _ in range(n):
        recv = collective_permute(acc, pairs)                     # Start
        transfers.append([(s, d, labels[s]) for s, d in pairs])
        labels = collective_permute(labels, pairs)
        schedule.append(list(labels))
        parts = [_rs_partial(mode, a[r], b[r], n, labels[r]) for r in range(n)]
        acc = [recv[r] + parts[r] for r in range(n)]               # Done + Add
    assert labels == list(range(n)), "ReduceScatter loop not aligned at end"
    return acc, schedule, transfers
