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
([OV] Section 2.1; CoCoNet's AllReduce split).  The bidirectional variant of
[OV] Section 5.4.2 (whose figures are not in the text) is pinned by exact
agreement with the monolithic definitions for N = 1..16, by the halved
iteration count that section states, by every rank still sending N-1 shards
to ring neighbours only, and by every shard / slice being covered once.
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
# case 3: batched operands (3-D arrays), the looped factor split on the batch dim
AG_BATCH_MODES = ("lhs_batch",)
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
      case 3 ([OV] 5.1): the looped factor is split on the batch dim; the
        local factor is DynamicSliced along its batch dim, at the looped
        shard's ID, with the looped shard's batch extent (the reading of the
        slice size), and the product is one matmul per batch element.
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
    if mode == "lhs_batch":         # held = A_s [b_s, m, K], local = B_r [N b_s, K, N]
        bs = held.shape[0]
        return np.matmul(held, local[shard_id * bs:(shard_id + 1) * bs])
    raise ValueError(mode)


def _ag_update(mode: str, out: np.ndarray, part: np.ndarray, shard_id: int):
    """Update of [OV] 5.1: DynamicUpdateSlice for cases 1 and 3 (along the
    batch dim for case 3), Addition for case 2."""
    if mode == "lhs_batch":
        bs = part.shape[0]
        out[shard_id * bs:(shard_id + 1) * bs] = part
    elif mode == "rhs_cols":
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
    if mode == "lhs_batch":
        return (n * shard.shape[0], shard.shape[1], local.shape[2])
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
    assert mode in AG_MODES + AG_BATCH_MODES and len(local) == n
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


# --------------------------------------------------------------------------
# Bidirectional data transfer ([OV] Section 5.4.2)
#
# Reading of the section (its Figures 9 and 10 are not in the text): every
# rank keeps two looped buffers (AllGather) or two accumulators
# (ReduceScatter), one travelling each way round the ring: "cw" along the
# loop's pairs of Section 5.1 (rank r sends to r-1) and "ccw" along the
# reversed pairs (rank r sends to r+1).  Each iteration computes the two
# partial einsums, one per direction, as one operation, so the loop has
# ceil(N/2) iterations instead of N.  The AllGather needs a prologue -- one
# ccw permute before the loop, so that the ccw buffer starts one shard away
# from the cw buffer -- and the ReduceScatter an epilogue -- one ccw permute
# after the loop that brings each ccw accumulator to the rank of its shard,
# followed by the sum of the two accumulators.  Both move N-1 shards per
# rank in total, like the one-way loop.
# --------------------------------------------------------------------------

def reversed_ring_pairs(n: int) -> list[tuple[int, int]]:
    """The loop's pairs with source and destination swapped: r -> r+1."""
    return [(d, s) for s, d in ring_pairs(n)]


def bidir_lengths(n: int) -> tuple[int, int]:
    """Iterations of the cw and the ccw stream: ceil(N/2) and floor(N/2)."""
    return (n + 1) // 2, n // 2


def simulate_allgather_einsum_bidir(mode: str, looped: list[np.ndarray],
                                    local: list[np.ndarray]):
    """Bidirectional looped AllGather-Einsum, rank by rank.

    Prologue: the ccw buffer of every rank receives its ccw neighbour's
    shard.  Iteration i computes the partial einsum on the cw buffer's shard
    and, while i < floor(N/2), on the ccw buffer's shard; then, unless the
    stream is done, each buffer is sent on in its direction.

    Returns (outputs, schedule, transfers):
      schedule[i][r]  -- (cw shard ID, ccw shard ID or None) of rank r;
      transfers       -- list of (phase, direction, src, dst, shard_id),
                         phase "prologue" or the iteration index.
    """
    n = len(looped)
    assert mode in AG_MODES + AG_BATCH_MODES and len(local) == n
    k_cw, k_ccw = bidir_lengths(n)
    cw_pairs, ccw_pairs = ring_pairs(n), reversed_ring_pairs(n)
    own = [(looped[r], r) for r in range(n)]
    cw = list(own)                                   # aligned at loop start
    transfers = []
    ccw = [None] * n
    if k_ccw > 0:                                    # prologue
        ccw = collective_permute(own, ccw_pairs)
        transfers += [("prologue", "ccw", s, d, own[s][1]) for s, d in ccw_pairs]
    outs = [np.zeros(_ag_out_shape(mode, n, looped[0], local[r])) for r in range(n)]
    schedule = []
    for i in range(k_cw):
        do_ccw = i < k_ccw
        schedule.append([(cw[r][1], ccw[r][1] if do_ccw else None) for r in range(n)])
        for r in range(n):
            for buf, sid in ([cw[r], ccw[r]] if do_ccw else [cw[r]]):
                part = _ag_partial(mode, buf, local[r], sid)
                outs[r] = _ag_update(mode, outs[r], part, sid)
        if i + 1 < k_cw:
            transfers += [(i, "cw", s, d, cw[s][1]) for s, d in cw_pairs]
            cw = collective_permute(cw, cw_pairs)
        if i + 1 < k_ccw:
            transfers += [(i, "ccw", s, d, ccw[s][1]) for s, d in ccw_pairs]
            ccw = collective_permute(ccw, ccw_pairs)
    return outs, schedule, transfers


def _start_labels(n: int, pairs, hops: int) -> list[int]:
    """Shard ID each rank must start an accumulator with so that after
    `hops` permutes along `pairs` the accumulator sits on the rank of its
    ID (markers pushed through the permutes, as reducescatter_start_ids)."""
    markers = list(range(n))
    for _ in range(hops):
        markers = collective_permute(markers, pairs)
    start = [None] * n
    for landing_rank, starting_rank in enumerate(markers):
        start[starting_rank] = landing_rank
    return start


def simulate_einsum_reducescatter_bidir(mode: str, a: list[np.ndarray],
                                        b: list[np.ndarray]):
    """Bidirectional looped Einsum-ReduceScatter, rank by rank.

    The cw accumulator of a shard makes ceil(N/2) - 1 hops and ends on the
    rank of its shard at loop end; the ccw accumulator makes floor(N/2) - 1
    hops in the loop and one more in the epilogue.  Each accumulator starts
    as its first partial (no zero buffer is sent) and adds one partial per
    rank it visits.  Epilogue: out[r] = cw[r] + ccw[r] after the ccw hop.

    Returns (outputs, schedule, transfers) with schedule[i][r] =
    (cw slice ID, ccw slice ID or None) and transfers as in
    simulate_allgather_einsum_bidir (phase "epilogue" for the last hop).
    """
    n = len(a)
    assert mode in RS_MODES and len(b) == n
    k_cw, k_ccw = bidir_lengths(n)
    cw_pairs, ccw_pairs = ring_pairs(n), reversed_ring_pairs(n)
    lab_cw = _start_labels(n, cw_pairs, k_cw - 1)
    lab_ccw = _start_labels(n, ccw_pairs, k_ccw) if k_ccw > 0 else [None] * n
    acc_cw, acc_ccw = [None] * n, [None] * n
    schedule, transfers = [], []
    for i in range(k_cw):
        do_ccw = i < k_ccw
        schedule.append([(lab_cw[r], lab_ccw[r] if do_ccw else None) for r in range(n)])
        for r in range(n):
            p = _rs_partial(mode, a[r], b[r], n, lab_cw[r])
            acc_cw[r] = p if i == 0 else acc_cw[r] + p
            if do_ccw:
                q = _rs_partial(mode, a[r], b[r], n, lab_ccw[r])
                acc_ccw[r] = q if i == 0 else acc_ccw[r] + q
        if i + 1 < k_cw:
            transfers += [(i, "cw", s, d, lab_cw[s]) for s, d in cw_pairs]
            acc_cw = collective_permute(acc_cw, cw_pairs)
            lab_cw = collective_permute(lab_cw, cw_pairs)
        if do_ccw:                                   # in the loop or the epilogue
            phase = i if i + 1 < k_ccw else "epilogue"
            transfers += [(phase, "ccw", s, d, lab_ccw[s]) for s, d in ccw_pairs]
            acc_ccw = collective_permute(acc_ccw, ccw_pairs)
            lab_ccw = collective_permute(lab_ccw, ccw_pairs)
    assert lab_cw == list(range(n)), "cw accumulators not aligned at loop end"
    if k_ccw > 0:
        assert lab_ccw == list(range(n)), "ccw accumulators not aligned after the epilogue"
        outs = [acc_cw[r] + acc_ccw[r] for r in range(n)]
    else:
        outs = acc_cw
    return outs, schedule, transfers
