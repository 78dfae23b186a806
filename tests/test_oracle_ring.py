"""Pins for the ring schedule and the brute-force loop simulation
(oracle.ring): the worked 2-way examples and the pair list of the
Wang et al. ASPLOS'23 page (Sections 4 and 5.1), the alignment rules of
Section 5.1, closed forms, and the collective identities of Section 2.1."""

import os

import numpy as np
import pytest

from oracle import ring, einsum

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(v) for v in line.split()])
    return rows


def _tiny(n, mode):
    """Shards and local operands with distinct integer values per shard."""
    rng = np.random.default_rng(123 + n)
    m, k, c = 3, 4, 2
    if mode == "rhs_cols":
        looped = [rng.integers(-3, 4, (k, c)).astype(float) for _ in range(n)]
        local = [rng.integers(-3, 4, (m, k)).astype(float) for _ in range(n)]
    elif mode == "lhs_rows":
        looped = [rng.integers(-3, 4, (m, k)).astype(float) for _ in range(n)]
        local = [rng.integers(-3, 4, (k, c)).astype(float) for _ in range(n)]
    elif mode == "lhs_cols":
        looped = [rng.integers(-3, 4, (m, k)).astype(float) for _ in range(n)]
        local = [rng.integers(-3, 4, (n * k, c)).astype(float) for _ in range(n)]
    else:
        looped = [rng.integers(-3, 4, (k, c)).astype(float) for _ in range(n)]
        local = [rng.integers(-3, 4, (m, n * k)).astype(float) for _ in range(n)]
    return looped, local


def test_ring_pairs_match_page():
    assert [list(p) for p in ring.ring_pairs(4)] == _load("ring_pairs_4.txt")


def test_2way_allgather_schedule_matches_page():
    looped, local = _tiny(2, "rhs_cols")
    _, sched, _ = ring.simulate_allgather_einsum("rhs_cols", looped, local)
    assert sched == _load("ag_2way_schedule.txt")


def test_2way_reducescatter_schedule_matches_page():
    a = [np.ones((4, 3)) for _ in range(2)]
    b = [np.ones((3, 2)) for _ in range(2)]
    _, sched, _ = ring.simulate_einsum_reducescatter("slice_lhs_rows", a, b)
    assert sched == _load("rs_2way_schedule.txt")


@pytest.mark.parametrize("n", list(range(1, 17)) + [31, 64])
def test_allgather_schedule_closed_form_and_alignment(n):
    looped = [np.full((1, 1), float(r)) for r in range(n)]
    local = [np.ones((1, 1)) for _ in range(n)]
    _, sched, transfers = ring.simulate_allgather_einsum("lhs_rows", looped, local)
    # aligned with the partition ID at loop start (Section 5.1)
    assert sched[0] == list(range(n))
    # closed form s(r, i) = (r + i) mod N; every rank sees every shard once
    for i in range(n):
        assert sched[i] == [(r + i) % n for r in range(n)]
    for r in range(n):
        assert sorted(sched[i][r] for i in range(n)) == list(range(n))
    # each transfer moves the sender's held shard to rank src - 1
    for i, tr in enumerate(transfers):
        for src, dst, sid in tr:
            assert dst == (src - 1) % n and sid == sched[i][src]


@pytest.mark.parametrize("n", list(range(1, 17)) + [31, 64])
def test_reducescatter_schedule_closed_form_and_alignment(n):
    a = [np.ones((n, 1)) for _ in range(n)]
    b = [np.ones((1, 1)) for _ in range(n)]
    _, sched, _ = ring.simulate_einsum_reducescatter("slice_lhs_rows", a, b)
    assert sched[-1] == list(range(n))           # aligned at loop end
    for i in range(n):
        assert sched[i] == [(r + i + 1) % n for r in range(n)]
    if n > 1:
        assert sched[0] != list(range(n))        # does not start at own ID


@pytest.mark.parametrize("mode", ring.AG_MODES)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 8])
def test_allgather_loop_equals_monolithic_exact(mode, n):
    looped, local = _tiny(n, mode)
    outs, _, _ = ring.simulate_allgather_einsum(mode, looped, local)
    ref = einsum.allgather_einsum(mode, looped, local)
    for o, r in zip(outs, ref):
        assert np.array_equal(o, r)


@pytest.mark.parametrize("mode", ring.RS_MODES)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 8])
def test_reducescatter_loop_equals_monolithic_exact(mode, n):
    rng = np.random.default_rng(n)
    if mode == "slice_lhs_rows":
        a = [rng.integers(-3, 4, (2 * n, 5)).astype(float) for _ in range(n)]
        b = [rng.integers(-3, 4, (5, 3)).astype(float) for _ in range(n)]
    else:
        a = [rng.integers(-3, 4, (2, 5)).astype(float) for _ in range(n)]
        b = [rng.integers(-3, 4, (5, 3 * n)).astype(float) for _ in range(n)]
    outs, _, _ = ring.simulate_einsum_reducescatter(mode, a, b)
    ref = einsum.einsum_reducescatter(mode, a, b)
    for o, r in zip(outs, ref):
        assert np.array_equal(o, r)


def test_allreduce_is_reducescatter_then_allgather():
    rng = np.random.default_rng(5)
    n = 4
    fulls = [rng.standard_normal((8, 3)) for _ in range(n)]
    rs = ring.reducescatter(fulls, axis=0)
    ag = ring.allgather(rs, axis=0)
    np.testing.assert_allclose(ag, ring.allreduce(fulls), rtol=0, atol=1e-14)


def test_collective_permute_is_a_ring_shift():
    n = 5
    got = ring.collective_permute(list(range(n)), ring.ring_pairs(n))
    # rank r receives what rank r+1 held
    assert got == [(r + 1) % n for r in range(n)]


# ---------------------------------------------------------------------------
# Bidirectional transfer (Section 5.4.2 of the same page)
# ---------------------------------------------------------------------------
def _rs_tiny(n, mode):
    rng = np.random.default_rng(321 + n)
    if mode == "slice_lhs_rows":
        a = [rng.integers(-3, 4, (2 * n, 5)).astype(float) for _ in range(n)]
        b = [rng.integers(-3, 4, (5, 3)).astype(float) for _ in range(n)]
    else:
        a = [rng.integers(-3, 4, (3, 5)).astype(float) for _ in range(n)]
        b = [rng.integers(-3, 4, (5, 2 * n)).astype(float) for _ in range(n)]
    return a, b


@pytest.mark.parametrize("n", list(range(1, 17)))
@pytest.mark.parametrize("mode", ring.AG_MODES)
def test_bidir_allgather_equals_monolithic_exact(n, mode):
    looped, local = _tiny(n, mode)
    outs, _, _ = ring.simulate_allgather_einsum_bidir(mode, looped, local)
    ref = einsum.allgather_einsum(mode, looped, local)
    for o, r in zip(outs, ref):
        assert np.array_equal(o, r)


@pytest.mark.parametrize("n", list(range(1, 17)))
@pytest.mark.parametrize("mode", ring.RS_MODES)
def test_bidir_reducescatter_equals_monolithic_exact(n, mode):
    a, b = _rs_tiny(n, mode)
    outs, _, _ = ring.simulate_einsum_reducescatter_bidir(mode, a, b)
    ref = einsum.einsum_reducescatter(mode, a, b)
    for o, r in zip(outs, ref):
        assert np.array_equal(o, r)


@pytest.mark.parametrize("n", list(range(1, 17)))
def test_bidir_halves_iterations_and_keeps_the_bytes(n):
    """Two partial einsums per iteration: ceil(N/2) iterations; every rank
    still sends N-1 shards, each to a ring neighbour, cw ones to r-1 and ccw
    ones to r+1."""
    looped, local = _tiny(n, "lhs_rows")
    a, b = _rs_tiny(n, "slice_lhs_rows")
    for sim, args in ((ring.simulate_allgather_einsum_bidir, ("lhs_rows", looped, local)),
                      (ring.simulate_einsum_reducescatter_bidir, ("slice_lhs_rows", a, b))):
        _, sched, transfers = sim(*args)
        assert len(sched) == (n + 1) // 2
        for r in range(n):
            assert sum(1 for t in transfers if t[2] == r) == n - 1
            assert sum(1 for t in transfers if t[3] == r) == n - 1
        for phase, direction, src, dst, _ in transfers:
            assert dst == ((src - 1) % n if direction == "cw" else (src + 1) % n)


@pytest.mark.parametrize("n", list(range(1, 17)))
def test_bidir_every_shard_once(n):
    """AllGather: each rank computes on every shard exactly once.
    ReduceScatter: each slice gets exactly one partial from every rank."""
    looped, local = _tiny(n, "rhs_cols")
    _, sched, _ = ring.simulate_allgather_einsum_bidir("rhs_cols", looped, local)
    for r in range(n):
        seen = [s for row in sched for s in row[r] if s is not None]
        assert sorted(seen) == list(range(n))
    a, b = _rs_tiny(n, "slice_rhs_cols")
    _, sched, _ = ring.simulate_einsum_reducescatter_bidir("slice_rhs_cols", a, b)
    for s in range(n):
        ranks = [r for row in sched for r in range(n) for t in row[r] if t == s]
        assert sorted(ranks) == list(range(n))


def test_bidir_2way_is_one_swap_each_way():
    """N = 2: the prologue (AllGather) or epilogue (ReduceScatter) is the
    only transfer, and the single iteration computes both shards."""
    looped, local = _tiny(2, "lhs_rows")
    _, sched, tr = ring.simulate_allgather_einsum_bidir("lhs_rows", looped, local)
    assert sched == [[(0, 1), (1, 0)]]
    assert [t[0] for t in tr] == ["prologue", "prologue"]
    a, b = _rs_tiny(2, "slice_lhs_rows")
    _, sched, tr = ring.simulate_einsum_reducescatter_bidir("slice_lhs_rows", a, b)
    assert sched == [[(0, 1), (1, 0)]]
    assert [t[0] for t in tr] == ["epilogue", "epilogue"]
