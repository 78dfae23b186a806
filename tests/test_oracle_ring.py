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
