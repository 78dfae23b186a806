"""Pins for the monolithic einsum definitions (oracle.einsum): a pure-Python
triple loop on tiny inputs, the N = 1 reduction to a plain matmul, the fp64
agreement of the simulated loop with the definition on random inputs."""

import numpy as np
import pytest

from oracle import einsum, ring


def _loop_matmul(a, b):
    m, k = a.shape
    k2, n = b.shape
    assert k == k2
    out = [[0.0] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            s = 0.0
            for t in range(k):
                s += float(a[i, t]) * float(b[t, j])
            out[i][j] = s
    return np.array(out)


def _shards(n, mode, rng):
    if mode == "rhs_cols":
        return ([rng.standard_normal((3, 2)) for _ in range(n)],
                [rng.standard_normal((4, 3)) for _ in range(n)])
    if mode == "lhs_rows":
        return ([rng.standard_normal((2, 3)) for _ in range(n)],
                [rng.standard_normal((3, 4)) for _ in range(n)])
    if mode == "lhs_cols":
        return ([rng.standard_normal((4, 2)) for _ in range(n)],
                [rng.standard_normal((2 * n, 3)) for _ in range(n)])
    return ([rng.standard_normal((2, 3)) for _ in range(n)],
            [rng.standard_normal((4, 2 * n)) for _ in range(n)])


@pytest.mark.parametrize("mode", ring.AG_MODES)
def test_allgather_einsum_vs_triple_loop(mode):
    rng = np.random.default_rng(11)
    n = 3
    looped, local = _shards(n, mode, rng)
    got = einsum.allgather_einsum(mode, looped, local)
    for r in range(n):
        # build the gathered operand element by element from partition IDs
        if mode in ("lhs_rows", "lhs_cols"):
            rows = []
            if mode == "lhs_rows":
                for s in range(n):
                    rows.extend(looped[s].tolist())
            else:
                m = looped[0].shape[0]
                rows = [sum((looped[s][i].tolist() for s in range(n)), [])
                        for i in range(m)]
            ref = _loop_matmul(np.array(rows), local[r])
        else:
            if mode == "rhs_cols":
                k = looped[0].shape[0]
                rows = [sum((looped[s][i].tolist() for s in range(n)), [])
                        for i in range(k)]
            else:
                rows = []
                for s in range(n):
                    rows.extend(looped[s].tolist())
            ref = _loop_matmul(local[r], np.array(rows))
        np.testing.assert_allclose(got[r], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("mode", ring.RS_MODES)
def test_einsum_reducescatter_vs_triple_loop(mode):
    rng = np.random.default_rng(12)
    n = 3
    if mode == "slice_lhs_rows":
        a = [rng.standard_normal((2 * n, 4)) for _ in range(n)]
        b = [rng.standard_normal((4, 3)) for _ in range(n)]
    else:
        a = [rng.standard_normal((2, 4)) for _ in range(n)]
        b = [rng.standard_normal((4, 2 * n)) for _ in range(n)]
    got = einsum.einsum_reducescatter(mode, a, b)
    for r in range(n):
        acc = None
        for q in range(n):
            full = _loop_matmul(a[q], b[q])
            part = full[2 * r:2 * r + 2, :] if mode == "slice_lhs_rows" \
                else full[:, 2 * r:2 * r + 2]
            acc = part if acc is None else acc + part
        np.testing.assert_allclose(got[r], acc, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("mode", ring.AG_MODES)
def test_n1_allgather_is_plain_matmul(mode):
    rng = np.random.default_rng(2)
    looped, local = _shards(1, mode, rng)
    got = einsum.allgather_einsum(mode, looped, local)[0]
    if mode in ("lhs_rows", "lhs_cols"):
        ref = looped[0] @ local[0]
    else:
        ref = local[0] @ looped[0]
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("mode", ring.RS_MODES)
def test_n1_reducescatter_is_plain_matmul(mode):
    rng = np.random.default_rng(3)
    a = [rng.standard_normal((5, 4))]
    b = [rng.standard_normal((4, 6))]
    np.testing.assert_array_equal(einsum.einsum_reducescatter(mode, a, b)[0],
                                  a[0] @ b[0])


@pytest.mark.parametrize("mode", ring.AG_MODES)
@pytest.mark.parametrize("n", [2, 4, 8])
def test_loop_agrees_with_definition_random_fp64(mode, n):
    rng = np.random.default_rng(100 + n)
    looped, local = _shards(n, mode, rng)
    outs, _, _ = ring.simulate_allgather_einsum(mode, looped, local)
    ref = einsum.allgather_einsum(mode, looped, local)
    for o, r in zip(outs, ref):
        np.testing.assert_allclose(o, r, rtol=1e-12, atol=1e-12)


def test_local_matmuls():
    rng = np.random.default_rng(4)
    a = [rng.standard_normal((3, 2)) for _ in range(2)]
    b = [rng.standard_normal((2, 4)) for _ in range(2)]
    for got, x, y in zip(einsum.local_matmuls(a, b), a, b):
        np.testing.assert_allclose(got, _loop_matmul(x, y), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("mode", ["rhs_cols", "lhs_rows"])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_allgather_einsum_backward_matches_autograd(mode, n):
    """The AllGather -> ReduceScatter duality of the backward pass, checked
    against torch autograd of the monolithic forward (float64, CPU)."""
    import torch
    rng = np.random.default_rng(77 + n)
    m, k, c = 5, 6, 3
    if mode == "rhs_cols":
        looped = [rng.standard_normal((k, c)) for _ in range(n)]       # B_s [K, n_s]
        local = [rng.standard_normal((m, k)) for _ in range(n)]        # A_r [M, K]
        d_out = [rng.standard_normal((m, n * c)) for _ in range(n)]
    else:
        looped = [rng.standard_normal((m, k)) for _ in range(n)]       # A_s [m_s, K]
        local = [rng.standard_normal((k, c)) for _ in range(n)]        # B_r [K, N]
        d_out = [rng.standard_normal((n * m, c)) for _ in range(n)]
    tl = [torch.tensor(x, requires_grad=True) for x in looped]
    tc = [torch.tensor(x, requires_grad=True) for x in local]
    if mode == "rhs_cols":
        full = torch.cat(tl, dim=1)
        ys = [a @ full for a in tc]
    else:
        full = torch.cat(tl, dim=0)
        ys = [full @ b for b in tc]
    loss = sum((y * torch.tensor(d)).sum() for y, d in zip(ys, d_out))
    loss.backward()
    d_looped, d_local = einsum.allgather_einsum_backward(mode, looped, local, d_out)
    for s in range(n):
        assert np.allclose(d_looped[s], tl[s].grad.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(d_local[s], tc[s].grad.numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Case 3 ([OV] 5.1): the looped LHS split on the batch dim
# ---------------------------------------------------------------------------
def _batch_shards(n, rng, bs=2, m=2, k=3, c=4, integer=False):
    draw = (lambda shape: rng.integers(-4, 5, size=shape).astype(np.float64)) if integer \
        else rng.standard_normal
    looped = [draw((bs, m, k)) for _ in range(n)]          # A_s [b_s, m, k]
    local = [draw((n * bs, k, c)) for _ in range(n)]       # B_r [N b_s, k, n]
    return looped, local


def test_allgather_batch_vs_triple_loop():
    rng = np.random.default_rng(21)
    n, bs = 3, 2
    looped, local = _batch_shards(n, rng, bs)
    got = einsum.allgather_einsum("lhs_batch", looped, local)
    for r in range(n):
        assert got[r].shape == (n * bs, 2, 4)
        for s in range(n):
            for e in range(bs):
                ref = _loop_matmul(looped[s][e], local[r][s * bs + e])
                np.testing.assert_allclose(got[r][s * bs + e], ref, rtol=1e-13, atol=1e-13)


def test_n1_allgather_batch_is_batched_matmul():
    rng = np.random.default_rng(22)
    looped, local = _batch_shards(1, rng, bs=3)
    got = einsum.allgather_einsum("lhs_batch", looped, local)[0]
    for e in range(3):
        np.testing.assert_allclose(got[e], _loop_matmul(looped[0][e], local[0][e]),
                                   rtol=1e-13, atol=1e-13)


def test_allgather_batch_reduces_to_case1_with_one_rhs():
    """When every batch slice of B_r is the same matrix, case 3 is case 1
    (looped LHS split on rows) applied to the shards' stacked rows."""
    rng = np.random.default_rng(23)
    n, bs, m, k, c = 4, 2, 3, 5, 6
    looped = [rng.standard_normal((bs, m, k)) for _ in range(n)]
    b0 = [rng.standard_normal((k, c)) for _ in range(n)]
    local = [np.broadcast_to(b, (n * bs, k, c)).copy() for b in b0]
    got = einsum.allgather_einsum("lhs_batch", looped, local)
    want = einsum.allgather_einsum("lhs_rows", [x.reshape(bs * m, k) for x in looped], b0)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g.reshape(n * bs * m, c), w, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n", [2, 3, 4, 8])
def test_batch_loop_agrees_with_definition(n):
    rng = np.random.default_rng(200 + n)
    looped, local = _batch_shards(n, rng)
    ref = einsum.allgather_einsum("lhs_batch", looped, local)
    outs, sched, _ = ring.simulate_allgather_einsum("lhs_batch", looped, local)
    for o, r in zip(outs, ref):
        np.testing.assert_allclose(o, r, rtol=1e-12, atol=1e-12)
    assert sched == [[(r + i) % n for r in range(n)] for i in range(n)]   # case 1's schedule
    outs2, _, _ = ring.simulate_allgather_einsum_bidir("lhs_batch", looped, local)
    for o, r in zip(outs2, ref):
        np.testing.assert_allclose(o, r, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n", [2, 5])
def test_batch_loop_bit_equal_on_integer_probes(n):
    rng = np.random.default_rng(300 + n)
    looped, local = _batch_shards(n, rng, integer=True)
    ref = einsum.allgather_einsum("lhs_batch", looped, local)
    for sim in (ring.simulate_allgather_einsum, ring.simulate_allgather_einsum_bidir):
        outs = sim("lhs_batch", looped, local)[0]
        for o, r in zip(outs, ref):
            assert np.array_equal(o, r)
