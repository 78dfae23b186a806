"""CPU tests of the C ABI library: it loads, exports every declared symbol,
its shard schedule is the oracle's, its stream/event plans are race-free and
overlap copies with GEMMs, and its host-side validation rejects bad shapes.
No GPU is needed: nothing here launches a kernel."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import ring
import plan_check

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cce.h")


@pytest.fixture(scope="module")
def cce():
    from collective_overlap_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libcce.so is not built (python -m collective_overlap_amd.build)")
    return _lib.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cce_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(cce):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(cce, n), n


def test_status_strings(cce):
    for s in range(5):
        assert cce.cce_status_string(s).decode().startswith("CCE_")
    assert cce.cce_version().decode().count(".") == 2


def test_debug_fail_op_validates(cce):
    """The error-path hook arms and disarms without a device; a negative
    index is rejected."""
    from collective_overlap_amd import cce_debug_fail_op
    from collective_overlap_amd._lib import CceError
    cce_debug_fail_op(3)
    cce_debug_fail_op(0)
    with pytest.raises(CceError) as e:
        cce_debug_fail_op(-1)
    assert e.value.status == 1


@pytest.mark.parametrize("n", list(range(1, 17)) + [31, 64])
def test_shard_schedule_is_the_oracles(n):
    from collective_overlap_amd import cce_shard_schedule
    looped = [np.zeros((1, 1)) for _ in range(n)]
    local = [np.zeros((1, 1)) for _ in range(n)]
    _, ag, _ = ring.simulate_allgather_einsum("lhs_rows", looped, local)
    assert cce_shard_schedule(n, 0) == ag
    a = [np.zeros((n, 1)) for _ in range(n)]
    b = [np.zeros((1, 1)) for _ in range(n)]
    _, rs, _ = ring.simulate_einsum_reducescatter("slice_lhs_rows", a, b)
    assert cce_shard_schedule(n, 1) == rs


def _plan(kind, n, mode, out_t=1, flags=0):
    from collective_overlap_amd import cce_describe_plan
    return cce_describe_plan(kind, n, mode, out_t, flags)


def _shards(op):
    return {int(k): int(v) for k, v in (p.split(":") for p in op.attrs["shard"].split(","))}


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("out_t", [0, 1])
@pytest.mark.parametrize("flags", [0, 1])
def test_allgather_plan_race_free(n, mode, out_t, flags):
    text = _plan(0, n, mode, out_t, flags)
    assert plan_check.check(text) == []


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("flags", [0, 1])
def test_reducescatter_plan_race_free(n, mode, flags):
    text = _plan(1, n, mode, 0, flags)
    assert plan_check.check(text) == []


@pytest.mark.parametrize("n", [2, 4, 8])
def test_allgather_plan_matches_simulated_loop(n):
    ops = plan_check.parse(_plan(0, n, 0))
    looped = [np.zeros((1, 1)) for _ in range(n)]
    _, sched, transfers = ring.simulate_allgather_einsum("lhs_rows", looped, looped)
    gemms = [o for o in ops if o.kind == "gemm"]
    copies = [o for o in ops if o.kind == "copy"]
    assert len(gemms) == n and len(copies) == n - 1        # N-1 hops per rank
    for o in gemms:
        i = int(o.attrs["it"])
        assert _shards(o) == {r: sched[i][r] for r in range(n)}
    for o in copies:
        i = int(o.attrs["it"])
        # the copy of iteration i lands the shard that the simulation's
        # permute of iteration i delivers to each destination rank
        want = {dst: sid for src, dst, sid in transfers[i]}
        assert _shards(o) == want


@pytest.mark.parametrize("n", [2, 4, 8])
def test_reducescatter_plan_matches_simulated_loop(n):
    ops = plan_check.parse(_plan(1, n, 0))
    a = [np.zeros((n, 1)) for _ in range(n)]
    b = [np.zeros((1, 1)) for _ in range(n)]
    _, sched, _ = ring.simulate_einsum_reducescatter("slice_lhs_rows", a, b)
    gemms = [o for o in ops if o.kind == "gemm"]
    assert len(gemms) == 2 * n
    for o in gemms:
        i = int(o.attrs["it"])
        assert _shards(o) == {r: sched[i][r] for r in range(n)}
    assert len([o for o in ops if o.kind == "copy"]) == 2 * (n - 1)


def _is(kind, it, h=None):
    def f(o):
        return (o.kind == kind and int(o.attrs["it"]) == it
                and (h is None or int(o.attrs["h"]) == h))
    return f


@pytest.mark.parametrize("n", [2, 4, 8])
def test_allgather_copy_overlaps_gemm(n):
    text = _plan(0, n, 1)
    for i in range(n - 1):
        assert plan_check.concurrent(text, _is("copy", i), _is("gemm", i))


@pytest.mark.parametrize("n", [2, 4, 8])
def test_reducescatter_half_copies_overlap_other_chain(n):
    text = _plan(1, n, 0)
    for i in range(n - 1):
        assert plan_check.concurrent(text, _is("copy", i, 0), _is("gemm", i, 1))
        assert plan_check.concurrent(text, _is("copy", i, 1), _is("gemm", i + 1, 0))


ONE_CHAIN = 0x40


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("flags", [ONE_CHAIN, ONE_CHAIN | 1, ONE_CHAIN | 0x10, ONE_CHAIN | 0x11])
def test_reducescatter_one_chain_plan_race_free(n, mode, flags):
    text = _plan(1, n, mode, 0, flags)
    assert plan_check.check(text) == []


@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("flags", [ONE_CHAIN, ONE_CHAIN | 1])
def test_reducescatter_one_chain_plan_matches_simulated_loop(n, flags):
    """CCE_FLAG_ONE_CHAIN: one whole-shard chain, n GEMM launches and n - 1
    permutes, each GEMM on the ring's schedule."""
    ops = plan_check.parse(_plan(1, n, 0, 0, flags))
    a = [np.zeros((n, 1)) for _ in range(n)]
    b = [np.zeros((1, 1)) for _ in range(n)]
    _, sched, _ = ring.simulate_einsum_reducescatter("slice_lhs_rows", a, b)
    gemms = [o for o in ops if o.kind == "gemm"]
    assert len(gemms) == n
    assert {int(o.attrs["h"]) for o in gemms} == {0}
    for o in gemms:
        i = int(o.attrs["it"])
        assert _shards(o) == {r: sched[i][r] for r in range(n)}
    assert len([o for o in ops if o.kind == "copy"]) == n - 1


def test_one_chain_leaves_the_fused_and_allgather_plans_alone():
    for kind, mode, fl in ((0, 0, 0), (0, 1, 1), (0, 0, 0x8), (1, 0, 0x8), (1, 1, 0x18)):
        assert _plan(kind, 4, mode, 1, fl | ONE_CHAIN) == _plan(kind, 4, mode, 1, fl)


def test_header_flags_match_the_binding():
    from collective_overlap_amd import _lib
    defs = dict(re.findall(r"#define (CCE_FLAG_[A-Z_]+) (0x[0-9a-f]+)u", open(HEADER).read()))
    assert len(defs) >= 7
    for name, val in defs.items():
        assert getattr(_lib, name) == int(val, 16), name


def test_serial_plan_has_no_copy_stream():
    for kind, mode in ((0, 0), (1, 0)):
        assert all(o.stream == "compute" for o in plan_check.parse(_plan(kind, 4, mode, 1, 1)))


@pytest.mark.parametrize("kind,mode", [(0, 0), (0, 2), (1, 0), (1, 1)])
def test_checker_flags_every_dropped_wait(kind, mode):
    """Each ordering wait of the overlapped plan is necessary: removing any
    single one (a mistake planted in the description, on the CPU) is flagged.
    Waits marked hint=1 only order dispatch (a GEMM waits until the permute
    beside it has started) and are exempt."""
    lines = _plan(kind, 4, mode, 1).strip().splitlines()
    waits = [i for i, l in enumerate(lines) if " wait " in l and "hint=1" not in l]
    assert waits
    for w in waits:
        broken = "\n".join(l for i, l in enumerate(lines) if i != w)
        assert plan_check.check(broken), f"dropping line {w} went unnoticed"


@pytest.mark.parametrize("kind,mode,n,expect", [(0, 1, 4, 3), (1, 0, 4, 6), (0, 1, 1, 0)])
def test_gemms_wait_for_the_permute_beside_them_to_start(kind, mode, n, expect):
    hints = [l for l in _plan(kind, n, mode, 1).splitlines() if "hint=1" in l]
    assert len(hints) == expect
    assert all(l.startswith("compute wait") for l in hints)


def test_checker_flags_wait_before_record():
    text = "copy wait ev=9\ncompute record ev=9\n"
    assert plan_check.check(text)


# ---------------------------------------------------------------------------
# Host-side validation (workspace queries need no device)
# ---------------------------------------------------------------------------

def _ws_ag(cce, n, mode, in_t, out_t, looped, out):
    from collective_overlap_amd._lib import cce_mat
    nb = ctypes.c_size_t()
    s = cce.cce_looped_allgather_einsum_workspace(n, mode, in_t, out_t, cce_mat(*looped),
                                                  cce_mat(*out), ctypes.byref(nb))
    return s, nb.value


def test_allgather_workspace_sizes(cce):
    # case 1, bf16, rhs_cols: two receive buffers of [512, 256] bf16 per rank
    # and direction (the size covers the bidirectional form)
    s, nb = _ws_ag(cce, 4, 1, 1, 1, (512, 256, 256), (64, 2048, 2048))
    assert s == 0 and nb == 2 * 2 * 4 * 512 * 256 * 2
    # case 2 with bf16 output adds an fp32 accumulator per rank
    s, nb2 = _ws_ag(cce, 4, 2, 1, 1, (64, 256, 256), (64, 512, 512))
    assert s == 0 and nb2 == 2 * 4 * 64 * 256 * 2 + 4 * 64 * 512 * 4
    # a single rank needs no workspace
    s, nb = _ws_ag(cce, 1, 1, 1, 1, (512, 256, 256), (64, 512, 512))
    assert s == 0 and nb == 0


@pytest.mark.parametrize("args,status", [
    ((0, 1, 1, 1, (8, 8, 8), (8, 0, 8)), 1),          # n < 1
    ((65, 1, 1, 1, (8, 8, 8), (8, 520, 520)), 2),     # n > max
    ((2, 7, 1, 1, (8, 8, 8), (8, 16, 16)), 1),        # bad mode
    ((2, 1, 5, 1, (8, 8, 8), (8, 16, 16)), 1),        # bad dtype
    ((2, 1, 1, 1, (8, 8, 4), (8, 16, 16)), 1),        # ld < cols
    ((2, 1, 1, 1, (8, 12, 12), (8, 16, 16)), 2),      # ld % 8
    ((2, 1, 1, 1, (8, 8, 8), (8, 24, 24)), 1),        # out cols != n * n_s
    ((2, 0, 1, 1, (8, 8, 8), (15, 8, 8)), 1),         # out rows != n * m_s
])
def test_allgather_validation(cce, args, status):
    s, _ = _ws_ag(cce, *args)
    assert s == status
    assert cce.cce_last_error().decode()


def test_reducescatter_workspace_and_validation(cce):
    from collective_overlap_amd._lib import cce_mat
    nb = ctypes.c_size_t()
    assert cce.cce_looped_einsum_reducescatter_workspace(
        8, 0, 0, cce_mat(2048, 4096, 4096), ctypes.byref(nb)) == 0
    # two chains, two directions; then the chunk signal words of the
    # fine-grained overlap: 2 per (64 x 64)-tile of each of the 8 outputs
    sig = 2 * 8 * (2048 // 64) * (4096 // 64) * 4
    assert nb.value == 2 * 2 * 8 * 2 * 1024 * 4096 * 4 + (sig + 255) // 256 * 256
    # bf16 travelling accumulator is not offered
    assert cce.cce_looped_einsum_reducescatter_workspace(
        8, 0, 1, cce_mat(2048, 4096, 4096), ctypes.byref(nb)) == 2
    assert cce.cce_looped_einsum_reducescatter_workspace(
        8, 3, 0, cce_mat(2048, 4096, 4096), ctypes.byref(nb)) == 1


def test_null_context_rejected_before_any_work(cce):
    from collective_overlap_amd._lib import cce_mat, ptr_array
    arr = ptr_array([0, 0])
    m = cce_mat(8, 8, 8)
    assert cce.cce_looped_allgather_einsum(None, 2, 1, 1, 1, arr, m, arr, m, arr,
                                           cce_mat(8, 16, 16), None, 0, 0, None) == 1
    assert cce.cce_grouped_gemm(None, 2, 1, 1, arr, m, arr, m, arr, m, 0, None) == 1
    import ctypes
    rows0 = (ctypes.c_int64 * 2)(0, 8)
    assert cce.cce_fused_reduce_epilogue_batched(None, 2, 1, 0, arr, m, None, 0, None, 0, 8,
                                                 0.1, 0, 0, rows0, 0, 8, arr, 0, 8, None, 0,
                                                 None) == 1
    assert cce.cce_looped_einsum_reducescatter_epilogue(None, 2, 0, 1, 1, arr, cce_mat(16, 8, 8),
                                                        arr, m, None, None, 8, 0.1, 0, 0, rows0,
                                                        0, 8, arr, m, None, 0, 0, None) == 1


# ---------------------------------------------------------------------------
# Fused permute: the GEMM sends the data itself (no copy stream)
# ---------------------------------------------------------------------------
FUSED = 0x8


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("kind,mode", [(0, 0), (0, 1), (0, 2), (0, 3), (0, 4), (1, 0), (1, 1)])
def test_fused_plans_race_free_and_copy_free(n, kind, mode):
    text = _plan(kind, n, mode, 1, FUSED)
    assert plan_check.check(text) == []
    ops = plan_check.parse(text)
    assert all(o.kind == "gemm" and o.stream == "compute" for o in ops)
    assert len(ops) == n


@pytest.mark.parametrize("n", [2, 4, 8])
def test_fused_allgather_forwards_what_the_ring_moves(n):
    ops = plan_check.parse(_plan(0, n, 0, 1, FUSED))
    looped = [np.zeros((1, 1)) for _ in range(n)]
    _, sched, transfers = ring.simulate_allgather_einsum("lhs_rows", looped, looped)
    for o in ops:
        i = int(o.attrs["it"])
        fwds = [{x for x in w if not x.startswith("out")} for _, w in o.items]
        if i == n - 1:
            assert all(not f for f in fwds)
            continue
        for src, dst, sid in transfers[i]:
            # rank src computes on shard sid and forwards it to rank dst
            assert sched[i][src] == sid
            assert fwds[src] == {f"recv{dst}.p{(i + 1) % 2}"}


def test_fused_reducescatter_sends_accumulators_down_the_ring():
    n = 4
    ops = plan_check.parse(_plan(1, n, 0, 1, FUSED))
    for o in ops[:-1]:
        i = int(o.attrs["it"])
        for r, (_, w) in enumerate(o.items):
            assert w == {f"acc{(r - 1) % n}.p{(i + 1) % 2}.h0"}
    for r, (_, w) in enumerate(ops[-1].items):
        assert w == {f"out{r}.h0"}


def test_checker_flags_intra_launch_conflict():
    """Plant a forward into the buffer another rank reads in the same launch."""
    lines = _plan(0, 4, 0, 1, FUSED).strip().splitlines()
    bad = lines[1].replace(">out0.h0.s1+recv3.p0", ">out0.h0.s1+recv1.p1")
    assert bad != lines[1]
    assert plan_check.check("\n".join([lines[0], bad] + lines[2:]))


# ---------------------------------------------------------------------------
# Bidirectional transfer (Wang et al. ASPLOS'23, Section 5.4.2)
# ---------------------------------------------------------------------------
BIDIR = 0x10


def _items(op):
    """(rank, shard) of each item of a gemm / copy / sum op, in order."""
    return [tuple(int(v) for v in p.split(":")) for p in op.attrs["shard"].split(",")]


@pytest.mark.parametrize("n", list(range(1, 17)) + [31, 32])
def test_bidir_shard_schedule_is_the_oracles(n):
    from collective_overlap_amd import cce_shard_schedule
    looped = [np.zeros((1, 1)) for _ in range(n)]
    _, ag, _ = ring.simulate_allgather_einsum_bidir("lhs_rows", looped, looped)
    assert cce_shard_schedule(n, 2) == ag
    a = [np.zeros((n, 1)) for _ in range(n)]
    b = [np.zeros((1, 1)) for _ in range(n)]
    _, rs, _ = ring.simulate_einsum_reducescatter_bidir("slice_lhs_rows", a, b)
    assert cce_shard_schedule(n, 3) == rs


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 16, 32])
@pytest.mark.parametrize("kind,mode", [(0, 0), (0, 1), (0, 4), (1, 0), (1, 1)])
@pytest.mark.parametrize("extra", [0, 1, 8])
def test_bidir_plans_race_free(n, kind, mode, extra):
    text = _plan(kind, n, mode, 1, BIDIR | extra)
    assert plan_check.check(text) == []


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("flags", [BIDIR, BIDIR | 8])
def test_bidir_allgather_plan_matches_simulated_loop(n, flags):
    """GEMM items follow the oracle's two-way schedule; the transfers (copies,
    or forwards in the fused form) are the oracle's, prologue included."""
    ops = plan_check.parse(_plan(0, n, 0, 1, flags))
    looped = [np.zeros((1, 1)) for _ in range(n)]
    _, sched, transfers = ring.simulate_allgather_einsum_bidir("lhs_rows", looped, looped)
    gemms = [o for o in ops if o.kind == "gemm"]
    assert len(gemms) == (n + 1) // 2
    for o in gemms:
        i = int(o.attrs["it"])
        want = [(r, sched[i][r][0]) for r in range(n)]
        want += [(r, sched[i][r][1]) for r in range(n) if sched[i][r][1] is not None]
        assert _items(o) == want
    # every (destination, shard) the oracle moves appears once: as a copy
    # item, or (fused form) as the forward destination of a GEMM item
    moved = sorted((t[3], t[4]) for t in transfers)
    got = [(r, sid) for o in ops if o.kind == "copy" for r, sid in _items(o)]
    for o in gemms:
        for (_, w), (_, sid) in zip(o.items, _items(o)):
            for x in w:
                m = re.match(r"recv(?:ccw)?(\d+)\.p", x)
                if m:
                    got.append((int(m.group(1)), sid))
    assert sorted(got) == moved


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8])
def test_bidir_reducescatter_plan_matches_simulated_loop(n):
    ops = plan_check.parse(_plan(1, n, 0, 1, BIDIR))
    a = [np.zeros((n, 1)) for _ in range(n)]
    b = [np.zeros((1, 1)) for _ in range(n)]
    _, sched, transfers = ring.simulate_einsum_reducescatter_bidir("slice_lhs_rows", a, b)
    gemms = [o for o in ops if o.kind == "gemm"]
    assert len(gemms) == 2 * ((n + 1) // 2)                 # two chains (halves)
    for o in gemms:
        i = int(o.attrs["it"])
        want = [(r, sched[i][r][0]) for r in range(n)]
        want += [(r, sched[i][r][1]) for r in range(n) if sched[i][r][1] is not None]
        assert _items(o) == want
    copies = [o for o in ops if o.kind == "copy"]
    got = sorted((r, sid) for o in copies if int(o.attrs["h"]) == 0 for r, sid in _items(o))
    assert got == sorted((t[3], t[4]) for t in transfers)
    sums = [o for o in ops if o.kind == "sum"]
    assert len(sums) == (2 if n > 1 else 0)


@pytest.mark.parametrize("kind,mode,n", [(0, 0, 4), (0, 1, 5), (1, 0, 4), (1, 1, 5), (1, 0, 2)])
def test_bidir_checker_flags_every_dropped_wait(kind, mode, n):
    lines = _plan(kind, n, mode, 1, BIDIR).strip().splitlines()
    waits = [i for i, l in enumerate(lines) if " wait " in l and "hint=1" not in l]
    assert waits
    for w in waits:
        broken = "\n".join(l for i, l in enumerate(lines) if i != w)
        assert plan_check.check(broken), f"dropping line {w} went unnoticed"


@pytest.mark.parametrize("n", [4, 8])
def test_bidir_copies_overlap_gemms(n):
    text = _plan(0, n, 1, 1, BIDIR)
    for i in range((n + 1) // 2 - 1):
        assert plan_check.concurrent(text, _is("copy", i), _is("gemm", i))
    text = _plan(1, n, 0, 1, BIDIR)
    for i in range((n + 1) // 2):
        assert plan_check.concurrent(text, _is("copy", i, 0), _is("gemm", i, 1))


def test_bidir_rejects_case2_and_too_many_ranks(cce):
    from collective_overlap_amd._lib import CceError
    with pytest.raises(CceError):
        _plan(0, 4, 2, 1, BIDIR)
    with pytest.raises(CceError):
        _plan(1, 33, 0, 1, BIDIR)


# ---------------------------------------------------------------------------
# Enabling rule and candidate choice (Wang et al. ASPLOS'23, Section 5.5)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("comp,comm,ring_,epi,want", [
    (10.0, 4.0, 8.0, 1.0, 1),     # ring hidden under the einsum: 14 >= 10 + 1
    (10.0, 4.0, 16.0, 1.0, 0),    # ring slower than einsum + collective: 14 < 17
    (10.0, 4.0, 13.0, 1.0, 1),    # boundary: 14 >= 13 + 1 -> loop
    (10.0, 4.0, 8.0, 4.5, 0),     # epilogue too costly: 14 < 14.5
    (2.0, 10.0, 12.0, 0.0, 1),    # communication-bound, ring equal to the original + comp
    (0.0, 0.0, 0.0, 0.0, 1),      # degenerate: equal times loop
    (-1.0, 1.0, 1.0, 0.0, -1),
    (float("nan"), 1.0, 1.0, 0.0, -1),
])
def test_overlap_enabling_rule(cce, comp, comm, ring_, epi, want):
    assert cce.cce_overlap_beneficial(comp, comm, ring_, epi) == want


def test_overlap_enabling_rule_properties(cce):
    """Monotone in each argument: more ring time or epilogue never turns the
    loop on; more original communication never turns it off."""
    rng = np.random.default_rng(0)
    for _ in range(200):
        c, m, r, e = rng.uniform(0, 10, 4)
        d = rng.uniform(0, 5)
        base = cce.cce_overlap_beneficial(c, m, r, e)
        assert cce.cce_overlap_beneficial(c, m, r + d, e) <= base
        assert cce.cce_overlap_beneficial(c, m, r, e + d) <= base
        assert cce.cce_overlap_beneficial(c, m + d, r, e) >= base


@pytest.mark.parametrize("comp,c0,s0,c1,s1,want", [
    (1.0, 5.0, 100.0, 6.0, 50.0, 1),   # einsum faster than both: smaller shard
    (1.0, 5.0, 50.0, 6.0, 100.0, 0),
    (1.0, 5.0, 70.0, 6.0, 70.0, 0),    # tie on shard size -> candidate 0
    (8.0, 5.0, 50.0, 6.0, 100.0, 1),   # otherwise the longer collective
    (8.0, 7.0, 50.0, 6.0, 10.0, 0),
    (5.5, 5.0, 50.0, 6.0, 10.0, 1),    # faster than only one: longer collective
    (1.0, -5.0, 50.0, 6.0, 10.0, -1),
])
def test_overlap_candidate_choice(cce, comp, c0, s0, c1, s1, want):
    assert cce.cce_overlap_choose(comp, c0, s0, c1, s1) == want


# ---------------------------------------------------------------------------
# The build's spill guard (collective_overlap_amd/build.py)
# ---------------------------------------------------------------------------
def test_spill_guard_reads_the_compiler_remarks():
    from collective_overlap_amd import build
    remarks = "\n".join([
        "x.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]",
    ])
    sc = build.scratch_by_kernel(remarks)
    assert sc == {"kern_a": 0, "kern_b": 12}
    assert build.check_spills(sc, known={}) == ["kern_b: 12 bytes/lane (allowed 0)"]
    assert build.check_spills(sc, known={"kern_b": 12}) == []
    assert build.check_spills(sc, known={"kern_b": 8}) == ["kern_b: 12 bytes/lane (allowed 8)"]



def test_sources_of_a_revision_are_that_revisions():
    """build.py --rev writes a revision's library sources beside the working
    tree for an A/B build: for HEAD they are the committed files, byte for
    byte, and the header is that revision's."""
    import subprocess
    from collective_overlap_amd import build
    if subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True).returncode != 0:
        pytest.skip("not a git checkout")
    csrc = build.sources_at("HEAD")
    ls = subprocess.run(["git", "-C", ROOT, "ls-tree", "--name-only", "HEAD:collective_overlap_amd/csrc"],
                        capture_output=True, text=True).stdout.split()
    assert "gemm.hip" in ls and sorted(os.listdir(csrc)) == sorted(ls)
    for f in ls:
        want = subprocess.run(["git", "-C", ROOT, "show", f"HEAD:collective_overlap_amd/csrc/{f}"],
                              capture_output=True).stdout
        assert open(os.path.join(csrc, f), "rb").read() == want, f
    hdr = os.path.join(os.path.dirname(os.path.dirname(csrc)), "include", "cce.h")
    want = subprocess.run(["git", "-C", ROOT, "show", "HEAD:include/cce.h"], capture_output=True).stdout
    assert open(hdr, "rb").read() == want
