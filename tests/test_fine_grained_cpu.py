"""CPU tests of the fine-grained overlap (CCE_FLAG_FINE_GRAINED; CoCoNet's
fine-grained overlap of a MatMul with the collective that consumes it, chunk
by chunk): the plans the library builds for it, checked for races, and the
per-chunk claim protocol its last launch runs, checked by exhaustive search
over every interleaving of two producers.  No GPU is needed."""

import re

import pytest

import plan_check

FUSED, BIDIR, SERIAL, FINE = 0x8, 0x10, 0x1, 0x20


def _plan(kind, n, mode, flags, out_t=1):
    from collective_overlap_amd import cce_describe_plan
    return cce_describe_plan(kind, n, mode, out_t, flags)


# ---------------------------------------------------------------------------
# Plans
# ---------------------------------------------------------------------------
FORMS = [
    (1, BIDIR | FUSED), (2, BIDIR | FUSED),                 # two-way fused
    (2, 0), (2, FUSED), (2, SERIAL),                        # one-way with the epilogue
    (1, 0), (1, FUSED),                                     # one-way, no consumer to move
]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 16, 32])
@pytest.mark.parametrize("kind,flags", FORMS)
@pytest.mark.parametrize("mode", [0, 1])
def test_fine_plans_race_free(n, kind, flags, mode):
    if flags & BIDIR and n > 32:
        pytest.skip("two-way ring takes at most 32 ranks")
    assert plan_check.check(_plan(kind, n, mode, flags | FINE)) == []


def _final(ops):
    return [o for o in ops if o.kind == "gemm" and o.attrs["epi"] == "2"]


@pytest.mark.parametrize("n", [2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("kind", [1, 2])
def test_two_way_last_launch_consumes_every_chunk(n, kind):
    """The align-and-sum op is gone; the last GEMM launch writes every
    output.  With n even both last partials of output s are in that launch
    (the cw item of rank s and the ccw item of rank s-1) and form a declared
    pair; with n odd the ccw chain ended one launch earlier and the cw item
    reads its finished accumulator."""
    ops = plan_check.parse(_plan(kind, n, 0, BIDIR | FUSED | FINE))
    assert not any(o.kind == "sum" for o in ops)
    fin = _final(ops)
    assert len(fin) == 1 and fin[0] is [o for o in ops if o.kind == "gemm"][-1]
    op = fin[0]
    outs = {}
    for q, (r, w) in enumerate(op.items):
        out = [b for b in w if b.startswith("out")]
        assert len(out) == 1
        outs.setdefault(out[0], []).append(q)
    assert sorted(outs) == sorted(f"out{s}.h0" for s in range(n))
    ranks = [int(x.split(":")[0]) for x in op.attrs["shard"].split(",")]
    if n % 2 == 0:
        pairs = {tuple(sorted(p)) for p in op.pairs}
        assert pairs == {tuple(sorted(v)) for v in outs.values()}
        for s in range(n):
            cw, ccw = outs[f"out{s}.h0"]
            assert ranks[cw] == s and ranks[ccw] == (s - 1) % n
            # each stores its partial at its own final accumulator when first
            assert f"acc{s}.p{(n // 2 - 1) % 2}.h0" in op.items[cw][1]
            assert f"accccw{s}.p{(n // 2) % 2}.h0" in op.items[ccw][1]
    else:
        assert op.pairs == []
        for s in range(n):
            (cw,) = outs[f"out{s}.h0"]
            assert ranks[cw] == s
            assert f"accccw{s}.p{(n // 2) % 2}.h0" in op.items[cw][0]


@pytest.mark.parametrize("n", [2, 3, 8])
@pytest.mark.parametrize("flags", [0, FUSED, SERIAL])
def test_one_way_epilogue_consumed_in_the_last_launches(n, flags):
    ops = plan_check.parse(_plan(2, n, 0, flags | FINE))
    base = plan_check.parse(_plan(2, n, 0, flags))
    fin = _final(ops)
    halves = 1 if flags & FUSED else 2
    assert len(fin) == halves
    for o in fin:
        assert o.pairs == []
        assert all(any(b.startswith("out") for b in w) for _, w in o.items)
    # otherwise the same operations in the same order
    assert [(o.stream, o.kind) for o in ops] == [(o.stream, o.kind) for o in base]


def test_flag_changes_nothing_without_a_consumer():
    for flags in (0, FUSED, SERIAL):
        assert _plan(1, 8, 0, flags | FINE) == _plan(1, 8, 0, flags)


def test_two_way_with_copies_rejected():
    from collective_overlap_amd import _lib
    with pytest.raises(_lib.CceError) as e:
        _plan(1, 4, 0, BIDIR | FINE)
    assert e.value.status == _lib.CCE_EUNSUPPORTED


def test_checker_exempts_only_declared_pairs():
    """Drop the pairs= annotation: the two items writing one output chunk are
    then a conflict.  Plant another shared write into a declared pair: still
    a conflict."""
    text = _plan(1, 4, 0, BIDIR | FUSED | FINE)
    assert plan_check.check(text) == []
    assert plan_check.check(re.sub(r" pairs=\S+", "", text))
    lines = text.strip().splitlines()
    k = next(i for i, l in enumerate(lines) if " epi=2 " in l)
    op = plan_check.parse(lines[k])[0]
    i, j = op.pairs[0]
    meet_i = sorted(b for b in op.items[i][1] if not b.startswith("out"))[0]
    bad = lines[k]
    xs = bad.split(" x=")[1].split(" ")[0].split(",")
    xs[j] = xs[j] + "+" + meet_i
    bad = bad.replace(" x=" + bad.split(" x=")[1].split(" ")[0], " x=" + ",".join(xs))
    assert plan_check.check("\n".join(lines[:k] + [bad] + lines[k + 1:]))


# ---------------------------------------------------------------------------
# The per-chunk claim protocol (claim_chunk / publish_chunk in the GEMM),
# explored over every interleaving of its two producers' atomic steps.
#
# Producer program, in order:
#   claim:   old = counter; counter = old + 1   (one atomic read-modify-write)
#   old == 0 (first):  store its partial; publish (ready = 1, unless the
#                      test hook withholds it); done
#   old == 1 (second): poll ready up to `cap` times; if seen: read the
#                      pair's partial, write the output chunk; else count a
#                      give-up and write nothing; done
# ---------------------------------------------------------------------------
def _explore(cap, publish=True, fair=False):
    """Every interleaving (fair: only those in which a producer polls again
    only after the other has taken a step, or has finished -- both
    workgroups run at once on the GPU and a poll sleeps); returns the set of
    final outcomes and checks the safety properties on every path."""
    outcomes = set()

    def step(state, who):
        st = dict(state)
        pc = st[f"pc{who}"]
        if pc == "claim":
            st[f"role{who}"] = 1 if st["counter"] == 0 else 2
            st["counter"] += 1
            st[f"pc{who}"] = "store" if st[f"role{who}"] == 1 else "poll"
        elif pc == "store":
            st[f"part{who}"] = True
            st[f"pc{who}"] = "publish"
        elif pc == "publish":
            if publish:
                st["ready"] = True
            st[f"pc{who}"] = "done"
        elif pc == "poll":
            if st["ready"]:
                st[f"pc{who}"] = "read"
            else:
                st[f"polls{who}"] += 1
                if st[f"polls{who}"] >= cap:
                    st["gaveup"] += 1
                    st[f"pc{who}"] = "done"
        elif pc == "read":
            other = 1 - who
            # the pair's partial must already be stored when it is read
            assert st[f"part{other}"], "read before the partner's store"
            st[f"pc{who}"] = "write"
        elif pc == "write":
            st["writes"] += 1
            st[f"pc{who}"] = "done"
        return st

    start = {"counter": 0, "ready": False, "writes": 0, "gaveup": 0,
             "pc0": "claim", "pc1": "claim", "role0": 0, "role1": 0,
             "part0": False, "part1": False, "polls0": 0, "polls1": 0, "last": -1}
    stack = [(start, 0)]
    while stack:
        st, depth = stack.pop()
        assert depth < 64, "a producer never finishes"
        live = [w for w in (0, 1) if st[f"pc{w}"] != "done"]
        if not live:
            outcomes.add((st["writes"], st["gaveup"], st["role0"], st["role1"]))
            continue
        for w in live:
            if (fair and st[f"pc{w}"] == "poll" and st["last"] == w
                    and st[f"pc{1 - w}"] != "done"):
                continue
            nxt = step(st, w)
            nxt["last"] = w
            stack.append((nxt, depth + 1))
    return outcomes


@pytest.mark.parametrize("cap", [1, 3, 6])
def test_claim_protocol_safe_on_every_interleaving(cap):
    """Whoever claims first stores and publishes; the chunk is written at
    most once, only by the second claimant and only after the first's
    partial is stored (asserted inside the search); both producers finish;
    a chunk left unwritten is always counted as a give-up."""
    for writes, gaveup, r0, r1 in _explore(cap=cap):
        assert {r0, r1} == {1, 2}
        assert writes + gaveup == 1


@pytest.mark.parametrize("cap", [3, 6, 1 << 18])
def test_claim_protocol_no_give_up_when_both_run(cap):
    """With both producers making progress (fair interleavings), the second
    sees the ready word within the first's two remaining steps: three polls
    suffice, and the kernels allow 2^18."""
    assert _explore(cap=cap, fair=True) == {(1, 0, 1, 2), (1, 0, 2, 1)}


@pytest.mark.parametrize("cap", [1, 2, 5])
def test_claim_protocol_give_up_when_ready_is_withheld(cap):
    """The test hook's condition: the first producer does not publish.  The
    second polls cap times, counts one give-up, writes nothing, and both
    producers finish on every interleaving."""
    outs = _explore(cap=cap, publish=False)
    assert outs == {(0, 1, 1, 2), (0, 1, 2, 1)}


def test_claim_protocol_counter_layout_matches_workspace():
    """Two 32-bit words per chunk (claim, ready), one chunk per (64 x 64)
    tile of each output (the smallest tile of any GEMM kernel): the workspace
    query holds them after the accumulators."""
    import ctypes
    from collective_overlap_amd import _lib
    lib = _lib.lib()
    nb = ctypes.c_size_t()
    for n, rows, cols in [(2, 64, 64), (8, 1024, 12288), (3, 129, 257)]:
        assert lib.cce_looped_einsum_reducescatter_workspace(
            n, 0, 0, _lib.cce_mat(rows, cols, cols + (-cols) % 8), ctypes.byref(nb)) == 0
        words = 2 * n * (-(-rows // 64)) * (-(-cols // 64))
        h0 = (rows + 1) // 2
        ld2, ld1 = cols + (-cols) % 8, cols + (-cols) % 8
        slot2 = -(-h0 * ld2 * 4 // 256) * 256
        slot1 = -(-rows * ld1 * 4 // 256) * 256
        region = max(2 * n * slot1, 2 * n * 2 * slot2)
        assert nb.value == 2 * region + -(-4 * words // 256) * 256
