"""Happens-before race checker for the library's plan descriptions
(cce_describe_plan).  Pure Python, CPU only.

Model: ops on one stream run in the order they were enqueued; a `wait ev=e`
orders everything after it on its stream after everything up to the most
recent `record ev=e` enqueued before the wait (a wait with no earlier record
waits for nothing).  The caller's own work is modelled as a virtual op at the
start and one at the end of the compute stream that touch every buffer.

A plan is race-free when every pair of operations that touch a common buffer,
at least one of them writing it, is ordered by happens-before in the same
direction as the host enqueue order (which is the sequential semantics: the
serial plan runs exactly that order on one stream).
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass
class POp:
    idx: int
    stream: str
    kind: str
    attrs: dict = field(default_factory=dict)
    reads: set = field(default_factory=set)
    writes: set = field(default_factory=set)
    items: list = field(default_factory=list)   # per rank: (reads, writes)
    pairs: list = field(default_factory=list)   # item pairs that claim chunks together


def parse(text: str) -> list[POp]:
    ops = []
    for line in text.strip().splitlines():
        parts = line.split()
        stream, kind = parts[0], parts[1]
        attrs = {}
        for p in parts[2:]:
            k, v = p.split("=", 1)
            attrs[k] = v
        op = POp(len(ops), stream, kind, attrs)
        if kind in ("gemm", "copy", "sum"):
            op.reads = set(attrs["r"].split(","))
            op.writes = set(attrs["w"].split(","))
            op.items = [(set(x.split(">")[0].split("+")), set(x.split(">")[1].split("+")))
                        for x in attrs.get("x", "").split(",") if x]
            op.pairs = [tuple(int(v) for v in pr.split(":"))
                        for pr in attrs.get("pairs", "").split(",") if pr]
        ops.append(op)
    return ops


def _with_caller(ops: list[POp]) -> list[POp]:
    bufs = set()
    for o in ops:
        bufs |= o.reads | o.writes
    start = POp(0, "compute", "caller", {}, set(), set(bufs))
    body = [POp(o.idx + 1, o.stream, o.kind, o.attrs, o.reads, o.writes) for o in ops]
    end = POp(len(ops) + 1, "compute", "caller", {}, set(bufs), set(bufs))
    return [start] + body + [end]


def happens_before(ops: list[POp], hints: bool = True):
    """Return (succ adjacency, problems) for the HB graph.  Waits marked
    hint=1 only order dispatch; with hints=False they are left out, so a plan
    must be race-free without them."""
    n = len(ops)
    succ = [set() for _ in range(n)]
    problems = []
    last_on = {}
    last_record = {}
    for o in ops:
        prev = last_on.get(o.stream)
        if prev is not None:
            succ[prev].add(o.idx)
        last_on[o.stream] = o.idx
        if o.kind == "record":
            last_record[o.attrs["ev"]] = o.idx
        elif o.kind == "wait":
            if not hints and o.attrs.get("hint") == "1":
                continue
            r = last_record.get(o.attrs["ev"])
            if r is None:
                problems.append(f"op {o.idx}: wait on ev={o.attrs['ev']} before any record")
            else:
                succ[r].add(o.idx)
    return succ, problems


def _reach(succ):
    n = len(succ)
    reach = []
    for s in range(n):
        seen = set()
        stack = [s]
        while stack:
            u = stack.pop()
            for v in succ[u]:
                if v not in seen:
                    seen.add(v)
                    stack.append(v)
        reach.append(seen)
    return reach


def intra_op_conflicts(op: POp) -> list[str]:
    """The items of one operation run concurrently (one kernel, or one
    batch of copies): no item may write what another item touches, and an
    item may overlap its own reads only by updating a buffer in place
    (its accumulator input is its output).  The one exception is a declared
    pair of a fine-grained launch (pairs=i:j): both name the output chunk
    among their writes, and the chunk claim lets exactly one of them write
    it; every other buffer they share is still a conflict."""
    out = []
    paired = {(i, j) for i, j in op.pairs} | {(j, i) for i, j in op.pairs}
    for i, (ri, wi) in enumerate(op.items):
        for j, (rj, wj) in enumerate(op.items):
            if i == j:
                continue
            shared = wi & (rj | wj)
            if (i, j) in paired:
                shared = {b for b in shared if not (b.startswith("out") and b in wj and b not in rj)}
            if shared:
                out.append(f"op {op.idx}: item {i} writes {sorted(shared)} used by item {j}")
        own = wi & ri
        if own and not (op.kind == "gemm" and len(own) == 1 and len(ri) == 3):
            out.append(f"op {op.idx}: item {i} reads and writes {sorted(own)}")
    return out


def check(text: str) -> list[str]:
    """List of problems (empty when the plan is race-free)."""
    problems = []
    for op in parse(text):
        problems += intra_op_conflicts(op)
    ops = _with_caller(parse(text))
    succ, hb_problems = happens_before(ops, hints=False)
    problems += hb_problems
    reach = _reach(succ)
    acc = [o for o in ops if o.kind in ("gemm", "copy", "sum", "caller")]
    for i, x in enumerate(acc):
        for y in acc[i + 1:]:
            conflict = (x.writes & (y.reads | y.writes)) or (y.writes & x.reads)
            if conflict and y.idx not in reach[x.idx]:
                problems.append(f"race: op {x.idx} ({x.stream} {x.kind} {x.attrs.get('it')}) "
                                f"and op {y.idx} ({y.stream} {y.kind} {y.attrs.get('it')}) "
                                f"on {sorted(conflict)[:3]}")
    return problems


def concurrent(text: str, a_pred, b_pred) -> bool:
    """True if some op matching a_pred and some op matching b_pred are not
    ordered by happens-before (they may overlap in time)."""
    ops = parse(text)
    succ, _ = happens_before(ops)
    reach = _reach(succ)
    for x in ops:
        if not a_pred(x):
            continue
        for y in ops:
            if y is x or not b_pred(y):
                continue
            if y.idx not in reach[x.idx] and x.idx not in reach[y.idx]:
                return True
    return False
