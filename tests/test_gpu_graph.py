"""The entry points under HIP graph capture (torch.cuda.CUDAGraph).

A call with a caller-supplied workspace allocates nothing and clears what
must start at zero with a fill kernel, never with a memset; the fused and
serial forms run on the caller's stream alone, and the stream form forks its
copy stream from the caller's stream by events and joins it back, which
capture turns into graph edges.  So a looped step can be captured once and
replayed: that removes the host's per-launch work, which is most of a
latency-bound step.

Each case runs the call eagerly first (the reference bits), captures it,
and replays the graph several times.  Between replays the program does eager
work of its own on the same buffers: the outputs are poisoned with NaN and
the same entry point runs eagerly on other inputs into the same outputs and
workspace, followed by a synchronisation.  Every replay must then reproduce
the reference bit for bit: a graph that depended on state an eager call
leaves behind, or a captured node that misbehaved on a later replay, would
fail."""

import pytest
import torch

import workloads as W
from gpu_util import sync

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16
REPLAYS = 3


@pytest.fixture(scope="module")
def ctx():
    import collective_overlap_amd as cce
    c = cce.Context(0)
    yield c
    sync()
    c.close()


def _bits(t):
    return t.view(torch.int16 if t.dtype == BF else torch.int32)


def _replay_and_check(run, run_other, outs):
    """run(): the captured call (writes `outs`); run_other(): the same entry
    point on other inputs into the same outputs and workspace (eager)."""
    run()
    sync()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    sync()
    for rep in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        run_other()
        sync()
        g.replay()
        sync()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(_bits(o), _bits(r)), f"replay {rep}: output {i} differs"
    del g
    sync()


# permute forms: fused two-way (the benchmark's), fused one-way, copy stream
# (fork/join), serial (the runtime's copies on the caller's stream)
FORMS = [0x18, 0x8, 0x0, 0x1]


@pytest.mark.parametrize("flags", FORMS)
def test_allgather_einsum_with_gelu(ctx, flags):
    import collective_overlap_amd as cce
    print(f"[gpu] graph allgather flags={flags:#x}", flush=True)
    n, m, k, c = 4, 200, 264, 136
    sets = [([W.normal((c, k), 0.05, 10 * s + r, device=DEV, dtype=BF) for r in range(n)],
             [W.normal((m, k), 1.0, 10 * s + 5 + r, device=DEV, dtype=BF) for r in range(n)])
            for s in (0, 1)]
    out = [torch.empty((m, n * c), device=DEV, dtype=BF) for _ in range(n)]
    ws = torch.empty(cce.cce_looped_allgather_einsum_workspace(n, "rhs_cols", BF, BF, (c, k), (m, n * c)),
                     dtype=torch.uint8, device=DEV)
    f = flags | cce.CCE_FLAG_GELU

    def call(s):
        cce.cce_looped_allgather_einsum(ctx, "rhs_cols", sets[s][0], sets[s][1], out,
                                        workspace=ws, flags=f)

    _replay_and_check(lambda: call(0), lambda: call(1), out)


@pytest.mark.parametrize("flags", FORMS + [0x38, 0x28])   # + fine-grained, two-way / one-way
def test_reducescatter_with_epilogue(ctx, flags):
    import collective_overlap_amd as cce
    print(f"[gpu] graph reducescatter+epilogue flags={flags:#x}", flush=True)
    n, s, k, c = 4, 136, 264, 200
    sets = [([W.normal((n * s, k), 1.0, 10 * q + r, device=DEV, dtype=BF) for r in range(n)],
             [W.normal((c, k), 0.05, 10 * q + 5 + r, device=DEV, dtype=BF) for r in range(n)])
            for q in (2, 3)]
    bias = W.normal((c,), 0.02, 90, device=DEV, dtype=BF)
    res = [W.normal((s, c), 1.0, 91 + r, device=DEV, dtype=BF) for r in range(n)]
    out = [torch.empty((s, c), device=DEV, dtype=BF) for _ in range(n)]
    ws = torch.empty(cce.cce_looped_einsum_reducescatter_workspace(n, "slice_lhs_rows", (s, c, c)),
                     dtype=torch.uint8, device=DEV)
    rows0 = [r * s for r in range(n)]

    def call(q):
        cce.cce_looped_einsum_reducescatter_epilogue(
            ctx, "slice_lhs_rows", sets[q][0], sets[q][1], bias, res, out, 0.1, 7, 3,
            mask_row0=rows0, mask_col0=0, mask_ld=c, workspace=ws, flags=flags)

    _replay_and_check(lambda: call(0), lambda: call(1), out)
    ctx.check_signals()           # no fine-grained consumer gave up


def test_epilogue_and_grouped_gemm(ctx):
    import collective_overlap_amd as cce
    print("[gpu] graph epilogue + grouped gemm", flush=True)
    rows, cols = 192, 320
    parts = [[W.normal((rows, cols), 1.0, 10 * q + k, device=DEV) for k in range(3)] for q in (4, 5)]
    bias = W.normal((cols,), 0.02, 60, device=DEV)
    res = W.normal((rows, cols), 1.0, 61, device=DEV)
    out = torch.empty((rows, cols), device=DEV, dtype=BF)
    a = [[W.normal((300, 128), 1.0, 70 + 10 * q + g, device=DEV, dtype=BF) for g in range(3)] for q in (0, 1)]
    b = [[W.normal((264, 128), 0.05, 75 + 10 * q + g, device=DEV, dtype=BF) for g in range(3)] for q in (0, 1)]
    cg = [torch.empty((300, 264), device=DEV, dtype=BF) for _ in range(3)]

    def call(q):
        cce.cce_fused_reduce_epilogue(ctx, parts[q], bias, res, out, 0.1, 5, 0)
        cce.cce_grouped_gemm(ctx, a[q], b[q], cg, gelu=True)

    _replay_and_check(lambda: call(0), lambda: call(1), [out] + cg)


def test_benchmark_step_of_the_two_rank_fp32_workload(ctx):
    """The latency-bound workload's whole step (fp32 AllGather-Einsum in the
    benchmark's form and the fused epilogue), as bench.py replays it."""
    import collective_overlap_amd as cce
    import bench
    print("[gpu] graph ag_fp32_n2 step", flush=True)
    steps = [bench.WORKLOADS["ag_fp32_n2"](DEV) for _ in range(2)]
    for t in steps[1].X + steps[1].Wt + steps[1].P:
        t.mul_(0.5)
    steps[1].Y, steps[1].out = steps[0].Y, steps[0].out      # same outputs
    f = cce.CCE_FLAG_FUSED_PERMUTE | bench.preferred_bid("ag_fp32_n2")
    _replay_and_check(lambda: steps[0].run(ctx, f), lambda: steps[1].run(ctx, f),
                      steps[0].Y + [steps[0].out])
