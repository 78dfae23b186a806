"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Sizes here finish in the oracle within seconds yet span several tiles and
ragged tails in M, N and K.  Float results are compared with the float64
oracle on the exact bf16/fp32 input values; integer-valued probes make every
fp32 sum exact, so those must match bit for bit."""

import numpy as np
import pytest
import torch

from oracle import einsum as oe
from oracle import numerics
import workloads as W
from gpu_util import np64, assert_bf16_close, assert_f32_close, sync

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def ctx():
    import collective_overlap_amd as cce
    print(f"[gpu] libcce {cce.cce_version()} on {torch.cuda.get_device_name(0)}", flush=True)
    c = cce.Context(0)
    yield c
    sync()
    c.close()


def _t(shape, k, dtype, probe, ld=None):
    rows, cols = shape
    full_cols = ld if ld is not None else cols
    if probe:
        x = W.int_probe((rows, full_cols), k, device=DEV, dtype=dtype)
    else:
        x = W.normal((rows, full_cols), 1.0, k, device=DEV, dtype=dtype)
    return x[:, :cols] if ld is not None else x


# ---------------------------------------------------------------------------
# grouped GEMM
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K,G", [(256, 256, 64, 1), (300, 200, 136, 3), (1000, 520, 264, 2),
                                     (2048, 1024, 512, 4), (17, 24, 8, 2), (512, 768, 0, 1)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_grouped_gemm(ctx, M, N, K, G, dt):
    import collective_overlap_amd as cce
    print(f"[gpu] grouped_gemm M={M} N={N} K={K} G={G} {dt}", flush=True)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    a = [_t((M, K), 10 + g, dtype, False) for g in range(G)]
    b = [_t((N, K), 20 + g, dtype, False) for g in range(G)]
    c32 = [torch.full((M, N), float("nan"), device=DEV) for _ in range(G)]
    cce.cce_grouped_gemm(ctx, a, b, c32)
    c16 = [torch.empty((M, N), device=DEV, dtype=torch.bfloat16) for _ in range(G)]
    cce.cce_grouped_gemm(ctx, a, b, c16)
    sync()
    for g in range(G):
        ref = oe.local_matmuls([np64(a[g])], [np64(b[g]).T])[0]
        assert_f32_close(np64(c32[g]), ref, f"group {g} fp32 out", tol=1e-5)
        assert_bf16_close(np64(c16[g]), ref, f"group {g} bf16 out")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_grouped_gemm_integer_probe_bit_exact(ctx, dt):
    import collective_overlap_amd as cce
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    M, N, K, G = 600, 392, 1032, 3
    a = [_t((M, K), 30 + g, dtype, True) for g in range(G)]
    b = [_t((N, K), 40 + g, dtype, True) for g in range(G)]
    c = [torch.empty((M, N), device=DEV) for _ in range(G)]
    cce.cce_grouped_gemm(ctx, a, b, c)
    sync()
    for g in range(G):
        ref = np64(a[g]) @ np64(b[g]).T
        assert np.array_equal(np64(c[g]), ref)


def test_gelu_device_values_within_the_erf_bound(ctx):
    """The store epilogue's GELU, element by element, against the exact
    fp64 definition.  The GEMM passes every bf16 value x in [-2^4, 2^4)
    through exactly (A[:, 0] = x, B^T[:, 0] = 1, all else 0), so the fp32
    output is GELU evaluated at x.  The device forms erf with the rational
    approximation of Abramowitz and Stegun 7.1.26 (|error| <= 1.5e-7) in
    fp32; allowing 6e-7 more for the fp32 evaluation of that formula, the
    error of 1 + erf is below 7.5e-7, hence the bound 0.5 |x| 7.5e-7 plus
    two fp32 ulps of the result."""
    import collective_overlap_amd as cce
    sign = np.array([1.0, -1.0])[:, None, None]
    exps = np.arange(-20, 4)[None, :, None].astype(np.float64)
    mant = (1.0 + np.arange(128) / 128.0)[None, None, :]
    x = np.concatenate([(sign * mant * 2.0 ** exps).ravel(), [0.0]])
    M, K, N = x.size, 8, 8
    a = torch.zeros((M, K), dtype=torch.bfloat16)
    a[:, 0] = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(a[:, 0].double().numpy(), x)        # exact in bf16
    b = torch.zeros((N, K), dtype=torch.bfloat16)
    b[:, 0] = 1.0
    c = torch.full((M, N), float("nan"), device=DEV)
    cce.cce_grouped_gemm(ctx, [a.to(DEV)], [b.to(DEV)], [c], gelu=True)
    sync()
    got = np64(c)
    ref = numerics.gelu(x)[:, None]
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    bound = 0.5 * np.abs(x)[:, None] * 7.5e-7 + 2 * ulp
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), (f"x={x[worst[0]]!r} got={got[worst]!r} ref={ref[worst[0], 0]!r} "
                                  f"err={err[worst]:.3e} bound={bound[worst]:.3e}")
    assert got[-1, 0] == 0.0                                   # GELU(0) = 0


# bf16 results of launches with more tiles than CUs (several rounds of
# workgroups), ragged rows (edge tiles take the element-wise store path),
# one to 17 k tiles, the 256 x 128 tile shape, and a padded output row
# stride whose padding must stay untouched.
MANY_TILE_CASES = [
    # G, M, N, K, output ld (None: N)
    (2, 4000, 4096, 200, None),       # 512 tiles of 256x256, ragged rows, 4 k tiles
    (1, 8192, 8192, 64, None),        # 1024 tiles, one k tile
    (3, 1024, 4096, 1000, 4104),      # 192 tiles of 256x256 -> 256x128 tiles, padded ld
    (4, 2048, 2048, 1032, None),      # 256 tiles: one per workgroup, 17 k tiles
]


@pytest.mark.parametrize("G,M,N,K,ld", MANY_TILE_CASES)
def test_grouped_gemm_many_tiles_bf16_integer_probe(ctx, G, M, N, K, ld):
    import collective_overlap_amd as cce
    print(f"[gpu] grouped_gemm many tiles G={G} M={M} N={N} K={K} ld={ld}", flush=True)
    a = [_t((M, K), 60 + g, torch.bfloat16, True) for g in range(G)]
    b = [_t((N, K), 70 + g, torch.bfloat16, True) for g in range(G)]
    if ld is None:
        bigs = [torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16) for _ in range(G)]
        c = bigs
    else:
        bigs = [torch.zeros((M, ld), device=DEV, dtype=torch.bfloat16) for _ in range(G)]
        c = [x[:, :N] for x in bigs]
    cce.cce_grouped_gemm(ctx, a, b, c)
    sync()
    for g in range(G):
        # exact integers in fp32, rounded once to bf16
        ref = numerics.bf16_round(np64(a[g]) @ np64(b[g]).T)
        assert np.array_equal(np64(c[g]), ref), f"group {g}"
        if ld is not None:
            assert torch.count_nonzero(bigs[g][:, N:]) == 0     # padding untouched


def test_grouped_gemm_gelu_and_strided(ctx):
    import collective_overlap_amd as cce
    M, N, K = 384, 261, 200
    a = [_t((M, K), 50, torch.bfloat16, False, ld=208)]
    b = [_t((N, K), 51, torch.bfloat16, False, ld=216)]
    big = torch.zeros((M, 272), device=DEV, dtype=torch.bfloat16)
    c = [big[:, :N]]
    cce.cce_grouped_gemm(ctx, a, b, c, gelu=True)
    sync()
    ref = numerics.gelu(np64(a[0]) @ np64(b[0]).T)
    assert_bf16_close(np64(c[0]), ref, "gelu strided")
    assert torch.count_nonzero(big[:, N:]) == 0     # padding untouched


# ---------------------------------------------------------------------------
# looped AllGather-Einsum
# ---------------------------------------------------------------------------
def _ag_inputs(mode, n, dims, dtype, probe, seed=0):
    """Storage-orientation device tensors and math-orientation oracle inputs."""
    m, k, c = dims           # m: rows-ish, k: contraction per shard, c: cols-ish
    if mode == "lhs_rows":
        looped = [_t((m, k), seed + r, dtype, probe) for r in range(n)]          # A_s [m_s, K]
        local = [_t((c, k), seed + 100 + r, dtype, probe) for r in range(n)]     # B_r^T [N, K]
        out_shape = (n * m, c)
        o_looped = [np64(x) for x in looped]
        o_local = [np64(x).T for x in local]
    elif mode == "rhs_cols":
        looped = [_t((c, k), seed + r, dtype, probe) for r in range(n)]          # B_s^T [n_s, K]
        local = [_t((m, k), seed + 100 + r, dtype, probe) for r in range(n)]     # A_r [M, K]
        out_shape = (m, n * c)
        o_looped = [np64(x).T for x in looped]
        o_local = [np64(x) for x in local]
    elif mode == "lhs_cols":
        looped = [_t((m, k), seed + r, dtype, probe) for r in range(n)]          # A_s [M, k_s]
        local = [_t((c, n * k), seed + 100 + r, dtype, probe) for r in range(n)] # B_r^T [N, n k_s]
        out_shape = (m, c)
        o_looped = [np64(x) for x in looped]
        o_local = [np64(x).T for x in local]
    else:  # rhs_rows
        looped = [_t((c, k), seed + r, dtype, probe) for r in range(n)]          # B_s^T [N, k_s]
        local = [_t((m, n * k), seed + 100 + r, dtype, probe) for r in range(n)] # A_r [M, n k_s]
        out_shape = (m, c)
        o_looped = [np64(x).T for x in looped]
        o_local = [np64(x) for x in local]
    return looped, local, out_shape, o_looped, o_local


AG_CASES = [("lhs_rows", (136, 200, 264)), ("rhs_cols", (300, 136, 200)),
            ("lhs_cols", (264, 136, 296)), ("rhs_rows", (200, 264, 136))]


@pytest.mark.parametrize("mode,dims", AG_CASES)
@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_allgather_einsum(ctx, mode, dims, n, out_dt):
    import collective_overlap_amd as cce
    print(f"[gpu] allgather {mode} n={n} dims={dims} out={out_dt}", flush=True)
    odt = torch.bfloat16 if out_dt == "bf16" else torch.float32
    looped, local, oshape, ol, oc = _ag_inputs(mode, n, dims, torch.bfloat16, False, seed=n)
    out = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, mode, looped, local, out)
    out_s = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, mode, looped, local, out_s, flags=cce.CCE_FLAG_SERIAL)
    sync()
    ref = oe.allgather_einsum(mode, ol, oc)
    for r in range(n):
        if out_dt == "bf16":
            assert_bf16_close(np64(out[r]), ref[r], f"rank {r}")
        else:
            assert_f32_close(np64(out[r]), ref[r], f"rank {r}")
        assert torch.equal(out[r], out_s[r]), "overlapped and serial results differ"


@pytest.mark.parametrize("mode,dims", AG_CASES)
@pytest.mark.parametrize("n", [2, 4])
def test_allgather_einsum_integer_probe_bit_exact(ctx, mode, dims, n):
    import collective_overlap_amd as cce
    looped, local, oshape, ol, oc = _ag_inputs(mode, n, dims, torch.bfloat16, True, seed=7)
    out = [torch.empty(oshape, device=DEV) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, mode, looped, local, out)
    sync()
    ref = oe.allgather_einsum(mode, ol, oc)
    for r in range(n):
        assert np.array_equal(np64(out[r]), ref[r]), f"rank {r}"


@pytest.mark.parametrize("mode,dims", [AG_CASES[1], AG_CASES[2]])
def test_allgather_einsum_gelu(ctx, mode, dims):
    import collective_overlap_amd as cce
    n = 3
    looped, local, oshape, ol, oc = _ag_inputs(mode, n, dims, torch.bfloat16, False, seed=11)
    out = [torch.empty(oshape, device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, mode, looped, local, out, flags=cce.CCE_FLAG_GELU)
    sync()
    ref = oe.allgather_einsum(mode, ol, oc)
    for r in range(n):
        assert_bf16_close(np64(out[r]), numerics.gelu(ref[r]), f"rank {r}")


def test_allgather_einsum_fp32_inputs(ctx):
    import collective_overlap_amd as cce
    n = 2
    looped, local, oshape, ol, oc = _ag_inputs("rhs_cols", n, (72, 264, 136), torch.float32, False)
    out = [torch.empty(oshape, device=DEV) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, "rhs_cols", looped, local, out)
    sync()
    ref = oe.allgather_einsum("rhs_cols", ol, oc)
    for r in range(n):
        assert_f32_close(np64(out[r]), ref[r], f"rank {r}")


# ---------------------------------------------------------------------------
# looped Einsum-ReduceScatter
# ---------------------------------------------------------------------------
def _rs_inputs(mode, n, dims, dtype, probe, seed=0):
    s, k, c = dims
    if mode == "slice_lhs_rows":
        a = [_t((n * s, k), seed + r, dtype, probe) for r in range(n)]     # [n m_s, K]
        b = [_t((c, k), seed + 50 + r, dtype, probe) for r in range(n)]    # B^T [N, K]
        oshape = (s, c)
    else:
        a = [_t((c, k), seed + r, dtype, probe) for r in range(n)]         # [M, K]
        b = [_t((n * s, k), seed + 50 + r, dtype, probe) for r in range(n)]  # B^T [n n_s, K]
        oshape = (c, s)
    return a, b, oshape, [np64(x) for x in a], [np64(x).T for x in b]


RS_CASES = [("slice_lhs_rows", (200, 264, 296)), ("slice_rhs_cols", (136, 264, 200)),
            ("slice_lhs_rows", (1, 64, 40)), ("slice_rhs_cols", (8, 64, 40))]


@pytest.mark.parametrize("mode,dims", RS_CASES)
@pytest.mark.parametrize("n", [1, 2, 3, 5])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_einsum_reducescatter(ctx, mode, dims, n, out_dt):
    import collective_overlap_amd as cce
    print(f"[gpu] reducescatter {mode} n={n} dims={dims} out={out_dt}", flush=True)
    odt = torch.bfloat16 if out_dt == "bf16" else torch.float32
    a, b, oshape, oa, ob = _rs_inputs(mode, n, dims, torch.bfloat16, False, seed=3 * n)
    out = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, out)
    out_s = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, out_s, flags=cce.CCE_FLAG_SERIAL)
    # one whole-shard chain instead of two half-shard chains, with copies
    # beside the GEMMs and serialised
    one = cce.CCE_FLAG_ONE_CHAIN
    out_1 = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, out_1, flags=one)
    out_1s = [torch.full(oshape, float("nan"), device=DEV, dtype=odt) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, out_1s, flags=one | cce.CCE_FLAG_SERIAL)
    sync()
    ref = oe.einsum_reducescatter(mode, oa, ob)
    for r in range(n):
        if out_dt == "bf16":
            assert_bf16_close(np64(out[r]), ref[r], f"rank {r}")
        else:
            assert_f32_close(np64(out[r]), ref[r], f"rank {r}")
        assert torch.equal(out[r], out_s[r]), "overlapped and serial results differ"
        assert torch.equal(out[r], out_1[r]), "one chain and two chains differ"
        assert torch.equal(out[r], out_1s[r]), "serial one chain and two chains differ"


@pytest.mark.parametrize("mode,dims", RS_CASES[:2])
@pytest.mark.parametrize("n", [2, 4, 8])
def test_einsum_reducescatter_integer_probe_bit_exact(ctx, mode, dims, n):
    import collective_overlap_amd as cce
    a, b, oshape, oa, ob = _rs_inputs(mode, n, dims, torch.bfloat16, True, seed=5)
    out = [torch.empty(oshape, device=DEV) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, out)
    sync()
    ref = oe.einsum_reducescatter(mode, oa, ob)
    for r in range(n):
        assert np.array_equal(np64(out[r]), ref[r]), f"rank {r}"


def test_repeated_calls_reuse_events(ctx):
    """Back-to-back calls on one context (events reused) stay correct."""
    import collective_overlap_amd as cce
    n = 4
    a, b, oshape, oa, ob = _rs_inputs("slice_lhs_rows", n, (64, 128, 96), torch.bfloat16, True, 9)
    ref = oe.einsum_reducescatter("slice_lhs_rows", oa, ob)
    outs = []
    for _ in range(5):
        out = [torch.empty(oshape, device=DEV) for _ in range(n)]
        cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", a, b, out)
        outs.append(out)
    sync()
    for out in outs:
        for r in range(n):
            assert np.array_equal(np64(out[r]), ref[r])


def test_invalid_arguments_enqueue_nothing(ctx):
    import collective_overlap_amd as cce
    from collective_overlap_amd._lib import CceError
    a = [torch.zeros((16, 12), device=DEV, dtype=torch.bfloat16)]   # K % 8 != 0
    b = [torch.zeros((16, 12), device=DEV, dtype=torch.bfloat16)]
    c = [torch.zeros((16, 16), device=DEV, dtype=torch.bfloat16)]
    with pytest.raises(CceError) as e:
        cce.cce_grouped_gemm(ctx, a, b, c)
    assert e.value.status in (1, 2)
    x = torch.zeros((64, 64), device=DEV, dtype=torch.bfloat16)
    with pytest.raises(CceError) as e:       # output aliases an input
        cce.cce_grouped_gemm(ctx, [x], [x], [x])
    assert e.value.status == 1
    assert torch.count_nonzero(x) == 0


# ---------------------------------------------------------------------------
# Fused permute (the GEMM sends the data itself): bit-identical to the
# copy-stream form, which the tests above compare with the oracle.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode,dims", AG_CASES)
@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
def test_allgather_fused_permute_matches(ctx, mode, dims, n, in_dt):
    import collective_overlap_amd as cce
    idt = torch.bfloat16 if in_dt == "bf16" else torch.float32
    looped, local, oshape, ol, oc = _ag_inputs(mode, n, dims, idt, False, seed=20 + n)
    outs = []
    for flags in (0, cce.CCE_FLAG_FUSED_PERMUTE):
        out = [torch.full(oshape, float("nan"), device=DEV, dtype=torch.bfloat16) for _ in range(n)]
        cce.cce_looped_allgather_einsum(ctx, mode, looped, local, out, flags=flags)
        outs.append(out)
    sync()
    ref = oe.allgather_einsum(mode, ol, oc)
    for r in range(n):
        assert torch.equal(outs[0][r], outs[1][r]), f"rank {r}"
        assert_bf16_close(np64(outs[1][r]), ref[r], f"rank {r}")


@pytest.mark.parametrize("mode,dims", RS_CASES)
@pytest.mark.parametrize("n", [1, 2, 3, 5])
def test_reducescatter_fused_permute_matches(ctx, mode, dims, n):
    import collective_overlap_amd as cce
    a, b, oshape, oa, ob = _rs_inputs(mode, n, dims, torch.bfloat16, False, seed=30 + n)
    outs = []
    for flags in (0, cce.CCE_FLAG_FUSED_PERMUTE):
        out = [torch.full(oshape, float("nan"), device=DEV) for _ in range(n)]
        cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, out, flags=flags)
        outs.append(out)
    sync()
    ref = oe.einsum_reducescatter(mode, oa, ob)
    for r in range(n):
        assert torch.equal(outs[0][r], outs[1][r]), f"rank {r}"
        assert_f32_close(np64(outs[1][r]), ref[r], f"rank {r}")


# ---------------------------------------------------------------------------
# Accumulate launches at the large tile shapes: whole tiles with more k tiles
# than accumulator blocks take the accumulator input during the last k tiles,
# edge tiles in the epilogue.  Integer probes make every order exact.
# ---------------------------------------------------------------------------
FOLD_CASES = [
    # mode, n, shard extent s, other extent c, K, flags.
    # copy stream: half-shard launches of 500 rows, 256x128 tiles, ragged
    # rows, a K tail (18 k tiles)
    ("slice_lhs_rows", 4, 1000, 4096, 1096, 0),
    # fused permute: 256x256 tiles, exactly one more k tile than blocks (17)
    ("slice_lhs_rows", 4, 1024, 4096, 1088, 0x8),
    # two-way ring, fused permute: 256x256 tiles, ragged rows
    ("slice_lhs_rows", 2, 1000, 4096, 1280, 0x18),
    # fused permute, one way: 256x128 tiles, ragged rows
    ("slice_lhs_rows", 2, 1000, 4096, 1280, 0x8),
    # column shards: 256x256 tiles, ragged rows, a K tail
    ("slice_rhs_cols", 4, 4096, 1000, 1096, 0x8),
]


@pytest.mark.parametrize("mode,n,s,c,K,flags", FOLD_CASES)
def test_reducescatter_large_tiles_integer_probe(ctx, mode, n, s, c, K, flags):
    import collective_overlap_amd as cce
    print(f"[gpu] reducescatter large tiles {mode} n={n} s={s} c={c} K={K} flags={flags:#x}",
          flush=True)
    a, b, oshape, _, _ = _rs_inputs(mode, n, (s, K, c), torch.bfloat16, True, seed=11)
    out = [torch.full(oshape, float("nan"), device=DEV) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, mode, a, b, out, flags=flags)
    sync()
    # sampled rows, tile edges and the ragged last tile included
    m_ext = s if mode == "slice_lhs_rows" else c
    rows = np.unique(np.concatenate([_rows_sample(24, m_ext, 3),
                                     [0, 255, 256, 767, 768, m_ext - 1]]))
    rows = rows[rows < m_ext]
    if mode == "slice_lhs_rows":
        oa = [np.concatenate([np64(x[t * s + rows]) for t in range(n)]) for x in a]
        ob = [np64(y).T for y in b]
    else:
        oa = [np64(x[rows]) for x in a]
        ob = [np64(y).T for y in b]
    ref = oe.einsum_reducescatter(mode, oa, ob)
    for r in range(n):
        assert np.array_equal(np64(out[r][rows]), ref[r]), f"rank {r}"


def _rows_sample(k, total, seed):
    g = np.random.default_rng(seed)
    return np.sort(g.choice(total, size=min(k, total), replace=False))


# ---------------------------------------------------------------------------
# Largest rank counts and empty extents
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("flags", [0, 0x1, 0x8])
def test_max_ranks_integer_probe(ctx, flags):
    """CCE_MAX_RANKS = 64 ranks (one launch of 64 groups), bit-exact."""
    import collective_overlap_amd as cce
    n = 64
    looped, local, oshape, ol, oc = _ag_inputs("rhs_cols", n, (40, 64, 16), torch.bfloat16, True, 4)
    out = [torch.empty(oshape, device=DEV) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, "rhs_cols", looped, local, out, flags=flags)
    a, b, rshape, oa, ob = _rs_inputs("slice_lhs_rows", n, (8, 64, 24), torch.bfloat16, True, 8)
    rout = [torch.empty(rshape, device=DEV) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", a, b, rout, flags=flags)
    sync()
    ref = oe.allgather_einsum("rhs_cols", ol, oc)
    rref = oe.einsum_reducescatter("slice_lhs_rows", oa, ob)
    for r in range(n):
        assert np.array_equal(np64(out[r]), ref[r]), f"allgather rank {r}"
        assert np.array_equal(np64(rout[r]), rref[r]), f"reducescatter rank {r}"


def test_empty_extents_are_noops(ctx):
    """Zero rows or columns: the call succeeds and touches nothing."""
    import collective_overlap_amd as cce
    n = 3
    looped = [torch.zeros((0, 64), device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    local = [torch.zeros((32, 64), device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    out = [torch.zeros((32, 0), device=DEV) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, "rhs_cols", looped, local, out)
    a = [torch.zeros((0, 64), device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    b = [torch.zeros((16, 64), device=DEV, dtype=torch.bfloat16) for _ in range(n)]
    rout = [torch.zeros((0, 16), device=DEV) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", a, b, rout)
    parts = [torch.zeros((0, 16), device=DEV)]
    cce.cce_fused_reduce_epilogue(ctx, parts, None, None, torch.zeros((0, 16), device=DEV), 0.1)
    sync()


# ---------------------------------------------------------------------------
# The largest operand the ABI takes (2^30 - 256 bytes)
# ---------------------------------------------------------------------------
def test_largest_operand_bit_exact_and_one_row_more_rejected(ctx):
    """A bf16 left factor of 65535 x 8192 (2^30 - 16384 bytes, the most whole
    rows of that width under the 2^30 - 256 byte limit): integer probes,
    bit-exact on the first and last tile rows, the ragged last tile
    included.  One row more (2^30 bytes) is rejected before anything is
    enqueued."""
    import collective_overlap_amd as cce
    from collective_overlap_amd._lib import CceError
    M, N, K = 65535, 256, 8192
    print(f"[gpu] largest operand M={M} N={N} K={K}", flush=True)
    big = W.int_probe((M + 1, K), 60, device=DEV, dtype=torch.bfloat16)
    a = big[:M]
    b = W.int_probe((N, K), 61, device=DEV, dtype=torch.bfloat16)
    assert a.numel() * 2 == (1 << 30) - 16384
    c = torch.full((M, N), float("nan"), device=DEV)
    cce.cce_grouped_gemm(ctx, [a], [b], [c])
    sync()
    rows = [0, 1, 255, 256, 65279, 65280, 65533, 65534]
    ref = np64(a[rows]) @ np64(b).T
    assert np.array_equal(np64(c[rows]), ref)
    assert not torch.isnan(c).any()
    c2 = torch.full((M + 1, N), float("nan"), device=DEV)
    with pytest.raises(CceError) as e:
        cce.cce_grouped_gemm(ctx, [big], [b], [c2])
    assert e.value.status == 2 and "1 GiB" in str(e.value)
    sync()
    assert torch.isnan(c2).all()
