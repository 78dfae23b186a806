"""Full-size parity of the five workloads, in the launch configuration the
benchmark times, on outputs the oracle computes element block by element
block (sampled rows x sampled columns of every checked rank)."""

import numpy as np
import pytest
import torch

from oracle import einsum as oe
from oracle import epilogue as oep
from oracle import numerics
import workloads as W
from gpu_util import np64, assert_bf16_close, assert_f32_close, sync

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16


@pytest.fixture(scope="module")
def ctx():
    import collective_overlap_amd as cce
    c = cce.Context(0)
    yield c
    sync()
    c.close()


def _rows(n, total, seed):
    g = np.random.default_rng(seed)
    return np.sort(g.choice(total, size=min(n, total), replace=False))


@pytest.mark.parametrize("flags", [0, 0x8, 0x18])   # copy stream; fused; fused two-way
def test_ag_fp32_n2_full(ctx, flags):
    """N=2 fp32 AllGather-Einsum case 1 and the 2-partial epilogue, compared
    in full."""
    import collective_overlap_amd as cce
    w = W.WORKLOADS["ag_fp32_n2"]
    n = 2
    X = [W.uniform(w.shapes["X"], r, device=DEV) for r in range(n)]
    # weight shards W_k [256, 512] stored as [512, 256]
    Wt = [W.uniform((512, 256), 10 + r, device=DEV) for r in range(n)]
    Y = [torch.empty((64, 1024), device=DEV) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, "rhs_cols", Wt, X, Y, flags=flags)
    P = [W.uniform(w.shapes["P"], 20 + k, device=DEV) for k in range(n)]
    b = W.uniform(w.shapes["bias"], 30, device=DEV)
    R = W.uniform(w.shapes["R"], 31, device=DEV)
    out = torch.empty((64, 256), device=DEV)
    mask = torch.empty((64, 256), device=DEV, dtype=torch.uint8)
    cce.cce_fused_reduce_epilogue(ctx, P, b, R, out, 0.1, 0, 0, mask_out=mask)
    sync()
    ref = oe.allgather_einsum("rhs_cols", [np64(t).T for t in Wt], [np64(x) for x in X])
    for r in range(n):
        assert_f32_close(np64(Y[r]), ref[r], f"rank {r}")
    eref, keep = oep.fused_reduce_epilogue([np64(p) for p in P], np64(b), np64(R), 0.1, 0, 0)
    assert np.array_equal(mask.cpu().numpy().astype(bool), keep)
    assert_f32_close(np64(out), eref, "epilogue", tol=1e-6)


@pytest.mark.parametrize("allreduce", [False, True])
def test_attn_outproj_n8_full(ctx, allreduce):
    """8 local partial GEMMs [8192,1024] x [1024,8192] and the 8-partial fused
    epilogue at full size (one output, or the FusedAllReduce's 8 replicas);
    sampled rows of each."""
    import collective_overlap_amd as cce
    n = 8
    IN = [W.normal((8192, 1024), 1.0, k, device=DEV) for k in range(n)]
    Wt = [W.weight_store(1024, 8192, 0.02, 10 + k, device=DEV) for k in range(n)]
    P = [torch.empty((8192, 8192), device=DEV, dtype=BF) for _ in range(n)]
    cce.cce_grouped_gemm(ctx, IN, Wt, P)
    b = W.normal((8192,), 0.02, 20, device=DEV)
    R = W.normal((8192, 8192), 1.0, 21, device=DEV)
    out = torch.empty((8192, 8192), device=DEV, dtype=BF)
    mask = torch.empty((8192, 8192), device=DEV, dtype=torch.uint8)
    if allreduce:
        reps = [out] + [torch.empty_like(out) for _ in range(n - 1)]
        cce.cce_fused_allreduce_epilogue(ctx, P, b, R, reps, 0.1, 0, 0, mask_out=mask)
    else:
        cce.cce_fused_reduce_epilogue(ctx, P, b, R, out, 0.1, 0, 0, mask_out=mask)
    sync()
    if allreduce:
        for q in (1, 7):
            assert torch.equal(reps[q].view(torch.int16), out.view(torch.int16)), f"replica {q}"
    rows = _rows(48, 8192, 1)
    cols = _rows(512, 8192, 2)
    for q in (0, 3, 7):
        ref = np64(IN[q][rows]) @ np64(Wt[q][cols]).T
        assert_bf16_close(np64(P[q][rows][:, cols]), ref, f"partial {q}")
    # keep mask of sampled rows, bit-exact
    from oracle import philox
    for r in rows:
        want = philox.keep_mask(1, 8192, 0.1, 0, 0, row0=int(r), col0=0, ld=8192)[0]
        assert np.array_equal(mask[int(r)].cpu().numpy().astype(bool), want)
    # end to end for a few full rows: the oracle forms the partials itself
    # (rounded to bf16, the partials' storage type) and applies the epilogue
    for r in rows[:4]:
        r = int(r)
        parts = [numerics.bf16_round((np64(IN[q][r:r + 1]) @ np64(Wt[q]).T).astype(np.float32))
                 for q in range(n)]
        ref, _ = oep.fused_reduce_epilogue(parts, np64(b), np64(R[r:r + 1]), 0.1, 0, 0,
                                           row0=r, col0=0, mask_ld=8192)
        assert_bf16_close(np64(out[r:r + 1]), ref, f"epilogue row {r}")


@pytest.mark.parametrize("flags", [0, 0x8, 0x18])   # copy stream; fused; fused two-way
def test_mlp2_n4_full(ctx, flags):
    """2-layer MLP, 4-way: layer 1 looped AllGather (W1 shards [4096,4096])
    with GELU, layer 2 looped AllGather (W2 shards [16384,1024]).  For the
    sampled rows the oracle derives H from X itself (rounded to bf16, H's
    storage type) and feeds that to layer 2."""
    import collective_overlap_amd as cce
    n = 4
    X = [W.normal((2048, 4096), 1.0, r, device=DEV) for r in range(n)]
    W1 = [W.weight_store(4096, 4096, 0.02, 10 + s, device=DEV) for s in range(n)]
    W2 = [W.weight_store(16384, 1024, 0.02, 20 + s, device=DEV) for s in range(n)]
    H = [torch.empty((2048, 16384), device=DEV, dtype=BF) for _ in range(n)]
    Y = [torch.empty((2048, 4096), device=DEV, dtype=BF) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, "rhs_cols", W1, X, H, flags=flags | cce.CCE_FLAG_GELU)
    cce.cce_looped_allgather_einsum(ctx, "rhs_cols", W2, H, Y, flags=flags)
    sync()
    rows = _rows(6, 2048, 3)
    cols = _rows(384, 4096, 4)
    w1_full = np.concatenate([np64(w) for w in W1], axis=0)     # [16384, 4096] = W1^T
    for r in (0, 2):
        h_ref = numerics.gelu(np64(X[r][rows]) @ w1_full.T)      # [6, 16384]
        assert_bf16_close(np64(H[r][rows]), h_ref, f"H rank {r}")
        # layer 2 from the oracle's own H, rounded to bf16 as stored
        h_bf = numerics.bf16_round(h_ref.astype(np.float32)).astype(np.float64)
        w2c = np.concatenate([np64(w) for w in W2], axis=0)[cols]   # [384, 16384]
        y_ref = h_bf @ w2c.T
        assert_bf16_close(np64(Y[r][rows][:, cols]), y_ref, f"Y rank {r}")


@pytest.mark.parametrize("flags", [0, 0x8, 0x18])   # copy stream; fused; fused two-way
def test_rs_n8_full(ctx, flags):
    """Einsum-ReduceScatter, 8 ranks, X [16384,2048] x W [2048,4096], fp32
    accumulator shards [2048,4096]; sampled whole rows of every shard (its
    first and last row included)."""
    import collective_overlap_amd as cce
    n = 8
    X = [W.normal((16384, 2048), 1.0, r, device=DEV) for r in range(n)]
    Wt = [W.weight_store(2048, 4096, 0.02, 10 + r, device=DEV) for r in range(n)]
    out = [torch.empty((2048, 4096), device=DEV) for _ in range(n)]
    cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", X, Wt, out, flags=flags)
    sync()
    rows = np.unique(np.concatenate([[0, 2047], _rows(14, 2048, 5)]))
    ref = oe.einsum_reducescatter(
        "slice_lhs_rows",
        [np.concatenate([np64(X[q][s * 2048 + rows]) for s in range(n)]) for q in range(n)],
        [np64(Wt[q]).T for q in range(n)])
    for r in range(n):
        assert_f32_close(np64(out[r][rows]), ref[r], f"shard {r}")


@pytest.mark.parametrize("flags,batched,in_rs", [(0, False, False), (0x8, True, False),
                                                 (0x18, True, False), (0x18, True, True),
                                                 (0x8, True, True)])
def test_gpt3_ffn_n8_full(ctx, flags, batched, in_rs):
    """GPT-3 FFN, 8-way: looped AllGather into W1 shards with GELU, looped
    ReduceScatter out of W2 shards, fused bias+dropout+residual; sampled.
    Run in the copy-stream form with one epilogue per rank, in the fused
    permute (one-way and two-way ring) with the batched epilogue, and with the
    epilogue inside the ReduceScatter (the benchmark's configuration: fused
    permute, two-way ring), whose output must equal the two-call path's bit
    for bit."""
    import collective_overlap_amd as cce
    print(f"[gpu] gpt3_ffn_n8 full flags={flags} batched={batched} in_rs={in_rs}", flush=True)
    n = 8
    X = [W.normal((1024, 12288), 1.0, s, device=DEV) for s in range(n)]
    W1 = [W.weight_store(12288, 6144, 0.02, 10 + r, device=DEV) for r in range(n)]
    W2 = [W.weight_store(6144, 12288, 0.02, 20 + r, device=DEV) for r in range(n)]
    b = W.normal((12288,), 0.02, 30, device=DEV)
    R = [W.normal((1024, 12288), 1.0, 40 + r, device=DEV) for r in range(n)]
    H = [torch.empty((8192, 6144), device=DEV, dtype=BF) for _ in range(n)]
    acc = [torch.empty((1024, 12288), device=DEV) for _ in range(n)]
    out = [torch.empty((1024, 12288), device=DEV, dtype=BF) for _ in range(n)]
    cce.cce_looped_allgather_einsum(ctx, "lhs_rows", X, W1, H, flags=flags | cce.CCE_FLAG_GELU)
    cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", H, W2, acc, flags=flags)
    if batched:
        cce.cce_fused_reduce_epilogue_batched(ctx, [[a] for a in acc], b, R, out, 0.1, 0, 0,
                                              mask_row0=[r * 1024 for r in range(n)],
                                              mask_col0=0, mask_ld=12288)
    else:
        for r in range(n):
            cce.cce_fused_reduce_epilogue(ctx, [acc[r]], b, R[r], out[r], 0.1, 0, 0,
                                          mask_row0=r * 1024, mask_col0=0, mask_ld=12288)
    if in_rs:
        fused = [torch.empty((1024, 12288), device=DEV, dtype=BF) for _ in range(n)]
        cce.cce_looped_einsum_reducescatter_epilogue(
            ctx, "slice_lhs_rows", H, W2, b, R, fused, 0.1, 0, 0,
            mask_row0=[r * 1024 for r in range(n)], mask_col0=0, mask_ld=12288, flags=flags)
        sync()
        for r in range(n):
            assert torch.equal(fused[r].view(torch.int16), out[r].view(torch.int16)), f"rank {r}"
    sync()
    # layer 1: H_r rows (global tokens) x sampled FFN columns
    grow = _rows(8, 8192, 7)
    hcols = _rows(256, 6144, 8)
    xg = np.stack([np64(X[g // 1024][g % 1024]) for g in grow])
    for r in (0, 5):
        ref = numerics.gelu(xg @ np64(W1[r][hcols]).T)
        assert_bf16_close(np64(H[r][grow][:, hcols]), ref, f"H rank {r}")
    # layer 2 + epilogue end to end for sampled rows of two shards: the oracle
    # rebuilds the needed H rows from X (rounded to bf16, H's storage type),
    # sums the partials over ranks and applies the epilogue
    cols = _rows(384, 12288, 10)
    # (shard, row in shard): the first, second, a middle and the last row of
    # every shard
    picks = [(sh, i) for sh in range(n) for i in (0, 1, 517, 1023)]
    xr = np.stack([np64(X[sh][i]) for sh, i in picks])   # token rows sh*1024 + i
    acc_ref = np.zeros((len(picks), len(cols)))
    for q in range(n):
        hq = numerics.gelu(xr @ np64(W1[q]).T)
        hq = numerics.bf16_round(hq.astype(np.float32)).astype(np.float64)
        acc_ref += hq @ np64(W2[q][cols]).T
    for k, (sh, i) in enumerate(picks):
        assert_f32_close(np64(acc[sh][i][cols]), acc_ref[k], f"acc shard {sh} row {i}", tol=2e-3)
        full_row = np.zeros((1, 12288))
        full_row[0, cols] = acc_ref[k]
        ref, _ = oep.fused_reduce_epilogue([full_row], np64(b), np64(R[sh][i:i + 1]), 0.1, 0, 0,
                                           row0=sh * 1024 + i, col0=0, mask_ld=12288)
        assert_bf16_close(np64(out[sh][i][cols]), ref[0, cols], f"out shard {sh} row {i}")


# Whole-tensor equality of the permute forms at full size.  The sampled
# oracle checks above see a few rows of every shard; a copy or forwarding
# mistake confined to other rows would pass them, but not these.  The
# stream, serial and fused forms of one ring direction, with one or two
# accumulator chains, accumulate every element in the same order, so their
# outputs agree bit for bit.
def _forms(cce, bid):
    return {"stream": bid, "serial": bid | cce.CCE_FLAG_SERIAL,
            "serial one-chain": bid | cce.CCE_FLAG_SERIAL | cce.CCE_FLAG_ONE_CHAIN,
            "fused": bid | cce.CCE_FLAG_FUSED_PERMUTE}


@pytest.mark.parametrize("bid", [0, 0x10])     # one-way ring; two-way ring
def test_rs_n8_full_forms_equal(ctx, bid):
    import collective_overlap_amd as cce
    print(f"[gpu] rs_n8 full, whole-tensor form equality bid={bid:#x}", flush=True)
    n = 8
    X = [W.normal((16384, 2048), 1.0, r, device=DEV) for r in range(n)]
    Wt = [W.weight_store(2048, 4096, 0.02, 10 + r, device=DEV) for r in range(n)]
    outs = {}
    for name, fl in _forms(cce, bid).items():
        o = [torch.full((2048, 4096), float("nan"), device=DEV) for _ in range(n)]
        cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", X, Wt, o, flags=fl)
        outs[name] = o
    sync()
    for name in ("serial", "serial one-chain", "fused"):
        for r in range(n):
            assert torch.equal(outs["stream"][r].view(torch.int32), outs[name][r].view(torch.int32)), \
                f"{name} differs from stream, shard {r}"
    assert all(bool(torch.isfinite(o).all()) for o in outs["stream"])


@pytest.mark.parametrize("bid", [0, 0x10])
def test_gpt3_ffn_n8_full_forms_equal(ctx, bid):
    """Both layers: H (AllGather, bf16 with GELU) and the fp32 accumulator
    (ReduceScatter) over every element of every rank."""
    import collective_overlap_amd as cce
    print(f"[gpu] gpt3_ffn_n8 full, whole-tensor form equality bid={bid:#x}", flush=True)
    n = 8
    X = [W.normal((1024, 12288), 1.0, s, device=DEV) for s in range(n)]
    W1 = [W.weight_store(12288, 6144, 0.02, 10 + r, device=DEV) for r in range(n)]
    W2 = [W.weight_store(6144, 12288, 0.02, 20 + r, device=DEV) for r in range(n)]
    Hs, accs = {}, {}
    for name, fl in _forms(cce, bid).items():
        H = [torch.full((8192, 6144), float("nan"), device=DEV, dtype=BF) for _ in range(n)]
        acc = [torch.full((1024, 12288), float("nan"), device=DEV) for _ in range(n)]
        cce.cce_looped_allgather_einsum(ctx, "lhs_rows", X, W1, H, flags=fl | cce.CCE_FLAG_GELU)
        cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", H, W2, acc, flags=fl)
        Hs[name], accs[name] = H, acc
    sync()
    for name in ("serial", "serial one-chain", "fused"):
        for r in range(n):
            assert torch.equal(Hs["stream"][r].view(torch.int16), Hs[name][r].view(torch.int16)), \
                f"H: {name} differs from stream, rank {r}"
            assert torch.equal(accs["stream"][r].view(torch.int32), accs[name][r].view(torch.int32)), \
                f"acc: {name} differs from stream, rank {r}"
    assert all(bool(torch.isfinite(h).all()) for h in Hs["stream"])
    assert all(bool(torch.isfinite(a).all()) for a in accs["stream"])


@pytest.mark.parametrize("bid", [0, 0x10])
def test_mlp2_n4_full_forms_equal(ctx, bid):
    """Both MLP layers (looped weight shards, rhs_cols; GELU between) over
    every element of every rank, in every permute form."""
    import collective_overlap_amd as cce
    print(f"[gpu] mlp2_n4 full, whole-tensor form equality bid={bid:#x}", flush=True)
    n, B, F, Hh = 4, 2048, 4096, 16384
    X = [W.normal((B, F), 1.0, r, device=DEV) for r in range(n)]
    W1 = [W.weight_store(F, Hh // n, 0.02, 10 + s, device=DEV) for s in range(n)]
    W2 = [W.weight_store(Hh, F // n, 0.02, 20 + s, device=DEV) for s in range(n)]
    Hs, Ys = {}, {}
    for name, fl in _forms(cce, bid).items():
        H = [torch.full((B, Hh), float("nan"), device=DEV, dtype=BF) for _ in range(n)]
        Y = [torch.full((B, F), float("nan"), device=DEV, dtype=BF) for _ in range(n)]
        cce.cce_looped_allgather_einsum(ctx, "rhs_cols", W1, X, H, flags=fl | cce.CCE_FLAG_GELU)
        cce.cce_looped_allgather_einsum(ctx, "rhs_cols", W2, H, Y, flags=fl)
        Hs[name], Ys[name] = H, Y
    sync()
    for name in ("serial", "fused"):
        for r in range(n):
            assert torch.equal(Hs["stream"][r].view(torch.int16), Hs[name][r].view(torch.int16)), \
                f"H: {name} differs from stream, rank {r}"
            assert torch.equal(Ys["stream"][r].view(torch.int16), Ys[name][r].view(torch.int16)), \
                f"Y: {name} differs from stream, rank {r}"
    assert all(bool(torch.isfinite(h).all()) for h in Hs["stream"])
    assert all(bool(torch.isfinite(y).all()) for y in Ys["stream"])
