#!/usr/bin/env python3
"""Benchmark of the looped CollectiveEinsum hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input.
The default workload is the GPT-3-scale FFN layer, 8-way: a looped
AllGather-Einsum into the W1 shards with GELU fused into its store, a looped
Einsum-ReduceScatter out of the W2 shards with an fp32 travelling
accumulator, and the fused bias + dropout + residual epilogue on every rank's
shard.  All 8 logical ranks are separate HBM buffers on the one GPU.

The timed step uses the fused permute by default (each partial GEMM sends
the data itself: the AllGather forwards the shard it stages through LDS, the
ReduceScatter's accumulate epilogue stores into the next rank's
accumulator); --permute stream times the form with async copies on a second
stream instead.  Both, and the same kernels serialised on one stream, are
reported.  The ring is two-way by default (two partial einsums per
iteration, one per direction) for every workload but the ReduceScatter
alone (rs_n8), whose one-way ring is faster; --transfer picks either.

Prints one JSON line: whole-step bf16 TFLOP/s (value), the dominant kernel's
roofline, the epilogue's HBM rate, the looped-vs-serial comparison with the
hidden copy fraction, and the CPU oracle timed on a bounded sample (rank 0,
N = 1 only), which doubles as an end-to-end parity check of the timed
outputs.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "looped einsum bf16 TFLOP/s (% MFMA peak); fused reduce-epilogue HBM GB/s"
CPU_SAMPLE_S = 12.0      # target seconds of oracle work in the CPU baseline
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}     # dense MFMA, MI355X datasheet
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------
class Gpt3Ffn:
    name = "gpt3_ffn_n8"
    has_rs = True              # a looped Einsum-ReduceScatter (two chains with copies)
    sample_default, sample_cap = 8, 1024       # tokens per shard in the oracle sample
    dtype = "bf16"

    def __init__(self, dev):
        import torch
        import workloads as W
        self.n, self.T, self.Hd, self.F = 8, 8192, 12288, 49152
        n, ts, fs = self.n, self.T // self.n, self.F // self.n
        self.ts, self.fs = ts, fs
        bf = torch.bfloat16
        self.X = [W.normal((ts, self.Hd), 1.0, s, device=dev) for s in range(n)]
        self.W1 = [W.weight_store(self.Hd, fs, 0.02, 10 + r, device=dev) for r in range(n)]
        self.W2 = [W.weight_store(fs, self.Hd, 0.02, 20 + r, device=dev) for r in range(n)]
        self.b = W.normal((self.Hd,), 0.02, 30, device=dev)
        self.R = [W.normal((ts, self.Hd), 1.0, 40 + r, device=dev) for r in range(n)]
        self.H = [torch.empty((self.T, fs), device=dev, dtype=bf) for _ in range(n)]
        self.acc = [torch.empty((ts, self.Hd), device=dev) for _ in range(n)]
        self.out = [torch.empty((ts, self.Hd), device=dev, dtype=bf) for _ in range(n)]
        import collective_overlap_amd as cce
        self.ws_ag = torch.empty(cce.cce_looped_allgather_einsum_workspace(
            n, "lhs_rows", "bf16", "bf16", (ts, self.Hd), (self.T, fs)), dtype=torch.uint8,
            device=dev)
        self.ws_rs = torch.empty(cce.cce_looped_einsum_reducescatter_workspace(
            n, "slice_lhs_rows", (ts, self.Hd)), dtype=torch.uint8, device=dev)
        self.flops = 2 * (2.0 * self.T * self.Hd * fs * n)
        self.p = 0.1
        # The fused epilogue's algorithmic bytes per step: one fp32 partial
        # (the reduced result), the bf16 residual and output, the bias.  The
        # two-way ring's epilogue reads two fp32 accumulators (cw and ccw),
        # so the bytes it moves exceed these by one fp32 plane.
        self.epi_alg_bytes = self.T * self.Hd * (4 + 2 + 2) + self.Hd * 2

    def config(self):
        return {"workload": self.name, "n_ranks": self.n, "tokens": self.T, "hidden": self.Hd,
                "ffn": self.F, "w1_shard": [self.Hd, self.fs], "w2_shard": [self.fs, self.Hd],
                "p_drop": self.p, "acc_dtype": "f32", "global_batch": self.T}

    # False: the ReduceScatter stores its fp32 result, and a second call
    # applies the epilogue (bench.py --separate-epilogue)
    fuse_epilogue = True

    def run(self, ctx, flags=0):
        import collective_overlap_amd as cce
        # (the fine-grained flag concerns the ReduceScatter's chunk consumer)
        cce.cce_looped_allgather_einsum(ctx, "lhs_rows", self.X, self.W1, self.H, self.ws_ag,
                                        flags=(flags & ~cce.CCE_FLAG_FINE_GRAINED) |
                                        cce.CCE_FLAG_GELU)
        rows0 = [r * self.ts for r in range(self.n)]
        if self.fuse_epilogue:
            # The ReduceScatter hands its accumulators straight to the fused
            # bias + dropout + residual epilogue (one launch over the ranks).
            cce.cce_looped_einsum_reducescatter_epilogue(
                ctx, "slice_lhs_rows", self.H, self.W2, self.b, self.R, self.out, self.p, 0, 0,
                mask_row0=rows0, mask_col0=0, mask_ld=self.Hd, workspace=self.ws_rs, flags=flags)
            return
        cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", self.H, self.W2, self.acc,
                                            self.ws_rs, flags=flags)
        # One launch for the 8 ranks' shards (each rank's slice of the
        # reduced tensor gets bias, dropout and residual).
        cce.cce_fused_reduce_epilogue_batched(
            ctx, [[a] for a in self.acc], self.b, self.R, self.out, self.p, 0, 0,
            mask_row0=rows0, mask_col0=0, mask_ld=self.Hd)

    def monolithic(self):
        """The same two layers unlooped, on pre-gathered operands: one grouped
        GEMM per layer (H_r = GELU(X_all W1_r), P_r = H_r W2_r in fp32, the
        full per-rank partial that a plain ReduceScatter would then reduce).
        Returns a callable running both; no permutes, no epilogue."""
        import torch
        import collective_overlap_amd as cce
        x_all = torch.cat(self.X)                       # [T, Hd], gathered
        parts = [torch.empty((self.T, self.Hd), device=x_all.device) for _ in range(self.n)]

        def run(ctx):
            cce.cce_grouped_gemm(ctx, [x_all] * self.n, self.W1, self.H, gelu=True)
            cce.cce_grouped_gemm(ctx, self.H, self.W2, parts)
        return run

    def oracle_sample(self, t=8):
        """The oracle end to end on t tokens of every shard; returns
        (seconds, flops, description, rel error vs the device outputs)."""
        import numpy as np
        from oracle import einsum as oe, epilogue as oep, numerics
        f64 = _f64
        xs = [f64(x[:t]) for x in self.X]
        w1 = [f64(w).T for w in self.W1]
        w2 = [f64(w).T for w in self.W2]
        b, rr = f64(self.b), [f64(r[:t]) for r in self.R]
        t0 = time.perf_counter()
        h = oe.allgather_einsum("lhs_rows", xs, w1)
        h = [numerics.bf16_round(numerics.gelu(x).astype(np.float32)).astype(np.float64) for x in h]
        a = oe.einsum_reducescatter("slice_lhs_rows", h, w2)
        t1 = time.perf_counter()
        outs = [oep.fused_reduce_epilogue([a[r]], b, rr[r], self.p, 0, 0, row0=r * self.ts,
                                          col0=0, mask_ld=self.Hd)[0] for r in range(self.n)]
        dt = time.perf_counter() - t0
        # the epilogue's share (its vectorised Philox included), timed apart
        self.epi_oracle = (time.perf_counter() - t1, self.n * t * self.Hd)
        got = np.concatenate([f64(o[:t]) for o in self.out])
        ref = np.concatenate(outs)
        err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        flops = 2 * (2.0 * self.n * t * self.Hd * self.fs * self.n)
        return dt, flops, f"{t} tokens per shard ({self.n * t} of {self.T}), all 8 ranks, " \
                          f"float64 NumPy oracle end to end", err


class AttnOutProj:
    name = "attn_outproj_n8"
    sample_default, sample_cap = 16, 8192      # token rows in the oracle sample
    dtype = "bf16"
    has_permute = False        # local GEMMs, then the fused reduction: no ring

    def __init__(self, dev):
        import torch
        import workloads as W
        self.n, self.M, self.K, self.N = 8, 8192, 1024, 8192
        n = self.n
        bf = torch.bfloat16
        self.IN = [W.normal((self.M, self.K), 1.0, k, device=dev) for k in range(n)]
        self.Wt = [W.weight_store(self.K, self.N, 0.02, 10 + k, device=dev) for k in range(n)]
        self.P = [torch.empty((self.M, self.N), device=dev, dtype=bf) for _ in range(n)]
        self.b = W.normal((self.N,), 0.02, 20, device=dev)
        self.R = W.normal((self.M, self.N), 1.0, 21, device=dev)
        self.out = torch.empty((self.M, self.N), device=dev, dtype=bf)
        self.flops = 2.0 * self.M * self.N * self.K * n
        self.p = 0.1
        self.epi_alg_bytes = self.M * self.N * 2 * (n + 2) + self.N * 2   # 8 partials + R + out, bias

    def config(self):
        return {"workload": self.name, "n_ranks": self.n, "tokens": self.M, "in_shard": self.K,
                "hidden": self.N, "p_drop": self.p, "global_batch": self.M}

    def use_allreduce(self):
        """FusedAllReduce form: the result lands on all 8 ranks (8 replicas)."""
        import torch
        self.outs = [self.out] + [torch.empty_like(self.out) for _ in range(self.n - 1)]

    def run(self, ctx, flags=0):
        import collective_overlap_amd as cce
        cce.cce_grouped_gemm(ctx, self.IN, self.Wt, self.P)
        if getattr(self, "outs", None):
            cce.cce_fused_allreduce_epilogue(ctx, self.P, self.b, self.R, self.outs, self.p, 0, 0)
        else:
            cce.cce_fused_reduce_epilogue(ctx, self.P, self.b, self.R, self.out, self.p, 0, 0)

    def oracle_sample(self, t=16):
        import numpy as np
        from oracle import einsum as oe, epilogue as oep, numerics
        f64 = _f64
        ins = [f64(x[:t]) for x in self.IN]
        ws = [f64(w).T for w in self.Wt]
        b, rr = f64(self.b), f64(self.R[:t])
        t0 = time.perf_counter()
        parts = oe.local_matmuls(ins, ws)
        parts = [numerics.bf16_round(p.astype(np.float32)).astype(np.float64) for p in parts]
        ref, _ = oep.fused_reduce_epilogue(parts, b, rr, self.p, 0, 0, mask_ld=self.N)
        dt = time.perf_counter() - t0
        err = float(np.linalg.norm(f64(self.out[:t]) - ref) / np.linalg.norm(ref))
        return dt, 2.0 * t * self.K * self.N * self.n, \
            f"{t} of {self.M} token rows, all 8 partials, float64 NumPy oracle", err


class Mlp2:
    name = "mlp2_n4"
    sample_default, sample_cap = 8, 2048       # rows per rank in the oracle sample
    dtype = "bf16"

    def __init__(self, dev):
        import torch
        import workloads as W
        self.n, self.B, self.F, self.Hh = 4, 2048, 4096, 16384
        n = self.n
        bf = torch.bfloat16
        self.X = [W.normal((self.B, self.F), 1.0, r, device=dev) for r in range(n)]
        self.W1 = [W.weight_store(self.F, self.Hh // n, 0.02, 10 + s, device=dev) for s in range(n)]
        self.W2 = [W.weight_store(self.Hh, self.F // n, 0.02, 20 + s, device=dev) for s in range(n)]
        self.H = [torch.empty((self.B, self.Hh), device=dev, dtype=bf) for _ in range(n)]
        self.Y = [torch.empty((self.B, self.F), device=dev, dtype=bf) for _ in range(n)]
        import collective_overlap_amd as cce
        w1, w2 = self.W1[0], self.W2[0]
        self.ws1 = torch.empty(cce.cce_looped_allgather_einsum_workspace(
            n, "rhs_cols", "bf16", "bf16", tuple(w1.shape), (self.B, self.Hh)), dtype=torch.uint8,
            device=dev)
        self.ws2 = torch.empty(cce.cce_looped_allgather_einsum_workspace(
            n, "rhs_cols", "bf16", "bf16", tuple(w2.shape), (self.B, self.F)), dtype=torch.uint8,
            device=dev)
        self.flops = 2 * (2.0 * self.B * self.F * self.Hh * n)

    def config(self):
        return {"workload": self.name, "n_ranks": self.n, "batch": self.B, "features": self.F,
                "hidden": self.Hh, "global_batch": self.B * self.n}

    def run(self, ctx, flags=0):
        import collective_overlap_amd as cce
        flags &= ~cce.CCE_FLAG_FINE_GRAINED      # (a ReduceScatter flag)
        cce.cce_looped_allgather_einsum(ctx, "rhs_cols", self.W1, self.X, self.H, self.ws1,
                                        flags=flags | cce.CCE_FLAG_GELU)
        cce.cce_looped_allgather_einsum(ctx, "rhs_cols", self.W2, self.H, self.Y, self.ws2,
                                        flags=flags)

    def monolithic(self):
        """Both layers unlooped: each rank multiplies by the gathered weights
        (the shards concatenated), one grouped GEMM per layer."""
        import torch
        import collective_overlap_amd as cce
        w1, w2 = torch.cat(self.W1), torch.cat(self.W2)     # [Hh, F], [F, Hh]

        def run(ctx):
            cce.cce_grouped_gemm(ctx, self.X, [w1] * self.n, self.H, gelu=True)
            cce.cce_grouped_gemm(ctx, self.H, [w2] * self.n, self.Y)
        return run

    def oracle_sample(self, t=8):
        import numpy as np
        from oracle import einsum as oe, numerics
        f64 = _f64
        xs = [f64(x[:t]) for x in self.X]
        w1 = [f64(w).T for w in self.W1]
        w2 = [f64(w).T for w in self.W2]
        t0 = time.perf_counter()
        h = oe.allgather_einsum("rhs_cols", w1, xs)
        h = [numerics.bf16_round(numerics.gelu(x).astype(np.float32)).astype(np.float64) for x in h]
        y = oe.allgather_einsum("rhs_cols", w2, h)
        dt = time.perf_counter() - t0
        got = np.concatenate([f64(o[:t]) for o in self.Y])
        ref = np.concatenate(y)
        err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        return dt, 2 * (2.0 * t * self.F * self.Hh * self.n), \
            f"{t} of {self.B} rows per rank, all 4 ranks, float64 NumPy oracle", err


class RsN8:
    name = "rs_n8"
    has_rs = True
    # The one-way ring is this workload's faster form (2.20 against 2.27 ms
    # per step, interleaved in one process): the two-way ring's closing
    # align-and-sum launch costs more than its fewer, larger launches save.
    transfer = "one-way"
    sample_default, sample_cap = 16, 2048      # rows of every shard in the oracle sample
    dtype = "bf16"

    def __init__(self, dev):
        import torch
        import workloads as W
        self.n, self.T, self.K, self.N = 8, 16384, 2048, 4096
        n = self.n
        self.X = [W.normal((self.T, self.K), 1.0, r, device=dev) for r in range(n)]
        self.Wt = [W.weight_store(self.K, self.N, 0.02, 10 + r, device=dev) for r in range(n)]
        self.out = [torch.empty((self.T // n, self.N), device=dev) for _ in range(n)]
        self.flops = 2.0 * self.T * self.K * self.N * n

    def config(self):
        return {"workload": self.name, "n_ranks": self.n, "tokens": self.T, "k_shard": self.K,
                "hidden": self.N, "acc_dtype": "f32", "global_batch": self.T}

    def run(self, ctx, flags=0):
        import collective_overlap_amd as cce
        cce.cce_looped_einsum_reducescatter(ctx, "slice_lhs_rows", self.X, self.Wt, self.out,
                                            flags=flags)

    def monolithic(self):
        """Every rank's full fp32 partial X_r W_r (what a plain ReduceScatter
        would then reduce), one grouped GEMM."""
        import torch
        import collective_overlap_amd as cce
        parts = [torch.empty((self.T, self.N), device=self.X[0].device) for _ in range(self.n)]

        def run(ctx):
            cce.cce_grouped_gemm(ctx, self.X, self.Wt, parts)
        return run

    def oracle_sample(self, t=16):
        import numpy as np
        from oracle import einsum as oe
        f64 = _f64
        ms = self.T // self.n
        a = [np.concatenate([f64(x[s * ms:s * ms + t]) for s in range(self.n)]) for x in self.X]
        b = [f64(w).T for w in self.Wt]
        t0 = time.perf_counter()
        ref = oe.einsum_reducescatter("slice_lhs_rows", a, b)
        dt = time.perf_counter() - t0
        got = np.concatenate([f64(o[:t]) for o in self.out])
        err = float(np.linalg.norm(got - np.concatenate(ref)) / np.linalg.norm(np.concatenate(ref)))
        return dt, 2.0 * self.n * t * self.K * self.N * self.n, \
            f"{t} of {ms} rows of every shard, float64 NumPy oracle", err


class AgFp32N2:
    name = "ag_fp32_n2"
    dtype = "f32"
    # launch-bound (microseconds per kernel): also timed as a captured graph
    graph = True

    def __init__(self, dev):
        import torch
        import workloads as W
        self.n = 2
        self.X = [W.uniform((64, 256), r, device=dev) for r in range(2)]
        self.Wt = [W.uniform((512, 256), 10 + r, device=dev) for r in range(2)]
        self.Y = [torch.empty((64, 1024), device=dev) for _ in range(2)]
        self.P = [W.uniform((64, 256), 20 + k, device=dev) for k in range(2)]
        self.b = W.uniform((256,), 30, device=dev)
        self.R = W.uniform((64, 256), 31, device=dev)
        self.out = torch.empty((64, 256), device=dev)
        import collective_overlap_amd as cce
        self.ws = torch.empty(cce.cce_looped_allgather_einsum_workspace(
            2, "rhs_cols", "f32", "f32", (512, 256), (64, 1024)), dtype=torch.uint8, device=dev)
        self.flops = 2.0 * 64 * 256 * 1024 * 2

    def config(self):
        return {"workload": self.name, "n_ranks": 2, "x": [64, 256], "w_shard": [256, 512],
                "epilogue": [64, 256], "p_drop": 0.1, "global_batch": 128}

    def run(self, ctx, flags=0):
        import collective_overlap_amd as cce
        cce.cce_looped_allgather_einsum(ctx, "rhs_cols", self.Wt, self.X, self.Y, self.ws,
                                        flags=flags & ~cce.CCE_FLAG_FINE_GRAINED)
        cce.cce_fused_reduce_epilogue(ctx, self.P, self.b, self.R, self.out, 0.1, 0, 0)

    def oracle_sample(self, t=64):
        import numpy as np
        from oracle import einsum as oe
        f64 = _f64
        t0 = time.perf_counter()
        ref = oe.allgather_einsum("rhs_cols", [f64(w).T for w in self.Wt], [f64(x) for x in self.X])
        dt = time.perf_counter() - t0
        err = float(max(np.linalg.norm(f64(y) - r) / np.linalg.norm(r) for y, r in zip(self.Y, ref)))
        return dt, self.flops, "whole workload, float64 NumPy oracle", err


WORKLOADS = {c.name: c for c in (Gpt3Ffn, AttnOutProj, Mlp2, RsN8, AgFp32N2)}
# the configurations in the order the workload list of the benchmark names them
WORKLOAD_ORDER = ["ag_fp32_n2", "attn_outproj_n8", "mlp2_n4", "rs_n8", "gpt3_ffn_n8"]


def _f64(t):
    import numpy as np
    return t.detach().float().cpu().numpy().astype(np.float64)


# ---------------------------------------------------------------------------
# Measurement helpers
# ---------------------------------------------------------------------------
def timed(step, ctx, steps, flags, profile):
    import torch
    torch.cuda.synchronize()
    if profile:
        ctx.set_profiling(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step.run(ctx, flags)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    recs = []
    if profile:
        recs = ctx.read_profile()
        ctx.set_profiling(False)
    return wall, recs


def gemm_roofline(recs, dtype, steps):
    """Dominant GEMM kernel: the launch shape (by FLOPs per launch) with the
    largest total time."""
    groups = {}
    for r in recs:
        if r["kind"] != "gemm":
            continue
        groups.setdefault(r["flops"], []).append(r["ms"])
    if not groups:
        return None, {}
    per = {}
    for fl, ms in groups.items():
        avg = sum(ms) / len(ms)
        per[fl] = dict(flops_per_launch=fl, launches=len(ms), avg_ms=avg,
                       tflops=fl / (avg * 1e-3) / 1e12, total_ms=sum(ms) / steps)
    dom = max(per.values(), key=lambda d: d["total_ms"])
    peak = PEAK_TFLOPS[dtype]
    roof = {"bound": "mfma", "achieved": round(dom["tflops"], 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(dom["tflops"] / peak, 4), "traffic": None,
            "kernel": "grouped GEMM launch", "flops_per_launch": dom["flops_per_launch"],
            "avg_launch_ms": round(dom["avg_ms"], 4), "launches": dom["launches"]}
    return roof, per


def measured_traffic(workload, permute, transfer):
    """HBM bytes per GEMM launch from the committed FETCH_SIZE / WRITE_SIZE
    counter runs (profiles/traffic_<workload>.json), scaled by the factors a
    plain copy of known size gave.  None when no such run exists for this
    workload, permute form and ring direction, or when the GEMM source has
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    with open(os.path.join(ROOT, t["kernel_source"]), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if (sha != t["kernel_source_sha256"] or t.get("permute") != permute
            or t.get("transfer", "one-way") != transfer):
        return None
    return t["gemm_bytes_per_launch"]["mean"]


def epilogue_summary(recs, step):
    """Rates of the fused epilogue launches: over the bytes each launch moves,
    and over the workload's algorithmic bytes (one reduced partial) when
    those differ (the two-way ring's epilogue reads both chains' fp32
    accumulators)."""
    epi = [r for r in recs if r["kind"] == "epilogue"]
    if not epi:
        return None
    tb = sum(r["bytes"] for r in epi)
    tm = sum(r["ms"] for r in epi)
    gbs = tb / (tm * 1e-3) / 1e9
    out = {"GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
           "launches": len(epi), "avg_launch_ms": round(tm / len(epi), 4),
           "bytes_per_launch": tb / len(epi), "bytes": "moved by the launch"}
    alg = getattr(step, "epi_alg_bytes", None)
    if alg and abs(alg - tb / len(epi)) > 1e-3 * alg:
        ag = alg / (tm / len(epi) * 1e-3) / 1e9
        out["algorithmic"] = {"bytes_per_launch": alg, "GB/s": round(ag, 1),
                              "frac_of_hbm_peak": round(ag / PEAK_HBM_GBS, 4),
                              "bytes": "one reduced fp32 partial + residual + output + bias"}
    return out


def measure(step, ctx, workload, steps, warmup, main_flags, bid, permute, transfer, serial=True):
    """One workload: the timed steps (with the library's per-launch timing
    events), the dominant GEMM launch's roofline, the epilogue's HBM rate, the
    unlooped (monolithic) comparison, and the permute forms (stream, serial,
    fused) with the hidden copy fraction."""
    import torch
    import collective_overlap_amd as cce
    log(f"{workload}: warmup")
    for _ in range(warmup):
        step.run(ctx, main_flags)
    log(f"{workload}: timed region (permute {permute})")
    wall, recs = timed(step, ctx, steps, main_flags, profile=True)
    ms_per_step = wall / steps * 1e3
    value = step.flops * steps / wall / 1e12
    roof, per_shape = gemm_roofline(recs, step.dtype, steps)
    if roof is not None:
        roof["traffic"] = measured_traffic(workload, permute, transfer)
        if roof["traffic"] is not None:
            roof["traffic_unit"] = "bytes per launch (HBM, rocprofv3 counters)"
    epi_info = epilogue_summary(recs, step)
    gemm_ms = sum(r["ms"] for r in recs if r["kind"] == "gemm") / steps

    mono = None
    if hasattr(step, "monolithic") and serial:
        # The decomposition's cost: the same FLOPs as one grouped GEMM per
        # layer on pre-gathered operands, against the looped step.
        log(f"{workload}: the same layers unlooped (monolithic grouped GEMMs)")
        run_mono = step.monolithic()
        for _ in range(max(1, warmup // 2)):
            run_mono(ctx)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run_mono(ctx)
        torch.cuda.synchronize()
        mono_ms = (time.perf_counter() - t0) / steps * 1e3
        # the looped step again, like the monolithic one without the
        # library's timing events (they add a marker around every launch)
        w_plain, _ = timed(step, ctx, steps, main_flags, profile=False)
        plain_ms = w_plain / steps * 1e3
        mono = {"ms": round(mono_ms, 4), "TFLOP/s": round(step.flops / (mono_ms * 1e-3) / 1e12, 2),
                "looped_ms_without_timing_events": round(plain_ms, 4),
                "looped_step_over_monolithic": round(plain_ms / mono_ms, 4),
                "looped_gemms_over_monolithic": round(gemm_ms / mono_ms, 4)}
        del run_mono
        torch.cuda.empty_cache()

    overlap = None
    if serial and getattr(step, "has_permute", True):
        log(f"{workload}: copies on a second stream; the same kernels serialised")
        res = {}
        for name, fl in (("stream", bid), ("serial", cce.CCE_FLAG_SERIAL | bid)):
            for _ in range(max(1, warmup // 2)):
                step.run(ctx, fl)
            w, r = timed(step, ctx, steps, fl, profile=True)
            res[name] = (w / steps * 1e3, r)
        fused_ms = ms_per_step if main_flags & cce.CCE_FLAG_FUSED_PERMUTE else None
        if fused_ms is None:
            fl = cce.CCE_FLAG_FUSED_PERMUTE | bid
            for _ in range(max(1, warmup // 2)):
                step.run(ctx, fl)
            w, _ = timed(step, ctx, steps, fl, profile=False)
            fused_ms = w / steps * 1e3
        s_ms, srecs = res["serial"]
        st_ms = res["stream"][0]
        copy_ms = sum(r["ms"] for r in srecs if r["kind"] == "copy") / steps
        copy_bytes = sum(r["bytes"] for r in srecs if r["kind"] == "copy") / steps
        base = s_ms - copy_ms            # the same GEMMs and epilogues without the copies
        hidden = (round(min(1.0, max(0.0, 1.0 - (st_ms - base) / copy_ms)), 4)
                  if copy_ms > 0 else None)
        # The fused form has no copies to hide: the GEMMs send the data
        # themselves.  Its baseline is the serial form with the same GEMMs:
        # the ReduceScatter's stream and serial forms run two half-shard
        # chains, the fused form one whole-shard chain, so the serial run is
        # repeated with CCE_FLAG_ONE_CHAIN.  What the fused step takes beyond
        # that run less its copies is the cost of forwarding.
        s1_ms, copy1_ms = s_ms, copy_ms
        if getattr(step, "has_rs", False):
            fl = cce.CCE_FLAG_SERIAL | cce.CCE_FLAG_ONE_CHAIN | bid
            for _ in range(max(1, warmup // 2)):
                step.run(ctx, fl)
            w, r1 = timed(step, ctx, steps, fl, profile=True)
            s1_ms = w / steps * 1e3
            copy1_ms = sum(r["ms"] for r in r1 if r["kind"] == "copy") / steps
        base1 = s1_ms - copy1_ms
        overlap = {"serial_ms": round(s_ms, 3), "stream_ms": round(st_ms, 3),
                   "copy_ms_serial": round(copy_ms, 3),
                   "copy_GB/s_serial": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1) if copy_ms else None,
                   "hidden_copy_frac_stream": hidden,
                   "fused": {"permute": "eliminated: the GEMMs forward the data (no copies)",
                             "step_ms": round(fused_ms, 3),
                             "serial_same_gemms_ms": round(s1_ms, 3),
                             "copy_ms_same_gemms": round(copy1_ms, 3),
                             "forwarding_cost_ms": round(fused_ms - base1, 3),
                             "forwarding_cost_over_copies": (round((fused_ms - base1) / copy1_ms, 4)
                                                             if copy1_ms > 0 else None)},
                   "speedup_vs_serial": round(s_ms / ms_per_step, 4)}
    return {"ms_per_step": ms_per_step, "value": value, "roofline": roof, "per_shape": per_shape,
            "epilogue": epi_info, "gemm_ms": gemm_ms, "monolithic": mono, "overlap": overlap}


def copy_ceiling(dev, reps=10):
    """The plain read+write rate of this GPU's memory: a 1 GiB device copy
    (PyTorch's copy, the runtime's blit kernel), the practical ceiling the
    epilogue's HBM rate is set against beside the 8 TB/s peak."""
    import torch
    nb = 1 << 30
    src = torch.ones(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * nb / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"op": "plain device copy of 1 GiB (Tensor.copy_)", "bytes_moved": 2 * nb,
            "ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def graph_replay_ms(step, ctx, flags, steps, warmup):
    """The step captured once into a graph (torch.cuda.CUDAGraph over the
    library's calls: every entry point is capturable when the caller passes
    its workspace) and replayed: per-step time without the host's work per
    launch."""
    import torch
    step.run(ctx, flags)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run(ctx, flags)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    del g
    torch.cuda.synchronize()
    return ms


def preferred_bid(name):
    """The ring form a workload is benchmarked in: two-way unless its class
    says otherwise (the attention out-projection has no ring)."""
    import collective_overlap_amd as cce
    cls = WORKLOADS[name]
    if not getattr(cls, "has_permute", True) or getattr(cls, "transfer", "bidir") != "bidir":
        return 0
    return cce.CCE_FLAG_BIDIRECTIONAL


def config_summary(name, dev, ctx, steps, warmup, cpu_leg=True):
    """A workload other than the headline, measured in the benchmark's form
    (fused permute, the workload's ring form), for the same JSON line:
    per-step time and rate, the dominant GEMM launch's roofline, the
    epilogue's HBM rate, the permute forms and the unlooped comparison.
    With `cpu_leg` (the CPU-baseline leg, off with --no-cpu-baseline) the
    oracle also runs on a small sample of the workload on the host: its
    rate is the entry's cpu_baseline, and the timed outputs are checked
    against it (parity)."""
    import torch
    import collective_overlap_amd as cce
    step = WORKLOADS[name](dev)
    bid = preferred_bid(name)
    flags = cce.CCE_FLAG_FUSED_PERMUTE | bid
    m = measure(step, ctx, name, steps, warmup, flags, bid, "fused",
                "bidir" if bid else "one-way", serial=True)
    graph = None
    if getattr(step, "graph", False):
        g_ms = graph_replay_ms(step, ctx, flags, max(steps, 100), warmup)
        graph = {"ms_per_step": round(g_ms, 4), "TFLOP/s": round(step.flops / (g_ms * 1e-3) / 1e12, 3),
                 "how": "the step captured once (torch.cuda.CUDAGraph) and replayed"}
    else:
        step.run(ctx, flags)
        torch.cuda.synchronize()
    # CPU-baseline leg: the oracle on a small sample, which also checks the
    # outputs (they hold the last step's results: the last graph replay's
    # where the step was replayed)
    cpu, parity = None, None
    bar = 2e-2 if step.dtype == "bf16" else 1e-5
    if cpu_leg:
        dt, fl, desc, err = step.oracle_sample()
        if graph:
            desc += " (outputs of the last graph replay)"
        cpu = {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "kind": "oracle",
               "sample": desc, "seconds": round(dt, 3)}
        parity = {"rel_fro_err_vs_oracle": err, "bar": bar, "ok": err <= bar, "sample": desc}
    roof = m["roofline"]
    cfg = dict(step.config(), permute="fused")
    if getattr(step, "has_permute", True):
        cfg["transfer"] = "bidirectional" if bid else "one-way"
    out = {"config": cfg, "dtype": step.dtype,
           "ms_per_step": round(m["ms_per_step"], 4),
           "TFLOP/s": round(m["value"], 2),
           "frac_of_mfma_peak": round(m["value"] / PEAK_TFLOPS[step.dtype], 4),
           "gemm_launch": None if roof is None else {
               k: roof[k] for k in ("achieved", "frac", "avg_launch_ms", "flops_per_launch",
                                    "launches")},
           "epilogue": m["epilogue"], "overlap": m["overlap"], "monolithic": m["monolithic"],
           **({"graph_replay": graph} if graph else {}),
           "cpu_baseline": cpu, "parity": parity}
    del step
    torch.cuda.empty_cache()
    return out


def cpu_info():
    """The host's CPU model (from /proc/cpuinfo) and the cores this process
    may run on."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return model, affinity


VENDOR_SHAPES = [
    # name, groups, M, N, K (C = A B^T per group, bf16 operands, bf16 result)
    ("square_8192", 1, 8192, 8192, 8192),
    ("gpt3_ffn_layer1_looped", 16, 1024, 6144, 12288),
    ("gpt3_ffn_layer1_unlooped", 8, 8192, 6144, 12288),
    ("gpt3_ffn_layer2_looped", 16, 512, 12288, 6144),
    ("attn_outproj_local", 8, 8192, 8192, 1024),
]


def vendor_gemm(dev, steps, warmup):
    """The grouped GEMM against the vendor library on the same operands, in
    one process: hipBLASLt through torch.bmm (right factor passed as a
    contiguous [K, N] batch) and cce_grouped_gemm (right factor [N, K]), both
    bf16 in, fp32 accumulation, bf16 out.  Each shape's GEMM time from HIP
    events around `steps` back-to-back calls.  Both results are compared
    element by element (they differ only in accumulation order)."""
    import torch
    import collective_overlap_amd as cce
    import workloads as W
    ctx = cce.Context(0)
    rows = []
    for name, g, m, n, k in VENDOR_SHAPES:
        log(f"vendor gemm {name}: {g} x {m}x{n}x{k}")
        a = W.normal((g, m, k), 1.0, 1, device=dev)
        bt = W.normal((g, n, k), 0.02, 2, device=dev)          # [N, K] per group
        b_kn = bt.transpose(1, 2).contiguous()                  # [K, N] per group
        ours = torch.empty((g, m, n), device=dev, dtype=torch.bfloat16)
        lib_out = torch.empty_like(ours)
        al, bl, cl = list(a.unbind(0)), list(bt.unbind(0)), list(ours.unbind(0))

        def run_ours():
            cce.cce_grouped_gemm(ctx, al, bl, cl)

        def run_lib():
            torch.bmm(a, b_kn, out=lib_out)
        res = {}
        for tag, fn in (("hipblaslt", run_lib), ("ours", run_ours)):
            for _ in range(warmup):
                fn()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(steps):
                fn()
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / steps
            res[tag] = {"ms": round(ms, 4), "TFLOP/s": round(2.0 * g * m * n * k / (ms * 1e-3) / 1e12, 1)}
        d = (ours.float() - lib_out.float()).norm() / lib_out.float().norm()
        rows.append({"shape": name, "groups": g, "M": m, "N": n, "K": k, **res,
                     "ours_over_hipblaslt": round(res["ours"]["TFLOP/s"] / res["hipblaslt"]["TFLOP/s"], 4),
                     "rel_fro_diff": float(d)})
        del a, bt, b_kn, ours, lib_out, al, bl, cl
        torch.cuda.empty_cache()
    ctx.close()
    return rows


def epilogue_ceiling(dev, steps, warmup):
    """The fused epilogue's kernels on the benchmark shapes, each in two
    forms: the full epilogue (bias, dropout p = 0.1, residual) and the same
    partials with p = 0 and no bias or residual, which leaves the kernel
    moving data with one add per partial.  The ratio of the two rates is the
    cost of the epilogue's arithmetic; the second rate is what the kernel's
    access pattern reaches on this GPU.  Beside them, PyTorch's own
    elementwise kernels move the same bytes (`vendor_streaming`): the sum of
    the partials into a bf16 output, as one launch over the stacked batch,
    and a plain copy of every partial, as a streaming ceiling that does not
    come from this library (each working set exceeds the memory-side
    cache)."""
    import torch
    import collective_overlap_amd as cce
    import workloads as W
    ctx = cce.Context(0)
    rows = []
    shapes = [
        # name, partials, rows, cols, partial dtype, batch (ranks)
        ("attn_outproj_n8: 8 bf16 partials [8192, 8192]", 8, 8192, 8192, torch.bfloat16, 1),
        ("gpt3_ffn_n8: 2 fp32 accumulators [1024, 12288] x 8 ranks", 2, 1024, 12288, torch.float32, 8),
        ("gpt3_ffn_n8 one-way: 1 fp32 accumulator [1024, 12288] x 8 ranks", 1, 1024, 12288,
         torch.float32, 8),
    ]
    for name, n, r, c, pdt, nb in shapes:
        log(f"epilogue ceiling {name}")
        parts = [[W.normal((r, c), 1.0, 300 + 10 * b + k, device=dev, dtype=pdt) for k in range(n)]
                 for b in range(nb)]
        bias = W.normal((c,), 0.02, 90, device=dev)
        res = [W.normal((r, c), 1.0, 91 + b, device=dev) for b in range(nb)]
        out = [torch.empty((r, c), device=dev, dtype=torch.bfloat16) for _ in range(nb)]
        row0 = [b * r for b in range(nb)]
        esz = torch.tensor([], dtype=pdt).element_size()
        full_bytes = nb * r * c * (n * esz + 2 + 2) + c * 2
        bare_bytes = nb * r * c * (n * esz + 2)
        res_ = {}
        for tag, fn in (
                ("full", lambda: cce.cce_fused_reduce_epilogue_batched(
                    ctx, parts, bias, res, out, 0.1, 0, 0, mask_row0=row0, mask_col0=0, mask_ld=c)),
                ("data_only", lambda: cce.cce_fused_reduce_epilogue_batched(
                    ctx, parts, None, None, out, 0.0, 0, 0, mask_row0=row0, mask_col0=0, mask_ld=c))):
            for _ in range(warmup):
                fn()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(steps):
                fn()
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / steps
            nbytes = full_bytes if tag == "full" else bare_bytes
            res_[tag] = {"ms": round(ms, 4), "bytes": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del parts, res, out
        torch.cuda.empty_cache()
        # PyTorch's kernels over the same bytes: stacked partials [n, nb, r, c]
        stack = torch.stack([W.normal((nb, r, c), 1.0, 400 + k, device=dev, dtype=pdt)
                             for k in range(n)])
        o16 = torch.empty((nb, r, c), device=dev, dtype=torch.bfloat16)
        ocp = torch.empty_like(stack)
        if n == 1:
            vsum = ("cast copy to bf16 (Tensor.copy_)", lambda: o16.copy_(stack[0]))
        elif n == 2:
            vsum = ("add into bf16 (torch.add, out=)", lambda: torch.add(stack[0], stack[1], out=o16))
        else:
            vsum = ("sum over the partials into bf16 (torch.sum, dim=0, out=)",
                    lambda: torch.sum(stack, dim=0, out=o16))
        vendor = {}
        for tag, (what, fn), nbytes in (
                ("sum_like_data_only", vsum, bare_bytes),
                ("copy", ("plain copy of every partial (Tensor.copy_)", lambda: ocp.copy_(stack)),
                 2 * n * nb * r * c * esz)):
            for _ in range(warmup):
                fn()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(steps):
                fn()
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / steps
            vendor[tag] = {"op": what, "ms": round(ms, 4), "bytes": nbytes,
                           "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                           "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        rows.append({"shape": name, **res_,
                     "full_over_data_only_rate": round(res_["full"]["GB/s"] / res_["data_only"]["GB/s"], 4),
                     "vendor_streaming": vendor,
                     "data_only_over_vendor_sum": round(res_["data_only"]["GB/s"] /
                                                        vendor["sum_like_data_only"]["GB/s"], 4)})
        del stack, o16, ocp
        torch.cuda.empty_cache()
    ctx.close()
    return rows


def k_sweep(dev, steps, warmup):
    """The grouped GEMM of the GPT-3 FFN's AllGather launch shape (16 groups
    of 1024 x 6144, bf16 out) at several contraction lengths, with and
    without GELU: a straight-line fit of launch time against K gives the
    cost that does not scale with K (the tile's pipeline fill, epilogue and
    stores, the launch itself), and the difference between the two forms the
    cost of GELU.  Every launch does its whole work."""
    import torch
    import collective_overlap_amd as cce
    import workloads as W
    ctx = cce.Context(0)
    G, M, N = 16, 1024, 6144
    ks = [768, 1536, 3072, 6144, 12288]
    data = {}
    for k in ks:
        a = [W.normal((M, k), 1.0, g, device=dev) for g in range(G)]
        b = [W.normal((N, k), 0.02, 10 + g, device=dev) for g in range(G)]
        c = [torch.empty((M, N), device=dev, dtype=torch.bfloat16) for _ in range(G)]
        data[k] = (a, b, c)
    res = {(k, gl): [] for k in ks for gl in (False, True)}
    for _ in range(3):                      # rounds, interleaved
        for k in ks:
            for gl in (False, True):
                a, b, c = data[k]
                for _ in range(warmup):
                    cce.cce_grouped_gemm(ctx, a, b, c, gelu=gl)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    cce.cce_grouped_gemm(ctx, a, b, c, gelu=gl)
                e1.record()
                torch.cuda.synchronize()
                res[(k, gl)].append(e0.elapsed_time(e1) / steps)
    rows, fit = [], {}
    for gl in (False, True):
        pts = []
        for k in ks:
            v = sorted(res[(k, gl)])[1]
            pts.append((k, v))
            rows.append({"K": k, "gelu": gl, "ms": round(v, 4),
                         "TFLOP/s": round(2.0 * G * M * N * k / (v * 1e-3) / 1e12, 1)})
        # least squares over the two longest K (the linear regime)
        (k1, t1), (k2, t2) = pts[-2], pts[-1]
        slope = (t2 - t1) / (k2 - k1)
        fit["gelu" if gl else "no_gelu"] = {"ms_per_1024_k": round(slope * 1024, 5),
                                            "fixed_ms": round(t2 - slope * k2, 4)}
    gelu_ms = [round(sorted(res[(k, True)])[1] - sorted(res[(k, False)])[1], 4) for k in ks]
    ctx.close()
    return {"shape": f"{G} x {M} x {N} x K, bf16 out", "launches": rows, "fit": fit,
            "gelu_cost_ms_by_K": dict(zip(ks, gelu_ms))}


def hip_runtime():
    """The HIP runtime PyTorch already loaded (found by its soname)."""
    import ctypes
    import torch  # noqa: F401
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    return hip


def cu_masked_stream(hip, n_cus, cus):
    """A new stream (default priority) whose kernels run only on the compute
    units `cus` (indices into the runtime's CU mask)."""
    import ctypes
    words = (ctypes.c_uint32 * ((n_cus + 31) // 32))()
    for c in cus:
        words[c // 32] |= 1 << (c % 32)
    h = ctypes.c_void_p()
    err = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), len(words), words)
    if err != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({err})")
    return h.value


def cu_mask_sweep(dev, steps, warmup):
    """The stream form (copies on a second stream) with compute-unit masks:
    the copy stream limited to a few CUs, alone or with the GEMMs' stream
    limited to the others, against the context's own unmasked copy stream.
    The hidden fraction uses the serial step (same GEMMs, every copy on the
    compute stream) and its copy time from the same run."""
    import torch
    import collective_overlap_amd as cce
    from collective_overlap_amd._lib import CceError
    hip = hip_runtime()
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    ctx = cce.Context(0)
    out = []
    for wl in ("gpt3_ffn_n8", "rs_n8"):
        log(f"cu-mask sweep {wl}")
        step = WORKLOADS[wl](dev)
        bid = cce.CCE_FLAG_BIDIRECTIONAL
        for _ in range(warmup):
            step.run(ctx, cce.CCE_FLAG_SERIAL | bid)
        w, recs = timed(step, ctx, steps, cce.CCE_FLAG_SERIAL | bid, profile=True)
        s_ms = w / steps * 1e3
        copy_ms = sum(r["ms"] for r in recs if r["kind"] == "copy") / steps
        base = s_ms - copy_ms
        forms = [("own copy stream (no mask)", None, None)]
        for n in (8, 32):
            for layout, cus in (("first", list(range(n))),
                                ("strided", list(range(0, n_cus, n_cus // n))[:n])):
                rest = sorted(set(range(n_cus)) - set(cus))
                forms.append((f"copy on {n} CUs ({layout})", cus, None))
                forms.append((f"copy on {n} CUs ({layout}), GEMMs on the other {n_cus - n}",
                              cus, rest))
        forms.append(("copy stream with a mask of every CU", list(range(n_cus)), None))
        rows = []
        stop = False
        for name, ccus, gcus in forms:
            try:
                cs = cu_masked_stream(hip, n_cus, ccus) if ccus else None
            except RuntimeError as e:
                rows.append({"form": name, "error": str(e)})
                continue
            try:
                gs = cu_masked_stream(hip, n_cus, gcus) if gcus else None
            except RuntimeError as e:
                hip.hipStreamDestroy(cs)
                rows.append({"form": name, "error": str(e)})
                continue
            ctx.set_copy_stream(cs)
            try:
                with torch.cuda.stream(torch.cuda.ExternalStream(gs) if gs
                                       else torch.cuda.current_stream()):
                    for _ in range(warmup):
                        step.run(ctx, bid)
                    w, _ = timed(step, ctx, steps, bid, profile=False)
            except CceError as e:
                # A runtime that cannot give the masked stream a queue fails
                # its first launch, and may fail later launches too: stop.
                rows.append({"form": name, "error": str(e)})
                stop = True
            finally:
                try:
                    torch.cuda.synchronize()
                except Exception as e:     # (the runtime's state after such a failure)
                    rows.append({"form": name, "synchronize_error": str(e).splitlines()[0]})
                    stop = True
                ctx.set_copy_stream(None)
                for h in (cs, gs):
                    if h:
                        hip.hipStreamDestroy(h)
            if stop:
                break
            ms = w / steps * 1e3
            rows.append({"form": name, "step_ms": round(ms, 3),
                         "hidden_copy_frac": round(1.0 - (ms - base) / copy_ms, 4)})
        out.append({"workload": wl, "serial_ms": round(s_ms, 3), "copy_ms_serial": round(copy_ms, 3),
                    "n_cus": n_cus, "stream_form": rows})
        del step
        if stop:
            break
        torch.cuda.empty_cache()
    if not stop:
        ctx.close()
    return out


def mfma_ceiling(iters=200000):
    """Run the MFMA ceiling program (collective_overlap_amd/mfma_ceiling, a
    child process) and summarise its measurements: median TFLOP/s per
    variant and its fraction of the bf16 peak."""
    import subprocess
    exe = os.path.join(ROOT, "collective_overlap_amd", "mfma_ceiling")
    if not os.path.exists(exe):
        raise SystemExit(f"{exe} is missing: build with `python -m collective_overlap_amd.build`")
    r = subprocess.run([exe, str(iters)], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        raise SystemExit(f"mfma_ceiling failed ({r.returncode}): {r.stderr.strip()}")
    rows = [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]
    out = {}
    for row in rows:
        out.setdefault((row["mfma"], row["operands"]), []).append(row["TFLOP/s"])
    res = []
    for (mf, op), v in out.items():
        v = sorted(v)
        med = v[len(v) // 2]
        res.append({"mfma": mf, "operands": op, "TFLOP/s": med, "all": v,
                    "frac_of_peak": round(med / PEAK_TFLOPS["bf16"], 4)})
    return res


def hbm_ceiling(reps=5):
    """Run the HBM streaming ceiling program (collective_overlap_amd/
    hbm_ceiling, a child process): for each read:write mix, the fastest of its
    variants (unroll depth, cache hint, grid) and the whole sweep."""
    import subprocess
    exe = os.path.join(ROOT, "collective_overlap_amd", "hbm_ceiling")
    if not os.path.exists(exe):
        raise SystemExit(f"{exe} is missing: build with `python -m collective_overlap_amd.build`")
    r = subprocess.run([exe, str(reps)], capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise SystemExit(f"hbm_ceiling failed ({r.returncode}): {r.stderr.strip()}")
    rows = [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]
    best = {}
    for row in rows:
        if row["mix"] not in best or row["GB/s"] > best[row["mix"]]["GB/s"]:
            best[row["mix"]] = row
    summary = [{"mix": m, "GB/s": b["GB/s"], "frac_of_hbm_peak": round(b["GB/s"] / PEAK_HBM_GBS, 4),
                "unroll": b["unroll"], "nontemporal": b["nontemporal"],
                "workgroups": b["workgroups"], "loop": b["loop"]} for m, b in best.items()]
    return {"best": summary, "sweep": rows}


def ab_libs(dev, paths, workloads, rounds, steps, warmup):
    """A/B timing of library builds: the benchmark's form (fused permute,
    the workload's ring form) of each workload's step under every build in `paths`
    (e.g. two git revisions built with `python -m collective_overlap_amd.build
    --rev REV --out PATH`), interleaved round by round in one process so that
    clock and power drift hit every build alike.  Per build: the median,
    minimum and maximum of the rounds' mean step times."""
    import torch
    import collective_overlap_amd as cce
    from collective_overlap_amd import _lib
    builds = {}
    for p in paths:
        _lib._lib = None
        _lib.LIB_PATH = os.path.abspath(p)
        builds[p] = (_lib.lib(), cce.Context(0))
    out = []
    for wl in workloads:
        log(f"a/b {wl}")
        flags = cce.CCE_FLAG_FUSED_PERMUTE | preferred_bid(wl)
        step = WORKLOADS[wl](dev)
        res = {p: [] for p in paths}
        for _ in range(rounds):
            for p in paths:
                lib, ctx = builds[p]
                _lib._lib = lib
                for _ in range(warmup):
                    step.run(ctx, flags)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(steps):
                    step.run(ctx, flags)
                torch.cuda.synchronize()
                res[p].append((time.perf_counter() - t0) / steps * 1e3)
        rows = []
        for p in paths:
            v = sorted(res[p])
            rows.append({"lib": p, "median_ms": round(v[len(v) // 2], 4), "min_ms": round(v[0], 4),
                         "max_ms": round(v[-1], 4), "rounds": [round(x, 4) for x in res[p]]})
        base = rows[0]["median_ms"]
        for r in rows:
            r["over_first"] = round(r["median_ms"] / base, 4)
        out.append({"workload": wl, "builds": rows})
        del step
        torch.cuda.empty_cache()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt3_ffn_n8", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-serial", action="store_true", help="skip the unoverlapped comparison")
    ap.add_argument("--permute", choices=("fused", "stream", "serial", "dma"), default="fused",
                    help="fused: each partial GEMM sends the data itself; stream: async "
                         "copies on a second stream ordered by events; serial: the stream "
                         "form's kernels, every copy on the caller's stream; dma: the stream "
                         "form with the copies on the SDMA engines")
    ap.add_argument("--transfer", choices=("bidir", "one-way"), default=None,
                    help="bidir: two-way ring, two partial einsums per iteration, ceil(n/2) "
                         "iterations; one-way: the ring of the loop's pairs only (default: the "
                         "workload's faster form, two-way except rs_n8)")
    ap.add_argument("--allreduce", action="store_true",
                    help="attn_outproj_n8: FusedAllReduce epilogue, the result on every rank")
    ap.add_argument("--separate-epilogue", action="store_true",
                    help="gpt3_ffn_n8: the ReduceScatter stores its fp32 result and a second "
                         "call applies the epilogue (default: one call, the accumulators go "
                         "straight into the epilogue)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (by default each is measured after the "
                         "headline one and reported under `configs` of the same JSON line)")
    ap.add_argument("--fine-grained", action="store_true",
                    help="the ReduceScatter's chunk consumer (epilogue or align-and-sum) runs "
                         "inside its last launch (CCE_FLAG_FINE_GRAINED; fused permute)")
    ap.add_argument("--ab", nargs="+", metavar="LIB",
                    help="only time the listed library builds against each other (A/B, "
                         "interleaved rounds in one process); prints one JSON line")
    ap.add_argument("--ab-workloads", default="gpt3_ffn_n8,rs_n8",
                    help="comma-separated workloads for --ab")
    ap.add_argument("--ab-rounds", type=int, default=8, help="interleaved rounds for --ab")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only run the MFMA ceiling program: the bf16 rate the matrix cores "
                         "sustain on MFMAs and LDS operand reads alone; prints one JSON line")
    ap.add_argument("--k-sweep", action="store_true",
                    help="only time the GPT-3 AllGather launch shape at several K, with and "
                         "without GELU (fixed cost per launch, cost of GELU); one JSON line")
    ap.add_argument("--cu-mask-sweep", action="store_true",
                    help="only time the stream form of gpt3_ffn_n8 and rs_n8 with the copy "
                         "stream (and optionally the GEMMs' stream) limited to some compute "
                         "units; prints one JSON line")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only compare the grouped GEMM with hipBLASLt (torch.bmm) on the "
                         "headline shapes; prints one JSON line")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="only run the HBM streaming ceiling program (read, write, copy and the "
                         "epilogue's read:write mixes); prints one JSON line")
    ap.add_argument("--epilogue-ceiling", action="store_true",
                    help="only time the fused epilogue's kernels on the benchmark shapes, full "
                         "and reduced to moving data; prints one JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MiB",
                    help="only run `steps` plain device copies of MiB mebibytes (the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    a = ap.parse_args(argv)

    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU: all N logical ranks live as "
                                   "separate HBM buffers of a single MI355X; --gpus must be 1",
                          "n_gpus": a.gpus}), flush=True)
        return 2

    if a.mfma_ceiling:
        # (before this process touches the GPU: the program is a child)
        print(json.dumps({"mfma_ceiling": mfma_ceiling(), "peak_TFLOP/s": PEAK_TFLOPS["bf16"],
                          "loop": "128 x 128 x 32 wave tile per iteration, operands read "
                                  "from LDS, no global memory traffic, one workgroup per CU"}),
              flush=True)
        return 0
    if a.hbm_ceiling:
        # (a child process, like the MFMA ceiling)
        print(json.dumps({"hbm_ceiling": hbm_ceiling(), "peak_GB/s": PEAK_HBM_GBS,
                          "streams": "1 GiB each, 16-byte vectors, XOR of the inputs written"}),
              flush=True)
        return 0
    import torch
    import collective_overlap_amd as cce
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = "cuda:0"
    if a.calibrate_copy:
        nb = a.calibrate_copy * 2**20
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(a.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / a.steps
        print(json.dumps({"calibrate_copy_bytes": nb, "read_bytes": nb, "write_bytes": nb,
                          "steps": a.steps, "GB/s": round(2 * nb / dt / 1e9, 1)}), flush=True)
        return 0
    if a.epilogue_ceiling:
        print(json.dumps({"epilogue_ceiling": epilogue_ceiling(dev, a.steps, a.warmup),
                          "hbm_peak_GB/s": PEAK_HBM_GBS}), flush=True)
        return 0
    if a.ab:
        wls = a.ab_workloads.split(",")
        for w in wls:
            if w not in WORKLOADS:
                raise SystemExit(f"unknown workload {w}")
        print(json.dumps({"ab": ab_libs(dev, a.ab, wls, a.ab_rounds, a.steps, a.warmup),
                          "form": "fused permute, each workload's ring form", "steps_per_round": a.steps}),
              flush=True)
        return 0
    if a.cu_mask_sweep:
        print(json.dumps({"cu_mask_sweep": cu_mask_sweep(dev, a.steps, a.warmup)}), flush=True)
        return 0
    if a.k_sweep:
        print(json.dumps({"k_sweep": k_sweep(dev, a.steps, a.warmup)}), flush=True)
        return 0
    if a.vendor_gemm:
        print(json.dumps({"vendor_gemm": vendor_gemm(dev, a.steps, a.warmup),
                          "peak_TFLOP/s": PEAK_TFLOPS["bf16"]}), flush=True)
        return 0
    log(f"device {torch.cuda.get_device_name(0)}; workload {a.workload}")
    step = WORKLOADS[a.workload](dev)
    if a.allreduce:
        if not hasattr(step, "use_allreduce"):
            raise SystemExit("--allreduce applies to attn_outproj_n8 only")
        step.use_allreduce()
    if a.separate_epilogue:
        if not hasattr(step, "fuse_epilogue"):
            raise SystemExit("--separate-epilogue applies to gpt3_ffn_n8 only")
        step.fuse_epilogue = False
    ctx = cce.Context(0)
    torch.cuda.synchronize()
    if a.transfer is None:
        a.transfer = "bidir" if preferred_bid(a.workload) else "one-way"
    bid = cce.CCE_FLAG_BIDIRECTIONAL if a.transfer == "bidir" else 0
    main_flags = {"fused": cce.CCE_FLAG_FUSED_PERMUTE, "stream": 0, "serial": cce.CCE_FLAG_SERIAL,
                  "dma": cce.CCE_FLAG_COPY_DMA}[a.permute] | bid
    if a.fine_grained:
        main_flags |= cce.CCE_FLAG_FINE_GRAINED
    m = measure(step, ctx, a.workload, a.steps, a.warmup, main_flags, bid, a.permute,
                a.transfer, serial=not a.no_serial)
    ms_per_step, value, roof, per_shape = m["ms_per_step"], m["value"], m["roofline"], m["per_shape"]
    epi_info, gemm_ms, mono, overlap = m["epilogue"], m["gemm_ms"], m["monolithic"], m["overlap"]

    cpu = None
    parity = None
    if not a.no_cpu_baseline:
        log("cpu baseline: oracle on a bounded sample")
        try:
            from threadpoolctl import threadpool_info
            threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        except Exception:
            threads = os.cpu_count()
        # A short calibration run sizes the sample to about CPU_SAMPLE_S of
        # oracle work on this host (capped by the workload's rows).
        dt, fl, desc, err = step.oracle_sample()
        cap = getattr(step, "sample_cap", 0)
        t = getattr(step, "sample_default", 0)
        for _ in range(2):       # the oracle runs faster per row on larger samples
            if not cap or dt >= 0.8 * CPU_SAMPLE_S or t >= cap:
                break
            t_next = min(cap, int(t * CPU_SAMPLE_S / max(dt, 1e-3)))
            if t_next <= t:
                break
            log(f"cpu baseline: {t_next} rows ({dt:.2f} s at {t})")
            t = t_next
            dt, fl, desc, err = step.oracle_sample(t)
        model, affinity = cpu_info()
        cpu = {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle", "sample": desc, "seconds": round(dt, 3),
               "host_cpus": os.cpu_count(), "affinity_cpus": affinity, "blas_threads": threads,
               "cpu_model": model}
        parity = {"rel_fro_err_vs_oracle": err, "bar": 2e-2 if step.dtype == "bf16" else 1e-5,
                  "ok": err <= (2e-2 if step.dtype == "bf16" else 1e-5)}
        if getattr(step, "epi_oracle", None):
            es, elems = step.epi_oracle
            # bytes the device epilogue moves per element (fp32 partial, bf16
            # residual and output), for a rate comparable with its GB/s
            cpu["epilogue_oracle"] = {"seconds": round(es, 4), "elements": elems,
                                      "Melements/s": round(elems / es / 1e6, 2),
                                      "GB/s_at_device_bytes": round(8.0 * elems / es / 1e9, 3)}

    ceiling = copy_ceiling(dev)
    if epi_info is not None:
        epi_info["frac_of_copy_ceiling"] = round(epi_info["GB/s"] / ceiling["GB/s"], 4)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": step.dtype,
        "data": "synthetic (seeded torch generators; no dataset)",
        "config": dict(step.config(), permute=a.permute,
                       **({"chunk_consumer": "in the last launch"} if a.fine_grained else {}),
                       **({"epilogue": "fused_allreduce"} if a.allreduce else {}),
                       **({"epilogue": "in the ReduceScatter" if step.fuse_epilogue
                           else "separate call"} if hasattr(step, "fuse_epilogue") else {}),
                       **({"transfer": "bidirectional" if bid else "one-way"}
                          if a.workload != "attn_outproj_n8" else {})),
        "frac_of_mfma_peak": round(value / PEAK_TFLOPS[step.dtype], 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "epilogue": epi_info,
        "hbm_copy_ceiling": ceiling,
        "overlap": overlap,
        "monolithic": mono,
        "gemm_ms_per_step": round(gemm_ms, 3),
        "gemm_shapes": list(per_shape.values()),
        "parity": parity,
    }
    if not a.no_configs:
        # Every other workload, in the benchmark's form, under one key.
        configs = {}
        for name in WORKLOAD_ORDER:
            if name == a.workload:
                continue
            log(f"config {name}")
            configs[name] = config_summary(name, dev, ctx, min(a.steps, 10), max(2, a.warmup),
                                           cpu_leg=not a.no_cpu_baseline)
        out["configs"] = configs
    print(json.dumps(out), flush=True)
    ctx.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
