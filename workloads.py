"""Seeded synthetic inputs and the named workload shapes.

This module holds no arithmetic of the method: it only draws random tensors
with fixed seeds and names the shapes of the five workloads.  Both the CPU
oracle's tests and the device path's tests and benchmark take their inputs
from here, so the two sides see identical values.

Recipe: tensor number k of a workload is drawn from its own
``torch.Generator(device).manual_seed(1000 * base_seed + k)``; N(0, s) is
``randn * s``, U(-1, 1) is ``rand * 2 - 1``.  Values that the device stores in
bf16 are rounded to bf16 here (torch's conversion), and the oracle receives
those exact bf16 values upcast to float64.  Weights are drawn directly in the
device's storage orientation [out_features, in_features] (the nn.Linear
layout); the mathematical factor [in, out] is their transpose, which the
tests hand to the oracle.  The entries are i.i.d., so the orientation in which
they are drawn does not change the distribution.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    desc: str
    n_ranks: int
    dtype: str                    # "f32" or "bf16"
    shapes: dict = field(default_factory=dict)


# The five workloads.  Shapes are [rows, cols] in mathematical orientation
# unless the key says "_store" (device storage orientation [out, in]).
WORKLOADS = {
    "ag_fp32_n2": Workload(
        "ag_fp32_n2",
        "N=2 fp32 AllGather-Einsum case 1 (weight shards split on columns) "
        "plus a fused epilogue over 2 partials",
        2, "f32",
        dict(X=(64, 256), W_shard=(256, 512), P=(64, 256), bias=(256,),
             R=(64, 256), p_drop=0.1)),
    "attn_outproj_n8": Workload(
        "attn_outproj_n8",
        "Megatron attention out-projection, 8 ranks, bf16: in[8192,1024] x "
        "w[1024,8192] per rank sliced on the contraction dim, then the fused "
        "reduce epilogue over the 8 local partials",
        8, "bf16",
        dict(IN=(8192, 1024), W=(1024, 8192), bias=(8192,), R=(8192, 8192),
             p_drop=0.1)),
    "mlp2_n4": Workload(
        "mlp2_n4",
        "2-layer MLP, 4-way, bf16: X[2048,4096]; W1[4096,16384] and "
        "W2[16384,4096] gathered by looped AllGather-Einsum; GELU between",
        4, "bf16",
        dict(X=(2048, 4096), W1_shard=(4096, 4096), W2_shard=(16384, 1024))),
    "rs_n8": Workload(
        "rs_n8",
        "Einsum-ReduceScatter, 8 ranks, bf16 operands / fp32 accumulator: "
        "X[16384,2048] x W[2048,4096] per rank, out shard [2048,4096]",
        8, "bf16",
        dict(X=(16384, 2048), W=(2048, 4096))),
    "gpt3_ffn_n8": Workload(
        "gpt3_ffn_n8",
        "GPT-3-scale FFN, 8-way, bf16: 8192 tokens, hidden 12288, FFN 49152; "
        "looped AllGather-Einsum into W1 shards, GELU, looped "
        "Einsum-ReduceScatter out of W2 shards, fused bias+dropout+residual",
        8, "bf16",
        dict(X_shard=(1024, 12288), W1=(12288, 6144), W2=(6144, 12288),
             bias=(12288,), R=(1024, 12288), p_drop=0.1)),
}


def _gen(device, base_seed: int, k: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(1000 * base_seed + k)
    return g


def normal(shape, std: float, k: int, device="cpu", base_seed: int = 0,
           dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, std) in float32, then converted to `dtype`."""
    x = torch.randn(tuple(shape), generator=_gen(device, base_seed, k),
                    device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def uniform(shape, k: int, device="cpu", base_seed: int = 0,
            dtype=torch.float32) -> torch.Tensor:
    """U(-1, 1) in float32, then converted to `dtype`."""
    x = torch.rand(tuple(shape), generator=_gen(device, base_seed, k),
                   device=device, dtype=torch.float32)
    return (x * 2.0 - 1.0).to(dtype)


def int_probe(shape, k: int, lo: int = -4, hi: int = 4, device="cpu",
              base_seed: int = 7, dtype=torch.float32) -> torch.Tensor:
    """Small integers in [lo, hi]: every product and every partial sum of a
    contraction of length <= 2^24 / (hi^2) is then an exact float32 integer,
    whatever the summation order."""
    x = torch.randint(lo, hi + 1, tuple(shape),
                      generator=_gen(device, base_seed, k), device=device)
    return x.to(dtype)


def weight_store(in_features: int, out_features: int, std: float, k: int,
                 device="cpu", base_seed: int = 0,
                 dtype=torch.bfloat16) -> torch.Tensor:
    """A weight in storage orientation [out_features, in_features]."""
    return normal((out_features, in_features), std, k, device, base_seed, dtype)
