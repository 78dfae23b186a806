"""Helpers shared by the GPU parity tests (no arithmetic of the method)."""

from __future__ import annotations

import numpy as np
import torch


def np64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a (bf16 or fp32) tensor."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def assert_bf16_close(got, ref, what=""):
    """Bar for bf16 storage with fp32 accumulation: relative Frobenius error
    <= 2e-2, and every element within 2^-7 relative (one bf16 rounding of
    the result plus fp32 accumulation error) of the float64 reference, with
    an absolute floor scaled to the tensor's magnitude."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    e = rel_fro(got, ref)
    assert e <= 2e-2, f"{what}: rel Frobenius error {e:.3e}"
    scale = np.sqrt(np.mean(ref * ref)) if ref.size else 1.0
    bad = np.abs(got - ref) > (2.0 ** -7) * np.abs(ref) + 1e-3 * scale
    assert not bad.any(), f"{what}: {bad.sum()} elements off, first at {np.argwhere(bad)[0]}"


def assert_f32_close(got, ref, what="", tol=1e-5):
    e = rel_fro(got, ref)
    assert e <= tol, f"{what}: rel Frobenius error {e:.3e} > {tol}"


def sync():
    torch.cuda.synchronize()
