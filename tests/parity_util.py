"""Helpers shared by the GPU parity tests: device upload of seeded inputs, oracle values of
the same inputs, and the per-tensor error bound.

Tolerance (per output tensor, floating point): max|gpu - ref| / max|ref| <= 1e-2 and
||gpu - ref||_F / ||ref||_F <= 4e-3, against the float64 oracle on the identical rounded
inputs.  Integer and byte outputs (int4 codes, scales, dequantised bits) must match exactly.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

MAX_RATIO = 1e-2
FROB = 4e-3


def bits_to_dev(bits: np.ndarray, dev="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(dev).view(torch.bfloat16)


def to_dev(inp, name: str, dev="cuda") -> torch.Tensor:
    a = getattr(inp, name)
    if a.dtype == np.uint16:
        return bits_to_dev(a, dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def values(inp, name: str) -> np.ndarray:
    """Exact float64 values of an input as both sides see it."""
    a = getattr(inp, name)
    if a.dtype == np.uint16:
        return oracle.bf16_bits_to_f64(a)
    return a.astype(np.float64)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    d = got - ref
    mr = np.max(np.abs(ref)) if ref.size else 0.0
    ratio = (np.max(np.abs(d)) / mr) if mr > 0 else float(np.max(np.abs(d), initial=0.0))
    fr = np.linalg.norm(ref)
    frob = (np.linalg.norm(d) / fr) if fr > 0 else float(np.linalg.norm(d))
    return float(ratio), float(frob)


def assert_close(name: str, got, ref, max_ratio=MAX_RATIO, frob=FROB):
    ratio, fr = errors(got, ref)
    print(f"    {name}: max-ratio {ratio:.3e}  frob {fr:.3e}", flush=True)
    assert ratio <= max_ratio, f"{name}: max|err|/max|ref| = {ratio:.3e} > {max_ratio}"
    assert fr <= frob, f"{name}: relative Frobenius error {fr:.3e} > {frob}"


def sample_rows(M: int, seed: int = 0, extra: int = 24):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 15, 16, 127, 128, 255, 256, 257, M // 2, M - 257, M - 256, M - 2, M - 1]
    rows = {r for r in fixed if 0 <= r < M}
    rows |= set(rng.integers(0, M, size=min(extra, M)).tolist())
    return np.array(sorted(rows))
