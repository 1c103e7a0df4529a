"""Seeded synthetic inputs for the LoRA / QLoRA layer, shared by the tests, the bench
and the oracle's callers.

This module draws random numbers and rounds them to the storage type; it holds
none of the layer's arithmetic.  Recipe (the workloads' own definition):

* one NumPy ``Generator(PCG64(seed))`` per input set, drawing float64 tensors in
  the fixed order X, W, A, B, dY;
* X, dY ~ N(0, 1); W ~ N(0, 1/K); A ~ U(-1/sqrt(K), 1/sqrt(K));
  B ~ N(0, 0.02) read as variance 0.02 (``b_dist="var"``, the default) or as
  standard deviation 0.02 (``b_dist="std"``);
* each tensor is rounded once: float64 -> fp32 (round to nearest even), then, for
  bf16 workloads, fp32 -> bf16 by torch's conversion (round to nearest even);
* for int4 workloads W stays fp32: it is the quantiser's input.

bf16 tensors are returned as ``uint16`` bit patterns so that every consumer sees
the identical bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# The layer shapes these workloads stand in for: a LoRA attention projection with
# the tutorial's 4096 x 4096 base weight and rank-16 adapters, a SwiGLU MLP's
# gate/up and down projections, and a QLoRA FFN projection of width 27648.
WORKLOADS = {
    "tiny_f32": dict(dtype="f32", M=64, N=256, K=256, R=8, alpha=16.0, seed=1, int4=False),
    "attn_proj": dict(dtype="bf16", M=8192, N=4096, K=4096, R=16, alpha=32.0, seed=2, int4=False),
    "mlp_gate_up": dict(dtype="bf16", M=8192, N=14336, K=4096, R=16, alpha=32.0, seed=3, int4=False),
    "mlp_down": dict(dtype="bf16", M=8192, N=4096, K=14336, R=16, alpha=32.0, seed=3, int4=False),
    "qlora_ffn": dict(dtype="bf16", M=4096, N=27648, K=5120, R=16, alpha=32.0, seed=4, int4=True),
    "decode_up": dict(dtype="bf16", M=1, N=27648, K=5120, R=16, alpha=32.0, seed=5, int4=True),
    "decode_down": dict(dtype="bf16", M=1, N=5120, K=27648, R=16, alpha=32.0, seed=5, int4=True),
}
DECODE_M = (1, 4, 8)


@dataclass
class Inputs:
    M: int
    N: int
    K: int
    R: int
    alpha: float
    dtype: str            # "f32" or "bf16": the type X, W, A, B, dY are stored in
    int4: bool
    seed: int
    X: np.ndarray         # float32 (f32) or uint16 bf16 bits (bf16)
    W: np.ndarray         # same as X; for int4 workloads the fp32 quantiser input
    A: np.ndarray
    B: np.ndarray
    dY: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return self.alpha / self.R


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _round(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return _to_bf16_bits(x32)
    raise ValueError(dtype)


def make_inputs(M: int, N: int, K: int, R: int, *, seed: int, dtype: str = "bf16",
                alpha: Optional[float] = None, int4: bool = False, b_dist: str = "var",
                with_dy: bool = True) -> Inputs:
    """Draw one input set (see the module docstring for the recipe)."""
    if alpha is None:
        alpha = 2.0 * R
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K)) * np.sqrt(1.0 / K)
    a = 1.0 / np.sqrt(K)
    A = rng.uniform(-a, a, size=(R, K))
    if b_dist == "var":
        bsd = np.sqrt(0.02)
    elif b_dist == "std":
        bsd = 0.02
    else:
        raise ValueError(b_dist)
    B = rng.standard_normal((N, R)) * bsd
    dY = rng.standard_normal((M, N)) if with_dy else None
    inp = Inputs(
        M=M, N=N, K=K, R=R, alpha=float(alpha), dtype=dtype, int4=int4, seed=seed,
        X=_round(X, dtype),
        W=W.astype(np.float32) if int4 else _round(W, dtype),
        A=_round(A, dtype),
        B=_round(B, dtype),
        dY=None if dY is None else _round(dY, dtype),
        meta=dict(b_dist=b_dist, numpy=np.__version__),
    )
    return inp


def workload_inputs(name: str, *, M: Optional[int] = None, b_dist: str = "var",
                    with_dy: bool = True) -> Inputs:
    w = dict(WORKLOADS[name])
    if M is not None:
        w["M"] = M
    return make_inputs(w["M"], w["N"], w["K"], w["R"], seed=w["seed"], dtype=w["dtype"],
                       alpha=w["alpha"], int4=w["int4"], b_dist=b_dist,
                       with_dy=with_dy and not name.startswith("decode"))


@dataclass
class SwigluInputs:
    """One input set of the SwiGLU gate/up pair (bf16 bit patterns, uint16)."""
    M: int
    N: int
    K: int
    R: int
    alpha: float
    seed: int
    X: np.ndarray
    Wg: np.ndarray
    Wu: np.ndarray
    Ag: np.ndarray
    Au: np.ndarray
    Bg: np.ndarray
    Bu: np.ndarray
    dH: Optional[np.ndarray]

    @property
    def scale(self) -> float:
        return self.alpha / self.R

    @property
    def Wgu(self) -> np.ndarray:
        """The gate and up weights stacked by rows, [Wg; Wu] (2N x K)."""
        return np.concatenate([self.Wg, self.Wu], axis=0)


def make_swiglu_inputs(M: int, N: int, K: int, R: int, *, seed: int, alpha: Optional[float] = None,
                       with_dh: bool = True) -> SwigluInputs:
    """Draw a SwiGLU input set: the distributions of make_inputs (X, dH ~ N(0,1); each W ~
    N(0, 1/K); each A ~ U(+-1/sqrt K); each B ~ N(0, variance 0.02)), drawn in the order X, Wg,
    Wu, Ag, Au, Bg, Bu, dH and rounded once to bf16."""
    if alpha is None:
        alpha = 2.0 * R
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((M, K))
    Wg = rng.standard_normal((N, K)) * np.sqrt(1.0 / K)
    Wu = rng.standard_normal((N, K)) * np.sqrt(1.0 / K)
    a = 1.0 / np.sqrt(K)
    Ag = rng.uniform(-a, a, size=(R, K))
    Au = rng.uniform(-a, a, size=(R, K))
    Bg = rng.standard_normal((N, R)) * np.sqrt(0.02)
    Bu = rng.standard_normal((N, R)) * np.sqrt(0.02)
    dH = rng.standard_normal((M, N)) if with_dh else None
    r = lambda v: None if v is None else _round(v, "bf16")
    return SwigluInputs(M=M, N=N, K=K, R=R, alpha=float(alpha), seed=seed, X=r(X), Wg=r(Wg), Wu=r(Wu),
                        Ag=r(Ag), Au=r(Au), Bg=r(Bg), Bu=r(Bu), dH=r(dH))


@dataclass
class NormInputs:
    """Seeded inputs of the RMSNorm ahead of a projection, as bf16 bit patterns (uint16)."""
    M: int
    K: int
    eps: float
    seed: int
    X: np.ndarray   # M x K
    g: np.ndarray   # K
    dY: Optional[np.ndarray]  # M x K


def make_norm_inputs(M: int, K: int, *, seed: int, eps: float = 1e-5, with_dy: bool = True) -> NormInputs:
    """Draw an RMSNorm input set: hidden-state rows X ~ N(0, 1) each scaled by exp(U(-2, 2)) (rows
    of different magnitude, so the reciprocal RMS varies over e^4), the per-feature scale
    g ~ U(0.5, 1.5), and dY ~ N(0, 1); drawn in that order and rounded once to bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((M, K)) * np.exp(rng.uniform(-2.0, 2.0, size=(M, 1)))
    g = rng.uniform(0.5, 1.5, size=K)
    dY = rng.standard_normal((M, K)) if with_dy else None
    return NormInputs(M=M, K=K, eps=float(eps), seed=seed, X=_round(X, "bf16"), g=_round(g, "bf16"),
                      dY=None if dY is None else _round(dY, "bf16"))


@dataclass
class CeInputs:
    """Seeded inputs of the cross-entropy over an LM head: X, W as bf16 bit patterns, labels int32."""
    M: int
    K: int
    V: int
    seed: int
    X: np.ndarray       # M x K
    W: np.ndarray       # V x K
    labels: np.ndarray  # M


def make_ce_inputs(M: int, K: int, V: int, *, seed: int, logit_std: float = 1.0) -> CeInputs:
    """Hidden states X ~ N(0, 1), the LM head W ~ N(0, logit_std^2 / K) (logits of standard deviation
    about logit_std), labels uniform in [0, V); drawn in that order, X and W rounded once to bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((V, K)) * (logit_std / np.sqrt(K))
    labels = rng.integers(0, V, size=M).astype(np.int32)
    return CeInputs(M=M, K=K, V=V, seed=seed, X=_round(X, "bf16"), W=_round(W, "bf16"), labels=labels)
