"""Float64 CPU oracle for the fused LoRA / QLoRA linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never imports it, and this
module imports nothing from the product package: the two share no code.

What it computes, and where the pages define it
-----------------------------------------------
Sources are the web pages on Unsloth.  They are cited by page title and section:

* LoRA layer: tutorial ch. 5 "加速原理：Triton kernel 与 fused LoRA", §5.3, the
  LoRA equation ``y = W x + (alpha/r) B A x`` with ``A`` (r x d), ``B`` (d x r);
  the same equation appears in tutorial ch. 1 "项目背景与定位", §1.2, as
  ``Delta W = (alpha/r) B A``.
* Row form of the equation: a batch of row vectors X (M x K) gives
  ``Y = X W^T + (alpha/r) (X A^T) B^T``; the rank-r product X A^T is formed first and
  ``B A`` is never materialised (it is only the brute-force check in the tests).
* Backward: §5.3's paragraph on the fused backward (gradients for X, A, B; W only
  "if trained", and here W is frozen) and the hand-derived-backward section of
  the wisestudy.cn Unsloth essay.  The gradients below are derived by hand from
  the loss convention ``L = <dY, Y>_F``.
* SwiGLU gate/up pair: tutorial ch. 5 §5.6 "fused SwiGLU",
  ``SwiGLU(x) = (W_g x ⊙ σ(W_g x)) ⊙ W_u x`` (σ the logistic function; the output
  projection W_d is another linear layer), with §5.3's LoRA update on the gate and
  on the up projection; gradients derived by hand from ``L = <dH, H>_F``.
* RMSNorm: tutorial ch. 5 §5.4 "fused RMSNorm", ``x / sqrt(mean(x^2) + eps) * g``
  over the hidden dimension, g a learnable per-feature scale; the gradients are
  derived by hand from ``L = <dY, Y>_F``.
* Chunked cross-entropy: tutorial ch. 5 §5.7, the LM head's logits X W^T are never
  formed for the whole batch; chunks of tokens each compute their logits, loss and
  gradient and drop the logits, and the chunk losses are summed.  Gradients derived by
  hand: d loss_m / d logits_m = softmax(logits_m) - onehot(label_m).
* RoPE: tutorial ch. 5 §5.5, each pair of coordinates of q and k rotated by an angle; the
  pairing of the page's listing (x_j with x_{j + rot/2}, the rest passed through) and the
  usual frequencies theta_j = pos * base^(-2j/rot); the backward is the inverse rotation.
* FP4 weights: the same page names FP4 beside INT4 for the 4-bit weights.  Its
  format is read as the OCP Microscaling (MX) FP4: blocks of 32 consecutive k share
  a power-of-two scale 2^(E-127) (E8M0), each element an E2M1 value (sign, 2
  exponent bits with bias 1, 1 mantissa bit; no infinities or NaN), the block
  exponent floor(log2(absmax)) - 2, round to nearest even with saturation at 6.
* 4-bit weights: "探微索隐：Unsloth 如何加速 LLM 推理？（以 Qwen 27B 为例）", §二.3
  (4-bit weights read compactly, unpacked in registers by a scaling coefficient,
  restored to FP16/BF16 before the matrix units).  The concrete format (symmetric
  int4 in -7..7, two per byte, groups of 64 along K, fp16 scale = absmax/7) is
  this repository's workload definition; the pages fix none of its details.

Readings taken where the pages are silent:
  row-major tokens, W is (N x K) = (out x in), A is (R x K), B is (N x R);
  scale = alpha / r passed as a number; no dropout; dW is not computed;
  XA = X A^T is the unscaled fp32 panel saved for backward; gradients overwrite;
  int4: low nibble holds the even k, 4-bit two's complement, ties to even,
  a group whose fp16 scale is 0 stores q = 0, dequantised weight =
  bf16_rne(q * s) (the product is exact in fp32).

Precision: every matrix product is a float64 NumPy matmul on the exact values of
the rounded inputs; nothing inside is rounded.  Integer decisions (the int4
codes) are taken on exact values (see ``quantize_int4``).

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle.py`` (brute force, closed forms, finite differences,
invariants, library witnesses, hand-worked fixtures under ``tests/golden/``).
"""
from __future__ import annotations

import numpy as np

GROUP = 64
QMAX = 7

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (uint16): the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    IEEE-754 rounding written on the bit pattern: add 0x7FFF plus the lowest kept
    bit, then drop the low 16 bits.  Inputs here are finite (no NaN handling needed).
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def fp16_rne(x: np.ndarray) -> np.ndarray:
    """Correctly rounded float64 -> IEEE binary16 (NumPy's cast rounds to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


# ---------------------------------------------------------------------------
# int4 groupwise format (page "探微索隐 ...", §二.3; format details are readings)
# ---------------------------------------------------------------------------


def quantize_int4(w: np.ndarray, group: int = GROUP):
    """Symmetric groupwise int4 quantisation of an fp32 weight ``w`` (N x K).

    Per row n and group g of ``group`` consecutive k:
      a = max |w|                       (exact)
      s = fp16_rne(a / 7)               (float64 quotient, one rounding to fp16)
      q = clip(rint(w / s), -7, 7)      (ties to even) ; q = 0 for the group if s == 0

    The code decision is exact: the float64 quotient w/s of an fp32 w and an fp16 s
    never lands on a half-integer unless the exact quotient is one, so ``rint``
    sees the exact tie or the exact side of it.

    Returns (q int8 N x K, s float16 N x K/group).
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    wg = w.astype(np.float64).reshape(n, k // group, group)
    a = np.abs(wg).max(axis=2)
    if np.any(a / QMAX > 65504.0):
        raise ValueError("group absmax too large for an fp16 scale")
    s16 = fp16_rne(a / QMAX)
    s = s16.astype(np.float64)
    safe = np.where(s == 0.0, 1.0, s)
    q = np.rint(wg / safe[:, :, None])
    q = np.clip(q, -QMAX, QMAX)
    q = np.where((s == 0.0)[:, :, None], 0.0, q)
    return q.reshape(n, k).astype(np.int8), s16


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two 4-bit two's-complement codes per byte; the low nibble holds the even k."""
    q = np.asarray(q, dtype=np.int8)
    n, k = q.shape
    if k % 2:
        raise ValueError("K must be even")
    lo = q[:, 0::2].astype(np.int16) & 0xF
    hi = q[:, 1::2].astype(np.int16) & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_int4``: sign-extend each nibble (0x8..0xF -> -8..-1)."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    n, kb = p.shape
    q = np.empty((n, 2 * kb), dtype=np.int8)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    return q


def dequant_int4_bits(packed: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Dequantised weight as bf16 bits: bf16_rne(float32(q) * float32(s)).

    The product of a 4-bit integer and an fp16 scale has at most 3 + 11 significant
    bits, so it is exact in fp32; the only rounding is the one to bf16.
    """
    q = unpack_int4(packed).astype(np.float64)
    n, k = q.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    s = np.repeat(s, group, axis=1)
    prod = (q * s).astype(np.float32)  # exact
    return f32_to_bf16_rne(prod)


def dequant_int4(packed: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Dequantised weight as float64 values (the exact bf16 values)."""
    return bf16_bits_to_f64(dequant_int4_bits(packed, scales, group))


# ---------------------------------------------------------------------------
# The LoRA layer (tutorial ch. 5 §5.3 equation; tutorial ch. 1 §1.2 equation)
# ---------------------------------------------------------------------------


def _f64(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def lora_forward(X, W, A, B, scale):
    """The §5.3 LoRA equation y = W x + (alpha/r) B (A x), applied to each row x of X.

    X: M x K, W: N x K, A: R x K, B: N x R, scale = alpha / r.
    Returns (Y, P) in float64: Y (M x N) the layer output and P = X A^T (M x R), the
    unscaled rank-R projection of every token (the state the backward reuses).
    """
    X, W, A, B = _f64(X, W, A, B)
    P = lora_projection(X, A)
    Y = X @ W.T + float(scale) * (P @ B.T)
    return Y, P


def lora_projection(X, A):
    """P = X A^T (M x R): the rank-R projection A x of every token row x, float64."""
    X, A = _f64(X, A)
    return X @ A.T


def lora_backward(dY, X, W, A, B, scale, XA=None):
    """Hand-derived gradients of L = <dY, Y>_F with W frozen.

    G  = dY B                     (M x R)
    dX = dY W + scale * G A       (M x K)
    dA = scale * G^T X            (R x K)
    dB = scale * dY^T (X A^T)     (N x R)
    """
    dY, X, W, A, B = _f64(dY, X, W, A, B)
    s = float(scale)
    xa = X @ A.T if XA is None else np.asarray(XA, dtype=np.float64)
    G = dY @ B
    dX = dY @ W + s * (G @ A)
    dA = s * (G.T @ X)
    dB = s * (dY.T @ xa)
    return dX, dA, dB


def lora_backward_adapters(dY, X, A, B, scale, XA=None):
    """The adapter gradients of ``lora_backward`` alone (no dX, so W is not needed):

    dA = scale * (dY B)^T X   (R x K),   dB = scale * dY^T (X A^T)   (N x R).

    Returns (dA, dB), float64.  XA, when given, is the saved X A^T.
    """
    dY, X, A, B = _f64(dY, X, A, B)
    s = float(scale)
    xa = X @ A.T if XA is None else np.asarray(XA, dtype=np.float64)
    G = dY @ B
    return s * (G.T @ X), s * (dY.T @ xa)


def lora_forward_rows(X, W, A, B, scale, rows):
    """Rows ``rows`` of (Y, XA), computed one row set at a time (for full-size sampling)."""
    rows = np.asarray(rows)
    return lora_forward(np.asarray(X)[rows], W, A, B, scale)


def lora_backward_dx_rows(dY, W, A, B, scale, rows):
    """Rows ``rows`` of dX = dY W + scale * (dY B) A."""
    rows = np.asarray(rows)
    dYr, W, A, B = _f64(np.asarray(dY)[rows], W, A, B)
    return dYr @ W + float(scale) * ((dYr @ B) @ A)


# ---------------------------------------------------------------------------
# SwiGLU gate/up pair with LoRA on both projections
# (tutorial ch. 5 §5.6, fused SwiGLU: SwiGLU(x) = (W_g x ⊙ σ(W_g x)) ⊙ W_u x, the output
# projection W_d being a separate linear layer; §5.3's LoRA update on the gate and the up
# projection; gradients derived by hand from L = <dH, H>_F)
# ---------------------------------------------------------------------------


def sigmoid(g):
    """Logistic function 1 / (1 + exp(-g)) in float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):  # exp(-g) = inf for g < -709 gives exactly 0
        return 1.0 / (1.0 + np.exp(-g))


def silu(g):
    """g * sigmoid(g): the gate's activation in §5.6's SwiGLU."""
    g = np.asarray(g, dtype=np.float64)
    return g * sigmoid(g)


def silu_grad(g):
    """d silu / d g = sigmoid(g) * (1 + g * (1 - sigmoid(g)))."""
    g = np.asarray(g, dtype=np.float64)
    s = sigmoid(g)
    return s * (1.0 + g * (1.0 - s))


def swiglu_lora_forward(X, Wg, Wu, Ag, Au, Bg, Bu, scale):
    """H = silu(G) ⊙ U with G = X Wg^T + scale (X Ag^T) Bg^T and U likewise with Wu, Au, Bu.

    X: M x K; Wg, Wu: N x K; Ag, Au: R x K; Bg, Bu: N x R.
    Returns (H, G, U, XAg, XAu), float64: H, G, U are M x N, XAg, XAu are M x R.
    """
    G, xag = lora_forward(X, Wg, Ag, Bg, scale)
    U, xau = lora_forward(X, Wu, Au, Bu, scale)
    return silu(G) * U, G, U, xag, xau


def swiglu_lora_backward(dH, X, Wg, Wu, Ag, Au, Bg, Bu, scale):
    """Gradients of L = <dH, H>_F with Wg, Wu frozen.

    dU = dH ⊙ silu(G),  dG = dH ⊙ U ⊙ silu'(G), then the LoRA backward of each projection:
    dX = dXg + dXu; returns (dX, dAg, dAu, dBg, dBu).
    """
    dH = np.asarray(dH, dtype=np.float64)
    G, _ = lora_forward(X, Wg, Ag, Bg, scale)
    U, _ = lora_forward(X, Wu, Au, Bu, scale)
    dU = dH * silu(G)
    dG = dH * U * silu_grad(G)
    dXg, dAg, dBg = lora_backward(dG, X, Wg, Ag, Bg, scale)
    dXu, dAu, dBu = lora_backward(dU, X, Wu, Au, Bu, scale)
    return dXg + dXu, dAg, dAu, dBg, dBu


def swiglu_lora_backward_adapters(dH, X, Wg, Wu, Ag, Au, Bg, Bu, scale):
    """The four adapter gradients of ``swiglu_lora_backward`` without dX: the same dG and dU
    from the forward's G and U, then ``lora_backward_adapters`` of each projection.
    Returns (dAg, dAu, dBg, dBu), float64."""
    dH = np.asarray(dH, dtype=np.float64)
    G, xag = lora_forward(X, Wg, Ag, Bg, scale)
    U, xau = lora_forward(X, Wu, Au, Bu, scale)
    dU = dH * silu(G)
    dG = dH * U * silu_grad(G)
    dAg, dBg = lora_backward_adapters(dG, X, Ag, Bg, scale, XA=xag)
    dAu, dBu = lora_backward_adapters(dU, X, Au, Bu, scale, XA=xau)
    return dAg, dAu, dBg, dBu


def swiglu_lora_rows(X, Wg, Wu, Ag, Au, Bg, Bu, scale, rows):
    """Rows ``rows`` of (H, G, U) (for full-size sampling)."""
    rows = np.asarray(rows)
    G, _ = lora_forward_rows(X, Wg, Ag, Bg, scale, rows)
    U, _ = lora_forward_rows(X, Wu, Au, Bu, scale, rows)
    return silu(G) * U, G, U


def swiglu_lora_backward_dx_rows(dH, X, Wg, Wu, Ag, Au, Bg, Bu, scale, rows):
    """Rows ``rows`` of dX of the SwiGLU pair (each row needs only its own G, U and dH)."""
    rows = np.asarray(rows)
    H, G, U = swiglu_lora_rows(X, Wg, Wu, Ag, Au, Bg, Bu, scale, rows)
    dHr = np.asarray(dH, dtype=np.float64)[rows]
    dU = dHr * silu(G)
    dG = dHr * U * silu_grad(G)
    return (lora_backward_dx_rows(dG, Wg, Ag, Bg, scale, np.arange(len(rows)))
            + lora_backward_dx_rows(dU, Wu, Au, Bu, scale, np.arange(len(rows))))


# ---------------------------------------------------------------------------
# RMSNorm (tutorial ch. 5 §5.4, fused RMSNorm: each row divided by the root of its mean
# square plus eps, then scaled per feature by g; gradients derived by hand from L = <dY, Y>_F)
# ---------------------------------------------------------------------------


def rmsnorm_forward(X, g, eps):
    """Y[m, k] = X[m, k] * r[m] * g[k] with r[m] = 1 / sqrt(mean_k X[m, k]^2 + eps).

    X: M x K, g: K.  Returns (Y, r), float64: Y is M x K, r (the reciprocal RMS the
    backward reuses) has M entries.
    """
    X, g = _f64(X, g)
    ms = np.mean(X * X, axis=1)
    r = 1.0 / np.sqrt(ms + float(eps))
    return X * r[:, None] * g[None, :], r


def rmsnorm_backward(dY, X, g, eps):
    """Gradients of L = <dY, Y>_F: returns (dX, dg), float64.

    With xh = X * r (row-wise) and dr / dX[m, j] = -r^3 X[m, j] / K:
      dX[m, j] = r (g[j] dY[m, j] - xh[m, j] * (1/K) sum_k g[k] dY[m, k] xh[m, k]),
      dg[k]    = sum_m dY[m, k] xh[m, k].
    """
    dY, X, g = _f64(dY, X, g)
    K = X.shape[1]
    _, r = rmsnorm_forward(X, g, eps)
    xh = X * r[:, None]
    gdy = dY * g[None, :]
    c = np.sum(gdy * xh, axis=1) / K
    dX = r[:, None] * (gdy - xh * c[:, None])
    dg = np.sum(dY * xh, axis=0)
    return dX, dg


# ---------------------------------------------------------------------------
# MXFP4 weights ("探微索隐：Unsloth 如何加速 LLM 推理？（以 Qwen 27B 为例）", §二.3 names FP4
# beside INT4; the block format is the OCP Microscaling FP4: 32 E2M1 elements per E8M0 scale)
# ---------------------------------------------------------------------------

FP4_BLOCK = 32


def fp4_e2m1_value(code):
    """Value of 4-bit E2M1 codes from the bit fields: sign s (bit 3), exponent e (bits 2..1,
    bias 1), mantissa m (bit 0); e = 0 is subnormal: m * 0.5, else (1 + m/2) * 2^(e-1)."""
    c = np.asarray(code, dtype=np.int64)
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def mxfp4_block_exponent(amax):
    """Shared exponent of a block: floor(log2(amax)) - 2 (2 is E2M1's largest exponent), clamped to
    [-125, 125] so that every nonzero element and the largest value stay normal in bf16; a block
    of zeros takes 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))  # amax = f 2^ex, f in [0.5, 1)
    se = np.clip(ex - 1 - 2, -125, 125)
    return np.where(amax > 0, se, 0).astype(np.int64)


def quantize_mxfp4(w):
    """MXFP4 codes of an fp32 weight W (N x K, K a multiple of 32), decided on exact values.

    Each element's magnitude |w| / 2^se is rounded to the nearest E2M1 magnitude
    {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the one with mantissa bit 0, values past 6 to 6; the
    sign bit is set for w < 0 (also when the magnitude rounds to 0).  Returns (codes, E): codes
    uint8 in 0..15 (N x K), E = se + 127 as uint8 (N x K/32).
    """
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    N, K = w.shape
    if K % FP4_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blk = w.reshape(N, K // FP4_BLOCK, FP4_BLOCK)
    se = mxfp4_block_exponent(np.max(np.abs(blk), axis=2))
    x = np.abs(blk) / np.exp2(se)[:, :, None]  # exact: a power-of-two scaling
    grid = fp4_e2m1_value(np.arange(8))
    dist = np.abs(x[..., None] - grid)
    best = dist.min(axis=-1, keepdims=True)
    tied = dist == best
    # among the nearest (one, or two at a midpoint) take the even code: its mantissa bit is 0
    even = tied & (np.arange(8) % 2 == 0)
    mag = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(tied, axis=-1))
    codes = (mag | np.where(blk < 0, 8, 0)).astype(np.uint8).reshape(N, K)
    return codes, (se + 127).astype(np.uint8)


def pack_fp4(codes):
    """Two codes per byte, even k in the low nibble: N x K -> N x K/2 uint8."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def dequant_mxfp4(packed, E):
    """W~[n][k] = e2m1(code) * 2^(E[n][k/32] - 127), float64 (exact; also exact in bf16, since it has
    at most two significant bits and the clamped exponents keep it normal)."""
    codes = unpack_fp4(packed)
    se = np.asarray(E, dtype=np.int64) - 127
    return fp4_e2m1_value(codes) * np.exp2(np.repeat(se, FP4_BLOCK, axis=1))


# ---------------------------------------------------------------------------
# Chunked cross-entropy over an LM head (tutorial ch. 5 §5.7: chunks of tokens each compute
# their logits, loss and gradient, the logits of the whole batch are never formed, and the
# chunk losses are summed; gradients derived by hand)
# ---------------------------------------------------------------------------


def cross_entropy_rows(X, W, labels):
    """Per-token loss of the logits X W^T: loss_m = logsumexp_v(logits[m]) - logits[m, label_m].

    X: M x K, W: V x K (the LM head), labels: M ints in [0, V).  Returns (loss, lse), float64,
    each with M entries; the log-sum-exp is taken around the row maximum.
    """
    X, W = _f64(X, W)
    labels = np.asarray(labels, dtype=np.int64)
    logits = X @ W.T
    mx = logits.max(axis=1)
    lse = mx + np.log(np.sum(np.exp(logits - mx[:, None]), axis=1))
    return lse - logits[np.arange(len(labels)), labels], lse


def cross_entropy_grad(X, W, labels, grad_scale):
    """dX of L = grad_scale * sum_m loss_m: dlogits = grad_scale (softmax - onehot), dX = dlogits W.
    Returns (dX, dlogits), float64."""
    X, W = _f64(X, W)
    labels = np.asarray(labels, dtype=np.int64)
    logits = X @ W.T
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    p[np.arange(len(labels)), labels] -= 1.0
    dlogits = grad_scale * p
    return dlogits @ W, dlogits


def cross_entropy_chunked(X, W, labels, chunk=256):
    """The page's procedure: for each chunk of `chunk` tokens, its logits, losses and gradient
    (for the mean loss over all M tokens), then the logits are dropped and the losses summed.
    Returns (mean loss, dX)."""
    X = np.asarray(X, dtype=np.float64)
    M = X.shape[0]
    total, dX = 0.0, np.zeros_like(X)
    for c0 in range(0, M, chunk):
        sl = slice(c0, min(M, c0 + chunk))
        loss, _ = cross_entropy_rows(X[sl], W, labels[sl])
        total += float(np.sum(loss))
        dX[sl] = cross_entropy_grad(X[sl], W, labels[sl], 1.0 / M)[0]
    return total / M, dX


# ---------------------------------------------------------------------------
# RoPE (tutorial ch. 5 §5.5: each coordinate pair of q and k multiplied by a 2 x 2 rotation; the
# listing pairs x_j with x_{j + rot/2} for j < rot/2 and passes the remaining coordinates through)
# ---------------------------------------------------------------------------


def rope_angles(positions, rot, base):
    """theta[t, j] = pos_t * base^(-2 j / rot), j < rot/2, float64."""
    pos = np.asarray(positions, dtype=np.float64)
    j = np.arange(rot // 2, dtype=np.float64)
    return pos[:, None] * np.power(float(base), -2.0 * j / rot)[None, :]


def rope_apply(x, positions, rot, base, inverse=False):
    """Rotate x (M x H x D: tokens, heads, head dimension) by the angles of each token's position:
    (x_j, x_{j+rot/2}) -> (x_j cos - x_{j+rot/2} sin, x_{j+rot/2} cos + x_j sin), by -theta when
    inverse (the gradient of the rotation); coordinates rot .. D-1 unchanged.  Returns float64."""
    x = np.asarray(x, dtype=np.float64)
    th = rope_angles(positions, rot, base) * (-1.0 if inverse else 1.0)
    c, s = np.cos(th)[:, None, :], np.sin(th)[:, None, :]
    h = rot // 2
    out = x.copy()
    a, b = x[..., :h], x[..., h:rot]
    out[..., :h] = a * c - b * s
    out[..., h:rot] = b * c + a * s
    return out
