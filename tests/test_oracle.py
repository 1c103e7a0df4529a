"""CPU pins of the float64 oracle (no GPU).

Each test checks the oracle against something other than itself: hand-worked
fixtures under tests/golden/, exact rational brute force, finite differences,
Euler-homogeneity invariants, special cases that reduce to a library routine, and
library witnesses (torch float64 autograd, torch's bf16 conversion, the struct
module's IEEE half conversion).  A dropped term, a wrong sign, a transposed
operand or a wrong rounding rule in ``oracle/`` fails at least one of them.
"""
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def test_bf16_rne_hand_cases():
    with open(os.path.join(GOLDEN, "bf16_rne_cases.txt")) as f:
        rows = [l.split()[:2] for l in f if l.strip() and not l.startswith("#")]
    src = np.array([int(a, 16) for a, _ in rows], dtype=np.uint32).view(np.float32)
    want = np.array([int(b, 16) for _, b in rows], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16_rne(src), want)


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1 << 20).astype(np.float32)
    # force many exact ties and near-ties
    u = x.view(np.uint32).copy()
    u[: 1 << 16] = (u[: 1 << 16] & 0xFFFF0000) | 0x8000
    u[1 << 16: 1 << 17] = (u[1 << 16: 1 << 17] & 0xFFFF0000) | 0x7FFF
    x = u.view(np.float32)
    torch_bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16_rne(x), torch_bits)


def test_bf16_bits_to_f64_roundtrip():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite only
    vals = oracle.bf16_bits_to_f64(bits)
    witness = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(vals, witness)


def test_fp16_rne_against_struct_half():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000) * 0.01, rng.standard_normal(2000) * 1e-6,
                        # exact fp16 ties: midpoints between neighbouring halves
                        (np.arange(1025, 1100, dtype=np.float64) + 0.5) * 2.0 ** -10])
    got = oracle.fp16_rne(x)
    want = np.array([np.frombuffer(struct.pack("<e", v), dtype=np.float16)[0] for v in x])
    np.testing.assert_array_equal(got.view(np.uint16), want.view(np.uint16))


# ---------------------------------------------------------------------------
# LoRA forward
# ---------------------------------------------------------------------------

def _fixture_lora():
    f = _read_fixture("lora_worked_example.txt")
    M, K, N, R = (int(f[k][0]) for k in ("M", "K", "N", "R"))
    alpha = float(f["alpha"][0])

    def mat(key, r, c):
        return np.array([float(v) for v in f[key]]).reshape(r, c)

    return dict(M=M, K=K, N=N, R=R, s=alpha / R, X=mat("X", M, K), W=mat("W", N, K),
                A=mat("A", R, K), B=mat("B", N, R), dY=mat("dY", M, N), XA=mat("XA", M, R),
                Y=mat("Y", M, N), dX=mat("dX", M, K), dA=mat("dA", R, K), dB=mat("dB", N, R))


def test_forward_hand_worked_example():
    f = _fixture_lora()
    Y, XA = oracle.lora_forward(f["X"], f["W"], f["A"], f["B"], f["s"])
    np.testing.assert_array_equal(Y, f["Y"])
    np.testing.assert_array_equal(XA, f["XA"])


def test_backward_hand_worked_example():
    f = _fixture_lora()
    dX, dA, dB = oracle.lora_backward(f["dY"], f["X"], f["W"], f["A"], f["B"], f["s"])
    np.testing.assert_array_equal(dX, f["dX"])
    np.testing.assert_array_equal(dA, f["dA"])
    np.testing.assert_array_equal(dB, f["dB"])


def _frac_matrix(a):
    return [[Fraction(float(v)) for v in row] for row in np.asarray(a)]


@pytest.mark.parametrize("M,K,N,R,zero_w", [(3, 5, 4, 2, False), (4, 8, 6, 3, False),
                                            (2, 7, 3, 1, True), (5, 4, 7, 4, False)])
def test_forward_against_materialised_delta_w(M, K, N, R, zero_w):
    """Brute force: Y = X (W + s B A)^T with Delta W built explicitly, in exact rationals."""
    rng = np.random.default_rng(10 + M * 100 + K)
    X = rng.standard_normal((M, K)).astype(np.float32).astype(np.float64)
    W = np.zeros((N, K)) if zero_w else rng.standard_normal((N, K)).astype(np.float32).astype(np.float64)
    A = rng.uniform(-1, 1, (R, K)).astype(np.float32).astype(np.float64)
    B = rng.standard_normal((N, R)).astype(np.float32).astype(np.float64)
    s = Fraction(3, 2)
    Xf, Wf, Af, Bf = map(_frac_matrix, (X, W, A, B))
    dW = [[sum(Bf[n][i] * Af[i][k] for i in range(R)) * s for k in range(K)] for n in range(N)]
    Weff = [[Wf[n][k] + dW[n][k] for k in range(K)] for n in range(N)]
    exact = [[sum(Xf[m][k] * Weff[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
    Y, XA = oracle.lora_forward(X, W, A, B, float(s))
    ex = np.array([[float(v) for v in row] for row in exact])
    assert np.max(np.abs(Y - ex)) <= 1e-12 * max(1.0, np.max(np.abs(ex)))
    xa_exact = np.array([[float(sum(Xf[m][k] * Af[i][k] for k in range(K))) for i in range(R)]
                         for m in range(M)])
    assert np.max(np.abs(XA - xa_exact)) <= 1e-12 * max(1.0, np.max(np.abs(xa_exact)))


def test_forward_zero_adapter_is_plain_matmul_bitwise():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((17, 64))
    W = rng.standard_normal((48, 64))
    A = rng.standard_normal((8, 64))
    Y, _ = oracle.lora_forward(X, W, A, np.zeros((48, 8)), 2.0)
    np.testing.assert_array_equal(Y, np.matmul(X, W.T))
    Y0, _ = oracle.lora_forward(X, W, A, rng.standard_normal((48, 8)), 0.0)
    np.testing.assert_array_equal(Y0, np.matmul(X, W.T))


def test_forward_rows_matches_full():
    rng = np.random.default_rng(4)
    X, W = rng.standard_normal((40, 32)), rng.standard_normal((24, 32))
    A, B = rng.standard_normal((4, 32)), rng.standard_normal((24, 4))
    Y, XA = oracle.lora_forward(X, W, A, B, 2.0)
    rows = [0, 7, 39, 13]
    Yr, XAr = oracle.lora_forward_rows(X, W, A, B, 2.0, rows)
    np.testing.assert_allclose(Yr, Y[rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(XAr, XA[rows], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# LoRA backward
# ---------------------------------------------------------------------------

def _loss(dY, X, W, A, B, s):
    Y, _ = oracle.lora_forward(X, W, A, B, s)
    return float(np.sum(dY * Y))


@pytest.mark.parametrize("M,K,N,R", [(3, 5, 4, 2), (6, 4, 7, 3)])
def test_backward_central_differences(M, K, N, R):
    """L = <dY, Y> is linear in X, in A and in B separately, so a central difference
    with a unit step has no truncation error: it equals the gradient up to rounding."""
    rng = np.random.default_rng(20 + M)
    X, W = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    A, B = rng.standard_normal((R, K)), rng.standard_normal((N, R))
    dY, s = rng.standard_normal((M, N)), 1.75
    dX, dA, dB = oracle.lora_backward(dY, X, W, A, B, s)

    def fd(which, shape):
        g = np.zeros(shape)
        for idx in np.ndindex(*shape):
            args = {"X": X, "A": A, "B": B}
            plus = {k: v.copy() for k, v in args.items()}
            minus = {k: v.copy() for k, v in args.items()}
            plus[which][idx] += 1.0
            minus[which][idx] -= 1.0
            g[idx] = (_loss(dY, plus["X"], W, plus["A"], plus["B"], s)
                      - _loss(dY, minus["X"], W, minus["A"], minus["B"], s)) / 2.0
        return g

    for name, got in (("X", dX), ("A", dA), ("B", dB)):
        want = fd(name, got.shape)
        np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-9)


def test_backward_against_torch_autograd_float64():
    rng = np.random.default_rng(5)
    M, K, N, R, s = 33, 40, 24, 6, 2.0
    X, W = rng.standard_normal((M, K)), rng.standard_normal((N, K)) / np.sqrt(K)
    A, B = rng.uniform(-0.2, 0.2, (R, K)), rng.standard_normal((N, R)) * 0.14
    dY = rng.standard_normal((M, N))
    tX, tA, tB = (torch.tensor(v, dtype=torch.float64, requires_grad=True) for v in (X, A, B))
    tW = torch.tensor(W, dtype=torch.float64)
    Y = tX @ tW.T + (tX @ tA.T @ tB.T) * s
    Y.backward(torch.tensor(dY, dtype=torch.float64))
    dX, dA, dB = oracle.lora_backward(dY, X, W, A, B, s)
    np.testing.assert_allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, tA.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dB, tB.grad.numpy(), rtol=1e-12, atol=1e-12)
    Yo, _ = oracle.lora_forward(X, W, A, B, s)
    np.testing.assert_allclose(Yo, Y.detach().numpy(), rtol=1e-12, atol=1e-12)


def test_backward_homogeneity_invariants():
    """Euler: <dX, X> = <dY, Y>; <dA, A> = <dB, B> = s <dY, XA B^T> (the LoRA part of L)."""
    rng = np.random.default_rng(6)
    M, K, N, R, s = 96, 80, 72, 8, 2.0
    X, W = rng.standard_normal((M, K)), rng.standard_normal((N, K)) / np.sqrt(K)
    A, B = rng.uniform(-0.1, 0.1, (R, K)), rng.standard_normal((N, R)) * 0.14
    dY = rng.standard_normal((M, N))
    Y, XA = oracle.lora_forward(X, W, A, B, s)
    dX, dA, dB = oracle.lora_backward(dY, X, W, A, B, s)
    L = np.sum(dY * Y)
    Lr = s * np.sum(dY * np.matmul(np.matmul(X, A.T), B.T))
    assert abs(np.sum(dX * X) - L) <= 1e-10 * max(1.0, abs(L))
    assert abs(np.sum(dA * A) - Lr) <= 1e-10 * max(1.0, abs(Lr))
    assert abs(np.sum(dB * B) - Lr) <= 1e-10 * max(1.0, abs(Lr))


def test_backward_zero_adapter_cases():
    rng = np.random.default_rng(7)
    M, K, N, R = 12, 16, 8, 4
    X, W, dY = rng.standard_normal((M, K)), rng.standard_normal((N, K)), rng.standard_normal((M, N))
    A, B = rng.standard_normal((R, K)), rng.standard_normal((N, R))
    dX, dA, dB = oracle.lora_backward(dY, X, W, A, np.zeros((N, R)), 2.0)
    assert not dA.any()
    np.testing.assert_array_equal(dX, np.matmul(dY, W))
    dX, dA, dB = oracle.lora_backward(dY, X, W, np.zeros((R, K)), B, 2.0)
    assert not dB.any()


def test_backward_dx_rows_matches_full():
    rng = np.random.default_rng(8)
    M, K, N, R = 30, 24, 20, 4
    X, W, dY = rng.standard_normal((M, K)), rng.standard_normal((N, K)), rng.standard_normal((M, N))
    A, B = rng.standard_normal((R, K)), rng.standard_normal((N, R))
    dX, _, _ = oracle.lora_backward(dY, X, W, A, B, 2.0)
    rows = [29, 0, 11]
    np.testing.assert_allclose(oracle.lora_backward_dx_rows(dY, W, A, B, 2.0, rows), dX[rows],
                               rtol=1e-13, atol=1e-13)


def test_backward_adapters_hand_worked_example():
    # the adapter gradients alone reproduce the hand-worked fixture's dA and dB exactly, with and
    # without the saved panel
    f = _fixture_lora()
    dA, dB = oracle.lora_backward_adapters(f["dY"], f["X"], f["A"], f["B"], f["s"])
    np.testing.assert_array_equal(dA, f["dA"])
    np.testing.assert_array_equal(dB, f["dB"])
    dA2, dB2 = oracle.lora_backward_adapters(f["dY"], f["X"], f["A"], f["B"], f["s"], XA=f["XA"])
    np.testing.assert_array_equal(dA2, f["dA"])
    np.testing.assert_array_equal(dB2, f["dB"])


@pytest.mark.parametrize("M,K,N,R", [(3, 5, 4, 2), (6, 4, 7, 3)])
def test_backward_adapters_central_differences(M, K, N, R):
    # L = <dY, Y> is linear in A and in B separately: unit-step central differences are exact
    rng = np.random.default_rng(40 + M)
    X, W = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    A, B = rng.standard_normal((R, K)), rng.standard_normal((N, R))
    dY, s = rng.standard_normal((M, N)), 1.25
    dA, dB = oracle.lora_backward_adapters(dY, X, A, B, s)
    for name, got in (("A", dA), ("B", dB)):
        want = np.zeros(got.shape)
        for idx in np.ndindex(*got.shape):
            p, m = {"A": A.copy(), "B": B.copy()}, {"A": A.copy(), "B": B.copy()}
            p[name][idx] += 1.0
            m[name][idx] -= 1.0
            want[idx] = (_loss(dY, X, W, p["A"], p["B"], s) - _loss(dY, X, W, m["A"], m["B"], s)) / 2.0
        np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-9)


def test_backward_adapters_invariants_and_full_backward():
    # <dA, A> = <dB, B> = s <dY, (X A^T) B^T>, and the same values as the full backward
    rng = np.random.default_rng(41)
    M, K, N, R, s = 64, 48, 40, 8, 2.0
    X, W = rng.standard_normal((M, K)), rng.standard_normal((N, K)) / np.sqrt(K)
    A, B = rng.uniform(-0.1, 0.1, (R, K)), rng.standard_normal((N, R)) * 0.14
    dY = rng.standard_normal((M, N))
    dA, dB = oracle.lora_backward_adapters(dY, X, A, B, s)
    Lr = s * np.sum(dY * np.matmul(np.matmul(X, A.T), B.T))
    assert abs(np.sum(dA * A) - Lr) <= 1e-10 * max(1.0, abs(Lr))
    assert abs(np.sum(dB * B) - Lr) <= 1e-10 * max(1.0, abs(Lr))
    _, dA2, dB2 = oracle.lora_backward(dY, X, W, A, B, s)
    np.testing.assert_array_equal(dA, dA2)
    np.testing.assert_array_equal(dB, dB2)
    # a planted mistake (dB from the scaled panel s X A^T) breaks the invariant
    bad = s * (dY.T @ (s * (X @ A.T)))
    assert abs(np.sum(bad * B) - Lr) > 1e-3 * abs(Lr)


# ---------------------------------------------------------------------------
# int4 format
# ---------------------------------------------------------------------------

def test_int4_hand_worked_group():
    f = _read_fixture("int4_format_example.txt")
    w = np.zeros((1, 64), dtype=np.float32)
    vals = [float(v) for v in f["values"]]
    w[0, : len(vals)] = vals
    q, s = oracle.quantize_int4(w)
    assert s.view(np.uint16)[0, 0] == int(f["scale_bits"][0], 16)
    codes = [int(v) for v in f["codes"]]
    np.testing.assert_array_equal(q[0, : len(codes)], codes)
    assert not q[0, len(codes):].any()
    packed = oracle.pack_int4(q)
    want = [int(b, 16) for b in f["bytes"]]
    np.testing.assert_array_equal(packed[0, : len(want)], want)
    assert not packed[0, len(want):].any()
    bits = oracle.dequant_int4_bits(packed, s)
    assert bits[0, 0] == int(f["dequant_k0_bf16"][0], 16)


def test_int4_pack_unpack_exhaustive():
    lo, hi = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8), indexing="ij")
    q = np.stack([lo.ravel(), hi.ravel()], axis=1).astype(np.int8).reshape(1, -1)
    p = oracle.pack_int4(q)
    assert sorted(p.ravel().tolist()) == list(range(256))
    np.testing.assert_array_equal(oracle.unpack_int4(p), q)


def test_int4_quantiser_properties():
    rng = np.random.default_rng(9)
    N, K = 64, 1024
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    q, s = oracle.quantize_int4(w)
    assert q.dtype == np.int8 and np.abs(q).max() <= 7
    wg = w.astype(np.float64).reshape(N, K // 64, 64)
    qg = q.reshape(N, K // 64, 64)
    sd = s.astype(np.float64)
    a = np.abs(wg).max(axis=2)
    # scale = fp16(absmax / 7), cross-checked with the struct module's IEEE half rounding
    want = np.array([[np.frombuffer(struct.pack("<e", v / 7.0), dtype=np.float16)[0] for v in row]
                     for row in a])
    np.testing.assert_array_equal(s.view(np.uint16), want.view(np.uint16))
    # the absmax element of every group maps to +-7
    arg = np.abs(wg).argmax(axis=2)
    top = np.take_along_axis(qg, arg[:, :, None], axis=2)[:, :, 0]
    np.testing.assert_array_equal(np.abs(top), 7)
    # nearest code: |w - q s| <= s / 2 (no clamping occurs below absmax * 7.5/7)
    err = np.abs(wg - qg * sd[:, :, None])
    assert np.all(err <= sd[:, :, None] / 2 * (1 + 1e-12))


def test_int4_exact_ties_go_to_even():
    s16 = np.float16(0.1)
    s = float(s16)
    ks = np.array([0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5, -0.5, -1.5, -6.5])
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 0] = 7 * s  # pins the scale to s exactly (7 s / 7 = s)
    w[0, 1: 1 + len(ks)] = ks * s  # exact in fp32 (<= 15 significant bits)
    assert np.all(w[0, 1: 1 + len(ks)].astype(np.float64) == ks * s)
    q, sc = oracle.quantize_int4(w)
    assert float(sc[0, 0]) == s
    np.testing.assert_array_equal(q[0, 1: 1 + len(ks)], [0, 2, 2, 4, 4, 6, 6, 0, -2, -6])


def test_int4_zero_and_underflow_groups():
    w = np.zeros((2, 128), dtype=np.float32)
    w[1, 64] = 1e-9  # absmax / 7 underflows to fp16 zero
    w[1, 65] = -5e-10
    q, s = oracle.quantize_int4(w)
    assert not s.astype(np.float64).any()
    assert not q.any()
    np.testing.assert_array_equal(oracle.dequant_int4_bits(oracle.pack_int4(q), s), 0)


def test_int4_dequant_enumeration_against_torch():
    """All 16 nibbles x sample scales: bf16(q s) via torch's float -> bf16 rounding."""
    rng = np.random.default_rng(11)
    scales = np.concatenate([rng.uniform(1e-4, 0.05, 60), [2.0 ** -24, 6.1e-5, 1.0, 65504.0 / 7]])
    s16 = scales.astype(np.float16)
    nib = np.arange(16, dtype=np.uint8)
    packed = np.repeat((nib | (nib << 4))[None, :], len(s16), axis=0)  # K = 32 per row
    packed = np.concatenate([packed, packed], axis=1)  # K = 64: one group per row
    bits = oracle.dequant_int4_bits(packed, s16[:, None])
    q = np.where(nib >= 8, nib.astype(np.int64) - 16, nib.astype(np.int64))
    exact = q[None, :] * s16.astype(np.float64)[:, None]  # exact products
    want = torch.tensor(exact).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits[:, 0:32:2], want)
    np.testing.assert_array_equal(bits[:, 1:32:2], want)


def test_qlora_forward_uses_dequantised_weight():
    """QLoRA = the LoRA formula with W := dequant(quant(W)); brute force on a tiny case."""
    rng = np.random.default_rng(12)
    M, K, N, R = 3, 64, 5, 2
    w = (rng.standard_normal((N, K)) / 8).astype(np.float32)
    q, s = oracle.quantize_int4(w)
    Wt = oracle.dequant_int4(oracle.pack_int4(q), s)
    # dequantised values are exactly representable in bf16 and close to q * s
    np.testing.assert_allclose(Wt, q * s.astype(np.float64).repeat(64, axis=1), rtol=2 ** -8, atol=0)
    X = rng.standard_normal((M, K))
    A, B = rng.standard_normal((R, K)), rng.standard_normal((N, R))
    Y, _ = oracle.lora_forward(X, Wt, A, B, 2.0)
    Xf, Wf, Af, Bf = map(_frac_matrix, (X, Wt, A, B))
    for m in range(M):
        for n in range(N):
            ex = sum(Xf[m][k] * (Wf[n][k] + 2 * sum(Bf[n][i] * Af[i][k] for i in range(R)))
                     for k in range(K))
            assert abs(Y[m, n] - float(ex)) <= 1e-12 * max(1.0, abs(float(ex)))


# ---------------------------------------------------------------------------
# SwiGLU gate/up pair with LoRA (tutorial ch. 5 §5.6)
# ---------------------------------------------------------------------------

def test_silu_closed_forms():
    # sigmoid(0) = 1/2, sigmoid(x) + sigmoid(-x) = 1; silu(0) = 0, silu'(0) = 1/2;
    # silu(g) -> g and silu'(g) -> 1 for large g, silu(g) -> 0 for very negative g;
    # silu(ln 3) = ln(3) * 3/4 exactly in the reals (sigmoid(ln 3) = 3/4)
    x = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(oracle.sigmoid(x) + oracle.sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    assert oracle.sigmoid(0.0) == 0.5 and oracle.silu(0.0) == 0.0 and oracle.silu_grad(0.0) == 0.5
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12 and abs(oracle.silu_grad(40.0) - 1.0) < 1e-12
    assert oracle.silu(-800.0) == 0.0
    assert abs(oracle.silu(np.log(3.0)) - 0.75 * np.log(3.0)) < 1e-15
    # derivative of silu against a central difference of silu itself
    g = np.linspace(-8, 8, 33)
    h = 1e-5
    fd = (oracle.silu(g + h) - oracle.silu(g - h)) / (2 * h)
    np.testing.assert_allclose(oracle.silu_grad(g), fd, rtol=0, atol=1e-9)


def _swiglu_case(rng, M, K, N, R):
    X = rng.standard_normal((M, K))
    Wg, Wu = rng.standard_normal((N, K)) / np.sqrt(K), rng.standard_normal((N, K)) / np.sqrt(K)
    Ag, Au = rng.uniform(-0.3, 0.3, (R, K)), rng.uniform(-0.3, 0.3, (R, K))
    Bg, Bu = rng.standard_normal((N, R)) * 0.14, rng.standard_normal((N, R)) * 0.14
    dH = rng.standard_normal((M, N))
    return X, Wg, Wu, Ag, Au, Bg, Bu, dH


@pytest.mark.parametrize("M,K,N,R", [(5, 7, 6, 2), (9, 16, 12, 4)])
def test_swiglu_backward_central_differences(M, K, N, R):
    """L = <dH, H> is smooth: central differences agree with the hand-derived gradients to
    O(h^2) (here ~1e-9 relative)."""
    rng = np.random.default_rng(40 + M)
    X, Wg, Wu, Ag, Au, Bg, Bu, dH = _swiglu_case(rng, M, K, N, R)
    s = 2.0
    args = [X, Wg, Wu, Ag, Au, Bg, Bu]

    def loss(a):
        H, *_ = oracle.swiglu_lora_forward(*a, s)
        return np.sum(dH * H)

    grads = oracle.swiglu_lora_backward(dH, *args, s)
    h = 1e-5
    for gi, ai in zip(grads, (0, 3, 4, 5, 6)):  # dX, dAg, dAu, dBg, dBu
        fd = np.zeros_like(args[ai])
        for idx in np.ndindex(*args[ai].shape):
            p = [a.copy() for a in args]
            p[ai][idx] += h
            lp = loss(p)
            p[ai][idx] -= 2 * h
            fd[idx] = (lp - loss(p)) / (2 * h)
        np.testing.assert_allclose(gi, fd, rtol=1e-6, atol=1e-8)


def test_swiglu_against_torch_autograd_float64():
    rng = np.random.default_rng(47)
    M, K, N, R, s = 33, 40, 24, 6, 2.0
    X, Wg, Wu, Ag, Au, Bg, Bu, dH = _swiglu_case(rng, M, K, N, R)
    t = lambda v, g=False: torch.tensor(v, dtype=torch.float64, requires_grad=g)
    tX, tAg, tAu, tBg, tBu = t(X, True), t(Ag, True), t(Au, True), t(Bg, True), t(Bu, True)
    tWg, tWu = t(Wg), t(Wu)
    G = tX @ tWg.T + (tX @ tAg.T @ tBg.T) * s
    U = tX @ tWu.T + (tX @ tAu.T @ tBu.T) * s
    H = torch.nn.functional.silu(G) * U
    H.backward(t(dH))
    Ho, Go, Uo, _, _ = oracle.swiglu_lora_forward(X, Wg, Wu, Ag, Au, Bg, Bu, s)
    np.testing.assert_allclose(Ho, H.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Go, G.detach().numpy(), rtol=1e-12, atol=1e-12)
    got = oracle.swiglu_lora_backward(dH, X, Wg, Wu, Ag, Au, Bg, Bu, s)
    for g, ref in zip(got, (tX, tAg, tAu, tBg, tBu)):
        np.testing.assert_allclose(g, ref.grad.numpy(), rtol=1e-11, atol=1e-12)
    # the adapter-only form against the same autograd witness
    ad = oracle.swiglu_lora_backward_adapters(dH, X, Wg, Wu, Ag, Au, Bg, Bu, s)
    for g, ref in zip(ad, (tAg, tAu, tBg, tBu)):
        np.testing.assert_allclose(g, ref.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_swiglu_rows_matches_full():
    rng = np.random.default_rng(48)
    X, Wg, Wu, Ag, Au, Bg, Bu, _ = _swiglu_case(rng, 40, 24, 16, 4)
    rows = np.array([0, 7, 39, 13])
    H, G, U, _, _ = oracle.swiglu_lora_forward(X, Wg, Wu, Ag, Au, Bg, Bu, 2.0)
    Hr, Gr, Ur = oracle.swiglu_lora_rows(X, Wg, Wu, Ag, Au, Bg, Bu, 2.0, rows)
    np.testing.assert_array_equal(Hr, H[rows])
    np.testing.assert_array_equal(Gr, G[rows])
    np.testing.assert_array_equal(Ur, U[rows])


def test_swiglu_planted_mistake_fails_the_difference_pin():
    # dropping the (1 + g (1 - sigmoid)) factor of silu' (a plausible slip) is caught
    rng = np.random.default_rng(49)
    X, Wg, Wu, Ag, Au, Bg, Bu, dH = _swiglu_case(rng, 4, 6, 5, 2)
    s = 2.0
    G, _ = oracle.lora_forward(X, Wg, Ag, Bg, s)
    U, _ = oracle.lora_forward(X, Wu, Au, Bu, s)
    wrong = oracle.lora_backward(dH * U * oracle.sigmoid(G), X, Wg, Ag, Bg, s)[0] + \
        oracle.lora_backward(dH * oracle.silu(G), X, Wu, Au, Bu, s)[0]
    right = oracle.swiglu_lora_backward(dH, X, Wg, Wu, Ag, Au, Bg, Bu, s)[0]
    assert np.max(np.abs(wrong - right)) > 1e-3


def test_swiglu_dx_rows_matches_full():
    rng = np.random.default_rng(50)
    X, Wg, Wu, Ag, Au, Bg, Bu, dH = _swiglu_case(rng, 30, 24, 16, 4)
    rows = np.array([29, 0, 11])
    dX = oracle.swiglu_lora_backward(dH, X, Wg, Wu, Ag, Au, Bg, Bu, 2.0)[0]
    got = oracle.swiglu_lora_backward_dx_rows(dH, X, Wg, Wu, Ag, Au, Bg, Bu, 2.0, rows)
    np.testing.assert_allclose(got, dX[rows], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# RMSNorm (tutorial ch. 5 §5.4)
# ---------------------------------------------------------------------------


def _rmsnorm_fixture(case):
    f = _read_fixture("rmsnorm_worked_example.txt")
    get = lambda k: [float(Fraction(v)) for v in f[f"{case}.{k}"]]
    M, K = int(f[f"{case}.M"][0]), int(f[f"{case}.K"][0])
    mat = lambda k: np.array(get(k)).reshape(M, K)
    return dict(eps=get("eps")[0], g=np.array(get("g")), x=mat("x"), r=np.array(get("r")), y=mat("y"),
                dy=mat("dy"), dx=mat("dx"), dg=np.array(get("dg")))


@pytest.mark.parametrize("case", ["A", "B"])
def test_rmsnorm_hand_worked_examples(case):
    f = _rmsnorm_fixture(case)
    Y, r = oracle.rmsnorm_forward(f["x"], f["g"], f["eps"])
    np.testing.assert_allclose(r, f["r"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(Y, f["y"], rtol=1e-15, atol=0)
    dX, dg = oracle.rmsnorm_backward(f["dy"], f["x"], f["g"], f["eps"])
    np.testing.assert_allclose(dX, f["dx"], rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(dg, f["dg"], rtol=1e-15, atol=1e-16)


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(60)
    M, K = 7, 48
    X = rng.standard_normal((M, K))
    g = rng.uniform(0.5, 1.5, K)
    # eps = 0: the output does not change when a row is scaled by a positive number
    Y0, _ = oracle.rmsnorm_forward(X, g, 0.0)
    for a in (1e-3, 7.0, 1e5):
        np.testing.assert_allclose(oracle.rmsnorm_forward(a * X, g, 0.0)[0], Y0, rtol=1e-13, atol=0)
    # the RMS of Y / g over a row is sqrt(ms / (ms + eps)); r from the Euclidean norm
    eps = 0.3
    Y, r = oracle.rmsnorm_forward(X, g, eps)
    ms = np.linalg.norm(X, axis=1) ** 2 / K
    np.testing.assert_allclose(np.sqrt(np.mean((Y / g) ** 2, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)
    np.testing.assert_allclose(r, (ms + eps) ** -0.5, rtol=1e-14)
    # a constant row c gives c / sqrt(c^2 + eps) g
    c = -2.5
    Yc, _ = oracle.rmsnorm_forward(np.full((1, K), c), g, eps)
    np.testing.assert_allclose(Yc[0], c / np.sqrt(c * c + eps) * g, rtol=1e-14)


def _rmsnorm_case(rng, M, K):
    return (rng.standard_normal((M, K)), rng.uniform(0.5, 1.5, K), rng.standard_normal((M, K)))


def test_rmsnorm_backward_central_differences():
    """L = <dY, Y> is smooth in X and g: central differences agree with the hand-derived
    gradients to O(h^2)."""
    rng = np.random.default_rng(61)
    X, g, dY = _rmsnorm_case(rng, 5, 24)
    eps = 0.05
    dX, dg = oracle.rmsnorm_backward(dY, X, g, eps)
    L = lambda X_, g_: float(np.sum(dY * oracle.rmsnorm_forward(X_, g_, eps)[0]))
    h = 1e-5
    num = np.zeros_like(X)
    for idx in np.ndindex(*X.shape):
        E = np.zeros_like(X)
        E[idx] = h
        num[idx] = (L(X + E, g) - L(X - E, g)) / (2 * h)
    np.testing.assert_allclose(num, dX, rtol=1e-6, atol=1e-8)
    numg = np.array([(L(X, g + h * np.eye(len(g))[k]) - L(X, g - h * np.eye(len(g))[k])) / (2 * h)
                     for k in range(len(g))])
    np.testing.assert_allclose(numg, dg, rtol=1e-6, atol=1e-8)


def test_rmsnorm_against_torch_autograd_float64():
    rng = np.random.default_rng(62)
    X, g, dY = _rmsnorm_case(rng, 9, 40)
    eps = 1e-5
    tX = torch.tensor(X, requires_grad=True)
    tg = torch.tensor(g, requires_grad=True)
    tY = tX / torch.sqrt(torch.mean(tX * tX, dim=1, keepdim=True) + eps) * tg
    tY.backward(torch.tensor(dY))
    Y, _ = oracle.rmsnorm_forward(X, g, eps)
    dX, dg = oracle.rmsnorm_backward(dY, X, g, eps)
    np.testing.assert_allclose(Y, tY.detach().numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dX, tX.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_rmsnorm_backward_invariants():
    # <dX_m, X_m> = <dY_m, Y_m> eps r_m^2 per row (scaling a row changes Y only through eps);
    # <dg, g> = <dY, Y> (Y is linear in g)
    rng = np.random.default_rng(63)
    X, g, dY = _rmsnorm_case(rng, 6, 32)
    for eps in (0.0, 0.7):
        Y, r = oracle.rmsnorm_forward(X, g, eps)
        dX, dg = oracle.rmsnorm_backward(dY, X, g, eps)
        np.testing.assert_allclose(np.sum(dX * X, axis=1), np.sum(dY * Y, axis=1) * eps * r * r, rtol=1e-10,
                                   atol=1e-12)
        np.testing.assert_allclose(np.dot(dg, g), np.sum(dY * Y), rtol=1e-12)


def test_rmsnorm_planted_mistakes_fail_the_pins():
    rng = np.random.default_rng(64)
    X, g, dY = _rmsnorm_case(rng, 4, 16)
    eps = 0.0
    Y, r = oracle.rmsnorm_forward(X, g, eps)
    # backward without the mean term: dX = r g dY breaks <dX, X> = 0 at eps = 0
    wrong_dx = r[:, None] * g[None, :] * dY
    assert np.max(np.abs(np.sum(wrong_dx * X, axis=1))) > 1e-3
    # sum instead of mean of the squares breaks the RMS closed form
    wrong_r = 1.0 / np.sqrt(np.sum(X * X, axis=1) + eps)
    assert not np.allclose(np.sqrt(np.mean((X * wrong_r[:, None]) ** 2, axis=1)), 1.0, rtol=1e-3)
    np.testing.assert_allclose(np.sqrt(np.mean((Y / g) ** 2, axis=1)), 1.0, rtol=1e-13)


# ---------------------------------------------------------------------------
# MXFP4 weights
# ---------------------------------------------------------------------------


def _mx_fixture():
    f = _read_fixture("mxfp4_format_example.txt")
    return f


def test_mxfp4_code_table():
    f = _mx_fixture()
    np.testing.assert_array_equal(oracle.fp4_e2m1_value(np.arange(16)), [float(v) for v in f["values"]])
    # the sign of code 8 is kept: -0.0
    assert np.signbit(oracle.fp4_e2m1_value(8))


@pytest.mark.parametrize("blk", ["A", "B", "C"])
def test_mxfp4_hand_worked_blocks(blk):
    f = _mx_fixture()
    vals = [float(Fraction(v)) for v in f[f"{blk}.w"]]
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, :len(vals)] = vals
    codes, E = oracle.quantize_mxfp4(w)
    assert int(E[0, 0]) == int(f[f"{blk}.E"][0])
    np.testing.assert_array_equal(codes[0, :len(vals)], [int(c) for c in f[f"{blk}.codes"]])
    assert not codes[0, len(vals):].any()


def test_mxfp4_packing():
    f = _mx_fixture()
    line = f["pack"]
    i = line.index("->")
    codes = np.array([[int(c) for c in line[:i]]], dtype=np.uint8)
    want = [int(b, 16) for b in line[i + 1:]]
    np.testing.assert_array_equal(oracle.pack_fp4(codes)[0], want)
    np.testing.assert_array_equal(oracle.unpack_fp4(oracle.pack_fp4(codes)), codes)


def test_mxfp4_round_trip_and_error_bound():
    rng = np.random.default_rng(70)
    N, K = 16, 256
    w = (rng.standard_normal((N, K)) * np.exp(rng.uniform(-8, 8, size=(N, 1)))).astype(np.float32)
    codes, E = oracle.quantize_mxfp4(w)
    wt = oracle.dequant_mxfp4(oracle.pack_fp4(codes), E)
    se = np.repeat(E.astype(np.int64) - 127, 32, axis=1)
    x = np.abs(w.astype(np.float64)) / np.exp2(se)
    # error within half the grid spacing at x (0.25 below 2, 0.5 below 4, 1 below 6), or the
    # saturation gap past 6; the block's largest element is never below 4 after scaling
    half = np.where(x <= 2, 0.25, np.where(x <= 4, 0.5, 1.0))
    err = np.abs(w - wt) / np.exp2(se)
    assert np.all(err <= np.maximum(half, x - 6) + 1e-12)
    amax = np.abs(w).reshape(N, K // 32, 32).max(axis=2) / np.exp2(E.astype(np.int64) - 127)
    assert np.all((amax >= 4) & (amax < 8))
    # values already on the scaled grid come back exactly
    g = oracle.fp4_e2m1_value(codes) * np.exp2(se)
    c2, E2 = oracle.quantize_mxfp4(g.astype(np.float32))
    np.testing.assert_array_equal(oracle.dequant_mxfp4(oracle.pack_fp4(c2), E2), oracle.fp4_e2m1_value(codes) * np.exp2(se))


def test_mxfp4_exponent_clamps_and_zero_blocks():
    w = np.zeros((1, 96), dtype=np.float32)
    w[0, 32] = 2.0 ** -130  # tiny block: exponent clamped to -125 -> rounds to 0
    w[0, 64] = 3.0e38        # huge block: floor(log2) = 127, se = 125
    codes, E = oracle.quantize_mxfp4(w)
    np.testing.assert_array_equal(E[0], [127, 2, 252])
    assert codes[0, 32] == 0 and codes[0, 64] == 7 and not codes[0, :32].any()


def test_mxfp4_planted_mistakes_fail_the_fixture():
    # ties rounded away from zero would turn 2.5 into 3 and 0.25 into 0.5
    grid = oracle.fp4_e2m1_value(np.arange(8))
    x = np.array([5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25])
    away = np.array([np.argmin(np.abs(v - grid) - 1e-9 * grid) for v in x])
    assert list(away) != [6, 6, 4, 4, 2, 2, 0]
    # swapped nibbles would pack 6, 14 as 0x6E
    assert int(oracle.pack_fp4(np.array([[6, 14]], dtype=np.uint8))[0, 0]) == 0xE6


# ---------------------------------------------------------------------------
# Chunked cross-entropy over an LM head (tutorial ch. 5 §5.7)
# ---------------------------------------------------------------------------


def _term(t):
    import math
    if "*ln(" in t:
        a, b = t.split("*ln(")
        return float(Fraction(a)) * math.log(float(Fraction(b.rstrip(")"))))
    return float(Fraction(t))


def test_cross_entropy_hand_worked_example():
    f = _read_fixture("cross_entropy_worked_example.txt")
    vec = lambda k: np.array([_term(t) for t in f[k]])
    W, X = vec("W").reshape(3, 2), vec("X").reshape(2, 2)
    labels = np.array([int(v) for v in f["labels"]])
    loss, lse = oracle.cross_entropy_rows(X, W, labels)
    np.testing.assert_allclose(loss, vec("loss"), rtol=1e-14)
    np.testing.assert_allclose(lse, vec("lse"), rtol=1e-14)
    dX, dl = oracle.cross_entropy_grad(X, W, labels, 1.0)
    np.testing.assert_allclose(dl, vec("dlogits").reshape(2, 3), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dX, vec("dX").reshape(2, 2), rtol=1e-14, atol=1e-15)


def test_cross_entropy_closed_forms_and_invariants():
    rng = np.random.default_rng(90)
    M, K, V = 9, 16, 50
    X, W = rng.standard_normal((M, K)), rng.standard_normal((V, K))
    labels = rng.integers(0, V, M)
    # X = 0: uniform softmax, loss = ln V, dX = mean of W's rows minus the label's row
    loss0, _ = oracle.cross_entropy_rows(np.zeros((M, K)), W, labels)
    np.testing.assert_allclose(loss0, np.log(V), rtol=1e-15)
    dX0, _ = oracle.cross_entropy_grad(np.zeros((M, K)), W, labels, 1.0)
    np.testing.assert_allclose(dX0, W.mean(axis=0)[None, :] - W[labels], rtol=1e-12, atol=1e-14)
    # a constant added to every logit (a constant feature in X with a constant column in W)
    # changes neither the loss nor the gradient, and the gradient's component on that feature is
    # sum_v dlogits_v * c = 0
    Xc, Wc = np.hstack([X, np.full((M, 1), 1.0)]), np.hstack([W, np.full((V, 1), 7.5)])
    np.testing.assert_allclose(oracle.cross_entropy_rows(Xc, Wc, labels)[0], oracle.cross_entropy_rows(X, W, labels)[0],
                               rtol=1e-12)
    dXc, dl = oracle.cross_entropy_grad(Xc, Wc, labels, 1.0)
    np.testing.assert_allclose(dXc[:, :K], oracle.cross_entropy_grad(X, W, labels, 1.0)[0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dXc[:, K], 0.0, atol=1e-12)
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-13)
    # huge logits (1e4 apart) stay finite: the log-sum-exp is taken around the maximum
    Xb = X * 1e3
    assert np.all(np.isfinite(oracle.cross_entropy_rows(Xb, W, labels)[0]))


def test_cross_entropy_central_differences_and_torch():
    rng = np.random.default_rng(91)
    M, K, V = 5, 8, 13
    X, W = rng.standard_normal((M, K)), rng.standard_normal((V, K))
    labels = rng.integers(0, V, M)
    g = 0.37
    L = lambda X_: g * float(np.sum(oracle.cross_entropy_rows(X_, W, labels)[0]))
    dX, _ = oracle.cross_entropy_grad(X, W, labels, g)
    h = 1e-5
    num = np.zeros_like(X)
    for idx in np.ndindex(*X.shape):
        E = np.zeros_like(X)
        E[idx] = h
        num[idx] = (L(X + E) - L(X - E)) / (2 * h)
    np.testing.assert_allclose(num, dX, rtol=1e-6, atol=1e-9)
    tX = torch.tensor(X, requires_grad=True)
    tl = torch.nn.functional.cross_entropy(tX @ torch.tensor(W).T, torch.tensor(labels), reduction="none")
    (g * tl.sum()).backward()
    np.testing.assert_allclose(oracle.cross_entropy_rows(X, W, labels)[0], tl.detach().numpy(), rtol=1e-12)
    np.testing.assert_allclose(dX, tX.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_cross_entropy_chunked_equals_whole_batch():
    # the page's chunked procedure gives the whole batch's mean loss and gradient
    rng = np.random.default_rng(92)
    M, K, V = 700, 12, 40
    X, W = rng.standard_normal((M, K)), rng.standard_normal((V, K))
    labels = rng.integers(0, V, M)
    mean, dX = oracle.cross_entropy_chunked(X, W, labels, chunk=256)
    np.testing.assert_allclose(mean, np.mean(oracle.cross_entropy_rows(X, W, labels)[0]), rtol=1e-13)
    np.testing.assert_allclose(dX, oracle.cross_entropy_grad(X, W, labels, 1.0 / M)[0], rtol=1e-12, atol=1e-15)


def test_cross_entropy_planted_mistake_fails():
    # forgetting the onehot term leaves gradient rows that do not sum to zero
    rng = np.random.default_rng(93)
    X, W = rng.standard_normal((4, 6)), rng.standard_normal((10, 6))
    logits = X @ W.T
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.max(np.abs(p.sum(axis=1))) > 0.5  # the invariant pinned above would catch it


# ---------------------------------------------------------------------------
# RoPE (tutorial ch. 5 §5.5)
# ---------------------------------------------------------------------------


def _trig_expr(t):
    import math
    import re
    total = 0.0
    for sign, coef, fn, arg in re.findall(r"([+-]?)([0-9.]+)\*(cos|sin)\(([0-9.]+)\)", t):
        v = float(coef) * (math.cos if fn == "cos" else math.sin)(float(arg))
        total += -v if sign == "-" else v
    return total if "(" in t else float(t)


def test_rope_hand_worked_example():
    f = _read_fixture("rope_worked_example.txt")
    x = np.array([float(v) for v in f["x"]]).reshape(2, 1, 6)
    pos = [int(v) for v in f["positions"]]
    want = np.array([_trig_expr(t) for t in f["out"]]).reshape(2, 1, 6)
    np.testing.assert_allclose(oracle.rope_apply(x, pos, 4, 10000.0), want, rtol=1e-14, atol=1e-15)


def test_rope_properties():
    rng = np.random.default_rng(95)
    M, H, D, rot, base = 9, 3, 16, 12, 500000.0
    pos = rng.integers(0, 8192, M)
    x = rng.standard_normal((M, H, D))
    y = oracle.rope_apply(x, pos, rot, base)
    # the inverse rotation undoes it; position 0 is the identity; the pass-through part is untouched
    np.testing.assert_allclose(oracle.rope_apply(y, pos, rot, base, inverse=True), x, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(oracle.rope_apply(x, np.zeros(M, int), rot, base), x)
    np.testing.assert_array_equal(y[..., rot:], x[..., rot:])
    # each pair keeps its length
    h = rot // 2
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:rot] ** 2, x[..., :h] ** 2 + x[..., h:rot] ** 2, rtol=1e-12)
    # the defining property: <R(m) q, R(n) k> depends only on m - n
    q, k = rng.standard_normal((1, 1, D)), rng.standard_normal((1, 1, D))
    dot = lambda m, n: float(np.sum(oracle.rope_apply(q, [m], rot, base) * oracle.rope_apply(k, [n], rot, base)))
    for m, n in ((5, 2), (105, 102), (3000, 2997)):
        np.testing.assert_allclose(dot(m, n), dot(3, 0), rtol=1e-9)
    # the gradient of L = <dY, rope(x)> is the inverse rotation of dY
    dY = rng.standard_normal((M, H, D))
    L = lambda x_: float(np.sum(dY * oracle.rope_apply(x_, pos, rot, base)))
    E = np.zeros_like(x)
    E[2, 1, 3] = 1e-6
    np.testing.assert_allclose((L(x + E) - L(x - E)) / 2e-6, oracle.rope_apply(dY, pos, rot, base, inverse=True)[2, 1, 3],
                               rtol=1e-7)


def test_rope_rotation_matrix_form_agrees():
    # §5.5's formula: each coordinate pair multiplied by the 2 x 2 rotation [[cos, -sin], [sin, cos]].
    # Written here as one explicit D x D matrix per token, acting on the half-split pairs
    # (j, j + rot/2) and the identity on the pass-through coordinates, applied by a matrix product
    rng = np.random.default_rng(96)
    M, H, D, rot, base = 5, 2, 10, 8, 10000.0
    pos = rng.integers(0, 100, M)
    x = rng.standard_normal((M, H, D))
    th = oracle.rope_angles(pos, rot, base)
    h = rot // 2
    want = np.empty_like(x)
    for t in range(M):
        Rm = np.eye(D)
        for j in range(h):
            c, s_ = np.cos(th[t, j]), np.sin(th[t, j])
            Rm[j, j], Rm[j, j + h] = c, -s_
            Rm[j + h, j], Rm[j + h, j + h] = s_, c
        want[t] = x[t] @ Rm.T
    np.testing.assert_allclose(oracle.rope_apply(x, pos, rot, base), want, rtol=1e-13, atol=1e-14)
    # a planted mistake (pairs (2i, 2i+1) instead of the half split) disagrees with it
    wrong = x.copy()
    wrong[..., 0:rot:2] = x[..., 0:rot:2] * np.cos(th)[:, None, :] - x[..., 1:rot:2] * np.sin(th)[:, None, :]
    wrong[..., 1:rot:2] = x[..., 1:rot:2] * np.cos(th)[:, None, :] + x[..., 0:rot:2] * np.sin(th)[:, None, :]
    assert not np.allclose(wrong, want)
