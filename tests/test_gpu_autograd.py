"""The torch.autograd wrappers of the layer (the forward saves X A^T for the backward, as the
LoRA path is packaged as a custom autograd function): gradients through autograd equal the
direct C ABI calls bit for bit, and the outputs stay within tolerance of the float64 oracle."""
import pytest
import torch

import oracle
from parity_util import assert_close, host, to_dev, values
from qlora_fine_tuning_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu


def _grad_leaves(*ts):
    return [t.detach().clone().requires_grad_(True) for t in ts]


@pytest.mark.parametrize("M,N,K,R", [(300, 512, 320, 16), (65, 256, 1024, 8)])
def test_lora_autograd_matches_direct_calls(gpu_lib, M, N, K, R):
    print(f"case lora autograd M={M} N={N} K={K} R={R}", flush=True)
    inp = make_inputs(M, N, K, R, seed=900 + M, dtype="bf16")
    X, W, A, B, dY = (to_dev(inp, n) for n in ("X", "W", "A", "B", "dY"))
    Xg, Ag, Bg = _grad_leaves(X, A, B)
    Y = gpu_lib.LoRALinearFunction.apply(Xg, W, Ag, Bg, inp.scale)
    Y.backward(dY)
    Yd, XA = gpu_lib.lora_fwd(X, W, A, B, inp.scale)
    dX, dA, dB = gpu_lib.lora_bwd(dY, X, W, A, B, XA, inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yd)
    assert torch.equal(Xg.grad, dX)
    assert torch.equal(Ag.grad, dA.to(A.dtype)) and torch.equal(Bg.grad, dB.to(B.dtype))
    x, w, a, b, dy = (values(inp, n) for n in ("X", "W", "A", "B", "dY"))
    dXr, dAr, dBr = oracle.lora_backward(dy, x, w, a, b, inp.scale)
    assert_close("dX", host(Xg.grad), dXr)
    assert_close("dA", host(Ag.grad), dAr)
    assert_close("dB", host(Bg.grad), dBr)


# 200 tokens: the tiled int4 kernels; 4 tokens with K a multiple of 1024: the decode forward
@pytest.mark.parametrize("M,N,K,R", [(200, 512, 1024, 16), (4, 320, 2048, 16)])
def test_qlora_autograd_matches_direct_calls(gpu_lib, M, N, K, R):
    print(f"case qlora autograd M={M} N={N} K={K} R={R}", flush=True)
    inp = make_inputs(M, N, K, R, seed=950 + M, dtype="bf16", int4=True)
    Wq, Ws = gpu_lib.qlora_quantize(torch.from_numpy(inp.W).cuda())
    X, A, B, dY = (to_dev(inp, n) for n in ("X", "A", "B", "dY"))
    Xg, Ag, Bg = _grad_leaves(X, A, B)
    Y = gpu_lib.QLoRALinearFunction.apply(Xg, Wq, Ws, Ag, Bg, inp.scale)
    Y.backward(dY)
    Yd, XA = gpu_lib.qlora_fwd(X, Wq, Ws, A, B, inp.scale)
    dX, dA, dB = gpu_lib.qlora_bwd(dY, X, Wq, Ws, A, B, XA, inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yd)
    assert torch.equal(Xg.grad, dX)
    assert torch.equal(Ag.grad, dA.to(A.dtype)) and torch.equal(Bg.grad, dB.to(B.dtype))
    assert Wq.grad is None and Ws.grad is None
    # the oracle's own quantisation of the same fp32 weight
    q, sc = oracle.quantize_int4(inp.W)
    wd = oracle.dequant_int4(oracle.pack_int4(q), sc)
    x, a, b, dy = (values(inp, n) for n in ("X", "A", "B", "dY"))
    Yr, _ = oracle.lora_forward(x, wd, a, b, inp.scale)
    dXr, dAr, dBr = oracle.lora_backward(dy, x, wd, a, b, inp.scale)
    assert_close("Y", host(Y), Yr)
    assert_close("dX", host(Xg.grad), dXr)
    assert_close("dA", host(Ag.grad), dAr)
    assert_close("dB", host(Bg.grad), dBr)
