"""GPU parity of the chunked cross-entropy over an LM head against the float64 oracle (through the
C ABI): per-token losses, the scaled total and dX at shapes with ragged chunks and a partial last
column tile, peaky logits, the pages' two LM heads on sampled rows (at the default chunk, at the
pages' 256-token chunk, and at an 8192-token chunk whose fp32 logits pass 4 GiB), an out-of-range
label, determinism, the empty batch, and the autograd wrapper with an upstream gradient."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import assert_close, bits_to_dev, host
from qlora_fine_tuning_amd.workloads import make_ce_inputs

pytestmark = pytest.mark.gpu


def _dev(inp):
    return bits_to_dev(inp.X), bits_to_dev(inp.W), torch.from_numpy(inp.labels).cuda()


def _vals(inp):
    return oracle.bf16_bits_to_f64(inp.X), oracle.bf16_bits_to_f64(inp.W), inp.labels.astype(np.int64)


@pytest.mark.parametrize("M,K,V,chunk,std", [(300, 256, 1024, 128, 1.0), (65, 512, 320, 0, 1.0), (1, 128, 64, 0, 1.0),
                                             (513, 384, 2112, 200, 6.0)])
def test_ce_shapes(gpu_lib, M, K, V, chunk, std):
    print(f"case ce M={M} K={K} V={V} chunk={chunk} std={std}", flush=True)
    inp = make_ce_inputs(M, K, V, seed=40 + M, logit_std=std)
    X, W, lab = _dev(inp)
    loss_total, loss, dX = gpu_lib.lora_ce(X, W, lab, chunk=chunk)
    torch.cuda.synchronize()
    x, w, labels = _vals(inp)
    lr, _ = oracle.cross_entropy_rows(x, w, labels)
    dXr, _ = oracle.cross_entropy_grad(x, w, labels, 1.0 / M)
    assert_close("loss", loss.cpu().numpy().astype(np.float64), lr)
    assert abs(float(loss_total[0]) - lr.mean()) <= 1e-5 * abs(lr.mean()) + 1e-6
    assert_close("dX", host(dX), dXr)
    # the loss alone (no gradient pass) gives the same bits
    _, loss2, dX2 = gpu_lib.lora_ce(X, W, lab, chunk=chunk, grad=False)
    torch.cuda.synchronize()
    assert dX2 is None and torch.equal(loss, loss2)


@pytest.mark.parametrize("V,K,chunk", [(128000, 4096, 0), (152064, 5120, 0), (128000, 4096, 256)])
def test_ce_lm_heads_sampled(gpu_lib, V, K, chunk):
    # the pages' vocabularies: 128000 (the chunked cross-entropy section) over 4096 hidden features,
    # and 152064 (the architecture table of the Qwen 27B inference post, section three) over 5120;
    # 2048 tokens at the default chunk (1024 and 768 tokens: the 768 one leaves a 512-token tail)
    # and at the section's 256-token chunk (the input gradient then splits V into 16 ranges)
    M = 2048
    C = chunk or gpu_lib.lora_ce_default_chunk(V)
    print(f"case ce M={M} K={K} V={V} chunk={C} (sampled rows)", flush=True)
    inp = make_ce_inputs(M, K, V, seed=5 + V % 7, logit_std=3.0)
    X, W, lab = _dev(inp)
    loss_total, loss, dX = gpu_lib.lora_ce(X, W, lab, chunk=chunk)
    torch.cuda.synchronize()
    edges = {0, 1, C - 1, C, C + 1, 2 * C - 1, 2 * C, M - 1} & set(range(M))
    rows = np.array(sorted(edges | set(np.random.default_rng(5).integers(0, M, 12))))
    x, w, labels = _vals(inp)
    lr, _ = oracle.cross_entropy_rows(x[rows], w, labels[rows])
    dXr, _ = oracle.cross_entropy_grad(x[rows], w, labels[rows], 1.0 / M)
    idx = torch.from_numpy(rows).cuda()
    assert_close("loss", loss[idx].cpu().numpy().astype(np.float64), lr)
    assert_close("dX", host(dX[idx]), dXr)
    assert torch.isfinite(loss).all() and torch.isfinite(dX.float()).all()
    # the total is the fixed-order sum of the per-token losses times 1/M
    l64 = loss.double().cpu().numpy()
    assert abs(float(loss_total[0]) - l64.mean()) <= 1e-5 * abs(l64.mean())


def test_ce_large_chunk_logits_past_4gib(gpu_lib):
    # 8200 tokens at the 152064-word head over 5120 features in 8192-token chunks: the first
    # chunk's fp32 logits (4.98 GB as two 16-bit planes) pass 2^32 bytes of workspace, then an
    # 8-token tail chunk
    M, K, V = 8200, 5120, 152064
    print(f"case ce M={M} K={K} V={V} chunk 8192 (sampled rows)", flush=True)
    inp = make_ce_inputs(M, K, V, seed=17, logit_std=3.0)
    X, W, lab = _dev(inp)
    loss_total, loss, dX = gpu_lib.lora_ce(X, W, lab, chunk=8192)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 7060, 7061, 7062, 7063, 8191, 8192, 8199} | set(np.random.default_rng(6).integers(0, M, 8))))
    x, w, labels = _vals(inp)
    lr, _ = oracle.cross_entropy_rows(x[rows], w, labels[rows])
    dXr, _ = oracle.cross_entropy_grad(x[rows], w, labels[rows], 1.0 / M)
    idx = torch.from_numpy(rows).cuda()
    assert_close("loss", loss[idx].cpu().numpy().astype(np.float64), lr)
    assert_close("dX", host(dX[idx]), dXr)
    assert torch.isfinite(loss).all() and torch.isfinite(dX.float()).all()


def test_ce_out_of_range_label_gives_nan(gpu_lib):
    print("case ce label out of range", flush=True)
    inp = make_ce_inputs(40, 128, 256, seed=3)
    inp.labels[7] = 256
    X, W, lab = _dev(inp)
    _, loss, _ = gpu_lib.lora_ce(X, W, lab, grad=False)
    torch.cuda.synchronize()
    l = loss.cpu().numpy()
    assert np.isnan(l[7]) and np.isfinite(np.delete(l, 7)).all()


def test_ce_determinism_empty_batch_and_autograd(gpu_lib):
    print("case ce determinism / empty / autograd", flush=True)
    inp = make_ce_inputs(200, 256, 640, seed=4)
    X, W, lab = _dev(inp)
    a = gpu_lib.lora_ce(X, W, lab, chunk=64)
    b = gpu_lib.lora_ce(X, W, lab, chunk=64)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    s0, l0, d0 = gpu_lib.lora_ce(X[:0], W, lab[:0])
    torch.cuda.synchronize()
    assert float(s0[0]) == 0.0 and l0.numel() == 0 and d0.shape == (0, 256)
    Xl = X.detach().clone().requires_grad_(True)
    mean = gpu_lib.LMHeadCrossEntropyFunction.apply(Xl, W, lab, 64)
    mean.backward()
    torch.cuda.synchronize()
    assert torch.equal(mean, a[0][0]) and torch.equal(Xl.grad, a[2])
    # an upstream gradient: the scaled objective's gradient, scaled on the device
    x, w, labels = _vals(inp)
    dXr, _ = oracle.cross_entropy_grad(x, w, labels, 1.0 / 200)
    Xl.grad = None
    mean = gpu_lib.LMHeadCrossEntropyFunction.apply(Xl, W, lab, 64)
    (mean * 2.5).backward()
    torch.cuda.synchronize()
    assert_close("dX x 2.5", host(Xl.grad), 2.5 * dXr)
    # the scaling entry point alone: bf16(dX g) for each value, in place too
    g = torch.tensor([-0.375], dtype=torch.float32, device="cuda")
    out = gpu_lib.lora_ce_scale_grad(a[2], g)
    ref = (a[2].double() * -0.375).cpu().numpy()
    got = out.double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8)
    same = a[2].clone()
    gpu_lib.lora_ce_scale_grad(same, g, out=same)
    torch.cuda.synchronize()
    assert torch.equal(same, out)
