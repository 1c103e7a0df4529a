"""GPU parity of RoPE against the float64 oracle (through the C ABI): Q and K heads at several
head sizes, partial rotary dimensions and bases, positions of packed sequences, the inverse
(backward) rotation, the Llama-3-8B attention shape in full, the pass-through coordinates bit for
bit, the autograd wrapper and the empty batch."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import assert_close, bits_to_dev, host
from qlora_fine_tuning_amd.workloads import _round

pytestmark = pytest.mark.gpu


def _packed_positions(M, rng, max_len=2048):
    pos, t = [], 0
    while t < M:
        n = int(rng.integers(1, max_len + 1))
        pos.extend(range(min(n, M - t)))
        t += n
    return np.array(pos[:M], dtype=np.int32)


def _case(M, H, Hk, D, seed, max_len=2048):
    rng = np.random.default_rng(seed)
    q = _round(rng.standard_normal((M, H, D)), "bf16")
    k = _round(rng.standard_normal((M, Hk, D)), "bf16")
    return q, k, _packed_positions(M, rng, max_len)


@pytest.mark.parametrize("M,H,Hk,D,rot,base,inverse", [
    (300, 4, 2, 128, 128, 10000.0, False), (65, 3, 1, 64, 32, 500000.0, False), (1, 1, 1, 16, 16, 10000.0, True),
    (257, 5, 0, 96, 48, 10000.0, True), (130, 8, 8, 256, 128, 1000000.0, False)])
def test_rope_shapes(gpu_lib, M, H, Hk, D, rot, base, inverse):
    print(f"case rope M={M} H={H} Hk={Hk} D={D} rot={rot} base={base} inverse={inverse}", flush=True)
    q, k, pos = _case(M, H, Hk, D, seed=M + D)
    Q, K = bits_to_dev(q).view(M, H, D), bits_to_dev(k).view(M, Hk, D)
    gpu_lib.lora_rope(Q, K if Hk else None, torch.from_numpy(pos).cuda(), base, rot=rot, inverse=inverse)
    torch.cuda.synchronize()
    for name, got, x in (("Q", Q, q), ("K", K, k)):
        if x.shape[1] == 0:
            continue
        ref = oracle.rope_apply(oracle.bf16_bits_to_f64(x), pos, rot, base, inverse=inverse)
        assert_close(name, host(got), ref)
        # the pass-through coordinates keep their bits
        assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16)[..., rot:], x[..., rot:])


def test_rope_llama3_attention_shape_in_full(gpu_lib):
    # 8192 tokens of packed sequences, 32 query and 8 key heads of 128, base 500000, every element
    M, H, Hk, D = 8192, 32, 8, 128
    print(f"case rope full M={M} H={H} Hk={Hk} D={D}", flush=True)
    q, k, pos = _case(M, H, Hk, D, seed=8, max_len=4096)
    Q, K = bits_to_dev(q).view(M, H, D), bits_to_dev(k).view(M, Hk, D)
    gpu_lib.lora_rope(Q, K, torch.from_numpy(pos).cuda(), 500000.0)
    torch.cuda.synchronize()
    assert_close("Q", host(Q), oracle.rope_apply(oracle.bf16_bits_to_f64(q), pos, D, 500000.0))
    assert_close("K", host(K), oracle.rope_apply(oracle.bf16_bits_to_f64(k), pos, D, 500000.0))


def test_rope_autograd_and_empty(gpu_lib):
    print("case rope autograd / empty", flush=True)
    M, H, Hk, D = 100, 4, 2, 64
    q, k, pos = _case(M, H, Hk, D, seed=3)
    Q = bits_to_dev(q).view(M, H, D).requires_grad_(True)
    K = bits_to_dev(k).view(M, Hk, D).requires_grad_(True)
    P = torch.from_numpy(pos).cuda()
    Qr, Kr = gpu_lib.RoPEFunction.apply(Q, K, P, 10000.0)
    gq, gk = torch.randn_like(Qr), torch.randn_like(Kr)
    (Qr.float() * gq.float()).sum().add((Kr.float() * gk.float()).sum()).backward()
    torch.cuda.synchronize()
    # the inputs were not modified; the gradients are the inverse rotations of the upstream ones
    assert torch.equal(Q.detach(), bits_to_dev(q).view(M, H, D))
    refq = oracle.rope_apply(host(gq), pos, D, 10000.0, inverse=True)
    assert_close("dQ", host(Q.grad), refq)
    assert_close("dK", host(K.grad), oracle.rope_apply(host(gk), pos, D, 10000.0, inverse=True))
    E = torch.empty((0, H, D), dtype=torch.bfloat16, device="cuda")
    gpu_lib.lora_rope(E, None, torch.empty(0, dtype=torch.int32, device="cuda"), 10000.0)
