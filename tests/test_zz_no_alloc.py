"""The decode entry point that allocates nothing (static scratch) against qlora_fwd / mxfp4_decode_fwd
with a workspace: bitwise equal outputs on two calls in a row, the second with fewer tokens."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import assert_close, host, to_dev, values
from qlora_fine_tuning_amd.workloads import workload_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["decode_up", "decode_down"])
@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_decode_noalloc_matches_workspace_path(gpu_lib, name, fmt):
    print(f"case noalloc {fmt} {name}", flush=True)
    lora = gpu_lib
    inp = workload_inputs(name, M=8)
    N, K, R = inp.N, inp.K, inp.R
    W32 = torch.from_numpy(inp.W).cuda()
    Wq, Ws = lora.qlora_quantize(W32) if fmt == "int4" else lora.mxfp4_quantize(W32)
    del W32
    A, B, Xall = to_dev(inp, "A"), to_dev(inp, "B"), to_dev(inp, "X")
    for M in (8, 3):  # two calls in a row, the second with a smaller input
        X = Xall[:M].contiguous()
        need = lora.qlora_fwd_workspace_bytes(M, N, K, R)
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        if fmt == "int4":
            Yr, XAr = lora.qlora_fwd(X, Wq, Ws, A, B, inp.scale, ws=ws)
        else:
            Yr, XAr = lora.mxfp4_decode_fwd(X, Wq, Ws, A, B, inp.scale, ws=ws)
        Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        XA = torch.full((M, R), float("nan"), dtype=torch.float32, device="cuda")
        lora.qlora_decode_fwd_noalloc(X, Wq, Ws, A, B, inp.scale, Y=Y, XA=XA)
        torch.cuda.synchronize()
        assert torch.equal(Y, Yr), f"Y differs at M={M}"
        assert torch.equal(XA, XAr), f"XA differs at M={M}"
        if M == 3:  # and against the oracle on the dequantised weight
            if fmt == "int4":
                q, s = oracle.quantize_int4(inp.W)
                wt = oracle.dequant_int4(oracle.pack_int4(q), s)
            else:
                c, e = oracle.quantize_mxfp4(inp.W)
                wt = oracle.dequant_mxfp4(oracle.pack_fp4(c), e)
            x, a, b = values(inp, "X")[:M], values(inp, "A"), values(inp, "B")
            Yo, XAo = oracle.lora_forward(x, wt, a, b, inp.scale)
            assert_close("Y", host(Y), Yo)
            assert_close("XA", host(XA), XAo)
