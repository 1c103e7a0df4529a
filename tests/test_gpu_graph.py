"""A LoRA training step (forward + backward through the C ABI) recorded into a HIP graph and
replayed: every replay, with unrelated eager work and synchronisations between replays, must give
the eager step's outputs bit for bit.  The kernels allocate nothing and record no memset nodes
(counters and partials are cleared by kernels), and every reduction runs in a fixed order."""
import pytest
import torch

from parity_util import bits_to_dev
from qlora_fine_tuning_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu


def test_training_step_graph_replays_match_eager(gpu_lib):
    lib = gpu_lib
    M, N, K, R = 512, 512, 384, 16
    print(f"case graph step M={M} N={N} K={K} R={R}", flush=True)
    inp = make_inputs(M, N, K, R, seed=77)
    X, W, A, B, dY = (bits_to_dev(getattr(inp, n)) for n in ("X", "W", "A", "B", "dY"))
    ws_bytes = lib.lora_bwd_workspace_bytes(1, M, N, K, R)

    def buffers():
        return dict(Y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                    XA=torch.empty((M, R), dtype=torch.float32, device="cuda"),
                    dX=torch.empty((M, K), dtype=torch.bfloat16, device="cuda"),
                    dA=torch.empty((R, K), dtype=torch.float32, device="cuda"),
                    dB=torch.empty((N, R), dtype=torch.float32, device="cuda"),
                    ws=torch.empty(ws_bytes, dtype=torch.uint8, device="cuda"))

    def step(b):
        lib.lora_fwd(X, W, A, B, inp.scale, Y=b["Y"], XA=b["XA"])
        lib.lora_bwd(dY, X, W, A, B, b["XA"], inp.scale, dX=b["dX"], dA=b["dA"], dB=b["dB"], ws=b["ws"])

    eager = buffers()
    step(eager)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in eager.items() if k != "ws"}

    g_buf = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream once, as graph capture expects
        step(g_buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_buf)
    other = buffers()
    for rep in range(4):
        for k in ("Y", "dX", "dA", "dB"):
            g_buf[k].zero_()
        torch.cuda.synchronize()
        graph.replay()
        step(other)  # unrelated eager work between replays
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(g_buf[k], v), f"replay {rep}: {k} differs from the eager step"
