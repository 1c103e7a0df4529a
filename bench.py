#!/usr/bin/env python3
"""Benchmark of the fused LoRA layer on one MI355X.

One step = lora_fwd + lora_bwd (every kernel of the bf16 path: the fused forward with its
rank-R panel and low-rank epilogue, the fused input gradient with its panel, the split-K
adapter-gradient partials and their fixed-order reduction) on the LoRA attention projection
M = 8192 tokens (4 x 2048), K = N = 4096, r = 16, alpha = 32, bf16 with fp32 accumulation,
synthetic seeded inputs already resident in HBM.

Prints one JSON line.  `value` is algorithmic TFLOP/s (4MNK + 6Mr(K+N) per step) over the
timed steps.  `roofline` reports the dominant kernel, the fused input gradient (the only
kernel of a lora_bwd_dx call), timed live with HIP events on its stream; its `traffic` is the
per-launch HBM byte count recorded under profiles/ from rocprofv3 counters, or null when the
kernel's sources have changed since the counters were taken.  `cpu_baseline` times the float64
oracle on a bounded sample of the same workload.  `secondary` holds the QLoRA fwd+bwd rate
on the int4 FFN projection, the decode matrix-vector bandwidth, and the same attention
projection layer run unfused through torch (hipBLASLt GEMMs), for comparison.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk (AMD MI355X spec)
PEAK_HBM_GBS = 8000.0       # HBM3E, AMD MI355X spec
METRIC = "fused LoRA fwd+bwd TFLOP/s (% bf16 MFMA peak), M=8192 K=N=4096 r=16"


def lora_flops(M, N, K, R):
    return 4.0 * M * N * K + 6.0 * M * R * (K + N)


def fwd_flops(M, N, K, R):
    return 2.0 * M * N * K + 2.0 * M * R * (K + N)


def dx_flops(M, N, K, R):
    # dY W (2MNK) + the rank-R panel G = dY B (2MNR) + its epilogue G A (2MRK)
    return 2.0 * M * N * K + 2.0 * M * R * (K + N)


DX_SOURCES = ("qlora_fine_tuning_amd/csrc/dx.hip", "qlora_fine_tuning_amd/csrc/common.hpp")
TRAFFIC_PROFILE = "profiles/lora_fwd_bwd_attn_proj_hbm_traffic.md"


def source_sha(files):
    import hashlib

    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel, files):
    """HBM bytes per launch of `kernel` from the committed counter summary, if still current."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    sha = source_sha(files)
    for line in open(path):
        f = line.split()
        if len(f) == 4 and f[0] == "roofline_traffic" and f[1] == kernel and f[3] == f"source_sha={sha}":
            return float(f[2].split("=")[1])
    return None


def dev_bits(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def event_time_ms(fn, reps, stream):
    """Average milliseconds of fn() over reps calls, HIP events recorded on `stream`."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


def cpu_baseline(inp, min_seconds):
    """The float64 oracle, as it stands, on the whole workload, repeated for >= min_seconds, with
    the BLAS thread pool pinned to the cores this process may run on."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = len(os.sched_getaffinity(0))
    x, dy, w, a, b = (oracle.bf16_bits_to_f64(getattr(inp, n)) for n in ("X", "dY", "W", "A", "B"))
    with threadpool_limits(limits=cores):
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        reps, t0 = 0, time.perf_counter()
        while True:
            Y, XA = oracle.lora_forward(x, w, a, b, inp.scale)
            oracle.lora_backward(dy, x, w, a, b, inp.scale, XA=XA)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds or reps >= 200:
                break
    fl = lora_flops(inp.M, inp.N, inp.K, inp.R) * reps
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 fwd+bwd of the whole workload ({inp.M} tokens), {reps} repetitions "
                      f"({fl:.3e} FLOP in {dt:.2f} s)"}


def bench_torch_unfused(torch, X, W, A, B, dY, scale, reps):
    """The same layer as separate library GEMMs (no fusion): Y = X W^T + s (X A^T) B^T and its
    backward with W frozen, in bf16 through torch.matmul (hipBLASLt)."""
    def step():
        XA = X @ A.t()
        Y = torch.addmm(X @ W.t(), XA, B.t(), alpha=scale)
        G = dY @ B
        dX = torch.addmm(dY @ W, G, A, alpha=scale)
        dA = (G.t() @ X) * scale
        dB = (dY.t() @ XA) * scale
        return Y, dX, dA, dB

    for _ in range(10):
        step()
    ms = event_time_ms(step, reps, torch.cuda.current_stream())
    M, K = X.shape
    N, R = W.shape[0], A.shape[0]
    return {"workload": "attn_proj", "ms_per_step": round(ms, 4),
            "TFLOP/s": round(lora_flops(M, N, K, R) / ms / 1e9, 2),
            "note": "bf16 torch.matmul / addmm, one GEMM per product, fp32 accumulation inside each"}


def bench_qlora_ffn(lora, torch, dev, reps, group=64):
    """QLoRA fwd+bwd on the FFN shape; group 64: int4 weights with fp16 scales, group 32: MXFP4."""
    from qlora_fine_tuning_amd.workloads import workload_inputs

    inp = workload_inputs("qlora_ffn")
    M, N, K, R = inp.M, inp.N, inp.K, inp.R
    Wq, Ws = lora.qlora_quantize(torch.from_numpy(inp.W).to(dev), group=group)
    X, A, B, dY = (dev_bits(getattr(inp, n), dev) for n in ("X", "A", "B", "dY"))
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    XA = torch.empty(M, R, dtype=torch.float32, device=dev)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(R, K, dtype=torch.float32, device=dev)
    dB = torch.empty(N, R, dtype=torch.float32, device=dev)
    ws = torch.empty(lora.qlora_bwd_workspace_bytes(M, N, K, R), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        lora.qlora_fwd(X, Wq, Ws, A, B, inp.scale, Y=Y, XA=XA)
        lora.qlora_bwd(dY, X, Wq, Ws, A, B, XA, inp.scale, dX=dX, dA=dA, dB=dB, ws=ws)

    for _ in range(10):
        step()
    torch.cuda.synchronize()
    ms = event_time_ms(step, reps, stream)
    fl = lora_flops(M, N, K, R)
    return {"workload": "qlora_ffn", "weights": "int4" if group == 64 else "mxfp4", "M": M, "N": N, "K": K,
            "r": R, "ms_per_step": round(ms, 4),
            "TFLOP/s": round(fl / ms / 1e9, 2), "frac_bf16_peak": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}


def bench_mlp(lora, torch, dev, reps):
    """The MLP projections of the same layer type (bf16): gate/up K=4096 -> N=14336 and down
    K=14336 -> N=4096, M=8192, r=16; fwd+bwd TFLOP/s of each."""
    from qlora_fine_tuning_amd.workloads import workload_inputs

    out = []
    for name in ("mlp_gate_up", "mlp_down"):
        inp = workload_inputs(name)
        M, N, K, R = inp.M, inp.N, inp.K, inp.R
        X, W, A, B, dY = (dev_bits(getattr(inp, n), dev) for n in ("X", "W", "A", "B", "dY"))
        Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        XA = torch.empty(M, R, dtype=torch.float32, device=dev)
        dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
        dA = torch.empty(R, K, dtype=torch.float32, device=dev)
        dB = torch.empty(N, R, dtype=torch.float32, device=dev)
        ws = torch.empty(lora.lora_bwd_workspace_bytes(lora.LORA_BF16, M, N, K, R), dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream()

        def step():
            lora.lora_fwd(X, W, A, B, inp.scale, Y=Y, XA=XA, stream=stream)
            lora.lora_bwd(dY, X, W, A, B, XA, inp.scale, dX=dX, dA=dA, dB=dB, ws=ws, stream=stream)

        for _ in range(10):
            step()
        torch.cuda.synchronize()
        ms = event_time_ms(step, reps, stream)
        fl = lora_flops(M, N, K, R)
        out.append({"workload": name, "M": M, "N": N, "K": K, "r": R, "ms_per_step": round(ms, 4),
                    "TFLOP/s": round(fl / ms / 1e9, 2), "frac_bf16_peak": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4)})
        del X, W, A, B, dY, Y, XA, dX, dA, dB, ws
    return out


def bench_swiglu(lora, torch, dev, reps):
    """The SwiGLU gate/up pair with LoRA on both projections at the MLP gate/up shape (M=8192,
    K=4096 -> N=14336, r=16): fwd+bwd TFLOP/s counting the two projections' LoRA work."""
    from qlora_fine_tuning_amd.workloads import make_swiglu_inputs

    M, N, K, R = 8192, 14336, 4096, 16
    inp = make_swiglu_inputs(M, N, K, R, seed=3)
    X, Wgu, Ag, Au, Bg, Bu, dH = (dev_bits(getattr(inp, n), dev) for n in ("X", "Wgu", "Ag", "Au", "Bg", "Bu", "dH"))
    H = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    GU = torch.empty(M, 2 * N, dtype=torch.bfloat16, device=dev)
    XA = torch.empty(M, 2 * R, dtype=torch.float32, device=dev)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dA = [torch.empty(R, K, dtype=torch.float32, device=dev) for _ in range(2)]
    dB = [torch.empty(N, R, dtype=torch.float32, device=dev) for _ in range(2)]
    wsf = torch.empty(lora.lora_swiglu_fwd_workspace_bytes(M, N, K, R), dtype=torch.uint8, device=dev)
    wsb = torch.empty(lora.lora_swiglu_bwd_workspace_bytes(M, N, K, R), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        lora.lora_swiglu_fwd(X, Wgu, Ag, Au, Bg, Bu, inp.scale, H=H, GU=GU, XA=XA, ws=wsf, stream=stream)

    def bwd():
        lora.lora_swiglu_bwd(dH, X, Wgu, Ag, Au, Bg, Bu, GU, XA, inp.scale, dX=dX, dAg=dA[0], dAu=dA[1],
                             dBg=dB[0], dBu=dB[1], ws=wsb, stream=stream)

    def step():
        fwd()
        bwd()

    for _ in range(10):
        step()
    torch.cuda.synchronize()
    ms = event_time_ms(step, reps, stream)
    fwd_ms = event_time_ms(fwd, reps, stream)
    fl = 2 * lora_flops(M, N, K, R)
    return {"workload": "mlp_swiglu", "M": M, "N": N, "K": K, "r": R, "ms_per_step": round(ms, 4),
            "fwd_ms": round(fwd_ms, 4), "TFLOP/s": round(fl / ms / 1e9, 2),
            "frac_bf16_peak": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "note": "gate and up projections as one LoRA GEMM over the stacked weight, H = silu(G) * U in its epilogue"}


def bench_rmsnorm(lora, torch, dev, reps):
    """RMSNorm ahead of a projection at the hidden-state shapes of the attention projection
    (M=8192, K=4096) and the QLoRA FFN (M=4096, K=5120): forward, backward with g frozen and with
    dg, rotating over buffer sets whose total exceeds the 256 MB MALL so that HBM is measured.
    Algorithmic bytes: every row read and written once (forward X in, Y out; backward dY and X in,
    dX out), plus g, r and dg."""
    from qlora_fine_tuning_amd.workloads import make_norm_inputs

    out = []
    stream = torch.cuda.current_stream()
    for M, K in ((8192, 4096), (4096, 5120)):
        inp = make_norm_inputs(M, K, seed=7)
        copies = max(3, -(-640 * 2**20 // (6 * M * K)))  # > 640 MB touched per rotation
        X0 = dev_bits(inp.X, dev)
        g = dev_bits(inp.g, dev)
        Xs = [X0] + [X0.clone() for _ in range(copies - 1)]
        dYs = [dev_bits(inp.dY, dev)] + [None] * (copies - 1)
        for i in range(1, copies):
            dYs[i] = dYs[0].clone()
        Ys = [torch.empty_like(X0) for _ in range(copies)]
        rs = [torch.empty(M, dtype=torch.float32, device=dev) for _ in range(copies)]
        dXs = [torch.empty_like(X0) for _ in range(copies)]
        dg = torch.empty(K, dtype=torch.float32, device=dev)
        ws = torch.empty(lora.lora_rmsnorm_bwd_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
        # the calls are ~20 us: the C entry points are called with arguments marshalled once, so
        # that Python's per-call cost does not set the pace
        lib, sp = lora.load(), ctypes.c_void_p(stream.cuda_stream)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        fargs = [(M, K, inp.eps, p(Xs[i]), p(g), p(Ys[i]), p(rs[i]), sp) for i in range(copies)]
        bargs = {dgf: [(M, K, p(dYs[i]), p(Xs[i]), p(g), p(rs[i]), p(dXs[i]), p(dg) if dgf else None,
                        p(ws) if dgf else None, ws.numel() if dgf else 0, sp) for i in range(copies)]
                 for dgf in (False, True)}
        state = {"i": 0}

        def fwd():
            i = state["i"] = (state["i"] + 1) % copies
            assert lib.lora_rmsnorm_fwd(*fargs[i]) == 0

        def bwd(need_dg):
            def call():
                i = state["i"] = (state["i"] + 1) % copies
                assert lib.lora_rmsnorm_bwd(*bargs[need_dg][i]) == 0
            return call

        row = {"workload": "rmsnorm", "M": M, "K": K}
        for name, fn, nbytes in (("fwd", fwd, 4 * M * K + 2 * K + 4 * M),
                                 ("bwd", bwd(False), 6 * M * K + 2 * K + 4 * M),
                                 ("bwd_dg", bwd(True), 6 * M * K + 2 * K + 4 * M + 4 * K)):
            for _ in range(copies):
                fn()
            torch.cuda.synchronize()
            ms = event_time_ms(fn, reps * copies, stream)
            row[name + "_us"] = round(ms * 1e3, 2)
            row[name + "_GB/s"] = round(nbytes / ms / 1e6, 1)
            row[name + "_frac_hbm_peak"] = round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)
        out.append(row)
        del Xs, dYs, Ys, dXs
    return out


def bench_ce(lora, torch, dev, reps):
    """Chunked cross-entropy over an LM head at the page's workload (batch 8 x 2048 tokens, vocabulary
    128000, hidden 4096): loss and dX per call at the library's default chunk (its fp32 logits within
    512 MiB) and at the page's 256-token chunk, TFLOP/s counting 4 M V K (the logits and the dX
    products; each is formed once), with the workspace each needs."""
    from qlora_fine_tuning_amd.workloads import make_ce_inputs

    M, K, V = 16384, 4096, 128000
    inp = make_ce_inputs(M, K, V, seed=8, logit_std=3.0)
    X, W = dev_bits(inp.X, dev), dev_bits(inp.W, dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    loss = torch.empty(M, dtype=torch.float32, device=dev)
    dX = torch.empty_like(X)
    out = []
    for chunk in (0, 256):
        ws = torch.empty(lora.lora_ce_workspace_bytes(M, V, K, chunk, True), dtype=torch.uint8, device=dev)
        call = lambda: lora.lora_ce(X, W, lab, loss=loss, dX=dX, ws=ws, chunk=chunk)
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        ms = event_time_ms(call, reps, torch.cuda.current_stream())
        out.append({"workload": "lm_head_ce", "M": M, "K": K, "V": V,
                    "chunk": chunk or lora.lora_ce_default_chunk(V), "default_chunk": chunk == 0,
                    "ms_per_call": round(ms, 3), "TFLOP/s": round(4 * M * V * K / ms / 1e9, 1),
                    "frac_bf16_peak": round(4 * M * V * K / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                    "workspace_GB": round(ws.numel() / 1e9, 3), "full_fp32_logits_GB": round(M * V * 4 / 1e9, 2)})
        del ws
    del X, W, dX
    return out


def bench_rope(lora, torch, dev, reps, copies=4):
    """RoPE in place on the Llama-3-8B attention shape (8192 tokens, 32 query and 8 key heads of 128,
    base 500000), rotating over buffer sets (> 256 MB MALL); bytes: Q and K read and written once."""
    M, H, Hk, D = 8192, 32, 8, 128
    Qs = [torch.randn(M, H, D, device=dev).to(torch.bfloat16) for _ in range(copies)]
    Ks = [torch.randn(M, Hk, D, device=dev).to(torch.bfloat16) for _ in range(copies)]
    pos = (torch.arange(M, device=dev, dtype=torch.int32) % 2048).contiguous()
    lib, sp = lora.load(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    args = [(M, H, Hk, D, D, 500000.0, 0, p(pos), p(Qs[i]), p(Ks[i]), sp) for i in range(copies)]
    state = {"i": 0}

    def call():
        i = state["i"] = (state["i"] + 1) % copies
        assert lib.lora_rope(*args[i]) == 0

    for _ in range(copies):
        call()
    torch.cuda.synchronize()
    ms = event_time_ms(call, reps * copies, torch.cuda.current_stream())
    nbytes = 2 * M * (H + Hk) * D * 2 + M * 4
    del Qs, Ks
    return {"workload": "rope", "M": M, "H": H, "Hk": Hk, "D": D, "us_per_call": round(ms * 1e3, 2),
            "GB/s": round(nbytes / ms / 1e6, 1), "frac_hbm_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)}


def bench_decode(lora, torch, dev, reps, copies=6):
    """Decode matrix-vector rate, rotating over `copies` distinct weight copies (> 256 MB MALL), with
    the int4 weight (group 64, fp16 scales) and with the MXFP4 weight (blocks of 32, E8M0 scales):
    both move 0.5 + 1/32 bytes per weight.  The C entry points are called with their arguments
    marshalled once (a call is ~15 us: Python must not set the pace)."""
    from qlora_fine_tuning_amd.workloads import workload_inputs

    out = []
    lib = lora.load()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    for fmt in ("int4", "mxfp4"):
        for name in ("decode_up", "decode_down"):
            inp = workload_inputs(name, M=8)
            N, K, R = inp.N, inp.K, inp.R
            W32 = torch.from_numpy(inp.W).to(dev)
            Wq0, Ws0 = lora.qlora_quantize(W32) if fmt == "int4" else lora.mxfp4_quantize(W32)
            del W32
            Wqs = [Wq0] + [Wq0.clone() for _ in range(copies - 1)]
            Wss = [Ws0] + [Ws0.clone() for _ in range(copies - 1)]
            A, B = dev_bits(inp.A, dev), dev_bits(inp.B, dev)
            Xall = dev_bits(inp.X, dev)
            stream = torch.cuda.current_stream()
            sp = ctypes.c_void_p(stream.cuda_stream)
            for M in (1, 4, 8):
                X = Xall[:M].contiguous()
                Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
                need = lora.qlora_fwd_workspace_bytes(M, N, K, R)
                ws = torch.zeros(need, dtype=torch.uint8, device=dev)
                if fmt == "int4":
                    args = [(M, N, K, R, inp.scale, 64, p(X), p(Wqs[i]), p(Wss[i]), p(A), p(B), p(Y), None,
                             p(ws), need, sp) for i in range(copies)]
                    fn = lib.qlora_fwd
                else:
                    args = [(M, N, K, R, inp.scale, p(X), p(Wqs[i]), p(Wss[i]), p(A), p(B), p(Y), None, p(ws), need,
                             sp) for i in range(copies)]
                    fn = lib.mxfp4_decode_fwd
                state = {"i": 0}

                def call():
                    i = state["i"]
                    state["i"] = (i + 1) % copies
                    assert fn(*args[i]) == 0

                for _ in range(copies):
                    call()
                torch.cuda.synchronize()
                ms = event_time_ms(call, reps * copies, stream)
                assert lora.qlora_decode_status(ws) == 0
                wbytes = N * K // 2 + (N * (K // 64) * 2 if fmt == "int4" else N * (K // 32))
                nbytes = wbytes + R * K * 2 + N * R * 2 + M * K * 2 + M * N * 2
                out.append({"workload": name, "weights": fmt, "M": M, "N": N, "K": K,
                            "us_per_call": round(ms * 1e3, 3), "GB/s": round(nbytes / ms / 1e6, 1),
                            "frac_hbm_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)})
            del Wqs, Wss
    return out


def measure_ceilings(lora, torch, dev, stream, iters=4000, read_mb=96, copies=6, reads=30):
    """The chip's practical ceilings, measured after the timed steps: the bf16 MFMA rate when
    every SIMD issues nothing but independent MFMAs (the chip's own power and clock limits set the
    clock), and the streaming-read rate over buffers larger than the 256 MB last-level cache."""
    out = None
    for _ in range(2):  # the second run is reported
        out = lora.lora_probe_mfma(256, iters, stream=stream)
        torch.cuda.synchronize()
    d = out.cpu().numpy().astype(np.float64)
    us = d[:, 1] / 100.0
    mfmas = 64.0 * iters
    tflops = float((mfmas * 16384.0 / us).sum() / 1e6)
    bufs = [torch.zeros(read_mb << 20, dtype=torch.uint8, device=dev) for _ in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for b in bufs:
        lora.lora_probe_hbm_read(b, sink, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reads):
        lora.lora_probe_hbm_read(bufs[i % copies], sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    tbs = reads * (read_mb << 20) / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del bufs
    return {"mfma_bf16_TFLOP/s": round(tflops, 1), "mfma_frac_of_nominal_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "mfma_clock_MHz": round(float(np.median(d[:, 0] / us)), 1),
            "cycles_per_mfma": round(float(np.median(d[:, 0] / mfmas)), 2),
            "hbm_read_TB/s": round(tbs, 3), "hbm_read_frac_of_peak": round(tbs / (PEAK_HBM_GBS / 1000), 4),
            "how": "lora_probe_mfma: 256 workgroups x 4 waves, each 64 independent bf16 16x16x32 MFMAs into "
                   f"AGPRs per block, {iters} blocks, nothing else issued; lora_probe_hbm_read: {reads} reads of "
                   f"{copies} rotating {read_mb} MiB buffers, 1 KB contiguous per wave load"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU's clocks settle over the first tens of milliseconds of sustained matrix work: the
    # timed steps come after 100 untimed ones (about 50 ms)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-secondary", action="store_true", help="skip the QLoRA and decode lines")
    ap.add_argument("--only", default=None, help="comma-separated secondary lines to run (e.g. decode)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle baseline (whole workload, repeated)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (HBM counter calibration under rocprofv3)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer's data-parallel sharding (token slices per GPU, "
              "one all-reduce of dA and dB per layer) is not implemented here. Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch

    from qlora_fine_tuning_amd import lora
    from qlora_fine_tuning_amd.workloads import workload_inputs

    if not os.path.exists(lora.LIB_PATH):
        from qlora_fine_tuning_amd import build

        build.build()
    lora.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    inp = workload_inputs("attn_proj")
    M, N, K, R = inp.M, inp.N, inp.K, inp.R
    X, W, A, B, dY = (dev_bits(getattr(inp, n), dev) for n in ("X", "W", "A", "B", "dY"))
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    XA = torch.empty(M, R, dtype=torch.float32, device=dev)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(R, K, dtype=torch.float32, device=dev)
    dB = torch.empty(N, R, dtype=torch.float32, device=dev)
    ws = torch.empty(lora.lora_bwd_workspace_bytes(lora.LORA_BF16, M, N, K, R), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        lora.lora_fwd(X, W, A, B, inp.scale, Y=Y, XA=XA, stream=stream)

    # lora_bwd as its two halves (bit for bit the same calls): the input gradient, whose kernel is
    # the dominant one and is timed on its own inside the timed region, then the adapter gradients
    def bwd_dx():
        lora.lora_bwd_dx(dY, W, A, B, inp.scale, ws=ws, dX=dX, stream=stream)

    def bwd_dadb():
        lora.lora_bwd_dadb(dY, X, XA, inp.scale, R, ws=ws, dA=dA, dB=dB, stream=stream)

    for _ in range(args.warmup):
        fwd()
        bwd_dx()
        bwd_dadb()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    t_step = [ev() for _ in range(args.steps + 1)]   # step boundaries
    t_dx = [(ev(), ev()) for _ in range(args.steps)]  # around each input-gradient kernel
    t0 = time.perf_counter()
    t_step[0].record(stream)
    for i in range(args.steps):
        fwd()
        t_dx[i][0].record(stream)
        bwd_dx()
        t_dx[i][1].record(stream)
        bwd_dadb()
        t_step[i + 1].record(stream)
    clk = lora.lora_probe_sclk(2000, stream=stream)  # right after the last step: 20 us spin
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = t_step[0].elapsed_time(t_step[-1]) / args.steps
    steps_ms = np.array([t_step[i].elapsed_time(t_step[i + 1]) for i in range(args.steps)])
    dx_each = np.array([a.elapsed_time(b) for a, b in t_dx])
    cyc, ticks = (int(v) for v in clk.cpu().tolist())
    fl = lora_flops(M, N, K, R)
    value = fl / ms / 1e9

    dx_ms = float(dx_each.mean())
    reps = max(args.steps, 10)
    fwd_ms = event_time_ms(fwd, reps, stream)
    ach = dx_flops(M, N, K, R) / dx_ms / 1e9
    kernel = "dx_mfma_kernel<16,false,false,false>"
    roofline = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": profiled_traffic(kernel, DX_SOURCES),
                "traffic_unit": "HBM bytes per launch", "kernel": kernel,
                "kernel_ms": round(dx_ms, 4), "kernel_ms_source": "HIP events around each timed step's lora_bwd_dx",
                "fwd_ms": round(fwd_ms, 4), "fwd_frac": round(fwd_flops(M, N, K, R) / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    step_stats = {"median": round(float(np.median(steps_ms)), 4), "p10": round(float(np.percentile(steps_ms, 10)), 4),
                  "p90": round(float(np.percentile(steps_ms, 90)), 4), "min": round(float(steps_ms.min()), 4),
                  "max": round(float(steps_ms.max()), 4)}
    sclk = {"mhz_after_timed_steps": round(100.0 * cyc / ticks, 1) if ticks else None,
            "how": "shader-cycle counter against the 100 MHz real-time counter over a 20 us spin enqueued "
                   "right after the last timed step"}

    ceilings = measure_ceilings(lora, torch, dev, stream)
    roofline["frac_of_measured_mfma_ceiling"] = round(ach / ceilings["mfma_bf16_TFLOP/s"], 4)

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) / N(0,1/K) / U(+-1/sqrt K) / N(0,0.02 variance) inputs)",
        "config": {"workload": "attn_proj: LoRA attention projection, M=8192 (4x2048) K=N=4096 r=16 alpha=32",
                   "global_batch": 4, "seq_len": 2048, "parallelism": "single GPU"},
        "frac_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "wall_s_timed": round(wall, 3),
        "step_ms": step_stats,
        "sclk": sclk,
        "roofline": roofline,
        "ceilings": ceilings,
    }
    if not args.no_secondary:
        lines = {"mlp": lambda: bench_mlp(lora, torch, dev, 20),
                 "mlp_swiglu": lambda: bench_swiglu(lora, torch, dev, 20),
                 "qlora": lambda: bench_qlora_ffn(lora, torch, dev, 20),
                 "qlora_mxfp4": lambda: bench_qlora_ffn(lora, torch, dev, 20, group=32),
                 "decode": lambda: bench_decode(lora, torch, dev, 20),
                 "rmsnorm": lambda: bench_rmsnorm(lora, torch, dev, 20),
                 "lm_head_ce": lambda: bench_ce(lora, torch, dev, 5),
                 "rope": lambda: bench_rope(lora, torch, dev, 20),
                 "torch_unfused": lambda: bench_torch_unfused(torch, X, W, A, B, dY, inp.scale, 20)}
        only = set(args.only.split(",")) if args.only else None
        result["secondary"] = {k: f() for k, f in lines.items() if only is None or k in only}
        for row in result["secondary"].get("decode", []):
            row["frac_hbm_read_ceiling"] = round(row["GB/s"] / (ceilings["hbm_read_TB/s"] * 1000), 4)
    if args.calib_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
