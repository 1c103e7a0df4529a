"""Python binding of the C ABI in include/lora.h (ctypes; argument marshalling only).

Every entry point keeps the C name.  Tensors are torch CUDA tensors used as device memory;
outputs and workspaces that the caller does not pass are allocated here with torch.  All
arithmetic runs in the gfx950 HIP library: if it is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# QLORA_AMD_LIB may name another build of the same library (the host-sanitized one)
LIB_PATH = os.environ.get("QLORA_AMD_LIB") or os.path.join(_PKG, "liblora_mi355x.so")

LORA_F32, LORA_BF16 = 0, 1
GROUP = 64
MXFP4_GROUP = 32  # the group argument that selects MXFP4 weights
STATUS = {
    0: "LORA_OK", 1: "LORA_ERR_NULL", 2: "LORA_ERR_SHAPE", 3: "LORA_ERR_RANK", 4: "LORA_ERR_ALIGN",
    5: "LORA_ERR_DTYPE", 6: "LORA_ERR_WORKSPACE", 7: "LORA_ERR_GROUP", 8: "LORA_ERR_VALUE",
    9: "LORA_ERR_HIP",
}

# C signatures: name -> (restype, argtypes)
_i64, _i32, _f32, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "lora_fwd": (_i32, [_i32, _i64, _i64, _i64, _i32, _f32, _p, _p, _p, _p, _p, _p, _p]),
    "lora_bwd_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64, _i32]),
    "lora_bwd": (_i32, [_i32, _i64, _i64, _i64, _i32, _f32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "lora_bwd_dx": (_i32, [_i32, _i64, _i64, _i64, _i32, _f32, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "lora_bwd_dadb": (_i32, [_i32, _i64, _i64, _i64, _i32, _f32, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "qlora_bwd_dx": (_i32, [_i64, _i64, _i64, _i32, _f32, _i32, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "qlora_quantize": (_i32, [_i64, _i64, _i32, _p, _p, _p, _p]),
    "qlora_dequant": (_i32, [_i64, _i64, _i32, _p, _p, _p, _p]),
    "qlora_fwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "qlora_fwd": (_i32, [_i64, _i64, _i64, _i32, _f32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "qlora_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "qlora_bwd": (_i32, [_i64, _i64, _i64, _i32, _f32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "lora_swiglu_fwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "lora_swiglu_fwd": (_i32, [_i64, _i64, _i64, _i32, _f32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "lora_swiglu_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "lora_swiglu_bwd": (_i32, [_i64, _i64, _i64, _i32, _f32] + [_p] * 15 + [_sz, _p]),
    "lora_rmsnorm_fwd": (_i32, [_i64, _i64, _f32, _p, _p, _p, _p, _p]),
    "lora_rmsnorm_bwd_workspace_bytes": (_sz, [_i64, _i64]),
    "lora_rmsnorm_bwd": (_i32, [_i64, _i64, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "mxfp4_quantize": (_i32, [_i64, _i64, _p, _p, _p, _p]),
    "mxfp4_dequant": (_i32, [_i64, _i64, _p, _p, _p, _p]),
    "mxfp4_decode_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "mxfp4_decode_fwd": (_i32, [_i64, _i64, _i64, _i32, _f32, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "lora_ce_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i32]),
    "lora_ce_default_chunk": (_i64, [_i64]),
    "lora_ce_scale_grad": (_i32, [_i64, _i64, _p, _p, _p, _p]),
    "lora_ce": (_i32, [_i64, _i64, _i64, _i64, _f32, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "lora_rope": (_i32, [_i64, _i32, _i32, _i32, _i32, _f32, _i32, _p, _p, _p, _p]),
    "qlora_swiglu_fwd": (_i32, [_i64, _i64, _i64, _i32, _f32, _i32] + [_p] * 11 + [_sz, _p]),
    "qlora_swiglu_bwd": (_i32, [_i64, _i64, _i64, _i32, _f32, _i32] + [_p] * 16 + [_sz, _p]),
    "lora_probe_sclk": (_i32, [_p, ctypes.c_uint32, _p]),
    "lora_probe_mfma": (_i32, [_p, _i32, ctypes.c_uint32, _p]),
    "lora_probe_mfma_issue": (_i32, [_p, _i32, ctypes.c_uint32, _i32, _p]),
    "lora_probe_hbm_read": (_i32, [_p, _sz, _p, _p]),
    "qlora_decode_status": (_i32, [_p, _sz, _p, _i32, _p]),
    "qlora_decode_fwd_noalloc": (_i32, [_i64, _i64, _i64, _i32, _f32, _i32, _p, _p, _p, _p, _p, _p, _p, _p]),
    "qlora_decode_set_hold": (_i32, [_p, _sz, _i32, _p]),
    "lora_status_str": (ctypes.c_char_p, [_i32]),
    "lora_last_hip_error": (ctypes.c_char_p, []),
}

_LIB = None


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = _LIB
        msg = lib.lora_status_str(status).decode() if lib is not None else STATUS.get(status, str(status))
        if status == 9 and lib is not None:
            msg += f" ({lib.lora_last_hip_error().decode()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


def load(path: Optional[str] = None):
    """Load the HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m qlora_fine_tuning_amd.build` "
                           "(the layer has no other implementation)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, st: int):
    if st != 0:
        raise LoraError(fn, st)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LORA_F32
    if t.dtype == torch.bfloat16:
        return LORA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _want(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def lora_fwd(X, W, A, B, scale: float, *, Y=None, XA=None, save_xa: bool = True,
             stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Y = X W^T + scale (X A^T) B^T; returns (Y, XA) with XA = X A^T in fp32 (or None)."""
    lib = load()
    dt = _dtype_code(X)
    for t, n in ((X, "X"), (W, "W"), (A, "A"), (B, "B")):
        _want(t, n, X.dtype)
    M, K = X.shape
    N, R = W.shape[0], A.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=X.dtype, device=X.device)
    if XA is None and save_xa:
        XA = torch.empty((M, R), dtype=torch.float32, device=X.device)
    st = lib.lora_fwd(dt, M, N, K, R, float(scale), _ptr(X), _ptr(W), _ptr(A), _ptr(B), _ptr(Y),
                      _ptr(XA), _stream(stream))
    _check("lora_fwd", st)
    return Y, XA


def lora_bwd_workspace_bytes(dt: int, M: int, N: int, K: int, R: int) -> int:
    return int(load().lora_bwd_workspace_bytes(dt, M, N, K, R))


def lora_bwd(dY, X, W, A, B, XA, scale: float, *, dX=None, dA=None, dB=None, ws=None,
             stream=None):
    """Returns (dX, dA, dB): dX in X's dtype, dA (R x K) and dB (N x R) in fp32."""
    lib = load()
    dt = _dtype_code(X)
    M, K = X.shape
    N, R = W.shape[0], A.shape[0]
    dev = X.device
    if dX is None:
        dX = torch.empty((M, K), dtype=X.dtype, device=dev)
    if dA is None:
        dA = torch.empty((R, K), dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty((N, R), dtype=torch.float32, device=dev)
    need = lib.lora_bwd_workspace_bytes(dt, M, N, K, R)
    if ws is None:
        ws = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    st = lib.lora_bwd(dt, M, N, K, R, float(scale), _ptr(dY), _ptr(X), _ptr(W), _ptr(A), _ptr(B),
                      _ptr(XA), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), ws.numel() * ws.element_size(),
                      _stream(stream))
    _check("lora_bwd", st)
    return dX, dA, dB


def _ws_for(lib, dt, M, N, K, R, ws, dev):
    need = lib.lora_bwd_workspace_bytes(dt, M, N, K, R)
    if ws is None:
        ws = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    return ws, ws.numel() * ws.element_size()


def lora_bwd_dx(dY, W, A, B, scale: float, *, ws, dX=None, stream=None):
    """Input-gradient half of lora_bwd: dX, and G = dY B left in `ws` for lora_bwd_dadb."""
    lib = load()
    dt = _dtype_code(dY)
    M, N = dY.shape
    K, R = W.shape[1], A.shape[0]
    if dX is None:
        dX = torch.empty((M, K), dtype=dY.dtype, device=dY.device)
    ws, wsb = _ws_for(lib, dt, M, N, K, R, ws, dY.device)
    st = lib.lora_bwd_dx(dt, M, N, K, R, float(scale), _ptr(dY), _ptr(W), _ptr(A), _ptr(B), _ptr(dX),
                         _ptr(ws), wsb, _stream(stream))
    _check("lora_bwd_dx", st)
    return dX


def lora_bwd_dadb(dY, X, XA, scale: float, R: int, *, ws, dA=None, dB=None, stream=None):
    """Adapter-gradient half of lora_bwd, reading G from `ws` (left by lora_bwd_dx / qlora_bwd_dx)."""
    lib = load()
    dt = _dtype_code(X)
    M, K = X.shape
    N = dY.shape[1]
    if dA is None:
        dA = torch.empty((R, K), dtype=torch.float32, device=X.device)
    if dB is None:
        dB = torch.empty((N, R), dtype=torch.float32, device=X.device)
    ws, wsb = _ws_for(lib, dt, M, N, K, R, ws, X.device)
    st = lib.lora_bwd_dadb(dt, M, N, K, R, float(scale), _ptr(dY), _ptr(X), _ptr(XA), _ptr(dA), _ptr(dB),
                           _ptr(ws), wsb, _stream(stream))
    _check("lora_bwd_dadb", st)
    return dA, dB


def qlora_bwd_dx(dY, Wq, Ws, A, B, scale: float, *, ws, dX=None, stream=None):
    lib = load()
    M, N = dY.shape
    K, R = Wq.shape[1] * 2, A.shape[0]
    if dX is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dY.device)
    ws, wsb = _ws_for(lib, LORA_BF16, M, N, K, R, ws, dY.device)
    st = lib.qlora_bwd_dx(M, N, K, R, float(scale), _group_of(Ws), _ptr(dY), _ptr(Wq), _ptr(Ws), _ptr(A), _ptr(B),
                          _ptr(dX), _ptr(ws), wsb, _stream(stream))
    _check("qlora_bwd_dx", st)
    return dX


def _group_of(Ws) -> int:
    """The 4-bit format from its scales: fp16 per 64 k (int4) or E8M0 bytes per 32 k (MXFP4)."""
    return MXFP4_GROUP if Ws.dtype == torch.uint8 else GROUP


def qlora_quantize(W32, *, group: int = GROUP, stream=None):
    """fp32 W (N x K) -> (Wq uint8 N x K/2, Ws): group 64, int4 codes with fp16 scales (N x K/64);
    group 32, MXFP4 (E2M1 codes, E8M0 exponent bytes N x K/32)."""
    lib = load()
    _want(W32, "W", torch.float32)
    N, K = W32.shape
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=W32.device)
    sdt = torch.uint8 if group == MXFP4_GROUP else torch.float16
    Ws = torch.empty((N, max(K // group, 1)), dtype=sdt, device=W32.device)
    st = lib.qlora_quantize(N, K, group, _ptr(W32), _ptr(Wq), _ptr(Ws), _stream(stream))
    _check("qlora_quantize", st)
    return Wq, Ws


def qlora_dequant(Wq, Ws, *, out=None, stream=None):
    """Dequantised weight bf16_rne(q * s) as a bf16 N x K tensor."""
    lib = load()
    N, K = Wq.shape[0], Wq.shape[1] * 2
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=Wq.device)
    st = lib.qlora_dequant(N, K, _group_of(Ws), _ptr(Wq), _ptr(Ws), _ptr(out), _stream(stream))
    _check("qlora_dequant", st)
    return out


def qlora_fwd_workspace_bytes(M: int, N: int, K: int, R: int) -> int:
    return int(load().qlora_fwd_workspace_bytes(M, N, K, R))


def qlora_fwd(X, Wq, Ws, A, B, scale: float, *, Y=None, XA=None, save_xa: bool = True, ws=None,
              stream=None):
    lib = load()
    M, K = X.shape
    N, R = Wq.shape[0], A.shape[0]
    dev = X.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if XA is None and save_xa:
        XA = torch.empty((M, R), dtype=torch.float32, device=dev)
    need = lib.qlora_fwd_workspace_bytes(M, N, K, R)
    if ws is None and need:
        # the decode path's arrival counters must start at zero (each call leaves them zero)
        ws = torch.zeros(int(need), dtype=torch.uint8, device=dev)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib.qlora_fwd(M, N, K, R, float(scale), _group_of(Ws), _ptr(X), _ptr(Wq), _ptr(Ws), _ptr(A), _ptr(B),
                       _ptr(Y), _ptr(XA), _ptr(ws), wsb, _stream(stream))
    _check("qlora_fwd", st)
    return Y, XA


def qlora_bwd_workspace_bytes(M: int, N: int, K: int, R: int) -> int:
    return int(load().qlora_bwd_workspace_bytes(M, N, K, R))


def qlora_bwd(dY, X, Wq, Ws, A, B, XA, scale: float, *, dX=None, dA=None, dB=None, ws=None,
              stream=None):
    lib = load()
    M, K = X.shape
    N, R = Wq.shape[0], A.shape[0]
    dev = X.device
    if dX is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    if dA is None:
        dA = torch.empty((R, K), dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty((N, R), dtype=torch.float32, device=dev)
    need = lib.qlora_bwd_workspace_bytes(M, N, K, R)
    if ws is None:
        ws = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    st = lib.qlora_bwd(M, N, K, R, float(scale), _group_of(Ws), _ptr(dY), _ptr(X), _ptr(Wq), _ptr(Ws), _ptr(A),
                       _ptr(B), _ptr(XA), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                       ws.numel() * ws.element_size(), _stream(stream))
    _check("qlora_bwd", st)
    return dX, dA, dB


class LoRALinearFunction(torch.autograd.Function):
    """Autograd wrapper: the forward saves X A^T (fp32) for the backward."""

    @staticmethod
    def forward(ctx, X, W, A, B, scale):
        Y, XA = lora_fwd(X, W, A, B, scale)
        ctx.save_for_backward(X, W, A, B, XA)
        ctx.scale = scale
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, W, A, B, XA = ctx.saved_tensors
        dX, dA, dB = lora_bwd(dY.contiguous(), X, W, A, B, XA, ctx.scale)
        return dX, None, dA.to(A.dtype), dB.to(B.dtype), None


class QLoRALinearFunction(torch.autograd.Function):
    """Autograd wrapper for the int4 base weight: Wq and Ws are frozen (no gradient), the forward
    saves X A^T (fp32) for the backward, and A, B receive their gradients in their own dtype."""

    @staticmethod
    def forward(ctx, X, Wq, Ws, A, B, scale):
        Y, XA = qlora_fwd(X, Wq, Ws, A, B, scale)
        ctx.save_for_backward(X, Wq, Ws, A, B, XA)
        ctx.scale = scale
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, Wq, Ws, A, B, XA = ctx.saved_tensors
        dX, dA, dB = qlora_bwd(dY.contiguous(), X, Wq, Ws, A, B, XA, ctx.scale)
        return dX, None, None, dA.to(A.dtype), dB.to(B.dtype), None


def lora_swiglu_fwd_workspace_bytes(M: int, N: int, K: int, R: int) -> int:
    return int(load().lora_swiglu_fwd_workspace_bytes(M, N, K, R))


def lora_swiglu_bwd_workspace_bytes(M: int, N: int, K: int, R: int) -> int:
    return int(load().lora_swiglu_bwd_workspace_bytes(M, N, K, R))


def lora_swiglu_fwd(X, Wgu, Ag, Au, Bg, Bu, scale: float, *, H=None, GU=None, XA=None, save_xa: bool = True,
                    ws=None, stream=None):
    """SwiGLU gate/up pair with LoRA on both: H = silu(G) * U over the stacked weight Wgu = [Wg; Wu]
    (2N x K).  Returns (H, GU, XA): GU = [G | U] (M x 2N bf16) and XA = [X Ag^T | X Au^T] (fp32)."""
    lib = load()
    for t, n in ((X, "X"), (Wgu, "Wgu"), (Ag, "Ag"), (Au, "Au"), (Bg, "Bg"), (Bu, "Bu")):
        _want(t, n, torch.bfloat16)
    M, K = X.shape
    N, R = Wgu.shape[0] // 2, Ag.shape[0]
    dev = X.device
    if H is None:
        H = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if GU is None:
        GU = torch.empty((M, 2 * N), dtype=torch.bfloat16, device=dev)
    if XA is None and save_xa:
        XA = torch.empty((M, 2 * R), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(int(lib.lora_swiglu_fwd_workspace_bytes(M, N, K, R)), 1), dtype=torch.uint8, device=dev)
    st = lib.lora_swiglu_fwd(M, N, K, R, float(scale), _ptr(X), _ptr(Wgu), _ptr(Ag), _ptr(Au), _ptr(Bg), _ptr(Bu),
                             _ptr(H), _ptr(GU), _ptr(XA), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("lora_swiglu_fwd", st)
    return H, GU, XA


def lora_swiglu_bwd(dH, X, Wgu, Ag, Au, Bg, Bu, GU, XA, scale: float, *, dX=None, dAg=None, dAu=None, dBg=None,
                    dBu=None, ws=None, stream=None):
    """Returns (dX, dAg, dAu, dBg, dBu): dX bf16, the adapter gradients fp32."""
    lib = load()
    M, K = X.shape
    N, R = Wgu.shape[0] // 2, Ag.shape[0]
    dev = X.device
    f32 = dict(dtype=torch.float32, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if dX is None else dX
    dAg = torch.empty((R, K), **f32) if dAg is None else dAg
    dAu = torch.empty((R, K), **f32) if dAu is None else dAu
    dBg = torch.empty((N, R), **f32) if dBg is None else dBg
    dBu = torch.empty((N, R), **f32) if dBu is None else dBu
    if ws is None:
        ws = torch.empty(max(int(lib.lora_swiglu_bwd_workspace_bytes(M, N, K, R)), 1), dtype=torch.uint8, device=dev)
    st = lib.lora_swiglu_bwd(M, N, K, R, float(scale), _ptr(dH), _ptr(X), _ptr(Wgu), _ptr(Ag), _ptr(Au), _ptr(Bg),
                             _ptr(Bu), _ptr(GU), _ptr(XA), _ptr(dX), _ptr(dAg), _ptr(dAu), _ptr(dBg), _ptr(dBu),
                             _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("lora_swiglu_bwd", st)
    return dX, dAg, dAu, dBg, dBu


class SwiGLULoRAFunction(torch.autograd.Function):
    """Autograd wrapper of the SwiGLU gate/up pair: Wgu frozen; the forward saves [G | U] and the
    stacked X A^T, the backward recomputes sigmoid(G) from them."""

    @staticmethod
    def forward(ctx, X, Wgu, Ag, Au, Bg, Bu, scale):
        H, GU, XA = lora_swiglu_fwd(X, Wgu, Ag, Au, Bg, Bu, scale)
        ctx.save_for_backward(X, Wgu, Ag, Au, Bg, Bu, GU, XA)
        ctx.scale = scale
        return H

    @staticmethod
    def backward(ctx, dH):
        X, Wgu, Ag, Au, Bg, Bu, GU, XA = ctx.saved_tensors
        dX, dAg, dAu, dBg, dBu = lora_swiglu_bwd(dH.contiguous(), X, Wgu, Ag, Au, Bg, Bu, GU, XA, ctx.scale)
        return dX, None, dAg.to(Ag.dtype), dAu.to(Au.dtype), dBg.to(Bg.dtype), dBu.to(Bu.dtype), None


def lora_rmsnorm_fwd(X, g, eps: float, *, Y=None, r=None, stream=None):
    """RMSNorm of the rows of X (M x K bf16) with the per-feature scale g (K bf16).  Returns
    (Y, r): Y (M x K bf16), the input of the following projection; r (M fp32), the reciprocal RMS
    the backward reuses."""
    lib = load()
    _want(X, "X", torch.bfloat16)
    _want(g, "g", torch.bfloat16)
    M, K = X.shape
    if Y is None:
        Y = torch.empty_like(X)
    if r is None:
        r = torch.empty(M, dtype=torch.float32, device=X.device)
    st = lib.lora_rmsnorm_fwd(M, K, float(eps), _ptr(X), _ptr(g), _ptr(Y), _ptr(r), _stream(stream))
    _check("lora_rmsnorm_fwd", st)
    return Y, r


def lora_rmsnorm_bwd_workspace_bytes(M: int, K: int) -> int:
    return int(load().lora_rmsnorm_bwd_workspace_bytes(M, K))


def lora_rmsnorm_bwd(dY, X, g, r, *, need_dg: bool = True, dX=None, dg=None, ws=None, stream=None):
    """Returns (dX, dg): dX (M x K bf16); dg (K fp32), or None when need_dg is False (g frozen)."""
    lib = load()
    for t, n in ((dY, "dY"), (X, "X"), (g, "g")):
        _want(t, n, torch.bfloat16)
    _want(r, "r", torch.float32)
    M, K = X.shape
    if dX is None:
        dX = torch.empty_like(X)
    if need_dg:
        if dg is None:
            dg = torch.empty(K, dtype=torch.float32, device=X.device)
        if ws is None:
            ws = torch.empty(max(lora_rmsnorm_bwd_workspace_bytes(M, K), 1), dtype=torch.uint8, device=X.device)
    else:
        dg = None
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib.lora_rmsnorm_bwd(M, K, _ptr(dY), _ptr(X), _ptr(g), _ptr(r), _ptr(dX), _ptr(dg), _ptr(ws), nbytes,
                              _stream(stream))
    _check("lora_rmsnorm_bwd", st)
    return dX, dg


class RMSNormFunction(torch.autograd.Function):
    """Autograd wrapper of the RMSNorm ahead of a projection: the forward saves X and the
    reciprocal RMS; dg is computed only when g requires a gradient."""

    @staticmethod
    def forward(ctx, X, g, eps):
        Y, r = lora_rmsnorm_fwd(X, g, eps)
        ctx.save_for_backward(X, g, r)
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, g, r = ctx.saved_tensors
        dX, dg = lora_rmsnorm_bwd(dY.contiguous(), X, g, r, need_dg=ctx.needs_input_grad[1])
        return dX, (dg.to(g.dtype) if dg is not None else None), None


def mxfp4_quantize(W32, *, stream=None):
    """MXFP4 codes and E8M0 block exponents of an fp32 weight (N x K): (Wq uint8 N x K/2,
    We uint8 N x K/32)."""
    lib = load()
    _want(W32, "W", torch.float32)
    N, K = W32.shape
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=W32.device)
    We = torch.empty((N, K // 32), dtype=torch.uint8, device=W32.device)
    _check("mxfp4_quantize", lib.mxfp4_quantize(N, K, _ptr(W32), _ptr(Wq), _ptr(We), _stream(stream)))
    return Wq, We


def mxfp4_dequant(Wq, We, *, out=None, stream=None):
    lib = load()
    N, K = Wq.shape[0], Wq.shape[1] * 2
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=Wq.device)
    _check("mxfp4_dequant", lib.mxfp4_dequant(N, K, _ptr(Wq), _ptr(We), _ptr(out), _stream(stream)))
    return out


def mxfp4_decode_workspace_bytes(M: int, N: int, K: int, R: int) -> int:
    return int(load().mxfp4_decode_workspace_bytes(M, N, K, R))


def mxfp4_decode_fwd(X, Wq, We, A, B, scale: float, *, Y=None, XA=None, save_xa: bool = True, ws=None,
                     stream=None):
    """Decode forward (1 <= M <= 8, K a multiple of 1024) with the MXFP4 weight.  Returns (Y, XA).
    A workspace passed in must have been zeroed before its first use (every call leaves it so)."""
    lib = load()
    for t, n in ((X, "X"), (A, "A"), (B, "B")):
        _want(t, n, torch.bfloat16)
    M, K = X.shape
    N, R = Wq.shape[0], A.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    if XA is None and save_xa:
        XA = torch.empty((M, R), dtype=torch.float32, device=X.device)
    if ws is None:
        ws = torch.zeros(max(mxfp4_decode_workspace_bytes(M, N, K, R), 256), dtype=torch.uint8, device=X.device)
    st = lib.mxfp4_decode_fwd(M, N, K, R, float(scale), _ptr(X), _ptr(Wq), _ptr(We), _ptr(A), _ptr(B), _ptr(Y),
                              _ptr(XA), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("mxfp4_decode_fwd", st)
    return Y, XA


def lora_ce_workspace_bytes(M: int, V: int, K: int, chunk: int = 0, grad: bool = True) -> int:
    return int(load().lora_ce_workspace_bytes(M, V, K, chunk, int(grad)))


def lora_ce_default_chunk(V: int) -> int:
    return int(load().lora_ce_default_chunk(V))


def lora_ce(X, W, labels, *, grad: bool = True, grad_scale: Optional[float] = None, chunk: int = 0, loss=None,
            dX=None, ws=None, stream=None):
    """Cross-entropy of the logits X W^T (X: M x K bf16, W: the V x K bf16 LM head, labels: M int32) in
    chunks of tokens.  Returns (loss_total (1,) fp32 = grad_scale * the sum of the losses, loss (M,) fp32,
    dX (M x K bf16) or None), dX being the gradient of loss_total (grad_scale defaults to 1/M: the mean
    loss)."""
    lib = load()
    _want(X, "X", torch.bfloat16)
    _want(W, "W", torch.bfloat16)
    _want(labels, "labels", torch.int32)
    M, K = X.shape
    V = W.shape[0]
    dev = X.device
    if grad_scale is None:
        grad_scale = 1.0 / max(M, 1)
    if loss is None:
        loss = torch.empty(M, dtype=torch.float32, device=dev)
    loss_total = torch.empty(4, dtype=torch.float32, device=dev)
    if grad and dX is None:
        dX = torch.empty_like(X)
    if not grad:
        dX = None
    if ws is None:
        ws = torch.empty(max(lora_ce_workspace_bytes(M, V, K, chunk, grad), 256), dtype=torch.uint8, device=dev)
    st = lib.lora_ce(M, V, K, chunk, float(grad_scale), _ptr(X), _ptr(W), _ptr(labels), _ptr(loss),
                     _ptr(loss_total), _ptr(dX), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("lora_ce", st)
    return loss_total[:1], loss, dX


def lora_ce_scale_grad(dX, g, *, out=None, stream=None):
    """out = bf16(dX * g) with g a one-element fp32 device tensor (read on the device)."""
    lib = load()
    _want(dX, "dX", torch.bfloat16)
    if g.dtype != torch.float32 or g.numel() != 1 or g.device != dX.device:
        raise ValueError("g: one fp32 value on dX's device")
    g = g.reshape(1).contiguous()
    M, K = dX.shape
    if out is None:
        out = torch.empty_like(dX)
    _check("lora_ce_scale_grad", lib.lora_ce_scale_grad(M, K, _ptr(g), _ptr(dX), _ptr(out), _stream(stream)))
    return out


class LMHeadCrossEntropyFunction(torch.autograd.Function):
    """Mean cross-entropy of the logits X W^T with W frozen: the forward runs the chunked loss and
    gradient together (the gradient of the logits is never kept past its chunk) and saves dX; the
    backward scales it by the upstream gradient on the device."""

    @staticmethod
    def forward(ctx, X, W, labels, chunk=0):
        M = X.shape[0]
        loss_total, _, dX = lora_ce(X, W, labels, grad=True, grad_scale=1.0 / max(M, 1), chunk=chunk)
        ctx.save_for_backward(dX)
        return loss_total[0]

    @staticmethod
    def backward(ctx, g):
        (dX,) = ctx.saved_tensors
        return lora_ce_scale_grad(dX, g.float()), None, None, None


def lora_rope(Q, K, positions, base: float, *, rot: Optional[int] = None, inverse: bool = False, stream=None):
    """Rotate Q (M x H x D) and K (M x Hk x D, or None) in place by the positions' angles (inverse:
    by the negated angles, the backward).  Returns (Q, K)."""
    lib = load()
    _want(Q, "Q", torch.bfloat16)
    _want(positions, "positions", torch.int32)
    M, H, D = Q.shape
    Hk = 0
    if K is not None:
        _want(K, "K", torch.bfloat16)
        Hk = K.shape[1]
    rot = D if rot is None else rot
    st = lib.lora_rope(M, H, Hk, D, rot, float(base), int(inverse), _ptr(positions), _ptr(Q), _ptr(K),
                       _stream(stream))
    _check("lora_rope", st)
    return Q, K


class RoPEFunction(torch.autograd.Function):
    """Autograd wrapper: rotates copies of Q and K (the inputs stay as they are); the backward
    rotates the incoming gradients back in place."""

    @staticmethod
    def forward(ctx, Q, K, positions, base, rot=None):
        Qr, Kr = Q.clone(), K.clone()
        lora_rope(Qr, Kr, positions, base, rot=rot)
        ctx.save_for_backward(positions)
        ctx.base, ctx.rot = base, rot
        return Qr, Kr

    @staticmethod
    def backward(ctx, dQ, dK):
        (positions,) = ctx.saved_tensors
        dQ, dK = dQ.contiguous().clone(), dK.contiguous().clone()
        lora_rope(dQ, dK, positions, ctx.base, rot=ctx.rot, inverse=True)
        return dQ, dK, None, None, None


def qlora_swiglu_fwd(X, Wguq, Wgus, Ag, Au, Bg, Bu, scale: float, *, H=None, GU=None, XA=None,
                     save_xa: bool = True, ws=None, stream=None):
    """The SwiGLU pair over the stacked 4-bit weight (Wguq, Wgus from qlora_quantize of [Wg; Wu]; the
    format follows Wgus: fp16 scales int4, uint8 exponents MXFP4).  Returns (H, GU, XA)."""
    lib = load()
    for t, n in ((X, "X"), (Ag, "Ag"), (Au, "Au"), (Bg, "Bg"), (Bu, "Bu")):
        _want(t, n, torch.bfloat16)
    M, K = X.shape
    N, R = Wguq.shape[0] // 2, Ag.shape[0]
    dev = X.device
    H = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if H is None else H
    GU = torch.empty((M, 2 * N), dtype=torch.bfloat16, device=dev) if GU is None else GU
    if XA is None and save_xa:
        XA = torch.empty((M, 2 * R), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(lora_swiglu_fwd_workspace_bytes(M, N, K, R), 1), dtype=torch.uint8, device=dev)
    st = lib.qlora_swiglu_fwd(M, N, K, R, float(scale), _group_of(Wgus), _ptr(X), _ptr(Wguq), _ptr(Wgus), _ptr(Ag),
                              _ptr(Au), _ptr(Bg), _ptr(Bu), _ptr(H), _ptr(GU), _ptr(XA), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream))
    _check("qlora_swiglu_fwd", st)
    return H, GU, XA


def qlora_swiglu_bwd(dH, X, Wguq, Wgus, Ag, Au, Bg, Bu, GU, XA, scale: float, *, ws=None, stream=None):
    """Returns (dX, dAg, dAu, dBg, dBu) for the 4-bit stacked weight."""
    lib = load()
    M, K = X.shape
    N, R = Wguq.shape[0] // 2, Ag.shape[0]
    dev = X.device
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dAg, dAu = (torch.empty((R, K), dtype=torch.float32, device=dev) for _ in range(2))
    dBg, dBu = (torch.empty((N, R), dtype=torch.float32, device=dev) for _ in range(2))
    if ws is None:
        ws = torch.empty(max(lora_swiglu_bwd_workspace_bytes(M, N, K, R), 1), dtype=torch.uint8, device=dev)
    st = lib.qlora_swiglu_bwd(M, N, K, R, float(scale), _group_of(Wgus), _ptr(dH), _ptr(X), _ptr(Wguq), _ptr(Wgus),
                              _ptr(Ag), _ptr(Au), _ptr(Bg), _ptr(Bu), _ptr(GU), _ptr(XA), _ptr(dX), _ptr(dAg),
                              _ptr(dAu), _ptr(dBg), _ptr(dBu), _ptr(ws), ws.numel() * ws.element_size(),
                              _stream(stream))
    _check("qlora_swiglu_bwd", st)
    return dX, dAg, dAu, dBg, dBu


def lora_probe_sclk(ticks: int = 2000, *, out=None, stream=None) -> torch.Tensor:
    """Enqueue the shader-clock probe; returns the device tensor [shader cycles, 100 MHz ticks]
    (int64), to be read after the stream has run it."""
    lib = load()
    if out is None:
        out = torch.zeros(2, dtype=torch.int64, device="cuda")
    _check("lora_probe_sclk", lib.lora_probe_sclk(_ptr(out), int(ticks), _stream(stream)))
    return out


def lora_probe_mfma(blocks: int = 256, iters: int = 2000, *, out=None, stream=None) -> torch.Tensor:
    """Enqueue the matrix-core ceiling probe; returns the device tensor [waves, 3] (int64) of
    (shader cycles, 100 MHz ticks, live value) per wave, to be read after the stream has run it."""
    lib = load()
    if out is None:
        out = torch.zeros(blocks * 4, 3, dtype=torch.int64, device="cuda")
    _check("lora_probe_mfma", lib.lora_probe_mfma(_ptr(out), int(blocks), int(iters), _stream(stream)))
    return out


def lora_probe_mfma_issue(mode: int, blocks: int = 256, iters: int = 1000, *, out=None, stream=None) -> torch.Tensor:
    """Enqueue the MFMA issue-cost probe in `mode` (0-7); returns the device tensor [waves, 3]
    (int64) of (shader cycles, 100 MHz ticks, live value) per wave; each wave issues 128 x iters
    MFMAs."""
    lib = load()
    if out is None:
        out = torch.zeros(blocks * 4, 3, dtype=torch.int64, device="cuda")
    _check("lora_probe_mfma_issue",
           lib.lora_probe_mfma_issue(_ptr(out), int(blocks), int(iters), int(mode), _stream(stream)))
    return out


def lora_probe_hbm_read(buf: torch.Tensor, sink: torch.Tensor, *, stream=None) -> None:
    """Enqueue one streaming read of `buf` (its whole storage); `sink`: one int32 on the device."""
    lib = load()
    _check("lora_probe_hbm_read", lib.lora_probe_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                          _stream(stream)))


def qlora_decode_status(ws: torch.Tensor, *, clear: bool = False, stream=None) -> int:
    """Status word of a decode workspace (0: normal; 1: a bounded wait gave up); waits for the stream.
    With clear, the control block is zeroed so the workspace can be used again."""
    lib = load()
    out = ctypes.c_uint32(0)
    _check("qlora_decode_status", lib.qlora_decode_status(_ptr(ws), ws.numel() * ws.element_size(),
                                                          ctypes.byref(out), int(clear), _stream(stream)))
    return int(out.value)


def qlora_decode_set_hold(ws: torch.Tensor, hold: bool, *, stream=None) -> None:
    """Test hook: with hold, decode calls on `ws` withhold their X A^T partials, so their bounded waits give up."""
    lib = load()
    _check("qlora_decode_set_hold", lib.qlora_decode_set_hold(_ptr(ws), ws.numel() * ws.element_size(), int(hold),
                                                              _stream(stream)))


def qlora_decode_fwd_noalloc(X, Wq, Ws, A, B, scale: float, *, Y, XA=None, stream=None) -> None:
    """The decode product with the library's static scratch (no workspace; the caller passes Y)."""
    lib = load()
    M, K = X.shape
    N, R = Wq.shape[0], A.shape[0]
    st = lib.qlora_decode_fwd_noalloc(M, N, K, R, float(scale), _group_of(Ws), _ptr(X), _ptr(Wq), _ptr(Ws), _ptr(A),
                                      _ptr(B), _ptr(Y), _ptr(XA), _stream(stream))
    _check("qlora_decode_fwd_noalloc", st)
