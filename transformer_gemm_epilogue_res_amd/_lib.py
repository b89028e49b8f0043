"""ctypes binding of libcoda.so (include/coda.h). Argument marshalling only.

torch tensors supply device memory and the current stream; every step of the
chain runs in the library's HIP kernels. If the library is missing this module
raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_float, c_int, c_int64, c_size_t, c_void_p

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# CODA_LIB may name another build of the library (e.g. a tuning variant).
LIB_PATH = os.environ.get("CODA_LIB") or os.path.join(PKG, "libcoda.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "coda.h")

CODA_OK, CODA_ERR_NULL, CODA_ERR_SHAPE, CODA_ERR_ALIGN, CODA_ERR_WORKSPACE, CODA_ERR_ARG, CODA_ERR_HIP = range(7)
CODA_BF16, CODA_F32 = 0, 1
(CODA_OP_FWD, CODA_OP_BWD, CODA_OP_UNFUSED_FWD, CODA_OP_UNFUSED_BWD, CODA_OP_FWD_SWIGLU, CODA_OP_BWD_SWIGLU,
 CODA_OP_CE_FWD, CODA_OP_CE_BWD, CODA_OP_UNFUSED_FWD_SWIGLU, CODA_OP_UNFUSED_BWD_SWIGLU,
 CODA_OP_UNFUSED_CE_FWD, CODA_OP_UNFUSED_CE_BWD) = range(12)
CODA_ROW, CODA_COL = 0, 1
CODA_FWD_STAGES, CODA_BWD_STAGES = 3, 5
FWD_STAGE_NAMES = ("gemm0_residual_ssq", "rms_combine", "gemm1_rowscale")
BWD_STAGE_NAMES = ("gr_transpose", "wgrad_rowdot", "s_combine", "dgrad_rmsnorm_bwd", "dgamma_combine")


class FwdArgs(ctypes.Structure):
    _fields_ = [("M", c_int64), ("K0", c_int64), ("D", c_int64), ("N", c_int64), ("eps", c_float),
                ("x", c_void_p), ("W0", c_void_p), ("z", c_void_p), ("gamma", c_void_p), ("W1", c_void_p),
                ("h", c_void_p), ("g", c_void_p), ("r", c_void_p), ("y", c_void_p), ("y_dtype", c_int)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("M", c_int64), ("D", c_int64), ("N", c_int64),
                ("dY", c_void_p), ("y", c_void_p), ("h", c_void_p), ("g", c_void_p), ("r", c_void_p),
                ("gamma", c_void_p), ("W1", c_void_p),
                ("da", c_void_p), ("dgamma", c_void_p), ("dW1", c_void_p), ("s", c_void_p),
                ("da_dtype", c_int), ("dW1_dtype", c_int)]


class GemmArgs(ctypes.Structure):
    _fields_ = [("M", c_int64), ("N", c_int64), ("K", c_int64),
                ("A", c_void_p), ("lda", c_int64), ("a_layout", c_int),
                ("B", c_void_p), ("ldb", c_int64), ("b_layout", c_int),
                ("C", c_void_p), ("ldc", c_int64), ("c_dtype", c_int)]


class BwdGemm0Args(ctypes.Structure):
    _fields_ = [("M", c_int64), ("K0", c_int64), ("D", c_int64),
                ("dh", c_void_p), ("x", c_void_p), ("W0", c_void_p), ("dx", c_void_p), ("dW0", c_void_p),
                ("dx_dtype", c_int), ("dW0_dtype", c_int)]


class FwdSwigluArgs(ctypes.Structure):
    _fields_ = [("chain", FwdArgs), ("o", c_void_p), ("o_dtype", c_int)]


class BwdSwigluArgs(ctypes.Structure):
    _fields_ = [("M", c_int64), ("D", c_int64), ("N", c_int64), ("E", c_int64),
                ("dOut", c_void_p), ("W2", c_void_p), ("o", c_void_p),
                ("y", c_void_p), ("h", c_void_p), ("g", c_void_p), ("r", c_void_p),
                ("gamma", c_void_p), ("W1", c_void_p),
                ("dY", c_void_p), ("da", c_void_p), ("dgamma", c_void_p), ("dW1", c_void_p), ("dW2", c_void_p),
                ("s", c_void_p), ("da_dtype", c_int), ("dW1_dtype", c_int), ("dW2_dtype", c_int)]


class CeFwdArgs(ctypes.Structure):
    _fields_ = [("M", c_int64), ("D", c_int64), ("V", c_int64), ("h", c_void_p), ("W", c_void_p),
                ("targets", c_void_p), ("lse", c_void_p), ("loss", c_void_p), ("logits", c_void_p)]


class CeBwdArgs(ctypes.Structure):
    _fields_ = [("M", c_int64), ("D", c_int64), ("V", c_int64), ("h", c_void_p), ("W", c_void_p),
                ("targets", c_void_p), ("lse", c_void_p), ("dloss", c_void_p),
                ("dlogits", c_void_p), ("dh", c_void_p), ("dW", c_void_p), ("dh_dtype", c_int), ("dW_dtype", c_int),
                ("logits", c_void_p)]


class CodaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcoda.so (built by __graft_entry__.build() / build.py); raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        L.coda_workspace_bytes.restype = c_size_t
        L.coda_workspace_bytes.argtypes = [c_int, c_int64, c_int64, c_int64]
        for name, argt in (("coda_validate_fwd", [POINTER(FwdArgs), c_void_p, c_size_t]),
                           ("coda_validate_bwd", [POINTER(BwdArgs), c_void_p, c_size_t]),
                           ("coda_validate_gemm", [POINTER(GemmArgs)]),
                           ("coda_validate_unfused", [c_int, c_void_p, c_void_p, c_size_t]),
                           ("coda_fwd", [POINTER(FwdArgs), c_void_p, c_size_t, c_void_p]),
                           ("coda_validate_fwd_noalloc", [POINTER(FwdArgs)]),
                           ("coda_fwd_noalloc", [POINTER(FwdArgs), c_void_p]),
                           ("coda_bwd", [POINTER(BwdArgs), c_void_p, c_size_t, c_void_p]),
                           ("coda_unfused_ref", [c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
                           ("coda_fwd_stage", [c_int, POINTER(FwdArgs), c_void_p, c_size_t, c_void_p]),
                           ("coda_bwd_stage", [c_int, POINTER(BwdArgs), c_void_p, c_size_t, c_void_p]),
                           ("coda_gemm", [POINTER(GemmArgs), c_void_p]),
                           ("coda_validate_bwd_gemm0", [POINTER(BwdGemm0Args)]),
                           ("coda_bwd_gemm0", [POINTER(BwdGemm0Args), c_void_p]),
                           ("coda_validate_fwd_swiglu", [POINTER(FwdSwigluArgs), c_void_p, c_size_t]),
                           ("coda_validate_bwd_swiglu", [POINTER(BwdSwigluArgs), c_void_p, c_size_t]),
                           ("coda_fwd_swiglu", [POINTER(FwdSwigluArgs), c_void_p, c_size_t, c_void_p]),
                           ("coda_bwd_swiglu", [POINTER(BwdSwigluArgs), c_void_p, c_size_t, c_void_p]),
                           ("coda_validate_ce_fwd", [POINTER(CeFwdArgs), c_void_p, c_size_t]),
                           ("coda_validate_ce_bwd", [POINTER(CeBwdArgs)]),
                           ("coda_ce_fwd", [POINTER(CeFwdArgs), c_void_p, c_size_t, c_void_p]),
                           ("coda_ce_bwd", [POINTER(CeBwdArgs), c_void_p])):
            fn = getattr(L, name)
            fn.restype = c_int
            fn.argtypes = argt
        L.coda_status_string.restype = ctypes.c_char_p
        L.coda_status_string.argtypes = [c_int]
        _lib = L
    return _lib


def declared_functions() -> list:
    """Names of the functions include/coda.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\*?\s+\**(coda_[a-z0-9_]+)\s*\(", text, re.M)))


def status_string(s: int) -> str:
    return lib().coda_status_string(s).decode()


def _check(status: int, where: str):
    if status != CODA_OK:
        raise CodaError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(dtype) -> int:
    if dtype == torch.bfloat16:
        return CODA_BF16
    if dtype == torch.float32:
        return CODA_F32
    raise ValueError(f"unsupported output dtype {dtype}")


def _want(t, name, dtype, shape=None, device=None):
    """t must be a contiguous GPU tensor of `dtype` (or one of a tuple of dtypes), `shape` and, when
    given, on `device`: every pointer handed to the library is then device memory of the stated size."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise TypeError(f"{name}: expected {' or '.join(map(str, dts))}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor (got one on {t.device})")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name}: on {t.device}, the other tensors are on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


OUT_DTYPES = (torch.bfloat16, torch.float32)


def _ws_bytes(ws, device) -> int:
    """Byte size of a workspace tensor (any dtype), after checking it is contiguous GPU memory on device."""
    if not isinstance(ws, torch.Tensor):
        raise TypeError(f"ws: expected a torch.Tensor, got {type(ws).__name__}")
    if not ws.is_cuda or ws.device != torch.device(device):
        raise ValueError(f"ws: must be a GPU tensor on {device} (got one on {ws.device})")
    if not ws.is_contiguous():
        raise ValueError("ws: must be contiguous")
    return ws.numel() * ws.element_size()


def _stream(device) -> c_void_p:
    return c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_bytes(op: int, M: int, D: int, N: int) -> int:
    return int(lib().coda_workspace_bytes(op, M, D, N))


def workspace(op: int, M: int, D: int, N: int, device) -> torch.Tensor:
    return torch.empty(max(workspace_bytes(op, M, D, N), 16), dtype=torch.uint8, device=device)


def _fwd_args(x, W0, z, gamma, W1, eps, h, g, r, y):
    _want(x, "x", torch.bfloat16)
    _want(W1, "W1", torch.bfloat16)
    M, K0 = x.shape
    D, N = W1.shape
    dev = x.device
    _want(x, "x", torch.bfloat16, (M, K0), dev)
    _want(W0, "W0", torch.bfloat16, (K0, D), dev)
    _want(z, "z", torch.bfloat16, (M, D), dev)
    _want(gamma, "gamma", torch.bfloat16, (D,), dev)
    _want(W1, "W1", torch.bfloat16, (D, N), dev)
    _want(h, "h", torch.bfloat16, (M, D), dev)
    if g is not None:
        _want(g, "g", torch.bfloat16, (M, D), dev)
    _want(r, "r", torch.float32, (M,), dev)
    _want(y, "y", OUT_DTYPES, (M, N), dev)
    return FwdArgs(M, K0, D, N, float(eps), _ptr(x), _ptr(W0), _ptr(z), _ptr(gamma), _ptr(W1),
                   _ptr(h), _ptr(g), _ptr(r), _ptr(y), _dt(y.dtype))


def fwd(x, W0, z, gamma, W1, eps, y_dtype=torch.bfloat16, ws=None, out=None, unfused=False):
    """Forward of the chain. Returns dict(h, g, r, y) (g is None for the unfused baseline)."""
    M, D, N = x.shape[0], W1.shape[0], W1.shape[1]
    dev = x.device
    if out is None:
        out = {"h": torch.empty(M, D, dtype=torch.bfloat16, device=dev),
               "g": None if unfused else torch.empty(M, D, dtype=torch.bfloat16, device=dev),
               "r": torch.empty(M, dtype=torch.float32, device=dev),
               "y": torch.empty(M, N, dtype=y_dtype, device=dev)}
    a = _fwd_args(x, W0, z, gamma, W1, eps, out["h"], out["g"], out["r"], out["y"])
    op = CODA_OP_UNFUSED_FWD if unfused else CODA_OP_FWD
    if ws is None:
        ws = workspace(op, M, D, N, dev)
    if unfused:
        st = lib().coda_unfused_ref(CODA_OP_FWD, ctypes.byref(a), _ptr(ws), _ws_bytes(ws, dev), _stream(dev))
    else:
        st = lib().coda_fwd(ctypes.byref(a), _ptr(ws), _ws_bytes(ws, dev), _stream(dev))
    _check(st, "coda_unfused_ref(fwd)" if unfused else "coda_fwd")
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20


def fwd_noalloc(x, W0, z, gamma, W1, eps, y_dtype=torch.bfloat16, out=None):
    """coda_fwd_noalloc: the fused forward with its partials in the library's own device scratch (no
    workspace argument; the outputs in `out` are the caller's). Returns dict(h, g, r, y)."""
    M, D, N = x.shape[0], W1.shape[0], W1.shape[1]
    dev = x.device
    if out is None:
        out = {"h": torch.empty(M, D, dtype=torch.bfloat16, device=dev),
               "g": torch.empty(M, D, dtype=torch.bfloat16, device=dev),
               "r": torch.empty(M, dtype=torch.float32, device=dev),
               "y": torch.empty(M, N, dtype=y_dtype, device=dev)}
    a = _fwd_args(x, W0, z, gamma, W1, eps, out["h"], out["g"], out["r"], out["y"])
    _check(lib().coda_fwd_noalloc(ctypes.byref(a), _stream(dev)), "coda_fwd_noalloc")
    return out


def _bwd_args(dY, y, h, g, r, gamma, W1, da, dgamma, dW1, s):
    _want(dY, "dY", torch.bfloat16)
    _want(W1, "W1", torch.bfloat16)
    M, N = dY.shape
    D = W1.shape[0]
    dev = dY.device
    _want(dY, "dY", torch.bfloat16, (M, N), dev)
    _want(y, "y", torch.bfloat16, (M, N), dev)
    _want(h, "h", torch.bfloat16, (M, D), dev)
    _want(g, "g", torch.bfloat16, (M, D), dev)
    _want(r, "r", torch.float32, (M,), dev)
    _want(gamma, "gamma", torch.bfloat16, (D,), dev)
    _want(W1, "W1", torch.bfloat16, (D, N), dev)
    _want(da, "da", OUT_DTYPES, (M, D), dev)
    _want(dgamma, "dgamma", torch.float32, (D,), dev)
    _want(dW1, "dW1", OUT_DTYPES, (D, N), dev)
    _want(s, "s", torch.float32, (M,), dev)
    return BwdArgs(M, D, N, _ptr(dY), _ptr(y), _ptr(h), _ptr(g), _ptr(r), _ptr(gamma), _ptr(W1),
                   _ptr(da), _ptr(dgamma), _ptr(dW1), _ptr(s), _dt(da.dtype), _dt(dW1.dtype))


def bwd(dY, y, h, g, r, gamma, W1, da_dtype=torch.bfloat16, dW1_dtype=torch.bfloat16, ws=None, out=None,
        unfused=False):
    """Backward of the chain. Returns dict(da, dgamma, dW1, s)."""
    M, N = dY.shape
    D = W1.shape[0]
    dev = dY.device
    if out is None:
        out = {"da": torch.empty(M, D, dtype=da_dtype, device=dev),
               "dgamma": torch.empty(D, dtype=torch.float32, device=dev),
               "dW1": torch.empty(D, N, dtype=dW1_dtype, device=dev),
               "s": torch.empty(M, dtype=torch.float32, device=dev)}
    a = _bwd_args(dY, y, h, g, r, gamma, W1, out["da"], out["dgamma"], out["dW1"], out["s"])
    op = CODA_OP_UNFUSED_BWD if unfused else CODA_OP_BWD
    if ws is None:
        ws = workspace(op, M, D, N, dev)
    if unfused:
        st = lib().coda_unfused_ref(CODA_OP_BWD, ctypes.byref(a), _ptr(ws), _ws_bytes(ws, dev), _stream(dev))
    else:
        st = lib().coda_bwd(ctypes.byref(a), _ptr(ws), _ws_bytes(ws, dev), _stream(dev))
    _check(st, "coda_unfused_ref(bwd)" if unfused else "coda_bwd")
    return out


def _bwd_gemm0_args(dh, x, W0, dx, dW0):
    _want(dh, "dh", torch.bfloat16)
    _want(x, "x", torch.bfloat16)
    M, D = dh.shape
    K0 = x.shape[1]
    dev = dh.device
    _want(dh, "dh", torch.bfloat16, (M, D), dev)
    _want(x, "x", torch.bfloat16, (M, K0), dev)
    _want(W0, "W0", torch.bfloat16, (K0, D), dev)
    _want(dx, "dx", OUT_DTYPES, (M, K0), dev)
    _want(dW0, "dW0", OUT_DTYPES, (K0, D), dev)
    return BwdGemm0Args(M, K0, D, _ptr(dh), _ptr(x), _ptr(W0), _ptr(dx), _ptr(dW0), _dt(dx.dtype), _dt(dW0.dtype))


def bwd_gemm0(dh, x, W0, dx_dtype=torch.bfloat16, dW0_dtype=torch.bfloat16, out=None):
    """Backward through h = x @ W0 + z for the upstream gradient dh: dict(dx, dW0) (dz is dh)."""
    M, D = dh.shape
    K0 = x.shape[1]
    dev = dh.device
    if out is None:
        out = {"dx": torch.empty(M, K0, dtype=dx_dtype, device=dev),
               "dW0": torch.empty(K0, D, dtype=dW0_dtype, device=dev)}
    a = _bwd_gemm0_args(dh, x, W0, out["dx"], out["dW0"])
    _check(lib().coda_bwd_gemm0(ctypes.byref(a), _stream(dev)), "coda_bwd_gemm0")
    return out


def _fwd_swiglu_args(x, W0, z, gamma, W1, eps, out):
    _want(out["o"], "o", OUT_DTYPES, (x.shape[0], W1.shape[1] // 2), x.device)
    return FwdSwigluArgs(_fwd_args(x, W0, z, gamma, W1, eps, out["h"], out["g"], out["r"], out["y"]),
                         _ptr(out["o"]), _dt(out["o"].dtype))


def fwd_swiglu(x, W0, z, gamma, W1, eps, o_dtype=torch.bfloat16, ws=None, out=None, unfused=False):
    """Forward of the chain followed by SwiGLU on y's interleaved (gate, up) columns.
    Returns dict(h, g, r, y, o); y is bf16, o is [M, N/2] in o_dtype. unfused: the SwiGLU
    step as a separate row kernel on the stored y (coda_unfused_ref)."""
    M, D, N = x.shape[0], W1.shape[0], W1.shape[1]
    dev = x.device
    if out is None:
        out = {"h": torch.empty(M, D, dtype=torch.bfloat16, device=dev),
               "g": torch.empty(M, D, dtype=torch.bfloat16, device=dev),
               "r": torch.empty(M, dtype=torch.float32, device=dev),
               "y": torch.empty(M, N, dtype=torch.bfloat16, device=dev),
               "o": torch.empty(M, N // 2, dtype=o_dtype, device=dev)}
    a = _fwd_swiglu_args(x, W0, z, gamma, W1, eps, out)
    if ws is None:
        ws = workspace(CODA_OP_UNFUSED_FWD_SWIGLU if unfused else CODA_OP_FWD_SWIGLU, M, D, N, dev)
    if unfused:
        _check(lib().coda_unfused_ref(CODA_OP_FWD_SWIGLU, ctypes.byref(a), _ptr(ws), _ws_bytes(ws, dev), _stream(dev)),
               "coda_unfused_ref(fwd_swiglu)")
    else:
        _check(lib().coda_fwd_swiglu(ctypes.byref(a), _ptr(ws), _ws_bytes(ws, dev), _stream(dev)), "coda_fwd_swiglu")
    return out


def _bwd_swiglu_args(dOut, W2, o, y, h, g, r, gamma, W1, out):
    _want(dOut, "dOut", torch.bfloat16)
    _want(W1, "W1", torch.bfloat16)
    _want(W2, "W2", torch.bfloat16)
    M, E = dOut.shape
    D, N = W1.shape
    F = W2.shape[0]
    dev = dOut.device
    _want(dOut, "dOut", torch.bfloat16, (M, E), dev)
    _want(W2, "W2", torch.bfloat16, (N // 2, E), dev)
    _want(o, "o", torch.bfloat16, (M, F), dev)
    _want(y, "y", torch.bfloat16, (M, N), dev)
    _want(h, "h", torch.bfloat16, (M, D), dev)
    _want(g, "g", torch.bfloat16, (M, D), dev)
    _want(r, "r", torch.float32, (M,), dev)
    _want(gamma, "gamma", torch.bfloat16, (D,), dev)
    _want(W1, "W1", torch.bfloat16, (D, N), dev)
    _want(out["dY"], "dY", torch.bfloat16, (M, N), dev)
    _want(out["da"], "da", OUT_DTYPES, (M, D), dev)
    _want(out["dgamma"], "dgamma", torch.float32, (D,), dev)
    _want(out["dW1"], "dW1", OUT_DTYPES, (D, N), dev)
    _want(out["dW2"], "dW2", OUT_DTYPES, (F, E), dev)
    _want(out["s"], "s", torch.float32, (M,), dev)
    return BwdSwigluArgs(M, D, N, E, _ptr(dOut), _ptr(W2), _ptr(o), _ptr(y), _ptr(h), _ptr(g), _ptr(r),
                         _ptr(gamma), _ptr(W1), _ptr(out["dY"]), _ptr(out["da"]), _ptr(out["dgamma"]),
                         _ptr(out["dW1"]), _ptr(out["dW2"]), _ptr(out["s"]),
                         _dt(out["da"].dtype), _dt(out["dW1"].dtype), _dt(out["dW2"].dtype))


def bwd_swiglu(dOut, W2, o, y, h, g, r, gamma, W1, da_dtype=torch.bfloat16, dW1_dtype=torch.bfloat16,
               dW2_dtype=torch.bfloat16, ws=None, out=None, unfused=False):
    """Backward of SwiGLU + output projection out = o @ W2 and of the chain under it.
    Returns dict(dY, da, dgamma, dW1, dW2, s). unfused: dO stored, then a separate
    SwiGLU-backward row kernel (coda_unfused_ref)."""
    M, E = dOut.shape
    D, N = W1.shape
    dev = dOut.device
    if out is None:
        out = {"dY": torch.empty(M, N, dtype=torch.bfloat16, device=dev),
               "da": torch.empty(M, D, dtype=da_dtype, device=dev),
               "dgamma": torch.empty(D, dtype=torch.float32, device=dev),
               "dW1": torch.empty(D, N, dtype=dW1_dtype, device=dev),
               "dW2": torch.empty(N // 2, E, dtype=dW2_dtype, device=dev),
               "s": torch.empty(M, dtype=torch.float32, device=dev)}
    a = _bwd_swiglu_args(dOut, W2, o, y, h, g, r, gamma, W1, out)
    if ws is None:
        ws = workspace(CODA_OP_UNFUSED_BWD_SWIGLU if unfused else CODA_OP_BWD_SWIGLU, M, D, N, dev)
    if unfused:
        _check(lib().coda_unfused_ref(CODA_OP_BWD_SWIGLU, ctypes.byref(a), _ptr(ws), _ws_bytes(ws, dev), _stream(dev)),
               "coda_unfused_ref(bwd_swiglu)")
    else:
        _check(lib().coda_bwd_swiglu(ctypes.byref(a), _ptr(ws), _ws_bytes(ws, dev), _stream(dev)), "coda_bwd_swiglu")
    return out


class BoundSwiglu:
    """coda_fwd_swiglu / coda_bwd_swiglu with arguments marshalled once (benchmarks)."""

    def __init__(self, kind, args, ws, keep):
        self.kind, self.args, self.ws, self._keep = kind, args, ws, keep

    def run(self, stream, unfused=False):
        if unfused:
            op = CODA_OP_FWD_SWIGLU if self.kind == "fwd" else CODA_OP_BWD_SWIGLU
            _check(lib().coda_unfused_ref(op, ctypes.byref(self.args), _ptr(self.ws), _ws_bytes(self.ws, self.ws.device), stream),
                   f"coda_unfused_ref({self.kind}_swiglu)")
            return
        fn = lib().coda_fwd_swiglu if self.kind == "fwd" else lib().coda_bwd_swiglu
        _check(fn(ctypes.byref(self.args), _ptr(self.ws), _ws_bytes(self.ws, self.ws.device), stream), f"coda_{self.kind}_swiglu")


def bind_fwd_swiglu(x, W0, z, gamma, W1, eps, out, ws):
    return BoundSwiglu("fwd", _fwd_swiglu_args(x, W0, z, gamma, W1, eps, out), ws, (x, W0, z, gamma, W1, out))


def bind_bwd_swiglu(dOut, W2, o, y, h, g, r, gamma, W1, out, ws):
    return BoundSwiglu("bwd", _bwd_swiglu_args(dOut, W2, o, y, h, g, r, gamma, W1, out), ws,
                       (dOut, W2, o, y, h, g, r, gamma, W1, out))


def _ce_fwd_args(h, W, targets, lse, loss, logits=None):
    _want(h, "h", torch.bfloat16)
    _want(W, "W", torch.bfloat16)
    M, D = h.shape
    V = W.shape[0]
    dev = h.device
    _want(h, "h", torch.bfloat16, (M, D), dev)
    _want(W, "W", torch.bfloat16, (V, D), dev)
    _want(targets, "targets", torch.int64, (M,), dev)
    _want(lse, "lse", torch.float32, (M,), dev)
    _want(loss, "loss", torch.float32, (M,), dev)
    if logits is not None:
        _want(logits, "logits", torch.float32, (M, V), dev)
    return CeFwdArgs(M, D, V, _ptr(h), _ptr(W), _ptr(targets), _ptr(lse), _ptr(loss),
                     None if logits is None else _ptr(logits))


def ce_fwd(h, W, targets, ws=None, out=None, unfused=False, store_logits=False):
    """Cross-entropy of the LM-head logits h @ W^T against targets (int64; outside [0, V) = ignored).
    Returns dict(lse, loss), both [M] fp32. unfused: the fp32 logits stored in the workspace, then
    a row kernel (coda_unfused_ref). store_logits: the epilogue also writes the fp32 logits
    (out["logits"], [M, V]) for ce_bwd(logits=...)."""
    M, D = h.shape
    V = W.shape[0]
    dev = h.device
    if out is None:
        out = {"lse": torch.empty(M, dtype=torch.float32, device=dev),
               "loss": torch.empty(M, dtype=torch.float32, device=dev)}
        if store_logits:
            out["logits"] = torch.empty(M, V, dtype=torch.float32, device=dev)
    a = _ce_fwd_args(h, W, targets, out["lse"], out["loss"], out.get("logits"))
    if ws is None:
        ws = workspace(CODA_OP_UNFUSED_CE_FWD if unfused else CODA_OP_CE_FWD, M, D, V, dev)
    if unfused:
        _check(lib().coda_unfused_ref(CODA_OP_CE_FWD, ctypes.byref(a), _ptr(ws), _ws_bytes(ws, dev), _stream(dev)),
               "coda_unfused_ref(ce_fwd)")
    else:
        _check(lib().coda_ce_fwd(ctypes.byref(a), _ptr(ws), _ws_bytes(ws, dev), _stream(dev)), "coda_ce_fwd")
    return out


def _ce_bwd_args(h, W, targets, lse, dloss, out, logits=None):
    _want(h, "h", torch.bfloat16)
    _want(W, "W", torch.bfloat16)
    M, D = h.shape
    V = W.shape[0]
    dev = h.device
    _want(h, "h", torch.bfloat16, (M, D), dev)
    _want(W, "W", torch.bfloat16, (V, D), dev)
    _want(targets, "targets", torch.int64, (M,), dev)
    _want(lse, "lse", torch.float32, (M,), dev)
    _want(dloss, "dloss", torch.float32, (M,), dev)
    _want(out["dlogits"], "dlogits", torch.bfloat16, (M, V), dev)
    _want(out["dh"], "dh", OUT_DTYPES, (M, D), dev)
    _want(out["dW"], "dW", OUT_DTYPES, (V, D), dev)
    if logits is not None:
        _want(logits, "logits", torch.float32, (M, V), dev)
    return CeBwdArgs(M, D, V, _ptr(h), _ptr(W), _ptr(targets), _ptr(lse), _ptr(dloss), _ptr(out["dlogits"]),
                     _ptr(out["dh"]), _ptr(out["dW"]), _dt(out["dh"].dtype), _dt(out["dW"].dtype),
                     None if logits is None else _ptr(logits))


def ce_bwd(h, W, targets, lse, dloss, dh_dtype=torch.bfloat16, dW_dtype=torch.bfloat16, out=None, unfused=False,
           ws=None, logits=None):
    """Backward of sum_i dloss_i loss_i: dict(dlogits [M,V] bf16, dh [M,D], dW [V,D]).
    unfused: the fp32 logits stored in a workspace, then a dlogits row kernel. logits: the
    forward's stored fp32 logits, read instead of recomputed."""
    M, D = h.shape
    V = W.shape[0]
    dev = h.device
    if out is None:
        out = {"dlogits": torch.empty(M, V, dtype=torch.bfloat16, device=dev),
               "dh": torch.empty(M, D, dtype=dh_dtype, device=dev),
               "dW": torch.empty(V, D, dtype=dW_dtype, device=dev)}
    a = _ce_bwd_args(h, W, targets, lse, dloss, out, logits)
    if unfused:
        if ws is None:
            ws = workspace(CODA_OP_UNFUSED_CE_BWD, M, D, V, dev)
        _check(lib().coda_unfused_ref(CODA_OP_CE_BWD, ctypes.byref(a), _ptr(ws), _ws_bytes(ws, dev), _stream(dev)),
               "coda_unfused_ref(ce_bwd)")
    else:
        _check(lib().coda_ce_bwd(ctypes.byref(a), _stream(dev)), "coda_ce_bwd")
    return out


class BoundCe:
    """coda_ce_fwd / coda_ce_bwd with arguments marshalled once (benchmarks)."""

    def __init__(self, kind, args, ws, keep):
        self.kind, self.args, self.ws, self._keep = kind, args, ws, keep

    def run(self, stream, unfused_ws=None):
        """unfused_ws: run coda_unfused_ref (stored fp32 logits) in that workspace instead."""
        if unfused_ws is not None:
            op = CODA_OP_CE_FWD if self.kind == "fwd" else CODA_OP_CE_BWD
            _check(lib().coda_unfused_ref(op, ctypes.byref(self.args), _ptr(unfused_ws), _ws_bytes(unfused_ws, unfused_ws.device), stream),
                   f"coda_unfused_ref(ce_{self.kind})")
        elif self.kind == "fwd":
            _check(lib().coda_ce_fwd(ctypes.byref(self.args), _ptr(self.ws), _ws_bytes(self.ws, self.ws.device), stream), "coda_ce_fwd")
        else:
            _check(lib().coda_ce_bwd(ctypes.byref(self.args), stream), "coda_ce_bwd")


def bind_ce_fwd(h, W, targets, out, ws, logits=None):
    return BoundCe("fwd", _ce_fwd_args(h, W, targets, out["lse"], out["loss"], logits), ws, (h, W, targets, out, logits))


def bind_ce_bwd(h, W, targets, lse, dloss, out, logits=None):
    return BoundCe("bwd", _ce_bwd_args(h, W, targets, lse, dloss, out, logits), None,
                   (h, W, targets, lse, dloss, out, logits))


class BoundGemm0:
    """coda_bwd_gemm0 with its arguments marshalled once (benchmarks)."""

    def __init__(self, dh, x, W0, out):
        self.args, self._keep = _bwd_gemm0_args(dh, x, W0, out["dx"], out["dW0"]), (dh, x, W0, out)

    def run(self, stream):
        _check(lib().coda_bwd_gemm0(ctypes.byref(self.args), stream), "coda_bwd_gemm0")


class Bound:
    """A forward or backward call with its arguments marshalled once, for repeated
    launches (benchmarks): .run() enqueues the whole call, .stage(i) one stage."""

    def __init__(self, kind, args, ws, keep):
        self.kind, self.args, self.ws, self._keep = kind, args, ws, keep
        self.nstages = CODA_FWD_STAGES if kind == "fwd" else CODA_BWD_STAGES

    def stage(self, i, stream):
        fn = lib().coda_fwd_stage if self.kind == "fwd" else lib().coda_bwd_stage
        _check(fn(i, ctypes.byref(self.args), _ptr(self.ws), _ws_bytes(self.ws, self.ws.device), stream), f"coda_{self.kind}_stage({i})")

    def run(self, stream, unfused=False):
        if unfused:
            op = CODA_OP_FWD if self.kind == "fwd" else CODA_OP_BWD
            _check(lib().coda_unfused_ref(op, ctypes.byref(self.args), _ptr(self.ws), _ws_bytes(self.ws, self.ws.device), stream),
                   "coda_unfused_ref")
        else:
            fn = lib().coda_fwd if self.kind == "fwd" else lib().coda_bwd
            _check(fn(ctypes.byref(self.args), _ptr(self.ws), _ws_bytes(self.ws, self.ws.device), stream), f"coda_{self.kind}")


def bind_fwd(x, W0, z, gamma, W1, eps, out, ws):
    return Bound("fwd", _fwd_args(x, W0, z, gamma, W1, eps, out["h"], out["g"], out["r"], out["y"]), ws,
                 (x, W0, z, gamma, W1, out))


def bind_bwd(dY, y, h, g, r, gamma, W1, out, ws):
    return Bound("bwd", _bwd_args(dY, y, h, g, r, gamma, W1, out["da"], out["dgamma"], out["dW1"], out["s"]), ws,
                 (dY, y, h, g, r, gamma, W1, out))


def current_stream(device="cuda:0") -> c_void_p:
    return _stream(device)


def gemm(A, B, a_layout=CODA_ROW, b_layout=CODA_ROW, out_dtype=torch.float32, M=None, N=None, K=None):
    """C[M,N] = A @ B with the shared mainloop. Layouts as in coda_layout_t."""
    _want(A, "A", torch.bfloat16)
    _want(B, "B", torch.bfloat16, device=A.device)
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    if M is None:
        M, K = (A.shape[0], A.shape[1]) if a_layout == CODA_ROW else (A.shape[1], A.shape[0])
    if N is None:
        N = B.shape[1] if b_layout == CODA_ROW else B.shape[0]
    # the logical [M, K] and [K, N] operands must lie inside the stored tensors
    a_ext = (M, K) if a_layout == CODA_ROW else (K, M)
    b_ext = (K, N) if b_layout == CODA_ROW else (N, K)
    if A.shape[0] < a_ext[0] or A.shape[1] < a_ext[1] or B.shape[0] < b_ext[0] or B.shape[1] < b_ext[1]:
        raise ValueError(f"gemm: M={M}, N={N}, K={K} exceed A {tuple(A.shape)} or B {tuple(B.shape)}")
    C = torch.empty(M, N, dtype=out_dtype, device=A.device)
    a = GemmArgs(M, N, K, _ptr(A), A.shape[1], a_layout, _ptr(B), B.shape[1], b_layout, _ptr(C), N, _dt(out_dtype))
    _check(lib().coda_gemm(ctypes.byref(a), _stream(A.device)), "coda_gemm")
    return C
