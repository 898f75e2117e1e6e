"""Python binding of libqlora_nf4, the gfx950 QLoRA NF4 linear-layer library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory (outputs and workspaces are allocated
here with torch.empty) and the current stream.  The functions carry the names
of the C entry points in include/qlora_nf4.h.

If the shared library has not been built, every entry point raises; there is
no fallback implementation.
"""
import ctypes
import os
from typing import NamedTuple, Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora_nf4.so")

QLORA_OK = 0
_lib = None


class _Nf4Weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("absmax_q", ctypes.c_void_p),
                ("absmax_scale", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64)]


_SIGS = {
    "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_version": (ctypes.c_char_p, []),
    "qlora_nf4_levels": (ctypes.c_int, [ctypes.c_void_p]),
    "qlora_nf4_thresholds": (ctypes.c_int, [ctypes.c_void_p]),
    "qlora_nf4_codes_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "qlora_nf4_absmax_q_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "qlora_nf4_scale_count": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "qlora_nf4_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p]),
    "qlora_nf4_dequantize": (ctypes.c_int, [ctypes.POINTER(_Nf4Weight), ctypes.c_void_p,
                                            ctypes.c_void_p]),
    "qlora_linear_fwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64,
                                                           ctypes.c_int64, ctypes.c_int]),
    "qlora_linear_fwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.POINTER(_Nf4Weight), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]),
    "qlora_linear_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64,
                                                           ctypes.c_int64, ctypes.c_int]),
    "qlora_linear_bwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.POINTER(_Nf4Weight), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]),
    "qlora_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "qlora_profile_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int64)]),
    "qlora_profile_reset": (ctypes.c_int, []),
}

EXPORTED = tuple(_SIGS)


def lib():
    """Load libqlora_nf4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_fine_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().qlora_status_string(status).decode()


class QloraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")
        self.status = status


def _check(fn: str, status: int):
    if status != QLORA_OK:
        raise QloraError(fn, status)


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, dtype):
    """The C entry points trust their pointers to hold the documented
    [rows, cols] layout, so tensors are checked here before a call: first
    dtype, shape and contiguity of every argument, then (_on_gpu) that all
    of them sit on the same GPU."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(named):
    """named: (name, tensor or None) pairs; the first tensor's GPU is the one."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _check_weight(w):
    import torch
    n_codes, n_blocks = w.N * w.K // 2, w.N * w.K // 64
    _need(w.codes, "w.codes", (n_codes,), torch.uint8)
    _need(w.absmax_q, "w.absmax_q", (n_blocks,), torch.uint8)
    _need(w.absmax_scale, "w.absmax_scale", ((n_blocks + 255) // 256,), torch.float32)
    return [("w.codes", w.codes), ("w.absmax_q", w.absmax_q),
            ("w.absmax_scale", w.absmax_scale)]


def _check_adapters(A, B, w):
    import torch
    if A is None or B is None:
        if A is not None or B is not None:
            raise ValueError("A and B go together (both None selects r = 0)")
        return 0
    if A.dim() != 2:
        raise ValueError("A must be [K, r]")
    r = A.shape[1]
    _need(A, "A", (w.K, r), torch.bfloat16)
    _need(B, "B", (r, w.N), torch.bfloat16)
    return r


class NF4Weight(NamedTuple):
    codes: "torch.Tensor"          # uint8 [N*K/2]
    absmax_q: "torch.Tensor"       # uint8 [N*K/64]
    absmax_scale: "torch.Tensor"   # float32 [ceil(N*K/16384)]
    N: int
    K: int

    def _c(self) -> _Nf4Weight:
        return _Nf4Weight(self.codes.data_ptr(), self.absmax_q.data_ptr(),
                          self.absmax_scale.data_ptr(), self.N, self.K)

    def nbytes(self) -> int:
        return (self.codes.numel() + self.absmax_q.numel()
                + 4 * self.absmax_scale.numel())


def qlora_nf4_levels():
    """The 16 NF4 levels (list of float)."""
    buf = (ctypes.c_float * 16)()
    _check("qlora_nf4_levels", lib().qlora_nf4_levels(buf))
    return list(buf)


def qlora_nf4_thresholds():
    buf = (ctypes.c_float * 15)()
    _check("qlora_nf4_thresholds", lib().qlora_nf4_thresholds(buf))
    return list(buf)


def qlora_nf4_quantize(W, out: Optional[NF4Weight] = None) -> NF4Weight:
    """Quantize a float32 [N, K] CUDA tensor to NF4 + double-quantized constants."""
    import torch
    if W.dim() != 2:
        raise ValueError("W must be [N, K]")
    N, K = W.shape
    _need(W, "W", (N, K), torch.float32)
    _on_gpu([("W", W)] + (_check_weight(out) if out is not None else []))
    L = lib()
    if out is None:
        out = NF4Weight(
            torch.empty(L.qlora_nf4_codes_bytes(N, K), dtype=torch.uint8, device=W.device),
            torch.empty(L.qlora_nf4_absmax_q_bytes(N, K), dtype=torch.uint8, device=W.device),
            torch.empty(L.qlora_nf4_scale_count(N, K), dtype=torch.float32, device=W.device),
            N, K)
    _check("qlora_nf4_quantize",
           L.qlora_nf4_quantize(_ptr(W), N, K, _ptr(out.codes), _ptr(out.absmax_q),
                                _ptr(out.absmax_scale), _stream(W)))
    return out


def qlora_nf4_dequantize(w: NF4Weight):
    """bf16 [N, K] dequantized copy of an NF4 weight."""
    import torch
    _on_gpu(_check_weight(w))
    out = torch.empty((w.N, w.K), dtype=torch.bfloat16, device=w.codes.device)
    cw = w._c()
    _check("qlora_nf4_dequantize",
           lib().qlora_nf4_dequantize(ctypes.byref(cw), _ptr(out), _stream(out)))
    return out


def _ws(nbytes: int, device):
    import torch
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def qlora_linear_fwd(X, w: NF4Weight, A=None, B=None, s: float = 1.0,
                     Y=None, T=None, workspace=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Y = X . deq(W)^T + s . (X . A) . B.  Returns (Y bf16 [M,N], T fp32 [M,r])."""
    import torch
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    M = X.shape[0]
    _need(X, "X", (M, w.K), torch.bfloat16)
    wt = _check_weight(w)
    r = _check_adapters(A, B, w)
    if Y is not None:
        _need(Y, "Y", (M, w.N), torch.bfloat16)
    if T is not None and r > 0:
        _need(T, "T", (M, r), torch.float32)
    if workspace is not None:
        _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
    _on_gpu([("X", X)] + wt + [("A", A), ("B", B), ("Y", Y), ("T", T if r > 0 else None),
                               ("workspace", workspace)])
    dev = X.device
    if Y is None:
        Y = torch.empty((M, w.N), dtype=torch.bfloat16, device=dev)
    if T is None and r > 0:
        T = torch.empty((M, r), dtype=torch.float32, device=dev)
    need = lib().qlora_linear_fwd_workspace_bytes(M, w.N, w.K, r)
    if workspace is None or workspace.numel() < need:
        workspace = _ws(need, X.device)
    cw = w._c()
    _check("qlora_linear_fwd",
           lib().qlora_linear_fwd(_ptr(X), M, ctypes.byref(cw), _ptr(A), _ptr(B), r,
                                  float(s), _ptr(Y), _ptr(T), _ptr(workspace), need,
                                  _stream(X)))
    return Y, T


def qlora_linear_bwd(dY, X, w: NF4Weight, A=None, B=None, s: float = 1.0, T=None,
                     need_dx: bool = True, dX=None, dA=None, dB=None, workspace=None):
    """Returns (dX bf16 [M,K] or None, dA bf16 [K,r], dB bf16 [r,N]).

    T is the forward's T = X . A; None recomputes it (gradient checkpointing).
    """
    import torch
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    M = X.shape[0]
    _need(X, "X", (M, w.K), torch.bfloat16)
    _need(dY, "dY", (M, w.N), torch.bfloat16)
    wt = _check_weight(w)
    r = _check_adapters(A, B, w)
    if T is not None and r > 0:
        _need(T, "T", (M, r), torch.float32)
    if need_dx and dX is not None:
        _need(dX, "dX", (M, w.K), torch.bfloat16)
    if r > 0 and dA is not None:
        _need(dA, "dA", (w.K, r), torch.bfloat16)
    if r > 0 and dB is not None:
        _need(dB, "dB", (r, w.N), torch.bfloat16)
    if workspace is not None:
        _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
    _on_gpu([("X", X), ("dY", dY)] + wt +
            [("A", A), ("B", B), ("T", T if r > 0 else None),
             ("dX", dX if need_dx else None), ("dA", dA if r > 0 else None),
             ("dB", dB if r > 0 else None), ("workspace", workspace)])
    dev = X.device
    if need_dx and dX is None:
        dX = torch.empty((M, w.K), dtype=torch.bfloat16, device=dev)
    if r > 0:
        if dA is None:
            dA = torch.empty((w.K, r), dtype=torch.bfloat16, device=dev)
        if dB is None:
            dB = torch.empty((r, w.N), dtype=torch.bfloat16, device=dev)
    need = lib().qlora_linear_bwd_workspace_bytes(M, w.N, w.K, r)
    if workspace is None or workspace.numel() < need:
        workspace = _ws(need, dev)
    cw = w._c()
    _check("qlora_linear_bwd",
           lib().qlora_linear_bwd(_ptr(dY), _ptr(X), M, ctypes.byref(cw), _ptr(A), _ptr(B),
                                  r, float(s), _ptr(T), _ptr(dX if need_dx else None),
                                  _ptr(dA), _ptr(dB), _ptr(workspace), need, _stream(X)))
    return (dX if need_dx else None), dA, dB


def qlora_profile_enable(enable: bool = True):
    _check("qlora_profile_enable", lib().qlora_profile_enable(int(enable)))


def qlora_profile_reset():
    _check("qlora_profile_reset", lib().qlora_profile_reset())


def qlora_profile_read(family: int):
    """(total milliseconds, launches) of a timed kernel family."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check("qlora_profile_read", lib().qlora_profile_read(family, ctypes.byref(ms),
                                                           ctypes.byref(n)))
    return ms.value, n.value


PROFILE_FAMILIES = {0: "fwd_gemm", 1: "dx_gemm", 2: "fwd_decode", 3: "quantize", 4: "rank"}
