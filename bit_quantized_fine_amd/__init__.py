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
QLORA_ERR_SCRATCH = 7
QLORA_ERR_FORMAT = 8
CODEBOOKS = {"nf4": 0, "int4": 1, "fp4": 2}   # qlora_codebook of the header
NOALLOC_SCRATCH_BYTES = 32 << 20   # QLORA_NOALLOC_SCRATCH_BYTES of the header
_lib = None


class _Nf4Weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("absmax_q", ctypes.c_void_p),
                ("absmax_scale", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64)]


class _Q4Weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("absmax_q", ctypes.c_void_p),
                ("absmax_scale", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("codebook", ctypes.c_int32),
                ("double_quant", ctypes.c_int32)]


class _AdamWConfig(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


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
    "qlora_linear_fwd_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64,
                                                ctypes.POINTER(_Nf4Weight), ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                                ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p]),
    "qlora_linear_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64,
                                                           ctypes.c_int64, ctypes.c_int]),
    "qlora_linear_bwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.POINTER(_Nf4Weight), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]),
    "qlora_block_fwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int,
                                                          ctypes.c_int64, ctypes.c_int64,
                                                          ctypes.c_int]),
    "qlora_block_fwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(_Nf4Weight),
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]),
    "qlora_block_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int,
                                                          ctypes.c_int64, ctypes.c_int64,
                                                          ctypes.c_int]),
    "qlora_block_bwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.POINTER(_Nf4Weight), ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]),
    "qlora_lora16_fwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64,
                                                           ctypes.c_int64, ctypes.c_int]),
    "qlora_lora16_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64,
                                                           ctypes.c_int64, ctypes.c_int]),
    "qlora_lora16_fwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]),
    "qlora_lora16_bwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]),
    "qlora_q4_levels": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p]),
    "qlora_q4_thresholds": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p]),
    "qlora_q4_scale_count": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]),
    "qlora_q4_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "qlora_q4_dequantize": (ctypes.c_int, [ctypes.POINTER(_Q4Weight), ctypes.c_void_p,
                                           ctypes.c_void_p]),
    "qlora_q4_linear_fwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.POINTER(_Q4Weight), ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p]),
    "qlora_q4_linear_bwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.POINTER(_Q4Weight), ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p]),
    "qlora_adamw_step": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.POINTER(_AdamWConfig), ctypes.c_int64,
                                        ctypes.c_void_p]),
    "qlora_paged_state_create": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int,
                                                ctypes.POINTER(ctypes.c_void_p)]),
    "qlora_paged_state_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "qlora_paged_state_page_out": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "qlora_paged_state_page_in": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "qlora_paged_state_pointers": (ctypes.c_int, [ctypes.c_void_p,
                                                  ctypes.POINTER(ctypes.c_void_p),
                                                  ctypes.POINTER(ctypes.c_void_p)]),
    "qlora_paged_state_resident": (ctypes.c_int, [ctypes.c_void_p]),
    "qlora_paged_state_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]),
    "qlora_paged_state_write": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p]),
    "qlora_probe_hbm_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_void_p]),
    "qlora_probe_mfma_bf16": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
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
    if out is not None and (out.N, out.K) != (N, K):
        raise ValueError(f"out is a {out.N} x {out.K} weight, W is {N} x {K}")
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


def _fwd(fn, X, w, wt, cw, A, B, s, Y, T, workspace):
    """Marshal a forward call: fn is the C entry point's name, wt the weight's
    tensors (checked), cw its C struct."""
    import torch
    M = X.shape[0]
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
    _check(fn, getattr(lib(), fn)(_ptr(X), M, ctypes.byref(cw), _ptr(A), _ptr(B), r, float(s),
                                  _ptr(Y), _ptr(T), _ptr(workspace), need, _stream(X)))
    return Y, T


def _x_rows(X, K):
    import torch
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    _need(X, "X", (X.shape[0], K), torch.bfloat16)
    return X.shape[0]


def qlora_linear_fwd(X, w: NF4Weight, A=None, B=None, s: float = 1.0,
                     Y=None, T=None, workspace=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Y = X . deq(W)^T + s . (X . A) . B.  Returns (Y bf16 [M,N], T fp32 [M,r])."""
    _x_rows(X, w.K)
    return _fwd("qlora_linear_fwd", X, w, _check_weight(w), w._c(), A, B, s, Y, T, workspace)


def qlora_linear_fwd_noalloc(X, w: NF4Weight, A=None, B=None, s: float = 1.0,
                             Y=None, T=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """qlora_linear_fwd on the library's fixed per-GPU scratch instead of a
    workspace (for callers that cannot allocate device memory; pass Y and T
    to keep this call allocation-free on the Python side too).  Calls that
    overlap on one GPU race on that scratch."""
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
    _on_gpu([("X", X)] + wt + [("A", A), ("B", B), ("Y", Y), ("T", T if r > 0 else None)])
    if Y is None:
        Y = torch.empty((M, w.N), dtype=torch.bfloat16, device=X.device)
    if T is None and r > 0:
        T = torch.empty((M, r), dtype=torch.float32, device=X.device)
    cw = w._c()
    _check("qlora_linear_fwd_noalloc",
           lib().qlora_linear_fwd_noalloc(_ptr(X), M, ctypes.byref(cw), _ptr(A), _ptr(B), r,
                                          float(s), _ptr(Y), _ptr(T), _stream(X)))
    return Y, T


def _bwd(fn, dY, X, w, wt, cw, A, B, s, T, need_dx, dX, dA, dB, workspace):
    """Marshal a backward call (as _fwd)."""
    import torch
    M = X.shape[0]
    _need(dY, "dY", (M, w.N), torch.bfloat16)
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
    _check(fn, getattr(lib(), fn)(_ptr(dY), _ptr(X), M, ctypes.byref(cw), _ptr(A), _ptr(B), r,
                                  float(s), _ptr(T), _ptr(dX if need_dx else None), _ptr(dA),
                                  _ptr(dB), _ptr(workspace), need, _stream(X)))
    return (dX if need_dx else None), dA, dB


def qlora_linear_bwd(dY, X, w: NF4Weight, A=None, B=None, s: float = 1.0, T=None,
                     need_dx: bool = True, dX=None, dA=None, dB=None, workspace=None):
    """Returns (dX bf16 [M,K] or None, dA bf16 [K,r], dB bf16 [r,N]).

    T is the forward's T = X . A; None recomputes it (gradient checkpointing).
    """
    _x_rows(X, w.K)
    return _bwd("qlora_linear_bwd", dY, X, w, _check_weight(w), w._c(), A, B, s, T, need_dx,
                dX, dA, dB, workspace)


class Q4Weight(NamedTuple):
    """A 4-bit weight of any codebook: with double quantization the NF4
    format's constants, else absmax_q is None and absmax_scale holds one
    fp32 absmax per 64-block."""
    codes: "torch.Tensor"                    # uint8 [N*K/2]
    absmax_q: Optional["torch.Tensor"]       # uint8 [N*K/64], or None
    absmax_scale: "torch.Tensor"             # float32 [ceil(N*K/16384)] or [N*K/64]
    N: int
    K: int
    codebook: str                            # "nf4", "int4" or "fp4"
    double_quant: bool

    def _c(self) -> _Q4Weight:
        return _Q4Weight(self.codes.data_ptr(),
                         self.absmax_q.data_ptr() if self.absmax_q is not None else None,
                         self.absmax_scale.data_ptr(), self.N, self.K,
                         CODEBOOKS[self.codebook], int(self.double_quant))

    def nbytes(self) -> int:
        return (self.codes.numel() + (self.absmax_q.numel() if self.absmax_q is not None else 0)
                + 4 * self.absmax_scale.numel())


def _codebook_id(codebook: str) -> int:
    if codebook not in CODEBOOKS:
        raise ValueError(f"codebook must be one of {sorted(CODEBOOKS)}, got {codebook!r}")
    return CODEBOOKS[codebook]


def _check_q4_weight(w: Q4Weight):
    import torch
    _codebook_id(w.codebook)
    n_codes, n_blocks = w.N * w.K // 2, w.N * w.K // 64
    _need(w.codes, "w.codes", (n_codes,), torch.uint8)
    if w.double_quant:
        _need(w.absmax_q, "w.absmax_q", (n_blocks,), torch.uint8)
        _need(w.absmax_scale, "w.absmax_scale", ((n_blocks + 255) // 256,), torch.float32)
    else:
        _need(w.absmax_scale, "w.absmax_scale", (n_blocks,), torch.float32)
    return [("w.codes", w.codes), ("w.absmax_q", w.absmax_q),
            ("w.absmax_scale", w.absmax_scale)]


def qlora_q4_levels(codebook: str = "nf4"):
    """The 16 levels of a codebook (list of float)."""
    buf = (ctypes.c_float * 16)()
    _check("qlora_q4_levels", lib().qlora_q4_levels(_codebook_id(codebook), buf))
    return list(buf)


def qlora_q4_thresholds(codebook: str = "nf4"):
    """The 15 quantizer thresholds of a codebook (code = #{j : x > t_j})."""
    buf = (ctypes.c_float * 15)()
    _check("qlora_q4_thresholds", lib().qlora_q4_thresholds(_codebook_id(codebook), buf))
    return list(buf)


def qlora_q4_quantize(W, codebook: str = "nf4", double_quant: bool = True) -> Q4Weight:
    """Quantize a float32 [N, K] CUDA tensor with a codebook ("nf4", "int4",
    "fp4"), with double-quantized or fp32 block constants."""
    import torch
    cb = _codebook_id(codebook)
    if W.dim() != 2:
        raise ValueError("W must be [N, K]")
    N, K = W.shape
    _need(W, "W", (N, K), torch.float32)
    _on_gpu([("W", W)])
    L = lib()
    dq = bool(double_quant)
    out = Q4Weight(
        torch.empty(L.qlora_nf4_codes_bytes(N, K), dtype=torch.uint8, device=W.device),
        torch.empty(L.qlora_nf4_absmax_q_bytes(N, K), dtype=torch.uint8, device=W.device)
        if dq else None,
        torch.empty(L.qlora_q4_scale_count(N, K, int(dq)), dtype=torch.float32, device=W.device),
        N, K, codebook, dq)
    _check("qlora_q4_quantize",
           L.qlora_q4_quantize(_ptr(W), N, K, cb, int(dq), _ptr(out.codes), _ptr(out.absmax_q),
                               _ptr(out.absmax_scale), _stream(W)))
    return out


def qlora_q4_dequantize(w: Q4Weight):
    """bf16 [N, K] dequantized copy of a 4-bit weight."""
    import torch
    _on_gpu(_check_q4_weight(w))
    out = torch.empty((w.N, w.K), dtype=torch.bfloat16, device=w.codes.device)
    cw = w._c()
    _check("qlora_q4_dequantize",
           lib().qlora_q4_dequantize(ctypes.byref(cw), _ptr(out), _stream(out)))
    return out


def qlora_q4_linear_fwd(X, w: Q4Weight, A=None, B=None, s: float = 1.0, Y=None, T=None,
                        workspace=None):
    """qlora_linear_fwd for a weight of any codebook and constant format."""
    _x_rows(X, w.K)
    return _fwd("qlora_q4_linear_fwd", X, w, _check_q4_weight(w), w._c(), A, B, s, Y, T,
                workspace)


def qlora_q4_linear_bwd(dY, X, w: Q4Weight, A=None, B=None, s: float = 1.0, T=None,
                        need_dx: bool = True, dX=None, dA=None, dB=None, workspace=None):
    """qlora_linear_bwd for a weight of any codebook and constant format."""
    _x_rows(X, w.K)
    return _bwd("qlora_q4_linear_bwd", dY, X, w, _check_q4_weight(w), w._c(), A, B, s, T,
                need_dx, dX, dA, dB, workspace)


def _addr(x):
    """A torch tensor's data pointer, or an int address as it is."""
    return ctypes.c_void_p(x if isinstance(x, int) else x.data_ptr())


def qlora_adamw_step(param, grad, exp_avg, exp_avg_sq, step: int, lr: float = 2e-4,
                     beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                     weight_decay: float = 0.0):
    """One AdamW step, in place: param (bf16, 1-D) and the fp32 moments.
    exp_avg / exp_avg_sq are fp32 tensors on param's GPU, or device-visible
    addresses (ints) such as PagedState.pointers() gives."""
    import torch
    if param.dim() != 1:
        raise ValueError("param must be a flat [n] tensor (adapters as slices of one buffer)")
    n = param.numel()
    _need(param, "param", (n,), torch.bfloat16)
    _need(grad, "grad", (n,), torch.bfloat16)
    named = [("param", param), ("grad", grad)]
    for name, t in (("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        if not isinstance(t, int):
            _need(t, name, (n,), torch.float32)
            named.append((name, t))
    _on_gpu(named)
    cfg = _AdamWConfig(lr, beta1, beta2, eps, weight_decay)
    _check("qlora_adamw_step",
           lib().qlora_adamw_step(_ptr(param), _ptr(grad), _addr(exp_avg), _addr(exp_avg_sq), n,
                                  ctypes.byref(cfg), int(step), _stream(param)))


class PagedState:
    """The library's paged optimizer state for n parameters: fp32 moments in
    HBM while resident, in pinned host memory (read and written by the GPU
    directly) when paged out."""

    def __init__(self, n: int, on_host: bool = False):
        h = ctypes.c_void_p()
        _check("qlora_paged_state_create",
               lib().qlora_paged_state_create(int(n), int(bool(on_host)), ctypes.byref(h)))
        self._h, self.n = h, int(n)

    def close(self):
        if self._h:
            _check("qlora_paged_state_destroy", lib().qlora_paged_state_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _stream(self):
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def page_out(self):
        _check("qlora_paged_state_page_out",
               lib().qlora_paged_state_page_out(self._h, self._stream()))

    def page_in(self):
        _check("qlora_paged_state_page_in",
               lib().qlora_paged_state_page_in(self._h, self._stream()))

    @property
    def resident(self) -> bool:
        return bool(lib().qlora_paged_state_resident(self._h))

    def pointers(self):
        """(exp_avg, exp_avg_sq) device-visible addresses of the current copy."""
        m, v = ctypes.c_void_p(), ctypes.c_void_p()
        _check("qlora_paged_state_pointers",
               lib().qlora_paged_state_pointers(self._h, ctypes.byref(m), ctypes.byref(v)))
        return m.value, v.value

    def read(self, out=None):
        """The moments as a [2, n] fp32 tensor (m, v) on the current GPU."""
        import torch
        if out is None:
            out = torch.empty((2, self.n), dtype=torch.float32, device="cuda")
        _need(out, "out", (2, self.n), torch.float32)
        _check("qlora_paged_state_read",
               lib().qlora_paged_state_read(self._h, _ptr(out), self._stream()))
        return out

    def write(self, src):
        """Set the moments from a [2, n] fp32 tensor (m, v)."""
        import torch
        _need(src, "src", (2, self.n), torch.float32)
        _check("qlora_paged_state_write",
               lib().qlora_paged_state_write(self._h, _ptr(src), self._stream()))

    def step(self, param, grad, step: int, **hp):
        m, v = self.pointers()
        qlora_adamw_step(param, grad, m, v, step, **hp)


class _Shape(NamedTuple):
    N: int
    K: int


def _dense_weight(W):
    import torch
    if W.dim() != 2:
        raise ValueError("W must be [N, K]")
    _need(W, "W", tuple(W.shape), torch.bfloat16)
    return _Shape(int(W.shape[0]), int(W.shape[1]))


def qlora_lora16_fwd(X, W, A=None, B=None, s: float = 1.0, Y=None, T=None, workspace=None):
    """16-bit LoRA forward on the same kernels: Y = X . W^T + s . (X . A) . B
    with a bf16 base weight W [N, K].  Returns (Y bf16 [M,N], T fp32 [M,r])."""
    import torch
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    w = _dense_weight(W)
    M = X.shape[0]
    _need(X, "X", (M, w.K), torch.bfloat16)
    r = _check_adapters(A, B, w)
    if Y is not None:
        _need(Y, "Y", (M, w.N), torch.bfloat16)
    if T is not None and r > 0:
        _need(T, "T", (M, r), torch.float32)
    if workspace is not None:
        _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
    _on_gpu([("X", X), ("W", W), ("A", A), ("B", B), ("Y", Y), ("T", T if r > 0 else None),
             ("workspace", workspace)])
    dev = X.device
    if Y is None:
        Y = torch.empty((M, w.N), dtype=torch.bfloat16, device=dev)
    if T is None and r > 0:
        T = torch.empty((M, r), dtype=torch.float32, device=dev)
    need = lib().qlora_lora16_fwd_workspace_bytes(M, w.N, w.K, r)
    if workspace is None or workspace.numel() < need:
        workspace = _ws(need, dev)
    _check("qlora_lora16_fwd",
           lib().qlora_lora16_fwd(_ptr(X), M, _ptr(W), w.N, w.K, _ptr(A), _ptr(B), r, float(s),
                                  _ptr(Y), _ptr(T), _ptr(workspace), need, _stream(X)))
    return Y, T


def qlora_lora16_bwd(dY, X, W, A=None, B=None, s: float = 1.0, T=None, need_dx: bool = True,
                     dX=None, dA=None, dB=None, workspace=None):
    """16-bit LoRA backward: (dX bf16 [M,K] or None, dA bf16 [K,r], dB bf16
    [r,N]) with a bf16 base weight W [N, K]; T None recomputes X . A."""
    import torch
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    w = _dense_weight(W)
    M = X.shape[0]
    _need(X, "X", (M, w.K), torch.bfloat16)
    _need(dY, "dY", (M, w.N), torch.bfloat16)
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
    _on_gpu([("X", X), ("dY", dY), ("W", W), ("A", A), ("B", B), ("T", T if r > 0 else None),
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
    need = lib().qlora_lora16_bwd_workspace_bytes(M, w.N, w.K, r)
    if workspace is None or workspace.numel() < need:
        workspace = _ws(need, dev)
    _check("qlora_lora16_bwd",
           lib().qlora_lora16_bwd(_ptr(dY), _ptr(X), M, _ptr(W), w.N, w.K, _ptr(A), _ptr(B), r,
                                  float(s), _ptr(T), _ptr(dX if need_dx else None), _ptr(dA),
                                  _ptr(dB), _ptr(workspace), need, _stream(X)))
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


def _check_block_adapters(A, B, w, S):
    import torch
    if A is None or B is None or A.dim() != 2:
        raise ValueError("A [K, S*r] and B [r, S*nseg] are required")
    if A.shape[1] % S:
        raise ValueError(f"A has {A.shape[1]} columns, not a multiple of S = {S}")
    r = A.shape[1] // S
    _need(A, "A", (w.K, S * r), torch.bfloat16)
    _need(B, "B", (r, w.N), torch.bfloat16)
    return r


def qlora_block_fwd(X, w: NF4Weight, S: int, A, B, s: float = 1.0, Y=None, T=None,
                    workspace=None):
    """S projections sharing X, stacked along N in w: returns Y [M, S*nseg]
    (projection j in columns j*nseg ..) and T [M, S*r]."""
    import torch
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    M = X.shape[0]
    _need(X, "X", (M, w.K), torch.bfloat16)
    wt = _check_weight(w)
    if S < 1 or w.N % S:
        raise ValueError(f"w.N = {w.N} is not a multiple of S = {S}")
    r = _check_block_adapters(A, B, w, S)
    nseg = w.N // S
    if Y is not None:
        _need(Y, "Y", (M, w.N), torch.bfloat16)
    if T is not None:
        _need(T, "T", (M, S * r), torch.float32)
    _on_gpu([("X", X)] + wt + [("A", A), ("B", B), ("Y", Y), ("T", T), ("workspace", workspace)])
    if Y is None:
        Y = torch.empty((M, w.N), dtype=torch.bfloat16, device=X.device)
    if T is None:
        T = torch.empty((M, S * r), dtype=torch.float32, device=X.device)
    need = lib().qlora_block_fwd_workspace_bytes(M, S, nseg, w.K, r)
    if workspace is None or workspace.numel() < need:
        workspace = _ws(need, X.device)
    cw = w._c()
    _check("qlora_block_fwd",
           lib().qlora_block_fwd(_ptr(X), M, ctypes.byref(cw), S, _ptr(A), _ptr(B), r, float(s),
                                 _ptr(Y), _ptr(T), _ptr(workspace), need, _stream(X)))
    return Y, T


def qlora_block_bwd(dY, X, w: NF4Weight, S: int, A, B, s: float = 1.0, T=None,
                    need_dx: bool = True, dX=None, dA=None, dB=None, workspace=None):
    """Backward of the fused block: (dX [M, K] summed over the projections or
    None, dA [K, S*r], dB [r, S*nseg])."""
    import torch
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    M = X.shape[0]
    _need(X, "X", (M, w.K), torch.bfloat16)
    _need(dY, "dY", (M, w.N), torch.bfloat16)
    wt = _check_weight(w)
    if S < 1 or w.N % S:
        raise ValueError(f"w.N = {w.N} is not a multiple of S = {S}")
    r = _check_block_adapters(A, B, w, S)
    nseg = w.N // S
    if T is not None:
        _need(T, "T", (M, S * r), torch.float32)
    _on_gpu([("X", X), ("dY", dY)] + wt + [("A", A), ("B", B), ("T", T)])
    dev = X.device
    if need_dx and dX is None:
        dX = torch.empty((M, w.K), dtype=torch.bfloat16, device=dev)
    if dA is None:
        dA = torch.empty((w.K, S * r), dtype=torch.bfloat16, device=dev)
    if dB is None:
        dB = torch.empty((r, w.N), dtype=torch.bfloat16, device=dev)
    need = lib().qlora_block_bwd_workspace_bytes(M, S, nseg, w.K, r)
    if workspace is None or workspace.numel() < need:
        workspace = _ws(need, dev)
    cw = w._c()
    _check("qlora_block_bwd",
           lib().qlora_block_bwd(_ptr(dY), _ptr(X), M, ctypes.byref(cw), S, _ptr(A), _ptr(B), r,
                                 float(s), _ptr(T), _ptr(dX if need_dx else None), _ptr(dA),
                                 _ptr(dB), _ptr(workspace), need, _stream(X)))
    return (dX if need_dx else None), dA, dB


def qlora_probe_hbm_read(buf, workgroups: int, sink):
    """Enqueue one streaming read of the uint8 device tensor buf."""
    _check("qlora_probe_hbm_read",
           lib().qlora_probe_hbm_read(_ptr(buf), buf.numel(), _ptr(sink), workgroups,
                                      _stream(buf)))


def qlora_probe_mfma_bf16(iters: int, workgroups: int, sink):
    """Enqueue the bf16 MFMA loop; returns its flop count."""
    _check("qlora_probe_mfma_bf16",
           lib().qlora_probe_mfma_bf16(iters, workgroups, _ptr(sink), _stream(sink)))
    return workgroups * 4 * iters * 8 * 32768


PROFILE_FAMILIES = {0: "fwd_gemm", 1: "dx_gemm", 2: "fwd_decode", 3: "quantize", 4: "rank"}
