"""Python binding of libflashattn.so (exact softmax attention on MI355X).

Argument marshalling only: each function below has the name of the C entry
point it calls (see include/flash_attn.h), takes torch tensors that already
live on the GPU, passes their device pointers, sizes and the current HIP
stream, and raises :class:`FlashAttnError` on a non-zero status. Every step of
the computation runs in the library's HIP kernels; there is no fallback: if
the library is not built, the first call raises.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "FlashAttnError",
    "lib_path",
    "load_library",
    "flash_attn_fwd",
    "flash_attn_fwd_f32",
    "flash_attn_bwd",
    "flash_attn_bwd_f32",
    "flash_attn_bwd_workspace_bytes",
    "flash_attn_status_str",
    "attention_forward",
    "attention_backward",
]

_LIB = None
_HERE = os.path.dirname(os.path.abspath(__file__))


class FlashAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {flash_attn_status_str(status)} ({status})")


def lib_path() -> str:
    return os.path.join(_HERE, "libflashattn.so")


def load_library():
    """Load libflashattn.so once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -m online_softmax_flash_amd.build` "
            "(or __graft_entry__.build()) first; there is no non-HIP fallback")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.flash_attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.flash_attn_fwd.restype = I
    lib.flash_attn_fwd_f32.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.flash_attn_fwd_f32.restype = I
    lib.flash_attn_bwd.argtypes = [P] * 10 + [I, I, I, I, I, F, I, P]
    lib.flash_attn_bwd.restype = I
    lib.flash_attn_bwd_f32.argtypes = [P] * 10 + [I, I, I, I, I, F, I, P]
    lib.flash_attn_bwd_f32.restype = I
    lib.flash_attn_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.flash_attn_bwd_workspace_bytes.restype = Z
    lib.flash_attn_status_str.argtypes = [I]
    lib.flash_attn_status_str.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def flash_attn_status_str(status: int) -> str:
    return load_library().flash_attn_status_str(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(*tensors, dtype=None):
    import torch
    for t in tensors:
        if not isinstance(t, torch.Tensor):
            raise TypeError("expected torch tensors")
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"expected dtype {dtype}, got {t.dtype}")


def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, Hq, N, d = q.shape
    return int(B), int(Hq), int(k.shape[1]), int(N), int(d)


def _fwd(name, dt, q, k, v, o, lse, scale, causal, stream):
    import torch
    _check(q, k, v, o, dtype=dt)
    _check(lse, dtype=torch.float32)
    B, Hq, Hkv, N, d = _dims(q, k)
    st = getattr(load_library(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       B, Hq, Hkv, N, d, float(scale), int(bool(causal)), _stream(stream))
    if st != 0:
        raise FlashAttnError(name, st)


def flash_attn_fwd(q, k, v, o, lse, scale, causal, stream=None):
    """bf16 forward into caller-allocated o [B,Hq,N,d] (bf16) and lse [B,Hq,N] (fp32)."""
    import torch
    _fwd("flash_attn_fwd", torch.bfloat16, q, k, v, o, lse, scale, causal, stream)


def flash_attn_fwd_f32(q, k, v, o, lse, scale, causal, stream=None):
    """fp32 check-mode forward into caller-allocated o (fp32) and lse (fp32)."""
    import torch
    _fwd("flash_attn_fwd_f32", torch.float32, q, k, v, o, lse, scale, causal, stream)


def flash_attn_bwd_workspace_bytes(B, Hq, Hkv, N, d) -> int:
    return int(load_library().flash_attn_bwd_workspace_bytes(int(B), int(Hq), int(Hkv), int(N), int(d)))


def _bwd(name, dt, q, k, v, o, lse, dout, dq, dk, dv, workspace, scale, causal, stream):
    import torch
    _check(q, k, v, o, dout, dq, dk, dv, dtype=dt)
    _check(lse, dtype=torch.float32)
    _check(workspace)
    B, Hq, Hkv, N, d = _dims(q, k)
    need = flash_attn_bwd_workspace_bytes(B, Hq, Hkv, N, d)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace too small: need {need} bytes")
    st = getattr(load_library(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                       B, Hq, Hkv, N, d, float(scale), int(bool(causal)), _stream(stream))
    if st != 0:
        raise FlashAttnError(name, st)


def flash_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale, causal, stream=None):
    """bf16 backward into caller-allocated dq, dk, dv (bf16); workspace is a device buffer."""
    import torch
    _bwd("flash_attn_bwd", torch.bfloat16, q, k, v, o, lse, dout, dq, dk, dv, workspace, scale, causal, stream)


def flash_attn_bwd_f32(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale, causal, stream=None):
    """fp32 check-mode backward."""
    import torch
    _bwd("flash_attn_bwd_f32", torch.float32, q, k, v, o, lse, dout, dq, dk, dv, workspace, scale, causal,
         stream)


def attention_forward(q, k, v, scale, causal, stream=None):
    """Allocate o and lse with torch and run the forward of q's dtype (bf16 or fp32)."""
    import torch
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if q.dtype == torch.bfloat16:
        flash_attn_fwd(q, k, v, o, lse, scale, causal, stream)
    elif q.dtype == torch.float32:
        flash_attn_fwd_f32(q, k, v, o, lse, scale, causal, stream)
    else:
        raise ValueError("q must be bfloat16 or float32")
    return o, lse


def attention_backward(q, k, v, o, lse, dout, scale, causal, stream=None):
    """Allocate dq, dk, dv and the workspace with torch and run the backward."""
    import torch
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, Hq, Hkv, N, d = _dims(q, k)
    ws = torch.empty(max(flash_attn_bwd_workspace_bytes(B, Hq, Hkv, N, d), 256), dtype=torch.uint8,
                     device=q.device)
    fn = flash_attn_bwd if q.dtype == torch.bfloat16 else flash_attn_bwd_f32
    fn(q, k, v, o, lse, dout, dq, dk, dv, ws, scale, causal, stream)
    return dq, dk, dv
