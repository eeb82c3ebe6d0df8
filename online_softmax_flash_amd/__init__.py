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
    "flash_attn_fwd_kv",
    "flash_attn_fwd_varlen",
    "flash_attn_fwd_kv_noalloc",
    "flash_attn_fwd_kv_num_splits",
    "flash_attn_fwd_kv_workspace_bytes",
    "attention_forward",
    "attention_forward_kv",
    "flash_attn_naive_fwd",
    "flash_attn_naive_workspace_bytes",
    "attention_forward_varlen",
    "attention_backward",
    "flash_attn_bwd_kv",
    "flash_attn_bwd_varlen",
    "flash_attn_bwd_kv_workspace_bytes",
    "attention_backward_kv",
    "attention_backward_varlen",
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
    lib.flash_attn_bwd.argtypes = [P] * 10 + [Z, I, I, I, I, I, F, I, P]
    lib.flash_attn_bwd.restype = I
    lib.flash_attn_bwd_f32.argtypes = [P] * 10 + [Z, I, I, I, I, I, F, I, P]
    lib.flash_attn_bwd_f32.restype = I
    lib.flash_attn_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.flash_attn_bwd_workspace_bytes.restype = Z
    L = ctypes.c_longlong
    lib.flash_attn_fwd_kv.argtypes = [P] * 5 + [I] * 6 + [F, I, I, P, Z, P]
    lib.flash_attn_fwd_kv.restype = I
    lib.flash_attn_fwd_kv_noalloc.argtypes = [P] * 5 + [I] * 6 + [F, I, I, P]
    lib.flash_attn_fwd_kv_noalloc.restype = I
    lib.flash_attn_fwd_varlen.argtypes = [P] * 7 + [I] * 8 + [F, I, I, P, Z, P]
    lib.flash_attn_fwd_varlen.restype = I
    lib.flash_attn_fwd_kv_num_splits.argtypes = [I] * 6
    lib.flash_attn_fwd_kv_num_splits.restype = I
    lib.flash_attn_fwd_kv_workspace_bytes.argtypes = [L, I, I]
    lib.flash_attn_fwd_kv_workspace_bytes.restype = Z
    lib.flash_attn_naive_fwd.argtypes = [P] * 5 + [I] * 5 + [F, I, P, Z, P]
    lib.flash_attn_naive_fwd.restype = I
    lib.flash_attn_naive_workspace_bytes.argtypes = [I, I, I]
    lib.flash_attn_naive_workspace_bytes.restype = Z
    lib.flash_attn_bwd_kv.argtypes = [P] * 10 + [Z] + [I] * 6 + [F, I, P]
    lib.flash_attn_bwd_kv.restype = I
    lib.flash_attn_bwd_varlen.argtypes = [P] * 12 + [Z] + [I] * 8 + [F, I, P]
    lib.flash_attn_bwd_varlen.restype = I
    lib.flash_attn_bwd_kv_workspace_bytes.argtypes = [L, I]
    lib.flash_attn_bwd_kv_workspace_bytes.restype = Z
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


def _expect_shape(what, t, shape):
    """The C ABI sees only pointers: a tensor of another shape would be read or
    written out of bounds on the GPU, so every shape is checked here first."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch tensor")
    if tuple(int(x) for x in t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dims(q, k):
    import torch
    if not isinstance(q, torch.Tensor) or not isinstance(k, torch.Tensor):
        raise TypeError("expected torch tensors")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, Hq, N, d = (int(x) for x in q.shape)
    Hkv = int(k.shape[1])
    _expect_shape("k", k, (B, Hkv, N, d))
    return B, Hq, Hkv, N, d


def _check_fwd_shapes(q, k, v, o, lse):
    B, Hq, Hkv, N, d = _dims(q, k)
    _expect_shape("v", v, (B, Hkv, N, d))
    _expect_shape("o", o, (B, Hq, N, d))
    _expect_shape("lse", lse, (B, Hq, N))
    return B, Hq, Hkv, N, d


def _check_bwd_shapes(q, k, v, o, lse, dout, dq, dk, dv):
    B, Hq, Hkv, N, d = _check_fwd_shapes(q, k, v, o, lse)
    for what, t in (("dout", dout), ("dq", dq)):
        _expect_shape(what, t, (B, Hq, N, d))
    for what, t in (("dk", dk), ("dv", dv)):
        _expect_shape(what, t, (B, Hkv, N, d))
    return B, Hq, Hkv, N, d


def _fwd(name, dt, q, k, v, o, lse, scale, causal, stream):
    import torch
    B, Hq, Hkv, N, d = _check_fwd_shapes(q, k, v, o, lse)
    _check(q, k, v, o, dtype=dt)
    _check(lse, dtype=torch.float32)
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
    B, Hq, Hkv, N, d = _check_bwd_shapes(q, k, v, o, lse, dout, dq, dk, dv)
    _check(q, k, v, o, dout, dq, dk, dv, dtype=dt)
    _check(lse, dtype=torch.float32)
    _check(workspace)
    need = flash_attn_bwd_workspace_bytes(B, Hq, Hkv, N, d)
    if _ws_size(workspace) < need:
        raise ValueError(f"workspace too small: need {need} bytes")
    st = getattr(load_library(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), _ws_size(workspace),
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


def flash_attn_fwd_kv_num_splits(B, Hq, Hkv, Nq, Nk, d) -> int:
    return int(load_library().flash_attn_fwd_kv_num_splits(int(B), int(Hq), int(Hkv), int(Nq), int(Nk), int(d)))


def flash_attn_fwd_kv_workspace_bytes(rows, d, num_splits) -> int:
    return int(load_library().flash_attn_fwd_kv_workspace_bytes(int(rows), int(d), int(num_splits)))


def _ws_size(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def _check_kv_shapes(q, k, v, o, lse):
    import torch
    if not isinstance(q, torch.Tensor) or not isinstance(k, torch.Tensor):
        raise TypeError("expected torch tensors")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, Nq, d] and k, v [B, Hkv, Nk, d]")
    B, Hq, Nq, d = (int(x) for x in q.shape)
    Hkv, Nk = int(k.shape[1]), int(k.shape[2])
    _expect_shape("k", k, (B, Hkv, Nk, d))
    _expect_shape("v", v, (B, Hkv, Nk, d))
    _expect_shape("o", o, (B, Hq, Nq, d))
    _expect_shape("lse", lse, (B, Hq, Nq))
    return B, Hq, Hkv, Nq, Nk, d


def _check_varlen_shapes(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k):
    import torch
    if not isinstance(q, torch.Tensor) or not isinstance(k, torch.Tensor):
        raise TypeError("expected torch tensors")
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [Hq, Tq, d] and k, v [Hkv, Tk, d]")
    Hq, Tq, d = (int(x) for x in q.shape)
    Hkv, Tk = int(k.shape[0]), int(k.shape[1])
    _expect_shape("k", k, (Hkv, Tk, d))
    _expect_shape("v", v, (Hkv, Tk, d))
    _expect_shape("o", o, (Hq, Tq, d))
    _expect_shape("lse", lse, (Hq, Tq))
    for what, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not isinstance(t, torch.Tensor) or t.dim() != 1 or t.numel() < 2:
            raise ValueError(f"{what} must be a 1-D tensor of B+1 >= 2 offsets")
    if cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError(f"cu_seqlens_k has {cu_seqlens_k.numel()} entries, cu_seqlens_q {cu_seqlens_q.numel()}")
    return int(cu_seqlens_q.numel()) - 1, Hq, Hkv, Tq, Tk, d


def flash_attn_fwd_kv(q, k, v, o, lse, scale, causal, num_splits=1, workspace=None, stream=None):
    """bf16 forward with Nq queries and Nk keys (bottom-right causal), optionally
    split over keys: q, o [B,Hq,Nq,d], k, v [B,Hkv,Nk,d], lse [B,Hq,Nq] fp32."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = _check_kv_shapes(q, k, v, o, lse)
    _check(q, k, v, o, dtype=torch.bfloat16)
    _check(lse, dtype=torch.float32)
    if workspace is not None:
        _check(workspace)
    st = load_library().flash_attn_fwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                                          float(scale), int(bool(causal)), int(num_splits), _ptr(workspace),
                                          _ws_size(workspace), _stream(stream))
    if st != 0:
        raise FlashAttnError("flash_attn_fwd_kv", st)


def flash_attn_fwd_kv_noalloc(q, k, v, o, lse, scale, causal, num_splits=0, stream=None):
    """flash_attn_fwd_kv with the split partials in the library's static
    scratch: no workspace, no device allocation (FLASH_ATTN_SCRATCH_BYTES)."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = _check_kv_shapes(q, k, v, o, lse)
    _check(q, k, v, o, dtype=torch.bfloat16)
    _check(lse, dtype=torch.float32)
    st = load_library().flash_attn_fwd_kv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq,
                                                  Nk, d, float(scale), int(bool(causal)), int(num_splits),
                                                  _stream(stream))
    if st != 0:
        raise FlashAttnError("flash_attn_fwd_kv_noalloc", st)


def flash_attn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, causal,
                          num_splits=1, workspace=None, stream=None):
    """bf16 forward over a variable-length batch: q, o [Hq,Tq,d], k, v [Hkv,Tk,d],
    lse [Hq,Tq] fp32, cu_seqlens_* int32 [B+1] on the GPU."""
    import torch
    B, Hq, Hkv, Tq, Tk, d = _check_varlen_shapes(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k)
    _check(q, k, v, o, dtype=torch.bfloat16)
    _check(lse, dtype=torch.float32)
    _check(cu_seqlens_q, cu_seqlens_k, dtype=torch.int32)
    if workspace is not None:
        _check(workspace)
    st = load_library().flash_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                                              _ptr(cu_seqlens_k), B, Hq, Hkv, Tq, Tk, int(max_seqlen_q),
                                              int(max_seqlen_k), d, float(scale), int(bool(causal)),
                                              int(num_splits), _ptr(workspace), _ws_size(workspace),
                                              _stream(stream))
    if st != 0:
        raise FlashAttnError("flash_attn_fwd_varlen", st)


def _kv_workspace(rows, d, splits, device):
    import torch
    n = flash_attn_fwd_kv_workspace_bytes(rows, d, splits)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=device)


def attention_forward_kv(q, k, v, scale, causal, num_splits=0, stream=None):
    """Allocate o, lse and the workspace with torch and run flash_attn_fwd_kv
    (num_splits=0: the library's choice)."""
    import torch
    B, Hq, Nq, d = (int(x) for x in q.shape)
    Hkv, Nk = int(k.shape[1]), int(k.shape[2])
    splits = num_splits or flash_attn_fwd_kv_num_splits(B, Hq, Hkv, Nq, Nk, d)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    ws = _kv_workspace(B * Hq * Nq, d, splits, q.device)
    flash_attn_fwd_kv(q, k, v, o, lse, scale, causal, splits, ws, stream)
    return o, lse


def attention_forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, causal,
                             num_splits=0, stream=None):
    """Allocate o, lse and the workspace with torch and run flash_attn_fwd_varlen."""
    import torch
    Hq, Tq, d = (int(x) for x in q.shape)
    Hkv = int(k.shape[0])
    B = int(cu_seqlens_q.numel()) - 1
    splits = num_splits or flash_attn_fwd_kv_num_splits(B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    ws = _kv_workspace(Hq * Tq, d, splits, q.device)
    flash_attn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, causal,
                          splits, ws, stream)
    return o, lse


def flash_attn_naive_workspace_bytes(B, Hq, N) -> int:
    return int(load_library().flash_attn_naive_workspace_bytes(int(B), int(Hq), int(N)))


def flash_attn_naive_fwd(q, k, v, o, lse, scale, causal, workspace, stream=None):
    """Three-pass materialising baseline (bf16): same arguments as flash_attn_fwd
    plus a workspace of flash_attn_naive_workspace_bytes(B, Hq, N) bytes."""
    import torch
    B, Hq, Hkv, N, d = _check_fwd_shapes(q, k, v, o, lse)
    _check(q, k, v, o, dtype=torch.bfloat16)
    _check(lse, dtype=torch.float32)
    _check(workspace)
    st = load_library().flash_attn_naive_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                                             float(scale), int(bool(causal)), _ptr(workspace), _ws_size(workspace),
                                             _stream(stream))
    if st != 0:
        raise FlashAttnError("flash_attn_naive_fwd", st)


def flash_attn_bwd_kv_workspace_bytes(rows, d) -> int:
    return int(load_library().flash_attn_bwd_kv_workspace_bytes(int(rows), int(d)))


def _check_grads(q, k, dout, dq, dk, dv):
    for what, t in (("dout", dout), ("dq", dq)):
        _expect_shape(what, t, tuple(q.shape))
    for what, t in (("dk", dk), ("dv", dv)):
        _expect_shape(what, t, tuple(k.shape))


def flash_attn_bwd_kv(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale, causal, stream=None):
    """bf16 backward of flash_attn_fwd_kv's problem (Nq queries, Nk keys,
    bottom-right causal) into caller-allocated dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d]."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = _check_kv_shapes(q, k, v, o, lse)
    _check_grads(q, k, dout, dq, dk, dv)
    _check(q, k, v, o, dout, dq, dk, dv, dtype=torch.bfloat16)
    _check(lse, dtype=torch.float32)
    _check(workspace)
    need = flash_attn_bwd_kv_workspace_bytes(B * Hq * Nq, d)
    if _ws_size(workspace) < need:
        raise ValueError(f"workspace too small: need {need} bytes")
    st = load_library().flash_attn_bwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                          _ptr(dk), _ptr(dv), _ptr(workspace), _ws_size(workspace), B, Hq, Hkv, Nq,
                                          Nk, d, float(scale), int(bool(causal)), _stream(stream))
    if st != 0:
        raise FlashAttnError("flash_attn_bwd_kv", st)


def flash_attn_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                          workspace, scale, causal, stream=None):
    """bf16 backward of flash_attn_fwd_varlen's problem: q, o, dout, dq [Hq,Tq,d],
    k, v, dk, dv [Hkv,Tk,d], lse [Hq,Tq] fp32, cu_seqlens_* int32 [B+1] on the GPU."""
    import torch
    B, Hq, Hkv, Tq, Tk, d = _check_varlen_shapes(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k)
    _check_grads(q, k, dout, dq, dk, dv)
    _check(q, k, v, o, dout, dq, dk, dv, dtype=torch.bfloat16)
    _check(lse, dtype=torch.float32)
    _check(cu_seqlens_q, cu_seqlens_k, dtype=torch.int32)
    _check(workspace)
    need = flash_attn_bwd_kv_workspace_bytes(Hq * Tq, d)
    if _ws_size(workspace) < need:
        raise ValueError(f"workspace too small: need {need} bytes")
    st = load_library().flash_attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                              _ptr(dk), _ptr(dv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                              _ptr(workspace), _ws_size(workspace), B, Hq, Hkv, Tq, Tk,
                                              int(max_seqlen_q), int(max_seqlen_k), d, float(scale),
                                              int(bool(causal)), _stream(stream))
    if st != 0:
        raise FlashAttnError("flash_attn_bwd_varlen", st)


def attention_backward_kv(q, k, v, o, lse, dout, scale, causal, stream=None):
    """Allocate dq, dk, dv and the workspace with torch and run flash_attn_bwd_kv."""
    import torch
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, Hq, Nq, d = (int(x) for x in q.shape)
    ws = torch.empty(max(flash_attn_bwd_kv_workspace_bytes(B * Hq * Nq, d), 256), dtype=torch.uint8, device=q.device)
    flash_attn_bwd_kv(q, k, v, o, lse, dout, dq, dk, dv, ws, scale, causal, stream)
    return dq, dk, dv


def attention_backward_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale,
                              causal, stream=None):
    """Allocate dq, dk, dv and the workspace with torch and run flash_attn_bwd_varlen."""
    import torch
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    Hq, Tq, d = (int(x) for x in q.shape)
    ws = torch.empty(max(flash_attn_bwd_kv_workspace_bytes(Hq * Tq, d), 256), dtype=torch.uint8, device=q.device)
    flash_attn_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                          ws, scale, causal, stream)
    return dq, dk, dv
