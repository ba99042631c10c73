"""Python binding of libattn.so: exact attention forward/backward and fp8 preparation on gfx950.

Argument marshalling only.  Every step of the computation runs in the HIP kernels behind the C
ABI declared in include/attn.h; torch supplies device memory and the current stream.  There is
no fallback: if the library is missing or a call fails, these functions raise.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "load", "library_path", "fwd", "bwd", "bwd_phases", "fwd_fp8", "fp8_prep", "bwd_workspace_size",
    "fwd_splitkv", "fwd_splitkv_noalloc", "splitkv_workspace_size", "attention", "clock_probe", "mfma_probe", "hbm_probe", "fwd_ext", "bwd_ext", "fwd_varlen", "bwd_varlen", "bwd_varlen_workspace_size", "AttnError", "EXPORTS", "F16", "BF16", "FP8_E4M3", "F32",
]

F16, BF16, FP8_E4M3, F32 = 0, 1, 2, 3
EXPORTS = ("attn_fwd", "attn_fwd_ext", "attn_bwd_ext", "attn_fwd_varlen", "attn_bwd", "attn_bwd_workspace_size", "attn_bwd_preprocess", "attn_bwd_dkdv",
           "attn_bwd_dq", "attn_bwd_varlen", "attn_bwd_varlen_workspace_size", "attn_fwd_splitkv", "attn_fwd_splitkv_workspace_size", "attn_fp8_prep",
           "attn_fwd_splitkv_noalloc", "attn_clock_probe", "attn_mfma_probe", "attn_hbm_probe", "attn_status_string")

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class AttnError(RuntimeError):
    pass


def library_path() -> str:
    return os.path.join(_HERE, "libattn.so")


def load():
    """Load libattn.so (built in place by exact_attention_online_amd.build) and declare its ABI."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise AttnError(f"{path} is missing: build it with `python -m exact_attention_online_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp] * 5 + [i] * 6 + [f, i] + [vp] * 3 + [vp]
    lib.attn_fwd.restype = i
    lib.attn_bwd_workspace_size.argtypes = [i] * 5
    lib.attn_bwd_workspace_size.restype = sz
    lib.attn_bwd.argtypes = [vp] * 9 + [i] * 6 + [f, i, i, vp, sz, vp]
    lib.attn_bwd.restype = i
    lib.attn_bwd_preprocess.argtypes = [vp] * 5 + [i] * 6 + [vp, sz, vp]
    lib.attn_bwd_preprocess.restype = i
    lib.attn_bwd_dkdv.argtypes = [vp] * 7 + [i] * 6 + [f, i, i, vp, sz, vp]
    lib.attn_bwd_dkdv.restype = i
    lib.attn_bwd_dq.argtypes = [vp] * 6 + [i] * 6 + [f, i, i, vp, sz, vp]
    lib.attn_bwd_dq.restype = i
    lib.attn_fwd_ext.argtypes = [vp] * 5 + [i] * 6 + [f, i, i, vp, vp]
    lib.attn_fwd_varlen.argtypes = [vp] * 6 + [i] * 7 + [f, i, vp]
    lib.attn_fwd_varlen.restype = i
    lib.attn_fwd_ext.restype = i
    lib.attn_bwd_ext.argtypes = [vp] * 9 + [i] * 6 + [f, i, i, i, vp, vp, sz, vp]
    lib.attn_bwd_ext.restype = i
    lib.attn_bwd_varlen_workspace_size.argtypes = [i] * 5
    lib.attn_bwd_varlen_workspace_size.restype = sz
    lib.attn_bwd_varlen.argtypes = [vp] * 10 + [i] * 7 + [f, i, i, vp, sz, vp]
    lib.attn_bwd_varlen.restype = i
    lib.attn_fwd_splitkv_workspace_size.argtypes = [i] * 7
    lib.attn_fwd_splitkv_workspace_size.restype = sz
    lib.attn_fwd_splitkv.argtypes = [vp] * 5 + [i] * 7 + [f, i, i, vp, sz, vp]
    lib.attn_fwd_splitkv.restype = i
    lib.attn_fwd_splitkv_noalloc.argtypes = [vp] * 5 + [i] * 7 + [f, i, i, vp]
    lib.attn_fwd_splitkv_noalloc.restype = i
    lib.attn_fp8_prep.argtypes = [vp] * 4 + [i] * 5 + [vp]
    lib.attn_fp8_prep.restype = i
    lib.attn_clock_probe.argtypes = [vp, i, ctypes.c_longlong, vp]
    lib.attn_clock_probe.restype = i
    lib.attn_mfma_probe.argtypes = [vp, ctypes.c_longlong, vp, i, i, i, vp]
    lib.attn_mfma_probe.restype = i
    lib.attn_hbm_probe.argtypes = [vp, ctypes.c_longlong, vp, i, vp]
    lib.attn_hbm_probe.restype = i
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise AttnError(f"libattn error {rc}: {load().attn_status_string(rc).decode()}")


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise AttnError(f"unsupported dtype {t.dtype} (expected float16 or bfloat16)")


def _grad_dtype(q, grad_dtype):
    """(torch dtype, ABI code) of the gradients: the input dtype (None) or float32."""
    torch = _torch()
    if grad_dtype is None or grad_dtype == q.dtype:
        return q.dtype, _dtype_code(q)
    if grad_dtype == torch.float32:
        return torch.float32, F32
    raise AttnError(f"grad_dtype must be None, {q.dtype} or torch.float32, got {grad_dtype}")


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _req(device, **named):
    """Every tensor the library will dereference: contiguous, on `device`, and (where given) of
    the expected shape and dtype.  name=(tensor, shape or None, dtype or None).  A host tensor
    here would reach a kernel as a host address, so it is rejected before any call."""
    for name, (t, shape, dtype) in named.items():
        if not t.is_cuda or t.device != device or not t.is_contiguous():
            raise AttnError(f"{name} must be a contiguous tensor on {device}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise AttnError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if dtype is not None and t.dtype != dtype:
            raise AttnError(f"{name} must be {dtype}, got {t.dtype}")


def _shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise AttnError(f"expected q [B,Hq,N,d], k/v [B,Hkv,N,d]; got {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise AttnError("q and k/v disagree in B, N or d")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise AttnError("tensors must be contiguous device tensors")
        if t.device != q.device:
            raise AttnError("tensors must be on one device")
    return B, Hq, k.shape[1], N, d


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """O, LSE = attention(q, k, v) for fp16/bf16 q [B,Hq,N,d], k/v [B,Hkv,N,d] on one device."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    if not (q.dtype == k.dtype == v.dtype):
        raise AttnError("q, k, v must share a dtype")
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _req(q.device, out=(out, q.shape, q.dtype), lse=(lse, (B, Hq, N), torch.float32))
    _check(load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d, int(bool(causal)),
                           scale, dt, None, None, None, _stream(q.device)))
    return out, lse


def fwd_ext(q, k, v, causal: bool = False, scale: float | None = None, window: int = 0, alibi_slopes=None,
            out=None, lse=None):
    """attn_fwd with a sliding window (0 = none) and/or ALiBi slopes (float [Hq] device tensor)."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    if not (q.dtype == k.dtype == v.dtype):
        raise AttnError("q, k, v must share a dtype")
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    sl = None
    if alibi_slopes is not None:
        if (alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != Hq or not alibi_slopes.is_contiguous()
                or alibi_slopes.device != q.device):
            raise AttnError("alibi_slopes must be a contiguous float32 device tensor of Hq values")
        sl = _ptr(alibi_slopes)
    _req(q.device, out=(out, q.shape, q.dtype), lse=(lse, (B, Hq, N), torch.float32))
    _check(load().attn_fwd_ext(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d,
                               int(bool(causal)), scale, dt, int(window), sl, _stream(q.device)))
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False, scale: float | None = None, out=None,
               lse=None):
    """O [Hq,T,d], LSE [Hq,T] for sequences packed along T (q [Hq,T,d], k/v [Hkv,T,d]); cu_seqlens is a
    device int32 tensor [B+1] of sequence offsets."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise AttnError(f"expected q [Hq,T,d], k/v [Hkv,T,d]; got {tuple(q.shape)}, {tuple(k.shape)}")
    Hq, T, d = q.shape
    Hkv = k.shape[0]
    if k.shape[1] != T or k.shape[2] != d:
        raise AttnError("q and k/v disagree in T or d")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise AttnError("q, k, v must be contiguous device tensors of one dtype on one device")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda:
        raise AttnError("cu_seqlens must be an int32 device tensor [B+1]")
    B = cu_seqlens.numel() - 1
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    _req(q.device, out=(out, q.shape, q.dtype), lse=(lse, (Hq, T), torch.float32),
         cu_seqlens=(cu_seqlens, (B + 1,), torch.int32))
    _check(load().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens.contiguous()), B,
                                  Hq, Hkv, T, int(max_seqlen), d, int(bool(causal)), scale, dt, _stream(q.device)))
    return out, lse


def splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits=0) -> int:
    return int(load().attn_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits))


def fwd_splitkv(q, k, v, causal: bool = False, scale: float | None = None, num_splits: int = 0, workspace=None,
                out=None, lse=None):
    """O, LSE for q [B,Hq,Nq,d] against k/v [B,Hkv,Nk,d] (Nq <= Nk) with the keys split among
    workgroups (decoding); causal aligns the queries with the last Nq keys."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise AttnError(f"expected q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d]; got {tuple(q.shape)}, {tuple(k.shape)}")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise AttnError("q and k/v disagree in B or d")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise AttnError("q, k, v must be contiguous device tensors of one dtype on one device")
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    need = splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _req(q.device, out=(out, q.shape, q.dtype), lse=(lse, (B, Hq, Nq), torch.float32),
         workspace=(workspace, None, None))
    wsb = workspace.numel() * workspace.element_size()
    _check(load().attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                                   int(bool(causal)), scale, dt, int(num_splits), _ptr(workspace), wsb,
                                   _stream(q.device)))
    return out, lse


def fwd_splitkv_noalloc(q, k, v, out, lse, causal: bool = False, scale: float | None = None, num_splits: int = 0):
    """fwd_splitkv without a workspace: the split partials go to the library's static scratch buffer
    on the GPU (ATTN_SPLITKV_SCRATCH_BYTES, 8 MiB), so neither this call nor the library allocates;
    the caller passes out [B,Hq,Nq,d] and lse [B,Hq,Nq] (float32).  Calls that overlap on one GPU
    share that buffer and race: serialise them."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise AttnError(f"expected q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d]; got {tuple(q.shape)}, {tuple(k.shape)}")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise AttnError("q and k/v disagree in B or d")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise AttnError("q, k, v must be contiguous device tensors of one dtype on one device")
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _req(q.device, out=(out, q.shape, q.dtype), lse=(lse, (B, Hq, Nq), torch.float32))
    _check(load().attn_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                                           int(bool(causal)), scale, dt, int(num_splits), _stream(q.device)))
    return out, lse


def bwd_workspace_size(B, Hq, Hkv, N, d) -> int:
    return int(load().attn_bwd_workspace_size(B, Hq, Hkv, N, d))


def bwd(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None, workspace=None,
        dq=None, dk=None, dv=None, grad_dtype=None):
    """dQ, dK, dV of L = <O, dO>; recomputes the probabilities from q, k, v and lse.  The gradients
    come in q's dtype, or in float32 with grad_dtype=torch.float32."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    dt = _dtype_code(q)
    gdt, gcode = _grad_dtype(q, grad_dtype)
    for t in (o, do):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise AttnError("o and do must match q in shape, dtype and layout")
    if lse.shape != (B, Hq, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise AttnError("lse must be float32 [B,Hq,N]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = bwd_workspace_size(B, Hq, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q, dtype=gdt) if dq is None else dq
    dk = torch.empty_like(k, dtype=gdt) if dk is None else dk
    dv = torch.empty_like(v, dtype=gdt) if dv is None else dv
    _req(q.device, o=(o, q.shape, q.dtype), do=(do, q.shape, q.dtype), lse=(lse, (B, Hq, N), torch.float32),
         workspace=(workspace, None, None), dq=(dq, q.shape, gdt), dk=(dk, k.shape, gdt),
         dv=(dv, v.shape, gdt))
    _check(load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                           B, Hq, Hkv, N, d, int(bool(causal)), scale, dt, gcode, _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(q.device)))
    return dq, dk, dv


def bwd_ext(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None, window: int = 0, alibi_slopes=None,
            workspace=None, dq=None, dk=None, dv=None, grad_dtype=None):
    """Gradients of attn_fwd_ext (same window and ALiBi slopes); o, lse from fwd_ext; grad_dtype as for bwd."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    dt = _dtype_code(q)
    gdt, gcode = _grad_dtype(q, grad_dtype)
    for t in (o, do):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise AttnError("o and do must match q in shape, dtype and layout")
    if lse.shape != (B, Hq, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise AttnError("lse must be float32 [B,Hq,N]")
    sl = None
    if alibi_slopes is not None:
        if (alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != Hq or not alibi_slopes.is_contiguous()
                or alibi_slopes.device != q.device):
            raise AttnError("alibi_slopes must be a contiguous float32 device tensor of Hq values")
        sl = _ptr(alibi_slopes)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = bwd_workspace_size(B, Hq, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q, dtype=gdt) if dq is None else dq
    dk = torch.empty_like(k, dtype=gdt) if dk is None else dk
    dv = torch.empty_like(v, dtype=gdt) if dv is None else dv
    _req(q.device, o=(o, q.shape, q.dtype), do=(do, q.shape, q.dtype), lse=(lse, (B, Hq, N), torch.float32),
         workspace=(workspace, None, None), dq=(dq, q.shape, gdt), dk=(dk, k.shape, gdt),
         dv=(dv, v.shape, gdt))
    _check(load().attn_bwd_ext(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                               _ptr(dv), B, Hq, Hkv, N, d, int(bool(causal)), scale, dt, gcode, int(window), sl,
                               _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device)))
    return dq, dk, dv


def bwd_varlen_workspace_size(B, Hq, Hkv, max_seqlen, d) -> int:
    return int(load().attn_bwd_varlen_workspace_size(B, Hq, Hkv, max_seqlen, d))


def bwd_varlen(q, k, v, o, do, lse, cu_seqlens, max_seqlen: int, causal: bool = False, scale: float | None = None,
               workspace=None, dq=None, dk=None, dv=None, grad_dtype=None):
    """dQ [Hq,T,d], dK, dV [Hkv,T,d] for sequences packed along T, with o, lse from fwd_varlen (same
    cu_seqlens, max_seqlen, causal flag and scale).  Rows outside every sequence come back as zeros
    when the outputs are allocated here; grad_dtype as for bwd."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise AttnError(f"expected q [Hq,T,d], k/v [Hkv,T,d]; got {tuple(q.shape)}, {tuple(k.shape)}")
    Hq, T, d = q.shape
    Hkv = k.shape[0]
    if k.shape[1] != T or k.shape[2] != d:
        raise AttnError("q and k/v disagree in T or d")
    for t in (q, k, v, o, do):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise AttnError("q, k, v, o, do must be contiguous device tensors of one dtype on one device")
    for t in (o, do):
        if t.shape != q.shape:
            raise AttnError("o and do must match q in shape")
    if lse.shape != (Hq, T) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise AttnError("lse must be float32 [Hq,T]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda:
        raise AttnError("cu_seqlens must be an int32 device tensor [B+1]")
    B = cu_seqlens.numel() - 1
    dt = _dtype_code(q)
    gdt, gcode = _grad_dtype(q, grad_dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = bwd_varlen_workspace_size(B, Hq, Hkv, int(max_seqlen), d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq = torch.zeros_like(q, dtype=gdt) if dq is None else dq
    dk = torch.zeros_like(k, dtype=gdt) if dk is None else dk
    dv = torch.zeros_like(v, dtype=gdt) if dv is None else dv
    _req(q.device, o=(o, q.shape, q.dtype), do=(do, q.shape, q.dtype), lse=(lse, (Hq, T), torch.float32),
         cu_seqlens=(cu_seqlens, (B + 1,), torch.int32), workspace=(workspace, None, None),
         dq=(dq, q.shape, gdt), dk=(dk, k.shape, gdt), dv=(dv, v.shape, gdt))
    _check(load().attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(cu_seqlens.contiguous()), B, Hq, Hkv, T, int(max_seqlen), d,
                                  int(bool(causal)), scale, dt, gcode, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(q.device)))
    return dq, dk, dv


def bwd_phases(q, k, v, o, do, lse, causal, scale, workspace, dq, dk, dv, between=None):
    """attn_bwd as its three phases (preprocess, dK/dV, dQ); ``between(i)`` (if given) is called
    before phase i = 0, 1, 2 and after the last one with i = 3, e.g. to record stream events.
    The gradients come in dq's dtype (q's dtype or float32)."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    dt = _dtype_code(q)
    gdt, gcode = _grad_dtype(q, dq.dtype)
    _req(q.device, o=(o, q.shape, q.dtype), do=(do, q.shape, q.dtype), lse=(lse, (B, Hq, N), torch.float32),
         workspace=(workspace, None, None), dq=(dq, q.shape, gdt), dk=(dk, k.shape, gdt),
         dv=(dv, v.shape, gdt))
    lib, st = load(), _stream(q.device)
    wsb = workspace.numel() * workspace.element_size()
    hook = between or (lambda i: None)
    causal, scale = int(bool(causal)), float(scale)
    hook(0)
    _check(lib.attn_bwd_preprocess(_ptr(q), _ptr(k), _ptr(o), _ptr(do), _ptr(lse), B, Hq, Hkv, N, d, dt,
                                   _ptr(workspace), wsb, st))
    hook(1)
    _check(lib.attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d,
                             causal, scale, dt, gcode, _ptr(workspace), wsb, st))
    hook(2)
    _check(lib.attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(dq), B, Hq, Hkv, N, d, causal,
                           scale, dt, gcode, _ptr(workspace), wsb, st))
    hook(3)
    return dq, dk, dv


def fp8_prep(x, signs=None, out=None, descale=None, pow2_scale=False):
    """float32 x [B,H,N,d] -> (e4m3 codes as uint8 [B,H,N,d], float32 descale [B,H,ceil(N/128)]);
    pow2_scale: block scales rounded up to powers of two (what fwd_fp8 applies exactly to V)."""
    torch = _torch()
    if x.dim() != 4 or x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise AttnError("x must be a contiguous float32 device tensor [B,H,N,d]")
    B, H, N, d = x.shape
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if descale is None:
        descale = torch.empty((B, H, (N + 127) // 128), dtype=torch.float32, device=x.device)
    sp = None
    if signs is not None:
        if signs.dtype != torch.int8 or signs.numel() != d or not signs.is_cuda:
            raise AttnError("signs must be an int8 device tensor of length d")
        _req(x.device, signs=(signs, (d,), torch.int8))
        sp = _ptr(signs)
    _req(x.device, out=(out, x.shape, torch.uint8), descale=(descale, (B, H, (N + 127) // 128), torch.float32))
    _check(load().attn_fp8_prep(_ptr(x), _ptr(out), _ptr(descale), sp, B, H, N, d, int(bool(pow2_scale)),
                                _stream(x.device)))
    return out, descale


def fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, causal: bool = False, scale: float | None = None,
            out=None, lse=None):
    """Attention on e4m3 codes (uint8 [B,H,N,d]) with per-128-row float descales; O in bfloat16."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shapes(q8, k8, v8)
    for t in (q8, k8, v8):
        if t.dtype != torch.uint8:
            raise AttnError("fp8 operands are passed as uint8 e4m3 codes")
    nb = (N + 127) // 128
    for t, H in ((q_descale, Hq), (k_descale, Hkv), (v_descale, Hkv)):
        if t.shape != (B, H, nb) or t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise AttnError("descales must be float32 [B,H,ceil(N/128)] device tensors")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q8.device)
    _req(q8.device, q_descale=(q_descale, (B, Hq, nb), torch.float32), k_descale=(k_descale, (B, Hkv, nb), torch.float32),
         v_descale=(v_descale, (B, Hkv, nb), torch.float32), out=(out, q8.shape, torch.bfloat16),
         lse=(lse, (B, Hq, N), torch.float32))
    _check(load().attn_fwd(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d, int(bool(causal)),
                           scale, FP8_E4M3, _ptr(q_descale), _ptr(k_descale), _ptr(v_descale), _stream(q8.device)))
    return out, lse


def clock_probe(out, ticks: int, stream=None):
    """Launch attn_clock_probe: out is an int64 device tensor of 2 * groups entries (engine clocks
    and 100 MHz real-time ticks per workgroup, filled when the probe ends); it runs on `stream`
    (a torch.cuda.Stream, default: the current stream) for `ticks` real-time ticks.  Clock of
    workgroup i in GHz: 0.1 * out[2i] / out[2i + 1]."""
    torch = _torch()
    if out.dtype != torch.int64 or out.dim() != 1 or out.numel() % 2 or not out.is_cuda or not out.is_contiguous():
        raise AttnError("out must be a contiguous int64 device tensor of 2 * groups entries")
    st = (stream or torch.cuda.current_stream(out.device)).cuda_stream
    _check(load().attn_clock_probe(_ptr(out), out.numel() // 2, int(ticks), ctypes.c_void_p(st)))
    return out


def mfma_probe(data, out, iters: int, stream=None):
    """Launch attn_mfma_probe: data is a contiguous device tensor of operand bits, bf16 values (at
    least 8192, a multiple of 8) or uint8 e4m3 codes (at least 8192, a multiple of 32), out a
    float32 device tensor of 512 * groups entries; runs on `stream` (default: the current
    stream).  Returns the launch's flop count."""
    torch = _torch()
    if data.dtype == torch.bfloat16:
        dtype, per_mfma = BF16, 32768
    elif data.dtype == torch.uint8:
        dtype, per_mfma = FP8_E4M3, 131072
    else:
        raise AttnError("data must hold bf16 values or uint8 e4m3 codes")
    if not data.is_cuda or not data.is_contiguous():
        raise AttnError("data must be a contiguous device tensor")
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous() or out.numel() % 512:
        raise AttnError("out must be a contiguous float32 device tensor of 512 * groups entries")
    groups = out.numel() // 512
    st = (stream or torch.cuda.current_stream(out.device)).cuda_stream
    _check(load().attn_mfma_probe(_ptr(data), data.numel(), _ptr(out), groups, int(iters), dtype,
                                  ctypes.c_void_p(st)))
    return groups * 8 * 32 * int(iters) * per_mfma


def hbm_probe(data, out, stream=None):
    """Launch attn_hbm_probe: data is a contiguous device tensor (any dtype; its bytes a multiple
    of 16384 * groups), out an int32 device tensor of 64 * groups entries that receives each
    lane's sum modulo 2^32 of the 32-bit words it read; runs on `stream` (default: the current
    stream).  Returns the number of bytes read."""
    torch = _torch()
    if not data.is_cuda or not data.is_contiguous():
        raise AttnError("data must be a contiguous device tensor")
    if out.dtype != torch.int32 or not out.is_cuda or not out.is_contiguous() or out.numel() % 64:
        raise AttnError("out must be a contiguous int32 device tensor of 64 * groups entries")
    groups = out.numel() // 64
    nbytes = data.numel() * data.element_size()
    st = (stream or torch.cuda.current_stream(out.device)).cuda_stream
    _check(load().attn_hbm_probe(_ptr(data), nbytes, _ptr(out), groups, ctypes.c_void_p(st)))
    return nbytes


_AttentionFn = None


def attention(q, k, v, causal: bool = False, scale: float | None = None):
    """Differentiable attention for fp16/bf16 q [B,Hq,N,d], k/v [B,Hkv,N,d] on one device: the
    forward is attn_fwd (O and the logsumexp saved), the backward attn_bwd (probabilities
    recomputed); dK/dV are summed over each query-head group.  Gradients flow to q, k and v."""
    global _AttentionFn
    torch = _torch()
    if _AttentionFn is None:
        class _Fn(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q_, k_, v_, causal_, scale_):
                o, lse = fwd(q_, k_, v_, causal=causal_, scale=scale_)
                ctx.save_for_backward(q_, k_, v_, o, lse)
                ctx.causal, ctx.scale = causal_, scale_
                return o

            @staticmethod
            def backward(ctx, do):
                q_, k_, v_, o, lse = ctx.saved_tensors
                dq, dk, dv = bwd(q_, k_, v_, o, do.contiguous(), lse, causal=ctx.causal, scale=ctx.scale)
                return dq, dk, dv, None, None

        _AttentionFn = _Fn
    return _AttentionFn.apply(q, k, v, bool(causal), scale)
