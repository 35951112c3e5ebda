"""Python binding of libfa.so: argument marshalling only.

The functions named like the C entry points (``fa_fwd``, ``fa_fwd_fp32``,
``fa_decode``, ``fa_decode_noalloc``, ``fa_decode_workspace_size``,
``fa_status_string`` and the others in ``EXPORTED``) take the
same arguments as in ``include/fa.h``; pointer arguments may be torch tensors
(their ``data_ptr()``), plain integers or None, and ``stream`` may be a
``torch.cuda.Stream``, a raw handle or None (torch's current stream).  They
return the C status code.

``attention``, ``attention_varlen``, ``attention_fp8`` and ``decode`` are conveniences on top:
they check tensor shapes, allocate the outputs with torch (device memory is
all torch provides here) and raise ``FAError`` on a non-zero status.  Every
arithmetic step runs in the library's kernels; there is no other path.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_WORKSPACE = -3
FA_ERR_LAUNCH = -4

EXPORTED = ("fa_fwd", "fa_fwd_fp32", "fa_fwd_kvcache", "fa_bwd_workspace_size", "fa_bwd",
            "fa_decode_workspace_size", "fa_decode", "fa_decode_noalloc", "fa_fwd_fp8",
            "fa_status_string")

# bytes of the per-GPU device array behind fa_decode_noalloc
FA_DECODE_SCRATCH_BYTES = 80 << 20

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {fa_status_string(status)} ({status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m io_aware_exact_19_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    fwd_args = [P, P, P, P, P, I, I, I, I, I, F, I, I, P, P, P]
    lib.fa_fwd.argtypes = fwd_args
    lib.fa_fwd.restype = I
    lib.fa_fwd_fp32.argtypes = fwd_args
    lib.fa_fwd_fp32.restype = I
    lib.fa_fwd_kvcache.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.fa_fwd_kvcache.restype = I
    lib.fa_bwd_workspace_size.argtypes = [I, I, I]
    lib.fa_bwd_workspace_size.restype = Z
    lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, P, Z, P]
    lib.fa_bwd.restype = I
    lib.fa_decode_workspace_size.argtypes = [I, I, I, I, I]
    lib.fa_decode_workspace_size.restype = Z
    lib.fa_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, F, I, P, Z, P]
    lib.fa_decode.restype = I
    lib.fa_decode_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, F, I, P]
    lib.fa_decode_noalloc.restype = I
    lib.fa_fwd_fp8.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.fa_fwd_fp8.restype = I
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


# ------------------------------------------------------------- same names


def fa_fwd(q, k, v, o, lse, batch, heads, seqlen_q, seqlen_k, d, scale, causal, window_left,
           cu_seqlens_q=None, cu_seqlens_k=None, stream=None) -> int:
    return load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), batch, heads,
                                 seqlen_q, seqlen_k, d, scale, int(causal), window_left,
                                 _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _stream(stream))


def fa_fwd_fp32(q, k, v, o, lse, batch, heads, seqlen_q, seqlen_k, d, scale, causal,
                window_left, cu_seqlens_q=None, cu_seqlens_k=None, stream=None) -> int:
    return load_library().fa_fwd_fp32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), batch,
                                      heads, seqlen_q, seqlen_k, d, scale, int(causal),
                                      window_left, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                      _stream(stream))


def fa_fwd_kvcache(q, k_cache, v_cache, seqlens_k, o, lse, batch, heads, seqlen_q, max_len, d,
                   scale, causal, window_left, stream=None) -> int:
    return load_library().fa_fwd_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k),
                                         _ptr(o), _ptr(lse), batch, heads, seqlen_q, max_len, d,
                                         scale, int(causal), window_left, _stream(stream))


def fa_bwd_workspace_size(batch, heads, seqlen_q) -> int:
    return int(load_library().fa_bwd_workspace_size(batch, heads, seqlen_q))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, batch, heads, seqlen_q, seqlen_k, d, scale, causal,
           window_left, workspace, workspace_bytes, stream=None) -> int:
    return load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                 _ptr(dq), _ptr(dk), _ptr(dv), batch, heads, seqlen_q, seqlen_k,
                                 d, scale, int(causal), window_left, _ptr(workspace),
                                 workspace_bytes, _stream(stream))


def fa_decode_workspace_size(batch, heads, max_len, d, chunk) -> int:
    return int(load_library().fa_decode_workspace_size(batch, heads, max_len, d, chunk))


def fa_decode(q, k_cache, v_cache, seqlens_k, o, lse, batch, heads, max_len, d, scale, chunk,
              workspace, workspace_bytes, stream=None) -> int:
    return load_library().fa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k),
                                    _ptr(o), _ptr(lse), batch, heads, max_len, d, scale, chunk,
                                    _ptr(workspace), workspace_bytes, _stream(stream))


def fa_decode_noalloc(q, k_cache, v_cache, seqlens_k, o, lse, batch, heads, max_len, d, scale,
                      chunk, stream=None) -> int:
    return load_library().fa_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(seqlens_k), _ptr(o), _ptr(lse), batch, heads,
                                            max_len, d, scale, chunk, _stream(stream))


def fa_fwd_fp8(q, k, v, o, lse, descale_q, descale_k, descale_v, batch, heads, seqlen_q, seqlen_k,
               d, scale, causal, window_left, stream=None) -> int:
    return load_library().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                     _ptr(descale_q), _ptr(descale_k), _ptr(descale_v), batch,
                                     heads, seqlen_q, seqlen_k, d, scale, int(causal), window_left,
                                     _stream(stream))


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


# ------------------------------------------------------------ conveniences


def _check_tensor(name, t, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(ws):
    if not isinstance(ws, torch.Tensor) or ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the GPU")


def attention(q, k, v, *, scale=None, causal=False, window_left=-1, return_lse=True, out=None,
              lse_out=None, stream=None):
    """Dense attention: q [B, n_q, H, d], k/v [B, n_k, H, d], bf16 or fp32.
    Returns (o [B, n_q, H, d], lse [B, H, n_q] fp32 or None)."""
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bfloat16 or float32")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, dtype, 4)
    B, n_q, H, d = q.shape
    if k.shape[0] != B or k.shape[2] != H or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    n_k = k.shape[1]
    o = torch.empty_like(q) if out is None else out
    _check_tensor("out", o, dtype, 4)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    lse = None
    if return_lse:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device) if lse_out is None else lse_out
        _check_tensor("lse", lse, torch.float32, 3)
        if tuple(lse.shape) != (B, H, n_q):
            raise ValueError(f"lse_out must be [B, H, n_q] = {(B, H, n_q)}, got {tuple(lse.shape)}")
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    fn = fa_fwd if dtype == torch.bfloat16 else fa_fwd_fp32
    st = fn(q, k, v, o, lse, B, H, n_q, n_k, d, s, int(causal), int(window_left), None, None,
            stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd" if dtype == torch.bfloat16 else "fa_fwd_fp32")
    return o, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *,
                     scale=None, causal=False, window_left=-1, return_lse=True, stream=None):
    """Packed attention: q [total_q, H, d], k/v [total_k, H, d] bf16;
    cu_seqlens_* int32 [nseq + 1] on the GPU.  Returns (o, lse [H, total_q])."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.bfloat16, 3)
    _check_tensor("cu_seqlens_q", cu_seqlens_q, torch.int32, 1)
    _check_tensor("cu_seqlens_k", cu_seqlens_k, torch.int32, 1)
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have nseq + 1 entries")
    total_q, H, d = q.shape
    if k.shape[1] != H or k.shape[2] != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    nseq = cu_seqlens_q.numel() - 1
    o = torch.empty_like(q)
    lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device) if return_lse else None
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = fa_fwd(q, k, v, o, lse, nseq, H, int(max_seqlen_q), int(max_seqlen_k), d, s,
                int(causal), int(window_left), cu_seqlens_q, cu_seqlens_k, stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd (varlen)")
    return o, lse


def attention_kvcache(q, k_cache, v_cache, seqlens_k, *, scale=None, causal=True, window_left=-1,
                      return_lse=True, out=None, stream=None):
    """q [B, n_new, H, d] (the last n_new positions of each sequence), caches
    [B, max_len, H, d] bf16 holding them, seqlens_k int32 [B] on the GPU.
    Returns (o [B, n_new, H, d], lse [B, H, n_new])."""
    _check_tensor("q", q, torch.bfloat16, 4)
    _check_tensor("k_cache", k_cache, torch.bfloat16, 4)
    _check_tensor("v_cache", v_cache, torch.bfloat16, 4)
    _check_tensor("seqlens_k", seqlens_k, torch.int32, 1)
    B, n_new, H, d = q.shape
    if k_cache.shape[0] != B or k_cache.shape[2] != H or k_cache.shape[3] != d:
        raise ValueError("cache shape mismatch")
    if v_cache.shape != k_cache.shape or seqlens_k.numel() != B:
        raise ValueError("cache/seqlens shape mismatch")
    o = torch.empty_like(q) if out is None else out
    _check_tensor("out", o, torch.bfloat16, 4)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    lse = torch.empty((B, H, n_new), dtype=torch.float32, device=q.device) if return_lse else None
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = fa_fwd_kvcache(q, k_cache, v_cache, seqlens_k, o, lse, B, H, n_new, k_cache.shape[1], d,
                        s, int(causal), int(window_left), stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_kvcache")
    return o, lse


def attention_backward(q, k, v, o, lse, dout, *, scale=None, causal=False, window_left=-1,
                       workspace=None, stream=None):
    """Gradients of dense bf16 attention: q/o/dout [B, n_q, H, d], k/v
    [B, n_k, H, d], lse [B, H, n_q] fp32 from ``attention``.  Returns
    (dq, dk, dv)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, torch.bfloat16, 4)
    _check_tensor("lse", lse, torch.float32, 3)
    B, n_q, H, d = q.shape
    n_k = k.shape[1]
    if k.shape != (B, n_k, H, d) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch")
    if lse.shape != (B, H, n_q):
        raise ValueError("lse must be [B, H, n_q]")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = fa_bwd_workspace_size(B, H, n_q)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, n_q, n_k, d, s, int(causal),
                int(window_left), workspace, workspace.numel() * workspace.element_size(), stream)
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv


def decode(q, k_cache, v_cache, seqlens_k, *, scale=None, chunk=256, workspace=None,
           return_lse=True, out=None, stream=None):
    """q [B, 1, H, d], caches [B, max_len, H, d] bf16, seqlens_k int32 [B] on
    the GPU.  Returns (o [B, 1, H, d], lse [B, H])."""
    _check_tensor("q", q, torch.bfloat16, 4)
    _check_tensor("k_cache", k_cache, torch.bfloat16, 4)
    _check_tensor("v_cache", v_cache, torch.bfloat16, 4)
    _check_tensor("seqlens_k", seqlens_k, torch.int32, 1)
    B, one, H, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per sequence")
    if k_cache.shape[0] != B or k_cache.shape[2] != H or k_cache.shape[3] != d:
        raise ValueError("cache shape mismatch")
    if v_cache.shape != k_cache.shape or seqlens_k.numel() != B:
        raise ValueError("cache/seqlens shape mismatch")
    max_len = k_cache.shape[1]
    need = fa_decode_workspace_size(B, H, max_len, d, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace)
    o = torch.empty_like(q) if out is None else out
    _check_tensor("out", o, torch.bfloat16, 4)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if return_lse else None
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = fa_decode(q, k_cache, v_cache, seqlens_k, o, lse, B, H, max_len, d, s, chunk,
                   workspace, workspace.numel() * workspace.element_size(), stream)
    if st != FA_OK:
        raise FAError(st, "fa_decode")
    return o, lse


def attention_fp8(q, k, v, descale_q, descale_k, descale_v, *, scale=None, causal=False,
                  window_left=-1, return_lse=True, stream=None):
    """Dense attention on e4m3 codes: q [B, n_q, H, 128], k/v [B, n_k, H, 128]
    torch.uint8 (or torch.float8_e4m3fn) on the GPU, descale_* fp32 [B * H]
    (or [B, H]).  Returns (o [B, n_q, H, 128] bf16, lse [B, H, n_q] fp32 or None)."""
    q, k, v = (t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t for t in (q, k, v))
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.uint8, 4)
    B, n_q, H, d = q.shape
    if k.shape[0] != B or k.shape[2] != H or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    n_k = k.shape[1]
    ds = []
    for name, t in (("descale_q", descale_q), ("descale_k", descale_k), ("descale_v", descale_v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.float32:
            raise ValueError(f"{name} must be a float32 tensor on the GPU")
        if t.numel() != B * H or not t.is_contiguous():
            raise ValueError(f"{name} must hold batch * heads contiguous values")
        ds.append(t)
    o = torch.empty((B, n_q, H, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device) if return_lse else None
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = fa_fwd_fp8(q, k, v, o, lse, ds[0], ds[1], ds[2], B, H, n_q, n_k, d, s, int(causal),
                    int(window_left), stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_fp8")
    return o, lse
