"""ctypes binding of libfa.so (the C ABI declared in include/fa.h).

Argument marshalling only: shapes are checked, outputs allocated with torch,
and device pointers plus torch's current HIP stream are handed to the C entry
points of the same names. Every step of the computation runs in the library's
HIP kernels; there is no fallback of any kind. If libfa.so is missing or
cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
_lib = None

# name -> (restype, argtypes)
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "fa_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "fa_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P]),
    "fa_decode": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "fa_decode_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "fa_decode_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "fa_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _S, _P]),
    "fa_bwd_workspace_bytes": (_S, [_I, _I, _I]),
    "fa_naive_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _S, _P]),
    "fa_naive_workspace_bytes": (_S, [_I, _I, _I]),
    "fa_status_str": (ctypes.c_char_p, [_I]),
    "fa_last_hip_error": (_I, []),
    "fa_shutdown": (None, []),
}


class FaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load()
        msg = f"{fn} failed: {lib.fa_status_str(status).decode()} ({status})"
        if status == -3:
            msg += f", hipError_t {lib.fa_last_hip_error()}"
        super().__init__(msg)
        self.status = status


def load():
    """Loads libfa.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first (python -m exact_io_aware_74_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(fn: str, status: int):
    if status != FA_OK:
        raise FaError(fn, status)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def default_scale(d: int) -> float:
    """1/sqrt(d), rounded to float32."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, return_lse: bool = True):
    """Fused attention forward. q, k, v: [B,H,N,d] bf16 (fa_fwd) or fp32 (fa_fwd_f32).

    Returns (o, lse); lse is [B,H,N] float32 (None if return_lse is False and
    no lse buffer is passed).
    """
    lib = load()
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or o.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    fn = "fa_fwd" if q.dtype == torch.bfloat16 else "fa_fwd_f32"
    with torch.cuda.device(q.device):
        st = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)),
                              scale, _stream(q))
    _check(fn, st)
    return o, lse


def fwd_fp8(q, k, v, descales, causal: bool = False, scale: float | None = None, out=None, lse=None,
            return_lse: bool = True):
    """Fused forward on FP8 (e4m3) inputs. q, k, v: [B,H,N,d] uint8 device tensors holding e4m3 codes
    (or torch.float8_e4m3fn); descales: (q_descale, k_descale, v_descale). Returns (o bf16, lse float32)."""
    lib = load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError(f"{name} must be a contiguous uint8 / float8_e4m3fn device tensor")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must have the same [B,H,N,d] shape")
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    qd, kd, vd = (float(x) for x in descales)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
    if o.shape != q.shape or o.dtype != torch.bfloat16 or not o.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor of q's shape")
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse if return_lse else None), B, H, N, d,
                            int(bool(causal)), scale, qd, kd, vd, _stream(q))
    _check("fa_fwd_fp8", st)
    return o, (lse if return_lse else None)


def decode(q, kcache, vcache, nsplit: int = 64, out=None, noalloc: bool = False):
    """Split-KV decode. q: [B,H,d] (or [B,H,1,d]) bf16; caches [B,H,Lkv,d] bf16. Returns o like q.

    noalloc=True calls fa_decode_noalloc (partials in the library's fixed per-device array; pass
    ``out`` as well to allocate nothing at all)."""
    lib = load()
    q3 = q.reshape(q.shape[0], q.shape[1], q.shape[-1]) if q.dim() == 4 else q
    for name, t in (("q", q3), ("kcache", kcache), ("vcache", vcache)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bfloat16 device tensor")
    if q3.dim() != 3 or kcache.dim() != 4 or kcache.shape != vcache.shape:
        raise ValueError("q must be [B,H,d]; kcache and vcache [B,H,Lkv,d]")
    B, H, d = q3.shape
    if kcache.shape[0] != B or kcache.shape[1] != H or kcache.shape[3] != d:
        raise ValueError("cache shape does not match q")
    Lkv = kcache.shape[2]
    o = torch.empty_like(q) if out is None else out
    if o.numel() != q3.numel() or o.dtype != torch.bfloat16 or not o.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor like q")
    fn = "fa_decode_noalloc" if noalloc else "fa_decode"
    with torch.cuda.device(q.device):
        st = getattr(lib, fn)(_ptr(q3), _ptr(kcache), _ptr(vcache), _ptr(o), B, H, Lkv, d, int(nsplit), _stream(q))
    _check(fn, st)
    return o


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, nsplit: int = 64, out=None):
    """Split-KV decode over a paged cache.

    q: [B,H,d] (or [B,H,1,d]) bf16; k_pages, v_pages: [num_pages,H,page_size,d]
    bf16 pools; block_table: int32 [B,max_pages] and seq_lens: int32 [B], both
    on the device. Returns o like q.
    """
    lib = load()
    q3 = q.reshape(q.shape[0], q.shape[1], q.shape[-1]) if q.dim() == 4 else q
    for name, t in (("q", q3), ("k_pages", k_pages), ("v_pages", v_pages)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bfloat16 device tensor")
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.int32:
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if q3.dim() != 3 or k_pages.dim() != 4 or k_pages.shape != v_pages.shape or block_table.dim() != 2:
        raise ValueError("q must be [B,H,d], the pools [num_pages,H,page_size,d], block_table [B,max_pages]")
    B, H, d = q3.shape
    num_pages, ph, page_size, pd = k_pages.shape
    if ph != H or pd != d or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("pool, table or length shapes do not match q")
    o = torch.empty_like(q) if out is None else out
    if o.numel() != q3.numel() or o.dtype != torch.bfloat16 or not o.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor like q")
    with torch.cuda.device(q.device):
        st = lib.fa_decode_paged(_ptr(q3), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), _ptr(o),
                                 B, H, d, page_size, num_pages, block_table.shape[1], int(nsplit), _stream(q))
    _check("fa_decode_paged", st)
    return o


def bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load().fa_bwd_workspace_bytes(B, H, N))


def bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None, out=None, workspace=None):
    """Gradients (dq, dk, dv) of fwd(q, k, v, causal, scale) for the upstream gradient dout.

    q, k, v, o, dout: [B,H,N,d] bfloat16; lse: the float32 [B,H,N] that fwd
    returned. ``out`` may pass preallocated (dq, dk, dv); ``workspace`` a
    device buffer of at least bwd_workspace_bytes(B, H, N) bytes.
    """
    lib = load()
    _check_qkv(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("bwd takes bfloat16 tensors")
    for name, t in (("o", o), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like q")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be the contiguous float32 [B, H, N] tensor fwd returned")
    scale = default_scale(d) if scale is None else float(scale)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3)) if out is None else out
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like q")
    need = bwd_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 16) // 4, dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                        B, H, N, d, int(bool(causal)), scale, _ptr(workspace),
                        workspace.numel() * workspace.element_size(), _stream(q))
    _check("fa_bwd", st)
    return dq, dk, dv


def naive_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load().fa_naive_workspace_bytes(B, H, N))


def decode_workspace_bytes(B: int, H: int, Lkv: int, d: int, nsplit: int) -> int:
    return int(load().fa_decode_workspace_bytes(B, H, Lkv, d, nsplit))


def naive_fwd(q, k, v, causal: bool = False, scale: float | None = None, workspace=None, out=None, lse=None):
    """The three-kernel ablation (S and P materialised in HBM). bf16 q, k, v. Returns (o, lse).

    ``out`` and ``lse`` may pass preallocated outputs, ``workspace`` a float32 device buffer of at least
    naive_workspace_bytes(B, H, N) bytes."""
    lib = load()
    _check_qkv(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("naive_fwd takes bfloat16 inputs")
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    need = naive_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=q.device)
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or o.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    with torch.cuda.device(q.device):
        st = lib.fa_naive_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)), scale,
                              _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q))
    _check("fa_naive_fwd", st)
    return o, lse


def shutdown():
    load().fa_shutdown()
