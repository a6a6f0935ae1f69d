"""ctypes binding of libattnres.so: its C-ABI entry points, same names.

Argument marshalling only.  Tensors are passed by device pointer together with
the current HIP stream; every computation happens in the library's gfx950
kernels.  There is no fallback: if the library is missing or a tensor is not
on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattnres.so")

F32, BF16, P24 = 0, 1, 2
ATTNRES_MAX_D = 16384
ATTNRES_MAX_SOURCES = 32
ATTNRES_MAX_SOURCES_MULTI = 16
ATTNRES_MAX_GROUP_SOURCES = 16
ATTNRES_MAX_T = 2147483647
ATTNRES_MAX_QUERIES = 4096
ATTNRES_MAX_STRIDE = 1 << 40

EXPORTED = ("attnres_phase1", "attnres_phase1_first_prenorm", "attnres_phase1_workspace_bytes", "attnres_phase2_merge", "attnres_phase2_merge_multi",
            "attnres_full", "attnres_block_accumulate", "attnres_site_backward", "attnres_site_backward_workspace_bytes",
            "attnres_phase2_backward", "attnres_phase2_backward_workspace_bytes", "attnres_phase1_backward",
            "attnres_phase1_backward_workspace_bytes", "attnres_status_string")


class AttnResError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__("%s failed: %s (status %d)" % (fn, msg, code))
        self.code = code


_lib = None


def load(path: Optional[str] = None):
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libattnres.so not found at %s: build it with "
                           "`python -m transformer_depth_wise_amd.build`" % p)
    lib = ctypes.CDLL(p)
    V, I, F, E = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.attnres_phase1.argtypes = [E, V, I, I, I, I, V, V, I, F, V, V, V, V, I, V]
    lib.attnres_phase1_first_prenorm.argtypes = [E, V, I, I, I, I, V, V, I, F, V, V, V, V, V, V, V, I, V]
    lib.attnres_phase1_workspace_bytes.argtypes = [I, I, I, I]
    lib.attnres_phase1_workspace_bytes.restype = ctypes.c_int64
    lib.attnres_phase2_merge.argtypes = [E, I, I, V, V, E, V, V, V, E, V, V, V, V, F, V, V, V]
    lib.attnres_phase2_merge_multi.argtypes = [E, I, I, V, V, V, I, I, V, V, V, F, V, V, V]
    lib.attnres_full.argtypes = [E, V, I, I, I, I, V, V, V, F, V, V, V, V]
    lib.attnres_site_backward.argtypes = [E, V, I, I, I, I, V, V, V, E, F, V, V, I, V, V, V, V, I, V]
    lib.attnres_site_backward_workspace_bytes.argtypes = [I, I]
    lib.attnres_site_backward_workspace_bytes.restype = ctypes.c_int64
    lib.attnres_block_accumulate.argtypes = [E, I, I, E, V, V, V, V, V]
    lib.attnres_phase2_backward.argtypes = [E, I, I, V, V, E, V, V, V, V, V, V, E, F, V, V, V, V, V, V, V, V, V, I,
                                            V]
    lib.attnres_phase2_backward_workspace_bytes.argtypes = [I, I]
    lib.attnres_phase2_backward_workspace_bytes.restype = ctypes.c_int64
    lib.attnres_phase1_backward.argtypes = [E, V, I, I, I, I, V, V, I, F, V, I, V, V, V, I, E, V, V, V, I, V]
    lib.attnres_phase1_backward_workspace_bytes.argtypes = [I, I, I, I]
    lib.attnres_phase1_backward_workspace_bytes.restype = ctypes.c_int64
    for fn in ("attnres_phase1", "attnres_phase1_first_prenorm", "attnres_phase2_merge", "attnres_phase2_merge_multi", "attnres_full",
               "attnres_block_accumulate", "attnres_site_backward", "attnres_phase2_backward",
               "attnres_phase1_backward"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.attnres_status_string.argtypes = [ctypes.c_int]
    lib.attnres_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().attnres_status_string(int(code)).decode()


def dtype_code(t: torch.dtype) -> int:
    """float32 -> F32, bfloat16 -> BF16; a uint8 tensor holds a partial sum in
    the 24-bit split format (P24, 3 bytes per element)."""
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    if t == torch.uint8:
        return P24
    raise TypeError("unsupported storage dtype %s (float32, bfloat16, or uint8 for a P24 partial)" % t)


def p24_partial(T: int, d: int, device) -> torch.Tensor:
    """An uninitialised partial-sum buffer in the P24 format."""
    return torch.empty((3 * T * d,), dtype=torch.uint8, device=device)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor is not on a GPU; the AttnRes library computes on the GPU only")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, rc: int):
    if rc != 0:
        raise AttnResError(fn, rc, status_string(rc))


def attnres_phase1_workspace_bytes(T: int, d: int, n_src: int, S: int) -> int:
    return int(load().attnres_phase1_workspace_bytes(T, d, n_src, S))


def attnres_phase1(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                   eps: float, out: Optional[torch.Tensor], m_out: Optional[torch.Tensor], lse_out: torch.Tensor,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """src: [>=n_src, T, d] slabs (sources 0..n_src-1 at stride src.stride(0));
    w, key_gain: [S, d] fp32; out: [S, T, d] or None (statistics only);
    m_out, lse_out: [S, T] fp32; workspace: device tensor of at least
    attnres_phase1_workspace_bytes bytes."""
    S, T = lse_out.shape
    d = src.shape[-1]
    stride = src.stride(0) if src.dim() == 3 else T * d
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().attnres_phase1(dtype_code(src.dtype), _ptr(src), n_src, stride, T, d, _ptr(w), _ptr(key_gain),
                               S, eps, _ptr(out), _ptr(m_out), _ptr(lse_out), _ptr(workspace), ws_bytes,
                               _stream(stream))
    _check("attnres_phase1", rc)


def attnres_phase1_first_prenorm(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                                 eps: float, out: Optional[torch.Tensor], m_out: Optional[torch.Tensor],
                                 lse_out: torch.Tensor, prenorm_gain: Optional[torch.Tensor], x_out: torch.Tensor,
                                 h_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                 stream=None) -> None:
    """As attnres_phase1, but query 0's output goes through the PreNorm into
    x_out ([T, d]; and as is into h_out when given) instead of out[0], which
    is scratch; out may be None only when n_src == 1."""
    S, T = lse_out.shape
    d = src.shape[-1]
    stride = src.stride(0) if src.dim() == 3 else T * d
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().attnres_phase1_first_prenorm(dtype_code(src.dtype), _ptr(src), n_src, stride, T, d, _ptr(w),
                                             _ptr(key_gain), S, eps, _ptr(out), _ptr(m_out), _ptr(lse_out),
                                             _ptr(prenorm_gain), _ptr(x_out), _ptr(h_out), _ptr(workspace),
                                             ws_bytes, _stream(stream))
    _check("attnres_phase1_first_prenorm", rc)


def attnres_phase2_merge(p1_out: torch.Tensor, p1_lse: torch.Tensor, partial_in: Optional[torch.Tensor],
                         sublayer_prev: Optional[torch.Tensor], partial_out: Optional[torch.Tensor],
                         w: torch.Tensor, key_gain: Optional[torch.Tensor], prenorm_gain: Optional[torch.Tensor],
                         eps: float, h_out: Optional[torch.Tensor], x_out: Optional[torch.Tensor],
                         stream=None, sublayer_prev2: Optional[torch.Tensor] = None) -> None:
    """p1_out: [T, d]; p1_lse: [T]; partial_in: [T, d] fp32 / storage dtype, or
    a P24 buffer; sublayer_prev, sublayer_prev2: [T, d] (partial sum
    p = partial_in + sublayer_prev2 + sublayer_prev, absent terms zero);
    partial_out: [T, d] fp32 or a P24 buffer; w, key_gain, prenorm_gain: [d]."""
    T, d = p1_out.shape
    pdt = dtype_code(partial_in.dtype) if partial_in is not None else F32
    podt = dtype_code(partial_out.dtype) if partial_out is not None else F32
    rc = load().attnres_phase2_merge(dtype_code(p1_out.dtype), T, d, _ptr(p1_out), _ptr(p1_lse), pdt,
                                     _ptr(partial_in), _ptr(sublayer_prev2), _ptr(sublayer_prev), podt,
                                     _ptr(partial_out), _ptr(w), _ptr(key_gain), _ptr(prenorm_gain), eps,
                                     _ptr(h_out), _ptr(x_out), _stream(stream))
    _check("attnres_phase2_merge", rc)


def attnres_phase2_merge_multi(p1_out: torch.Tensor, p1_lse: torch.Tensor, src: Optional[torch.Tensor], n_src: int,
                               w: Optional[torch.Tensor], key_gain: Optional[torch.Tensor],
                               prenorm_gain: Optional[torch.Tensor], eps: float, h_out: Optional[torch.Tensor],
                               x_out: Optional[torch.Tensor], stream=None) -> None:
    """p1_out: [T, d]; p1_lse: [T]; src: [>=n_src, T, d] slabs (the group's
    outputs so far, each its own source; None when n_src == 0); w, gains: [d]."""
    T, d = p1_out.shape
    stride = 0 if src is None else (src.stride(0) if src.dim() == 3 else T * d)
    rc = load().attnres_phase2_merge_multi(dtype_code(p1_out.dtype), T, d, _ptr(p1_out), _ptr(p1_lse), _ptr(src),
                                           n_src, stride, _ptr(w), _ptr(key_gain), _ptr(prenorm_gain), eps,
                                           _ptr(h_out), _ptr(x_out), _stream(stream))
    _check("attnres_phase2_merge_multi", rc)


def attnres_full(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                 prenorm_gain: Optional[torch.Tensor], eps: float, h_out: Optional[torch.Tensor],
                 x_out: Optional[torch.Tensor], lse_out: Optional[torch.Tensor], stream=None) -> None:
    """src: [>=n_src, T, d]; w, gains: [d] fp32; h_out/x_out: [T, d]; lse_out: [T]."""
    T, d = src.shape[-2], src.shape[-1]
    stride = src.stride(0) if src.dim() == 3 else T * d
    rc = load().attnres_full(dtype_code(src.dtype), _ptr(src), n_src, stride, T, d, _ptr(w), _ptr(key_gain),
                             _ptr(prenorm_gain), eps, _ptr(h_out), _ptr(x_out), _ptr(lse_out), _stream(stream))
    _check("attnres_full", rc)


def attnres_site_backward_workspace_bytes(T: int, d: int) -> int:
    return int(load().attnres_site_backward_workspace_bytes(T, d))


def attnres_site_backward(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                          prenorm_gain: Optional[torch.Tensor], prenorm: bool, eps: float, dx: torch.Tensor,
                          dsrc: torch.Tensor, dw: torch.Tensor, dkey_gain: Optional[torch.Tensor],
                          dprenorm_gain: Optional[torch.Tensor], workspace: torch.Tensor, stream=None) -> None:
    """src, dsrc: [>=n_src, T, d] slabs; dx: [T, d]; w, gains and their
    gradients: [d] fp32; workspace: device tensor of at least
    attnres_site_backward_workspace_bytes(T, d) bytes."""
    T, d = dx.shape
    stride = src.stride(0) if src.dim() == 3 else T * d
    dstride = dsrc.stride(0) if dsrc.dim() == 3 else T * d
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = load().attnres_site_backward(dtype_code(src.dtype), _ptr(src), n_src, stride, T, d, _ptr(w), _ptr(key_gain),
                                      _ptr(prenorm_gain), 1 if prenorm else 0, eps, _ptr(dx), _ptr(dsrc), dstride,
                                      _ptr(dw), _ptr(dkey_gain), _ptr(dprenorm_gain), _ptr(workspace), ws_bytes,
                                      _stream(stream))
    _check("attnres_site_backward", rc)


def attnres_phase2_backward_workspace_bytes(T: int, d: int) -> int:
    return int(load().attnres_phase2_backward_workspace_bytes(T, d))


def attnres_phase2_backward(p1_out: torch.Tensor, p1_lse: Optional[torch.Tensor], partial_in: Optional[torch.Tensor],
                            sublayer_prev: Optional[torch.Tensor], w: torch.Tensor, key_gain: Optional[torch.Tensor],
                            prenorm_gain: Optional[torch.Tensor], eps: float, dx: torch.Tensor,
                            dpartial: Optional[torch.Tensor], g_out: torch.Tensor, c_out: torch.Tensor,
                            gp_out: torch.Tensor, dw: Optional[torch.Tensor], dkey_gain: Optional[torch.Tensor],
                            dprenorm_gain: Optional[torch.Tensor], workspace: torch.Tensor, prenorm: bool = True,
                            sublayer_prev2: Optional[torch.Tensor] = None, stream=None) -> None:
    """One site's phase-2 backward: p1_out, dx, g_out: [T, d]; p1_lse, c_out
    (1 - beta), gp_out (G.p): [T]; the partial source as for
    attnres_phase2_merge; dpartial:
    [T, d] fp32, added to in place; dw, dkey_gain, dprenorm_gain: [d] fp32,
    added to."""
    T, d = p1_out.shape
    pdt = dtype_code(partial_in.dtype) if partial_in is not None else F32
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = load().attnres_phase2_backward(dtype_code(p1_out.dtype), T, d, _ptr(p1_out), _ptr(p1_lse), pdt,
                                        _ptr(partial_in), _ptr(sublayer_prev2), _ptr(sublayer_prev), _ptr(w),
                                        _ptr(key_gain), _ptr(prenorm_gain), 1 if prenorm else 0, eps, _ptr(dx),
                                        _ptr(dpartial), _ptr(g_out), _ptr(c_out), _ptr(gp_out), _ptr(dw),
                                        _ptr(dkey_gain), _ptr(dprenorm_gain), _ptr(workspace), ws_bytes,
                                        _stream(stream))
    _check("attnres_phase2_backward", rc)


def attnres_phase1_backward_workspace_bytes(T: int, d: int, n_src: int, S: int) -> int:
    return int(load().attnres_phase1_backward_workspace_bytes(T, d, n_src, S))


def attnres_phase1_backward(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                            eps: float, g_in: torch.Tensor, c_in: Optional[torch.Tensor],
                            gp_in: Optional[torch.Tensor], dsrc: torch.Tensor, dw: torch.Tensor,
                            dkey_gain: Optional[torch.Tensor], workspace: torch.Tensor, accumulate: bool = False,
                            stream=None) -> None:
    """The block sources' part of S sites: src: [>=n_src, T, d]; w, key_gain,
    dw, dkey_gain: [S, d] fp32; g_in: [S, T, d]; c_in, gp_in: [S, T] or None;
    dsrc: [>=n_src, T, d] fp32, written or (accumulate) added to."""
    S, d = w.shape
    T = g_in.shape[-2]
    stride = src.stride(0) if src.dim() == 3 else T * d
    gstride = g_in.stride(0) if g_in.dim() == 3 else T * d
    dstride = dsrc.stride(0) if dsrc.dim() == 3 else T * d
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = load().attnres_phase1_backward(dtype_code(src.dtype), _ptr(src), n_src, stride, T, d, _ptr(w), _ptr(key_gain),
                                        S, eps, _ptr(g_in), gstride, _ptr(c_in), _ptr(gp_in), _ptr(dsrc), dstride,
                                        1 if accumulate else 0, _ptr(dw), _ptr(dkey_gain), _ptr(workspace), ws_bytes,
                                        _stream(stream))
    _check("attnres_phase1_backward", rc)


def attnres_block_accumulate(partial_in: Optional[torch.Tensor], v: torch.Tensor, out: torch.Tensor,
                             stream=None, v2: Optional[torch.Tensor] = None) -> None:
    """out = (partial_in or 0) + (v2 or 0) + v; all [T, d] (partial_in may be
    a P24 buffer)."""
    T, d = v.shape
    pdt = dtype_code(partial_in.dtype) if partial_in is not None else F32
    rc = load().attnres_block_accumulate(dtype_code(v.dtype), T, d, pdt, _ptr(partial_in), _ptr(v2), _ptr(v),
                                         _ptr(out), _stream(stream))
    _check("attnres_block_accumulate", rc)
