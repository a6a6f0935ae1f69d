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

F32, BF16, P24, Q16 = 0, 1, 2, 3
ATTNRES_MAX_D = 16384
ATTNRES_MAX_SOURCES = 32
ATTNRES_MAX_SOURCES_MULTI = 16
ATTNRES_MAX_GROUP_SOURCES = 16
ATTNRES_MAX_T = 2147483647
ATTNRES_MAX_QUERIES = 4096
ATTNRES_MAX_STRIDE = 1 << 40
ATTNRES_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED = ("attnres_phase1", "attnres_phase1_first_prenorm", "attnres_phase1_workspace_bytes",
            "attnres_phase2_merge", "attnres_phase2_merge_multi", "attnres_full", "attnres_block_accumulate",
            "attnres_site_backward", "attnres_site_backward_accumulate", "attnres_site_backward_workspace_bytes",
            "attnres_phase2_backward", "attnres_phase2_backward_workspace_bytes", "attnres_phase1_backward",
            "attnres_phase1_backward_workspace_bytes", "attnres_stream_probe", "attnres_phase1_noalloc",
            "attnres_phase1_accumulate", "attnres_status_string")


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
    lib.attnres_phase1.argtypes = [E, E, V, I, I, I, I, V, V, I, F, V, V, V, V, I, V]
    lib.attnres_phase1_first_prenorm.argtypes = [E, V, I, I, I, I, V, V, I, F, V, V, V, V, V, V, V, I, V]
    lib.attnres_phase1_accumulate.argtypes = [E, E, V, I, I, I, I, V, V, I, F, E, V, E, V, V, V, V, V, V, V, V, V,
                                              I, V]
    lib.attnres_phase1_workspace_bytes.argtypes = [I, I, I, I]
    lib.attnres_phase1_workspace_bytes.restype = ctypes.c_int64
    lib.attnres_phase2_merge.argtypes = [E, I, I, V, V, E, V, V, V, E, V, V, V, V, F, V, V, V]
    lib.attnres_phase2_merge_multi.argtypes = [E, I, I, V, V, V, I, I, V, V, V, F, V, V, V]
    lib.attnres_full.argtypes = [E, V, I, I, I, I, V, V, V, F, V, V, V, V]
    lib.attnres_site_backward.argtypes = [E, V, I, I, I, I, V, V, V, E, F, V, V, I, V, V, V, V, I, V]
    lib.attnres_site_backward_accumulate.argtypes = lib.attnres_site_backward.argtypes
    lib.attnres_site_backward_workspace_bytes.argtypes = [I, I]
    lib.attnres_site_backward_workspace_bytes.restype = ctypes.c_int64
    lib.attnres_block_accumulate.argtypes = [E, I, I, E, V, V, V, V, E, V]
    lib.attnres_phase2_backward.argtypes = [E, I, I, V, V, E, V, V, V, V, V, V, E, F, V, V, V, V, V, V, V, V, V, I,
                                            V]
    lib.attnres_phase2_backward_workspace_bytes.argtypes = [I, I]
    lib.attnres_phase2_backward_workspace_bytes.restype = ctypes.c_int64
    lib.attnres_phase1_backward.argtypes = [E, E, V, I, I, I, I, V, V, I, F, V, I, V, V, V, I, E, V, V, V, I, V]
    lib.attnres_phase1_backward_workspace_bytes.argtypes = [I, I, I, I]
    lib.attnres_phase1_backward_workspace_bytes.restype = ctypes.c_int64
    lib.attnres_stream_probe.argtypes = [I, I, V, V, I, I, I, I, V]
    lib.attnres_phase1_noalloc.argtypes = [E, V, I, I, I, I, V, V, I, F, V, V, V, V]
    for fn in ("attnres_phase1_noalloc", "attnres_stream_probe", "attnres_phase1", "attnres_phase1_first_prenorm",
               "attnres_phase1_accumulate", "attnres_phase2_merge", "attnres_phase2_merge_multi",
               "attnres_full", "attnres_block_accumulate", "attnres_site_backward",
               "attnres_site_backward_accumulate", "attnres_phase2_backward", "attnres_phase1_backward"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.attnres_status_string.argtypes = [ctypes.c_int]
    lib.attnres_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().attnres_status_string(int(code)).decode()


def dtype_code(t: torch.dtype) -> int:
    """float32 -> F32, bfloat16 -> BF16; a uint8 tensor holds a partial sum in
    the 24-bit split format (P24, 3 bytes per element), an int16 tensor one in
    the 16-bit fixed-point format with row exponents (Q16)."""
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    if t == torch.uint8:
        return P24
    if t == torch.int16:
        return Q16
    raise TypeError("unsupported storage dtype %s (float32, bfloat16, or uint8 / int16 for a P24 / Q16 partial)" % t)


def p24_partial(T: int, d: int, device) -> torch.Tensor:
    """An uninitialised partial-sum buffer in the P24 format."""
    return torch.empty((3 * T * d,), dtype=torch.uint8, device=device)


def q16_partial(T: int, d: int, device) -> torch.Tensor:
    """An uninitialised partial-sum buffer in the Q16 format: T*d int16 values
    followed by T int32 row exponents (2 int16 elements each)."""
    return torch.empty((T * d + 2 * T,), dtype=torch.int16, device=device)


def _pow2(k: torch.Tensor) -> torch.Tensor:
    """Exactly 2^k in fp32 for integer k in [-126, 127] (built from its bits)."""
    return ((k + 127).to(torch.int32) << 23).view(torch.float32)


def q16_decode(buf: torch.Tensor, T: int, d: int) -> torch.Tensor:
    """The fp32 values of a Q16 partial: q * 2^(e - 15) per row, exact (for
    inspection and tests; the scale is applied as two exact powers of two)."""
    q = buf[:T * d].view(T, d).float()
    k = buf[T * d:T * d + 2 * T].view(torch.int32).view(T, 1) - 15
    k1 = torch.div(k, 2, rounding_mode="floor")
    return q * _pow2(k1) * _pow2(k - k1)


def _rows(t: Optional[torch.Tensor], name: str, T: int, d: int, dtype: torch.dtype, n: int = 1,
          optional: bool = False) -> int:
    """Check a [T, d] row set, or slabs [k >= n, T, d]: dtype, shape and
    contiguous rows (the slab stride is free).  Returns the slab stride in
    elements (T * d for a single [T, d] row set)."""
    if t is None:
        if optional:
            return 0
        raise ValueError("%s is required" % name)
    if t.dtype != dtype:
        raise TypeError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    sh = t.shape
    if len(sh) == 2 and n <= 1 and sh[0] == T and sh[1] == d:
        if t.is_contiguous():
            return T * d
        st = t.stride()
    elif len(sh) == 3 and sh[0] >= n and sh[1] == T and sh[2] == d:
        st = t.stride()
        if (d <= 1 or st[2] == 1) and (T <= 1 or st[1] == d):
            return st[0]
    else:
        raise ValueError("%s: shape %s, expected [%d, %d] or [>= %d, %d, %d]" % (name, tuple(sh), T, d, n, T, d))
    if (d > 1 and st[-1] != 1) or (T > 1 and st[-2] != d):
        raise ValueError("%s: rows must be contiguous (strides %s)" % (name, st))
    return T * d


def _fp32(t: Optional[torch.Tensor], name: str, shape: tuple, optional: bool = True) -> None:
    """Check a contiguous fp32 tensor of `shape` (leading size-1 dimensions
    may be present or absent)."""
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if t.dtype != torch.float32:
        raise TypeError("%s: dtype %s, expected torch.float32" % (name, t.dtype))
    sh = t.shape
    if sh == shape and t.is_contiguous():
        return
    got = tuple(sh)
    while len(got) > len(shape) and got[0] == 1:
        got = got[1:]
    want = tuple(shape)
    while len(want) > len(got) and want[0] == 1:
        want = want[1:]
    if got != want or not t.is_contiguous():
        raise ValueError("%s: shape %s (contiguous: %s), expected contiguous %s"
                         % (name, tuple(sh), t.is_contiguous(), tuple(shape)))


def _partial(t: Optional[torch.Tensor], name: str, T: int, d: int, dtype: torch.dtype,
             allow_storage: bool = True) -> int:
    """A running partial sum: fp32 [T, d], a P24 buffer (uint8, >= 3 T d
    bytes, contiguous), or (where allowed) [T, d] in the storage dtype.
    Returns its format code (F32 when absent)."""
    if t is None:
        return F32
    if t.dtype == torch.uint8:
        if not t.is_contiguous() or t.numel() < 3 * T * d:
            raise ValueError("%s: a P24 partial needs a contiguous uint8 buffer of >= %d bytes" % (name, 3 * T * d))
        return P24
    if t.dtype == torch.int16:
        if not t.is_contiguous() or t.numel() < T * d + 2 * T:
            raise ValueError("%s: a Q16 partial needs a contiguous int16 buffer of >= %d elements"
                             % (name, T * d + 2 * T))
        if t.data_ptr() % 16:
            raise ValueError("%s: a Q16 partial must be 16-byte aligned" % name)
        return Q16
    if t.dtype != torch.float32 and not (allow_storage and t.dtype == dtype):
        raise TypeError("%s: dtype %s, expected float32, uint8 (P24), int16 (Q16)%s"
                        % (name, t.dtype, (" or %s" % dtype) if allow_storage else ""))
    _rows(t, name, T, d, t.dtype)
    return dtype_code(t.dtype)


def _workspace(t: Optional[torch.Tensor], name: str = "workspace") -> int:
    """A contiguous device buffer; returns its size in bytes (0 when absent)."""
    if t is None:
        return 0
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.numel() * t.element_size()


def _storage(t: torch.Tensor, name: str) -> torch.dtype:
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("%s: rows must be float32 or bfloat16, got %s" % (name, t.dtype))
    return t.dtype


def _on_device(*ts: Optional[torch.Tensor]) -> None:
    """Every tensor given lives on the current GPU (the library launches on
    the current device's stream)."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensor is not on a GPU; the AttnRes library computes on the GPU only")
        if dev is None:
            dev = torch.cuda.current_device()
        if t.device.index != dev:
            raise ValueError("tensor on %s, but the current device is cuda:%d" % (t.device, dev))


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


def _fmt(t: Optional[torch.Tensor]) -> int:
    return F32 if t is None else dtype_code(t.dtype)


def _slab_stride(t: Optional[torch.Tensor], T: int, d: int) -> int:
    return 0 if t is None else (t.stride(0) if t.dim() == 3 else T * d)


# Every call below checks its tensors (dtype, shape, contiguous rows, current
# device) unless ``check=False``: a caller that built the tensors itself and
# checked them once (the driver) skips the per-call Python cost.  The C ABI
# validates sizes, alignment and aliasing either way.

def attnres_phase1_workspace_bytes(T: int, d: int, n_src: int, S: int) -> int:
    return int(load().attnres_phase1_workspace_bytes(T, d, n_src, S))


def _phase1_args(src, n_src, w, key_gain, out, m_out, lse_out):
    if lse_out is None or lse_out.dim() != 2:
        raise ValueError("lse_out must be an [S, T] fp32 tensor")
    S, T = lse_out.shape
    d = src.shape[-1]
    dt = _storage(src, "src")
    _rows(src, "src", T, d, dt, n=n_src)
    _fp32(w, "w", (S, d), optional=False)
    _fp32(key_gain, "key_gain", (S, d))
    # outputs of the sources' dtype, or bf16 outputs from fp32 sources
    odt = torch.bfloat16 if (out is not None and dt == torch.float32 and out.dtype == torch.bfloat16) else dt
    if out is not None and (out.dtype != odt or tuple(out.shape) != (S, T, d) or not out.is_contiguous()):
        raise ValueError("out: expected a contiguous [%d, %d, %d] %s tensor, got %s %s"
                         % (S, T, d, dt, out.dtype, tuple(out.shape)))
    _fp32(m_out, "m_out", (S, T))
    _fp32(lse_out, "lse_out", (S, T), optional=False)


def attnres_phase1(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                   eps: float, out: Optional[torch.Tensor], m_out: Optional[torch.Tensor], lse_out: torch.Tensor,
                   workspace: Optional[torch.Tensor] = None, stream=None, check: bool = True) -> None:
    """src: [>=n_src, T, d] slabs (sources 0..n_src-1 at stride src.stride(0));
    w, key_gain: [S, d] fp32; out: [S, T, d] or None (statistics only);
    m_out, lse_out: [S, T] fp32; workspace: device tensor of at least
    attnres_phase1_workspace_bytes bytes."""
    if check:
        _phase1_args(src, n_src, w, key_gain, out, m_out, lse_out)
        _workspace(workspace)
        _on_device(src, w, key_gain, out, m_out, lse_out, workspace)
    S, T = lse_out.shape
    d = src.shape[-1]
    out_dt = out.dtype if out is not None else src.dtype
    rc = load().attnres_phase1(dtype_code(out_dt), dtype_code(src.dtype), _ptr(src), n_src, _slab_stride(src, T, d),
                               T, d, _ptr(w),
                               _ptr(key_gain), S, eps, _ptr(out), _ptr(m_out), _ptr(lse_out), _ptr(workspace),
                               _workspace(workspace), _stream(stream))
    _check("attnres_phase1", rc)


def attnres_phase1_noalloc(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                           eps: float, out: Optional[torch.Tensor], m_out: Optional[torch.Tensor],
                           lse_out: torch.Tensor, stream=None, check: bool = True) -> None:
    """attnres_phase1 with the library's own device scratch as workspace
    (allocates nothing; calls overlapping in time on one GPU race on it)."""
    if check:
        _phase1_args(src, n_src, w, key_gain, out, m_out, lse_out)
        _on_device(src, w, key_gain, out, m_out, lse_out)
    S, T = lse_out.shape
    d = src.shape[-1]
    rc = load().attnres_phase1_noalloc(dtype_code(src.dtype), _ptr(src), n_src, _slab_stride(src, T, d), T, d,
                                       _ptr(w), _ptr(key_gain), S, eps, _ptr(out), _ptr(m_out), _ptr(lse_out),
                                       _stream(stream))
    _check("attnres_phase1_noalloc", rc)


def attnres_phase1_first_prenorm(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                                 eps: float, out: Optional[torch.Tensor], m_out: Optional[torch.Tensor],
                                 lse_out: torch.Tensor, prenorm_gain: Optional[torch.Tensor], x_out: torch.Tensor,
                                 h_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                 stream=None, check: bool = True) -> None:
    """As attnres_phase1, but query 0's output goes through the PreNorm into
    x_out ([T, d]; and as is into h_out when given) instead of out[0], which
    is scratch; out may be None only when n_src == 1."""
    if check:
        _phase1_args(src, n_src, w, key_gain, out, m_out, lse_out)
        T, d = lse_out.shape[1], src.shape[-1]
        _fp32(prenorm_gain, "prenorm_gain", (d,))
        _rows(x_out, "x_out", T, d, src.dtype)
        _rows(h_out, "h_out", T, d, src.dtype, optional=True)
        _workspace(workspace)
        _on_device(src, w, key_gain, out, m_out, lse_out, prenorm_gain, x_out, h_out, workspace)
    S, T = lse_out.shape
    d = src.shape[-1]
    rc = load().attnres_phase1_first_prenorm(dtype_code(src.dtype), _ptr(src), n_src, _slab_stride(src, T, d), T,
                                             d, _ptr(w), _ptr(key_gain), S, eps, _ptr(out), _ptr(m_out),
                                             _ptr(lse_out), _ptr(prenorm_gain), _ptr(x_out), _ptr(h_out),
                                             _ptr(workspace), _workspace(workspace), _stream(stream))
    _check("attnres_phase1_first_prenorm", rc)


def attnres_phase1_accumulate(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                              eps: float, partial_in: Optional[torch.Tensor], v2: Optional[torch.Tensor],
                              v: torch.Tensor, out: Optional[torch.Tensor], m_out: Optional[torch.Tensor],
                              lse_out: torch.Tensor, prenorm_gain: Optional[torch.Tensor] = None,
                              x_out: Optional[torch.Tensor] = None, h_out: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None, stream=None, check: bool = True) -> None:
    """attnres_phase1 (x_out None) or attnres_phase1_first_prenorm (x_out
    given) whose newest source src[n_src - 1] is first formed as
    (partial_in or 0) + (v2 or 0) + v and written there: v, v2 [T, d] sublayer
    outputs, partial_in a running partial (fp32, Q16 or P24 buffer, or v's
    dtype).  The outputs' dtype is out's (else the sources')."""
    if v is None or v.dim() != 2:
        raise ValueError("v must be a [T, d] tensor")
    odt = out.dtype if out is not None else src.dtype
    if check:
        _phase1_args(src, n_src, w, key_gain, out, m_out, lse_out)
        T, d = lse_out.shape[1], src.shape[-1]
        vdt = _storage(v, "v")
        _rows(v, "v", T, d, vdt)
        _rows(v2, "v2", T, d, vdt, optional=True)
        _partial(partial_in, "partial_in", T, d, vdt)
        _fp32(prenorm_gain, "prenorm_gain", (d,))
        _rows(x_out, "x_out", T, d, odt, optional=True)
        _rows(h_out, "h_out", T, d, odt, optional=True)
        _workspace(workspace)
        _on_device(src, w, key_gain, partial_in, v2, v, out, m_out, lse_out, prenorm_gain, x_out, h_out, workspace)
    S, T = lse_out.shape
    d = src.shape[-1]
    rc = load().attnres_phase1_accumulate(dtype_code(odt), dtype_code(src.dtype), _ptr(src), n_src,
                                          _slab_stride(src, T, d), T, d, _ptr(w), _ptr(key_gain), S, eps,
                                          _fmt(partial_in), _ptr(partial_in), dtype_code(v.dtype), _ptr(v2), _ptr(v),
                                          _ptr(out),
                                          _ptr(m_out), _ptr(lse_out), _ptr(prenorm_gain), _ptr(x_out), _ptr(h_out),
                                          _ptr(workspace), _workspace(workspace), _stream(stream))
    _check("attnres_phase1_accumulate", rc)


def attnres_phase2_merge(p1_out: torch.Tensor, p1_lse: torch.Tensor, partial_in: Optional[torch.Tensor],
                         sublayer_prev: Optional[torch.Tensor], partial_out: Optional[torch.Tensor],
                         w: torch.Tensor, key_gain: Optional[torch.Tensor], prenorm_gain: Optional[torch.Tensor],
                         eps: float, h_out: Optional[torch.Tensor], x_out: Optional[torch.Tensor],
                         stream=None, sublayer_prev2: Optional[torch.Tensor] = None, check: bool = True) -> None:
    """p1_out: [T, d]; p1_lse: [T]; partial_in: [T, d] fp32 / storage dtype, or
    a P24 buffer; sublayer_prev, sublayer_prev2: [T, d] (partial sum
    p = partial_in + sublayer_prev2 + sublayer_prev, absent terms zero);
    partial_out: [T, d] fp32 or a P24 buffer; w, key_gain, prenorm_gain: [d]."""
    if p1_out.dim() != 2:
        raise ValueError("p1_out must be a [T, d] tensor")
    T, d = p1_out.shape
    if check:
        dt = _storage(p1_out, "p1_out")
        _rows(p1_out, "p1_out", T, d, dt)
        _fp32(p1_lse, "p1_lse", (T,), optional=False)
        _partial(partial_in, "partial_in", T, d, dt)
        _partial(partial_out, "partial_out", T, d, dt, allow_storage=False)
        _rows(sublayer_prev, "sublayer_prev", T, d, dt, optional=True)
        _rows(sublayer_prev2, "sublayer_prev2", T, d, dt, optional=True)
        for t, name in ((w, "w"), (key_gain, "key_gain"), (prenorm_gain, "prenorm_gain")):
            _fp32(t, name, (d,))
        _rows(h_out, "h_out", T, d, dt, optional=True)
        _rows(x_out, "x_out", T, d, dt, optional=True)
        _on_device(p1_out, p1_lse, partial_in, sublayer_prev, sublayer_prev2, partial_out, w, key_gain,
                   prenorm_gain, h_out, x_out)
    rc = load().attnres_phase2_merge(dtype_code(p1_out.dtype), T, d, _ptr(p1_out), _ptr(p1_lse), _fmt(partial_in),
                                     _ptr(partial_in), _ptr(sublayer_prev2), _ptr(sublayer_prev), _fmt(partial_out),
                                     _ptr(partial_out), _ptr(w), _ptr(key_gain), _ptr(prenorm_gain), eps,
                                     _ptr(h_out), _ptr(x_out), _stream(stream))
    _check("attnres_phase2_merge", rc)


def attnres_phase2_merge_multi(p1_out: torch.Tensor, p1_lse: torch.Tensor, src: Optional[torch.Tensor], n_src: int,
                               w: Optional[torch.Tensor], key_gain: Optional[torch.Tensor],
                               prenorm_gain: Optional[torch.Tensor], eps: float, h_out: Optional[torch.Tensor],
                               x_out: Optional[torch.Tensor], stream=None, check: bool = True) -> None:
    """p1_out: [T, d]; p1_lse: [T]; src: [>=n_src, T, d] slabs (the group's
    outputs so far, each its own source; None when n_src == 0); w, gains: [d]."""
    if p1_out.dim() != 2:
        raise ValueError("p1_out must be a [T, d] tensor")
    T, d = p1_out.shape
    if check:
        dt = _storage(p1_out, "p1_out")
        _rows(p1_out, "p1_out", T, d, dt)
        _fp32(p1_lse, "p1_lse", (T,), optional=False)
        _rows(src, "src", T, d, dt, n=n_src, optional=n_src == 0)
        for t, name in ((w, "w"), (key_gain, "key_gain"), (prenorm_gain, "prenorm_gain")):
            _fp32(t, name, (d,))
        _rows(h_out, "h_out", T, d, dt, optional=True)
        _rows(x_out, "x_out", T, d, dt, optional=True)
        _on_device(p1_out, p1_lse, src, w, key_gain, prenorm_gain, h_out, x_out)
    rc = load().attnres_phase2_merge_multi(dtype_code(p1_out.dtype), T, d, _ptr(p1_out), _ptr(p1_lse), _ptr(src),
                                           n_src, _slab_stride(src, T, d), _ptr(w), _ptr(key_gain),
                                           _ptr(prenorm_gain), eps, _ptr(h_out), _ptr(x_out), _stream(stream))
    _check("attnres_phase2_merge_multi", rc)


def attnres_full(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                 prenorm_gain: Optional[torch.Tensor], eps: float, h_out: Optional[torch.Tensor],
                 x_out: Optional[torch.Tensor], lse_out: Optional[torch.Tensor], stream=None,
                 check: bool = True) -> None:
    """src: [>=n_src, T, d]; w, gains: [d] fp32; h_out/x_out: [T, d]; lse_out: [T]."""
    T, d = src.shape[-2], src.shape[-1]
    if check:
        dt = _storage(src, "src")
        _rows(src, "src", T, d, dt, n=n_src)
        _fp32(w, "w", (d,), optional=False)
        _fp32(key_gain, "key_gain", (d,))
        _fp32(prenorm_gain, "prenorm_gain", (d,))
        _rows(h_out, "h_out", T, d, dt, optional=True)
        _rows(x_out, "x_out", T, d, dt, optional=True)
        _fp32(lse_out, "lse_out", (T,))
        _on_device(src, w, key_gain, prenorm_gain, h_out, x_out, lse_out)
    rc = load().attnres_full(dtype_code(src.dtype), _ptr(src), n_src, _slab_stride(src, T, d), T, d, _ptr(w),
                             _ptr(key_gain), _ptr(prenorm_gain), eps, _ptr(h_out), _ptr(x_out), _ptr(lse_out),
                             _stream(stream))
    _check("attnres_full", rc)


def attnres_site_backward_workspace_bytes(T: int, d: int) -> int:
    return int(load().attnres_site_backward_workspace_bytes(T, d))


def attnres_site_backward(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                          prenorm_gain: Optional[torch.Tensor], prenorm: bool, eps: float, dx: torch.Tensor,
                          dsrc: torch.Tensor, dw: torch.Tensor, dkey_gain: Optional[torch.Tensor],
                          dprenorm_gain: Optional[torch.Tensor], workspace: torch.Tensor, stream=None,
                          check: bool = True) -> None:
    """src, dsrc: [>=n_src, T, d] slabs; dx: [T, d]; w, gains and their
    gradients: [d] fp32; workspace: device tensor of at least
    attnres_site_backward_workspace_bytes(T, d) bytes."""
    if dx.dim() != 2:
        raise ValueError("dx must be a [T, d] tensor")
    T, d = dx.shape
    if check:
        dt = _storage(src, "src")
        _rows(src, "src", T, d, dt, n=n_src)
        _rows(dx, "dx", T, d, dt)
        _rows(dsrc, "dsrc", T, d, dt, n=n_src)
        for t, name in ((w, "w"), (key_gain, "key_gain"), (prenorm_gain, "prenorm_gain"), (dw, "dw"),
                        (dkey_gain, "dkey_gain"), (dprenorm_gain, "dprenorm_gain")):
            _fp32(t, name, (d,), optional=name not in ("w", "dw"))
        _workspace(workspace)
        _on_device(src, dx, dsrc, w, key_gain, prenorm_gain, dw, dkey_gain, dprenorm_gain, workspace)
    rc = load().attnres_site_backward(dtype_code(src.dtype), _ptr(src), n_src, _slab_stride(src, T, d), T, d,
                                      _ptr(w), _ptr(key_gain), _ptr(prenorm_gain), 1 if prenorm else 0, eps,
                                      _ptr(dx), _ptr(dsrc), _slab_stride(dsrc, T, d), _ptr(dw), _ptr(dkey_gain),
                                      _ptr(dprenorm_gain), _ptr(workspace), _workspace(workspace),
                                      _stream(stream))
    _check("attnres_site_backward", rc)


def attnres_site_backward_accumulate(src: torch.Tensor, n_src: int, w: torch.Tensor,
                                     key_gain: Optional[torch.Tensor], prenorm_gain: Optional[torch.Tensor],
                                     prenorm: bool, eps: float, dx: torch.Tensor, dsrc: torch.Tensor,
                                     dw: torch.Tensor, dkey_gain: Optional[torch.Tensor],
                                     dprenorm_gain: Optional[torch.Tensor], workspace: torch.Tensor, stream=None,
                                     check: bool = True) -> None:
    """As attnres_site_backward, but dL/du_i is added to dsrc: [>=n_src, T, d]
    fp32 slabs."""
    if dx.dim() != 2:
        raise ValueError("dx must be a [T, d] tensor")
    T, d = dx.shape
    if check:
        dt = _storage(src, "src")
        _rows(src, "src", T, d, dt, n=n_src)
        _rows(dx, "dx", T, d, dt)
        _rows(dsrc, "dsrc", T, d, torch.float32, n=n_src)
        for t, name in ((w, "w"), (key_gain, "key_gain"), (prenorm_gain, "prenorm_gain"), (dw, "dw"),
                        (dkey_gain, "dkey_gain"), (dprenorm_gain, "dprenorm_gain")):
            _fp32(t, name, (d,), optional=name not in ("w", "dw"))
        _workspace(workspace)
        _on_device(src, dx, dsrc, w, key_gain, prenorm_gain, dw, dkey_gain, dprenorm_gain, workspace)
    rc = load().attnres_site_backward_accumulate(
        dtype_code(src.dtype), _ptr(src), n_src, _slab_stride(src, T, d), T, d, _ptr(w), _ptr(key_gain),
        _ptr(prenorm_gain), 1 if prenorm else 0, eps, _ptr(dx), _ptr(dsrc), _slab_stride(dsrc, T, d), _ptr(dw),
        _ptr(dkey_gain), _ptr(dprenorm_gain), _ptr(workspace), _workspace(workspace), _stream(stream))
    _check("attnres_site_backward_accumulate", rc)


def attnres_phase2_backward_workspace_bytes(T: int, d: int) -> int:
    return int(load().attnres_phase2_backward_workspace_bytes(T, d))


def attnres_phase2_backward(p1_out: torch.Tensor, p1_lse: Optional[torch.Tensor], partial_in: Optional[torch.Tensor],
                            sublayer_prev: Optional[torch.Tensor], w: torch.Tensor, key_gain: Optional[torch.Tensor],
                            prenorm_gain: Optional[torch.Tensor], eps: float, dx: torch.Tensor,
                            dpartial: Optional[torch.Tensor], g_out: torch.Tensor, c_out: torch.Tensor,
                            gp_out: torch.Tensor, dw: Optional[torch.Tensor], dkey_gain: Optional[torch.Tensor],
                            dprenorm_gain: Optional[torch.Tensor], workspace: torch.Tensor, prenorm: bool = True,
                            sublayer_prev2: Optional[torch.Tensor] = None, stream=None, check: bool = True) -> None:
    """One site's phase-2 backward: p1_out, dx, g_out: [T, d]; p1_lse, c_out
    (1 - beta), gp_out (G.p): [T]; the partial source as for
    attnres_phase2_merge; dpartial:
    [T, d] fp32, added to in place; dw, dkey_gain, dprenorm_gain: [d] fp32,
    added to."""
    if p1_out.dim() != 2:
        raise ValueError("p1_out must be a [T, d] tensor")
    T, d = p1_out.shape
    if check:
        dt = _storage(p1_out, "p1_out")
        _rows(p1_out, "p1_out", T, d, dt)
        _fp32(p1_lse, "p1_lse", (T,))
        _partial(partial_in, "partial_in", T, d, dt)
        _rows(sublayer_prev, "sublayer_prev", T, d, dt, optional=True)
        _rows(sublayer_prev2, "sublayer_prev2", T, d, dt, optional=True)
        _rows(dx, "dx", T, d, dt)
        _rows(dpartial, "dpartial", T, d, torch.float32, optional=True)
        _rows(g_out, "g_out", T, d, dt)
        _fp32(c_out, "c_out", (T,), optional=False)
        _fp32(gp_out, "gp_out", (T,), optional=False)
        for t, name in ((w, "w"), (key_gain, "key_gain"), (prenorm_gain, "prenorm_gain"), (dw, "dw"),
                        (dkey_gain, "dkey_gain"), (dprenorm_gain, "dprenorm_gain")):
            _fp32(t, name, (d,), optional=name != "w")
        _workspace(workspace)
        _on_device(p1_out, p1_lse, partial_in, sublayer_prev, sublayer_prev2, dx, dpartial, g_out, c_out, gp_out, w,
                   key_gain, prenorm_gain, dw, dkey_gain, dprenorm_gain, workspace)
    rc = load().attnres_phase2_backward(dtype_code(p1_out.dtype), T, d, _ptr(p1_out), _ptr(p1_lse),
                                        _fmt(partial_in), _ptr(partial_in), _ptr(sublayer_prev2),
                                        _ptr(sublayer_prev), _ptr(w), _ptr(key_gain), _ptr(prenorm_gain),
                                        1 if prenorm else 0, eps, _ptr(dx), _ptr(dpartial), _ptr(g_out),
                                        _ptr(c_out), _ptr(gp_out), _ptr(dw), _ptr(dkey_gain), _ptr(dprenorm_gain),
                                        _ptr(workspace), _workspace(workspace), _stream(stream))
    _check("attnres_phase2_backward", rc)


def attnres_phase1_backward_workspace_bytes(T: int, d: int, n_src: int, S: int) -> int:
    return int(load().attnres_phase1_backward_workspace_bytes(T, d, n_src, S))


def attnres_phase1_backward(src: torch.Tensor, n_src: int, w: torch.Tensor, key_gain: Optional[torch.Tensor],
                            eps: float, g_in: torch.Tensor, c_in: Optional[torch.Tensor],
                            gp_in: Optional[torch.Tensor], dsrc: torch.Tensor, dw: torch.Tensor,
                            dkey_gain: Optional[torch.Tensor], workspace: torch.Tensor, accumulate: bool = False,
                            stream=None, check: bool = True) -> None:
    """The block sources' part of S sites: src: [>=n_src, T, d]; w, key_gain,
    dw, dkey_gain: [S, d] fp32; g_in: [S, T, d]; c_in, gp_in: [S, T] or None;
    dsrc: [>=n_src, T, d] fp32, written or (accumulate) added to."""
    if w.dim() != 2:
        raise ValueError("w must be an [S, d] fp32 tensor")
    S, d = w.shape
    T = g_in.shape[-2]
    if check:
        dt = _storage(src, "src")
        _rows(src, "src", T, d, dt, n=n_src)
        # G of the sources' dtype, or bf16 G with fp32 sources
        gdt = torch.bfloat16 if (dt == torch.float32 and g_in.dtype == torch.bfloat16) else dt
        _rows(g_in, "g_in", T, d, gdt, n=S)
        _rows(dsrc, "dsrc", T, d, torch.float32, n=n_src)
        for t, name in ((w, "w"), (key_gain, "key_gain"), (dw, "dw"), (dkey_gain, "dkey_gain")):
            _fp32(t, name, (S, d), optional=name not in ("w", "dw"))
        _fp32(c_in, "c_in", (S, T))
        _fp32(gp_in, "gp_in", (S, T))
        _workspace(workspace)
        _on_device(src, w, key_gain, g_in, c_in, gp_in, dsrc, dw, dkey_gain, workspace)
    rc = load().attnres_phase1_backward(dtype_code(g_in.dtype), dtype_code(src.dtype), _ptr(src), n_src,
                                        _slab_stride(src, T, d), T, d,
                                        _ptr(w), _ptr(key_gain), S, eps, _ptr(g_in), _slab_stride(g_in, T, d),
                                        _ptr(c_in), _ptr(gp_in), _ptr(dsrc), _slab_stride(dsrc, T, d),
                                        1 if accumulate else 0, _ptr(dw), _ptr(dkey_gain), _ptr(workspace),
                                        _workspace(workspace), _stream(stream))
    _check("attnres_phase1_backward", rc)


def attnres_block_accumulate(partial_in: Optional[torch.Tensor], v: torch.Tensor, out: torch.Tensor,
                             stream=None, v2: Optional[torch.Tensor] = None, check: bool = True) -> None:
    """out = (partial_in or 0) + (v2 or 0) + v; all [T, d] (partial_in may be
    a P24 buffer; out may be fp32 for bf16 rows: the exact sum)."""
    if v.dim() != 2:
        raise ValueError("v must be a [T, d] tensor")
    T, d = v.shape
    if check:
        dt = _storage(v, "v")
        _rows(v, "v", T, d, dt)
        _rows(v2, "v2", T, d, dt, optional=True)
        _rows(out, "out", T, d, torch.float32 if (out is not None and out.dtype == torch.float32) else dt)
        _partial(partial_in, "partial_in", T, d, dt)
        _on_device(partial_in, v2, v, out)
    rc = load().attnres_block_accumulate(dtype_code(v.dtype), T, d, _fmt(partial_in), _ptr(partial_in), _ptr(v2),
                                         _ptr(v), _ptr(out), dtype_code(out.dtype), _stream(stream))
    _check("attnres_block_accumulate", rc)


def attnres_stream_probe(n_read: int, n_write: int, src: Optional[torch.Tensor], dst: torch.Tensor,
                         stream_bytes: int, workgroups_per_cu: int = 2, unroll: int = 2, nontemporal: bool = True,
                         stream=None) -> None:
    """Streaming-bandwidth probe: read ``n_read`` streams of ``stream_bytes``
    each from the start of ``src`` and write ``n_write`` streams to ``dst``
    (which needs at least 16 bytes when nothing is written), with the given
    launch shape and access policy."""
    need_r, need_w = n_read * stream_bytes, max(n_write * stream_bytes, 16)
    if n_read and (src is None or src.numel() * src.element_size() < need_r or not src.is_contiguous()):
        raise ValueError("src must be a contiguous tensor of at least %d bytes" % need_r)
    if dst.numel() * dst.element_size() < need_w or not dst.is_contiguous():
        raise ValueError("dst must be a contiguous tensor of at least %d bytes" % need_w)
    _on_device(src, dst)
    rc = load().attnres_stream_probe(n_read, n_write, _ptr(src), _ptr(dst), stream_bytes, workgroups_per_cu, unroll,
                                     1 if nontemporal else 0, _stream(stream))
    _check("attnres_stream_probe", rc)
