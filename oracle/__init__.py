"""fp64 CPU oracle for the Block / Full AttnRes depth aggregation.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
benchmark's CPU-baseline leg.  The product path (the HIP library and its
binding) never imports it.  The arithmetic lives in ``attnres_oracle.c``; this
module builds it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attnres_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at a deliberately broken copy of the oracle to
# check that the pins catch the planted mistake.
_LIB_OVERRIDE = os.environ.get("ATTNRES_ORACLE_LIB")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP over tokens, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not _LIB_OVERRIDE and not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        D = ctypes.c_double
        lib.oracle_rms.restype = D
        lib.oracle_rms.argtypes = [I, P, D]
        lib.oracle_rmsnorm.argtypes = [I, P, P, D, P]
        lib.oracle_depth_softmax.argtypes = [I, I, P, P, P, D, P, P, P, P, P]
        lib.oracle_partition_stats.argtypes = [I, I, P, P, P, D, P, P, P]
        lib.oracle_merge_two.argtypes = [I, D, D, P, D, D, P, P]
        lib.oracle_block_forward.argtypes = [I, I, I, P, I, P, P, P, P, P, P, D, ctypes.c_int,
                                             P, P, P, P, P, P, P, P]
        lib.oracle_full_forward.argtypes = [I, I, I, P, P, P, P, P, D, ctypes.c_int, P, P, P, P]
        lib.oracle_site_backward.argtypes = [I, I, P, P, P, P, ctypes.c_int, D, P, P, P, P, P]
        lib.oracle_site_backward_tokens.argtypes = [I, I, I, P, P, P, P, ctypes.c_int, D, P, P, P, P, P]
        lib.oracle_block_backward.argtypes = [I, I, I, P, I, P, P, P, P, P, P, D, ctypes.c_int,
                                              P, P, P, P, P, P, P]
        lib.oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _f32(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: widen exactly on the host
        a = a.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def threads() -> int:
    return int(_load().oracle_threads())


def rms(x, eps: float) -> float:
    x = _f64(x)
    return float(_load().oracle_rms(x.shape[-1], _p(x), eps))


def rmsnorm(x, gain=None, eps: float = 0.0) -> np.ndarray:
    x = _f64(x)
    y = np.empty_like(x)
    g = None if gain is None else _f64(gain)
    rc = _load().oracle_rmsnorm(x.shape[-1], _p(x), _p(g), eps, _p(y))
    assert rc == 0
    return y


def _ptr_array(rows: Sequence[np.ndarray]):
    arr = (ctypes.c_void_p * len(rows))(*[r.ctypes.data for r in rows])
    return arr


def depth_softmax(sources, w, g=None, eps: float = 1e-6):
    """One site for one token: returns dict(z, alpha, h, m, lse)."""
    rows = [_f64(s) for s in sources]
    n, d = len(rows), rows[0].shape[0]
    w = _f64(w)
    g = None if g is None else _f64(g)
    z = np.empty(n)
    a = np.empty(n)
    h = np.empty(d)
    m = ctypes.c_double()
    lse = ctypes.c_double()
    ptrs = _ptr_array(rows)
    rc = _load().oracle_depth_softmax(n, d, ctypes.cast(ptrs, ctypes.c_void_p), _p(w), _p(g), eps,
                                      _p(z), _p(a), _p(h), ctypes.byref(m), ctypes.byref(lse))
    assert rc == 0
    return {"z": z, "alpha": a, "h": h, "m": m.value, "lse": lse.value}


def partition_stats(sources, w, g=None, eps: float = 1e-6):
    rows = [_f64(s) for s in sources]
    n, d = len(rows), rows[0].shape[0]
    w = _f64(w)
    g = None if g is None else _f64(g)
    o = np.empty(d)
    m = ctypes.c_double()
    ell = ctypes.c_double()
    ptrs = _ptr_array(rows)
    rc = _load().oracle_partition_stats(n, d, ctypes.cast(ptrs, ctypes.c_void_p), _p(w), _p(g), eps,
                                        ctypes.byref(m), ctypes.byref(ell), _p(o))
    assert rc == 0
    return m.value, ell.value, o


def merge_two(mA, lA, oA, mB, lB, oB) -> np.ndarray:
    oA, oB = _f64(oA), _f64(oB)
    h = np.empty_like(oA)
    rc = _load().oracle_merge_two(oA.shape[0], mA, lA, _p(oA), mB, lB, _p(oB), _p(h))
    assert rc == 0
    return h


def block_forward(emb, v, w, g, gamma, blocks: Sequence[int], eps: float, given=None,
                  final_site: bool = True, want=("x", "h", "o1", "m1", "lse1", "lse", "hfinal", "reps")):
    """Block AttnRes forward for every token row of ``emb``.

    emb [n_tok, d]; v [L, n_tok, d]; w, g [L+1, d]; gamma [L, d];
    given [n_given, n_tok, d] or None.  Returns a dict of fp64 arrays."""
    emb = _f32(emb)
    n_tok, d = emb.shape
    L = int(sum(blocks))
    v = _f32(v) if L > 0 else None
    w = _f32(w)
    g = _f32(g)
    gamma = _f32(gamma)
    given = _f32(given)
    n_given = 0 if given is None else given.shape[0]
    nb = len(blocks)
    bl = np.ascontiguousarray(np.asarray(blocks, dtype=np.int64))
    out = {}

    def alloc(name, shape):
        if name in want:
            out[name] = np.empty(shape, dtype=np.float64)
            return out[name]
        return None

    x = alloc("x", (L, n_tok, d))
    h = alloc("h", (L, n_tok, d))
    o1 = alloc("o1", (L, n_tok, d))
    m1 = alloc("m1", (L, n_tok))
    lse1 = alloc("lse1", (L, n_tok))
    lse = alloc("lse", (L, n_tok))
    hf = alloc("hfinal", (n_tok, d)) if final_site else None
    reps = alloc("reps", (1 + n_given + nb, n_tok, d))
    rc = _load().oracle_block_forward(n_tok, d, nb, _p(bl), n_given, _p(emb), _p(given), _p(v),
                                      _p(w), _p(g), _p(gamma), eps, 1 if final_site else 0,
                                      _p(x), _p(h), _p(o1), _p(m1), _p(lse1), _p(lse), _p(hf), _p(reps))
    if rc != 0:
        raise RuntimeError("oracle_block_forward failed: %d" % rc)
    return out


def full_forward(emb, v, w, g, gamma, eps: float, final_site: bool = True,
                 want=("x", "h", "lse", "hfinal")):
    """Full AttnRes forward (every sublayer output its own source)."""
    emb = _f32(emb)
    n_tok, d = emb.shape
    v = _f32(v)
    L = v.shape[0]
    w, g, gamma = _f32(w), _f32(g), _f32(gamma)
    out = {}
    for name, shape in (("x", (L, n_tok, d)), ("h", (L, n_tok, d)), ("lse", (L, n_tok))):
        if name in want:
            out[name] = np.empty(shape, dtype=np.float64)
    if final_site and "hfinal" in want:
        out["hfinal"] = np.empty((n_tok, d), dtype=np.float64)
    rc = _load().oracle_full_forward(n_tok, d, L, _p(emb), _p(v), _p(w), _p(g), _p(gamma), eps,
                                     1 if final_site else 0, _p(out.get("x")), _p(out.get("h")),
                                     _p(out.get("lse")), _p(out.get("hfinal")))
    if rc != 0:
        raise RuntimeError("oracle_full_forward failed: %d" % rc)
    return out


def site_backward(src, w, g, gamma, eps: float, dx, prenorm: bool = True):
    """Backward of one aggregation site over tokens ("Attention Residuals
    阅读补充", gradients along the tangent; "Attention Residuals" notes,
    section 7, logit gradient).  src [n, T, d], dx [T, d], w/g/gamma [d]
    (g, gamma may be None: ones).  Returns dict(du [n, T, d], dw, dg, dgamma
    [d]) in fp64; dw, dg, dgamma are sums over the tokens."""
    s = _f32(src)
    n, T, d = s.shape
    dxa = _f32(dx)
    du = np.empty((n, T, d))
    dw = np.empty(d)
    dg = np.empty(d)
    dgm = np.empty(d)
    rc = _load().oracle_site_backward_tokens(T, n, d, _p(s), _p(_f32(w)), _p(_f32(g)), _p(_f32(gamma)),
                                             1 if prenorm else 0, eps, _p(dxa), _p(du), _p(dw), _p(dg),
                                             _p(dgm) if prenorm else None)
    assert rc == 0, rc
    return {"du": du, "dw": dw, "dg": dg, "dgamma": dgm if prenorm else None}


def block_backward(emb, v, w, g, gamma, blocks: Sequence[int], eps: float, dx, dhf=None, given=None,
                   final_site: bool = True):
    """Backward of block_forward with the sublayer outputs as inputs, for the
    loss sum_l dx_l . x_l + dhf . hfinal over the token rows of ``emb``
    (block sums exact).

    dx [L, n_tok, d]; dhf [n_tok, d] or None.  Returns fp64 arrays dv [L,
    n_tok, d], demb [n_tok, d], dgiven [n_given, n_tok, d], dw, dg [L+1, d]
    and dgamma [L, d] (parameter gradients summed over the tokens)."""
    emb = _f32(emb)
    n_tok, d = emb.shape
    L = int(sum(blocks))
    v = _f32(v) if L > 0 else None
    dx = _f32(dx) if L > 0 else None
    w, g, gamma = _f32(w), _f32(g), _f32(gamma)
    given = _f32(given)
    dhf = _f32(dhf)
    n_given = 0 if given is None else given.shape[0]
    bl = np.ascontiguousarray(np.asarray(blocks, dtype=np.int64))
    dv = np.empty((L, n_tok, d))
    dreps = np.empty((1 + n_given, n_tok, d))
    dw = np.empty((L + 1, d))
    dg = np.empty((L + 1, d))
    dgamma = np.empty((max(L, 1), d))
    rc = _load().oracle_block_backward(n_tok, d, len(blocks), _p(bl), n_given, _p(emb), _p(given), _p(v), _p(w),
                                       _p(g), _p(gamma), eps, 1 if final_site else 0,
                                       _p(dx), _p(dhf), _p(dv),
                                       _p(dreps), _p(dw), _p(dg), _p(dgamma))
    if rc != 0:
        raise RuntimeError("oracle_block_backward failed: %d" % rc)
    return {"dv": dv, "demb": dreps[0], "dgiven": dreps[1:], "dw": dw, "dg": dg, "dgamma": dgamma[:L]}
