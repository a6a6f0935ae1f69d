"""Parity harness: run a workload through the HIP path, capture sampled rows at
every aggregation site, and compare them with the fp64 oracle.

Metric (per output row): max_k |gpu_k - ref_k| / max_k |ref_k|.  Bars: 2e-2
for bf16 storage, 1e-5 for fp32 storage.  Statistics (lse) are compared as
|gpu - ref| / max(1, |ref|) against the same bar.
"""
from __future__ import annotations

import time
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle
import synth
from transformer_depth_wise_amd import BlockAttnRes, FullAttnRes

TOL = {"f32": 1e-5, "bf16": 2e-2}


def row_rel_err(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row max-abs-rel error over the last axis."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(gpu - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return num / np.maximum(den, 1e-300)


def stat_err(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(gpu - ref) / np.maximum(1.0, np.abs(ref))


def _host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Capture:
    """Collect sampled rows of every site's outputs on the device."""

    def __init__(self, idx: torch.Tensor):
        self.idx = idx
        self.rows: Dict[str, List[torch.Tensor]] = {}
        self.where: Dict[str, List[int]] = {}

    def __call__(self, site, **tensors):
        for k, t in tensors.items():
            if t is None:
                continue
            self.rows.setdefault(k, []).append(t.index_select(0, self.idx).clone())
            self.where.setdefault(k, []).append(site)

    def stacked(self, k) -> np.ndarray:
        return _host(torch.stack(self.rows[k]))

    def sites(self, k) -> List[int]:
        """The sites at which ``k`` was captured, in capture order."""
        return self.where[k]


def block_inputs(w: synth.Workload, device, t0: int = 0, t1: Optional[int] = None):
    t1 = w.T if t1 is None else t1
    scales = synth.sublayer_scales(w)
    emb = synth.embedding(w, t0, t1, device)
    given = [synth.given_block(w, n + 1, t0, t1, device) for n in range(w.n_given)]
    v = [synth.sublayer_output(w, l + 1, t0, t1, device, scales) for l in range(w.L)]
    return emb, given, v


def run_block_parity(w: synth.Workload, samples: Optional[Sequence[int]] = None, device="cuda",
                     keep_h: bool = True, x_ring: int = 4, partial: Optional[str] = None,
                     fuse_first: bool = True, training: bool = False) -> Dict[str, float]:
    """Block AttnRes on the GPU vs the oracle on sampled tokens.  Returns the
    worst error per output kind (already asserted against the bar).  With
    ``training`` the forward that keeps its activations runs (fp32 block
    representations for bf16 rows)."""
    dev = torch.device(device)
    emb, given, v = block_inputs(w, dev)
    prm = synth.params(w, dev)
    st = BlockAttnRes(w.T, w.d, w.block_sizes, w.torch_dtype, n_given=w.n_given, eps=w.eps, device=dev,
                      keep_h=keep_h, x_ring=x_ring, final_site=w.final_site, partial=partial,
                      fuse_first=fuse_first, training=training)
    st.reps[0].copy_(emb)
    for n, b in enumerate(given):
        st.reps[1 + n].copy_(b)
    samples = list(range(w.T)) if samples is None else list(samples)
    idx = torch.tensor(samples, dtype=torch.long, device=dev)
    cap = Capture(idx)
    st.forward(prm, lambda l, x: v[l], hook=cap)
    torch.cuda.synchronize()

    # oracle on the sampled tokens, from the very values the GPU saw
    o = oracle.block_forward(
        emb.index_select(0, idx), torch.stack([t.index_select(0, idx) for t in v]), prm["w"], prm["g"],
        prm["gamma"], w.block_sizes, w.eps,
        given=torch.stack([t.index_select(0, idx) for t in given]) if given else None,
        final_site=w.final_site)
    tol = TOL[w.dtype]
    worst = {}
    worst["x"] = float(row_rel_err(cap.stacked("x"), o["x"]).max())
    if keep_h:
        worst["h"] = float(row_rel_err(cap.stacked("h"), o["h"]).max())
    # (with the first sublayer fused into phase 1 and no h kept, o_0 of a
    # block with several sources is never stored)
    worst["o1"] = float(row_rel_err(cap.stacked("o1"), o["o1"][cap.sites("o1")]).max())
    worst["lse1"] = float(stat_err(cap.stacked("lse1"), o["lse1"]).max())
    worst["m1"] = float(stat_err(cap.stacked("m1"), o["m1"]).max())
    reps_gpu = _host(st.reps.index_select(1, idx))
    worst["reps"] = float(row_rel_err(reps_gpu, o["reps"]).max())
    if w.final_site:
        worst["hfinal"] = float(row_rel_err(_host(st.h_final.index_select(0, idx)), o["hfinal"]).max())
    for k, e in worst.items():
        assert e <= tol, "%s: %s max-abs-rel %.3e exceeds %.1e" % (w.name, k, e, tol)
    return worst


def run_full_parity(w: synth.Workload, samples: Optional[Sequence[int]] = None, device="cuda",
                    group: Optional[int] = None):
    """Full AttnRes on the GPU (one-shot sites, or the grouped two-phase
    schedule with ``group`` sublayers per group) vs the oracle's one-shot
    definition on sampled tokens."""
    dev = torch.device(device)
    scales = synth.sublayer_scales(w)
    prm = synth.params(w, dev)
    st = FullAttnRes(w.T, w.d, w.L, w.torch_dtype, eps=w.eps, device=dev, keep_h=True, final_site=w.final_site,
                     group=group)
    st.hist[0].copy_(synth.embedding(w, 0, w.T, dev))
    for l in range(w.L):
        st.hist[l + 1].copy_(synth.sublayer_output(w, l + 1, 0, w.T, dev, scales))
    samples = list(range(w.T)) if samples is None else list(samples)
    idx = torch.tensor(samples, dtype=torch.long, device=dev)
    cap = Capture(idx)
    st.forward(prm, lambda l, x: None, hook=cap)
    torch.cuda.synchronize()
    hist = st.hist.index_select(1, idx)
    o = oracle.full_forward(hist[0], hist[1:], prm["w"], prm["g"], prm["gamma"], w.eps, final_site=w.final_site)
    tol = TOL[w.dtype]
    worst = {
        "x": float(row_rel_err(cap.stacked("x"), o["x"]).max()),
        "h": float(row_rel_err(cap.stacked("h"), o["h"]).max()),
    }
    if group is None:  # the grouped merge returns no per-site statistics
        worst["lse"] = float(stat_err(cap.stacked("lse"), o["lse"]).max())
    if w.final_site:
        worst["hfinal"] = float(row_rel_err(_host(st.h_final.index_select(0, idx)), o["hfinal"]).max())
    for k, e in worst.items():
        assert e <= tol, "%s: %s max-abs-rel %.3e exceeds %.1e" % (w.name, k, e, tol)
    return worst


def run_block_backward_parity(w: synth.Workload, samples: Optional[Sequence[int]] = None, device="cuda",
                              params_too: bool = True, dx_from_outputs: bool = False,
                              tol: Optional[float] = None) -> Dict[str, float]:
    """Block AttnRes training forward + backward on the GPU vs the oracle's
    backward on sampled tokens: dL/dv_l of every site, dL/db_0 and the given
    block sums; with ``params_too`` (all tokens sampled) also dw, dg, dgamma.
    Upstream gradients dx_l, dh_final are seeded N(0,1) rows (or, with
    ``dx_from_outputs``, the sublayer outputs themselves, to save memory).

    The reference is the oracle's backward of the plain definition (block
    sums exact).  The training forward keeps the block representations in
    fp32 for that reason; dL/dh_final enters in h_final's dtype (fp32 there,
    the same values as the bf16 rows drawn here)."""
    dev = torch.device(device)
    emb, given, v = block_inputs(w, dev)
    prm = synth.params(w, dev)
    st = BlockAttnRes(w.T, w.d, w.block_sizes, w.torch_dtype, n_given=w.n_given, eps=w.eps, device=dev,
                      final_site=w.final_site, training=True)
    st.reps[0].copy_(emb)
    for n, b in enumerate(given):
        st.reps[1 + n].copy_(b)
    st.forward(prm, lambda l, x: v[l])
    gen = torch.Generator(device=dev).manual_seed(7000 + w.T + w.d)
    if dx_from_outputs:
        dx = [v[(l + 1) % w.L] for l in range(w.L)]
        dhf = v[0]
    else:
        dx = [torch.randn((w.T, w.d), generator=gen, device=dev).to(w.torch_dtype) for _ in range(w.L)]
        dhf = torch.randn((w.T, w.d), generator=gen, device=dev).to(w.torch_dtype)
    samples = list(range(w.T)) if samples is None else list(samples)
    idx = torch.tensor(samples, dtype=torch.long, device=dev)
    dv_rows = [None] * w.L

    def dx_for(l, dv):
        dv_rows[l] = dv.index_select(0, idx).clone()
        return dx[l]

    out = st.backward(prm, dx_for, dh_final=dhf.to(st.h_final.dtype) if w.final_site else None)
    torch.cuda.synchronize()
    sel = lambda t: t.index_select(0, idx)  # noqa: E731
    args = (sel(emb), torch.stack([sel(t) for t in v]), prm["w"], prm["g"], prm["gamma"], w.block_sizes, w.eps,
            torch.stack([sel(t) for t in dx]), sel(dhf) if w.final_site else None)
    kw = dict(given=torch.stack([sel(t) for t in given]) if given else None, final_site=w.final_site)
    exact = oracle.block_backward(*args, **kw)
    gpu = {"dv": _host(torch.stack(dv_rows)), "demb": _host(sel(out["demb"]))}
    if w.n_given:
        gpu["dgiven"] = _host(out["dgiven"].index_select(1, idx))
    if params_too:
        assert len(samples) == w.T, "parameter gradients are sums over every token"
        for k in ("dw", "dg", "dgamma"):
            gpu[k] = _host(out[k])
    bar = TOL[w.dtype] if tol is None else tol
    worst = {}
    for k, x in gpu.items():
        e = float(row_rel_err(x, exact[k]).max())
        worst[k] = e
        assert e <= bar, "%s: %s max-abs-rel %.3e exceeds %.1e" % (w.name, k, e, bar)
    return worst
