"""Drivers of the Block / Full AttnRes depth aggregation on one GPU.

The schedule follows the two-phase inference of "Attention Residuals" (notes,
section 10) for every block of sublayers:

    phase 1   attnres_phase1_first_prenorm  sources b_0..b_{n-1}, all S queries
              of the block; the first sublayer's PreNorm output x comes out
              of this pass (that sublayer has no partial-sum source)
    phase 2   attnres_phase2_merge  x (S - 1), sequentially; sublayer j's output
              is produced between two calls (here by a synthetic sublayer)
    block end attnres_block_accumulate  b_n = partial + v_S
    final     attnres_full        b_0..b_N with the final query (no PreNorm)

Buffers live in HBM for the whole pass: the block representations
``reps [1 + n_given + N, T, d]`` (slot 0 is the embedding b_0), the phase-1
outputs ``o1 [S_max, T, d]`` with their ``lse/m [S_max, T]`` (fp32) and the
phase-1 workspace (packed queries and softmax weights), the running
intra-block partial sum ``partial``, and a small ring of PreNorm outputs
``x``.  The partial sum is never stored in bf16: a bf16 running sum over a
24-sublayer block drifts by several percent of the row maximum.  For bf16
rows it is kept in the 16-bit fixed-point format with one power-of-two
exponent per row (Q16: 2 bytes per element, every element to within 2^-15 of
its row's largest magnitude; the 24-bit split format P24 remains selectable),
and in fp32 for fp32 rows; block sums are rounded to the storage dtype once,
when they are complete.  The partial is stored only at the even
positions j = 2, 4, ... of a block: sublayer j + 1 reads it with v_j and
writes nothing, sublayer j + 2 reads it with v_j and v_{j+1} and stores the
next one, so the two latest sublayer outputs must stay valid.

``plan()`` lists every launch of a pass with its algorithmic bytes (each row
the method must read or write, counted once).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional, Sequence

import torch

from . import _lib
from ._lib import (attnres_block_accumulate, attnres_full, attnres_phase1, attnres_phase1_backward,
                   attnres_site_backward_accumulate,
                   attnres_phase1_accumulate, attnres_phase1_first_prenorm, attnres_phase2_backward,
                   attnres_phase2_merge,
                   attnres_phase2_merge_multi)

SiteHook = Callable[..., None]
Sublayer = Callable[[int, torch.Tensor], torch.Tensor]


@dataclasses.dataclass
class Launch:
    kind: str       # "phase1", "phase2", "accumulate", "final", "full", "*_backward"
    bytes: int      # algorithmic bytes moved by this launch


def _esize(dt: torch.dtype) -> int:
    return 4 if dt == torch.float32 else 2


def _check_params(params: Dict[str, torch.Tensor], d: int, sites: int, norms: int, device: torch.device) -> None:
    """Checked once per pass, so that the per-launch calls can skip the
    binding's own checks: w, g fp32 [>= sites, d]; gamma fp32 [>= norms, d];
    contiguous; on the pass's device, which must be the current one."""
    for name, rows, required in (("w", sites, True), ("g", sites, False), ("gamma", norms, False)):
        t = params.get(name)
        if t is None:
            if required:
                raise ValueError("params['%s'] is required" % name)
            continue
        if (t.dtype != torch.float32 or t.dim() != 2 or t.shape[0] < rows or t.shape[1] != d or
                not t.is_contiguous()):
            raise ValueError("params['%s'] must be a contiguous fp32 [>= %d, %d] tensor, got %s %s"
                             % (name, rows, d, t.dtype, tuple(t.shape)))
        _lib._on_device(t)
    if device.index is not None and torch.cuda.current_device() != device.index:
        raise ValueError("the pass's buffers live on %s, but the current device is cuda:%d"
                         % (device, torch.cuda.current_device()))


def _checked_rows(t: torch.Tensor, name: str, T: int, d: int, dtype: torch.dtype) -> torch.Tensor:
    """A caller-supplied [T, d] row set (a sublayer's output or gradient)."""
    _lib._rows(t, name, T, d, dtype)
    _lib._on_device(t)
    return t


class BlockAttnRes:
    """Block AttnRes forward over T tokens of width d on the current GPU.

    ``block_sizes``: sublayers per block computed in this pass.
    ``n_given``: completed block sums supplied as inputs (a decode-shaped step
    starts at block n_given + 1).  ``x_ring``: number of PreNorm output
    buffers cycled through (a real model consumes x_l immediately).
    ``fuse_first``: the first sublayer of a block takes its PreNorm output
    from the phase-1 pass (False: a separate phase-2 launch computes it).
    ``training``: keep what ``backward`` needs -- every site's phase-1
    output and statistics, and every stored partial sum (each in its own
    buffer instead of in place); the first sublayer is then merged by a
    phase-2 launch so that its phase-1 output is stored too.  With bf16
    rows, training keeps the block representations (``reps``, and
    ``h_final``) in fp32: the notes' section 8 defines b_n as the sum of the
    block's outputs, and the backward differentiates the forward that reads
    those exact sums (phase 1 then reads fp32 sources and writes bf16
    outputs; the embedding and given block sums are copied in exactly).
    ``dh_final`` then comes in fp32 too.
    ``fuse_sum``: a block's sum b_n is formed by the next phase-1 call
    (attnres_phase1_accumulate, which sums inside the scoring pass over long
    token ranges) or by the final site's call, instead of by a block-sum
    launch at the end of the block (False); after the last block without a
    final site, a block-sum launch forms it either way.
    """

    def __init__(self, T: int, d: int, block_sizes: Sequence[int], dtype: torch.dtype, n_given: int = 0,
                 eps: float = 1e-6, device=None, x_ring: int = 4, keep_h: bool = False,
                 final_site: bool = True, partial: Optional[str] = None, fuse_first: bool = True,
                 training: bool = False, fuse_sum: bool = True):
        self.training = bool(training)
        self.fuse_sum = bool(fuse_sum)
        self.fuse_first = bool(fuse_first) and not self.training
        self.T, self.d, self.dtype = int(T), int(d), dtype
        self.block_sizes = [int(s) for s in block_sizes]
        self.n_given, self.eps = int(n_given), float(eps)
        self.L = sum(self.block_sizes)
        self.final_site = final_site
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.device = dev
        n_reps = 1 + self.n_given + len(self.block_sizes)
        if n_reps > _lib.ATTNRES_MAX_SOURCES:
            raise ValueError("too many sources for one aggregation site: %d" % n_reps)
        if any(s > 1 and 1 + self.n_given + b > _lib.ATTNRES_MAX_SOURCES_MULTI
               for b, s in enumerate(self.block_sizes)):
            raise ValueError("phase 1 with S >= 2 supports at most %d completed sources"
                             % _lib.ATTNRES_MAX_SOURCES_MULTI)
        if self.training:
            # the phase-1 backward of a block takes every site of the block at
            # once (at most 32) and, with the sites' partial-source terms, at
            # most ATTNRES_MAX_SOURCES_MULTI block sources, also for one-sublayer
            # blocks (whose forward could take more)
            for b, S in enumerate(self.block_sizes):
                if S > 32:
                    raise ValueError("the backward supports at most 32 sublayers per block, got %d" % S)
                if 1 + self.n_given + b > _lib.ATTNRES_MAX_SOURCES_MULTI:
                    raise ValueError("the backward of block %d would read %d completed sources (at most %d)"
                                     % (b, 1 + self.n_given + b, _lib.ATTNRES_MAX_SOURCES_MULTI))
        smax = max(self.block_sizes) if self.block_sizes else 1
        # the block representations' storage: fp32 in a bf16 training pass
        self.rep_dtype = torch.float32 if self.training else dtype
        self.reps = torch.empty((n_reps, T, d), dtype=self.rep_dtype, device=dev)
        self.device = dev = self.reps.device  # with its index
        self.o1 = torch.empty((smax, T, d), dtype=dtype, device=dev)
        self.m1 = torch.empty((smax, T), dtype=torch.float32, device=dev)
        self.lse1 = torch.empty((smax, T), dtype=torch.float32, device=dev)
        # the largest phase-1 workspace over the blocks (a one-query phase 1
        # without the first sublayer's PreNorm and with sources of the output
        # type, and the final site, need none)
        ws = 0
        for b, S in enumerate(self.block_sizes):
            if T > 0 and (S > 1 or self._fuse(S, 1 + self.n_given + b) or self.rep_dtype != dtype):
                ws = max(ws, _lib.attnres_phase1_workspace_bytes(T, d, 1 + self.n_given + b, S))
        self.workspace = torch.empty((max(ws, 16) // 4,), dtype=torch.float32, device=dev)
        # running partial sum: P24 (24-bit split) for bf16 rows, fp32 for fp32 rows
        self.partial_format = partial or ("q16" if dtype == torch.bfloat16 else "f32")
        if self.partial_format == "q16":
            self.partial = _lib.q16_partial(T, d, dev)
        elif self.partial_format == "p24":
            self.partial = _lib.p24_partial(T, d, dev)
        elif self.partial_format == "f32":
            self.partial = torch.empty((T, d), dtype=torch.float32, device=dev)
        else:
            raise ValueError("partial format must be 'q16', 'p24' or 'f32'")
        if self.training:
            # per block: phase-1 outputs and statistics of every site, and the
            # partial sums stored at positions j = 2, 4, ..., S - 1 (slot j // 2 - 1)
            self.o_blocks = [torch.empty((S, T, d), dtype=dtype, device=dev) for S in self.block_sizes]
            self.lse_blocks = [torch.empty((S, T), dtype=torch.float32, device=dev) for S in self.block_sizes]
            self.p_slots = [[self._new_partial() for _ in range(max(0, (S - 1) // 2))] for S in self.block_sizes]
            self.recipes: List[Optional[tuple]] = [None] * self.L
        self.x = torch.empty((max(1, x_ring), T, d), dtype=dtype, device=dev)
        self.h = torch.empty((T, d), dtype=dtype, device=dev) if keep_h else None
        self.h_final = torch.empty((T, d), dtype=self.rep_dtype, device=dev)
        self.lse_final = torch.empty((T,), dtype=torch.float32, device=dev)

    def _new_partial(self) -> torch.Tensor:
        if self.partial_format == "q16":
            return _lib.q16_partial(self.T, self.d, self.device)
        if self.partial_format == "p24":
            return _lib.p24_partial(self.T, self.d, self.device)
        return torch.empty((self.T, self.d), dtype=torch.float32, device=self.device)

    # ------------------------------------------------------------------ bytes
    def buffer_bytes(self) -> Dict[str, int]:
        """Device memory held by this pass's buffers (the AttnRes working set)."""
        out = {"block_reps": self.reps.numel() * self.reps.element_size(),
               "phase1_out": self.o1.numel() * self.o1.element_size(),
               "phase1_stats": 2 * self.m1.numel() * 4,
               "phase1_workspace": self.workspace.numel() * 4,
               "partial_sum": self.partial.numel() * self.partial.element_size(),
               "prenorm_out": self.x.numel() * self.x.element_size(),
               "final": self.h_final.numel() * self.h_final.element_size() + self.lse_final.numel() * 4}
        if self.h is not None:
            out["h"] = self.h.numel() * self.h.element_size()
        out["total"] = sum(out.values())
        return out

    def _fuse(self, S: int, n_done: int) -> bool:
        """Whether the block's first sublayer takes its PreNorm output from the
        phase-1 pass (that pass reads at most ATTNRES_MAX_SOURCES_MULTI
        sources; a one-query block with more merges its first site in phase 2)."""
        return self.fuse_first and (S > 1 or n_done <= _lib.ATTNRES_MAX_SOURCES_MULTI)

    def _partial_bytes(self) -> int:
        """Bytes of one stored partial sum (Q16: values and row exponents)."""
        es = {"q16": 2, "p24": 3, "f32": 4}[self.partial_format]
        return self.T * self.d * es + (self.T * 4 if self.partial_format == "q16" else 0)

    def _row(self, dt=None) -> int:
        return self.T * self.d * _esize(self.dtype if dt is None else dt)

    def plan(self) -> List[Launch]:
        """Algorithmic bytes of every launch of one pass, in launch order."""
        r = self._row()
        rr = self._row(self.rep_dtype)  # a block representation (fp32 in a bf16 training pass)
        r32 = self._partial_bytes()
        stat = self.T * 4
        out: List[Launch] = []
        n_done = 1 + self.n_given
        pend = 0  # bytes of the previous block's sum still to be formed (its pieces read, b_n written)
        for S in self.block_sizes:
            fuse = self._fuse(S, n_done)
            if fuse:  # + x of the first sublayer (phase 1 writes it instead of o_0)
                out.append(Launch("phase1", pend + (n_done * rr + S * r + S * 2 * stat if n_done > 1 else
                                                    rr + r + S * 2 * stat)))
            elif n_done == 1 and not self.training:
                # statistics only; phase 2 reads b_0 as its phase-1 output
                out.append(Launch("phase1", pend + rr + S * 2 * stat))
            else:
                out.append(Launch("phase1", pend + n_done * rr + S * (r + 2 * stat)))
            for j in range(S):
                if j == 0 and fuse:
                    continue
                if j == 0:
                    b = 2 * r + stat                  # o; x
                elif j == 1:
                    b = 3 * r + stat                  # o, v0; x
                elif j == 2:
                    b = 4 * r + r32 + stat            # o, v0, v1; p, x
                elif j % 2:
                    b = 3 * r + r32 + stat            # o, p, v; x
                else:
                    b = 4 * r + 2 * r32 + stat        # o, p, v, v; p, x
                out.append(Launch("phase2", b))
            if S == 1:
                acc = r + rr
            elif S == 2:
                acc = 2 * r + rr
            elif S % 2:
                acc = r + r32 + rr           # p (stored at S-1), v; b
            else:
                acc = 2 * r + r32 + rr       # p (stored at S-2), v, v; b
            if self.fuse_sum:
                pend = acc                   # formed by the next phase-1 (or the final site's) call
            else:
                out.append(Launch("accumulate", acc))
            n_done += 1
        if self.final_site:
            out.append(Launch("final", pend + (n_done + 1) * rr + stat))
        elif pend:
            out.append(Launch("accumulate", pend))
        return out

    def plan_survey(self) -> List[Launch]:
        """The same launches priced with the plain row model of the scope
        table (rows only, no statistics; every partial sum one row of the
        storage dtype): phase 1 of a block reads its n sources and writes S
        outputs; the first sublayer's merge reads o and writes x (2 rows; here
        it happens inside phase 1, so it is booked there); the second reads o
        and v_1 and writes x (3); every later one reads o, the partial and the
        previous output and writes the partial and x (5); the block sum reads
        the partial and the last output and writes b_n (3); the final site
        reads the N + 1 representations and writes h_final.  At the 16K
        chunk's layout this is 1146 rows per token, 874 of them in the 178
        merge launches."""
        r = self._row()
        out: List[Launch] = []
        n_done = 1 + self.n_given
        pend = 0  # a block sum formed inside the next call is booked there
        for S in self.block_sizes:
            fuse = self._fuse(S, n_done)
            out.append(Launch("phase1", pend + (n_done + S + (2 if fuse else 0)) * r))
            for j in range(S):
                if j == 0 and fuse:
                    continue
                out.append(Launch("phase2", (2 if j == 0 else 3 if j == 1 else 5) * r))
            if self.fuse_sum:
                pend = 3 * r
            else:
                out.append(Launch("accumulate", 3 * r))
            n_done += 1
        if self.final_site:
            out.append(Launch("final", pend + (n_done + 1) * r))
        elif pend:
            out.append(Launch("accumulate", pend))
        return out

    # ---------------------------------------------------------------- forward
    def forward(self, params: Dict[str, torch.Tensor], sublayer: Sublayer,
                hook: Optional[SiteHook] = None, stream=None,
                instrument: Optional[Callable[[str, bool], None]] = None) -> torch.Tensor:
        """One pass over the whole depth.  ``self.reps[0]`` must hold b_0 and
        ``self.reps[1:1+n_given]`` the supplied block sums.  ``params`` holds
        fp32 ``w``, ``g`` [L+1, d] and ``gamma`` [L, d] (``g``/``gamma`` may be
        None for unit gains).  ``sublayer(l, x_l)`` returns the output v_l of
        sublayer l (0-based), a [T, d] tensor that stays valid for the rest of
        the block (the last two of a block until the next block's phase-1
        call, or the final site's, has been issued: with ``fuse_sum`` that
        call forms the block's sum from them).  ``hook(site, x=, h=, o1=,
        lse1=, m1=)`` is called after each phase-2 launch.
        ``instrument(kind, begin)`` is called just before (begin=True) and
        after (begin=False) every launch."""
        _check_params(params, self.d, self.L + (1 if self.final_site else 0), self.L, self.device)
        w, g, gam = params["w"], params.get("g"), params.get("gamma")
        eps = self.eps
        n_done = 1 + self.n_given
        mark = instrument if instrument is not None else (lambda kind, begin: None)
        l0 = 0
        nx = self.x.shape[0]
        pending = None  # (partial, v_{S-2}, v_{S-1}) of the previous block, its sum not yet formed
        for b, S in enumerate(self.block_sizes):
            # with a single completed source (the embedding) every phase-1
            # output is that source: compute the statistics only and let
            # phase 2 read b_0 itself
            single = n_done == 1
            o1 = self.o_blocks[b] if self.training else self.o1[:S]
            lse1 = self.lse_blocks[b] if self.training else self.lse1[:S]
            slots = self.p_slots[b] if self.training else None
            fuse = self._fuse(S, n_done)
            mark("phase1", True)
            if pending is not None:
                # b_{n_done-1}, the previous block's sum, is formed by this call
                attnres_phase1_accumulate(self.reps, n_done, w[l0:l0 + S], None if g is None else g[l0:l0 + S],
                                          eps, *pending, o1, self.m1[:S], lse1,
                                          prenorm_gain=None if (gam is None or not fuse) else gam[l0],
                                          x_out=self.x[l0 % nx] if fuse else None, h_out=self.h if fuse else None,
                                          workspace=self.workspace, stream=stream, check=False)
                pending = None
            elif fuse:
                attnres_phase1_first_prenorm(self.reps, n_done, w[l0:l0 + S], None if g is None else g[l0:l0 + S],
                                             eps, None if single else self.o1[:S], self.m1[:S], self.lse1[:S],
                                             None if gam is None else gam[l0], self.x[l0 % nx], self.h,
                                             self.workspace, stream=stream, check=False)
            else:
                attnres_phase1(self.reps, n_done, w[l0:l0 + S], None if g is None else g[l0:l0 + S], eps,
                               o1 if (self.training or not single) else None, self.m1[:S], lse1,
                               self.workspace, stream=stream, check=False)
            mark("phase1", False)
            # the two latest outputs of the block stay alive (prev2, prev)
            prev2 = prev = None
            for j in range(S):
                site = l0 + j
                x = self.x[site % nx]
                kg = None if g is None else g[site]
                pg = None if gam is None else gam[site]
                # the partial p_j = v_0 + ... + v_{j-1} is stored at even j >= 2
                # (training: each in its own slot, j // 2 - 1)
                if slots is None:
                    p_prev = p_new = self.partial
                else:
                    p_prev = slots[(j - 1) // 2 - 1] if j >= 3 else None
                    p_new = slots[j // 2 - 1] if j >= 2 and j % 2 == 0 else None
                if j <= 1:
                    pin, v2, pout = None, None, None            # p = v_0 (j = 1) or none
                elif j == 2:
                    pin, v2, pout = None, prev2, p_new          # p = v_0 + v_1, stored
                elif j % 2:
                    pin, v2, pout = p_prev, None, None          # p = p_{j-1} + v_{j-1}
                else:
                    pin, v2, pout = p_prev, prev2, p_new        # p_{j-2} + v_{j-2} + v_{j-1}
                if self.training:
                    self.recipes[site] = (pin, v2, prev)
                o = self.reps[0] if (single and not self.training) else o1[j]
                if j == 0 and fuse:
                    # x (and h = o_0) came out of phase 1; slab 0 of o1 is scratch
                    o = self.reps[0] if single else self.h
                else:
                    mark("phase2", True)
                    attnres_phase2_merge(o, lse1[j], pin, prev, pout, w[site], kg, pg, eps,
                                         self.h, x, stream=stream, sublayer_prev2=v2, check=False)
                    mark("phase2", False)
                if hook is not None:
                    hook(site, x=x, h=self.h, o1=o, lse1=lse1[j], m1=self.m1[j])
                prev2, prev = prev, _checked_rows(sublayer(site, x), "output of sublayer %d" % site, self.T,
                                                  self.d, self.dtype)
            # b_n = ((p or 0) + (v_{S-2} or 0)) + v_{S-1}: the partial stored at
            # S-2 (S even) or S-1 (S odd), none for S <= 2
            p_last = self.partial if slots is None else (slots[-1] if slots else None)
            pending = (None if S <= 2 else p_last, prev2 if S % 2 == 0 else None, prev)
            if not self.fuse_sum or (b == len(self.block_sizes) - 1 and not self.final_site):
                mark("accumulate", True)
                attnres_block_accumulate(pending[0], pending[2], self.reps[n_done], stream=stream, v2=pending[1],
                                         check=False)
                mark("accumulate", False)
                pending = None
            n_done += 1
            l0 += S
        if self.final_site:
            mark("final", True)
            wf, gf = w[self.L:self.L + 1], None if g is None else g[self.L:self.L + 1]
            if pending is not None:
                attnres_phase1_accumulate(self.reps, n_done, wf, gf, eps, *pending, self.h_final.unsqueeze(0), None,
                                          self.lse_final.unsqueeze(0), workspace=self.workspace, stream=stream,
                                          check=False)
            else:
                attnres_phase1(self.reps, n_done, wf, gf, eps, self.h_final.unsqueeze(0), None,
                               self.lse_final.unsqueeze(0), self.workspace, stream=stream, check=False)
            mark("final", False)
        return self.h_final

    def plan_backward(self) -> List[Launch]:
        """Algorithmic bytes of every launch of ``backward``, in launch order
        (rows counted once; gradients of rows are fp32, read and written).
        Phase-2 backward of site j: o, dx and the partial source's terms
        read, G written, and (after the first sublayer) the fp32 running
        gradient read and written.  Phase-1 backward of a block: the n
        sources and S rows of G read once, the n fp32 source gradients read
        and written, plus the per-token coefficients (written and read back).
        The final site: N+1 sources and dL/dh_final read, N+1 fp32 gradients
        written."""
        r = self._row()
        rr = self._row(self.rep_dtype)  # a block representation (fp32 in a bf16 training pass)
        r32 = self.T * self.d * 4
        rp = self._partial_bytes()
        stat = self.T * 4
        out: List[Launch] = []
        n_reps = 1 + self.n_given + len(self.block_sizes)
        if self.final_site:   # the representations and dL/dh_final (h_final's dtype) read
            out.append(Launch("final_backward", (n_reps + 1) * rr + n_reps * r32 + stat))
        n = n_reps - 1
        for S in reversed(self.block_sizes):
            n -= 1
            for j in range(S - 1, -1, -1):
                if j == 0:
                    b = 2 * r + r + 2 * stat                      # o, dx; G
                elif j == 1:
                    b = 3 * r + 2 * r32 + r + 3 * stat            # o, dx, v0; R; G
                elif j == 2:
                    b = 4 * r + 2 * r32 + r + 3 * stat            # o, dx, v0, v1; R; G
                elif j % 2:
                    b = 3 * r + rp + 2 * r32 + r + 3 * stat       # o, dx, p, v; R; G
                else:
                    b = 4 * r + rp + 2 * r32 + r + 3 * stat       # o, dx, p, v, v; R; G
                out.append(Launch("phase2_backward", b))
            nsrc = n + 1
            out.append(Launch("phase1_backward", nsrc * rr + S * r + 2 * nsrc * r32 + 2 * S * stat +
                              2 * self.T * S * nsrc * 4))
        return out

    # --------------------------------------------------------------- backward
    def backward(self, params: Dict[str, torch.Tensor], dx_for: Callable[[int, torch.Tensor], torch.Tensor],
                 dh_final: Optional[torch.Tensor] = None, stream=None,
                 instrument: Optional[Callable[[str, bool], None]] = None) -> Dict[str, torch.Tensor]:
        """Backward of the last ``forward`` (built with ``training=True``),
        sites in reverse order.  ``dx_for(l, dv_l)`` is the sublayer's backward:
        it receives dL/dv_l (fp32 [T, d], valid only during the call) and
        returns dL/dx_l ([T, d], storage dtype).  ``dh_final``: dL/dh_final
        (needed with the final site).  Returns fp32 ``demb`` [T, d],
        ``dgiven`` [n_given, T, d], ``dw``, ``dg`` [L+1, d], ``dgamma`` [L, d]."""
        if not self.training:
            raise RuntimeError("backward needs a forward built with training=True")
        if self.final_site and dh_final is None:
            raise ValueError("dh_final is required with the final aggregation site")
        _check_params(params, self.d, self.L + (1 if self.final_site else 0), self.L, self.device)
        if self.final_site:
            _checked_rows(dh_final, "dh_final", self.T, self.d, self.h_final.dtype)
        w, g, gam = params["w"], params.get("g"), params.get("gamma")
        T, d, eps, dev = self.T, self.d, self.eps, self.device
        mark = instrument if instrument is not None else (lambda kind, begin: None)
        n_reps = self.reps.shape[0]
        smax = max(self.block_sizes) if self.block_sizes else 1
        dw = torch.zeros((self.L + 1, d), dtype=torch.float32, device=dev)
        dg = torch.zeros((self.L + 1, d), dtype=torch.float32, device=dev)
        dgamma = torch.zeros((max(self.L, 1), d), dtype=torch.float32, device=dev)
        G = torch.empty((smax, T, d), dtype=self.dtype, device=dev)
        cg = torch.empty((2, smax, T), dtype=torch.float32, device=dev)  # 1 - beta, G.p
        ws1 = max([_lib.attnres_phase1_backward_workspace_bytes(T, d, n_reps, 1) if self.final_site else 0] +
                  [_lib.attnres_phase1_backward_workspace_bytes(T, d, 1 + self.n_given + b, S)
                   for b, S in enumerate(self.block_sizes)])
        ws = torch.empty((max(ws1, _lib.attnres_phase2_backward_workspace_bytes(T, d), 16) + 3) // 4,
                         dtype=torch.float32, device=dev)
        # dL/db_i for b_0 .. b_N: the final site writes them all first
        if self.final_site:
            dB = torch.empty((n_reps, T, d), dtype=torch.float32, device=dev)
            mark("final_backward", True)
            attnres_phase1_backward(self.reps, n_reps, w[self.L:self.L + 1],
                                    None if g is None else g[self.L:self.L + 1], eps, dh_final.unsqueeze(0), None,
                                    None, dB, dw[self.L:self.L + 1], None if g is None else dg[self.L:self.L + 1],
                                    ws, accumulate=False, stream=stream, check=False)
            mark("final_backward", False)
        else:
            dB = torch.zeros((n_reps, T, d), dtype=torch.float32, device=dev)
        l_end = self.L
        for b in range(len(self.block_sizes) - 1, -1, -1):
            S = self.block_sizes[b]
            l0 = l_end - S
            n = 1 + self.n_given + b
            # the running gradient of the block's outputs starts as dL/db_n
            # (b_n is no source of this block) and gains dL/dp_j per site
            R = dB[n]
            for j in range(S - 1, -1, -1):
                l = l0 + j
                dx = _checked_rows(dx_for(l, R), "dL/dx of sublayer %d" % l, T, d, self.dtype)
                pin, v2, v = self.recipes[l] if j > 0 else (None, None, None)
                mark("phase2_backward", True)
                attnres_phase2_backward(self.o_blocks[b][j], self.lse_blocks[b][j], pin, v, w[l],
                                        None if g is None else g[l], None if gam is None else gam[l], eps, dx,
                                        R if j > 0 else None, G[j], cg[0, j], cg[1, j], dw[l],
                                        None if g is None else dg[l], dgamma[l], ws, sublayer_prev2=v2,
                                        stream=stream, check=False)
                mark("phase2_backward", False)
            mark("phase1_backward", True)
            attnres_phase1_backward(self.reps, n, w[l0:l0 + S], None if g is None else g[l0:l0 + S], eps, G[:S],
                                    cg[0, :S], cg[1, :S], dB, dw[l0:l0 + S], None if g is None else dg[l0:l0 + S],
                                    ws, accumulate=True, stream=stream, check=False)
            mark("phase1_backward", False)
            l_end = l0
        return {"demb": dB[0], "dgiven": dB[1:1 + self.n_given], "dw": dw, "dg": dg, "dgamma": dgamma[:self.L]}


class FullAttnRes:
    """Full AttnRes: every sublayer output is its own depth source ("Attention
    Residuals" notes, section 7).

    ``group=None``: one-shot per site, sublayer l aggregates hist[0..l] with
    attnres_full and PreNorm.  ``group=G``: the grouped two-phase schedule
    (reading notes, static queries and two-phase computation; notes section
    10): for each group of G consecutive sublayers, phase 1 scores the
    sources completed before the group for all G queries at once, then each
    sublayer merges that partition with the outputs produced inside the group
    so far (attnres_phase2_merge_multi).  The phase-1 call of a group reads
    at most ATTNRES_MAX_SOURCES_MULTI completed sources."""

    def __init__(self, T: int, d: int, L: int, dtype: torch.dtype, eps: float = 1e-6, device=None,
                 keep_h: bool = False, final_site: bool = True, group: Optional[int] = None):
        self.T, self.d, self.L, self.dtype, self.eps = int(T), int(d), int(L), dtype, float(eps)
        if L + 1 > _lib.ATTNRES_MAX_SOURCES:
            raise ValueError("Full AttnRes supports at most %d sources" % _lib.ATTNRES_MAX_SOURCES)
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.final_site = final_site
        self.group = None if group is None else int(group)
        self.hist = torch.empty((L + 1, T, d), dtype=dtype, device=dev)  # v_0 = embedding, v_1..v_L
        self.x = torch.empty((2, T, d), dtype=dtype, device=dev)
        self.h = torch.empty((T, d), dtype=dtype, device=dev) if keep_h else None
        self.lse = torch.empty((T,), dtype=torch.float32, device=dev)
        self.h_final = torch.empty((T, d), dtype=dtype, device=dev)
        if self.group is not None:
            G = self.group
            if not 1 <= G <= _lib.ATTNRES_MAX_GROUP_SOURCES:
                raise ValueError("group size must be in [1, %d]" % _lib.ATTNRES_MAX_GROUP_SOURCES)
            n_max = max(g0 + 1 for g0 in range(0, L, G))
            if n_max > _lib.ATTNRES_MAX_SOURCES_MULTI:
                raise ValueError("the last group's phase 1 would read %d sources (at most %d): use larger groups"
                                 % (n_max, _lib.ATTNRES_MAX_SOURCES_MULTI))
            self.o1 = torch.empty((G, T, d), dtype=dtype, device=dev)
            self.m1 = torch.empty((G, T), dtype=torch.float32, device=dev)
            self.lse1 = torch.empty((G, T), dtype=torch.float32, device=dev)
            ws = _lib.attnres_phase1_workspace_bytes(T, d, n_max, G)
            self.workspace = torch.empty((max(ws, 16) + 3) // 4, dtype=torch.float32, device=dev)

    def plan(self) -> List[Launch]:
        r = self.T * self.d * _esize(self.dtype)
        stat = self.T * 4
        if self.group is None:
            # site l reads its l sources and writes x (and h when kept)
            hr = r if self.h is not None else 0
            out = [Launch("full", (l + 1) * r + hr + stat) for l in range(1, self.L + 1)]
        else:
            out = []
            for g0 in range(0, self.L, self.group):
                S = min(self.group, self.L - g0)
                n = g0 + 1
                # + x of the group's first sublayer, written by phase 1
                out.append(Launch("phase1", (2 * r if n == 1 else n * r + S * r) + 2 * S * stat))
                for j in range(1, S):
                    out.append(Launch("phase2", (2 + j) * r + stat))   # o, j group outputs; x
        if self.final_site:
            out.append(Launch("final", (self.L + 2) * r + stat))
        return out

    def forward(self, params: Dict[str, torch.Tensor], sublayer: Callable[[int, torch.Tensor], None],
                hook: Optional[SiteHook] = None, stream=None,
                instrument: Optional[Callable[[str, bool], None]] = None) -> torch.Tensor:
        """``hist[0]`` must hold the embedding; ``sublayer(l, x_l)`` writes the
        output of sublayer l (0-based) into ``hist[l + 1]``."""
        _check_params(params, self.d, self.L + (1 if self.final_site else 0), self.L, self.hist.device)
        w, g, gam = params["w"], params.get("g"), params.get("gamma")
        mark = instrument if instrument is not None else (lambda kind, begin: None)
        if self.group is None:
            for l in range(self.L):
                x = self.x[l % 2]
                mark("full", True)
                attnres_full(self.hist, l + 1, w[l], None if g is None else g[l],
                             None if gam is None else gam[l], self.eps, self.h, x, self.lse, stream=stream,
                             check=False)
                mark("full", False)
                if hook is not None:
                    hook(l, x=x, h=self.h, lse=self.lse)
                sublayer(l, x)
        else:
            for g0 in range(0, self.L, self.group):
                S = min(self.group, self.L - g0)
                n = g0 + 1
                single = n == 1  # only the embedding: every phase-1 output is hist[0]
                mark("phase1", True)
                # the group's first sublayer has no in-group source: its
                # PreNorm output comes out of the phase-1 pass
                attnres_phase1_first_prenorm(self.hist, n, w[g0:g0 + S], None if g is None else g[g0:g0 + S],
                                             self.eps, None if single else self.o1[:S], self.m1[:S],
                                             self.lse1[:S], None if gam is None else gam[g0],
                                             self.x[g0 % 2], self.h, self.workspace, stream=stream, check=False)
                mark("phase1", False)
                for j in range(S):
                    l = g0 + j
                    x = self.x[l % 2]
                    o = self.hist[0] if single else self.o1[j]
                    if j:
                        mark("phase2", True)
                        attnres_phase2_merge_multi(o, self.lse1[j], self.hist[g0 + 1:g0 + 1 + j], j, w[l],
                                                   None if g is None else g[l], None if gam is None else gam[l],
                                                   self.eps, self.h, x, stream=stream, check=False)
                        mark("phase2", False)
                    if hook is not None:
                        hook(l, x=x, h=self.h, lse=None)
                    sublayer(l, x)
        if self.final_site:
            mark("final", True)
            attnres_full(self.hist, self.L + 1, w[self.L], None if g is None else g[self.L], None, self.eps,
                         self.h_final, None, None, stream=stream, check=False)
            mark("final", False)
        return self.h_final

    def plan_backward(self) -> List[Launch]:
        """Algorithmic bytes of ``backward``: per site its sources and dx
        (storage type) once, and the sources' fp32 gradient rows read and
        written once."""
        r = self.T * self.d * _esize(self.dtype)
        r32 = self.T * self.d * 4
        out = []
        if self.final_site:
            out.append(Launch("final_backward", (self.L + 1) * (r + 2 * r32) + r))
        for l in range(self.L - 1, -1, -1):
            out.append(Launch("site_backward", (l + 1) * (r + 2 * r32) + r))
        return out

    def backward(self, params: Dict[str, torch.Tensor], dx_for: Callable[[int, torch.Tensor], torch.Tensor],
                 dh_final: Optional[torch.Tensor] = None, stream=None,
                 instrument: Optional[Callable[[str, bool], None]] = None) -> Dict[str, torch.Tensor]:
        """Backward of the last ``forward`` (``hist`` unchanged since), sites
        in reverse order.  Both schedules compute the same sites, so both have
        the one-shot sites' gradient.  Every representation feeds all later
        sites ("Attention Residuals" notes, section 7), so its gradient is a
        sum over sites, accumulated in one fp32 row per representation.
        ``dx_for(l, dv_l)`` is the sublayer's backward: it receives dL/dv_l
        (= dL/dhist[l+1], fp32 [T, d], complete once every later site has run;
        valid only during the call) and returns dL/dx_l ([T, d], storage
        dtype).  ``dh_final``: dL/dh_final (needed with the final site).
        Returns fp32 ``demb`` [T, d], ``dw``, ``dg`` [L+1, d] (``dg`` stays
        zero without key gains), ``dgamma`` [L, d]."""
        if self.final_site and dh_final is None:
            raise ValueError("dh_final is required with the final aggregation site")
        T, d, L, eps = self.T, self.d, self.L, self.eps
        dev = self.hist.device
        _check_params(params, d, L + (1 if self.final_site else 0), L, dev)
        if self.final_site:
            _checked_rows(dh_final, "dh_final", T, d, self.dtype)
        w, g, gam = params["w"], params.get("g"), params.get("gamma")
        mark = instrument if instrument is not None else (lambda kind, begin: None)
        dH = torch.zeros((L + 1, T, d), dtype=torch.float32, device=dev)
        dw = torch.zeros((L + 1, d), dtype=torch.float32, device=dev)
        dg = torch.zeros((L + 1, d), dtype=torch.float32, device=dev)
        dgamma = torch.zeros((max(L, 1), d), dtype=torch.float32, device=dev)
        ws = torch.empty((max(_lib.attnres_site_backward_workspace_bytes(T, d), 16) + 3) // 4,
                         dtype=torch.float32, device=dev)
        if self.final_site:
            mark("final_backward", True)
            attnres_site_backward_accumulate(self.hist, L + 1, w[L], None if g is None else g[L], None, False, eps,
                                             dh_final, dH, dw[L], None if g is None else dg[L], None, ws,
                                             stream=stream, check=False)
            mark("final_backward", False)
        for l in range(L - 1, -1, -1):
            dx = _checked_rows(dx_for(l, dH[l + 1]), "dL/dx of sublayer %d" % l, T, d, self.dtype)
            mark("site_backward", True)
            attnres_site_backward_accumulate(self.hist, l + 1, w[l], None if g is None else g[l],
                                             None if gam is None else gam[l], True, eps, dx, dH, dw[l],
                                             None if g is None else dg[l], dgamma[l], ws, stream=stream,
                                             check=False)
            mark("site_backward", False)
        return {"demb": dH[0], "dw": dw, "dg": dg, "dgamma": dgamma[:L]}


def prefill_chunked(T_total: int, chunk: int, d: int, block_sizes: Sequence[int], dtype: torch.dtype,
                    params: Dict[str, torch.Tensor], fill_embedding: Callable[[int, int, torch.Tensor], None],
                    sublayer_for_chunk: Callable[[int, int], Sublayer],
                    on_chunk: Optional[Callable[[int, int, BlockAttnRes], None]] = None,
                    eps: float = 1e-6, hook_for_chunk=None) -> BlockAttnRes:
    """Long-context prefill on one GPU, streamed in chunks of ``chunk`` tokens
    ("Attention Residuals 阅读补充", Block AttnRes memory section; the notes'
    section 10 on sequence sharding and chunked prefill).  Depth attention
    never mixes tokens, so each chunk is an independent pass; the per-chunk
    buffers (block representations, phase-1 outputs, partial sum) are
    allocated once and reused, which bounds the resident block cache by the
    chunk length instead of the context length."""
    st = BlockAttnRes(min(chunk, T_total), d, block_sizes, dtype, eps=eps)
    for c0 in range(0, T_total, chunk):
        c1 = min(T_total, c0 + chunk)
        if c1 - c0 != st.T:  # ragged last chunk: release the full-size buffers first
            st = None
            st = BlockAttnRes(c1 - c0, d, block_sizes, dtype, eps=eps)
        fill_embedding(c0, c1, st.reps[0])
        hook = hook_for_chunk(c0, c1) if hook_for_chunk is not None else None
        st.forward(params, sublayer_for_chunk(c0, c1), hook=hook)
        if on_chunk is not None:
            on_chunk(c0, c1, st)
    return st
