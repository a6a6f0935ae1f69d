#!/usr/bin/env python3
"""Benchmark of the Block AttnRes depth-aggregation hot path on one MI355X.

One step = one pass of the whole path over the 16K-token prefill chunk
(T=16384, d=7168, bf16 storage, 186 sublayers in 7 blocks of 24 and a tail of
18, plus the final aggregation): 8 phase-1 launches, 186 phase-2 launches, 8
block sums and 1 final aggregation.  All inputs (embedding, the 186 synthetic
sublayer outputs, parameters) are resident in HBM before timing starts.

Prints one JSON line: token-sublayers/s, algorithmic HBM GB/s and its fraction
of the MI355X peak (8 TB/s), the roofline of the dominant kernel class timed
with HIP events on the launch stream, and the fp64 CPU oracle timed on a
bounded token sample on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "AttnRes token-sublayers/s + achieved HBM GB/s (% of MI355X peak)"


def cpu_baseline(w, emb, v, prm, target_s: float):
    """Time the fp64 oracle, as it stands, on a bounded token sample: batches
    of evenly spaced tokens (full depth each) until about ``target_s``
    seconds of oracle time have run."""
    import torch
    import oracle
    import synth

    oracle.build(force=False)
    w_h, g_h, gm_h = oracle._f32(prm["w"]), oracle._f32(prm["g"]), oracle._f32(prm["gamma"])
    order = synth.sample_tokens(w.T, w.T)  # every token, visited in a strided order below
    batch = 256
    stride = max(1, w.T // batch)
    done, spent, start = 0, 0.0, 0
    while spent < target_s and start < stride:
        tokens = order[start::stride][:batch]
        start += 1
        idx = torch.tensor(tokens, dtype=torch.long, device=emb.device)
        e_h = oracle._f32(emb.index_select(0, idx))
        v_h = oracle._f32(torch.stack([t.index_select(0, idx) for t in v]))
        t0 = time.perf_counter()
        oracle.block_forward(e_h, v_h, w_h, g_h, gm_h, w.block_sizes, w.eps, final_site=w.final_site,
                             want=("hfinal",))
        spent += time.perf_counter() - t0
        done += len(tokens)
    return {
        "value": round(done * w.L / spent, 1),
        "unit": "token-sublayers/s",
        "cores": oracle.threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": "%d tokens (batches of %d evenly spaced tokens) of the %d-token chunk, all %d sublayers "
                  "+ final site, fp64, %.1f s of oracle time" % (done, batch, w.T, w.L, spent),
    }


def cpu_model() -> str:
    """The host CPU's model name and logical core count, as the OS reports them."""
    name = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    import platform
    return "%s (%d logical cores visible)" % (name or platform.processor() or "unknown", os.cpu_count() or 0)


PROBE_SHAPES = [(g, u, nt) for g in (1, 2, 4) for u in (1, 2, 8) for nt in (False, True)]


def ceiling(dev, total_bytes: int = 4 << 30, reps: int = 6) -> dict:
    """Achievable HBM rate of plain streaming kernels (attnres_stream_probe:
    16-byte accesses, persistent grid-stride loop) with the read/write mixes
    of the path's kernels: read-only, write-only, copy, and the phase-2
    merge's two mixes (odd positions read o, the stored partial and v and
    write x: about 3 reads : 1 write; even positions also read the
    one-before-last output and store the partial: about 4 : 2), eight
    concurrent read streams (the scoring pass over the last blocks'
    sources), nine reads with one write (the final aggregation) and seven
    reads with 24 writes (the phase-1 output pass of a 7-source, 24-sublayer
    block).  Each mix
    is run in 18 launch shapes (1, 2 or 4 workgroups per CU; 1, 2 or 8
    chunks in flight per thread; plain or non-temporal accesses) and the
    best rate is reported with its shape.  Each dispatch moves
    ``total_bytes``, far beyond the 256 MB last-level cache; a rate is the
    mean over ``reps`` dispatches timed with HIP events on the launch
    stream."""
    import torch
    import transformer_depth_wise_amd as tdw

    src = torch.empty((total_bytes,), dtype=torch.uint8, device=dev)
    dst = torch.empty((total_bytes,), dtype=torch.uint8, device=dev)
    src.fill_(1)
    stream = torch.cuda.current_stream()
    out = {"bytes_per_dispatch": total_bytes, "unit": "GB/s",
           "note": "attnres_stream_probe: the rate a streaming kernel with this read:write mix reaches here"}
    for name, nr, nw in (("read", 1, 0), ("write", 0, 1), ("copy", 1, 1), ("mix_3r1w", 3, 1),
                         ("mix_4r2w", 4, 2), ("read_8", 8, 0), ("mix_9r1w", 9, 1), ("mix_7r24w", 7, 24)):
        sb = (total_bytes // (nr + nw)) // (1 << 20) * (1 << 20)
        best, shape = 0.0, None
        for g, u, nt in PROBE_SHAPES:
            tdw.attnres_stream_probe(nr, nw, src, dst, sb, g, u, nt)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                tdw.attnres_stream_probe(nr, nw, src, dst, sb, g, u, nt)
            e1.record(stream)
            e1.synchronize()
            rate = (nr + nw) * sb / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e9
            if rate > best:
                best, shape = rate, {"workgroups_per_cu": g, "unroll": u, "nontemporal": nt}
        out[name] = round(best, 1)
        out[name + "_shape"] = shape
    del src, dst
    torch.cuda.empty_cache()
    return out


def measured_traffic(path, kind, workload, alg_bytes_per_launch=None):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when there is none,
    the kernel's sources changed since the counters were taken, or the
    launch mix differs (the current plan's algorithmic bytes per launch are
    not the ones the counters were taken with)."""
    import hashlib
    if not os.path.exists(path):
        return None
    try:
        tr = json.load(open(path))
    except ValueError:
        return None
    if tr.get("kind") != kind or tr.get("workload") != workload:
        return None
    h = hashlib.sha256()
    for f in tr.get("sources", []):
        fp = os.path.join(ROOT, f)
        if not os.path.exists(fp):
            return None
        h.update(open(fp, "rb").read())
    if h.hexdigest()[:16] != tr.get("source_sha256_16"):
        return None
    if alg_bytes_per_launch is not None and int(alg_bytes_per_launch) != tr.get("algorithmic_bytes_per_launch"):
        return None
    return tr.get("bytes_per_launch")


def long_prefill_report(w, dev):
    """Peak device memory and throughput of the long-context prefill, streamed
    in chunks vs one unchunked pass.  Sublayer outputs are generated for the
    tokens at hand between phase-2 launches (the full context's outputs would
    not fit), so the times include that generation; the memory split reports
    the AttnRes buffers separately from the total peak."""
    import torch
    import synth
    import transformer_depth_wise_amd as tdw

    scales = synth.sublayer_scales(w)
    prm = synth.params(w, dev)
    res = {"metric": "long-context prefill peak device memory, chunked vs unchunked", "config": {
        "workload": w.name, "T": w.T, "chunk": w.chunk, "d": w.d, "sublayers": w.L,
        "blocks": list(w.block_sizes)}}
    for label, chunk in (("chunked", w.chunk), ("unchunked", w.T)):
        ledger = {}

        def fill(c0, c1, dst):
            dst.copy_(synth.embedding(w, c0, c1, dev))

        def sub_for(c0, c1):
            return lambda l, x: synth.sublayer_output(w, l + 1, c0, c1, dev, scales)

        def on_chunk(c0, c1, st):
            ledger.update(st.buffer_bytes())

        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        t0 = time.perf_counter()
        tdw.prefill_chunked(w.T, chunk, w.d, w.block_sizes, w.torch_dtype, prm, fill, sub_for,
                            on_chunk=on_chunk, eps=w.eps)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        res[label] = {"peak_gb": round((torch.cuda.max_memory_allocated() - base) / 1e9, 3),
                      "attnres_buffers_gb": round(ledger["total"] / 1e9, 3),
                      "block_reps_gb": round(ledger["block_reps"] / 1e9, 3),
                      "seconds_incl_generation": round(el, 3)}
    return res


def _time(fn, steps: int) -> float:
    """Seconds per call of ``fn`` over ``steps`` calls, GPU-synchronised."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        fn(k)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def backward_report(dev, steps: int):
    """Backward through the whole block structure of the 16K chunk
    (training): one training forward keeps the phase-1 outputs and partial
    sums, then ``max(2, steps // 4)`` backward passes are timed, and one more
    with HIP events around every launch gives the per-kernel times (such
    events cost a few microseconds each, so the timed passes carry none).
    The synthetic upstream gradient of sublayer l's input is another
    sublayer's output row (a model's sublayer backward would produce it from
    dL/dv_l)."""
    import torch
    import synth
    import transformer_depth_wise_amd as tdw

    w = synth.WORKLOADS["prefill_chunk_bf16"]
    prm = synth.params(w, dev)
    scales = synth.sublayer_scales(w)
    st = tdw.BlockAttnRes(w.T, w.d, w.block_sizes, w.torch_dtype, n_given=w.n_given, eps=w.eps, device=dev,
                          final_site=w.final_site, training=True)
    st.reps[0].copy_(synth.embedding(w, 0, w.T, dev))
    v = [synth.sublayer_output(w, l + 1, 0, w.T, dev, scales) for l in range(w.L)]
    st.forward(prm, lambda l, x: v[l])
    dx_for = lambda l, dv: v[(l + 1) % w.L]  # noqa: E731
    recs = []
    stream = torch.cuda.current_stream()

    def instrument(kind, begin):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        if begin:
            recs.append([kind, e, None])
        else:
            recs[-1][2] = e

    dhf = v[0].to(st.h_final.dtype)   # h_final is fp32 in a bf16 training pass
    st.backward(prm, dx_for, dh_final=dhf)
    nb = max(2, steps // 4)
    sec = _time(lambda k: st.backward(prm, dx_for, dh_final=dhf), nb)
    st.backward(prm, dx_for, dh_final=dhf, instrument=instrument)
    torch.cuda.synchronize()
    plan = st.plan_backward()
    b = sum(x.bytes for x in plan)
    kinds = {}
    for kind, e0, e1 in recs:
        kinds.setdefault(kind, [0.0, 0])
        kinds[kind][0] += e0.elapsed_time(e1)
        kinds[kind][1] += 1
    kb = {}
    for x in plan:
        kb[x.kind] = kb.get(x.kind, 0) + x.bytes
    out = {
        "config": {"T": w.T, "d": w.d, "blocks": list(w.block_sizes), "final_site": w.final_site},
        "ms_per_step": round(sec * 1e3, 4), "value": round(w.T * w.L / sec, 1), "unit": "token-sublayers/s",
        "hbm_gbps": round(b / sec / 1e9, 1), "bytes_per_step": b,
        "kernels": {k: {"ms_per_step": round(ms, 4), "launches_per_step": c,
                        "gbps": round(kb[k] / (ms * 1e-3) / 1e9, 1)} for k, (ms, c) in kinds.items()},
        "note": "backward only (the training forward that keeps its activations is not timed here)"}
    del st, v
    torch.cuda.empty_cache()
    return out


def full_backward_report(fulls, prm, steps: int) -> dict:
    """Backward of Full AttnRes over resident outputs (site backward passes
    accumulating every representation's gradient in fp32), rotating over the
    given FullAttnRes states; the synthetic sublayer backward returns another
    resident output row as dL/dx_l."""
    f0 = fulls[0]
    L = f0.L
    dxs = [f0.hist[(l + 2) % (L + 1)] for l in range(L)]
    dxf = lambda l, dv: dxs[l]  # noqa: E731
    for f in fulls:
        f.backward(prm, dxf, dh_final=f.hist[1])
    nf = len(fulls)
    sec = _time(lambda k: fulls[k % nf].backward(prm, dxf, dh_final=fulls[k % nf].hist[1]), max(steps, 20))
    b = sum(x.bytes for x in f0.plan_backward())
    return {"config": {"T": f0.T, "d": f0.d, "sublayers": L, "schedule": "site backward, reverse"},
            "ms_per_step": round(sec * 1e3, 4), "value": round(f0.T * L / sec, 1),
            "unit": "token-sublayers/s", "hbm_gbps": round(b / sec / 1e9, 1), "bytes_per_step": b,
            "note": "includes zeroing the fp32 gradient rows and parameter gradients"}


def full_states(w, dev, replicas: int):
    """FullAttnRes states over resident synthetic outputs of workload w."""
    import synth
    import transformer_depth_wise_amd as tdw
    prm = synth.params(w, dev)
    scales = synth.sublayer_scales(w)
    fulls = []
    for r in range(replicas):
        f = tdw.FullAttnRes(w.T, w.d, w.L, w.torch_dtype, eps=w.eps, device=dev, final_site=w.final_site)
        f.hist[0].copy_(synth.embedding(w, 0, w.T, dev))
        for l in range(w.L):
            f.hist[l + 1].copy_(synth.sublayer_output(w, l + 1, 0, w.T, dev, scales))
        fulls.append(f)
    return fulls, prm


def io_model(w, rows) -> dict:
    """The measured path's algorithmic rows per token and sublayer beside the
    pages' analytic residual I/O per layer (rows of d): at this workload's
    depth and block count, and at the pages' own L = 128, N = 8, S = 16."""
    from transformer_depth_wise_amd import costmodel as cm
    N = len(w.block_sizes)
    return {"this_path": round(rows, 3),
            "pages_model_here": cm.model_for(w.L, N),
            "pages_model_L128_N8_S16": {"standard_residual": cm.io_standard_residual(1),
                                        "mhc_m4": round(cm.io_mhc(4, w.d) / w.d, 3),
                                        "full_two_phase": cm.io_full_two_phase(16, 8, 1),
                                        "block_two_phase": cm.io_block_two_phase(8, 16, 1)},
            "note": "the pages give no breakdown of the 5 rows of their Block figure; this path counts "
                    "the write and re-read of the phase-1 outputs and its 24-bit partial sum explicitly"}


def other_workloads(dev, steps: int):
    """Shorter measurements of the other hot-path shapes, each pass over
    resident inputs: the decode-shaped block step (eager launches and one
    HIP-graph replay per pass), Full AttnRes (one-shot sites and the grouped
    schedule, each eager and as a graph replay; the backward), one aggregation site's backward, and one GPU's
    token share (2048 tokens) of the 16K chunk.  Working sets that fit the
    256 MB last-level cache rotate over 4 input replicas so that every pass
    reads from HBM."""
    import torch
    import synth
    import transformer_depth_wise_amd as tdw

    res = {}

    def block_states(w, replicas):
        sts, subs = [], []
        prm = synth.params(w, dev)
        scales = synth.sublayer_scales(w)
        for r in range(replicas):
            st = tdw.BlockAttnRes(w.T, w.d, w.block_sizes, w.torch_dtype, n_given=w.n_given, eps=w.eps,
                                  device=dev, final_site=w.final_site)
            st.reps[0].copy_(synth.embedding(w, 0, w.T, dev))
            for n in range(w.n_given):
                st.reps[1 + n].copy_(synth.given_block(w, n + 1, 0, w.T, dev))
            v = [synth.sublayer_output(w, l + 1, 0, w.T, dev, scales) for l in range(w.L)]
            sts.append(st)
            subs.append(lambda l, x, v=v: v[l])
        return sts, subs, prm

    def summary(w, st, sec):
        b = sum(x.bytes for x in st.plan())
        return {"config": {"T": w.T, "d": w.d, "blocks": list(w.block_sizes), "given_blocks": w.n_given},
                "ms_per_step": round(sec * 1e3, 4), "value": round(w.T * w.L / sec, 1),
                "unit": "token-sublayers/s", "hbm_gbps": round(b / sec / 1e9, 1),
                "bytes_per_step": b}

    # decode-shaped block step: T=256, one block of 24, 7 given block sums
    w = synth.WORKLOADS["decode_block_bf16"]
    sts, subs, prm = block_states(w, 4)
    for k in range(4):
        sts[k].forward(prm, subs[k])
    eager = _time(lambda k: sts[k % 4].forward(prm, subs[k % 4]), max(steps, 20))
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in range(4):
            sts[k].forward(prm, subs[k])
    torch.cuda.current_stream().wait_stream(side)
    for k in range(4):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sts[k].forward(prm, subs[k])
        graphs.append(g)
    replay = _time(lambda k: graphs[k % 4].replay(), max(steps, 20))
    res[w.name] = summary(w, sts[0], eager)
    res[w.name]["launches_per_step"] = len(sts[0].plan())
    res[w.name]["graph_replay"] = {"ms_per_step": round(replay * 1e3, 4),
                                   "value": round(w.T * w.L / replay, 1),
                                   "hbm_gbps": round(res[w.name]["bytes_per_step"] / replay / 1e9, 1)}
    del graphs, sts, subs

    # Full AttnRes: every sublayer output its own source, one-shot per site
    w = synth.WORKLOADS["full_bf16"]
    fulls, prm = full_states(w, dev, 4)
    noop = lambda l, x: None  # noqa: E731  (outputs are resident in hist)
    for f in fulls:
        f.forward(prm, noop)
    sec = _time(lambda k: fulls[k % 4].forward(prm, noop), max(steps, 20))
    b = sum(x.bytes for x in fulls[0].plan())
    res[w.name] = {"config": {"T": w.T, "d": w.d, "sublayers": w.L, "schedule": "one-shot sites"},
                   "ms_per_step": round(sec * 1e3, 4),
                   "value": round(w.T * w.L / sec, 1), "unit": "token-sublayers/s",
                   "hbm_gbps": round(b / sec / 1e9, 1), "bytes_per_step": b,
                   "note": "one-shot sites re-read earlier outputs; those re-reads partly hit the last-level cache"}
    # the grouped two-phase schedule over the same resident outputs (groups of 4)
    grouped = []
    for f in fulls:
        gr = tdw.FullAttnRes(w.T, w.d, w.L, w.torch_dtype, eps=w.eps, device=dev, final_site=w.final_site, group=4)
        gr.hist = f.hist
        grouped.append(gr)
    for gr in grouped:
        gr.forward(prm, noop)
    sec = _time(lambda k: grouped[k % 4].forward(prm, noop), max(steps, 20))
    b = sum(x.bytes for x in grouped[0].plan())
    res[w.name + "_grouped4"] = {"config": {"T": w.T, "d": w.d, "sublayers": w.L,
                                            "schedule": "grouped two-phase, groups of 4"},
                                 "ms_per_step": round(sec * 1e3, 4), "value": round(w.T * w.L / sec, 1),
                                 "unit": "token-sublayers/s", "hbm_gbps": round(b / sec / 1e9, 1),
                                 "bytes_per_step": b}
    # both schedules as one HIP-graph replay per pass (at 8 MB per row set the
    # launches, 17 one-shot against 32 grouped, weigh as much as the bytes)
    for key, states in ((w.name, fulls), (w.name + "_grouped4", grouped)):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for st in states:
                st.forward(prm, noop)
        torch.cuda.current_stream().wait_stream(side)
        gs = []
        for st in states:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                st.forward(prm, noop)
            gs.append(g)
        sec = _time(lambda k: gs[k % len(gs)].replay(), max(steps, 20))
        res[key]["graph_replay"] = {"ms_per_step": round(sec * 1e3, 4), "value": round(w.T * w.L / sec, 1),
                                    "hbm_gbps": round(res[key]["bytes_per_step"] / sec / 1e9, 1)}
        del gs
    res[w.name + "_backward"] = full_backward_report(fulls, prm, steps)
    del fulls, grouped
    torch.cuda.empty_cache()

    # a larger Full AttnRes shape, where the bytes rather than the launches
    # decide: one-shot sites re-read every earlier output (152 rows per token
    # at depth 16), the grouped schedule reads each completed source once per
    # group (groups of 4: 107 rows)
    wl = synth.scaled(w, name="full_bf16_T16384_d4096", T=16384, d=4096)
    fl, prm = full_states(wl, dev, 1)
    gl = tdw.FullAttnRes(wl.T, wl.d, wl.L, wl.torch_dtype, eps=wl.eps, device=dev, final_site=wl.final_site, group=4)
    gl.hist = fl[0].hist
    for name, st in (("one_shot", fl[0]), ("grouped4", gl)):
        st.forward(prm, noop)
        sec = _time(lambda k: st.forward(prm, noop), max(steps // 2, 10))
        b = sum(x.bytes for x in st.plan())
        res.setdefault(wl.name, {"config": {"T": wl.T, "d": wl.d, "sublayers": wl.L}})[name] = {
            "ms_per_step": round(sec * 1e3, 4), "value": round(wl.T * wl.L / sec, 1), "unit": "token-sublayers/s",
            "hbm_gbps": round(b / sec / 1e9, 1), "bytes_per_step": b, "launches_per_step": len(st.plan())}
    del fl, gl

    # backward of one aggregation site at the 16K chunk's final-site shape
    # (9 sources), with and without the PreNorm
    T, d, n = 16384, 7168, 9
    gen = torch.Generator(device=dev).manual_seed(77)
    src = torch.randn((n, T, d), generator=gen, device=dev).to(torch.bfloat16)
    dx = torch.randn((T, d), generator=gen, device=dev).to(torch.bfloat16)
    wq = torch.randn((d,), generator=gen, device=dev) * 0.02
    kg = torch.rand((d,), generator=gen, device=dev) * 0.4 + 0.8
    dsrc = torch.empty_like(src)
    dw, dkg, dgm = (torch.empty((d,), device=dev) for _ in range(3))
    ws = torch.empty(tdw.attnres_site_backward_workspace_bytes(T, d) // 4 + 4, device=dev)
    for prenorm in (True, False):
        f = lambda k: tdw.attnres_site_backward(src, n, wq, kg, kg if prenorm else None, prenorm, 1e-6, dx,  # noqa
                                                dsrc, dw, dkg, dgm if prenorm else None, ws)
        f(0)
        sec = _time(f, max(steps, 10))
        b = (2 * n + 1) * T * d * 2
        res["site_backward_n9" + ("_prenorm" if prenorm else "")] = {
            "config": {"T": T, "d": d, "sources": n, "prenorm": prenorm}, "ms_per_step": round(sec * 1e3, 4),
            "value": round(T / sec, 1), "unit": "tokens/s", "hbm_gbps": round(b / sec / 1e9, 1),
            "bytes_per_step": b, "note": "reads 9 source rows + dx, writes 9 gradient rows per token"}
    del src, dx, dsrc, ws

    # one GPU's share (16384 / 8 tokens) of the 16K chunk
    w = synth.scaled(synth.WORKLOADS["prefill_chunk_bf16"], T=2048, name="prefill_share_2048")
    sts, subs, prm = block_states(w, 1)
    sts[0].forward(prm, subs[0])
    sec = _time(lambda k: sts[0].forward(prm, subs[0]), steps)
    res[w.name] = summary(w, sts[0], sec)
    del sts, subs
    torch.cuda.empty_cache()

    res["block_backward_prefill_chunk"] = backward_report(dev, steps)
    torch.cuda.empty_cache()
    # the long-context workload: 131072 tokens in 16K chunks vs unchunked
    res["long_prefill_memory"] = long_prefill_report(synth.WORKLOADS["long_prefill_bf16"], dev)
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_chunk_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the decode / Full / per-GPU-share workloads")
    ap.add_argument("--backward", action="store_true",
                    help="time only a backward (one JSON line): through the 16K chunk's block structure, or "
                         "with --workload full_bf16 that of Full AttnRes")
    ap.add_argument("--probe", choices=["copy"], default=None,
                    help="run only a plain device copy of known size (counter calibration)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="rocprofv3 FETCH_SIZE/WRITE_SIZE summary for the dominant kernel")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the AttnRes aggregation never mixes tokens, so it shards by "
              "token with no communication; a run over several GPUs is not supported (use --gpus 1).",
              file=sys.stderr)
        return 2

    import torch
    import synth
    import transformer_depth_wise_amd as tdw

    tdw.load()  # fails loudly without the HIP library
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.probe == "copy":
        # 1 GiB read + 1 GiB written per dispatch, 4 dispatches
        a = torch.ones((1 << 29,), dtype=torch.bfloat16, device=dev)
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"probe": "copy", "bytes_read_per_dispatch": a.numel() * 2,
                          "bytes_written_per_dispatch": b.numel() * 2, "dispatches": 4}), flush=True)
        return 0
    w = synth.WORKLOADS[args.workload]
    if args.backward and w.full:
        fulls, prm = full_states(w, dev, 4)
        print(json.dumps({"metric": "AttnRes backward token-sublayers/s (Full AttnRes, %s)" % w.name,
                          **full_backward_report(fulls, prm, args.steps)}), flush=True)
        return 0
    if args.backward:
        print(json.dumps({"metric": "AttnRes backward token-sublayers/s (block structure, 16K chunk)",
                          **backward_report(dev, args.steps)}), flush=True)
        return 0
    if w.chunk:
        print(json.dumps(long_prefill_report(w, dev)), flush=True)
        return 0
    if w.full:
        raise SystemExit("bench.py times the block workloads only")

    # ---- inputs resident in HBM (untimed)
    scales = synth.sublayer_scales(w)
    emb = synth.embedding(w, 0, w.T, dev)
    v = [synth.sublayer_output(w, l + 1, 0, w.T, dev, scales) for l in range(w.L)]
    given = [synth.given_block(w, n + 1, 0, w.T, dev) for n in range(w.n_given)]
    prm = synth.params(w, dev)
    st = tdw.BlockAttnRes(w.T, w.d, w.block_sizes, w.torch_dtype, n_given=w.n_given, eps=w.eps, device=dev,
                          final_site=w.final_site)
    st.reps[0].copy_(emb)
    for n, b in enumerate(given):
        st.reps[1 + n].copy_(b)
    plan = st.plan()
    step_bytes = sum(x.bytes for x in plan)
    kind_bytes = {}
    kind_count = {}
    for x in plan:
        kind_bytes[x.kind] = kind_bytes.get(x.kind, 0) + x.bytes
        kind_count[x.kind] = kind_count.get(x.kind, 0) + 1
    # the scope table's plain row model of the same launches
    survey = st.plan_survey()
    survey_bytes = sum(x.bytes for x in survey)
    survey_kind = {}
    for x in survey:
        survey_kind[x.kind] = survey_kind.get(x.kind, 0) + x.bytes
    sub = lambda l, x: v[l]  # noqa: E731

    for _ in range(args.warmup):
        st.forward(prm, sub)
    torch.cuda.synchronize()

    # ---- timed region: K steps.  Every pass is bracketed by HIP events on
    # the launch stream; the last few passes also carry an event wherever the
    # launch kind changes (per-kernel times, the roofline's launch duration):
    # consecutive launches of one kind, such as a block's merges, which have
    # no other GPU work between them here, are timed as one group, so that an
    # event costs its few microseconds once per group instead of twice per
    # launch.  The other passes run without them.
    recs = []
    stream = torch.cuda.current_stream()
    n_instr = min(2, args.steps)
    group = {"kind": None}

    def instrument(kind, begin):
        if not begin or kind == group["kind"]:
            return
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        if recs and recs[-1][2] is None:
            recs[-1][2] = e
        recs.append([kind, e, None])
        group["kind"] = kind

    pass_ev = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        a = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        timed = i >= args.steps - n_instr
        st.forward(prm, sub, instrument=instrument if timed else None)
        if timed:
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            recs[-1][2] = e
            group["kind"] = None
        b = torch.cuda.Event(enable_timing=True)
        b.record(stream)
        pass_ev.append((a, b))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    kind_ms = {}
    for kind, a, b in recs:
        kind_ms[kind] = kind_ms.get(kind, 0.0) + a.elapsed_time(b) / n_instr
    spans = [a.elapsed_time(b) for a, b in pass_ev]
    plain = sorted(spans[:args.steps - n_instr]) or sorted(spans)
    instr = spans[args.steps - n_instr:]

    # ---- cold-cache pass: a 512 MiB scratch write between consecutive
    # launches evicts the 256 MB last-level cache (MALL), as the sublayers of
    # a model would; only the AttnRes launches are timed (events around each).
    scratch = torch.empty((1 << 28,), dtype=torch.float16, device=dev)
    crecs = []

    def instrument_cold(kind, begin):
        if begin:
            scratch.fill_(1.0)
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        if begin:
            crecs.append([kind, e, None])
        else:
            crecs[-1][2] = e

    cold_steps = max(1, min(3, args.steps))
    for _ in range(cold_steps):
        st.forward(prm, sub, instrument=instrument_cold)
    torch.cuda.synchronize()
    cold_kind = {}
    for kind, a, b in crecs:
        cold_kind[kind] = cold_kind.get(kind, 0.0) + a.elapsed_time(b) / cold_steps
    del scratch
    cold_ms = sum(cold_kind.values())
    steps = args.steps
    ms_per_step = elapsed * 1e3 / steps
    units = w.T * w.L
    gbps = step_bytes / (elapsed / steps) / 1e9
    kernels = {}
    for k in kind_ms:
        t_step = kind_ms[k]  # ms per step (mean over the instrumented passes)
        kernels[k] = {"ms_per_step": round(t_step, 4), "launches_per_step": kind_count[k],
                      "gbps": round(survey_kind[k] / (t_step * 1e-3) / 1e9, 1),
                      "bytes_per_step": survey_kind[k],
                      "path_gbps": round(kind_bytes[k] / (t_step * 1e-3) / 1e9, 1),
                      "path_bytes_per_step": kind_bytes[k]}
    dom = max(kind_ms, key=lambda k: kind_ms[k])
    launches = kind_count[dom]
    avg_launch_s = kind_ms[dom] / launches * 1e-3
    avg_bytes = kind_bytes[dom] / launches
    avg_survey = survey_kind[dom] / launches
    achieved = avg_survey / avg_launch_s / 1e9
    achieved_path = avg_bytes / avg_launch_s / 1e9
    traffic = measured_traffic(args.traffic, dom, w.name, int(avg_bytes))
    ceil = ceiling(dev)
    for k, mix in (("phase2", "mix_3r1w"), ("accumulate", "mix_3r1w"), ("final", "mix_9r1w")):
        if k in kernels:
            kernels[k]["frac_of_ceiling"] = {mix: round(kernels[k]["path_gbps"] / ceil[mix], 4)}
    survey_gbps = survey_bytes / (elapsed / steps) / 1e9
    out = {
        "metric": METRIC,
        "value": round(units * steps / elapsed, 1),
        "unit": "token-sublayers/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms": {"median": round(statistics.median(plain), 4),
                    "p90": round(plain[-(-9 * len(plain) // 10) - 1], 4),  # nearest rank
                    "min": round(plain[0], 4), "max": round(plain[-1], 4),
                    "instrumented": [round(x, 4) for x in instr],
                    "note": "per-pass HIP-event spans of the passes without per-launch events; "
                            "'instrumented': the last %d passes, which also time every group of launches of one kind" % n_instr},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "sublayers": w.L,
                   "blocks": list(w.block_sizes), "storage": w.dtype, "partial_sum": st.partial_format,
                   "parallelism": "single GPU"},
        "hbm_gbps": round(survey_gbps, 1),
        "hbm_frac": round(survey_gbps / PEAK_HBM_GBPS, 4),
        "bytes_per_step": survey_bytes,
        "byte_model": "the scope table's rows (phase 1: n + S, merges 2/3/5, block sum 3, final N + 2 rows per "
                      "token); path_bytes adds what this path really moves beyond it (the 24-bit partial "
                      "sum's extra byte plane, the stored-every-second-sublayer schedule, statistics)",
        "path_bytes": {"bytes_per_step": step_bytes, "hbm_gbps": round(gbps, 1),
                       "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4)},
        "bytes_per_token_sublayer": round(step_bytes / units, 1),
        "rows_per_token_sublayer": round(step_bytes / units / (w.d * w.elem_bytes), 3),
        "io_model": io_model(w, step_bytes / units / (w.d * w.elem_bytes)),
        "kernels": kernels,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "avg_launch_us": round(avg_launch_s * 1e6, 2),
                     "algorithmic_bytes_per_launch": int(avg_survey),
                     "frac_survey_bytes": round(achieved / PEAK_HBM_GBPS, 4),
                     "path_bytes_per_launch": int(avg_bytes),
                     "achieved_path_bytes": round(achieved_path, 1),
                     "frac_path_bytes": round(achieved_path / PEAK_HBM_GBPS, 4),
                     "frac_of_ceiling": {k: round(achieved_path / ceil[k], 4) for k in ("copy", "mix_3r1w",
                                                                                         "mix_4r2w")},
                     "note": "traffic is measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                             "copy-calibrated) and compares with path_bytes_per_launch; frac_of_ceiling "
                             "divides the path's bytes by the streaming probe's rate at the same mixes"},
        "ceiling": ceil,
        "cold_cache": {
            "note": "512 MiB scratch write between launches (MALL evicted), AttnRes kernels only",
            "ms_per_step": round(cold_ms, 4),
            "value": round(units / (cold_ms * 1e-3), 1),
            "hbm_gbps": round(survey_bytes / (cold_ms * 1e-3) / 1e9, 1),
            "path_hbm_gbps": round(step_bytes / (cold_ms * 1e-3) / 1e9, 1),
            "kernels_path_gbps": {k: round(kind_bytes[k] / (cold_kind[k] * 1e-3) / 1e9, 1) for k in cold_kind},
            "dominant_frac": round(survey_kind[dom] / (cold_kind[dom] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, emb, v, prm, args.cpu_seconds)
    if not args.no_other:
        del v, st, emb, sub, given
        torch.cuda.empty_cache()
        out["other_workloads"] = other_workloads(dev, args.steps)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
