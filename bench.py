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
        "kind": "oracle",
        "sample": "%d tokens (batches of %d evenly spaced tokens) of the %d-token chunk, all %d sublayers "
                  "+ final site, fp64, %.1f s of oracle time" % (done, batch, w.T, w.L, spent),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefill_chunk_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="rocprofv3 FETCH_SIZE/WRITE_SIZE summary for the dominant kernel")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the AttnRes aggregation never mixes tokens, so it shards by "
              "token with no communication; multi-GPU runs are not part of this build (--gpus 1).",
              file=sys.stderr)
        return 2

    import torch
    import synth
    import transformer_depth_wise_amd as tdw

    tdw.load()  # fails loudly without the HIP library
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    if w.full or w.chunk:
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
    sub = lambda l, x: v[l]  # noqa: E731

    for _ in range(args.warmup):
        st.forward(prm, sub)
    torch.cuda.synchronize()

    # ---- timed region: K steps, HIP events around every launch on its stream
    recs = []
    stream = torch.cuda.current_stream()

    def instrument(kind, begin):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        if begin:
            recs.append([kind, e, None])
        else:
            recs[-1][2] = e

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        st.forward(prm, sub, instrument=instrument)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    kind_ms = {}
    for kind, a, b in recs:
        kind_ms[kind] = kind_ms.get(kind, 0.0) + a.elapsed_time(b)
    steps = args.steps
    ms_per_step = elapsed * 1e3 / steps
    units = w.T * w.L
    gbps = step_bytes / (elapsed / steps) / 1e9
    kernels = {}
    for k in kind_ms:
        t_step = kind_ms[k] / steps  # ms per step
        kernels[k] = {"ms_per_step": round(t_step, 4), "launches_per_step": kind_count[k],
                      "gbps": round(kind_bytes[k] / (t_step * 1e-3) / 1e9, 1),
                      "bytes_per_step": kind_bytes[k]}
    dom = max(kind_ms, key=lambda k: kind_ms[k])
    launches = kind_count[dom]
    avg_launch_s = kind_ms[dom] / steps / launches * 1e-3
    avg_bytes = kind_bytes[dom] / launches
    achieved = avg_bytes / avg_launch_s / 1e9
    traffic = None
    if os.path.exists(args.traffic):
        try:
            tr = json.load(open(args.traffic))
            if tr.get("kind") == dom and tr.get("workload") == w.name:
                traffic = tr.get("bytes_per_launch")
        except Exception:
            traffic = None
    out = {
        "metric": METRIC,
        "value": round(units * steps / elapsed, 1),
        "unit": "token-sublayers/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "sublayers": w.L,
                   "blocks": list(w.block_sizes), "storage": w.dtype, "partial_sum": "f32",
                   "parallelism": "single GPU"},
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
        "bytes_per_token_sublayer": round(step_bytes / units, 1),
        "rows_per_token_sublayer": round(step_bytes / units / (w.d * w.elem_bytes), 3),
        "kernels": kernels,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "avg_launch_us": round(avg_launch_s * 1e6, 2), "algorithmic_bytes_per_launch": int(avg_bytes)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, emb, v, prm, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
