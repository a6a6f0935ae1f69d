"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Every workload runs through the C ABI in the launch configuration the
benchmark uses.  Each test prints the case it is about to run before any GPU
work, so a failure can be attributed from the log alone.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import TOL, Capture, row_rel_err, run_block_parity, run_full_parity, stat_err, _host
import transformer_depth_wise_amd as tdw

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    tdw.load()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ------------------------------------------------------------ full workloads
def test_tiny_block_f32_all_tokens():
    w = synth.WORKLOADS["tiny_block_f32"]
    _say("case tiny_block_f32 T=%d d=%d blocks=%s" % (w.T, w.d, w.block_sizes))
    worst = run_block_parity(w)
    _say("worst", worst)


def test_full_bf16_all_sites():
    w = synth.WORKLOADS["full_bf16"]
    _say("case full_bf16 T=%d d=%d L=%d (sampled 512 tokens)" % (w.T, w.d, w.L))
    worst = run_full_parity(w, samples=synth.sample_tokens(w.T, 512))
    _say("worst", worst)


def test_decode_block_bf16_all_tokens():
    w = synth.WORKLOADS["decode_block_bf16"]
    _say("case decode_block_bf16 T=%d d=%d S=24 given=%d" % (w.T, w.d, w.n_given))
    worst = run_block_parity(w)
    _say("worst", worst)


@pytest.mark.parametrize("partial", ["q16", "p24", "f32"])
def test_prefill_chunk_bf16_sampled(partial):
    w = synth.WORKLOADS["prefill_chunk_bf16"]
    _say("case prefill_chunk_bf16 T=%d d=%d blocks=%s partial=%s (64 sampled tokens)"
         % (w.T, w.d, w.block_sizes, partial))
    worst = run_block_parity(w, samples=synth.sample_tokens(w.T, 64), keep_h=True, partial=partial)
    _say("worst", worst)


def _p24_emulate(x: np.ndarray) -> np.ndarray:
    """The 24-bit split format's value of fp32 x: round to nearest even at
    bit 8 of the encoding, keep the upper 24 bits."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7F + ((u >> 8) & 1)) & 0xFFFFFF00
    return r.astype(np.uint32).view(np.float32)


def test_p24_partial_roundtrip_is_exact():
    _say("case P24 partial round trip")
    dev = torch.device("cuda")
    T, d = 37, 1032
    pin = (torch.randn((T, d), device=dev) * torch.logspace(-3, 3, d, device=dev)).float()
    pin[0, :8] = torch.tensor([0.0, -0.0, 1.0, -1.0, 1.0 + 2 ** -16, 1.0 + 3 * 2 ** -17, 3e-38, -65504.0])
    zeros = torch.zeros((T, d), dtype=torch.float32, device=dev)
    o = torch.randn((T, d), device=dev)
    lse = torch.zeros((T,), device=dev)
    p24 = tdw._lib.p24_partial(T, d, dev)
    x = torch.empty((T, d), device=dev)
    # p = pin + 0, stored as P24
    tdw.attnres_phase2_merge(o, lse, pin, zeros, p24, torch.zeros(d, device=dev), None, None, 1e-6, None, x)
    back = torch.empty((T, d), device=dev)
    tdw.attnres_block_accumulate(p24, zeros, back)  # P24 -> fp32 + 0
    torch.cuda.synchronize()
    got, want = back.cpu().numpy(), _p24_emulate(pin.cpu().numpy())
    # value comparison: the kernels compute pin + 0.0, which turns -0.0 into +0.0
    bad = np.argwhere(got != want)
    assert bad.size == 0, "P24 mismatch at %s: got %r want %r (input %r)" % (
        bad[:4].tolist(), got[tuple(bad[0])], want[tuple(bad[0])], pin.cpu().numpy()[tuple(bad[0])])
    rel = np.abs(back.cpu().numpy() - pin.cpu().numpy()) / np.maximum(np.abs(pin.cpu().numpy()), 1e-30)
    assert rel.max() <= 2.0 ** -16


def _q16_emulate(x: np.ndarray) -> np.ndarray:
    """The Q16 format's value of fp32 rows x: per row the exponent e of
    frexp(max |x|) (max |x| < 2^e), q = x * 2^(15 - e) rounded to nearest
    even and clamped to [-32767, 32767], value q * 2^(e - 15)."""
    x = x.astype(np.float64)
    e = np.frexp(np.abs(x).max(axis=1))[1][:, None].astype(np.float64)
    q = np.clip(np.rint(np.ldexp(x, (15 - e).astype(np.int64))), -32767, 32767)
    return np.ldexp(q, (e - 15).astype(np.int64))


def test_q16_partial_roundtrip_is_exact():
    _say("case Q16 partial round trip")
    dev = torch.device("cuda")
    T, d = 37, 1032
    row_scale = torch.logspace(-20, 20, T, device=dev)[:, None]
    pin = (torch.randn((T, d), device=dev) * row_scale).float()
    pin[0] = 0.0                                          # zero row: exponent 0, all zeros
    pin[1, :] = 0.25
    pin[1, 5] = -1.0                                      # largest magnitude exactly a power of two
    pin[2, :] = 1e-3
    pin[2, 7] = 1.0 - 2.0 ** -20                          # rounds to 32768 steps: clamped to 32767
    pin[3, :8] = torch.tensor([3.0, -3.0, 1.5, -0.0, 2.0 ** -16, 2.0 ** -17, 3 * 2.0 ** -17, 5 * 2.0 ** -18])
    zeros = torch.zeros((T, d), dtype=torch.float32, device=dev)
    o = torch.randn((T, d), device=dev)
    lse = torch.zeros((T,), device=dev)
    q16 = tdw._lib.q16_partial(T, d, dev)
    x = torch.empty((T, d), device=dev)
    # p = pin + 0, stored as Q16 (fp32 rows: the partial's format is independent of them)
    tdw.attnres_phase2_merge(o, lse, pin, zeros, q16, torch.zeros(d, device=dev), None, None, 1e-6, None, x)
    back = torch.empty((T, d), device=dev)
    tdw.attnres_block_accumulate(q16, zeros, back)  # Q16 -> fp32 + 0
    torch.cuda.synchronize()
    got, want = back.cpu().numpy().astype(np.float64), _q16_emulate(pin.cpu().numpy())
    bad = np.argwhere(got != want)
    assert bad.size == 0, "Q16 mismatch at %s: got %r want %r (input %r)" % (
        bad[:4].tolist(), got[tuple(bad[0])], want[tuple(bad[0])], pin.cpu().numpy()[tuple(bad[0])])
    assert np.all(got[0] == 0.0) and got[2, 7] == 32767 * 2.0 ** -15
    # every element within 2^-15 of its row's largest magnitude
    ref = pin.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-300)
    assert err.max() <= 2.0 ** -15
    # the Python-side decoder reads the same values
    np.testing.assert_array_equal(tdw._lib.q16_decode(q16, T, d).cpu().numpy(), got.astype(np.float32))


# -------------------------------------------------- ragged and edge shapes
EDGE = [
    # (T, d, blocks, n_given, dtype)
    (1, 8, (3, 2), 0, "f32"),
    (17, 24, (1, 4), 1, "f32"),
    (33, 136, (2, 3, 5), 0, "bf16"),
    (40, 1032, (5, 1, 2), 2, "bf16"),
    (19, 7168, (3,), 7, "bf16"),
    (50, 256, (33,), 0, "bf16"),          # S > 32: two query tiles in one phase-1 call
    (16, 64, (17, 2), 0, "f32"),           # S = 17: second query tile of 16 partly used
    (23, 512, (1,) * 15, 0, "bf16"),      # 16 completed sources at the last blocks
    (31, 16384, (4,), 0, "bf16"),          # widest supported row
    (9, 4104, (2, 1), 1, "f32"),           # fp32 final site over 513 chunks: workgroup per token, 2 chunks a thread
    (6, 8200, (2,), 2, "f32"),             # fp32 final site over 1025 chunks: 4 chunks a thread
    (300, 2048, (3, 3), 0, "bf16"),        # final site over 256 chunks: the widest wave-per-token row
    (5, 8, (2,) + (1,) * 18, 0, "f32"),    # one-query blocks past 16 sources: first merge in phase 2
    (37, 1032, (1,) * 20, 1, "bf16"),
]


@pytest.mark.parametrize("T,d,blocks,n_given,dt", EDGE)
def test_block_edge_shapes(T, d, blocks, n_given, dt):
    base = synth.WORKLOADS["tiny_block_f32"]
    w = synth.scaled(base, name="edge", T=T, d=d, block_sizes=tuple(blocks), n_given=n_given, dtype=dt,
                     unit_gains=False, seed=4242 + T + d)
    _say("case edge T=%d d=%d blocks=%s given=%d %s" % (T, d, blocks, n_given, dt))
    worst = run_block_parity(w)
    _say("worst", worst)


@pytest.mark.parametrize("T,d,L,dt", [
    (5, 8, 3, "bf16"), (18, 200, 31, "bf16"), (64, 1024, 9, "bf16"),
    (33, 520, 12, "bf16"),    # 65 chunks: two chunks per lane, the second mostly past the row
    (29, 2048, 31, "bf16"),   # four chunks per lane, 32 sources: batches of two
    (21, 1544, 10, "f32"),    # fp32, four chunks per lane, batches of one
    (40, 1032, 7, "f32"),     # fp32, two chunks per lane, ragged last batch
    (17, 2056, 5, "bf16"),    # 257 chunks: the 512-thread one-pass kernel, one chunk per thread
    (23, 4096, 9, "bf16"),    # 512 chunks, the widest with one chunk per thread
    (19, 4096, 17, "f32"),    # the same in fp32, 17 sources
    (11, 4104, 6, "bf16"),    # 513 chunks: two chunks per thread
    (7, 16384, 3, "bf16"),    # 2048 chunks, the widest row: four chunks per thread
])
def test_full_edge_shapes(T, d, L, dt):
    """One-shot sites over the row widths and source counts of the site
    kernels (one pass with a wave per token for rows of <= 256 chunks, one
    pass with a 512-thread workgroup per token up to the 2048 chunks of the
    widest row)."""
    base = synth.WORKLOADS["full_bf16"]
    w = synth.scaled(base, name="full_edge", T=T, d=d, block_sizes=(1,) * L, seed=777 + L + d, dtype=dt)
    _say("case full_edge T=%d d=%d L=%d %s" % (T, d, L, dt))
    run_full_parity(w)


@pytest.mark.parametrize("T,d,L,group", [(4096, 1024, 16, 4), (5, 8, 3, 2), (18, 200, 19, 5), (64, 1024, 9, 4),
                                         (33, 7168, 6, 6), (40, 16384, 4, 3)])
def test_full_grouped_two_phase(T, d, L, group):
    """Grouped two-phase Full AttnRes (phase 1 per group + multi-source merge)
    against the oracle's one-shot sites."""
    base = synth.WORKLOADS["full_bf16"]
    w = base if (T, d, L) == (base.T, base.d, base.L) else synth.scaled(
        base, name="full_grouped", T=T, d=d, block_sizes=(1,) * L, seed=991 + L + d)
    _say("case full grouped T=%d d=%d L=%d group=%d" % (T, d, L, group))
    samples = synth.sample_tokens(w.T, 256) if w.T > 256 else None
    worst = run_full_parity(w, samples, group=group)
    _say("worst", worst)


def test_empty_token_set_is_a_noop():
    _say("case T=0")
    dev = torch.device("cuda")
    z = torch.empty((3, 0, 64), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((2, 64), dtype=torch.float32, device=dev)
    out = torch.empty((2, 0, 64), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((2, 0), dtype=torch.float32, device=dev)
    tdw.attnres_phase1(z, 3, w, None, 1e-6, out, None, lse)
    torch.cuda.synchronize()


# ------------------------------------------------------- special cases
def test_zero_query_gives_mean_and_identical_sources_give_source():
    _say("case special: zero query / identical sources")
    dev = torch.device("cuda")
    T, d, n = 37, 7168, 9
    src = (torch.randn((n, T, d), device=dev) * 3).to(torch.bfloat16)
    h = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T,), dtype=torch.float32, device=dev)
    tdw.attnres_full(src, n, torch.zeros(d, device=dev), None, None, 1e-6, h, None, lse)
    mean = src.double().mean(0)
    assert row_rel_err(_host(h), mean.cpu().numpy()).max() <= 1e-2
    assert np.allclose(lse.cpu().numpy(), math.log(n), rtol=1e-6)
    same = src[:1].expand(n, T, d).contiguous()
    tdw.attnres_full(same, n, torch.randn(d, device=dev), None, None, 1e-6, h, None, lse)
    assert torch.equal(h, same[0])


def test_phase1_single_query_equals_full():
    _say("case phase1(S=1) vs full")
    dev = torch.device("cuda")
    T, d, n = 50, 1024, 6
    src = (torch.randn((n, T, d), device=dev)).to(torch.bfloat16)
    wq = torch.randn((1, d), device=dev) * 0.02
    g = torch.rand((1, d), device=dev) * 0.4 + 0.8
    out = torch.empty((1, T, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, T), dtype=torch.float32, device=dev)
    tdw.attnres_phase1(src, n, wq, g, 1e-6, out, None, lse)
    h = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    lse2 = torch.empty((T,), dtype=torch.float32, device=dev)
    tdw.attnres_full(src, n, wq[0], g[0], None, 1e-6, h, None, lse2)
    assert torch.equal(out[0], h)
    assert torch.equal(lse[0], lse2)


@pytest.mark.parametrize("T,d,L", [(300, 1024, 8), (97, 7168, 5)])
def test_block_of_single_sublayers_equals_full_and_grouped(T, d, L):
    """GPU against GPU on the same inputs: Block AttnRes with every block one
    sublayer long has Full AttnRes's sources at every site (structured notes
    on arXiv 2603.15031, section 8: N = L recovers Full), and the grouped
    two-phase Full schedule computes the one-shot sites exactly up to
    rounding (section 7, two-phase computation).  Each GPU result is within
    the parity tolerance of the same exact values, so they are compared at it."""
    _say("case block N=L vs full vs grouped T=%d d=%d L=%d" % (T, d, L))
    dev = torch.device("cuda")
    base = synth.WORKLOADS["full_bf16"]
    w = synth.scaled(base, name="block_vs_full", T=T, d=d, block_sizes=(1,) * L, seed=4242 + d)
    scales = synth.sublayer_scales(w)
    prm = synth.params(w, dev)
    emb = synth.embedding(w, 0, T, dev)
    v = [synth.sublayer_output(w, l + 1, 0, T, dev, scales) for l in range(L)]
    idx = torch.arange(T, device=dev)

    def full(group):
        st = tdw.FullAttnRes(T, d, L, w.torch_dtype, eps=w.eps, device=dev, keep_h=True, group=group)
        st.hist[0].copy_(emb)
        for l in range(L):
            st.hist[l + 1].copy_(v[l])
        cap = Capture(idx)
        st.forward(prm, lambda l, x: None, hook=cap)
        return cap, st.h_final.clone()

    blk = tdw.BlockAttnRes(T, d, w.block_sizes, w.torch_dtype, eps=w.eps, device=dev, keep_h=True)
    blk.reps[0].copy_(emb)
    bcap = Capture(idx)
    blk.forward(prm, lambda l, x: v[l], hook=bcap)
    torch.cuda.synchronize()
    one, one_hf = full(None)
    grp, grp_hf = full(4 if L > 4 else 2)
    tol = TOL[w.dtype]
    for other, hf in ((bcap, blk.h_final), (grp, grp_hf)):
        for k in ("x", "h"):
            e = float(row_rel_err(other.stacked(k), one.stacked(k)).max())
            assert e <= tol, (k, e)
        assert float(row_rel_err(_host(hf), _host(one_hf)).max()) <= tol
    # Block's one-query sites and Full's one-shot sites compute the same
    # softmax: their statistics agree to fp32 rounding
    assert float(stat_err(bcap.stacked("lse1"), one.stacked("lse")).max()) <= 1e-4


def test_block_runs_are_bitwise_deterministic():
    w = synth.scaled(synth.WORKLOADS["prefill_chunk_bf16"], T=2048, name="det")
    _say("case determinism T=%d" % w.T)
    dev = torch.device("cuda")
    from harness import block_inputs
    emb, given, v = block_inputs(w, dev)
    prm = synth.params(w, dev)
    outs = []
    for _ in range(2):
        st = tdw.BlockAttnRes(w.T, w.d, w.block_sizes, w.torch_dtype, device=dev, x_ring=1, keep_h=False)
        st.reps[0].copy_(emb)
        xs = []
        st.forward(prm, lambda l, x: v[l], hook=lambda site, x, **k: xs.append(x[::97].clone()))
        torch.cuda.synchronize()
        outs.append((st.h_final.clone(), st.reps.clone(), torch.stack(xs)))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("T,d,cut", [(1000, 7168, 333), (9001, 1024, 4001), (5000, 7168, 1000)])
def test_token_split_invariance(T, d, cut):
    """Tokens never interact: one call over T tokens equals calls over slices,
    every sublayer input and the final output bit for bit.  At 9001 tokens
    (64-thread teams, d = 1024) and 5000 tokens (256-thread teams, d = 7168)
    the whole range takes the merge's persistent loop and the slices its
    one-token-per-team path (4001 and 5000 tokens leave teams without a
    token in the last workgroup); at 5000 tokens the whole range also forms
    the first sublayer's input inside phase 1's token-order output kernel,
    the slices in the short-range kernels."""
    _say("case token split invariance T=%d d=%d" % (T, d))
    dev = torch.device("cuda")
    w = synth.scaled(synth.WORKLOADS["prefill_chunk_bf16"], T=T, d=d, block_sizes=(5, 7), name="split")
    from harness import block_inputs
    emb, given, v = block_inputs(w, dev)
    prm = synth.params(w, dev)

    def run(a, b):
        st = tdw.BlockAttnRes(b - a, w.d, w.block_sizes, w.torch_dtype, device=dev)
        st.reps[0].copy_(emb[a:b])
        xs = []
        st.forward(prm, lambda l, x: v[l][a:b].contiguous(), hook=lambda site, x, **k: xs.append(x.clone()))
        return st.h_final.clone(), xs

    whole, xw = run(0, T)
    for a, b in ((0, cut), (cut, T)):
        h, xs = run(a, b)
        assert torch.equal(h, whole[a:b]), (a, b)
        assert len(xs) == len(xw)
        for site, (x, y) in enumerate(zip(xs, xw)):
            assert torch.equal(x, y[a:b]), (a, b, site)


def test_token_permutation_equivariance():
    """Permuting the tokens permutes every output bitwise: no kernel lets a
    token's result depend on its position or neighbours (which wave, tile or
    workgroup computes it)."""
    _say("case token permutation")
    dev = torch.device("cuda")
    w = synth.scaled(synth.WORKLOADS["prefill_chunk_bf16"], T=777, block_sizes=(4, 3, 2), n_given=1,
                     name="perm")
    from harness import block_inputs
    emb, given, v = block_inputs(w, dev)
    prm = synth.params(w, dev)
    perm = torch.randperm(w.T, generator=torch.Generator().manual_seed(5)).to(dev)

    def run(e, gs, vs):
        st = tdw.BlockAttnRes(w.T, w.d, w.block_sizes, w.torch_dtype, n_given=1, keep_h=True, device=dev)
        st.reps[0].copy_(e)
        st.reps[1].copy_(gs[0])
        xs, hs = [], []

        def hook(site, **k):
            xs.append(k["x"].clone())
            hs.append(k["h"].clone())

        st.forward(prm, lambda l, x: vs[l], hook=hook)
        return st.h_final.clone(), st.reps.clone(), torch.stack(xs), torch.stack(hs)

    ref = run(emb, given, v)
    got = run(emb[perm].contiguous(), [gl[perm].contiguous() for gl in given], [vl[perm].contiguous() for vl in v])
    assert torch.equal(got[0], ref[0][perm])
    for a, b in zip(got[1:], ref[1:]):
        assert torch.equal(a, b[:, perm])


# ------------------------------------------------ decode step as a HIP graph
def test_decode_step_graph_replay_matches_eager():
    """The decode-shaped block step (T=256, one block of 24, 7 given block
    sums) captured once as a HIP graph: every replay, with eager work in
    between that overwrites all outputs, reproduces the eager pass bit for bit."""
    w = synth.WORKLOADS["decode_block_bf16"]
    _say("case decode step graph replay T=%d" % w.T)
    dev = torch.device("cuda")
    from harness import block_inputs
    emb, given, v = block_inputs(w, dev)
    prm = synth.params(w, dev)
    st = tdw.BlockAttnRes(w.T, w.d, w.block_sizes, w.torch_dtype, n_given=w.n_given, eps=w.eps, device=dev,
                          x_ring=w.L, final_site=w.final_site)
    st.reps[0].copy_(emb)
    for n, b in enumerate(given):
        st.reps[1 + n].copy_(b)
    sub = lambda l, x: v[l]  # noqa: E731
    st.forward(prm, sub)
    torch.cuda.synchronize()
    # outputs of the pass (the decode step has no final aggregation site)
    outs = lambda: [st.reps, st.x] + ([st.h_final] if w.final_site else [])  # noqa: E731
    ref = [t.clone() for t in outs()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.forward(prm, sub)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.forward(prm, sub)
    for k in range(3):
        st.h_final.fill_(float(k + 1))
        st.x.fill_(-1.0 - k)
        st.reps[1 + w.n_given:].fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("reps", "x", "h_final"), ref, outs()):
            if not torch.equal(a, b):
                bad = (a != b).nonzero()
                raise AssertionError("replay %d: %s differs at %d places, first %s: %r vs %r (max |diff| %.3e)"
                                     % (k, name, bad.shape[0], bad[0].tolist(), a[tuple(bad[0])].item(),
                                        b[tuple(bad[0])].item(), (a.float() - b.float()).abs().max().item()))


# ------------------------- phase 1 over long token ranges (wide-tile scoring)
WIDE = [
    # (dtype, d, n_src, S): ragged last K-block, single query, fp32, largest LDS use
    ("bf16", 7104, 8, 24),
    ("bf16", 7168, 9, 1),
    ("f32", 1032, 3, 20),
    ("bf16", 1024, 16, 32),
    # bf16 tiles take two scoring waves, each with a share of the sources: an
    # odd count (3 + 2, ragged K-blocks) and a single source (the second wave
    # only keeps the barriers)
    ("bf16", 2056, 5, 24),
    ("bf16", 1024, 1, 20),
]


@pytest.mark.parametrize("dt,d,n,S", WIDE)
def test_phase1_long_range_equals_slices_and_oracle(dt, d, n, S):
    """Phase 1 over a token range long enough for the wide scoring kernel (64
    tokens per workgroup, one workgroup per compute unit) gives, bit for bit,
    what calls over shorter slices (16-token tiles) give, also slices short
    enough for the softmax to run inside the output kernel and for the query
    tiles to be split over workgroups, and matches the oracle on sampled
    tokens."""
    dev = torch.device("cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    T = 64 * cus + 40                   # ragged last workgroup
    cut = 64 * cus // 2                 # both slices stay below 64 * cus tokens
    _say("case phase1 long range %s T=%d d=%d n=%d S=%d" % (dt, T, d, n, S))
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    g = torch.Generator(device=dev).manual_seed(9000 + d + n + S)
    src = torch.randn((n, T, d), generator=g, device=dev).to(tdt)
    w = torch.randn((S, d), generator=g, device=dev) * 0.02
    kg = torch.rand((S, d), generator=g, device=dev) * 0.4 + 0.8
    ws = torch.empty(tdw.attnres_phase1_workspace_bytes(T, d, n, S) // 4 + 4, device=dev)

    def call(t0, t1):
        out = torch.empty((S, t1 - t0, d), dtype=tdt, device=dev)
        m = torch.empty((S, t1 - t0), device=dev)
        lse = torch.empty((S, t1 - t0), device=dev)
        tdw.attnres_phase1(src[:, t0:t1], n, w, kg, 1e-6, out, m, lse, workspace=ws)
        return out, m, lse

    whole = call(0, T)
    parts = [call(0, cut), call(cut, T)]
    torch.cuda.synchronize()
    for k in range(3):
        assert torch.equal(whole[k], torch.cat([parts[0][k], parts[1][k]], dim=-2 if k == 0 else -1)), k
    for t0, t1 in ((0, 300), (T - 1000, T)):
        short = call(t0, t1)
        for k in range(3):
            assert torch.equal(short[k], whole[k][:, t0:t1]), (t0, t1, k)
    tol = TOL[dt]
    for t in synth.sample_tokens(T, 6):
        rows = [src[i, t].double().cpu().numpy() for i in range(n)]
        for q in (0, S - 1):
            # the oracle's partition statistics: max m, sum ell of e^{z - m}, and
            # the unnormalised sum o of e^{z_i - m} u_i
            m_ref, ell, o_ref = oracle.partition_stats(rows, w[q].cpu().numpy(), kg[q].cpu().numpy(), 1e-6)
            assert stat_err(np.array([whole[1][q, t].item()]), np.array([m_ref])).max() <= tol
            assert stat_err(np.array([whole[2][q, t].item()]), np.array([m_ref + math.log(ell)])).max() <= tol
            assert row_rel_err(_host(whole[0][q, t]), o_ref / ell) <= tol


# ------------------- phase 1 with the first sublayer's PreNorm in the same pass
FIRST = [
    # (T, d, n, S, dtype, h_out): T None = long enough for the token-order kernel
    (None, 7168, 8, 24, "bf16", False),
    (None, 1032, 3, 5, "bf16", True),      # ragged last chunk group
    (None, 13312, 2, 3, "bf16", False),    # widest row whose copy fits in LDS
    (None, 16384, 2, 2, "bf16", True),     # wider: phase 1 + a separate PreNorm launch
    (None, 4096, 4, 3, "f32", True),
    (None, 8192, 1, 4, "f32", False),      # one source: out may be NULL
    (None, 7168, 1, 24, "bf16", True),     # one source, the 16K chunk's first block (PreNorm-only merge launch)
    (37, 1032, 3, 4, "bf16", True),        # short range: item-order kernel + PreNorm launch
    (37, 64, 1, 3, "f32", True),           # short range, one source
    # short ranges, rows over 256 chunks: a workgroup per token with the PreNorm inside
    (37, 7168, 8, 24, "bf16", True),       # the decode step's shape
    (300, 4104, 3, 20, "bf16", False),     # ragged last chunk group (9 groups, the last of one chunk)
    (37, 2056, 4, 5, "f32", True),         # 257 chunks: 5 groups
    (200, 7168, 16, 24, "bf16", False),    # 16 sources
    (1500, 4104, 3, 20, "bf16", False),    # more tokens than workgroups: two tokens on some
]


@pytest.mark.parametrize("T,d,n,S,dt,with_h", FIRST)
def test_phase1_first_prenorm(T, d, n, S, dt, with_h):
    """attnres_phase1_first_prenorm gives the statistics and queries 1..S-1
    of attnres_phase1 bit for bit, h = o_0 bit for bit, and x bit for bit as
    the two-launch path (phase 1, then the first sublayer's merge: the fused
    PreNorm sums the squares in the merge's order); x matches the oracle on
    sampled tokens."""
    dev = torch.device("cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    T = 32 * cus + 40 if T is None else T
    _say("case phase1 first prenorm %s T=%d d=%d n=%d S=%d h=%s" % (dt, T, d, n, S, with_h))
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    g = torch.Generator(device=dev).manual_seed(5100 + d + n + S)
    scale = torch.exp(torch.rand((n, 1, 1), generator=g, device=dev) * 2.0)
    src = (torch.randn((n, T, d), generator=g, device=dev) * scale).to(tdt)
    w = torch.randn((S, d), generator=g, device=dev) * 0.02
    kg = torch.rand((S, d), generator=g, device=dev) * 0.4 + 0.8
    gamma = torch.rand((d,), generator=g, device=dev) * 0.4 + 0.8
    ws = torch.empty(tdw.attnres_phase1_workspace_bytes(T, d, n, S) // 4 + 4, device=dev)
    eps = 1e-6
    outA = torch.empty((S, T, d), dtype=tdt, device=dev)
    mA, lseA = torch.empty((S, T), device=dev), torch.empty((S, T), device=dev)
    hA, xA = torch.empty((T, d), dtype=tdt, device=dev), torch.empty((T, d), dtype=tdt, device=dev)
    tdw.attnres_phase1(src, n, w, kg, eps, outA, mA, lseA, workspace=ws)
    tdw.attnres_phase2_merge(outA[0], lseA[0], None, None, None, w[0], kg[0], gamma, eps, hA, xA)
    outB = None if n == 1 else torch.zeros((S, T, d), dtype=tdt, device=dev)
    mB, lseB = torch.empty((S, T), device=dev), torch.empty((S, T), device=dev)
    xB = torch.empty((T, d), dtype=tdt, device=dev)
    hB = torch.empty((T, d), dtype=tdt, device=dev) if with_h else None
    tdw.attnres_phase1_first_prenorm(src, n, w, kg, eps, outB, mB, lseB, gamma, xB, hB, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(mA, mB) and torch.equal(lseA, lseB)
    if outB is not None:
        assert torch.equal(outA[1:], outB[1:])
    if with_h:
        assert torch.equal(hB, outA[0])
    if not torch.equal(xA, xB):
        diff = (xA.float() - xB.float()).abs()
        raise AssertionError("x differs at %d places (max |diff| %.3e)" % (int((diff > 0).sum()), diff.max().item()))
    tol = TOL[dt]
    for t in synth.sample_tokens(T, 8):
        rows = [src[i, t].double().cpu().numpy() for i in range(n)]
        h = oracle.depth_softmax(rows, w[0].cpu().numpy(), kg[0].cpu().numpy(), eps)["h"]
        x = oracle.rmsnorm(h, gamma.cpu().numpy(), eps)
        assert row_rel_err(_host(xB[t]), x) <= tol, t


# ------------------------------------------------ backward of one site
BWD = [
    # (T, d, n, prenorm, dtype, query scale)
    (300, 1024, 5, True, "bf16", 0.02),
    (97, 7168, 9, True, "bf16", 0.02),
    (64, 7168, 9, False, "bf16", 0.2),      # peaked softmax
    (64, 256, 3, False, "f32", 0.1),
    (33, 136, 16, True, "f32", 0.05),       # most sources, ragged d
    (5, 8, 1, True, "f32", 1.0),            # one source: no score gradient
    (40, 16384, 2, True, "bf16", 0.02),     # widest row
    (2100, 2048, 4, True, "bf16", 0.02),    # many tokens per team
    (50, 1024, 17, True, "bf16", 0.02),     # more than 16 sources: rows re-read per pass
    (33, 7168, 32, True, "bf16", 0.02),     # the most sources
    (20, 16384, 24, False, "bf16", 0.02),   # widest row, many sources
    (40, 256, 25, True, "f32", 0.05),
]


@pytest.mark.parametrize("T,d,n,prenorm,dt,qs", BWD)
def test_site_backward_matches_oracle(T, d, n, prenorm, dt, qs):
    """dL/du_i, dL/dw, dL/dg and dL/dgamma of one aggregation site against
    the oracle's fp64 backward (itself pinned to finite differences)."""
    _say("case site backward T=%d d=%d n=%d prenorm=%s %s" % (T, d, n, prenorm, dt))
    dev = torch.device("cuda")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    g = torch.Generator(device=dev).manual_seed(5000 + T + d + n)
    scales = torch.exp(torch.rand((n, 1, 1), generator=g, device=dev) * 2.0)
    src = (torch.randn((n, T, d), generator=g, device=dev) * scales).to(tdt)
    w = torch.randn((d,), generator=g, device=dev) * qs
    kg = torch.rand((d,), generator=g, device=dev) * 0.4 + 0.8
    gm = torch.rand((d,), generator=g, device=dev) * 0.4 + 0.8
    dx = torch.randn((T, d), generator=g, device=dev).to(tdt)
    dsrc = torch.empty_like(src)
    dw = torch.empty((d,), device=dev)
    dkg = torch.empty((d,), device=dev)
    dgm = torch.empty((d,), device=dev)
    ws = torch.empty(tdw.attnres_site_backward_workspace_bytes(T, d) // 4 + 4, device=dev)
    tdw.attnres_site_backward(src, n, w, kg, gm if prenorm else None, prenorm, 1e-6, dx, dsrc, dw, dkg,
                              dgm if prenorm else None, ws)
    torch.cuda.synchronize()
    ref = oracle.site_backward(src, w, kg, gm if prenorm else None, 1e-6, dx, prenorm=prenorm)
    tol = TOL[dt]
    err = row_rel_err(_host(dsrc).reshape(n * T, d), ref["du"].reshape(n * T, d)).max()
    _say("worst du %.3e" % err)
    assert err <= tol
    for name, got in (("dw", dw), ("dg", dkg)) + ((("dgamma", dgm),) if prenorm else ()):
        e = float(row_rel_err(_host(got), ref[name if name != "dg" else "dg"]))
        _say("worst %s %.3e" % (name, e))
        assert e <= tol, name
    # a second run gives the same bits (fixed-order reductions, no atomics)
    d2 = torch.empty_like(dsrc)
    dw2 = torch.empty_like(dw)
    tdw.attnres_site_backward(src, n, w, kg, gm if prenorm else None, prenorm, 1e-6, dx, d2, dw2, None, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(d2, dsrc) and torch.equal(dw2, dw)


@pytest.mark.parametrize("T,d,n,prenorm,dt,qs", [BWD[1], BWD[3], BWD[8], BWD[9], BWD[11]])
def test_site_backward_accumulate_adds_the_gradient(T, d, n, prenorm, dt, qs):
    """attnres_site_backward_accumulate adds dL/du_i to fp32 rows already
    holding other contributions; the increment matches the oracle's
    backward, and dw/dg/dgamma equal the storing entry point's bit for bit."""
    _say("case site backward accumulate T=%d d=%d n=%d %s" % (T, d, n, dt))
    dev = torch.device("cuda")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    g = torch.Generator(device=dev).manual_seed(6000 + T + d + n)
    scales = torch.exp(torch.rand((n, 1, 1), generator=g, device=dev) * 2.0)
    src = (torch.randn((n, T, d), generator=g, device=dev) * scales).to(tdt)
    w = torch.randn((d,), generator=g, device=dev) * qs
    kg = torch.rand((d,), generator=g, device=dev) * 0.4 + 0.8
    gm = torch.rand((d,), generator=g, device=dev) * 0.4 + 0.8
    dx = torch.randn((T, d), generator=g, device=dev).to(tdt)
    ws = torch.empty(tdw.attnres_site_backward_workspace_bytes(T, d) // 4 + 4, device=dev)
    ref = oracle.site_backward(src, w, kg, gm if prenorm else None, 1e-6, dx, prenorm=prenorm)
    # other contributions of each row's own size (an offset far above a row
    # would round its increment away in fp32)
    row_max = torch.from_numpy(np.abs(ref["du"]).max(axis=-1, keepdims=True)).float().to(dev)
    start = torch.randn((n, T, d), generator=g, device=dev) * row_max
    acc = start.clone()
    dw, dkg, dgm = (torch.empty((d,), device=dev) for _ in range(3))
    tdw.attnres_site_backward_accumulate(src, n, w, kg, gm if prenorm else None, prenorm, 1e-6, dx, acc, dw, dkg,
                                         dgm if prenorm else None, ws)
    dsrc = torch.empty_like(src)
    dw2, dkg2, dgm2 = (torch.empty((d,), device=dev) for _ in range(3))
    tdw.attnres_site_backward(src, n, w, kg, gm if prenorm else None, prenorm, 1e-6, dx, dsrc, dw2, dkg2,
                              dgm2 if prenorm else None, ws)
    torch.cuda.synchronize()
    inc = _host(acc) - _host(start)
    err = row_rel_err(inc.reshape(n * T, d), ref["du"].reshape(n * T, d)).max()
    _say("worst du increment %.3e" % err)
    assert err <= TOL[dt]
    assert torch.equal(dw, dw2) and torch.equal(dkg, dkg2)
    if prenorm:
        assert torch.equal(dgm, dgm2)
    # the increment is the storing entry point's gradient before its rounding
    assert (acc - start - dsrc.float()).abs().max().item() <= \
        (2.0 ** -8 if dt == "bf16" else 1e-5) * dsrc.float().abs().max().item()


FULL_BWD = [
    # (T, d, L, dtype, group used by the forward)
    (64, 256, 4, "f32", None),
    (256, 1024, 16, "bf16", None),     # the Full workload's depth and width: 17 sources at the final site
    (256, 1024, 16, "bf16", 4),        # same, forward on the grouped two-phase schedule
    (33, 7168, 6, "bf16", None),
    (24, 520, 31, "bf16", None),       # 32 sources at the final site, ragged width
]


@pytest.mark.parametrize("T,d,L,dt,group", FULL_BWD)
def test_full_backward_matches_oracle(T, d, L, dt, group):
    """Full AttnRes backward (site backward passes accumulating in fp32) on
    the GPU against the oracle's backward of Block AttnRes with one sublayer
    per block, which is Full AttnRes (structured notes on arXiv 2603.15031,
    section 8): dL/dv_l of every sublayer, dL/db_0, dw, dg, dgamma."""
    _full_backward_case(T, d, L, dt, group)


def test_full_backward_unit_gains_without_final_site():
    """The same without the final aggregation and with the gains left out
    (None: ones) on the GPU side."""
    _full_backward_case(50, 256, 5, "bf16", None, final_site=False, gains=False)


def _full_backward_case(T, d, L, dt, group, final_site=True, gains=True):
    _say("case full backward T=%d d=%d L=%d %s group=%s final=%s gains=%s" % (T, d, L, dt, group, final_site,
                                                                              gains))
    dev = torch.device("cuda")
    base = synth.WORKLOADS["full_bf16"]
    w = synth.scaled(base, name="full_bwd", T=T, d=d, block_sizes=(1,) * L, seed=8100 + L + d, dtype=dt,
                     final_site=final_site, unit_gains=not gains)
    scales = synth.sublayer_scales(w)
    prm = synth.params(w, dev)
    gpu_prm = prm if gains else {"w": prm["w"], "g": None, "gamma": None}
    emb = synth.embedding(w, 0, T, dev)
    v = [synth.sublayer_output(w, l + 1, 0, T, dev, scales) for l in range(L)]
    st = tdw.FullAttnRes(T, d, L, w.torch_dtype, eps=w.eps, device=dev, group=group, final_site=final_site)
    st.hist[0].copy_(emb)
    for l in range(L):
        st.hist[l + 1].copy_(v[l])
    st.forward(gpu_prm, lambda l, x: None)
    gen = torch.Generator(device=dev).manual_seed(8200 + T + d)
    dx = [torch.randn((T, d), generator=gen, device=dev).to(w.torch_dtype) for _ in range(L)]
    dhf = torch.randn((T, d), generator=gen, device=dev).to(w.torch_dtype)
    dv = [None] * L

    def dx_for(l, g_v):
        dv[l] = g_v.clone()
        return dx[l]

    out = st.backward(gpu_prm, dx_for, dh_final=dhf if final_site else None)
    torch.cuda.synchronize()
    ref = oracle.block_backward(emb, torch.stack(v), prm["w"], prm["g"], prm["gamma"], w.block_sizes, w.eps,
                                torch.stack(dx), dhf if final_site else None, final_site=final_site)
    gpu = {"dv": _host(torch.stack(dv)), "demb": _host(out["demb"]), "dw": _host(out["dw"]),
           "dg": _host(out["dg"]), "dgamma": _host(out["dgamma"])}
    tol = TOL[dt]
    if not gains:  # no key gains: their gradient is not computed (stays zero)
        assert not gpu.pop("dg").any()
    for k, x in gpu.items():
        e = float(row_rel_err(x, ref[k]).max())
        _say("worst %s %.3e" % (k, e))
        assert e <= tol, (k, e)
    # a second backward gives the same bits (fixed-order reductions, no atomics)
    dv2 = [None] * L

    def dx_for2(l, g_v):
        dv2[l] = g_v.clone()
        return dx[l]

    out2 = st.backward(gpu_prm, dx_for2, dh_final=dhf if final_site else None)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(dv2, dv))
    for k in ("demb", "dw", "dg", "dgamma"):
        assert torch.equal(out2[k], out[k]), k


# --------------------------------------------- long context, chunked prefill
def _long_prefill(w, chunked: bool, samples, dev):
    """Run the whole depth over T tokens, streamed in 16K chunks or in one
    pass; sublayer outputs are produced on the fly for the tokens at hand
    (as a model's sublayers would), never for the whole context at once."""
    from harness import Capture
    scales = synth.sublayer_scales(w)
    prm = synth.params(w, dev)
    h_final = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=dev)
    caps = {}

    def fill(c0, c1, dst):
        dst.copy_(synth.embedding(w, c0, c1, dev))

    def sub_for(c0, c1):
        return lambda l, x: synth.sublayer_output(w, l + 1, c0, c1, dev, scales)

    def hook_for(c0, c1):
        local = [t - c0 for t in samples if c0 <= t < c1]
        if not local:
            return None
        cap = Capture(torch.tensor(local, dtype=torch.long, device=dev))
        caps[c0] = (local, cap)
        return cap

    def on_chunk(c0, c1, st):
        h_final[c0:c1].copy_(st.h_final)

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    tdw.prefill_chunked(w.T, w.chunk if chunked else w.T, w.d, w.block_sizes, w.torch_dtype, prm, fill, sub_for,
                        on_chunk=on_chunk, eps=w.eps, hook_for_chunk=hook_for)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    xs = {}
    for c0, (local, cap) in caps.items():
        x = torch.stack(cap.rows["x"])  # [L, k, d]
        for j, t in enumerate(local):
            xs[c0 + t] = x[:, j].clone()
    return h_final, xs, peak


def test_long_prefill_ragged_last_chunk():
    """A context that is not a whole number of chunks: the last, shorter
    chunk gets buffers of its own size after the full-size ones are released,
    so the peak stays that of whole chunks, and the output still equals the
    unchunked pass bit for bit."""
    base = synth.WORKLOADS["long_prefill_bf16"]
    dev = torch.device("cuda")
    w = synth.scaled(base, name="ragged_prefill", T=3 * 4096 + 1000, d=1024, chunk=4096, block_sizes=(4, 4, 3))
    whole = synth.scaled(w, T=3 * 4096)
    samples = synth.sample_tokens(w.T, 8)
    _say("case long_prefill ragged T=%d chunk=%d" % (w.T, w.chunk))
    hc, xc, peak_ragged = _long_prefill(w, True, samples, dev)
    hu, xu, _ = _long_prefill(w, False, samples, dev)
    _, _, peak_whole = _long_prefill(whole, True, synth.sample_tokens(whole.T, 8), dev)
    _say("peak: ragged %.3f GB, whole chunks %.3f GB" % (peak_ragged / 1e9, peak_whole / 1e9))
    assert torch.equal(hc, hu)
    for t in samples:
        assert torch.equal(xc[t], xu[t]), t
    assert peak_ragged <= peak_whole * 1.02


def test_long_prefill_chunked_equals_unchunked_and_oracle():
    w = synth.WORKLOADS["long_prefill_bf16"]
    dev = torch.device("cuda")
    samples = synth.sample_tokens(w.T, 24)
    _say("case long_prefill T=%d chunk=%d chunked pass" % (w.T, w.chunk))
    hc, xc, peak_c = _long_prefill(w, True, samples, dev)
    _say("case long_prefill unchunked pass")
    hu, xu, peak_u = _long_prefill(w, False, samples, dev)
    _say("peak AttnRes device memory: chunked %.2f GB, unchunked %.2f GB" % (peak_c / 1e9, peak_u / 1e9))
    # tokens never interact, so the chunking cannot change any bit
    assert torch.equal(hc, hu)
    for t in samples:
        assert torch.equal(xc[t], xu[t]), t
    assert peak_c * 4 < peak_u
    # oracle on the sampled tokens, from the generated inputs
    idx = torch.tensor(samples, dtype=torch.long, device=dev)
    scales = synth.sublayer_scales(w)
    emb = torch.cat([synth.embedding(w, t, t + 1, dev) for t in samples])
    v = torch.stack([torch.cat([synth.sublayer_output(w, l + 1, t, t + 1, dev, scales) for t in samples])
                     for l in range(w.L)])
    prm = synth.params(w, dev)
    o = oracle.block_forward(emb, v, prm["w"], prm["g"], prm["gamma"], w.block_sizes, w.eps,
                             want=("x", "hfinal"))
    gx = torch.stack([xc[t] for t in samples], dim=1)  # [L, k, d]
    ex = row_rel_err(_host(gx), o["x"]).max()
    eh = row_rel_err(_host(hc.index_select(0, idx)), o["hfinal"]).max()
    _say("worst x %.3e hfinal %.3e" % (ex, eh))
    assert ex <= TOL["bf16"] and eh <= TOL["bf16"]
