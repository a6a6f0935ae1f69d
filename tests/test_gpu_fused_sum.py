"""The block sum formed inside the next phase-1 call (attnres_phase1_accumulate)
against summing first (attnres_block_accumulate) and running phase 1 on the
result: the written block sum, the outputs, the statistics and the first
sublayer's PreNorm output must agree bit for bit, whether the library sums
inside the scoring pass (long token ranges, Q16 or fp32 partial) or runs the
block-sum kernel first.  The unfused path itself is checked against the oracle
elsewhere; the driver runs the fused form by default, so every Block AttnRes
parity test covers it too (needs an MI355X)."""
import sys

import pytest
import torch

import synth
from harness import Capture, block_inputs
import transformer_depth_wise_amd as tdw
from transformer_depth_wise_amd import _lib

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


def _partial(fmt, T, d, gen, dev):
    """A running partial in format fmt holding arbitrary valid contents."""
    if fmt is None:
        return None
    if fmt == "q16":
        buf = _lib.q16_partial(T, d, dev)
        buf[:T * d] = torch.randint(-32767, 32768, (T * d,), generator=gen, device=dev, dtype=torch.int32).to(torch.int16)
        buf[T * d:].view(torch.int32).copy_(torch.randint(-2, 5, (T,), generator=gen, device=dev, dtype=torch.int32))
        return buf
    if fmt == "p24":
        buf = _lib.p24_partial(T, d, dev)
        hi = (torch.randn((T * d,), generator=gen, device=dev) * 4).to(torch.bfloat16).view(torch.uint8)
        buf[:2 * T * d] = hi
        buf[2 * T * d:] = torch.randint(0, 256, (T * d,), generator=gen, device=dev, dtype=torch.int32).to(torch.uint8)
        return buf
    return torch.randn((T, d), generator=gen, device=dev) * 4


CASES = [
    # (T, d, n, S, partial, has_v2, dt (outputs), src_dt, pieces' dtype, prenorm)
    (16421, 1032, 5, 24, "q16", True, "bf16", "bf16", "bf16", True),   # wide path, ragged K-blocks and tiles
    (16421, 1032, 5, 24, "q16", True, "bf16", "bf16", "bf16", False),
    (16384, 256, 3, 7, "q16", False, "bf16", "bf16", "bf16", True),     # one query tile (S <= 16), no v2
    (16384, 512, 2, 24, "f32", True, "bf16", "bf16", "bf16", True),    # an fp32 partial, two sources
    (16384, 520, 4, 9, "q16", True, "bf16", "f32", "bf16", False),     # fp32 block sums (training), bf16 outputs
    (16384, 512, 3, 24, "q16", True, "f32", "f32", "bf16", False),     # fp32 sources and outputs, bf16 pieces
    (16384, 256, 4, 24, "f32", True, "f32", "f32", "f32", True),       # fp32 rows
    (16384, 256, 3, 5, "p24", True, "bf16", "bf16", "bf16", True),     # a 24-bit partial: block-sum kernel first
    (16384, 256, 3, 2, None, True, "bf16", "bf16", "bf16", True),      # no stored partial (blocks of 2)
    (300, 1032, 4, 24, "q16", True, "bf16", "bf16", "bf16", True),     # short range: block-sum kernel first
    (37, 7168, 3, 1, "q16", True, "bf16", "bf16", "bf16", False),      # one query without PreNorm: single pass
    (1000, 7168, 9, 1, "q16", True, "f32", "f32", "bf16", False),      # a training pass's final site
    (16384, 7168, 8, 18, "q16", True, "bf16", "bf16", "bf16", True),   # the 16K chunk's last block
    (16384, 256, 3, 40, "q16", True, "bf16", "bf16", "bf16", True),    # 40 queries: two query tiles
    (16384, 16384, 2, 3, "q16", True, "bf16", "bf16", "bf16", True),   # the widest rows
]
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.mark.parametrize("T,d,n,S,pfmt,has_v2,dt,sdt,vdt,prenorm", CASES)
def test_phase1_accumulate_equals_sum_then_phase1(T, d, n, S, pfmt, has_v2, dt, sdt, vdt, prenorm):
    _say("case phase1_accumulate T=%d d=%d n=%d S=%d partial=%s v2=%s out/src/pieces %s/%s/%s prenorm=%s"
         % (T, d, n, S, pfmt, has_v2, dt, sdt, vdt, prenorm))
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(9100 + T + d + n + S)
    odt, sdt_t, vdt_t = DT[dt], DT[sdt], DT[vdt]
    src = (torch.randn((n, T, d), generator=gen, device=dev) * 3).to(sdt_t)
    src[n - 1].fill_(float("nan"))  # overwritten by the call; never read
    v = (torch.randn((T, d), generator=gen, device=dev) * 2).to(vdt_t)
    v2 = (torch.randn((T, d), generator=gen, device=dev) * 2).to(vdt_t) if has_v2 else None
    pin = _partial(pfmt, T, d, gen, dev)
    w = torch.randn((S, d), generator=gen, device=dev) * 0.02
    kg = torch.rand((S, d), generator=gen, device=dev) * 0.4 + 0.8
    gm = torch.rand((d,), generator=gen, device=dev) * 0.4 + 0.8
    ws = torch.empty(((tdw.attnres_phase1_workspace_bytes(T, d, n, S) + 3) // 4 + 4,), device=dev)

    def outputs():
        return (torch.empty((S, T, d), dtype=odt, device=dev), torch.empty((S, T), device=dev),
                torch.empty((S, T), device=dev), torch.empty((T, d), dtype=odt, device=dev) if prenorm else None,
                torch.empty((T, d), dtype=odt, device=dev) if prenorm else None)

    # summing first, then phase 1
    ref = src.clone()
    tdw.attnres_block_accumulate(pin, v, ref[n - 1], v2=v2)
    o_r, m_r, l_r, x_r, h_r = outputs()
    if prenorm:
        tdw.attnres_phase1_first_prenorm(ref, n, w, kg, 1e-6, o_r, m_r, l_r, gm, x_r, h_r, workspace=ws)
    else:
        tdw.attnres_phase1(ref, n, w, kg, 1e-6, o_r, m_r, l_r, workspace=ws)
    # the fused call
    o_f, m_f, l_f, x_f, h_f = outputs()
    tdw.attnres_phase1_accumulate(src, n, w, kg, 1e-6, pin, v2, v, o_f, m_f, l_f,
                                  prenorm_gain=gm if prenorm else None, x_out=x_f, h_out=h_f, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(src[n - 1], ref[n - 1]), "block sum differs"
    assert torch.equal(src[:n - 1], ref[:n - 1]), "older sources changed"
    first = 1 if prenorm else 0  # slab 0 of out is scratch with the PreNorm
    assert torch.equal(o_f[first:], o_r[first:]), "phase-1 outputs differ"
    assert torch.equal(m_f, m_r) and torch.equal(l_f, l_r), "statistics differ"
    if prenorm:
        assert torch.equal(x_f, x_r) and torch.equal(h_f, h_r), "first sublayer's PreNorm output differs"


@pytest.mark.parametrize("training", [False, True])
def test_driver_fused_sums_equal_separate_launches(training):
    """The whole forward with block sums formed by the next phase-1 call (and
    the final site's) equals the one with a block-sum launch per block, bit for
    bit, at a long token range where the library sums inside the scoring pass."""
    base = synth.WORKLOADS["tiny_block_f32"]
    w = synth.scaled(base, name="fusedsum", T=16384, d=1024, block_sizes=(3, 4, 6, 1, 2, 5), n_given=0,
                     dtype="bf16", unit_gains=False, seed=9300, final_site=True)
    _say("case driver fuse_sum T=%d d=%d blocks=%s training=%s" % (w.T, w.d, w.block_sizes, training))
    dev = torch.device("cuda")
    emb, given, v = block_inputs(w, dev)
    prm = synth.params(w, dev)
    idx = torch.tensor(synth.sample_tokens(w.T, 64), device=dev)
    runs = []
    for fuse_sum in (True, False):
        st = tdw.BlockAttnRes(w.T, w.d, w.block_sizes, w.torch_dtype, eps=w.eps, device=dev, keep_h=True,
                              training=training, fuse_sum=fuse_sum)
        st.reps[0].copy_(emb)
        cap = Capture(idx)
        st.forward(prm, lambda l, x: v[l], hook=cap)
        torch.cuda.synchronize()
        runs.append((st.reps.clone(), st.h_final.clone(), st.lse_final.clone(),
                     torch.stack(cap.rows["x"]), torch.stack(cap.rows["h"])))
        del st
    for a, b, name in zip(runs[0], runs[1], ("reps", "h_final", "lse_final", "x", "h")):
        assert torch.equal(a, b), name
