"""The allocation-free phase 1 (attnres_phase1_noalloc, through the C ABI):
the same results as attnres_phase1 with a caller workspace, on two calls in a
row (the second smaller, so it runs over what the first left in the
library's scratch), for bf16 and fp32 rows; a call needing more than the
scratch holds is refused before any launch (needs an MI355X)."""
import sys

import pytest
import torch

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


def _inputs(T, d, n, S, dtype, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    scale = torch.exp(torch.rand((n, 1, 1), generator=g, device="cuda") * 2.0)
    src = (torch.randn((n, T, d), generator=g, device="cuda") * scale).to(dtype)
    w = torch.randn((S, d), generator=g, device="cuda") * 0.02
    kg = torch.rand((S, d), generator=g, device="cuda") * 0.4 + 0.8
    return src, w, kg


def _run(T, d, n, S, dtype, seed):
    src, w, kg = _inputs(T, d, n, S, dtype, seed)
    outs = []
    for fn in ("ref", "noalloc"):
        out = torch.empty((S, T, d), dtype=dtype, device="cuda")
        m = torch.empty((S, T), device="cuda")
        lse = torch.empty((S, T), device="cuda")
        if fn == "ref":
            ws = torch.empty((tdw.attnres_phase1_workspace_bytes(T, d, n, S) + 15) // 4, device="cuda")
            tdw.attnres_phase1(src, n, w, kg, 1e-6, out, m, lse, ws)
        else:
            torch.cuda.synchronize()
            before = torch.cuda.memory_allocated()
            tdw.attnres_phase1_noalloc(src, n, w, kg, 1e-6, out, m, lse)
            torch.cuda.synchronize()
            assert torch.cuda.memory_allocated() == before
        outs.append((out, m, lse))
    (o0, m0, l0), (o1, m1, l1) = outs
    diff = (o0.float() - o1.float()).abs().max().item()
    _say("  T=%d d=%d n=%d S=%d %s: max |out diff| %.3e" % (T, d, n, S, dtype, diff))
    # the same kernels on the same inputs: bit for bit
    assert torch.equal(o0, o1) and torch.equal(m0, m1) and torch.equal(l0, l1)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_equals_phase1_two_calls(dtype):
    _say("case noalloc two calls %s" % dtype)
    # a one-rank share of the 16K chunk's last block, then a smaller ragged call
    _run(2048, 7168, 8, 24, dtype, 11)
    _run(300, 1032, 3, 5, dtype, 12)


def test_noalloc_one_query_and_many_queries():
    _say("case noalloc S=1 with 20 sources; S=40 (two groups of queries)")
    _run(257, 2048, 20, 1, torch.bfloat16, 13)
    _run(129, 512, 4, 40, torch.bfloat16, 14)


def test_noalloc_refuses_more_than_its_scratch():
    _say("case noalloc beyond its scratch")
    T, d, n, S = 200000, 256, 16, 32
    assert tdw.attnres_phase1_workspace_bytes(T, d, n, S) > _lib.ATTNRES_NOALLOC_SCRATCH_BYTES
    src = torch.empty((n, T, d), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((S, d), device="cuda")
    lse = torch.empty((S, T), device="cuda")
    with pytest.raises(tdw.AttnResError) as e:
        tdw.attnres_phase1_noalloc(src, n, w, None, 1e-6, None, None, lse)
    assert e.value.code == 6
