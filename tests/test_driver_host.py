"""Host logic of the driver, on the CPU (no kernel is launched): launch plans
and their algorithmic bytes, the source-count limits, and argument checks
that fire before any launch.  The driver objects are built on the CPU device;
only the library's host functions (workspace sizes) are called."""
import pytest
import torch

import transformer_depth_wise_amd as tdw
from transformer_depth_wise_amd import _lib

BF, F32 = torch.bfloat16, torch.float32
K3 = (24,) * 7 + (18,)   # the 16K prefill chunk's depth layout


def rows_per_token_sublayer(plan, T, d, L, esize=2):
    return sum(x.bytes for x in plan) / (T * L * d * esize)


def test_block_plan_bytes_per_token_sublayer():
    # the forward at the prefill chunk's shape moves 5.953 rows of d per token
    # and sublayer with the Q16 partial (2 bytes per element plus a 4-byte row
    # exponent), 6.638 with the 24-bit one (every term is proportional to T;
    # the per-token statistics and exponents make the ratio depend slightly on
    # d); phase 1 writes S outputs per block except the first block's (its
    # only source is b_0)
    st = tdw.BlockAttnRes(16, 7168, K3, BF, device="cpu")
    assert st.partial_format == "q16"
    plan = st.plan()
    assert abs(rows_per_token_sublayer(plan, 16, 7168, 186) - 5.953) < 5e-4
    p24 = tdw.BlockAttnRes(16, 7168, K3, BF, device="cpu", partial="p24")
    assert abs(rows_per_token_sublayer(p24.plan(), 16, 7168, 186) - 6.638) < 5e-4
    kinds = [x.kind for x in plan]
    # every block's sum is formed by the next phase-1 call, the last one by the final site's
    assert kinds.count("phase1") == 8 and kinds.count("accumulate") == 0 and kinds.count("final") == 1
    assert kinds.count("phase2") == 186 - 8     # the first sublayer of each block leaves phase 1
    twice = tdw.BlockAttnRes(32, 7168, K3, BF, device="cpu").plan()
    assert sum(x.bytes for x in twice) == 2 * sum(x.bytes for x in plan)
    # the same bytes with a block-sum launch per block; without a final site
    # the last block's sum still needs one
    sep = tdw.BlockAttnRes(16, 7168, K3, BF, device="cpu", fuse_sum=False).plan()
    assert [x.kind for x in sep].count("accumulate") == 8
    assert sum(x.bytes for x in sep) == sum(x.bytes for x in plan)
    nofinal = [x.kind for x in tdw.BlockAttnRes(16, 7168, K3, BF, device="cpu", final_site=False).plan()]
    assert nofinal.count("accumulate") == 1 and nofinal[-1] == "accumulate" and "final" not in nofinal


def test_block_plan_survey_rows():
    # the plain row model of the scope table: 1146 rows per token at the 16K
    # chunk's layout (36 phase-1 reads + 186 phase-1 writes + 890 phase-2 +
    # 24 block sums + 10 final), 874 of them in the 178 merge launches
    T, d = 16, 7168
    st = tdw.BlockAttnRes(T, d, K3, BF, device="cpu")
    sv = st.plan_survey()
    r = T * d * 2
    assert sum(x.bytes for x in sv) == 1146 * r
    assert sum(x.bytes for x in sv if x.kind == "phase2") == 874 * r
    assert [x.kind for x in sv] == [x.kind for x in st.plan()]   # the same launches
    sep = tdw.BlockAttnRes(T, d, K3, BF, device="cpu", fuse_sum=False)
    assert [x.kind for x in sep.plan_survey()] == [x.kind for x in sep.plan()]
    assert sum(x.bytes for x in sep.plan_survey()) == 1146 * r
    unfused = tdw.BlockAttnRes(T, d, K3, BF, device="cpu", fuse_first=False).plan_survey()
    assert sum(x.bytes for x in unfused) == 1146 * r
    assert sum(x.bytes for x in unfused if x.kind == "phase2") == 890 * r


def test_block_plan_backward_bytes():
    # the 16K chunk's backward moves 501649047552 bytes with the Q16 partial
    # (every term is proportional to T): 16 tokens of it move 1/1024 of
    # that.  With the 24-bit partial: one byte more per element for each of
    # the 162 partial reads of the phase-2 backward (21 per block of 24, 15
    # for the block of 18), less their row exponents.  The block
    # representations are fp32 in a bf16 training pass: 46 rows per token
    # more than bf16 ones would move (the final site's 9 representations and
    # dL/dh_final, and the 1 + 2 + ... + 8 block-source reads of phase 1)
    st = tdw.BlockAttnRes(16, 7168, K3, BF, device="cpu", training=True)
    assert st.reps.dtype == torch.float32 and st.h_final.dtype == torch.float32
    assert sum(x.bytes for x in st.plan_backward()) * 1024 == 501649047552
    p24 = tdw.BlockAttnRes(16, 7168, K3, BF, device="cpu", training=True, partial="p24")
    assert sum(x.bytes for x in p24.plan_backward()) * 1024 == 520663793664
    assert 520663793664 - 501649047552 == 162 * 16384 * (7168 - 4)
    assert 520663793664 - 509859266560 == 46 * 16384 * 7168 * 2
    inf = tdw.BlockAttnRes(16, 7168, K3, BF, device="cpu")
    assert inf.reps.dtype == BF and inf.h_final.dtype == BF


def test_block_source_limits():
    with pytest.raises(ValueError, match="at most 16 completed sources"):
        tdw.BlockAttnRes(4, 64, (1,) * 15 + (2,), BF, n_given=1, device="cpu")
    with pytest.raises(ValueError, match="too many sources"):
        tdw.BlockAttnRes(4, 64, (1,) * 32, BF, device="cpu")
    tdw.BlockAttnRes(4, 64, (1,) * 31, BF, device="cpu")            # 32 sources at the final site
    tdw.BlockAttnRes(4, 64, (1,) * 15 + (2,), BF, device="cpu")      # 16 completed sources for S = 2


def test_training_limits_checked_before_any_forward():
    # the backward's limits are checked when the training state is built,
    # not after a whole forward: a one-sublayer block with 17 completed
    # sources runs forward (one query, up to 32 sources) but not backward
    tdw.BlockAttnRes(4, 64, (1,) * 16, BF, device="cpu")
    with pytest.raises(ValueError, match="would read 17 completed sources"):
        tdw.BlockAttnRes(4, 64, (1,) * 17, BF, device="cpu", training=True)
    with pytest.raises(ValueError, match="at most 32 sublayers per block"):
        tdw.BlockAttnRes(4, 64, (33,), BF, device="cpu", training=True)
    tdw.BlockAttnRes(4, 64, (32,) + (1,) * 15, BF, device="cpu", training=True)   # 16 sources, 32 sites
    # the final site's one-query backward takes up to 32 sources
    assert _lib.attnres_phase1_backward_workspace_bytes(64, 256, 32, 1) == \
        _lib.attnres_site_backward_workspace_bytes(64, 256)
    assert _lib.attnres_phase1_backward_workspace_bytes(64, 256, 17, 2) == -1
    assert _lib.attnres_phase1_backward_workspace_bytes(64, 256, 33, 1) == -1


def test_full_plan_and_limits():
    T, d, L = 8, 64, 16
    f = tdw.FullAttnRes(T, d, L, BF, device="cpu")
    r, r32 = T * d * 2, T * d * 4
    assert sum(x.bytes for x in f.plan_backward()) == \
        sum((l + 1) * (r + 2 * r32) + r for l in range(L + 1))
    assert [x.kind for x in f.plan()].count("full") == L
    # one-shot sites: site l reads its l sources and writes x; the final site
    # reads the L + 1 representations and writes h_final.  At the Full
    # workload's depth (L = 16) that is 152 + 18 = 170 rows per token.
    rows = sum(x.bytes for x in f.plan() if x.kind in ("full", "final")) / r
    assert rows == sum(l + 1 for l in range(1, L + 1)) + (L + 2) + (L + 1) * 4 / (d * 2) and \
        int(rows) == 170
    kept = tdw.FullAttnRes(T, d, L, BF, device="cpu", keep_h=True)
    assert sum(x.bytes for x in kept.plan()) == sum(x.bytes for x in f.plan()) + L * r
    with pytest.raises(ValueError, match="at most 32 sources"):
        tdw.FullAttnRes(T, d, 32, BF, device="cpu")
    with pytest.raises(ValueError, match="group size"):
        tdw.FullAttnRes(T, d, L, BF, device="cpu", group=17)
    with pytest.raises(ValueError, match="use larger groups"):
        tdw.FullAttnRes(T, d, 20, BF, device="cpu", group=1)


def test_backward_argument_checks_fire_first():
    prm = {"w": torch.zeros((5, 64)), "g": None, "gamma": None}
    f = tdw.FullAttnRes(8, 64, 4, BF, device="cpu")
    with pytest.raises(ValueError, match="dh_final is required"):
        f.backward(prm, lambda l, dv: None)
    st = tdw.BlockAttnRes(8, 64, (2, 2), BF, device="cpu")
    with pytest.raises(RuntimeError, match="training=True"):
        st.backward(prm, lambda l, dv: None, dh_final=torch.zeros((8, 64), dtype=BF))


def test_workspace_sizes_cover_the_site_backward_for_one_site():
    # a one-site phase-1 backward without c/gp runs on the site backward kernel
    for T, d, n in ((16384, 7168, 9), (100, 64, 3), (4096, 1024, 17 - 1)):
        assert _lib.attnres_phase1_backward_workspace_bytes(T, d, n, 1) >= \
            _lib.attnres_site_backward_workspace_bytes(T, d)


def test_bench_refuses_several_gpus():
    # one GPU's throughput is the measured value; several GPUs are not run
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "several GPUs is not supported" in r.stderr
    assert r.stdout == ""
