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
    # the forward at the prefill chunk's shape moves 6.638 rows of d per token
    # and sublayer (every term is proportional to T; the per-token statistics
    # make the ratio depend slightly on d); phase 1 writes S outputs per block
    # except the first block's (its only source is b_0)
    st = tdw.BlockAttnRes(16, 7168, K3, BF, device="cpu")
    plan = st.plan()
    assert abs(rows_per_token_sublayer(plan, 16, 7168, 186) - 6.638) < 5e-4
    kinds = [x.kind for x in plan]
    assert kinds.count("phase1") == 8 and kinds.count("accumulate") == 8 and kinds.count("final") == 1
    assert kinds.count("phase2") == 186 - 8     # the first sublayer of each block leaves phase 1
    twice = tdw.BlockAttnRes(32, 7168, K3, BF, device="cpu").plan()
    assert sum(x.bytes for x in twice) == 2 * sum(x.bytes for x in plan)


def test_block_plan_backward_bytes():
    # the 16K chunk's backward moves 509859266560 bytes (every term is
    # proportional to T): 16 tokens of it move 1/1024 of that
    st = tdw.BlockAttnRes(16, 7168, K3, BF, device="cpu", training=True)
    assert sum(x.bytes for x in st.plan_backward()) * 1024 == 509859266560


def test_block_source_limits():
    with pytest.raises(ValueError, match="at most 16 completed sources"):
        tdw.BlockAttnRes(4, 64, (1,) * 15 + (2,), BF, n_given=1, device="cpu")
    with pytest.raises(ValueError, match="too many sources"):
        tdw.BlockAttnRes(4, 64, (1,) * 32, BF, device="cpu")
    tdw.BlockAttnRes(4, 64, (1,) * 31, BF, device="cpu")            # 32 sources at the final site
    tdw.BlockAttnRes(4, 64, (1,) * 15 + (2,), BF, device="cpu")      # 16 completed sources for S = 2


def test_full_plan_and_limits():
    T, d, L = 8, 64, 16
    f = tdw.FullAttnRes(T, d, L, BF, device="cpu")
    r, r32 = T * d * 2, T * d * 4
    assert sum(x.bytes for x in f.plan_backward()) == \
        sum((l + 1) * (r + 2 * r32) + r for l in range(L + 1))
    assert [x.kind for x in f.plan()].count("full") == L
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
