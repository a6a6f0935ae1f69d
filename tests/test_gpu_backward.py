"""GPU parity of the backward through the block structure (phase-2 backward
per site, phase-1 backward per block) against the oracle's fp64 backward,
itself pinned to finite differences (needs an MI355X)."""
import sys

import pytest
import torch

import synth
from harness import run_block_backward_parity, run_block_parity
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


BWD_CASES = [
    # (T, d, blocks, n_given, dtype, final_site)
    (64, 256, (4, 4), 0, "f32", True),        # the tiny fp32 workload's shape
    (5, 8, (1, 2, 3), 0, "f32", True),        # smallest rows, a block of one sublayer
    (33, 64, (2, 3), 1, "f32", False),        # no final site
    (200, 1032, (3, 5, 2), 1, "bf16", True),  # ragged chunk groups
    (96, 2048, (6,), 3, "bf16", True),
    (40, 7168, (5, 4), 2, "bf16", True),
    (6, 16384, (3, 2), 1, "bf16", True),      # widest rows: 1024-thread teams
    (7, 10240, (2, 2), 0, "f32", True),       # fp32 rows past 8192
    (24, 256, (2, 2, 2, 2), 11, "bf16", True),  # up to 15 block sources
]


@pytest.mark.parametrize("T,d,blocks,n_given,dt,final_site", BWD_CASES)
def test_block_backward_matches_oracle(T, d, blocks, n_given, dt, final_site):
    base = synth.WORKLOADS["tiny_block_f32"]
    w = synth.scaled(base, name="bwd", T=T, d=d, block_sizes=tuple(blocks), n_given=n_given, dtype=dt,
                     unit_gains=False, seed=6100 + T + d, final_site=final_site)
    _say("case block backward T=%d d=%d blocks=%s given=%d %s final=%s" % (T, d, blocks, n_given, dt, final_site))
    worst = run_block_backward_parity(w)
    _say("worst", worst)


def test_block_backward_decode_shape():
    w = synth.WORKLOADS["decode_block_bf16"]
    _say("case block backward decode_block_bf16 T=%d d=%d S=24 given=%d" % (w.T, w.d, w.n_given))
    worst = run_block_backward_parity(w, samples=synth.sample_tokens(w.T, 24), params_too=False)
    _say("worst", worst)


def test_block_backward_prefill_chunk_sampled():
    """The 16K-token chunk, 186 sublayers in 8 blocks, at full size: every
    sampled token's dL/dv_l and dL/db_0 (upstream gradients are sublayer
    output rows, so no extra 44 GB of synthetic gradients is needed)."""
    w = synth.WORKLOADS["prefill_chunk_bf16"]
    _say("case block backward prefill_chunk_bf16 T=%d d=%d blocks=%s (8 sampled tokens)" % (w.T, w.d, w.block_sizes))
    worst = run_block_backward_parity(w, samples=synth.sample_tokens(w.T, 8), params_too=False, dx_from_outputs=True)
    _say("worst", worst)


TRAIN_FWD_CASES = [
    # (T, d, blocks, n_given, dtype): the training forward reads fp32 block
    # representations in phase 1 (bf16 outputs), sums blocks in fp32
    (64, 256, (4, 4), 0, "bf16"),
    (200, 1032, (3, 1, 2), 2, "bf16"),      # a one-sublayer block: one query on fp32 sources
    (33, 7168, (5, 3), 14, "bf16"),         # 16 sources in the last block
    (5, 8, (1, 2), 0, "f32"),
]


@pytest.mark.parametrize("T,d,blocks,n_given,dt", TRAIN_FWD_CASES)
def test_training_forward_matches_oracle(T, d, blocks, n_given, dt):
    base = synth.WORKLOADS["tiny_block_f32"]
    w = synth.scaled(base, name="trainfwd", T=T, d=d, block_sizes=tuple(blocks), n_given=n_given, dtype=dt,
                     unit_gains=False, seed=6300 + T + d)
    _say("case training forward T=%d d=%d blocks=%s given=%d %s" % (T, d, blocks, n_given, dt))
    worst = run_block_parity(w, training=True)
    _say("worst", worst)
    # the block sums are fp32 here: they carry the exact sums to fp32 rounding
    if dt == "bf16":
        assert worst["reps"] < 1e-4
