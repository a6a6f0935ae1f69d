"""The pages' analytic cost model (transformer_depth_wise_amd.costmodel)
against every number the pages print for it.  The printed values are rounded,
so each check allows half a unit of the last printed digit; each would fail
for a plausible slip (a dropped +1, a missing factor 2, the other form of a
formula)."""
import pytest

from transformer_depth_wise_amd import costmodel as cm

MiB, GiB = 1 << 20, 1 << 30
d = 7168


def near(x, printed, half_unit):
    return abs(x - printed) <= half_unit


def test_io_table_at_the_typical_setting():
    # "Attention Residuals" structured notes, section 10, analytic I/O table at
    # L = 128, N = 8, S = 16, m = 4: 3d, 34d + 48, 24d, 5.5d
    assert cm.io_standard_residual(d) == 3 * d
    assert cm.io_mhc(4, d) == 34 * d + 48
    assert cm.io_full_two_phase(16, 8, d) == 24 * d
    assert cm.io_block_two_phase(8, 16, d) == 5.5 * d
    # Block with N = L (one sublayer per block) is Full without the merge saving
    assert cm.io_block_two_phase(128, 1, d) == 133 * d


def test_batching_reads_each_history_row_once_per_group():
    # "Attention Residuals 阅读补充", static queries: 2 S R d b -> 2 R d b
    per_query, per_group = cm.batched_history_reads(16, 9, d, 2)
    assert per_query == 16 * per_group == 2 * 16 * 9 * d * 2


def test_full_arithmetic_and_parameters_at_k2_sizes():
    # "Attention Residuals 阅读补充", Full AttnRes arithmetic: L = 122, d = 7168
    assert cm.full_pairs(122) == 7503
    assert near(cm.full_forward_flops(122, d) / 1e9, 0.215, 5e-4)
    assert near(cm.full_train_flops(122, d) / 1e9, 0.645, 5e-4)
    assert near(cm.query_params(122, d) / 1e6, 1.75, 5e-3)
    # the forward share of a ~64 GFLOPs/token backbone: about 0.34%
    assert near(100 * cm.full_forward_flops(122, d) / 64e9, 0.34, 5e-3)


def test_full_history_memory():
    # reading notes, Full AttnRes history memory: B = 1, T = 32K, L = 128 -> about
    # 60 GB, about 7.5 GB on each of 8 sequence shards
    m = cm.full_prefill_bytes(1, 32 * 1024, 128, d)
    assert near(m / 1e9, 60, 1.0)
    assert near(m / 8 / 1e9, 7.5, 0.1)
    # decode: 123 depth states of one token, about 1.68 MiB
    assert near(cm.depth_state_bytes(123, d) / MiB, 1.68, 5e-3)
    # training: one 4096-token hidden state is 56 MiB; 123 of them 6.73 GiB
    assert cm.history_bytes(4096, 1, d) == 56 * MiB
    assert near(cm.history_bytes(4096, 123, d) / GiB, 6.73, 5e-3)


def test_block_history_memory():
    # reading notes, Block AttnRes activation memory: 8 to 9 block
    # representations of 4096 tokens, 448 to 504 MiB
    assert cm.history_bytes(4096, 8, d) == 448 * MiB
    assert cm.history_bytes(4096, 9, d) == 504 * MiB
    # reading notes, Block AttnRes history memory: B = 1, N = 8, T = 128K -> about
    # 15 GB, about 1.9 GB over 8 devices, below 0.3 GB with 16K chunks
    total = cm.block_prefill_bytes(1, 8, 128 * 1024, d)
    assert near(total / 1e9, 15, 0.5)
    assert near(cm.block_prefill_bytes(1, 8, 128 * 1024, d, P=8) / 1e9, 1.9, 0.05)
    assert cm.block_prefill_bytes(1, 8, 16 * 1024, d, P=8) / 1e9 < 0.3


def test_pipeline_communication_example():
    # structured notes, section 9: P = 4 physical stages, V = 2 virtual each ->
    # naive 28 N_p d, cached 22 N_p d, 6 block transfers fewer
    assert cm.pp_comm_naive(4, 2) == 28
    assert cm.pp_comm_cached(4, 2) == 22
    # one virtual stage per physical stage: nothing to cache
    assert cm.pp_comm_cached(5, 1) == cm.pp_comm_naive(5, 1)


@pytest.mark.parametrize("L,N,block", [(128, 8, 5.5), (186, 8, 5.344), (128, 128, 133.0)])
def test_model_for_uses_s_equal_l_over_n(L, N, block):
    assert cm.model_for(L, N)["block_two_phase"] == pytest.approx(block, abs=1e-3)
