"""Host-side plan: grouping by trailing shape, transposed members, chunking,
workspace sizing and every validation error.  Runs on the CPU (the plan does
no device work)."""
import json
import os

import pytest
import torch

from newton_schulz_05_amd import MuonError, MuonPlan
from newton_schulz_05_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_workloads.json")


def test_pages_fused_case_is_one_group():
    """74 params of [24, 10240] form one [74, 24, 10240] batch (RFC item 3)."""
    spec = json.load(open(GOLDEN))["fused_case"]
    plan = MuonPlan([tuple(spec["shape"])] * spec["count"], torch.bfloat16)
    g = plan.groups()
    assert len(g) == 1
    assert (g[0]["m"], g[0]["n"], g[0]["count"], g[0]["n_transposed"]) == (24, 10240, 74, 0)
    assert g[0]["n_chunks"] == 1


def test_pages_slab_is_batch_of_matrices():
    shapes = json.load(open(GOLDEN))["small_matrix_shapes"]
    plan = MuonPlan([tuple(s) for s in shapes], torch.bfloat16)
    g = plan.groups()
    assert len(g) == 1 and g[0]["count"] == 1 + 32


def test_c3_groups():
    plan = MuonPlan(W.WORKLOADS["c3"].shapes, torch.bfloat16)
    g = {(x["m"], x["n"]): x for x in plan.groups()}
    assert g[(1536, 2048)]["count"] == 8 and g[(1536, 2048)]["n_transposed"] == 8
    assert g[(24, 10240)]["count"] == 32 and g[(24, 10240)]["n_transposed"] == 0


def test_c4_merges_transposed_up_gate_with_down():
    plan = MuonPlan(W.WORKLOADS["c4"].shapes, torch.bfloat16)
    g = {(x["m"], x["n"]): x for x in plan.groups()}
    assert set(g) == {(4096, 4096), (4096, 14336)}
    assert g[(4096, 4096)]["count"] == 128 and g[(4096, 4096)]["n_transposed"] == 0
    assert g[(4096, 14336)]["count"] == 96 and g[(4096, 14336)]["n_transposed"] == 64
    # chunks cover the group; the per-launch table holds at most 80 matrices
    assert g[(4096, 4096)]["n_chunks"] >= 2


def test_mfma_chunks_leave_no_partial_round_when_they_can():
    # 256-tiles: 136 symmetric tiles per 4096-row matrix.  128 squares fit
    # 4 chunks of 32 (4352 tiles, 17 rounds of 256); the 96 wide matrices
    # fit 3 of 32 under the workspace cap, where the fewest chunks alone
    # would do too (one more chunk is taken only when it leaves fewer tiles
    # over, and 3 x 32 leaves none)
    plan = MuonPlan(W.WORKLOADS["c4"].shapes, torch.bfloat16)
    g = {(x["m"], x["n"]): x for x in plan.groups()}
    assert g[(4096, 4096)]["n_chunks"] == 4
    assert g[(4096, 14336)]["n_chunks"] == 3
    # the workspace holds the largest chunk of any group, under the 32 GiB cap
    assert plan.workspace_bytes <= (32 << 30) + (1 << 20)
    # a group that one chunk holds stays in one chunk
    assert [x["n_chunks"] for x in MuonPlan([(2048, 2048)] * 10, torch.bfloat16).groups()] == [1]


def test_c1_c2_c5_groups():
    assert [(x["m"], x["n"], x["count"]) for x in MuonPlan(W.WORKLOADS["c1"].shapes, torch.float32).groups()] \
        == [(64, 128, 4)]
    assert [(x["m"], x["n"], x["count"]) for x in MuonPlan(W.WORKLOADS["c5"].shapes, torch.bfloat16).groups()] \
        == [(8192, 28672, 2)]


def test_group_order_is_first_appearance():
    plan = MuonPlan([(5, 7), (3, 4), (7, 5), (4, 3)], torch.bfloat16)
    assert [(g["m"], g["n"], g["count"], g["n_transposed"]) for g in plan.groups()] == \
        [(5, 7, 2, 1), (3, 4, 2, 1)]


def test_workspace_grows_with_shape():
    small = MuonPlan([(128, 256)], torch.bfloat16).workspace_bytes
    big = MuonPlan([(1024, 2048)], torch.bfloat16).workspace_bytes
    assert 0 < small < big


def test_workspace_independent_of_param_order():
    a = MuonPlan([(100, 300), (24, 999)], torch.bfloat16).workspace_bytes
    b = MuonPlan([(24, 999), (100, 300)], torch.bfloat16).workspace_bytes
    assert a == b


@pytest.mark.parametrize("shape", [(0, 5), (5, 0), (0, 3, 4), (-1, 4)])
def test_bad_shapes_rejected(shape):
    with pytest.raises(MuonError) as e:
        MuonPlan([shape], torch.bfloat16)
    assert e.value.name == "MUON_ERR_SHAPE"


def test_mfma_width_limit():
    """bf16 MFMA-path groups address a 256-row operand tile with 32-bit
    buffer offsets, so max(rows, cols) is limited to 2^22 - 256 there (tall
    members too; a matrix that wide is also beyond the skinny path's
    co-resident slabs whatever its m); fp32 keeps wider matrices."""
    lim = (1 << 22) - 256
    MuonPlan([(64, lim)], torch.bfloat16)
    for shape in [(64, lim + 1), (lim + 1, 64)]:
        with pytest.raises(MuonError) as e:
            MuonPlan([shape], torch.bfloat16)
        assert e.value.name == "MUON_ERR_SHAPE"
    with pytest.raises(MuonError):
        MuonPlan([(24, lim + 1)], torch.bfloat16)
    MuonPlan([(64, lim + 1)], torch.float32)


def test_one_d_rejected():
    with pytest.raises(MuonError) as e:
        MuonPlan([(5,)], torch.bfloat16)
    assert e.value.name == "MUON_ERR_SHAPE"


def test_bad_dtype_rejected():
    with pytest.raises(MuonError) as e:
        MuonPlan([(5, 6)], torch.float16)
    assert e.value.name == "MUON_ERR_DTYPE"


def test_empty_plan_rejected():
    with pytest.raises(MuonError) as e:
        MuonPlan([], torch.bfloat16)
    assert e.value.name == "MUON_ERR_INVALID_ARG"
