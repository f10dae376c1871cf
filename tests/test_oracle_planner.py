"""Pins of the reference planner to the pages' rules and printed plans (CPU)."""
import json
import os

import numpy as np
import pytest

from oracle import planner, reference as ref
from oracle.planner import PlanError, parse_spec, plan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
XY = {"X": 4, "Y": 2}


def test_parse_forms():
    """learntpu.dev ch05 'Notation' table: subscripts and PartitionSpecs."""
    assert parse_spec("P('X', 'Y')") == (("X",), ("Y",))
    assert parse_spec("P(('X', 'Y'), None)") == (("X", "Y"), ())
    assert parse_spec("P(None, None)") == ((), ())
    assert parse_spec("P()") == ((), ())
    assert parse_spec("('X','Y'), None") == (("X", "Y"), ())
    assert parse_spec("P('X', None)") == (("X",), ())
    assert parse_spec("A[I_X, J_Y]") == (("X",), ("Y",))
    assert parse_spec("A[I_XY, J]") == (("X", "Y"), ())
    assert parse_spec("I, J") == ((), ())
    with pytest.raises(PlanError):
        parse_spec("P('X', 'Y', 'Z')")


def test_axis_reuse_forbidden():
    """lingze.zone 'Notation' and learntpu.dev ch05: A[I_X, J_X] is invalid."""
    with pytest.raises(PlanError) as ei:
        plan(XY, "A[I_X, J_X]", "P(None, None)", 8, 8, 8)
    assert ei.value.code == "AXIS_REUSED"
    with pytest.raises(PlanError) as ei:
        plan(XY, "P(None, None)", "P('Y', 'Y')", 8, 8, 8)
    assert ei.value.code == "AXIS_REUSED"


def test_unmentioned_axis_replicates():
    """learntpu.dev ch05: on {X:4, Y:2}, A[I_X, J] is held twice."""
    p = plan(XY, "A[I_X, J]", "P(None, None)", 8, 8, 8)
    assert p.a_copies == 2
    assert p.b_copies == 8


@pytest.mark.parametrize("a,b,case", [
    ("A[I_X, J]", "B[J, K_Y]", 1),        # lingze.zone Case 1 / learntpu four cases
    ("A[I, J_X]", "B[J, K]", 2),          # Case 2
    ("A[I, J_Y]", "B[J_Y, K]", 3),        # Case 3
    ("A[I_X, J_Y]", "B[J_Y, K]", 3),      # Case 3 generalisation
    ("A[I_X, J]", "B[J, K_X]", 4),        # Case 4
])
def test_case_vectors(a, b, case):
    assert plan(XY, a, b, 16, 16, 16).case == case


def test_megatron_second_matmul_is_case3_and_fsdp_is_case2():
    """learntpu.dev ch05: every Megatron layer's second matmul is case 3;
    every FSDP layer is case 2 on its weights (gather the weight)."""
    p = plan({"X": 4}, "H[B, F_X]", "W2[F_X, D]", 16, 16, 16)
    assert p.case == 3 and p.unreduced == ("X",)
    q = plan({"X": 4}, "X[B_X, D]", "W[D_X, F]", 16, 16, 16)
    assert q.case == 2 and q.gather_operand == "B" and q.gather_axes == ("X",)


def test_case1_output_and_gather_free():
    p = plan(XY, "A[I_X, J]", "B[J, K_Y]", 16, 8, 16)
    assert planner.notation("C", p.c_spec, ("I", "K")) == "C[I_X, K_Y]"
    assert p.n_partials == 1 and p.n_groups == 8 and p.c_copies == 1


def test_case4_diagonal_blocks_only():
    """lingze.zone 'Case 4': chip x can only form the diagonal block C[x,x];
    the off-diagonal blocks are produced by no chip."""
    p = plan({"X": 2}, "A[I_X, J]", "B[J, K_X]", 4, 3, 4)
    assert p.case == 4
    A = np.arange(12, dtype=np.float64).reshape(4, 3)
    B = np.arange(12, dtype=np.float64).reshape(3, 4) - 5
    formed = set()
    for r in range(p.n_ranks):
        bl = p.rank_blocks(r)
        formed.add((bl["A"][0], bl["B"][1]))
    assert formed == {(0, 0), (1, 1)}
    with pytest.raises(PlanError):
        ref.unit_partial(p, A, B, 0)
    # the fix: gather one operand, then case 1
    assert p.gather_operand in ("A", "B")
    q = plan({"X": 2}, "A[I, J]", "B[J, K_X]", 4, 3, 4)
    assert q.case == 1


def test_case4_gathers_the_smaller_input():
    """lingze.zone 'Case 4': the fix all-gathers one input, at a cost of V/W
    with V the bytes of the gathered input; the cheaper choice is the
    smaller one (ties: A, the page's own example)."""
    for (I, J, K), want in (((4, 3, 8), "A"), ((8, 3, 4), "B"), ((4, 3, 4), "A")):
        p = plan({"X": 2}, "A[I_X, J]", "B[J, K_X]", I, J, K)
        assert p.case == 4 and p.gather_operand == want and p.gather_axes == ("X",)
        q = planner.gathered(p)
        assert q.case == 1
        assert (q.a_copies, q.b_copies) == ((2, 1) if want == "A" else (1, 2))


def test_case4_checked_before_j_cases():
    """Reading: an illegal output layout (case 4) takes precedence."""
    assert plan(XY, "A[I_Y, J_X]", "B[J_X, K_Y]", 8, 8, 8).case == 4


def test_j_mismatch():
    with pytest.raises(PlanError) as ei:
        plan(XY, "A[I, J_X]", "B[J_Y, K]", 8, 8, 8)
    assert ei.value.code == "J_MISMATCH"


def test_indivisible():
    with pytest.raises(PlanError) as ei:
        plan(XY, "A[I_X, J]", "B[J, K]", 10, 8, 8)
    assert ei.value.code == "INDIVISIBLE"


def test_sandbox_default_plan():
    """learntpu.dev ch05 'Sharding sandbox' default plan, restated in
    tests/golden/sandbox_default_plan.json."""
    with open(os.path.join(GOLDEN, "sandbox_default_plan.json")) as f:
        g = json.load(f)
    I, J = g["A_shape"]
    K = g["B_shape"][1]
    p = plan(dict(g["mesh"]), g["A_spec"], g["B_spec"], I, J, K)
    assert planner.notation("A", p.a) == g["A_notation"]
    assert list(p.a_local) == g["A_shard"]
    assert round(p.shard_bytes("A") / 1e6, 1) == g["A_shard_MB"]
    assert p.a_copies == g["A_copies"]
    assert p.n_ranks == g["devices"]
    assert list(p.a_grid) == g["A_grid"]
    assert list(p.b_grid) == g["B_grid"]
    assert list(p.b_local) == g["B_shard"]
    assert p.case == g["case"]
    assert p.unreduced == (g["reduce_axis"],)
    assert planner.notation("C", p.c_spec, ("I", "K"), p.unreduced) == g["C_before_reduce"]
    assert planner.notation("C", p.c_spec, ("I", "K")) == g["C_after_allreduce"]
    assert round(p.shard_bytes("C", "bf16") / 1e6, 1) == g["C_bytes_per_device_MB"]
    assert round(p.local_flops() / 1e9) == g["local_matmul_GFLOP"]


def test_rank_numbering_and_units():
    """Reading: ranks row-major over the mesh axes; unit = g*N + y."""
    p = plan(XY, "P('X', 'Y')", "P('Y', None)", 16, 16, 16)
    assert p.coords(5) == {"X": 2, "Y": 1}
    assert [p.rank_unit(r) for r in range(8)] == list(range(8))
    assert p.n_groups == 4 and p.n_partials == 2
    assert p.c_rs_spec == (("X", "Y"), ())
    assert p.rs_rows(2, 1) == (2 * 4 + 2, 2)


def test_flatten_first_axis_major():
    """Reading: I_XY is split with X major (block = x*|Y| + y)."""
    p = plan(XY, "P(('X', 'Y'), None)", "P(None, None)", 16, 4, 4)
    for r in range(8):
        c = p.coords(r)
        assert p.rank_blocks(r)["A"] == (c["X"] * 2 + c["Y"], 0)


def test_replica_axis_units():
    """An axis used by neither operand replicates the work: units count
    distinct local products only."""
    p = plan({"X": 2, "Y": 2, "Z": 2}, "P('X', 'Y')", "P('Y', None)", 8, 8, 8)
    assert p.n_units == 4 and p.c_copies == 2
    seen = {}
    for r in range(p.n_ranks):
        seen.setdefault(p.rank_unit(r), []).append(r)
    assert all(len(v) == 2 for v in seen.values())
