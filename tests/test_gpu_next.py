"""GPU parity of the widened rows: case 2 / case 4 by composition (gather the
operand, re-plan, multiply) and the fused local-products + reduce kernel,
against the fp64 oracle through the C ABI."""
import numpy as np
import pytest
import torch

import local_shard_gemm_amd as sm
import workloads as wl
from oracle import planner, reference as ref

from hip_cases import DEV, REL_TOL, f32_bits_equal, guard_intact, guarded, run_partials, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu


def _stack_blocks(X: torch.Tensor, p_grid, axis_rows: bool):
    """Host-side stacked layout of a 2-D operand's blocks (block id =
    row_block * grid[1] + col_block)."""
    gr, gc = p_grid
    rows, cols = X.shape[0] // gr, X.shape[1] // gc
    return torch.stack([X[i * rows:(i + 1) * rows, j * cols:(j + 1) * cols].contiguous()
                        for i in range(gr) for j in range(gc)])


# ------------------------------------------------------------------ f1

@pytest.mark.parametrize("shape", [(512, 768, 640), (4096, 4096, 4096)], ids=["small", "case1-size"])
def test_case2_gather_then_multiply(shape):
    """lingze.zone 'Case 2': A[I, J_X] . B[J, K] -- all-gather A, then a
    case-1 product. A arrives as stacked per-rank column blocks."""
    I, J, K = shape
    say("case: case2 composition", shape)
    A = wl.random_ints((I, J), 601)
    B = wl.random_ints((J, K), 602)
    mesh = {"X": 4, "Y": 2}
    p = sm.sm_plan(mesh, "A[I, J_X]", "B[J, K]", I, J, K)
    q = planner.plan(mesh, "A[I, J_X]", "B[J, K]", I, J, K)
    assert p.kase == sm.SM_CASE2 and q.gather_operand == "A"
    stacked = to_dev(_stack_blocks(A, tuple(p.a_grid), False))
    Ag = torch.empty(I, J, dtype=torch.bfloat16, device=DEV)
    sm.sm_gather_shards(p, sm.SM_WHAT_A, sm.buf(stacked), sm.buf(Ag))
    assert torch.equal(Ag.cpu(), A)
    p2 = sm.sm_plan_gathered(p)
    q2 = planner.gathered(q)
    assert p2.kase == sm.SM_CASE1 == q2.case and p2.n_units == q2.n_units == 1
    Bd = to_dev(B)
    C = torch.empty(I, K, dtype=torch.float32, device=DEV)
    sm.sm_local_gemm(p2, sm.buf(Ag), sm.buf(Bd), sm.buf(C))
    Cn = C.cpu().numpy()
    if I * J * K <= 512 * 768 * 640:
        assert f32_bits_equal(Cn, ref.dense(A, B))
    else:
        assert ref.freivalds(A, (0, 0, I, J), B, (0, 0, J, K), Cn.astype(np.float64), trials=1) == 0.0
        rows = sample_rows(I, 4, 3)
        assert f32_bits_equal(Cn[rows], ref.matmul(A, B, rows=rows))


def test_case4_gather_smaller_then_multiply():
    """lingze.zone 'Case 4': A[I_X, J] . B[J, K_X] forms only diagonal
    blocks; all-gather the smaller operand and multiply as case 1."""
    I, J, K = 512, 256, 1024
    say("case: case4 composition")
    A = wl.random_ints((I, J), 611)
    B = wl.random_ints((J, K), 612)
    mesh = {"X": 4}
    p = sm.sm_plan(mesh, "A[I_X, J]", "B[J, K_X]", I, J, K)
    assert p.kase == sm.SM_CASE4 and p.gather_operand == 0  # A is smaller
    with pytest.raises(sm.ShardmmError) as ei:
        sm.sm_local_gemm(p, sm.buf(to_dev(A)), sm.buf(to_dev(B)),
                         sm.buf(torch.empty(4, I // 4, K // 4, device=DEV)))
    assert ei.value.status == sm.SM_ERR_NEEDS_GATHER
    stacked = to_dev(_stack_blocks(A, tuple(p.a_grid), True))
    Ag = torch.empty(I, J, dtype=torch.bfloat16, device=DEV)
    sm.sm_gather_shards(p, sm.SM_WHAT_A, sm.buf(stacked), sm.buf(Ag))
    p2 = sm.sm_plan_gathered(p)
    q2 = planner.gathered(planner.plan(mesh, "A[I_X, J]", "B[J, K_X]", I, J, K))
    assert p2.kase == sm.SM_CASE1 and p2.n_units == q2.n_units == 4
    Bd = to_dev(B)
    full, P = run_partials(p2, Ag, Bd)
    C = torch.empty(I, K, dtype=torch.float32, device=DEV)
    sm.sm_gather_shards(p2, sm.SM_WHAT_C_BLOCKS, sm.buf(P), sm.buf(C))
    assert f32_bits_equal(C.cpu().numpy(), ref.dense(A, B))
    assert guard_intact(full, P.numel())


# ------------------------------------------------------------------ f2

FUSED = [
    ({"X": 2, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 600, 400, 520),   # ragged: edge tiles
    ({"Y": 2}, "P(None, 'Y')", "P('Y', None)", 512, 512, 768),          # interior tiles
    ({"X": 2, "T": 4}, "P('X', 'T')", "P('T', None)", 2 * 256, 4 * 96, 256),
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: f"{c[3]}x{c[4]}x{c[5]}")
@pytest.mark.parametrize("mode", [sm.SM_ALLREDUCE, sm.SM_REDUCESCATTER], ids=["AR", "RS"])
def test_fused_reduce_bitexact(case, mode):
    mesh, sa, sb, I, J, K = case
    say("case: fused", case, mode)
    A = wl.random_ints((I, J), 701 + I)
    B = wl.random_ints((J, K), 702 + K)
    p = sm.sm_plan(mesh, sa, sb, I, J, K)
    q = planner.plan(mesh, sa, sb, I, J, K)
    Ad, Bd = to_dev(A), to_dev(B)
    parts = [ref.unit_partial(q, A, B, u) for u in range(q.n_units)]
    m, n = q.c_local
    N = q.n_partials
    # global layout
    fg, g = guarded((I, K), torch.float32)
    sm.sm_local_gemm_reduce(p, sm.buf(Ad), sm.buf(Bd), sm.buf(g), mode)
    want = ref.gather(q, ref.allreduce(q, parts))
    assert f32_bits_equal(g.cpu().numpy(), want)
    assert guard_intact(fg, g.numel())
    # stacked layout, with a padded block stride so RS row blocks are apart
    if mode == sm.SM_ALLREDUCE:
        blocks, rows = q.n_groups, m
    else:
        blocks, rows = q.n_groups * N, m // N
    stride = (rows + 3) * n
    fs = torch.full((blocks * stride + 64,), float("nan"), device=DEV)
    s = sm.sm_buf(fs.data_ptr(), n, stride, fs.numel())
    sm.sm_local_gemm_reduce(p, sm.buf(Ad), sm.buf(Bd), s, mode)
    fsn = fs.cpu().numpy()
    if mode == sm.SM_ALLREDUCE:
        sums = ref.allreduce(q, parts)
        for gi in range(q.n_groups):
            assert f32_bits_equal(fsn[gi * stride:gi * stride + m * n].reshape(m, n), sums[gi])
    else:
        rs = ref.reduce_scatter(q, parts)
        for (gi, y), blk in rs.items():
            o = (gi * N + y) * stride
            assert f32_bits_equal(fsn[o:o + rows * n].reshape(rows, n), blk)
    pad = np.concatenate([fsn[b * stride + rows * n:(b + 1) * stride] for b in range(blocks)])
    assert np.isnan(pad).all()  # nothing written between blocks


def test_fused_reduce_full_downproj():
    """The down-projection at full size: fused kernel == GEMM + reduce-scatter
    bit for bit on integers; within tolerance of the oracle on floats."""
    w = wl.get("downproj")
    for integer in (True, False):
        ww = wl.int_variant(w) if integer else w
        say("case: fused full downproj", "int" if integer else "float")
        A = wl.make_operand(ww.operand("A"))
        B = wl.make_operand(ww.operand("B"))
        I, J = A.shape
        K = B.shape[1]
        p = sm.sm_plan(dict(w.mesh), w.operand("A").spec, w.operand("B").spec, I, J, K)
        q = planner.plan(dict(w.mesh), w.operand("A").spec, w.operand("B").spec, I, J, K)
        Ad, Bd = to_dev(A), to_dev(B)
        fused = torch.empty(I, K, dtype=torch.float32, device=DEV)
        sm.sm_local_gemm_reduce(p, sm.buf(Ad), sm.buf(Bd), sm.buf(fused), sm.SM_REDUCESCATTER)
        if integer:
            _, P = run_partials(p, Ad, Bd)
            rs = torch.empty(I, K, dtype=torch.float32, device=DEV)
            sm.sm_reduce_partials(p, sm.buf(P), sm.buf(rs), sm.SM_REDUCESCATTER)
            assert torch.equal(fused, rs)
            assert ref.freivalds(A, (0, 0, I, J), B, (0, 0, J, K), fused.cpu().numpy().astype(np.float64),
                                 trials=1) == 0.0
        else:
            rows = sample_rows(I, 12, 77)
            want = ref.matmul(A, B, rows=rows)
            err = ref.rel_frobenius(fused[rows].cpu().numpy(), want)
            say("fused float rel err", err)
            assert err <= REL_TOL
        del Ad, Bd, fused
