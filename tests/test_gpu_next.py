"""GPU parity of the widened rows: case 2 / case 4 by composition (gather the
operand, re-plan, multiply) and the fused local-products + reduce kernel,
against the fp64 oracle through the C ABI."""
import numpy as np
import pytest
import torch

import local_shard_gemm_amd as sm
import workloads as wl
from oracle import planner, reference as ref

from hip_cases import (DEV, FREIVALDS_FLOAT_TOL, REL_TOL, f32_bits_equal, guard_intact, guarded, run_partials,
                       sample_rows, say, to_dev)

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
    s = sm.sm_buf(fs.data_ptr(), n, stride, fs.numel(), sm.SM_F32, 0)
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
            fr = ref.freivalds(A, (0, 0, I, J), B, (0, 0, J, K), fused.cpu().numpy(), trials=1, ints=False)
            say("fused whole-output Freivalds residual", fr)
            assert fr <= FREIVALDS_FLOAT_TOL
        del Ad, Bd, fused


# ------------------------------------------------------------------ f3

LN_TOL_INT = 1e-5   # exact pre-norm sums; float32 mean / variance / scaling
LN_TOL = REL_TOL


@pytest.mark.parametrize("integer", [True, False], ids=["int", "float"])
def test_sp_tail_reduce_scatter_layernorm(integer):
    """ana-alekseeva.com 'Sequence parallelism': RS, per-token layer norm on
    the owned rows, AG. Global output (AG in place) and stacked output then
    sm_gather_shards must agree bit for bit."""
    mesh, sa, sb, I, J, K = {"X": 2, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 512, 2 * 192, 520
    say("case: sp tail", "int" if integer else "float")
    mk = (lambda s, seed: wl.random_ints(s, seed)) if integer else (lambda s, seed: wl.random_normal(s, seed))
    A, B = mk((I, J), 801), mk((J, K), 802)
    p = sm.sm_plan(mesh, sa, sb, I, J, K)
    q = planner.plan(mesh, sa, sb, I, J, K)
    Ad, Bd = to_dev(A), to_dev(B)
    _, P = run_partials(p, Ad, Bd)
    rng = np.random.default_rng(803)
    gamma = rng.standard_normal(K).astype(np.float32)
    beta = rng.standard_normal(K).astype(np.float32)
    gd, bd = torch.from_numpy(gamma).to(DEV), torch.from_numpy(beta).to(DEV)
    parts = [ref.unit_partial(q, A, B, u) for u in range(q.n_units)]
    tol = LN_TOL_INT if integer else LN_TOL
    for g_, b_ in ((None, None), (gd, bd)):
        fo, out = guarded((I, K), torch.float32)
        sm.sm_reduce_scatter_layernorm(p, sm.buf(P), sm.buf(out), g_, b_, 1e-5)
        want = ref.sp_tail(q, parts, None if g_ is None else gamma, None if b_ is None else beta, 1e-5)
        err = ref.rel_frobenius(out.cpu().numpy(), want)
        say("sp tail rel err", err)
        assert err <= tol
        assert guard_intact(fo, out.numel())
        st = torch.empty(q.n_groups * q.n_partials, q.c_local[0] // q.n_partials, K, device=DEV)
        sm.sm_reduce_scatter_layernorm(p, sm.buf(P), sm.buf(st), g_, b_, 1e-5)
        ag = torch.empty(I, K, device=DEV)
        sm.sm_gather_shards(p, sm.SM_WHAT_C_SCATTERED, sm.buf(st), sm.buf(ag))
        assert torch.equal(ag, out)


def test_sp_tail_full_downproj():
    w = wl.get("downproj")
    say("case: sp tail full downproj")
    A = wl.make_operand(w.operand("A"))
    B = wl.make_operand(w.operand("B"))
    I, J = A.shape
    K = B.shape[1]
    p = sm.sm_plan(dict(w.mesh), w.operand("A").spec, w.operand("B").spec, I, J, K)
    q = planner.plan(dict(w.mesh), w.operand("A").spec, w.operand("B").spec, I, J, K)
    _, P = run_partials(p, to_dev(A), to_dev(B))
    out = torch.empty(I, K, device=DEV)
    sm.sm_reduce_scatter_layernorm(p, sm.buf(P), sm.buf(out), None, None, 1e-5)
    m = q.c_local[0]
    for g in (0, 3):
        rows = sample_rows(m, 4, 900 + g)
        parts = [ref.unit_partial(q, A, B, g * 2 + y, rows=rows) for y in range(2)]
        want = ref.layer_norm(ref.sum_ranked(parts))
        got = out[[g * m + r for r in rows]].cpu().numpy()
        assert ref.rel_frobenius(got, want) <= LN_TOL


def test_sp_tail_full_mlp_with_affine():
    """The tail as the benchmark runs it: the MLP's 4 partials [4096, 4096]
    (from the two-layer chain on the full workload), reduce-scattered, layer
    normed with gamma and beta, all-gathered; sampled rows of every owner
    within the float tolerance of the oracle."""
    w = wl.get("mlp")
    say("case: sp tail full mlp")
    X = wl.make_operand(w.operand("X"))
    W1 = wl.make_operand(w.operand("W1"))
    W2 = wl.make_operand(w.operand("W2"))
    B_, D = X.shape
    F = W1.shape[1]
    p1 = sm.sm_plan(dict(w.mesh), w.operand("X").spec, w.operand("W1").spec, B_, D, F, out_dtype=sm.SM_BF16)
    p2 = sm.sm_plan(dict(w.mesh), "P(None, 'T')", w.operand("W2").spec, B_, F, D)
    q2 = planner.plan(dict(w.mesh), "P(None, 'T')", w.operand("W2").spec, B_, F, D)
    H = torch.empty(B_, F, dtype=torch.bfloat16, device=DEV)
    sm.sm_local_gemm(p1, sm.buf(to_dev(X)), sm.buf(to_dev(W1)), sm.buf(H), sm.SM_EPI_GELU_TANH)
    _, P = run_partials(p2, H, to_dev(W2))
    rng = np.random.default_rng(811)
    gamma = rng.standard_normal(D).astype(np.float32)
    beta = rng.standard_normal(D).astype(np.float32)
    out = torch.empty(B_, D, device=DEV)
    sm.sm_reduce_scatter_layernorm(p2, sm.buf(P), sm.buf(out), torch.from_numpy(gamma).to(DEV),
                                   torch.from_numpy(beta).to(DEV), 1e-5)
    # oracle only: the chain's rank-ordered Z rows from the oracle's own H,
    # then the layer norm of each owned row
    q1 = planner.plan(dict(w.mesh), w.operand("X").spec, w.operand("W1").spec, B_, D, F)
    m = q2.c_local[0] // q2.n_partials
    for y in range(q2.n_partials):
        rows = [y * m + r for r in sample_rows(m, 3, 820 + y)]
        _, z = ref.mlp_chain(q1, q2, X, W1, W2, rows=rows)
        want = ref.layer_norm(z, gamma, beta, 1e-5)
        got = out[rows].cpu().numpy()
        assert ref.rel_frobenius(got, want) <= LN_TOL, y


# ------------------------------------------------------------------ f4

RESHARD = [
    ({"X": 4}, "A[I, J_X]", "A[I_X, J]", 512, 768),       # all-to-all
    ({"X": 4}, "A[I, J_X]", "A[I_X, J]", 4104, 96),       # 16 jobs of 1026 short rows, copied in source order
    ({"X": 2, "Y": 2}, "A[I_XY, J]", "A[I_X, J_Y]", 256, 512),
    ({"X": 4}, "A[I_X, J]", "P()", 256, 264),             # all-gather to replicated
    ({"X": 2, "Y": 3}, "A[I, J_X]", "A[I, J_Y]", 64, 48),  # blocks straddle blocks
]


def test_reshard_full_size_bitexact():
    """The all-to-all as the benchmark runs it: bf16 [4096, 4096] A[I,J_X] ->
    A[I_X,J] on {X:4}, stacked blocks in and out, bit for bit."""
    say("case: reshard full size")
    X = wl.random_normal((4096, 4096), 961)
    mesh = {"X": 4}
    src_blocks = ref.shard(ref.stored(X)[0], mesh, "A[I, J_X]")
    src = to_dev(torch.from_numpy(np.stack([src_blocks[b] for b in sorted(src_blocks)])).view(torch.bfloat16))
    dst = torch.empty(4, 1024, 4096, dtype=torch.bfloat16, device=DEV)
    sm.sm_reshard(mesh, "A[I, J_X]", "A[I_X, J]", 4096, 4096, sm.SM_BF16, sm.buf(src), sm.buf(dst))
    want = ref.reshard(src_blocks, mesh, "A[I, J_X]", "A[I_X, J]", 4096, 4096)
    got = ref.stored(dst.cpu())[0]
    for b in range(4):
        np.testing.assert_array_equal(got[b], want[b])


@pytest.mark.parametrize("case", RESHARD, ids=lambda c: f"{c[1]}->{c[2]}")
@pytest.mark.parametrize("dtype", [sm.SM_BF16, sm.SM_F32], ids=["bf16", "f32"])
def test_reshard_bitexact(case, dtype):
    mesh, frm, to, R, Cc = case
    say("case: reshard", case, dtype)
    X = wl.random_normal((R, Cc), 950 + R)
    if dtype == sm.SM_F32:
        X = X.float()
    tdt = torch.bfloat16 if dtype == sm.SM_BF16 else torch.float32
    src_blocks = ref.shard(ref.stored(X)[0], mesh, frm)
    src = to_dev(torch.from_numpy(np.stack([src_blocks[b] for b in sorted(src_blocks)])).view(tdt)
                 if dtype == sm.SM_BF16 else torch.from_numpy(np.stack([src_blocks[b] for b in sorted(src_blocks)])))
    want = ref.reshard(src_blocks, mesh, frm, to, R, Cc)
    nb = len(want)
    br, bc = next(iter(want.values())).shape
    full = torch.full((nb * br * bc + 256,), 7, dtype=tdt, device=DEV)
    dst = full[:nb * br * bc].view(nb, br, bc)
    sm.sm_reshard(mesh, frm, to, R, Cc, dtype, sm.buf(src), sm.buf(dst))
    got = ref.stored(dst.cpu())[0]
    for b in range(nb):
        np.testing.assert_array_equal(got[b], want[b])
    assert bool((full[nb * br * bc:] == 7).all())
    # global source layout gives the same blocks
    Xd = to_dev(X)
    dst2 = torch.empty_like(dst)
    sm.sm_reshard(mesh, frm, to, R, Cc, dtype, sm.buf(Xd, block_stride=0), sm.buf(dst2))
    assert torch.equal(dst2, dst)
