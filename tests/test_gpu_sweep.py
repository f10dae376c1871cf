"""Seeded random sweep of the whole path through the C ABI.

Random meshes (up to three axes, at most 8 ranks), random partition specs
of A[I,J] and B[J,K] (lingze.zone "Cheetsheet for the four cases of sharded
matmul": which dimension each mesh axis shards decides the case), random
ragged sizes and leading dimensions padded with NaN, integer-valued
inputs. Every
plan the library accepts runs through every call that applies to its case,
and every result is compared bit for bit with the oracle's dense product
A.B (fp64 from the stored inputs; integers keep every fp32 sum exact):

- case 1: the local products, gathered into the global layout;
- case 3: the partials against the oracle's unit partials, then
  sm_reduce_partials (all-reduce and, when the rows split, reduce-scatter),
  sm_local_gemm_reduce_ws, and the single-launch sm_local_gemm_reduce for
  products of more than 64 rows;
- reshards (a separate sweep): random source and target specs on random
  meshes, bf16 and float32, against the oracle's blocks;
- the sequence-parallel tail (a third sweep) on random case-3 plans with
  whole output rows, within 1e-5 of the oracle's tail;
- the GeLU -> bfloat16 epilogue (a fourth sweep) on random case-1 plans,
  within the derived bound of the oracle's round_bf16(gelu(.));
- cases 2 and 4: the operand the plan names gathered with
  sm_gather_shards and the re-plan from sm_plan_gathered, repeated until
  the plan is case 1 or 3 (a case-4 plan can leave a case-2 one), then as
  above.
"""
import itertools

import numpy as np
import pytest
import torch

import local_shard_gemm_amd as sm
from oracle import planner, reference as ref
import workloads as wl

from hip_cases import DEV, f32_bits_equal, say

pytestmark = pytest.mark.gpu

AXES = "XYZ"


def _spec_text(dims):
    def one(d):
        if not d:
            return "None"
        if len(d) == 1:
            return f"'{d[0]}'"
        return "(" + ", ".join(f"'{a}'" for a in d) + ")"
    return f"P({one(dims[0])}, {one(dims[1])})"


def _random_case(seed):
    rng = np.random.default_rng(7000 + seed)
    while True:
        n_axes = int(rng.integers(1, 4))
        sizes = [int(rng.choice([1, 2, 2, 3, 4])) for _ in range(n_axes)]
        if int(np.prod(sizes)) <= 8:
            break
    mesh = {AXES[a]: sizes[a] for a in range(n_axes)}

    def assign():
        dims = ([], [])
        for a in rng.permutation(n_axes):
            slot = int(rng.integers(0, 3))
            if slot < 2:
                dims[slot].append(AXES[a])
        return dims

    a_dims = assign()
    b_dims = assign()
    if rng.random() < 0.6:  # mostly matching J shardings, so that most plans are legal
        b_dims = (list(a_dims[1]), [x for x in b_dims[1] if x not in a_dims[1]])
    prod = lambda d: int(np.prod([mesh[x] for x in d])) if d else 1  # noqa: E731
    pj = int(np.lcm(prod(a_dims[1]), prod(b_dims[0])))
    I = prod(a_dims[0]) * int(rng.integers(1, 161))
    J = pj * int(rng.integers(1, 97))
    K = prod(b_dims[1]) * int(rng.integers(1, 161))
    return mesh, _spec_text(a_dims), _spec_text(b_dims), I, J, K


def _global(rows, cols, dtype, fill=float("nan")):
    """Device buffer [rows, ld] with ld padded to 16 bytes, NaN-filled."""
    q = 8 if dtype == torch.bfloat16 else 4
    ld = -(-cols // q) * q
    return torch.full((rows, ld), fill, dtype=dtype, device=DEV)


def _place(X):
    """X (CPU bf16 [rows, cols]) in a padded device buffer whose padding
    holds NaN: no byte past a view's columns may reach a stored result."""
    t = _global(X.shape[0], X.shape[1], X.dtype)
    t[:, :X.shape[1]] = X.to(DEV)
    return t


def _stacked(blocks, rows, cols, dtype, fill=float("nan")):
    q = 8 if dtype == torch.bfloat16 else 4
    ld = -(-cols // q) * q
    return torch.full((blocks, rows, ld), fill, dtype=dtype, device=DEV)


def _operand_blocks(X, grid, rows, cols):
    """Stacked padded blocks of a global operand, block id = row_block * grid[1] + col_block."""
    out = _stacked(grid[0] * grid[1], rows, cols, torch.bfloat16)
    for i, j in itertools.product(range(grid[0]), range(grid[1])):
        out[i * grid[1] + j, :, :cols] = X[i * rows:(i + 1) * rows, j * cols:(j + 1) * cols].to(DEV)
    return out


def _check_products(p, q, A, B, Ad, Bd, dense):
    """Cases 1 and 3 on device operands Ad, Bd (global, padded)."""
    I, K = dense.shape
    m, n = p.c_local
    P = _stacked(p.n_units, m, n, torch.float32)
    sm.sm_local_gemm(p, sm.buf(Ad), sm.buf(Bd), sm.buf(P))
    torch.cuda.synchronize()
    Pn = P[:, :, :n].cpu().numpy()
    for u in range(p.n_units):
        assert f32_bits_equal(Pn[u], ref.unit_partial(q, A, B, u)), ("unit", u)
    if p.kase == sm.SM_CASE1:
        C = _global(I, K, torch.float32)
        sm.sm_gather_shards(p, sm.SM_WHAT_C_BLOCKS, sm.buf(P), sm.buf(C))
        torch.cuda.synchronize()
        assert f32_bits_equal(C[:, :K].cpu().numpy(), dense)
        return
    assert p.kase == sm.SM_CASE3
    N = p.n_partials
    modes = [sm.SM_ALLREDUCE] + ([sm.SM_REDUCESCATTER] if m % N == 0 else [])
    for mode in modes:
        C = _global(I, K, torch.float32)
        sm.sm_reduce_partials(p, sm.buf(P), sm.buf(C), mode)
        nbytes = sm.sm_gemm_reduce_workspace(p)
        ws = torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device=DEV) if nbytes else None
        F = _global(I, K, torch.float32)
        sm.sm_local_gemm_reduce_ws(p, sm.buf(Ad), sm.buf(Bd), sm.buf(F), ws, mode)
        torch.cuda.synchronize()
        assert f32_bits_equal(C[:, :K].cpu().numpy(), dense), ("reduce", mode)
        assert f32_bits_equal(F[:, :K].cpu().numpy(), dense), ("fused ws", mode)
        if m > 64:
            S = _global(I, K, torch.float32)
            sm.sm_local_gemm_reduce(p, sm.buf(Ad), sm.buf(Bd), sm.buf(S), mode)
            torch.cuda.synchronize()
            assert f32_bits_equal(S[:, :K].cpu().numpy(), dense), ("fused", mode)


@pytest.mark.parametrize("seed", range(128))
def test_random_plans_bitexact(seed):
    mesh, sa, sb, I, J, K = _random_case(seed)
    say("case: sweep", seed, mesh, sa, sb, I, J, K)
    try:
        p = sm.sm_plan(mesh, sa, sb, I, J, K)
    except sm.ShardmmError as e:
        # refused plans are covered on the CPU (planner brute force); the
        # oracle planner must refuse it too
        with pytest.raises(planner.PlanError):
            planner.plan(mesh, sa, sb, I, J, K)
        say("refused", e.name)
        return
    q = planner.plan(mesh, sa, sb, I, J, K)
    assert p.kase == q.case
    A = wl.random_ints((I, J), 9100 + seed)
    B = wl.random_ints((J, K), 9200 + seed)
    dense = ref.dense(A, B)
    Ad, Bd = _place(A), _place(B)
    while p.kase in (sm.SM_CASE2, sm.SM_CASE4):
        # a case-4 plan can leave a case-2 one (J still sharded on one side)
        assert (p.gather_operand == 0) == (q.gather_operand == "A")
        which = sm.SM_WHAT_A if p.gather_operand == 0 else sm.SM_WHAT_B
        if which == sm.SM_WHAT_A:
            shards = _operand_blocks(A, tuple(p.a_grid), *p.a_local)
            Ag = _global(I, J, torch.bfloat16)
            sm.sm_gather_shards(p, which, sm.buf(shards), sm.buf(Ag))
            Ad = Ag
        else:
            shards = _operand_blocks(B, tuple(p.b_grid), *p.b_local)
            Bg = _global(J, K, torch.bfloat16)
            sm.sm_gather_shards(p, which, sm.buf(shards), sm.buf(Bg))
            Bd = Bg
        torch.cuda.synchronize()
        assert torch.equal(Ad[:, :J].cpu(), A) and torch.equal(Bd[:, :K].cpu(), B)
        try:
            p = sm.sm_plan_gathered(p)
        except sm.ShardmmError as e:
            # e.g. a case-4 plan whose J shardings still differ once its
            # I/K conflict is gathered: the oracle planner refuses it too
            with pytest.raises(planner.PlanError):
                planner.gathered(q)
            say("re-plan refused", e.name)
            return
        q = planner.gathered(q)
        assert p.kase == q.case
    _check_products(p, q, A, B, Ad, Bd, dense)


def _random_reshard(seed):
    rng = np.random.default_rng(8000 + seed)
    while True:
        n_axes = int(rng.integers(1, 4))
        sizes = [int(rng.choice([1, 2, 2, 3, 4])) for _ in range(n_axes)]
        if int(np.prod(sizes)) <= 12:
            break
    mesh = {AXES[a]: sizes[a] for a in range(n_axes)}

    def assign():
        dims = ([], [])
        for a in rng.permutation(n_axes):
            slot = int(rng.integers(0, 3))
            if slot < 2:
                dims[slot].append(AXES[a])
        return dims

    frm, to = assign(), assign()
    prod = lambda d: int(np.prod([mesh[x] for x in d])) if d else 1  # noqa: E731
    rows = int(np.lcm(prod(frm[0]), prod(to[0]))) * int(rng.integers(1, 41))
    cols = 8 * int(np.lcm(prod(frm[1]), prod(to[1]))) * int(rng.integers(1, 17))
    dtype = sm.SM_BF16 if rng.random() < 0.5 else sm.SM_F32
    return mesh, _spec_text(frm), _spec_text(to), rows, cols, dtype


@pytest.mark.parametrize("seed", range(48))
def test_random_reshards_bitexact(seed):
    """sm_reshard between random specs on random meshes (learntpu.dev ch05,
    "The four collectives and their cost": all-to-all, all-gather, slicing),
    stacked blocks in and out, bit for bit the oracle's blocks; the global
    source layout gives the same blocks."""
    mesh, frm, to, R, Cc, dtype = _random_reshard(seed)
    say("case: reshard sweep", seed, mesh, frm, to, R, Cc, dtype)
    tdt = torch.bfloat16 if dtype == sm.SM_BF16 else torch.float32
    X = wl.random_normal((R, Cc), 8500 + seed)
    if dtype == sm.SM_F32:
        X = X.float()
    stored = ref.stored(X)[0]
    src_blocks = ref.shard(stored, mesh, frm)
    want = ref.reshard(src_blocks, mesh, frm, to, R, Cc)
    src_np = np.stack([src_blocks[b] for b in sorted(src_blocks)])
    src = torch.from_numpy(src_np)
    src = (src.view(torch.bfloat16) if dtype == sm.SM_BF16 else src).to(DEV)
    nb = len(want)
    br, bc = next(iter(want.values())).shape
    full = torch.full((nb * br * bc + 256,), 7, dtype=tdt, device=DEV)
    dst = full[:nb * br * bc].view(nb, br, bc)
    sm.sm_reshard(mesh, frm, to, R, Cc, dtype, sm.buf(src), sm.buf(dst))
    dst2 = torch.empty_like(dst)
    sm.sm_reshard(mesh, frm, to, R, Cc, dtype, sm.buf(X.to(DEV), block_stride=0), sm.buf(dst2))
    torch.cuda.synchronize()
    got = ref.stored(dst.cpu())[0]
    for b in range(nb):
        np.testing.assert_array_equal(got[b], want[b])
    assert bool((full[nb * br * bc:] == 7).all())
    assert torch.equal(dst2, dst)


LN_TOL_INT = 1e-5  # exact pre-norm sums; float32 mean, variance and scaling


@pytest.mark.parametrize("seed", range(24))
def test_random_sp_tails(seed):
    """sm_reduce_scatter_layernorm (ana-alekseeva.com "Sequence parallelism":
    reduce-scatter, per-token layer norm on the owned rows, all-gather) on
    random case-3 plans with whole output rows, with and without gamma/beta,
    against the oracle's tail on the oracle's partials (integer inputs: the
    sums are exact, the norm is compared within 1e-5); the stacked output
    gathered equals the global one bit for bit."""
    rng = np.random.default_rng(8800 + seed)
    while True:
        n_axes = int(rng.integers(1, 4))
        sizes = [int(rng.choice([1, 2, 2, 3, 4])) for _ in range(n_axes)]
        if int(np.prod(sizes)) <= 8:
            break
    mesh = {AXES[a]: sizes[a] for a in range(n_axes)}
    i_ax, j_ax = [], []
    for a in rng.permutation(n_axes):
        (i_ax if rng.random() < 0.4 else j_ax).append(AXES[a])
    if not j_ax:
        j_ax, i_ax = i_ax[-1:], i_ax[:-1]
    prod = lambda d: int(np.prod([mesh[x] for x in d])) if d else 1  # noqa: E731
    N = prod(j_ax)
    I = prod(i_ax) * N * int(rng.integers(1, 41))
    J = N * int(rng.integers(1, 65))
    K = 4 * int(rng.integers(1, 300))
    sa, sb = _spec_text((i_ax, j_ax)), _spec_text((j_ax, []))
    say("case: sp tail sweep", seed, mesh, sa, sb, I, J, K)
    p = sm.sm_plan(mesh, sa, sb, I, J, K)
    q = planner.plan(mesh, sa, sb, I, J, K)
    assert p.kase == q.case == sm.SM_CASE3 and p.c_grid[1] == 1
    A = wl.random_ints((I, J), 8900 + seed)
    B = wl.random_ints((J, K), 8950 + seed)
    Ad, Bd = _place(A), _place(B)
    m, n = p.c_local
    P = _stacked(p.n_units, m, n, torch.float32)
    sm.sm_local_gemm(p, sm.buf(Ad), sm.buf(Bd), sm.buf(P))
    parts = [ref.unit_partial(q, A, B, u) for u in range(q.n_units)]
    gamma = rng.standard_normal(K).astype(np.float32)
    beta = rng.standard_normal(K).astype(np.float32)
    for g_, b_ in ((None, None), (gamma, beta)):
        gd = None if g_ is None else torch.from_numpy(g_).to(DEV)
        bd = None if b_ is None else torch.from_numpy(b_).to(DEV)
        out = torch.full((I, K), float("nan"), device=DEV)
        sm.sm_reduce_scatter_layernorm(p, sm.buf(P), sm.buf(out), gd, bd, 1e-5)
        st = torch.full((p.n_groups * p.n_partials, m // p.n_partials, K), float("nan"), device=DEV)
        sm.sm_reduce_scatter_layernorm(p, sm.buf(P), sm.buf(st), gd, bd, 1e-5)
        ag = torch.full((I, K), float("nan"), device=DEV)
        sm.sm_gather_shards(p, sm.SM_WHAT_C_SCATTERED, sm.buf(st), sm.buf(ag))
        torch.cuda.synchronize()
        want = ref.sp_tail(q, parts, g_, b_, 1e-5)
        err = ref.rel_frobenius(out.cpu().numpy(), want)
        assert err <= LN_TOL_INT, err
        assert torch.equal(ag, out)


@pytest.mark.parametrize("seed", range(32))
def test_random_gelu_epilogues(seed):
    """The GeLU(tanh) -> bfloat16 epilogue (ana-alekseeva.com "MLP block":
    GeLU applies to each column block of the first layer) on random case-1
    plans (random meshes, A sharded on I or not, B on K, ragged sizes, row
    padding holding NaN): every unit's stacked bfloat16 block within the
    derived bound of the oracle's round_bf16(gelu(A_u B_u)), and fewer than
    1 % of its elements differ at all."""
    from hip_cases import gelu_h_within_bound

    rng = np.random.default_rng(9300 + seed)
    while True:
        n_axes = int(rng.integers(1, 4))
        sizes = [int(rng.choice([1, 2, 2, 3, 4])) for _ in range(n_axes)]
        if int(np.prod(sizes)) <= 8:
            break
    mesh = {AXES[a]: sizes[a] for a in range(n_axes)}
    i_ax, k_ax = [], []
    for a in rng.permutation(n_axes):
        slot = int(rng.integers(0, 3))
        if slot == 0:
            i_ax.append(AXES[a])
        elif slot == 1:
            k_ax.append(AXES[a])
    prod = lambda d: int(np.prod([mesh[x] for x in d])) if d else 1  # noqa: E731
    I = prod(i_ax) * int(rng.integers(1, 161))
    J = int(rng.integers(1, 200))
    K = prod(k_ax) * int(rng.integers(1, 161))
    sa, sb = _spec_text((i_ax, [])), _spec_text(([], k_ax))
    say("case: gelu sweep", seed, mesh, sa, sb, I, J, K)
    p = sm.sm_plan(mesh, sa, sb, I, J, K, out_dtype=sm.SM_BF16)
    q = planner.plan(mesh, sa, sb, I, J, K)
    assert p.kase == q.case == sm.SM_CASE1
    X = wl.random_normal((I, J), 9400 + seed)
    W = wl.random_normal((J, K), 9450 + seed, 0.1)
    m, n = p.c_local
    H = _stacked(p.n_units, m, n, torch.bfloat16)
    sm.sm_local_gemm(p, sm.buf(_place(X)), sm.buf(_place(W)), sm.buf(H), sm.SM_EPI_GELU_TANH)
    torch.cuda.synchronize()
    Hg = H[:, :, :n].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    absdot = ref.matmul(np.abs(ref.widen(X)), np.abs(ref.widen(W)))
    for u in range(p.n_units):
        want = ref.round_bf16(ref.gelu_tanh(ref.unit_partial(q, X, W, u)))
        r0, c0, _, _ = q.unit_views(u)["C"]
        ok = gelu_h_within_bound(Hg[u], want, absdot[r0:r0 + m, c0:c0 + n], J)
        assert ok.all(), (u, int((~ok).sum()))
        assert (Hg[u] != want).mean() < 0.01, u
