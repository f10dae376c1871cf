"""GPU parity of the skinny split-J path with its fused rank-ordered reduce
(sm_local_gemm_reduce_ws): each rank forms Z_i = X_i A_i and the output is
Y = sum_i X_i A_i (mbrenndoerfer.com "Row Parallelism"), summed in rank
order inside the split-J kernel by the workgroup that finishes a column
block last. Checked through the C ABI against the fp64 oracle: bit for bit
on integer-valued inputs, within the float tolerance on random bfloat16."""
import numpy as np
import pytest
import torch

import local_shard_gemm_amd as sm
import workloads as wl
from oracle import planner, reference as ref

from hip_cases import DEV, FREIVALDS_FLOAT_TOL, REL_TOL, f32_bits_equal, guard_intact, guarded, run_partials, say, to_dev

pytestmark = pytest.mark.gpu


def _workspace(p, group_count=None):
    nbytes = sm.sm_gemm_reduce_workspace(p, group_count)
    return torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device=DEV)


def _ws_layout(p, ws, group_count):
    """(counters, partials) views of a workspace: 32-bit counters for every
    (group, 256-column block), then the partials [group_count * N, m, ldp]."""
    m, n = p.c_local
    ncb = -(-n // 256)
    cbytes = -(-(group_count * ncb * 4) // 256) * 256
    ldp = -(-n // 4) * 4
    counters = ws[:group_count * ncb]
    parts = ws[cbytes // 4:cbytes // 4 + group_count * p.n_partials * m * ldp].view(torch.float32)
    return counters, parts.view(group_count * p.n_partials, m, ldp)[:, :, :n]


CASES = [
    ({"T": 8}, "P(None, 'T')", "P('T', None)", 16, 8 * 512, 1024),       # eight partials, four column blocks
    ({"T": 4}, "P(None, 'T')", "P('T', None)", 5, 4 * 100, 296),        # ragged K (not a multiple of 16) and N
    ({"T": 2}, "P(None, 'T')", "P('T', None)", 64, 2 * 256, 512),       # two 32-row blocks
    ({"T": 16}, "P(None, 'T')", "P('T', None)", 32, 16 * 64, 256),      # sixteen partials, one column block
    ({"X": 2, "T": 4}, "P('X', 'T')", "P('T', None)", 2 * 24, 4 * 128, 512),  # two groups; RS blocks of 6 rows
    ({"X": 3, "T": 32}, "P('X', 'T')", "P('T', None)", 3 * 8, 32 * 32, 264),  # 32 partials: two launches
    ({"T": 1}, "P(None, 'T')", "P('T', None)", 16, 64, 256),            # one partial (axis of size 1)
    ({"T": 2, "Z": 4}, "P(None, 'T')", "P('T', 'Z')", 12, 2 * 64, 4 * 138),  # 138-column blocks: element path
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[3]}x{c[4]}x{c[5]}-{'x'.join(map(str, c[0].values()))}")
@pytest.mark.parametrize("mode", [sm.SM_ALLREDUCE, sm.SM_REDUCESCATTER], ids=["AR", "RS"])
def test_skinny_fused_reduce_bitexact(case, mode):
    mesh, sa, sb, I, J, K = case
    say("case: skinny fused", case, mode)
    A = wl.random_ints((I, J), 801 + J)
    B = wl.random_ints((J, K), 802 + K)
    p = sm.sm_plan(mesh, sa, sb, I, J, K)
    q = planner.plan(mesh, sa, sb, I, J, K)
    m, n = q.c_local
    N, G = q.n_partials, q.n_groups
    assert p.kase == sm.SM_CASE3 and m <= 64
    if mode == sm.SM_REDUCESCATTER and m % N:
        with pytest.raises(sm.ShardmmError) as ei:
            sm.sm_local_gemm_reduce_ws(p, sm.buf(to_dev(A)), sm.buf(to_dev(B)),
                                       sm.buf(torch.empty(I, K, device=DEV)), _workspace(p), mode)
        assert ei.value.status == sm.SM_ERR_INDIVISIBLE
        return
    Ad, Bd = to_dev(A), to_dev(B)
    parts = [ref.unit_partial(q, A, B, u) for u in range(q.n_units)]
    ws = _workspace(p)
    # global layout
    fg, g = guarded((I, K), torch.float32)
    sm.sm_local_gemm_reduce_ws(p, sm.buf(Ad), sm.buf(Bd), sm.buf(g), ws, mode)
    torch.cuda.synchronize()
    assert f32_bits_equal(g.cpu().numpy(), ref.gather(q, ref.allreduce(q, parts)))
    assert guard_intact(fg, g.numel())
    counters, wparts = _ws_layout(p, ws, G)
    assert int(counters.abs().sum().item()) == 0  # every counter back at zero
    wp = wparts.cpu().numpy()
    for u in range(q.n_units):  # the materialised partials are the oracle's, bit for bit
        assert f32_bits_equal(wp[u], parts[u]), u
    # stacked layout with a padded block stride, the same workspace again
    blocks, rows = (G, m) if mode == sm.SM_ALLREDUCE else (G * N, m // N)
    ld = -(-n // 4) * 4  # float32 rows start on 16 bytes
    stride = (rows + 3) * ld
    fs = torch.full((blocks * stride + 64,), float("nan"), device=DEV)
    s = sm.sm_buf(fs.data_ptr(), ld, stride, fs.numel(), sm.SM_F32, 0)
    sm.sm_local_gemm_reduce_ws(p, sm.buf(Ad), sm.buf(Bd), s, ws, mode)
    fsn = fs.cpu().numpy()
    if mode == sm.SM_ALLREDUCE:
        sums = ref.allreduce(q, parts)
        for gi in range(G):
            blk = fsn[gi * stride:gi * stride + m * ld].reshape(m, ld)[:, :n]
            assert f32_bits_equal(np.ascontiguousarray(blk), sums[gi]), gi
    else:
        for (gi, y), want in ref.reduce_scatter(q, parts).items():
            o = (gi * N + y) * stride
            blk = fsn[o:o + rows * ld].reshape(rows, ld)[:, :n]
            assert f32_bits_equal(np.ascontiguousarray(blk), want), (gi, y)
    written = np.zeros(fsn.shape, dtype=bool)
    for b in range(blocks):
        for r in range(rows):
            written[b * stride + r * ld:b * stride + r * ld + n] = True
    assert np.isnan(fsn[~written]).all()  # nothing written between rows or blocks
    assert int(counters.abs().sum().item()) == 0


def test_skinny_fused_reduce_group_subset_and_errors():
    """A call over a subset of groups writes only those groups; errors are
    raised on the host before anything is launched."""
    mesh, sa, sb, I, J, K = {"X": 2, "T": 4}, "P('X', 'T')", "P('T', None)", 2 * 24, 4 * 128, 512
    say("case: skinny fused subset")
    A = wl.random_ints((I, J), 811)
    B = wl.random_ints((J, K), 812)
    p = sm.sm_plan(mesh, sa, sb, I, J, K)
    q = planner.plan(mesh, sa, sb, I, J, K)
    Ad, Bd = to_dev(A), to_dev(B)
    parts = [ref.unit_partial(q, A, B, u) for u in range(q.n_units)]
    ws = _workspace(p, 1)
    out = torch.full((1, 24, K), float("nan"), device=DEV)
    sm.sm_local_gemm_reduce_ws(p, sm.buf(Ad), sm.buf(Bd), sm.buf(out), ws, sm.SM_ALLREDUCE, 1, 1)
    assert f32_bits_equal(out[0].cpu().numpy(), ref.allreduce(q, parts)[1])
    # too small a workspace, a misaligned one, and a missing one
    small = torch.zeros(ws.numel() - 64, dtype=torch.int32, device=DEV)
    for wsx, status in ((small, sm.SM_ERR_SHAPE), (ws[1:], sm.SM_ERR_ALIGN), (None, sm.SM_ERR_ARG)):
        with pytest.raises(sm.ShardmmError) as ei:
            sm.sm_local_gemm_reduce_ws(p, sm.buf(Ad), sm.buf(Bd), sm.buf(out), wsx, sm.SM_ALLREDUCE, 1, 1)
        assert ei.value.status == status, ei.value
    with pytest.raises(sm.ShardmmError) as ei:
        sm.sm_local_gemm_reduce(p, sm.buf(Ad), sm.buf(Bd), sm.buf(out), sm.SM_ALLREDUCE, 1, 1)
    assert ei.value.status == sm.SM_ERR_SHAPE


@pytest.mark.parametrize("integer", [True, False], ids=["int", "float"])
def test_full_skinny_fused_reduce(integer):
    """The skinny workload at full size (X[16,28672] . A[28672,8192], J
    split 8 ways): the fused kernel's all-reduce and reduce-scatter against
    the oracle (bit for bit on integers, within tolerance on floats), equal
    bit for bit to the split-J GEMM + sm_reduce_partials (the same rank-order
    sums), and bit for bit the same on a second run."""
    w = wl.get("skinny")
    if integer:
        w = wl.int_variant(w)
    say("case: full skinny fused", "int" if integer else "float")
    X = wl.make_operand(w.operand("X"))
    A = wl.make_operand(w.operand("A"))
    I, J = X.shape
    K = A.shape[1]
    p = sm.sm_plan(dict(w.mesh), w.operand("X").spec, w.operand("A").spec, I, J, K)
    q = planner.plan(dict(w.mesh), w.operand("X").spec, w.operand("A").spec, I, J, K)
    Xd, Ad = to_dev(X), to_dev(A)
    ws = _workspace(p)
    outs = {}
    for mode in (sm.SM_ALLREDUCE, sm.SM_REDUCESCATTER):
        fo, o = guarded((I, K), torch.float32)
        sm.sm_local_gemm_reduce_ws(p, sm.buf(Xd), sm.buf(Ad), sm.buf(o), ws, mode)
        o2 = torch.empty(I, K, device=DEV)
        sm.sm_local_gemm_reduce_ws(p, sm.buf(Xd), sm.buf(Ad), sm.buf(o2), ws, mode)
        torch.cuda.synchronize()
        assert guard_intact(fo, o.numel())
        assert torch.equal(o, o2)  # deterministic
        outs[mode] = o
    assert torch.equal(outs[sm.SM_ALLREDUCE], outs[sm.SM_REDUCESCATTER])
    _, P = run_partials(p, Xd, Ad)
    two = torch.empty(I, K, device=DEV)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(two), sm.SM_ALLREDUCE)
    assert torch.equal(outs[sm.SM_ALLREDUCE], two)
    parts = ref.partials(q, X, A)
    (s,) = ref.allreduce(q, parts)
    got = outs[sm.SM_ALLREDUCE].cpu().numpy()
    if integer:
        assert f32_bits_equal(got, s)
    else:
        err = ref.rel_frobenius(got, s)
        say("skinny fused rel err", err)
        assert err <= REL_TOL


# ------------------------------------------- taller products with few tiles

FEW_TILES = [
    ({"T": 8}, "P(None, 'T')", "P('T', None)", 128, 8 * 256, 1024),        # 4 tiles of 128 rows
    ({"X": 2, "T": 4}, "P('X', 'T')", "P('T', None)", 2 * 96, 4 * 100, 296),  # two groups, ragged K and N
    ({"T": 2}, "P(None, 'T')", "P('T', None)", 65, 2 * 64, 512),          # one ragged row tile
    ({"T": 4}, "P(None, 'T')", "P('T', None)", 300, 4 * 64, 256),          # 256-row tiles, ragged
]


@pytest.mark.parametrize("case", FEW_TILES, ids=lambda c: f"{c[3]}x{c[4]}x{c[5]}")
@pytest.mark.parametrize("mode", [sm.SM_ALLREDUCE, sm.SM_REDUCESCATTER], ids=["AR", "RS"])
def test_few_tile_products_reduce_through_the_workspace(case, mode):
    """Local products taller than 64 rows whose single launch over the whole
    J would have few tiles: with a workspace, the units' products and their
    rank-ordered sum (two launches), bit for bit the oracle's rank-order sums
    on integers and bit for bit sm_local_gemm + sm_reduce_partials; without
    one, the single launch, also exact on integers."""
    mesh, sa, sb, I, J, K = case
    say("case: few-tile fused", case, mode)
    A = wl.random_ints((I, J), 821 + I)
    B = wl.random_ints((J, K), 822 + K)
    p = sm.sm_plan(mesh, sa, sb, I, J, K)
    q = planner.plan(mesh, sa, sb, I, J, K)
    m, n = q.c_local
    N = q.n_partials
    if mode == sm.SM_REDUCESCATTER and m % N:
        return
    nbytes = sm.sm_gemm_reduce_workspace(p)
    assert nbytes == q.n_groups * N * m * (-(-n // 4) * 4) * 4
    Ad, Bd = to_dev(A), to_dev(B)
    ws = torch.full((nbytes // 4,), float("nan"), device=DEV)
    fg, g = guarded((I, K), torch.float32)
    sm.sm_local_gemm_reduce_ws(p, sm.buf(Ad), sm.buf(Bd), sm.buf(g), ws, mode)
    one = torch.full((I, K), float("nan"), device=DEV)
    sm.sm_local_gemm_reduce_ws(p, sm.buf(Ad), sm.buf(Bd), sm.buf(one), None, mode)
    _, P = run_partials(p, Ad, Bd)
    two = torch.empty(I, K, device=DEV)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(two), mode)
    torch.cuda.synchronize()
    parts = [ref.unit_partial(q, A, B, u) for u in range(q.n_units)]
    want = ref.gather(q, ref.allreduce(q, parts))
    assert f32_bits_equal(g.cpu().numpy(), want)
    assert guard_intact(fg, g.numel())
    assert torch.equal(g, two)
    assert f32_bits_equal(one.cpu().numpy(), want)


def test_full_medium_batch_fused_reduce():
    """A 128-row batch on the skinny workload's weights (float): the
    workspace call runs the 8 units' products and their rank-ordered sum,
    bit for bit sm_local_gemm + sm_reduce_partials; sampled rows within the
    float tolerance of the oracle's rank-order sums, the whole output by
    Freivalds' test; the single launch (no workspace) within the same
    bounds."""
    w = wl.get("skinny")
    say("case: full medium fused")
    X = wl.make_operand(w.operand("X"), shape=(128, 28672))
    A = wl.make_operand(w.operand("A"))
    args = (dict(w.mesh), w.operand("X").spec, w.operand("A").spec, 128, 28672, 8192)
    p, q = sm.sm_plan(*args), planner.plan(*args)
    Xd, Ad = to_dev(X), to_dev(A)
    ws = torch.empty(sm.sm_gemm_reduce_workspace(p) // 4, device=DEV)
    out = torch.empty(128, 8192, device=DEV)
    sm.sm_local_gemm_reduce_ws(p, sm.buf(Xd), sm.buf(Ad), sm.buf(out), ws, sm.SM_ALLREDUCE)
    _, P = run_partials(p, Xd, Ad)
    two = torch.empty(128, 8192, device=DEV)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(two), sm.SM_ALLREDUCE)
    one = torch.empty(128, 8192, device=DEV)
    sm.sm_local_gemm_reduce(p, sm.buf(Xd), sm.buf(Ad), sm.buf(one), sm.SM_ALLREDUCE)
    torch.cuda.synchronize()
    assert torch.equal(out, two)
    rows = [0, 1, 63, 64, 127]
    (s,) = ref.allreduce(q, [ref.unit_partial(q, X, A, u, rows=rows) for u in range(q.n_units)])
    for name, got in (("workspace", out), ("single launch", one)):
        g = got.cpu().numpy()
        err = ref.rel_frobenius(g[rows], s)
        fr = ref.freivalds(X, (0, 0, 128, 28672), A, (0, 0, 28672, 8192), g, trials=1, ints=False)
        say("medium fused", name, "rows rel err", err, "freivalds", fr)
        assert err <= REL_TOL and fr <= FREIVALDS_FLOAT_TOL


@pytest.mark.parametrize("mode", [sm.SM_ALLREDUCE, sm.SM_REDUCESCATTER], ids=["AR", "RS"])
def test_few_tile_products_stacked_subsets_and_fallback(mode):
    """The few-tile two-launch path with stacked outputs and a subset of the
    groups (group 1 of 2, then both), bit for bit the oracle's rank-order
    sums on integers; a workspace one word short of the partials falls back
    to the single launch, bit for bit sm_local_gemm_reduce."""
    mesh, sa, sb, I, J, K = {"X": 2, "T": 4}, "P('X', 'T')", "P('T', None)", 2 * 96, 4 * 100, 296
    say("case: few-tile stacked/subset", mode)
    A = wl.random_ints((I, J), 831)
    B = wl.random_ints((J, K), 832)
    p = sm.sm_plan(mesh, sa, sb, I, J, K)
    q = planner.plan(mesh, sa, sb, I, J, K)
    m, n = q.c_local
    N, G = q.n_partials, q.n_groups
    Ad, Bd = to_dev(A), to_dev(B)
    parts = [ref.unit_partial(q, A, B, u) for u in range(q.n_units)]
    sums = ref.allreduce(q, parts)
    rs = mode == sm.SM_REDUCESCATTER
    orows = m // N if rs else m
    nblk = N if rs else 1
    for g0, gc in ((1, 1), (0, 2)):
        nbytes = sm.sm_gemm_reduce_workspace(p, gc)
        assert nbytes == gc * N * m * 296 * 4
        ws = torch.full((nbytes // 4,), float("nan"), device=DEV)
        fs, st = guarded((gc * nblk, orows, n), torch.float32)
        sm.sm_local_gemm_reduce_ws(p, sm.buf(Ad), sm.buf(Bd), sm.buf(st, block_stride=orows * n), ws, mode, g0, gc)
        torch.cuda.synchronize()
        assert guard_intact(fs, st.numel())
        got = st.cpu().numpy()
        for i, g in enumerate(range(g0, g0 + gc)):
            for y in range(nblk):
                want = sums[g][y * orows:(y + 1) * orows]
                assert f32_bits_equal(got[i * nblk + y], want), (g, y)
    # fallback: a workspace too small for the partials
    nbytes = sm.sm_gemm_reduce_workspace(p)
    small = torch.empty(nbytes // 4 - 1, device=DEV)
    a = torch.full((I, K), float("nan"), device=DEV)
    sm.sm_local_gemm_reduce_ws(p, sm.buf(Ad), sm.buf(Bd), sm.buf(a), small, mode)
    b = torch.full((I, K), float("nan"), device=DEV)
    sm.sm_local_gemm_reduce(p, sm.buf(Ad), sm.buf(Bd), sm.buf(b), mode)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert f32_bits_equal(a.cpu().numpy(), ref.gather(q, sums))
