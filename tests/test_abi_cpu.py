"""C-ABI library checks that need no GPU: symbols, plan layout, the host
planner against the oracle's independent planner, and argument validation
(every check runs before any HIP call, so no device is touched)."""
import ctypes
import itertools
import os
import re

import pytest

import local_shard_gemm_amd as sm
from oracle import planner as ref_planner

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "shardmm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sm_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = sm.load()
    names = _declared_functions()
    assert "sm_plan" in names and "sm_local_gemm" in names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(sm.EXPORTED)


def test_plan_struct_layout_matches():
    lib = sm.load()
    assert lib.sm_plan_size() == ctypes.sizeof(sm.sm_plan_t)
    assert lib.sm_abi_version() == sm.SM_ABI_VERSION


def test_status_strings():
    assert sm.sm_status_str(sm.SM_ERR_UNREDUCED) == "SM_ERR_UNREDUCED"
    assert sm.sm_status_str(0) == "SM_OK"


# ---------------------------------------------------------- spec parsing

@pytest.mark.parametrize("text,dims", [
    ("P('X', 'Y')", ((0,), (1,))),
    ("P(('X', 'Y'), None)", ((0, 1), ())),
    ("P(None, None)", ((), ())),
    ("P()", ((), ())),
    ("('X','Y'), None", ((0, 1), ())),
    ("P('Y', None)", ((1,), ())),
    ("A[I_X, J_Y]", ((0,), (1,))),
    ("A[I_XY, J]", ((0, 1), ())),
    ("I, J_Y", ((), (1,))),
    ("", ((), ())),
])
def test_parse_spec_forms(text, dims):
    mesh = sm.sm_mesh_init({"X": 4, "Y": 2})
    assert sm.sm_parse_spec(mesh, text).dims() == dims
    assert ref_planner.parse_spec(text) == tuple(tuple("XY"[i] for i in d) for d in dims)


@pytest.mark.parametrize("text,code", [
    ("P('X', 'Y', 'X')", sm.SM_ERR_SPEC),
    ("P('Q', None)", sm.SM_ERR_SPEC),
    ("P('X'", sm.SM_ERR_SPEC),
    ("A[I_Q, J]", sm.SM_ERR_SPEC),
])
def test_parse_spec_errors(text, code):
    mesh = sm.sm_mesh_init({"X": 4, "Y": 2})
    with pytest.raises(sm.ShardmmError) as ei:
        sm.sm_parse_spec(mesh, text)
    assert ei.value.status == code


def test_mesh_errors():
    for axes in ({}, {"X": 0}, [("X", 2), ("X", 2)], {"A": 1, "B": 1, "C": 1, "D": 1, "E": 1}, {"TOOLONGNAME": 2}):
        with pytest.raises(sm.ShardmmError) as ei:
            sm.sm_mesh_init(axes)
        assert ei.value.status == sm.SM_ERR_MESH


# ------------------------------------------- planner vs reference planner

_CODE = {
    "SPEC": sm.SM_ERR_SPEC, "AXIS_REUSED": sm.SM_ERR_AXIS_REUSED, "INDIVISIBLE": sm.SM_ERR_INDIVISIBLE,
    "J_MISMATCH": sm.SM_ERR_J_MISMATCH, "SHAPE": sm.SM_ERR_SHAPE, "MESH": sm.SM_ERR_MESH,
}


def _all_specs(names):
    """Every 2-D spec over the mesh axes with ordered axis lists (len <= 2 per dim)."""
    lists = [()]
    for k in (1, 2):
        lists += list(itertools.permutations(names, k))
    for d0 in lists:
        for d1 in lists:
            yield (tuple(d0), tuple(d1))


def _to_c_spec(spec, names):
    s = sm.sm_spec()
    for d in range(2):
        s.n[d] = len(spec[d])
        for k, a in enumerate(spec[d]):
            s.axes[d][k] = names.index(a)
    return s


def _compare(mesh_axes, a, b, I, J, K):
    names = [n for n, _ in mesh_axes]
    mesh = sm.sm_mesh_init(mesh_axes)
    try:
        want = ref_planner.plan(mesh_axes, a, b, I, J, K)
        want_err = None
    except ref_planner.PlanError as e:
        want, want_err = None, e.code
    try:
        got = sm.sm_plan(mesh, _to_c_spec(a, names), _to_c_spec(b, names), I, J, K)
        got_err = None
    except sm.ShardmmError as e:
        got, got_err = None, e.status
    if want_err is not None:
        assert got_err == _CODE[want_err], (mesh_axes, a, b)
        return
    assert got_err is None, (mesh_axes, a, b, got_err)
    _compare_plans(got, want, names)
    if want.case in (2, 4):
        # the case-2/4 fix by composition: plan after gathering the operand
        try:
            want_g, want_g_err = ref_planner.gathered(want), None
        except ref_planner.PlanError as e:
            want_g, want_g_err = None, e.code
        try:
            got_g, got_g_err = sm.sm_plan_gathered(got), None
        except sm.ShardmmError as e:
            got_g, got_g_err = None, e.status
        if want_g_err is not None:
            assert got_g_err == _CODE[want_g_err], (mesh_axes, a, b)
        else:
            assert got_g_err is None, (mesh_axes, a, b, got_g_err)
            _compare_plans(got_g, want_g, names)
    else:
        with pytest.raises(sm.ShardmmError) as ei:
            sm.sm_plan_gathered(got)
        assert ei.value.status == sm.SM_ERR_CASE


def _compare_plans(got, want, names):
    assert got.kase == want.case
    assert got.n_ranks == want.n_ranks
    assert tuple(got.a_local) == want.a_local and tuple(got.b_local) == want.b_local
    assert tuple(got.c_local) == want.c_local
    assert tuple(got.a_grid) == want.a_grid and tuple(got.b_grid) == want.b_grid
    assert tuple(got.c_grid) == want.c_grid
    assert (got.a_copies, got.b_copies, got.c_copies) == (want.a_copies, want.b_copies, want.c_copies)
    assert got.n_partials == want.n_partials and got.n_groups == want.n_groups
    red = tuple(names[i] for i in range(len(names)) if got.reduce_axes >> i & 1)
    assert set(red) == set(want.unreduced)
    if want.gather_operand is None:
        assert got.gather_operand == -1
    else:
        assert got.gather_operand == "AB".index(want.gather_operand)
        assert {names[i] for i in range(len(names)) if got.gather_axes >> i & 1} == set(want.gather_axes)
    if want.case == 3:
        assert tuple(tuple(names[i] for i in d) for d in got.c_rs.dims()) == want.c_rs_spec
    for r in range(want.n_ranks):
        ri = sm.sm_rank_info(got, r)
        bl = want.rank_blocks(r)
        assert tuple(ri.a_block) == bl["A"] and tuple(ri.b_block) == bl["B"] and tuple(ri.c_block) == bl["C"]
        assert tuple(ri.coords[: len(names)]) == tuple(want.coords(r)[n] for n in names)
        if want.case in (1, 3):
            assert ri.unit == want.rank_unit(r)
            if want.case == 3 and want.c_local[0] % want.n_partials == 0:
                g, y = divmod(ri.unit, want.n_partials)
                assert (ri.rs_row0, ri.rs_rows) == want.rs_rows(g, y)
        else:
            assert ri.unit == -1


@pytest.mark.parametrize("mesh_axes", [
    [("X", 2)], [("X", 3)], [("X", 1)], [("X", 4), ("Y", 2)], [("X", 2), ("Y", 3)],
    [("X", 2), ("Y", 1), ("Z", 2)],
])
def test_planner_brute_force_against_reference(mesh_axes):
    """Every legal and illegal 2-D spec pair on small meshes: the library's
    planner and the oracle's planner agree on case, shapes, grids, copies,
    reduce axes, gather choice, rank blocks, units and RS ownership."""
    names = [n for n, _ in mesh_axes]
    specs = list(_all_specs(names))
    if len(names) == 3:
        specs = [s for s in specs if len(s[0]) + len(s[1]) <= 2]
    shapes = [(12, 12, 12), (24, 36, 12), (6, 5, 4)]
    for a in specs:
        for b in specs:
            for I, J, K in shapes[:2] if len(names) < 3 else shapes[:1]:
                _compare(mesh_axes, a, b, I, J, K)
    _compare(mesh_axes, specs[1], specs[1], *shapes[2])


@pytest.mark.parametrize("I,J,K", [(1 << 40, 1 << 40, 1 << 39), (1 << 39, 1 << 40, 1 << 40),
                                   (1 << 40, 1 << 40, 1 << 40), (2, 1 << 40, 4)])
def test_case4_extreme_shapes_match_reference(I, J, K):
    """Case 4 gathers the smaller input by bytes (I*J against J*K); at the
    largest accepted dimensions (2^40) those products reach 2^80, and the
    library's choice must still be the oracle planner's (exact integers)."""
    for mesh_axes, a, b in (([("X", 2)], ("X",), ("X",)), ([("X", 2), ("Y", 4)], ("XY",), ("XY",))):
        names = [n for n, _ in mesh_axes]
        sa = (tuple(a[0]), ())
        sb = ((), tuple(b[0]))
        _compare(mesh_axes, sa, sb, I, J, K)


def test_sandbox_default_through_the_library():
    p = sm.sm_plan({"X": 4, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 8192, 28672, 8192)
    assert p.kase == sm.SM_CASE3 and tuple(p.a_local) == (2048, 14336) and p.a_copies == 1
    assert tuple(p.a_grid) == (4, 2) and tuple(p.b_grid) == (2, 1) and p.n_ranks == 8
    assert p.n_partials == 2 and p.n_groups == 4


def test_plan_dtype_rules():
    with pytest.raises(sm.ShardmmError) as ei:
        sm.sm_plan({"X": 2}, "P(None, 'X')", "P('X', None)", 8, 8, 8, sm.SM_BF16, sm.SM_BF16)
    assert ei.value.status == sm.SM_ERR_DTYPE  # partials must stay float32
    with pytest.raises(sm.ShardmmError) as ei:
        sm.sm_plan({"X": 2}, "P()", "P()", 8, 8, 8, sm.SM_F32, sm.SM_F32)
    assert ei.value.status == sm.SM_ERR_DTYPE
    p = sm.sm_plan({"X": 2}, "P()", "P(None, 'X')", 8, 8, 8, sm.SM_BF16, sm.SM_BF16)
    assert p.kase == sm.SM_CASE1


# ------------------------------------------------ host-side validation

FAKE = 0x10000  # never dereferenced: every call below fails validation first


BF, F32 = sm.SM_BF16, sm.SM_F32


def _fb(ld, stride=0, elems=1 << 40, ptr=FAKE, dt=F32):
    return sm.sm_buf(ctypes.c_void_p(ptr), ld, stride, elems, dt, 0)


def _err(fn, *args):
    with pytest.raises(sm.ShardmmError) as ei:
        fn(*args)
    return ei.value.status


def test_local_gemm_validation():
    p3 = sm.sm_plan({"X": 2}, "P(None, 'X')", "P('X', None)", 64, 128, 64)
    p2 = sm.sm_plan({"X": 2}, "P(None, 'X')", "P()", 64, 128, 64)
    p4 = sm.sm_plan({"X": 2}, "P('X', None)", "P(None, 'X')", 64, 128, 64)
    p1 = sm.sm_plan({"X": 2}, "P('X', None)", "P()", 64, 128, 64)
    A, B = _fb(128, dt=BF), _fb(64, dt=BF)
    Cs = _fb(64, 64 * 64)
    assert _err(sm.sm_local_gemm, p2, A, B, Cs) == sm.SM_ERR_NEEDS_GATHER
    assert _err(sm.sm_local_gemm, p4, A, B, Cs) == sm.SM_ERR_NEEDS_GATHER
    assert _err(sm.sm_local_gemm, p3, A, B, _fb(64)) == sm.SM_ERR_UNREDUCED
    assert _err(sm.sm_local_gemm, p3, A, B, Cs, sm.SM_EPI_GELU_TANH) == sm.SM_ERR_CASE
    assert _err(sm.sm_local_gemm, p3, A, B, Cs, 7) == sm.SM_ERR_ARG
    assert _err(sm.sm_local_gemm, p3, A, B, Cs, 0, 1, 2) == sm.SM_ERR_ARG
    assert _err(sm.sm_local_gemm, p3, _fb(128, ptr=FAKE + 8, dt=BF), B, Cs) == sm.SM_ERR_ALIGN
    assert _err(sm.sm_local_gemm, p3, _fb(130, dt=BF), B, Cs) == sm.SM_ERR_ALIGN
    assert _err(sm.sm_local_gemm, p3, _fb(120, dt=BF), B, Cs) == sm.SM_ERR_SHAPE
    assert _err(sm.sm_local_gemm, p3, _fb(128, elems=64 * 128 - 1, dt=BF), B, Cs) == sm.SM_ERR_SHAPE
    assert _err(sm.sm_local_gemm, p3, A, B, _fb(64, 64 * 64, elems=2 * 64 * 64 - 1)) == sm.SM_ERR_SHAPE
    assert _err(sm.sm_local_gemm, p3, A, B, _fb(64, 63 * 64)) == sm.SM_ERR_SHAPE
    assert _err(sm.sm_local_gemm, p1, A, B, _fb(62)) == sm.SM_ERR_ALIGN
    assert _err(sm.sm_local_gemm, p1, A, B, _fb(60)) == sm.SM_ERR_SHAPE
    bad = sm.sm_plan_t()
    assert _err(sm.sm_local_gemm, bad, A, B, Cs) == sm.SM_ERR_ARG


def test_gathered_plan_examples():
    """lingze.zone 'Case 2': A[I,J_X].B[J,K] -> gather A -> case 1;
    'Case 4': A[I_X,J].B[J,K_X] -> gather the smaller operand -> case 1."""
    p2 = sm.sm_plan({"X": 4}, "A[I, J_X]", "B[J, K]", 64, 64, 64)
    q2 = sm.sm_plan_gathered(p2)
    assert p2.kase == sm.SM_CASE2 and q2.kase == sm.SM_CASE1 and q2.a.dims() == ((), ())
    p4 = sm.sm_plan({"X": 4}, "A[I_X, J]", "B[J, K_X]", 64, 32, 128)
    assert p4.kase == sm.SM_CASE4 and p4.gather_operand == 0  # A (64x32) smaller than B (32x128)
    q4 = sm.sm_plan_gathered(p4)
    assert q4.kase == sm.SM_CASE1 and q4.n_groups == 4
    # case 4 whose fix leaves A J-sharded: case 2 next, then case 1
    p = sm.sm_plan({"X": 2, "Y": 2}, "A[I_X, J_Y]", "B[J, K_X]", 16, 16, 32)
    q = sm.sm_plan_gathered(p)
    assert p.kase == sm.SM_CASE4 and q.kase == sm.SM_CASE2
    assert sm.sm_plan_gathered(q).kase == sm.SM_CASE1


def test_fused_reduce_validation():
    p3 = sm.sm_plan({"X": 2}, "P(None, 'X')", "P('X', None)", 160, 128, 64)
    p1 = sm.sm_plan({"X": 2}, "P('X', None)", "P()", 64, 128, 64)
    p2 = sm.sm_plan({"X": 2}, "P(None, 'X')", "P()", 64, 128, 64)
    A, B, out = _fb(128, dt=BF), _fb(64, dt=BF), _fb(64)
    assert _err(sm.sm_local_gemm_reduce, p1, A, B, out) == sm.SM_ERR_CASE
    assert _err(sm.sm_local_gemm_reduce, p2, A, B, out) == sm.SM_ERR_NEEDS_GATHER
    assert _err(sm.sm_local_gemm_reduce, p3, _fb(128, 64 * 128, dt=BF), B, out) == sm.SM_ERR_ARG
    for rows in (16, 64):  # skinny products (at most 64 rows) reduce through sm_reduce_partials
        sk = sm.sm_plan({"X": 2}, "P(None, 'X')", "P('X', None)", rows, 128, 64)
        assert _err(sm.sm_local_gemm_reduce, sk, A, B, out) == sm.SM_ERR_SHAPE
    assert _err(sm.sm_local_gemm_reduce, p3, A, B, out, 9) == sm.SM_ERR_ARG
    assert _err(sm.sm_local_gemm_reduce, p3, A, B, _fb(64, 16 * 64, elems=2 * 16 * 64), sm.SM_REDUCESCATTER) \
        == sm.SM_ERR_SHAPE
    q = sm.sm_plan({"X": 3}, "P(None, 'X')", "P('X', None)", 160, 96, 64)
    assert _err(sm.sm_local_gemm_reduce, q, _fb(96, dt=BF), B, out, sm.SM_REDUCESCATTER) == sm.SM_ERR_INDIVISIBLE


def test_skinny_fused_reduce_workspace_and_validation():
    """Workspace size of the fused split-J reduction (counters rounded up to
    256 bytes, then N partials [m, ld] per group, ld = n rounded up to 4),
    and the host checks of sm_local_gemm_reduce_ws before any launch."""
    sk = sm.sm_plan({"T": 8}, "P(None, 'T')", "P('T', None)", 16, 28672, 8192)
    assert sm.sm_gemm_reduce_workspace(sk) == 256 + 8 * 16 * 8192 * 4
    g2 = sm.sm_plan({"X": 2, "T": 4}, "P('X', 'T')", "P('T', None)", 48, 512, 300)
    assert sm.sm_gemm_reduce_workspace(g2, 1) == 256 + 4 * 24 * 300 * 4
    assert sm.sm_gemm_reduce_workspace(g2) == 256 + 2 * 4 * 24 * 300 * 4
    # taller products: the partials when a single launch would have fewer
    # than 256 tiles (here 1), none when it fills the GPU (the down-projection:
    # 4 groups x 8 x 32 tiles)
    few = sm.sm_plan({"T": 2}, "P(None, 'T')", "P('T', None)", 65, 128, 64)
    assert sm.sm_gemm_reduce_workspace(few) == 2 * 65 * 64 * 4
    dp = sm.sm_plan({"X": 4, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 8192, 28672, 8192)
    assert sm.sm_gemm_reduce_workspace(dp) == 0
    assert sm.sm_gemm_reduce_workspace(dp, 1) == 0  # one group: 256 tiles
    assert _err(sm.sm_gemm_reduce_workspace, sk, 2) == sm.SM_ERR_ARG
    assert _err(sm.sm_gemm_reduce_workspace, sm.sm_plan({"X": 2}, "P('X', None)", "P()", 64, 128, 64)) \
        == sm.SM_ERR_CASE
    X, A, out = _fb(28672, dt=BF), _fb(8192, dt=BF), _fb(8192)
    need = sm.sm_gemm_reduce_workspace(sk)
    ws = (FAKE, need)
    assert _err(sm.sm_local_gemm_reduce_ws, sk, X, A, out, None) == sm.SM_ERR_ARG
    assert _err(sm.sm_local_gemm_reduce_ws, sk, X, A, out, (FAKE, need - 4)) == sm.SM_ERR_SHAPE
    assert _err(sm.sm_local_gemm_reduce_ws, sk, X, A, out, (FAKE + 16, need)) == sm.SM_ERR_ALIGN
    assert _err(sm.sm_local_gemm_reduce_ws, sk, X, A, out, ws, 7) == sm.SM_ERR_ARG
    assert _err(sm.sm_local_gemm_reduce_ws, sk, X, A, _fb(8192, elems=15 * 8192), ws) == sm.SM_ERR_SHAPE
    assert _err(sm.sm_local_gemm_reduce_ws, sk, X, _fb(8192, 3584 * 8192, dt=BF), out, ws) == sm.SM_ERR_ARG
    odd = sm.sm_plan({"T": 3}, "P(None, 'T')", "P('T', None)", 16, 96, 64)
    assert _err(sm.sm_local_gemm_reduce_ws, odd, _fb(96, dt=BF), _fb(64, dt=BF), _fb(64), (FAKE, 1 << 30),
                sm.SM_REDUCESCATTER) == sm.SM_ERR_INDIVISIBLE
    many = sm.sm_plan({"T": 128}, "P(None, 'T')", "P('T', None)", 16, 128 * 16, 64)
    assert _err(sm.sm_local_gemm_reduce_ws, many, _fb(2048, dt=BF), _fb(64, dt=BF), _fb(64), (FAKE, 1 << 30)) \
        == sm.SM_ERR_SHAPE  # more than 64 partials per group
    # a valid call passes every argument check and reaches the device-memory
    # check, which refuses the fake pointers (or finds no device at all)
    assert _err(sm.sm_local_gemm_reduce_ws, sk, X, A, out, ws) in (sm.SM_ERR_ARG, sm.SM_ERR_HIP)
    assert "A: " in sm.sm_last_error()
    # few-tile taller products: a misaligned workspace is refused; a smaller
    # one, or none, is accepted (the single launch) and the call reaches the
    # device-memory check
    fA, fB, fo = _fb(128, dt=BF), _fb(64, dt=BF), _fb(64)
    fneed = sm.sm_gemm_reduce_workspace(few)
    assert _err(sm.sm_local_gemm_reduce_ws, few, fA, fB, fo, (FAKE + 16, fneed)) == sm.SM_ERR_ALIGN
    for w in ((FAKE, fneed), (FAKE, fneed - 4), None):
        assert _err(sm.sm_local_gemm_reduce_ws, few, fA, fB, fo, w) in (sm.SM_ERR_ARG, sm.SM_ERR_HIP)
        assert "A: " in sm.sm_last_error()


def test_reduce_and_gather_validation():
    p3 = sm.sm_plan({"X": 2, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 12, 16, 8)
    p1 = sm.sm_plan({"X": 2}, "P('X', None)", "P()", 8, 8, 8)
    parts = _fb(8, 6 * 8)
    out = _fb(8)
    assert _err(sm.sm_reduce_partials, p1, parts, out) == sm.SM_ERR_CASE
    assert _err(sm.sm_reduce_partials, p3, _fb(8), out) == sm.SM_ERR_UNREDUCED
    assert _err(sm.sm_reduce_partials, p3, parts, out, 5) == sm.SM_ERR_ARG
    assert _err(sm.sm_reduce_partials, p3, parts, out, sm.SM_ALLREDUCE, 1, 2) == sm.SM_ERR_ARG
    assert _err(sm.sm_reduce_partials, p3, _fb(8, 6 * 8, elems=4 * 6 * 8 - 1), out) == sm.SM_ERR_SHAPE
    q = sm.sm_plan({"X": 2, "Y": 4}, "P('X', 'Y')", "P('Y', None)", 12, 16, 8)  # m = 6, N = 4
    assert _err(sm.sm_reduce_partials, q, parts, out, sm.SM_REDUCESCATTER) == sm.SM_ERR_INDIVISIBLE
    assert _err(sm.sm_gather_shards, p3, sm.SM_WHAT_C_PARTIAL, parts, out) == sm.SM_ERR_UNREDUCED
    assert _err(sm.sm_gather_shards, p1, sm.SM_WHAT_C_SCATTERED, _fb(8, 32), out) == sm.SM_ERR_CASE
    assert _err(sm.sm_gather_shards, p1, sm.SM_WHAT_C_BLOCKS, _fb(8), out) == sm.SM_ERR_ARG
    assert _err(sm.sm_gather_shards, p1, sm.SM_WHAT_C_BLOCKS, _fb(8, 32), _fb(8, 64)) == sm.SM_ERR_ARG
    assert _err(sm.sm_gather_shards, p1, sm.SM_WHAT_C_BLOCKS, _fb(8, 32), _fb(4)) == sm.SM_ERR_SHAPE


def test_sp_tail_and_reshard_validation():
    p3 = sm.sm_plan({"X": 2, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 16, 16, 8)
    p1 = sm.sm_plan({"X": 2}, "P('X', None)", "P()", 8, 8, 8)
    pk = sm.sm_plan({"X": 2, "Y": 2}, "P(None, 'Y')", "P('Y', 'X')", 16, 16, 8)
    parts, out = _fb(8, 8 * 8), _fb(8)
    ln = sm.sm_reduce_scatter_layernorm
    assert _err(ln, p1, parts, out) == sm.SM_ERR_CASE
    assert _err(ln, pk, _fb(4, 16 * 4), _fb(8)) == sm.SM_ERR_CASE  # K sharded: rows are not whole
    assert _err(ln, p3, parts, out, None, None, -1.0) == sm.SM_ERR_ARG
    q = sm.sm_plan({"X": 2}, "P(None, 'X')", "P('X', None)", 8, 8, 6)
    assert _err(ln, q, _fb(8, 64), _fb(8)) == sm.SM_ERR_SHAPE  # row length 6 not a multiple of 4
    rs = sm.sm_reshard
    assert _err(rs, {"X": 2}, "A[I, J_X]", "A[I_X, J]", 8, 8, sm.SM_F32, _fb(8), _fb(8)) == sm.SM_ERR_ARG
    assert _err(rs, {"X": 3}, "A[I, J_X]", "A[I_X, J]", 8, 9, sm.SM_F32, _fb(4, 32), _fb(12, 48)) \
        == sm.SM_ERR_INDIVISIBLE
    assert _err(rs, {"X": 2}, "A[I_X, J_X]", "P()", 8, 8, sm.SM_F32, _fb(8, 32), _fb(8)) == sm.SM_ERR_AXIS_REUSED
    assert _err(rs, {"X": 2}, "A[I, J_X]", "P()", 8, 8, 7, _fb(8, 32), _fb(8)) == sm.SM_ERR_DTYPE


def test_buffer_element_type_is_checked():
    """A buffer is never addressed as another element type than it holds:
    a bfloat16 buffer given as the float32 output of a product (half the
    bytes the call would write), or float32 data given as a bfloat16 operand,
    is refused before anything is enqueued."""
    p = sm.sm_plan({"T": 4}, "P(None, None)", "P(None, 'T')", 64, 64, 256)  # fp32 output
    A, B = _fb(64, dt=BF), _fb(256, dt=BF)
    assert _err(sm.sm_local_gemm, p, A, B, _fb(256, dt=BF)) == sm.SM_ERR_DTYPE
    assert "bfloat16" in sm.sm_last_error() and "float32" in sm.sm_last_error()
    assert _err(sm.sm_local_gemm, p, _fb(64, dt=F32), B, _fb(256)) == sm.SM_ERR_DTYPE
    assert _err(sm.sm_local_gemm, p, A, B, _fb(256, dt=7)) == sm.SM_ERR_DTYPE
    pb = sm.sm_plan({"T": 4}, "P(None, None)", "P(None, 'T')", 64, 64, 256, sm.SM_BF16, sm.SM_BF16)
    assert _err(sm.sm_local_gemm, pb, A, B, _fb(256, dt=F32), sm.SM_EPI_GELU_TANH) == sm.SM_ERR_DTYPE
    p3 = sm.sm_plan({"X": 2}, "P(None, 'X')", "P('X', None)", 8, 16, 8)
    assert _err(sm.sm_reduce_partials, p3, _fb(8, 64, dt=BF), _fb(8)) == sm.SM_ERR_DTYPE
    assert _err(sm.sm_reshard, {"X": 2}, "A[I, J_X]", "A[I_X, J]", 8, 8, sm.SM_F32, _fb(8, 32, dt=BF),
                _fb(8, 32)) == sm.SM_ERR_DTYPE


def test_binding_sets_buffer_element_type():
    import torch

    assert sm.buf(torch.zeros(4, 8, dtype=torch.bfloat16)).dtype == sm.SM_BF16
    assert sm.buf(torch.zeros(2, 4, 8)).dtype == sm.SM_F32
    with pytest.raises(ValueError):
        sm.buf(torch.zeros(4, 8, dtype=torch.float16))


def test_empty_inputs_refused():
    """Zero-sized dimensions and empty unit / group ranges are refused on the
    host (the ABI computes on M, N, K >= 1), by the library and the oracle's
    planner alike."""
    for I, J, K in ((0, 8, 8), (8, 0, 8), (8, 8, 0)):
        with pytest.raises(sm.ShardmmError) as ei:
            sm.sm_plan({"X": 2}, "P()", "P()", I, J, K)
        assert ei.value.status == sm.SM_ERR_SHAPE
        with pytest.raises(ref_planner.PlanError) as pe:
            ref_planner.plan({"X": 2}, "P()", "P()", I, J, K)
        assert pe.value.code == "SHAPE"
    p1 = sm.sm_plan({"X": 2}, "P('X', None)", "P()", 64, 128, 64)
    p3 = sm.sm_plan({"X": 2}, "P(None, 'X')", "P('X', None)", 64, 128, 64)
    A, B = _fb(128, dt=BF), _fb(64, dt=BF)
    assert _err(sm.sm_local_gemm, p1, A, B, _fb(64, 32 * 64), 0, 0, 0) == sm.SM_ERR_ARG
    assert _err(sm.sm_reduce_partials, p3, _fb(64, 64 * 64), _fb(64), 0, 0, 0) == sm.SM_ERR_ARG
    assert _err(sm.sm_local_gemm_reduce, p3, A, B, _fb(64), 0, 0, 0) == sm.SM_ERR_ARG
    assert _err(sm.sm_reshard, {"X": 2}, "A[I, J_X]", "A[I_X, J]", 0, 8, sm.SM_F32, _fb(8, 32), _fb(8, 32)) \
        == sm.SM_ERR_SHAPE


def test_extent_checks_do_not_wrap():
    """Offsets and extents are computed without 64-bit wrap: an absurd ld or
    block_stride (here 2^62) cannot make an out-of-range block look in range."""
    p1 = sm.sm_plan({"X": 2}, "P('X', None)", "P()", 64, 128, 64)
    B, C = _fb(64, dt=BF), _fb(64, 32 * 64)
    huge = 1 << 62
    # 31 rows of ld 2^62 past a zero offset: 31 * 2^62 wraps negative in 64 bits
    assert _err(sm.sm_local_gemm, p1, _fb(huge, elems=1 << 40, dt=BF), B, C) == sm.SM_ERR_SHAPE
    # stacked input: unit 4 reads A block 4 at 4 * 2^62, which wraps to 0 in 64 bits
    p8 = sm.sm_plan({"X": 8}, "P('X', None)", "P()", 64, 64, 64)
    assert _err(sm.sm_local_gemm, p8, _fb(64, huge, elems=1 << 40, dt=BF), _fb(64, dt=BF), _fb(64, 8 * 64),
                sm.SM_EPI_STORE, 4, 1) == sm.SM_ERR_SHAPE
    p3 = sm.sm_plan({"X": 2}, "P(None, 'X')", "P('X', None)", 8, 16, 8)
    assert _err(sm.sm_reduce_partials, p3, _fb(8, huge, elems=1 << 40), _fb(8)) == sm.SM_ERR_SHAPE
    assert _err(sm.sm_gather_shards, p1, sm.SM_WHAT_C_BLOCKS, _fb(64, huge, elems=1 << 40), _fb(64)) \
        == sm.SM_ERR_SHAPE
    assert _err(sm.sm_reshard, {"X": 4}, "A[I, J_X]", "A[I_X, J]", 8, 16, sm.SM_F32, _fb(4, huge, elems=1 << 40),
                _fb(16, 32)) == sm.SM_ERR_SHAPE


def test_modified_plan_refused():
    """A plan is used only as sm_plan made it: editing any field afterwards
    (a zero partial count, a different local shape) is refused before any
    arithmetic uses it."""
    p = sm.sm_plan({"X": 2}, "P(None, 'X')", "P('X', None)", 64, 128, 64)
    A, B, C = _fb(128, dt=BF), _fb(64, dt=BF), _fb(64, 64 * 64)
    for field, value in (("n_partials", 0), ("n_units", 64), ("kase", sm.SM_CASE1)):
        q = sm.sm_plan_t.from_buffer_copy(p)
        setattr(q, field, value)
        assert _err(sm.sm_local_gemm, q, A, B, C) == sm.SM_ERR_ARG, field
        assert "modified" in sm.sm_last_error()
        assert _err(sm.sm_reduce_partials, q, C, _fb(64)) == sm.SM_ERR_ARG, field
    q = sm.sm_plan_t.from_buffer_copy(p)
    q.c_local[1] = 32
    assert _err(sm.sm_gather_shards, q, sm.SM_WHAT_C_BLOCKS, C, _fb(64)) == sm.SM_ERR_ARG
    # an untouched copy is accepted (it fails only at the launch, with no GPU here)
    q = sm.sm_plan_t.from_buffer_copy(p)
    assert _err(sm.sm_local_gemm, q, A, B, C) in (sm.SM_ERR_HIP, sm.SM_ERR_SHAPE)


def test_mesh_rank_limit():
    with pytest.raises(sm.ShardmmError) as ei:
        sm.sm_plan({"A": 1024, "B": 1025}, "P()", "P()", 8, 8, 8)
    assert ei.value.status == sm.SM_ERR_MESH
    assert sm.sm_plan({"A": 1024, "B": 1024}, "P()", "P()", 8, 8, 8).n_ranks == 1 << 20


def test_launch_grid_bound():
    """Local outputs whose tile grid could not be addressed by one launch are
    refused before any arithmetic on them (a [2^29, 2^29] block)."""
    p = sm.sm_plan({"X": 1}, "P()", "P()", 1 << 29, 64, 1 << 29)
    n = 1 << 29
    assert _err(sm.sm_local_gemm, p, _fb(64, dt=BF), _fb(n, dt=BF), _fb(n, elems=1 << 62)) == sm.SM_ERR_SHAPE
    assert "tiles" in sm.sm_last_error()
    pr = sm.sm_plan({"X": 1}, "P(None, 'X')", "P('X', None)", 1 << 29, 64, 1 << 29)
    assert _err(sm.sm_local_gemm_reduce, pr, _fb(64, dt=BF), _fb(n, dt=BF), _fb(n, elems=1 << 62),
                sm.SM_ALLREDUCE) == sm.SM_ERR_SHAPE
    assert "tiles" in sm.sm_last_error()
