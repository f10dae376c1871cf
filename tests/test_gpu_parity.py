"""GPU parity: the HIP path, called through the C-ABI, against the fp64 oracle.

Small and ragged shapes are checked element by element; the full workload
sizes are checked in the launch configuration the benchmark times, on
sampled output rows (float) or with exact Freivalds checks plus sampled
entries (integers).
"""
import numpy as np
import pytest
import torch

import local_shard_gemm_amd as sm
import workloads as wl
from oracle import planner, reference as ref

from hip_cases import (DEV, FREIVALDS_FLOAT_TOL, REL_TOL, f32_bits_equal, gelu_h_within_bound, guard_intact,
                       guarded, h_ulp_stats, run_partials,
                       sample_rows, say, to_dev)

pytestmark = pytest.mark.gpu


def _plans(mesh, a_spec, b_spec, I, J, K, out=sm.SM_F32):
    p = sm.sm_plan(mesh, a_spec, b_spec, I, J, K, sm.SM_BF16, out)
    q = planner.plan(mesh, a_spec, b_spec, I, J, K, "bf16", "f32" if out == sm.SM_F32 else "bf16")
    return p, q


def _int(shape, seed):
    return wl.random_ints(shape, seed)


# --------------------------------------------------------------- toy (C0)

def test_toy_case3_partials_allreduce_reducescatter_bitexact():
    w = wl.get("toy")
    say("case: toy", w.name)
    A = wl.make_operand(w.operand("A"))
    B = wl.make_operand(w.operand("B"))
    p, q = _plans(dict(w.mesh), w.operand("A").spec, w.operand("B").spec, 64, 128, 64)
    Ad, Bd = to_dev(A), to_dev(B)
    full, P = run_partials(p, Ad, Bd)
    parts = ref.partials(q, A, B)
    torch.cuda.synchronize()
    Pn = P.cpu().numpy()
    for u in range(2):
        assert f32_bits_equal(Pn[u], parts[u]), u
    assert guard_intact(full, P.numel())
    # all-reduce into the global layout
    fo, out = guarded((64, 64), torch.float32)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(out), sm.SM_ALLREDUCE)
    (s,) = ref.allreduce(q, parts)
    assert f32_bits_equal(out.cpu().numpy(), s)
    assert guard_intact(fo, out.numel())
    # reduce-scatter: stacked row halves and global layout
    frs, rs = guarded((2, 32, 64), torch.float32)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(rs), sm.SM_REDUCESCATTER)
    want = ref.reduce_scatter(q, parts)
    for y in range(2):
        assert f32_bits_equal(rs[y].cpu().numpy(), want[(0, y)])
    assert guard_intact(frs, rs.numel())
    g = torch.empty(64, 64, dtype=torch.float32, device=DEV)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(g), sm.SM_REDUCESCATTER)
    assert torch.equal(g, out)  # AR = RS + AG, bitwise
    g2 = torch.empty(64, 64, dtype=torch.float32, device=DEV)
    sm.sm_gather_shards(p, sm.SM_WHAT_C_SCATTERED, sm.buf(rs), sm.buf(g2))
    assert torch.equal(g2, out)
    # concatenation of partials is refused
    with pytest.raises(sm.ShardmmError) as ei:
        sm.sm_gather_shards(p, sm.SM_WHAT_C_PARTIAL, sm.buf(P), sm.buf(g2))
    assert ei.value.status == sm.SM_ERR_UNREDUCED


def test_two_by_two_worked_example():
    """semiaifoundry.com 'Engineering example' on the GPU (ld = 8 buffers)."""
    say("case: 2x2 worked example")
    A = torch.zeros(2, 8, dtype=torch.bfloat16)
    B = torch.zeros(2, 8, dtype=torch.bfloat16)
    A[:, :2] = torch.tensor([[1, 2], [3, 4]], dtype=torch.bfloat16)
    B[:, :2] = torch.tensor([[5, 6], [7, 8]], dtype=torch.bfloat16)
    p = sm.sm_plan({"X": 2}, "P(None, 'X')", "P('X', None)", 2, 2, 2)
    Ad, Bd = to_dev(A), to_dev(B)
    P = torch.full((2, 2, 8), float("nan"), dtype=torch.float32, device=DEV)
    sm.sm_local_gemm(p, sm.buf(Ad), sm.buf(Bd), sm.buf(P))
    Pc = P.cpu()
    assert Pc[0, :, :2].tolist() == [[5, 6], [15, 18]]
    assert Pc[1, :, :2].tolist() == [[14, 16], [28, 32]]
    assert torch.isnan(Pc[:, :, 2:]).all()  # nothing written outside the blocks
    rs = torch.zeros(2, 1, 8, dtype=torch.float32, device=DEV)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(rs), sm.SM_REDUCESCATTER)
    assert rs[0, 0, :2].tolist() == [19, 22] and rs[1, 0, :2].tolist() == [43, 50]
    ar = torch.zeros(2, 8, dtype=torch.float32, device=DEV)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(ar), sm.SM_ALLREDUCE)
    assert ar[:, :2].tolist() == [[19, 22], [43, 50]]


# ------------------------------------------------ ragged edges (integers)

RAGGED = [
    # mesh, A spec, B spec, I, J, K
    ({"X": 2, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 600, 400, 520),   # K_local 200, N 520
    ({"Y": 2}, "P(None, 'Y')", "P('Y', None)", 520, 256, 296),           # interior + edge tiles
    ({"X": 3}, "P('X', None)", "P()", 3 * 257, 96, 264),                 # case 1, all ragged
    ({"X": 2, "Y": 2}, "P('X', None)", "P(None, 'Y')", 2 * 512, 192, 2 * 256),  # case 1, interior only
    ({"T": 4}, "P(None, 'T')", "P('T', None)", 300, 4 * 72, 256),         # K not a multiple of 64
    ({"T": 2}, "P(None, 'T')", "P('T', None)", 33, 2 * 8, 17 * 8),        # tiny, one partial tile
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: f"{c[3]}x{c[4]}x{c[5]}")
def test_ragged_shapes_bitexact(case):
    mesh, sa, sb, I, J, K = case
    say("case: ragged", case)
    A = _int((I, J), 11 + I)
    B = _int((J, K), 12 + K)
    p, q = _plans(mesh, sa, sb, I, J, K)
    Ad, Bd = to_dev(A), to_dev(B)
    full, P = run_partials(p, Ad, Bd)
    torch.cuda.synchronize()
    Pn = P.cpu().numpy()
    for u in range(q.n_units):
        assert f32_bits_equal(Pn[u], ref.unit_partial(q, A, B, u)), u
    assert guard_intact(full, P.numel())
    if q.case == 3:
        out = torch.empty(I, K, dtype=torch.float32, device=DEV)
        sm.sm_reduce_partials(p, sm.buf(P), sm.buf(out), sm.SM_ALLREDUCE)
        want = ref.gather(q, ref.allreduce(q, [ref.unit_partial(q, A, B, u) for u in range(q.n_units)]))
        assert f32_bits_equal(out.cpu().numpy(), want)
        np.testing.assert_array_equal(want, ref.dense(A, B))
    else:
        g = torch.empty(I, K, dtype=torch.float32, device=DEV)
        sm.sm_gather_shards(p, sm.SM_WHAT_C_BLOCKS, sm.buf(P), sm.buf(g))
        assert f32_bits_equal(g.cpu().numpy(), ref.dense(A, B))
        # the global output layout of the local products gives the same bytes
        g2 = torch.empty(I, K, dtype=torch.float32, device=DEV)
        sm.sm_local_gemm(p, sm.buf(Ad), sm.buf(Bd), sm.buf(g2))
        assert torch.equal(g, g2)


def test_store_paths_bitexact():
    """The MFMA kernels' epilogue stores 4 consecutive columns per lane as
    one vector when the output views allow it. Covered here: (a) a logical
    width that is not a multiple of 4 inside padded stacked blocks (the last
    run of a row falls back to single elements, and the padding columns stay
    untouched); (b) column-block views that start off the 16-byte grid (every
    store falls back to single elements)."""
    say("case: store paths")
    # (a) case 3, n = 70 inside blocks of ld 72
    I, J, K = 300, 2 * 96, 70
    A, B = _int((I, J), 41), _int((J, K), 42)
    p, q = _plans({"Y": 2}, "P(None, 'Y')", "P('Y', None)", I, J, K)
    ld = 72
    Bp = torch.zeros(J, ld, dtype=torch.bfloat16)
    Bp[:, :K] = B
    full = torch.full((2 * I * ld + 256,), float("nan"), device=DEV)
    C = full[:2 * I * ld].view(2, I, ld)
    sm.sm_local_gemm(p, sm.buf(to_dev(A)), sm.buf(to_dev(Bp)), sm.buf(C, ld=ld))
    Cn = C.cpu().numpy()
    for u in range(2):
        assert f32_bits_equal(Cn[u, :, :K], ref.unit_partial(q, A, B, u)), u
    assert np.isnan(Cn[:, :, K:]).all()
    assert bool(torch.isnan(full[2 * I * ld:]).all())
    # (b) case 1, global layout, column blocks of width 6 (views at 24-byte steps)
    I, J, K = 260, 64, 2 * 6
    A, B = _int((I, J), 43), _int((J, K), 44)
    p, q = _plans({"Y": 2}, "P()", "P(None, 'Y')", I, J, K)
    Bp = torch.zeros(J, 16, dtype=torch.bfloat16)
    Bp[:, :K] = B
    fg, g = guarded((I, K), torch.float32)
    sm.sm_local_gemm(p, sm.buf(to_dev(A)), sm.buf(to_dev(Bp)), sm.buf(g))
    assert f32_bits_equal(g.cpu().numpy(), ref.dense(A, B))
    assert guard_intact(fg, g.numel())


def test_ragged_tiles_tight_buffers_bitexact():
    """Ragged tiles read A rows and B columns clamped into the views. Two
    layouts: (a) a B view whose last row ends exactly at the buffer's
    declared end with N not a multiple of 8 (the 16-byte chunk holding column
    N-1 would reach past it, so the launch goes to the element-wise kernel);
    (b) the same product with the row padded (the MFMA pipeline kernel takes
    the ragged tiles). Both bit for bit against the oracle, nothing outside C
    written."""
    say("case: ragged tiles, tight buffers")
    I, J, K, ld = 300, 64, 70, 72
    A, B = _int((I, J), 51), _int((J, K), 52)
    p, q = _plans({"X": 1}, "P()", "P()", I, J, K)
    Bp = torch.zeros(J, ld, dtype=torch.bfloat16)
    Bp[:, :K] = B
    Bd = to_dev(Bp)
    want = ref.dense(A, B)
    for elems in ((J - 1) * ld + K, J * ld):
        bb = sm.sm_buf(Bd.data_ptr(), ld, 0, elems, sm.SM_BF16, 0)
        fg, g = guarded((I, ld), torch.float32)
        g.fill_(float("nan"))
        sm.sm_local_gemm(p, sm.buf(to_dev(A)), bb, sm.buf(g))
        gn = g.cpu().numpy()
        assert f32_bits_equal(gn[:, :K], want), elems
        assert np.isnan(gn[:, K:]).all()  # padding columns of C untouched
        assert guard_intact(fg, g.numel())


def test_gelu_epilogue_unaligned_views():
    """GeLU -> bfloat16 into the global H layout with column blocks of width 6:
    half of the views start off the 8-byte grid, so the bfloat16 stores go
    element by element; H is within the derived bound of the oracle."""
    say("case: gelu epilogue unaligned views")
    X = wl.random_normal((96, 64), 45)
    W1 = wl.random_normal((64, 24), 46, 0.1)
    W2 = wl.random_normal((24, 64), 47, 0.1)
    p1, q1 = _plans({"T": 4}, "P(None, None)", "P(None, 'T')", 96, 64, 24, sm.SM_BF16)
    _, q2 = _plans({"T": 4}, "P(None, 'T')", "P('T', None)", 96, 24, 64)
    fh = torch.zeros(96 * 24 + 64, dtype=torch.bfloat16, device=DEV)
    H = fh[:96 * 24].view(96, 24)
    sm.sm_local_gemm(p1, sm.buf(to_dev(X)), sm.buf(to_dev(W1)), sm.buf(H), sm.SM_EPI_GELU_TANH)
    Hw, _ = ref.mlp_chain(q1, q2, X, W1, W2)
    Hg = H.cpu().view(torch.int16).numpy().view(np.uint16)
    absdot = ref.matmul(np.abs(ref.widen(X)), np.abs(ref.widen(W1)))
    assert gelu_h_within_bound(Hg, Hw, absdot, 64).all()
    assert (Hg != Hw).mean() < 0.01
    assert bool((fh[96 * 24:] == 0).all())


def test_gather_many_short_rows_bitexact():
    """Case-1 blocks of 1030 x 40 fp32 gathered into C[4120, 80]: 8240 short
    rows in 8 jobs, most lanes of each row's workgroup idle; the gathered C
    equals the dense product bit for bit and nothing outside C is written."""
    I, J, K = 4 * 1030, 64, 2 * 40
    say("case: gather many short rows")
    A, B = _int((I, J), 51), _int((J, K), 52)
    p, q = _plans({"X": 4, "Y": 2}, "P('X', None)", "P(None, 'Y')", I, J, K)
    Bp = torch.zeros(J, 88, dtype=torch.bfloat16)
    Bp[:, :K] = B
    _, P = run_partials(p, to_dev(A), to_dev(Bp))
    fg, g = guarded((I, K), torch.float32)
    sm.sm_gather_shards(p, sm.SM_WHAT_C_BLOCKS, sm.buf(P), sm.buf(g))
    assert f32_bits_equal(g.cpu().numpy(), ref.dense(A, B))
    assert guard_intact(fg, g.numel())


def test_many_units_and_jobs_bitexact():
    """Maximum batch sizes: 128 units in one sm_local_gemm call (two launches
    of at most 64 units), gathered through 128 row jobs (four launches of at
    most 32); and an 80-unit case 3 reduced through 80 row jobs, both modes."""
    say("case: many units and jobs")
    # case 1 on {X:16, Y:8}: 128 blocks of [24, 16]
    I, J, K = 16 * 24, 64, 8 * 16
    A, B = _int((I, J), 61), _int((J, K), 62)
    p, q = _plans({"X": 16, "Y": 8}, "P('X', None)", "P(None, 'Y')", I, J, K)
    assert p.n_units == 128
    full, P = run_partials(p, to_dev(A), to_dev(B))
    fg, g = guarded((I, K), torch.float32)
    sm.sm_gather_shards(p, sm.SM_WHAT_C_BLOCKS, sm.buf(P), sm.buf(g))
    assert f32_bits_equal(g.cpu().numpy(), ref.dense(A, B))
    assert guard_intact(full, P.numel()) and guard_intact(fg, g.numel())
    # case 3 on {X:40, Y:2}: 40 groups x 2 partials of [32, 48]
    I, J, K = 40 * 32, 2 * 64, 48
    A, B = _int((I, J), 63), _int((J, K), 64)
    p, q = _plans({"X": 40, "Y": 2}, "P('X', 'Y')", "P('Y', None)", I, J, K)
    assert p.n_units == 80
    _, P = run_partials(p, to_dev(A), to_dev(B))
    want = ref.dense(A, B)
    for mode in (sm.SM_ALLREDUCE, sm.SM_REDUCESCATTER):
        fo, out = guarded((I, K), torch.float32)
        sm.sm_reduce_partials(p, sm.buf(P), sm.buf(out), mode)
        assert f32_bits_equal(out.cpu().numpy(), want), mode
        assert guard_intact(fo, out.numel())


def test_single_partial_reduce_bitexact():
    """Degenerate case 3: J split over an axis of size 1 (N = 1). The reduce
    is a copy of the one partial, in both modes."""
    say("case: N = 1 reduce")
    I, J, K = 96, 64, 40
    A, B = _int((I, J), 65), _int((J, K), 66)
    p, q = _plans({"X": 1}, "P(None, 'X')", "P('X', None)", I, J, K)
    assert p.kase == sm.SM_CASE3 and p.n_partials == 1
    _, P = run_partials(p, to_dev(A), to_dev(B))
    for mode in (sm.SM_ALLREDUCE, sm.SM_REDUCESCATTER):
        out = torch.full((I, K), float("nan"), device=DEV)
        sm.sm_reduce_partials(p, sm.buf(P), sm.buf(out), mode)
        assert f32_bits_equal(out.cpu().numpy(), ref.dense(A, B)), mode


SKINNY = [
    ({"T": 4}, "P(None, 'T')", "P('T', None)", 5, 4 * 100, 296),    # ragged K and N
    ({"T": 8}, "P(None, 'T')", "P('T', None)", 16, 8 * 256, 1024),  # full tiles
    ({"T": 2}, "P(None, 'T')", "P('T', None)", 1, 2 * 64, 136),     # one row
    ({"X": 2}, "P()", "P(None, 'X')", 16, 96, 2 * 128),              # case 1, skinny
    ({"T": 2}, "P(None, 'T')", "P('T', None)", 16, 2 * 112, 768),   # 7 K steps over 4 waves, 3 column blocks
    ({"T": 2}, "P(None, 'T')", "P('T', None)", 3, 2 * 16, 512),     # one K step: three waves idle
    ({"T": 4}, "P(None, 'T')", "P('T', None)", 17, 4 * 128, 512),   # one row block, rows 16..31 kept
    ({"T": 4}, "P(None, 'T')", "P('T', None)", 32, 4 * 96, 264),    # one full row block, ragged N
    ({"T": 2}, "P(None, 'T')", "P('T', None)", 33, 2 * 128, 256),   # two row blocks, second has one row
    ({"T": 8}, "P(None, 'T')", "P('T', None)", 64, 8 * 256, 1024),  # two full row blocks
    ({"T": 4}, "P(None, 'T')", "P('T', None)", 48, 4 * 100, 296),   # two row blocks, ragged K and N
    # 65..128 rows (past the split-J kernel: the tile kernel with ragged row tiles)
    ({"T": 4}, "P(None, 'T')", "P('T', None)", 65, 4 * 128, 256),   # six blocks, the fifth has one row
    ({"T": 2}, "P(None, 'T')", "P('T', None)", 96, 2 * 100, 296),   # six full blocks, ragged K and N
    ({"T": 8}, "P(None, 'T')", "P('T', None)", 128, 8 * 256, 1024),  # eight full blocks, full column blocks
    ({"T": 4}, "P(None, 'T')", "P('T', None)", 100, 4 * 96, 264),   # eight blocks, 3 K steps over 4 waves
    ({"X": 2}, "P()", "P(None, 'X')", 97, 96, 2 * 128),              # case 1, 97 rows
    ({"T": 2}, "P(None, 'T')", "P('T', None)", 127, 2 * 16, 128),   # K below one step
]


@pytest.mark.parametrize("case", SKINNY, ids=lambda c: f"{c[3]}x{c[4]}x{c[5]}")
def test_skinny_shapes_bitexact(case):
    mesh, sa, sb, I, J, K = case
    say("case: skinny", case)
    A = _int((I, J), 21 + J)
    B = _int((J, K), 22 + K)
    p, q = _plans(mesh, sa, sb, I, J, K)
    full, P = run_partials(p, to_dev(A), to_dev(B))
    torch.cuda.synchronize()
    Pn = P.cpu().numpy()
    for u in range(q.n_units):
        assert f32_bits_equal(Pn[u], ref.unit_partial(q, A, B, u)), u
    assert guard_intact(full, P.numel())


@pytest.mark.parametrize("rows", [12, 40, 80, 128], ids=["rows12", "rows40", "rows80", "rows128"])
@pytest.mark.parametrize("width", [256, 288], ids=["interior", "ragged"])
def test_gelu_epilogue_skinny(width, rows):
    """The GeLU(tanh) -> bfloat16 epilogue for small batches (the split-J
    kernel up to 64 rows, ragged row tiles of the tile kernel above):
    column blocks of a small batch, within the derived bound of the oracle's
    round_bf16(gelu(.))."""
    say("case: gelu epilogue skinny", width, rows)
    F = 4 * width
    X = wl.random_normal((rows, 160), 34)
    W1 = wl.random_normal((160, F), 35, 0.1)
    W2 = wl.random_normal((F, 64), 36, 0.1)
    p1, q1 = _plans({"T": 4}, "P(None, None)", "P(None, 'T')", rows, 160, F, sm.SM_BF16)
    _, q2 = _plans({"T": 4}, "P(None, 'T')", "P('T', None)", rows, F, 64)
    H = torch.empty(rows, F, dtype=torch.bfloat16, device=DEV)
    sm.sm_local_gemm(p1, sm.buf(to_dev(X)), sm.buf(to_dev(W1)), sm.buf(H), sm.SM_EPI_GELU_TANH)
    Hw, _ = ref.mlp_chain(q1, q2, X, W1, W2)
    Hg = H.cpu().view(torch.int16).numpy().view(np.uint16)
    absdot = ref.matmul(np.abs(ref.widen(X)), np.abs(ref.widen(W1)))
    assert gelu_h_within_bound(Hg, Hw, absdot, 160).all()
    assert (Hg != Hw).mean() < 0.01


def test_gelu_epilogue_small():
    """Case-1 column block with the GeLU(tanh) epilogue stored as bfloat16:
    within one bfloat16 ulp of the oracle's round_bf16(gelu(.)), and the
    second layer's reduced output within the float tolerance."""
    say("case: gelu epilogue small")
    X = wl.random_normal((96, 128), 31)
    W1 = wl.random_normal((128, 4 * 160), 32, 0.1)
    W2 = wl.random_normal((4 * 160, 128), 33, 0.1)
    p1, q1 = _plans({"T": 4}, "P(None, None)", "P(None, 'T')", 96, 128, 640, sm.SM_BF16)
    p2, q2 = _plans({"T": 4}, "P(None, 'T')", "P('T', None)", 96, 640, 128)
    H = torch.empty(96, 640, dtype=torch.bfloat16, device=DEV)
    sm.sm_local_gemm(p1, sm.buf(to_dev(X)), sm.buf(to_dev(W1)), sm.buf(H), sm.SM_EPI_GELU_TANH)
    Hw, Zw = ref.mlp_chain(q1, q2, X, W1, W2)
    Hg = H.cpu().view(torch.int16).numpy().view(np.uint16)
    absdot = ref.matmul(np.abs(ref.widen(X)), np.abs(ref.widen(W1)))
    assert gelu_h_within_bound(Hg, Hw, absdot, 128).all()
    assert (Hg != Hw).mean() < 0.01
    P = torch.empty(4, 96, 128, dtype=torch.float32, device=DEV)
    sm.sm_local_gemm(p2, sm.buf(H), sm.buf(to_dev(W2)), sm.buf(P))
    Z = torch.empty(96, 128, dtype=torch.float32, device=DEV)
    sm.sm_reduce_partials(p2, sm.buf(P), sm.buf(Z), sm.SM_ALLREDUCE)
    assert ref.rel_frobenius(Z.cpu().numpy(), Zw) <= REL_TOL


def test_determinism_and_stream_argument():
    say("case: determinism")
    A = wl.random_normal((512, 2 * 384), 41)
    B = wl.random_normal((2 * 384, 512), 42)
    p = sm.sm_plan({"Y": 2}, "P(None, 'Y')", "P('Y', None)", 512, 768, 512)
    Ad, Bd = to_dev(A), to_dev(B)
    s = torch.cuda.Stream()
    outs = []
    for _ in range(3):
        P = torch.empty(2, 512, 512, dtype=torch.float32, device=DEV)
        with torch.cuda.stream(s):
            sm.sm_local_gemm(p, sm.buf(Ad), sm.buf(Bd), sm.buf(P), stream=s)
            out = torch.empty(512, 512, dtype=torch.float32, device=DEV)
            sm.sm_reduce_partials(p, sm.buf(P), sm.buf(out), sm.SM_ALLREDUCE, stream=s)
        s.synchronize()
        outs.append(out)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


def test_unit_subsets_match_full_batch():
    """Computing one X-group at a time equals the batched launch bitwise."""
    say("case: unit subsets")
    A = wl.random_normal((4 * 256, 2 * 256), 51)
    B = wl.random_normal((2 * 256, 512), 52)
    p = sm.sm_plan({"X": 4, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 1024, 512, 512)
    Ad, Bd = to_dev(A), to_dev(B)
    _, P = run_partials(p, Ad, Bd)
    for x in range(4):
        _, Px = run_partials(p, Ad, Bd, 2 * x, 2)
        assert torch.equal(Px, P[2 * x:2 * x + 2])


# ------------------------------------------------- full workload sizes

def _rel_err_rows(gpu_rows: np.ndarray, want_rows: np.ndarray) -> float:
    return ref.rel_frobenius(gpu_rows, want_rows)


@pytest.fixture(scope="module")
def downproj():
    w = wl.get("downproj")
    A = wl.make_operand(w.operand("A"))
    B = wl.make_operand(w.operand("B"))
    return w, A, B


def test_full_downproj_float(downproj):
    """Case-3 down-projection shard at full size, all 8 units in one launch
    and reduce-scatter of all 4 groups (the benchmarked configuration)."""
    w, A, B = downproj
    say("case: full downproj float")
    I, J = A.shape
    K = B.shape[1]
    p, q = _plans(dict(w.mesh), w.operand("A").spec, w.operand("B").spec, I, J, K)
    Ad, Bd = to_dev(A), to_dev(B)
    full, P = run_partials(p, Ad, Bd)
    rs = torch.empty(I, K, dtype=torch.float32, device=DEV)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(rs), sm.SM_REDUCESCATTER)
    torch.cuda.synchronize()
    assert guard_intact(full, P.numel())
    m = q.c_local[0]
    worst = 0.0
    sums = {}
    for u in range(q.n_units):
        rows = sample_rows(m, 6, 100 + u)
        want = ref.unit_partial(q, A, B, u, rows=rows)
        got = P[u][rows].cpu().numpy()
        worst = max(worst, _rel_err_rows(got, want))
        g, y = divmod(u, q.n_partials)
        sums.setdefault(g, []).append((rows, want))
    say("downproj partial rel err", worst)
    assert worst <= REL_TOL
    # reduce-scatter rows: oracle partial rows summed in rank order
    for g in range(q.n_groups):
        rows = sample_rows(m, 4, 200 + g)
        parts = [ref.unit_partial(q, A, B, g * q.n_partials + y, rows=rows) for y in range(q.n_partials)]
        want = ref.sum_ranked(parts)
        got = rs[[g * m + r for r in rows]].cpu().numpy()
        assert _rel_err_rows(got, want) <= REL_TOL
    # whole outputs: every partial against its unit's product, and the
    # reduce-scattered C against the dense product (Freivalds, Gaussian v)
    Pn = P.cpu().numpy()
    fr = [ref.freivalds(A, q.unit_views(u)["A"], B, q.unit_views(u)["B"], Pn[u], trials=1, seed=u, ints=False)
          for u in range(q.n_units)]
    fr.append(ref.freivalds(A, (0, 0, I, J), B, (0, 0, J, K), rs.cpu().numpy(), trials=1, seed=9, ints=False))
    say("downproj whole-output Freivalds residuals", max(fr))
    assert max(fr) <= FREIVALDS_FLOAT_TOL


def test_full_downproj_integer_exact():
    w = wl.int_variant(wl.get("downproj"))
    say("case: full downproj integer")
    A = wl.make_operand(w.operand("A"))
    B = wl.make_operand(w.operand("B"))
    I, J = A.shape
    K = B.shape[1]
    p, q = _plans(dict(w.mesh), w.operand("A").spec, w.operand("B").spec, I, J, K)
    _, P = run_partials(p, to_dev(A), to_dev(B))
    ar = torch.empty(4, *q.c_local, dtype=torch.float32, device=DEV)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(ar), sm.SM_ALLREDUCE)
    rs = torch.empty(I, K, dtype=torch.float32, device=DEV)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(rs), sm.SM_REDUCESCATTER)
    g = torch.empty(I, K, dtype=torch.float32, device=DEV)
    sm.sm_gather_shards(p, sm.SM_WHAT_C_BLOCKS, sm.buf(ar), sm.buf(g))
    assert torch.equal(g, rs)  # AR = RS + AG
    Pn = P.cpu().numpy()
    for u in range(q.n_units):
        v = q.unit_views(u)
        assert ref.freivalds(A, v["A"], B, v["B"], Pn[u].astype(np.float64), trials=1, seed=u) == 0.0, u
        rng = np.random.default_rng(u)
        ri = rng.integers(0, q.c_local[0], 256)
        ci = rng.integers(0, q.c_local[1], 256)
        want = ref.unit_entries(q, A, B, u, ri, ci)
        assert np.array_equal(Pn[u][ri, ci], want.astype(np.float32))
    # the reduced output against the dense product (exact), via Freivalds
    assert ref.freivalds(A, (0, 0, I, J), B, (0, 0, J, K), rs.cpu().numpy().astype(np.float64), trials=1) == 0.0


def test_full_case1_float_and_gather():
    w = wl.get("case1")
    say("case: full case1 float")
    A = wl.make_operand(w.operand("A"))
    B = wl.make_operand(w.operand("B"))
    p, q = _plans(dict(w.mesh), w.operand("A").spec, w.operand("B").spec, 4096, 4096, 4096)
    _, P = run_partials(p, to_dev(A), to_dev(B))
    C = torch.empty(4096, 4096, dtype=torch.float32, device=DEV)
    sm.sm_gather_shards(p, sm.SM_WHAT_C_BLOCKS, sm.buf(P), sm.buf(C))
    torch.cuda.synchronize()
    rows = sample_rows(4096, 24, 7)
    want = ref.matmul(A, B, rows=rows)
    assert _rel_err_rows(C[rows].cpu().numpy(), want) <= REL_TOL
    fr = ref.freivalds(A, (0, 0, 4096, 4096), B, (0, 0, 4096, 4096), C.cpu().numpy(), trials=2, ints=False)
    say("case1 whole-output Freivalds residual", fr)
    assert fr <= FREIVALDS_FLOAT_TOL


def test_full_case1_integer_exact():
    w = wl.int_variant(wl.get("case1"))
    say("case: full case1 integer")
    A = wl.make_operand(w.operand("A"))
    B = wl.make_operand(w.operand("B"))
    p, q = _plans(dict(w.mesh), w.operand("A").spec, w.operand("B").spec, 4096, 4096, 4096)
    _, P = run_partials(p, to_dev(A), to_dev(B))
    C = torch.empty(4096, 4096, dtype=torch.float32, device=DEV)
    sm.sm_gather_shards(p, sm.SM_WHAT_C_BLOCKS, sm.buf(P), sm.buf(C))
    Cn = C.cpu().numpy().astype(np.float64)
    assert ref.freivalds(A, (0, 0, 4096, 4096), B, (0, 0, 4096, 4096), Cn, trials=2) == 0.0
    rows = sample_rows(4096, 8, 8)
    assert f32_bits_equal(C[rows].cpu().numpy(), ref.matmul(A, B, rows=rows))


def test_full_mlp_chain():
    w = wl.get("mlp")
    say("case: full mlp chain")
    X = wl.make_operand(w.operand("X"))
    W1 = wl.make_operand(w.operand("W1"))
    W2 = wl.make_operand(w.operand("W2"))
    p1, q1 = _plans(dict(w.mesh), w.operand("X").spec, w.operand("W1").spec, 4096, 4096, 16384, sm.SM_BF16)
    p2, q2 = _plans(dict(w.mesh), "P(None, 'T')", w.operand("W2").spec, 4096, 16384, 4096)
    H = torch.empty(4096, 16384, dtype=torch.bfloat16, device=DEV)  # column blocks, global layout
    sm.sm_local_gemm(p1, sm.buf(to_dev(X)), sm.buf(to_dev(W1)), sm.buf(H), sm.SM_EPI_GELU_TANH)
    P = torch.empty(4, 4096, 4096, dtype=torch.float32, device=DEV)
    sm.sm_local_gemm(p2, sm.buf(H), sm.buf(to_dev(W2)), sm.buf(P))
    Z = torch.empty(4096, 4096, dtype=torch.float32, device=DEV)
    sm.sm_reduce_partials(p2, sm.buf(P), sm.buf(Z), sm.SM_ALLREDUCE)
    torch.cuda.synchronize()
    # H: every element against the oracle's round_bf16(gelu(X W1_u))
    Hw = ref.mlp_hidden(q1, X, W1)
    Hg = H.cpu().view(torch.int16).numpy().view(np.uint16)
    st = h_ulp_stats(Hg, Hw)
    say("H against the oracle, bf16 ulps:", st)
    ri, ci = np.nonzero(Hg != Hw)
    absdot = ref.view_entries(np.abs(ref.widen(X)), (0, 0, 4096, 4096), np.abs(ref.widen(W1)), (0, 0, 4096, 16384),
                              ri, ci)
    assert gelu_h_within_bound(Hg[ri, ci], Hw[ri, ci], absdot, 4096).all()
    assert st["differ"] < 0.01
    # Z: whole output against the oracle's H times W2 (Freivalds, Gaussian
    # v); the GPU's Z is built on the GPU's H, whose one-ulp flips (above)
    # move Z by about sqrt(differ) * 2^-8 relative, so the workload's
    # tolerance applies, not the pure-GEMM one
    fr = ref.freivalds(Hw, (0, 0, 4096, 16384), W2, (0, 0, 16384, 4096), Z.cpu().numpy(), trials=1, ints=False)
    say("chain whole-output Freivalds residual", fr)
    assert fr <= REL_TOL
    rows = sample_rows(4096, 8, 9)
    _, Zw = ref.mlp_chain(q1, q2, X, W1, W2, rows=rows)
    err = _rel_err_rows(Z[rows].cpu().numpy(), Zw)
    say("chain rel err", err)
    assert err <= REL_TOL


def test_full_mlp_integer_layers_exact():
    """Both GEMM shapes of the chain with the plain store epilogue on
    integer values (GeLU would break integrality)."""
    w = wl.int_variant(wl.get("mlp"))
    say("case: full mlp integer")
    X = wl.make_operand(w.operand("X"))
    W1 = wl.make_operand(w.operand("W1"))
    W2 = wl.make_operand(w.operand("W2"))
    p1, q1 = _plans(dict(w.mesh), w.operand("X").spec, w.operand("W1").spec, 4096, 4096, 16384)
    _, P1 = run_partials(p1, to_dev(X), to_dev(W1))
    for u in range(4):
        v = q1.unit_views(u)
        assert ref.freivalds(X, v["A"], W1, v["B"], P1[u].cpu().numpy().astype(np.float64), trials=1) == 0.0
    H = wl.random_ints((4096, 16384), 4600)
    p2, q2 = _plans(dict(w.mesh), "P(None, 'T')", w.operand("W2").spec, 4096, 16384, 4096)
    _, P2 = run_partials(p2, to_dev(H), to_dev(W2))
    Z = torch.empty(4096, 4096, dtype=torch.float32, device=DEV)
    sm.sm_reduce_partials(p2, sm.buf(P2), sm.buf(Z), sm.SM_ALLREDUCE)
    assert ref.freivalds(H, (0, 0, 4096, 16384), W2, (0, 0, 16384, 4096),
                         Z.cpu().numpy().astype(np.float64), trials=1) == 0.0


@pytest.mark.parametrize("integer", [False, True])
def test_full_skinny_all_outputs(integer):
    w = wl.get("skinny")
    if integer:
        w = wl.int_variant(w)
    say("case: full skinny", "int" if integer else "float")
    X = wl.make_operand(w.operand("X"))
    A = wl.make_operand(w.operand("A"))
    p, q = _plans(dict(w.mesh), w.operand("X").spec, w.operand("A").spec, 16, 28672, 8192)
    full, P = run_partials(p, to_dev(X), to_dev(A))
    out = torch.empty(16, 8192, dtype=torch.float32, device=DEV)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(out), sm.SM_ALLREDUCE)
    torch.cuda.synchronize()
    assert guard_intact(full, P.numel())
    parts = ref.partials(q, X, A)
    (s,) = ref.allreduce(q, parts)
    Pn = P.cpu().numpy()
    if integer:
        for u in range(8):
            assert f32_bits_equal(Pn[u], parts[u]), u
        assert f32_bits_equal(out.cpu().numpy(), s)
    else:
        worst = max(ref.rel_frobenius(Pn[u], parts[u]) for u in range(8))
        say("skinny partial rel err", worst)
        assert worst <= REL_TOL
        assert ref.rel_frobenius(out.cpu().numpy(), s) <= REL_TOL


@pytest.mark.parametrize("integer", [False, True])
def test_full_medium_batch(integer):
    """A 128-row batch on the skinny workload's weights (8 x [128,3584] .
    [3584,8192]): past the split-J kernel's 64 rows, the tile kernel with
    half-empty row tiles at its full launch size, against the oracle's
    partials and their sum."""
    w = wl.get("skinny")
    if integer:
        w = wl.int_variant(w)
    say("case: full medium batch", "int" if integer else "float")
    rows = 128
    X = wl.make_operand(w.operand("X"), shape=(rows, 28672))
    A = wl.make_operand(w.operand("A"))
    p, q = _plans(dict(w.mesh), w.operand("X").spec, w.operand("A").spec, rows, 28672, 8192)
    full, P = run_partials(p, to_dev(X), to_dev(A))
    out = torch.empty(rows, 8192, dtype=torch.float32, device=DEV)
    sm.sm_reduce_partials(p, sm.buf(P), sm.buf(out), sm.SM_ALLREDUCE)
    torch.cuda.synchronize()
    assert guard_intact(full, P.numel())
    parts = ref.partials(q, X, A)
    (s,) = ref.allreduce(q, parts)
    Pn = P.cpu().numpy()
    if integer:
        for u in range(8):
            assert f32_bits_equal(Pn[u], parts[u]), u
        assert f32_bits_equal(out.cpu().numpy(), s)
    else:
        worst = max(ref.rel_frobenius(Pn[u], parts[u]) for u in range(8))
        say("medium partial rel err", worst)
        assert worst <= REL_TOL
        assert ref.rel_frobenius(out.cpu().numpy(), s) <= REL_TOL


def test_host_memory_refused_before_launch():
    """A pageable host buffer (a CPU tensor) handed to a device entry point is
    refused on the host with SM_ERR_ARG before anything is launched; the
    device outputs are untouched."""
    say("case: host memory refused")
    I, J, K = 128, 128, 64  # more than 64 rows: not a skinny product, so the fused call gets as far as the buffers
    A, B = _int((I, J), 71), _int((J, K), 72)
    p, q = _plans({"X": 2}, "P(None, 'X')", "P('X', None)", I, J, K)
    Ad, Bd = to_dev(A), to_dev(B)
    P = torch.full((2, I, K), float("nan"), device=DEV)
    for args in ((sm.buf(A), sm.buf(Bd), sm.buf(P)), (sm.buf(Ad), sm.buf(Bd), sm.buf(torch.zeros(2, I, K)))):
        with pytest.raises(sm.ShardmmError) as ei:
            sm.sm_local_gemm(p, *args)
        assert ei.value.status == sm.SM_ERR_ARG and "GPU can address" in str(ei.value)
    torch.cuda.synchronize()
    assert bool(torch.isnan(P).all())
    sm.sm_local_gemm(p, sm.buf(Ad), sm.buf(Bd), sm.buf(P))
    out = torch.full((I, K), float("nan"), device=DEV)
    for call in (lambda: sm.sm_reduce_partials(p, sm.buf(P.cpu()), sm.buf(out)),
                 lambda: sm.sm_gather_shards(p, sm.SM_WHAT_C_SCATTERED, sm.buf(P.cpu()), sm.buf(out)),
                 lambda: sm.sm_local_gemm_reduce(p, sm.buf(A), sm.buf(Bd), sm.buf(out)),
                 lambda: sm.sm_reduce_scatter_layernorm(p, sm.buf(P), sm.buf(out), torch.ones(K), None),
                 lambda: sm.sm_reshard({"X": 2}, "A[I, J_X]", "A[I_X, J]", I, K, sm.SM_F32, sm.buf(out.cpu(), block_stride=0),
                                       sm.buf(P))):
        with pytest.raises(sm.ShardmmError) as ei:
            call()
        assert ei.value.status == sm.SM_ERR_ARG, ei.value
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all())
