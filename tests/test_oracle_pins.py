"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test names the fact it uses: a value the pages print, a closed form, a
library routine, or brute force on tiny inputs. A plausible slip in the
oracle (a dropped term, a swapped operand, a wrong sign or index, rounding
through float32) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import planner, reference as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _ints(shape, seed, lo=-4, hi=4):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float64)


# ----------------------------------------------------------- worked example

def test_two_by_two_partials_and_sum():
    """semiaifoundry.com, 'Engineering example': C0, C1 and their sum."""
    g = _golden("two_by_two_rs.json")
    A = np.array(g["A"], dtype=np.float64)
    B = np.array(g["B"], dtype=np.float64)
    p = planner.plan(dict(g["mesh"]), g["A_spec"], g["B_spec"], 2, 2, 2)
    assert p.case == 3 and p.n_partials == 2 and p.n_groups == 1
    parts = ref.partials(p, A, B)
    np.testing.assert_array_equal(parts[0], np.array(g["partials"]["0"], dtype=np.float64))
    np.testing.assert_array_equal(parts[1], np.array(g["partials"]["1"], dtype=np.float64))
    (s,) = ref.allreduce(p, parts)
    np.testing.assert_array_equal(s, np.array(g["sum"], dtype=np.float64))


def test_two_by_two_reduce_scatter_ownership_and_bytes():
    """Rank 0 keeps row 0, rank 1 keeps row 1; 8 B each way, 16 B per rank, 32 B total."""
    g = _golden("two_by_two_rs.json")
    A = np.array(g["A"], dtype=np.float64)
    B = np.array(g["B"], dtype=np.float64)
    p = planner.plan(dict(g["mesh"]), g["A_spec"], g["B_spec"], 2, 2, 2)
    rs = ref.reduce_scatter(p, ref.partials(p, A, B))
    for y in (0, 1):
        np.testing.assert_array_equal(rs[(0, y)], np.array(g["reduce_scatter_rows"][str(y)], dtype=np.float64))
        assert p.rank_unit(y) == y  # reduce coordinate y is rank y on {X:2}
    eb = p.exchange_bytes()
    assert eb["rs"] == g["payload_bytes_per_rank"]["reduce_scatter"]
    assert eb["ag"] == g["payload_bytes_per_rank"]["all_gather"]
    assert eb["ar"] == g["payload_bytes_per_rank"]["total"]
    assert eb["ar"] * p.n_ranks == g["payload_bytes_total"]


def test_concatenation_is_not_summation():
    """Concatenating the two 2x2 partials gives 4 unfinished rows; the
    oracle's gather refuses partials (semiaifoundry.com, 'The mechanism';
    mbrenndoerfer.com, partials need their sum, not their concatenation)."""
    g = _golden("two_by_two_rs.json")
    A = np.array(g["A"], dtype=np.float64)
    B = np.array(g["B"], dtype=np.float64)
    p = planner.plan(dict(g["mesh"]), g["A_spec"], g["B_spec"], 2, 2, 2)
    parts = ref.partials(p, A, B)
    cat = np.concatenate(parts, axis=0)
    assert cat.shape[0] == g["concatenated_partial_rows"]
    assert not np.array_equal(cat[:2], np.array(g["sum"], dtype=np.float64))
    with pytest.raises(planner.PlanError) as ei:
        ref.gather_partials(p, parts)
    assert ei.value.code == "UNREDUCED"


# ------------------------------------------------- products: library, brute

def test_matmul_equals_numpy_on_integers():
    """Integer data: every summation order is exact, so numpy's float64
    matmul (a library routine) must agree bit for bit."""
    A = _ints((37, 53), 1)
    B = _ints((53, 29), 2)
    np.testing.assert_array_equal(ref.matmul(A, B), A @ B)


def test_matmul_brute_force_tiny():
    """Pure-Python triple loop on tiny non-square shapes (catches transposes)."""
    rng = np.random.default_rng(3)
    A = rng.standard_normal((3, 5))
    B = rng.standard_normal((5, 4))
    want = [[sum(A[i, j] * B[j, k] for j in range(5)) for k in range(4)] for i in range(3)]
    np.testing.assert_allclose(ref.matmul(A, B), np.array(want), rtol=1e-14, atol=1e-14)


def test_matmul_reads_bf16_and_f32_storage_exactly():
    """bfloat16 / float32 storage is widened exactly: results match the
    float64 product of the widened values (library routine)."""
    x = torch.randn(17, 24, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    w = torch.randn(24, 9, generator=torch.Generator().manual_seed(5))
    want = x.double().numpy() @ w.double().numpy()
    np.testing.assert_allclose(ref.matmul(x, w), want, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(ref.widen(x), x.double().numpy())


def test_selected_rows_and_entries():
    A = _ints((40, 30), 6)
    B = _ints((30, 20), 7)
    full = A @ B
    rows = [0, 7, 39, 13]
    np.testing.assert_array_equal(ref.matmul(A, B, rows=rows), full[rows])
    ri, ci = [3, 39, 0], [19, 0, 5]
    got = ref.view_entries(A, (0, 0, 40, 30), B, (0, 0, 30, 20), ri, ci)
    np.testing.assert_array_equal(got, full[ri, ci])


def test_view_offsets_select_the_right_block():
    """A view (row0, col0, rows, cols) into a larger array."""
    A = _ints((12, 10), 8)
    B = _ints((10, 14), 9)
    got = ref.view_matmul(A, (4, 3, 5, 6), B, (2, 7, 6, 4))
    np.testing.assert_array_equal(got, A[4:9, 3:9] @ B[2:8, 7:11])


# ----------------------------------------------- block identity, outer view

@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_block_identity(N):
    """mbrenndoerfer.com 'Row Parallelism': X A = sum_i X_i A_i; each partial
    has the full output shape. Dense product computed separately (numpy)."""
    X = _ints((24, 64), 10 + N)
    A = _ints((64, 16), 20 + N)
    p = planner.plan({"T": N}, "P(None, 'T')", "P('T', None)", 24, 64, 16)
    parts = ref.partials(p, X, A)
    assert len(parts) == N and all(q.shape == (24, 16) for q in parts)
    np.testing.assert_array_equal(ref.allreduce(p, parts)[0], X @ A)
    if N > 1:
        assert not np.array_equal(parts[0], X @ A)


def test_outer_product_view():
    """ana-alekseeva.com: AB = sum_i a_i b_i^T (rank-one partials) -- case 3
    with N = J."""
    A = _ints((6, 8), 30)
    B = _ints((8, 5), 31)
    p = planner.plan({"T": 8}, "P(None, 'T')", "P('T', None)", 6, 8, 5)
    parts = ref.partials(p, A, B)
    for i, q in enumerate(parts):
        np.testing.assert_array_equal(q, np.outer(A[:, i], B[i, :]))
        assert np.linalg.matrix_rank(q) <= 1
    np.testing.assert_array_equal(ref.allreduce(p, parts)[0], A @ B)


def test_allreduce_equals_reducescatter_then_allgather():
    """learntpu.dev ch05 / lingze.zone: AllReduce = ReduceScatter + AllGather."""
    A = _ints((16, 24), 40)
    B = _ints((24, 12), 41)
    p = planner.plan({"X": 2, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 16, 24, 12)
    parts = ref.partials(p, A, B)
    ar = ref.gather(p, ref.allreduce(p, parts))
    rs = ref.gather_scattered(p, ref.reduce_scatter(p, parts))
    np.testing.assert_array_equal(ar, rs)
    np.testing.assert_array_equal(ar, A @ B)


def test_two_dimensional_output_grid():
    """Output blocks on a 2 x 2 grid (lingze.zone 'Case 1' C[I_X, K_Y]; 'Case 3'
    generalisation with K sharded too): gathering the case-1 blocks, the
    all-reduced blocks and the reduce-scattered row blocks must each give
    the dense product (numpy), and coordinate y of group (bi, bk) owns rows
    [bi m + y m/N, bi m + (y+1) m/N) of column block bk."""
    A = _ints((16, 24), 45)
    B = _ints((24, 12), 46)
    D = A @ B
    p1 = planner.plan({"X": 4, "Y": 2}, "A[I_X, J]", "B[J, K_Y]", 16, 24, 12)
    assert p1.case == 1 and p1.c_grid == (4, 2)
    np.testing.assert_array_equal(ref.gather(p1, ref.partials(p1, A, B)), D)
    p3 = planner.plan({"X": 2, "Y": 2, "Z": 2}, "P('X', 'Y')", "P('Y', 'Z')", 16, 24, 12)
    assert p3.case == 3 and p3.c_grid == (2, 2) and p3.n_partials == 2
    parts = ref.partials(p3, A, B)
    np.testing.assert_array_equal(ref.gather(p3, ref.allreduce(p3, parts)), D)
    rs = ref.reduce_scatter(p3, parts)
    np.testing.assert_array_equal(ref.gather_scattered(p3, rs), D)
    for (g, y), blk in rs.items():
        bi, bk = divmod(g, 2)
        assert p3.rs_rows(g, y) == (bi * 8 + y * 4, 4)
        np.testing.assert_array_equal(blk, D[bi * 8 + y * 4:bi * 8 + (y + 1) * 4, bk * 6:(bk + 1) * 6])


def test_generalised_case3_groups():
    """lingze.zone 'Case 3', generalisation: A[I_X,J_Y].B[J_Y,K] -> partial
    sums of C[I_X,K]; group x's block is rows x*m.. of the dense product."""
    A = _ints((32, 40), 50)
    B = _ints((40, 8), 51)
    p = planner.plan({"X": 4, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 32, 40, 8)
    sums = ref.allreduce(p, ref.partials(p, A, B))
    D = A @ B
    for g in range(4):
        np.testing.assert_array_equal(sums[g], D[g * 8:(g + 1) * 8])


def test_rank_outputs_after_allreduce():
    """semiaifoundry.com "Sharded matrix multiplication and result
    ownership" (The mechanism: after the all-reduce every rank holds the
    completed values of its block): on {X:2, Y:2} with A[I_X, J_Y], rank
    (x, y) holds rows x*m.. of the dense product (numpy), the same block for
    both y, and ranks of different x hold different row blocks."""
    A = _ints((16, 24), 55)
    B = _ints((24, 12), 56)
    D = A @ B
    p = planner.plan({"X": 2, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 16, 24, 12)
    held = ref.rank_outputs_allreduce(p, ref.partials(p, A, B))
    assert sorted(held) == [0, 1, 2, 3]
    for r, blk in held.items():
        x = r // 2  # row-major rank numbering over (X, Y)
        np.testing.assert_array_equal(blk, D[x * 8:(x + 1) * 8])
    np.testing.assert_array_equal(held[0], held[1])
    assert not np.array_equal(held[0], held[2])


def test_integer_exactness_bound():
    """Closed form (IEEE binary32 has a 24-bit significand): with entries in
    [-4, 4] every partial sum is an integer of magnitude <= 16 J, exact in
    float32 when 16 J < 2^24. All workload shapes satisfy it."""
    for J in (128, 4096, 14336, 16384, 3584):
        assert 16 * J < 2 ** 24
    A = _ints((8, 14336), 60)
    B = _ints((14336, 4), 61)
    d = ref.matmul(A, B)
    np.testing.assert_array_equal(d.astype(np.float32).astype(np.float64), d)


# ---------------------------------------------------------------- GeLU

def test_gelu_matches_torch_float64():
    x = np.linspace(-8, 8, 4001)
    want = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(ref.gelu_tanh(x), want, rtol=1e-14, atol=1e-15)


def test_gelu_identities():
    """gelu(0) = 0; gelu(x) - gelu(-x) = x (tanh is odd); gelu(x)/x -> 1."""
    x = np.linspace(0.01, 6, 600)
    assert ref.gelu_tanh(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(ref.gelu_tanh(x) - ref.gelu_tanh(-x), x, rtol=1e-13, atol=1e-15)
    assert abs(ref.gelu_tanh(np.array([30.0]))[0] - 30.0) < 1e-12


# ------------------------------------------------------- bfloat16 rounding

def test_round_bf16_matches_torch_on_float32_values():
    """For float32-representable inputs, rounding from double equals
    torch's float32 -> bfloat16 conversion (RNE)."""
    rng = np.random.default_rng(70)
    x32 = np.concatenate([rng.standard_normal(20000).astype(np.float32) * np.float32(s)
                          for s in (1e-30, 1e-3, 1.0, 1e3, 1e30)])
    got = ref.round_bf16(x32.astype(np.float64))
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)


def test_round_bf16_ties_and_no_double_rounding():
    """Hand-derived: bfloat16 spacing at 1 is 2^-7.
    1 + 2^-8 is a tie -> 1 (even); 1 + 3*2^-8 is a tie -> 1 + 2^-6 (even);
    1 + 2^-8 + 2^-40 is just above the tie -> 1 + 2^-7, which rounding
    through float32 first would get wrong (it would land on the tie)."""
    vals = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40,
                     -(1 + 2.0 ** -8 + 2.0 ** -40)])
    got = ref.bf16_bits_to_f64(ref.round_bf16(vals))
    np.testing.assert_array_equal(got, [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -(1 + 2.0 ** -7)])


def test_round_bf16_overflow_and_subnormal():
    big = (2 - 2.0 ** -7) * 2.0 ** 127
    half_ulp = 2.0 ** 119
    got = ref.round_bf16(np.array([big, big + half_ulp * 0.99, big + half_ulp, 2.0 ** -133,
                                   2.0 ** -134, 2.0 ** -134 * 1.01, 0.0, -0.0]))
    assert got[0] == 0x7F7F and got[1] == 0x7F7F
    assert got[2] == 0x7F80               # tie at the top rounds to even = infinity
    assert got[3] == 0x0001               # smallest subnormal
    assert got[4] == 0x0000               # tie between 0 and 2^-133 -> even (0)
    assert got[5] == 0x0001
    assert got[6] == 0x0000 and got[7] == 0x8000


# ----------------------------------------------------------- MLP chain

def test_mlp_chain_parts_and_commuting_split():
    """Column split of W1 commutes with the elementwise GeLU
    (ana-alekseeva.com 'MLP block'): the chain equals the unsharded
    round_bf16(gelu(X W1)) W2 computed with library routines."""
    X = torch.randn(8, 16, generator=torch.Generator().manual_seed(80)).to(torch.bfloat16)
    W1 = (0.2 * torch.randn(16, 32, generator=torch.Generator().manual_seed(81))).to(torch.bfloat16)
    W2 = (0.2 * torch.randn(32, 16, generator=torch.Generator().manual_seed(82))).to(torch.bfloat16)
    p1 = planner.plan({"T": 4}, "P(None, None)", "P(None, 'T')", 8, 16, 32)
    p2 = planner.plan({"T": 4}, "P(None, 'T')", "P('T', None)", 8, 32, 16)
    H, Z = ref.mlp_chain(p1, p2, X, W1, W2)
    y = X.double() @ W1.double()
    g = torch.nn.functional.gelu(y, approximate="tanh")
    h_ref = ref.round_bf16(g.numpy())
    np.testing.assert_array_equal(H, h_ref)
    z_ref = ref.bf16_bits_to_f64(h_ref) @ W2.double().numpy()
    np.testing.assert_allclose(Z, z_ref, rtol=1e-13, atol=1e-13)
    # the bf16 storage of H matters: without it the result differs
    z_unrounded = g.numpy() @ W2.double().numpy()
    assert not np.allclose(Z, z_unrounded, rtol=1e-9, atol=0)


# ----------------------------------------------------- layer norm, reshard

def test_layer_norm_hand_example_and_library():
    """Hand-worked: x = [1, 2, 3, 4]: mean 2.5, biased var 1.25, so
    y = (x - 2.5) / sqrt(1.25 + eps). Library: torch's float64 layer_norm."""
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    want = (x - 2.5) / np.sqrt(1.25 + 1e-5)
    np.testing.assert_allclose(ref.layer_norm(x), want, rtol=1e-15, atol=1e-15)
    rng = np.random.default_rng(120)
    X = rng.standard_normal((7, 33)) * 3 + 1
    g = rng.standard_normal(33)
    b = rng.standard_normal(33)
    t = torch.nn.functional.layer_norm(torch.from_numpy(X), (33,), torch.from_numpy(g), torch.from_numpy(b), 1e-5)
    np.testing.assert_allclose(ref.layer_norm(X, g, b), t.numpy(), rtol=1e-12, atol=1e-12)
    y = ref.layer_norm(X, eps=0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-13)


def test_sp_tail_equals_allreduce_then_norm():
    """ana-alekseeva.com 'Sequence parallelism': reduce-scatter, per-token
    norm, all-gather gives what all-reduce then the per-token norm gives."""
    A = _ints((16, 24), 130)
    B = _ints((24, 12), 131)
    p = planner.plan({"X": 2, "Y": 2}, "P('X', 'Y')", "P('Y', None)", 16, 24, 12)
    parts = ref.partials(p, A, B)
    np.testing.assert_allclose(ref.sp_tail(p, parts), ref.layer_norm(A @ B), rtol=1e-12, atol=1e-12)


def test_reshard_alltoall_blocks():
    """learntpu.dev ch05: AllToAll A[I, J_X] -> A[I_X, J] moves which
    dimension is sharded; an all-gather to P() gives the whole array."""
    X = np.arange(8 * 12, dtype=np.float64).reshape(8, 12)
    mesh = {"X": 4}
    cols = ref.shard(X, mesh, "A[I, J_X]")
    assert all(b.shape == (8, 3) for b in cols.values())
    rows = ref.reshard(cols, mesh, "A[I, J_X]", "A[I_X, J]", 8, 12)
    assert all(b.shape == (2, 12) for b in rows.values())
    for i in range(4):
        np.testing.assert_array_equal(rows[i], X[2 * i:2 * i + 2])
    whole = ref.reshard(rows, mesh, "A[I_X, J]", "P()", 8, 12)
    np.testing.assert_array_equal(whole[0], X)


# ------------------------------------------------------------- Freivalds

def test_freivalds_detects_one_wrong_entry():
    A = _ints((50, 40), 90)
    B = _ints((40, 30), 91)
    C = A @ B
    assert ref.freivalds(A, (0, 0, 50, 40), B, (0, 0, 40, 30), C) == 0.0
    bad = C.copy()
    bad[17, 23] += 1.0
    assert ref.freivalds(A, (0, 0, 50, 40), B, (0, 0, 40, 30), bad) > 0.0


def test_rel_frobenius():
    a = np.ones((4, 4))
    assert ref.rel_frobenius(a, a) == 0.0
    assert math.isclose(ref.rel_frobenius(a * 1.001, a), 1e-3, rel_tol=1e-9)
