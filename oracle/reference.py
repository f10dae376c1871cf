"""The sharded matmul's outputs, computed plainly in fp64 on the CPU.

TEST INFRASTRUCTURE (part of the oracle; see the package docstring).

What each function follows, and what pins it (tests/test_oracle_*.py):

* ``matmul`` / ``view_matmul`` -- C[i,k] = sum_j A[i,j] B[j,k], J
  contracted (lingze.zone "Cheetsheet ...", the product at the top).
  Pinned by the 2x2 worked example's numbers (semiaifoundry.com,
  "Engineering example"), by numpy's float64 matmul on integer data, and by
  pure-Python brute force on tiny shapes.
* ``unit_partial`` / ``partials`` -- each rank multiplies the slice of J it
  holds and gets an unreduced partial over the whole output block
  (lingze.zone "Case 3"; semiaifoundry.com "The mechanism", steps 2-3).
  Pinned by C0 = [[5,6],[15,18]] and C1 = [[14,16],[28,32]] of the 2x2
  example and by the block identity X A = sum_i X_i A_i (mbrenndoerfer.com
  "Row Parallelism", block-form equation) against a separate dense product.
* ``group_sum`` / ``allreduce`` / ``reduce_scatter`` / ``gather`` -- addition
  of matching coordinates in rank order; all-reduce leaves the sum on every
  rank of the group, reduce-scatter leaves row block y on reduce
  coordinate y, all-gather places finished blocks (learntpu.dev ch05, "The
  four collectives and their cost" table; semiaifoundry.com, "The
  mechanism" steps 4-5). Pinned by the 2x2 example's sum [[19,22],[43,50]]
  and its row ownership, by AllReduce = ReduceScatter + AllGather, and by
  the refusal to concatenate unfinished partials.
* ``gelu_tanh`` -- pinned by torch's float64 GeLU (tanh form) and by the
  identities gelu(0) = 0 and gelu(x) - gelu(-x) = x.
* ``round_bf16`` -- pinned by torch's float32 -> bfloat16 conversion on
  float32-representable values and by hand-derived ties and overflow.
* ``mlp_chain`` -- dense chain Z = round_bf16(gelu(X W1)) W2, summed over the
  row-split of W2 in rank order (ana-alekseeva.com "MLP block";
  mbrenndoerfer.com, the column/row pairing paragraph). Pinned by its parts
  and by the column split commuting with the elementwise GeLU.
* ``freivalds`` -- checks a full product through A (B v) = C v; pinned by a
  planted single-entry error that it must detect.

Random-valued configurations have no page-printed outputs: their expected
values are this oracle's, computed in fp64 from the exact stored inputs.

tests/test_oracle_mutants.py plants plausible slips in copies of this
module, the planner and oracle.c, and checks that some pin fails for each.
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .build import load_library
from .planner import Plan, PlanError

F64, F32, BF16 = 0, 1, 2


def stored(x) -> Tuple[np.ndarray, int]:
    """The stored bytes of an operand as a 2-D numpy array plus its kind."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            if x.dtype == torch.float64:
                return x.numpy(), F64
            raise TypeError(f"unsupported dtype {x.dtype}")
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(x)
    if a.dtype == np.float64:
        return a, F64
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    if np.issubdtype(a.dtype, np.integer):
        return a.astype(np.float64), F64
    raise TypeError(f"unsupported dtype {a.dtype}")


def widen(x) -> np.ndarray:
    """Exact float64 values of the stored operand."""
    a, kind = stored(x)
    if kind == F64:
        return a.astype(np.float64, copy=True)
    if kind == F32:
        return a.astype(np.float64)
    return bf16_bits_to_f64(a)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _ptr(a: np.ndarray, row0: int = 0, col0: int = 0) -> int:
    return a.ctypes.data + (row0 * a.shape[1] + col0) * a.itemsize


def view_matmul(A, a_view, B, b_view, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Product of the view A[r0:r0+m, c0:c0+k] and B[r0':r0'+k, c0':c0'+n].

    ``rows`` selects output rows (indices within the view) to compute.
    """
    lib = load_library()
    a, ak = stored(A)
    b, bk = stored(B)
    ar0, ac0, m, k = a_view
    br0, bc0, k2, n = b_view
    if k != k2:
        raise ValueError("contracted lengths differ")
    if rows is None:
        out = np.empty((m, n), dtype=np.float64)
        rc = lib.orc_matmul(_ptr(a, ar0, ac0), ak, a.shape[1], _ptr(b, br0, bc0), bk, b.shape[1],
                            out.ctypes.data, n, m, k, n, None, 0)
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((len(r), n), dtype=np.float64)
        rc = lib.orc_matmul(_ptr(a, ar0, ac0), ak, a.shape[1], _ptr(b, br0, bc0), bk, b.shape[1],
                            out.ctypes.data, n, m, k, n, r.ctypes.data, len(r))
    if rc:
        raise RuntimeError("orc_matmul failed")
    return out


def matmul(A, B, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    a, _ = stored(A)
    b, _ = stored(B)
    return view_matmul(A, (0, 0, a.shape[0], a.shape[1]), B, (0, 0, b.shape[0], b.shape[1]), rows)


def dense(A, B) -> np.ndarray:
    """The unsharded product, computed separately from any partial."""
    return matmul(A, B)


def view_entries(A, a_view, B, b_view, ri, ci) -> np.ndarray:
    lib = load_library()
    a, ak = stored(A)
    b, bk = stored(B)
    ar0, ac0, m, k = a_view
    br0, bc0, k2, n = b_view
    ri = np.ascontiguousarray(np.asarray(ri, dtype=np.int64))
    ci = np.ascontiguousarray(np.asarray(ci, dtype=np.int64))
    if ri.size and (ri.min() < 0 or ri.max() >= m or ci.min() < 0 or ci.max() >= n):
        raise IndexError("entry outside the view")
    out = np.empty(len(ri), dtype=np.float64)
    rc = lib.orc_entries(_ptr(a, ar0, ac0), ak, a.shape[1], _ptr(b, br0, bc0), bk, b.shape[1], k,
                         ri.ctypes.data, ci.ctypes.data, len(ri), out.ctypes.data)
    if rc:
        raise RuntimeError("orc_entries failed")
    return out


def view_matvec(M, view, v: np.ndarray) -> np.ndarray:
    lib = load_library()
    a, kind = stored(M)
    r0, c0, rows, cols = view
    v = np.ascontiguousarray(v, dtype=np.float64)
    assert v.shape == (cols,)
    y = np.empty(rows, dtype=np.float64)
    rc = lib.orc_matvec(_ptr(a, r0, c0), kind, a.shape[1], rows, cols, v.ctypes.data, y.ctypes.data)
    if rc:
        raise RuntimeError("orc_matvec failed")
    return y


# ------------------------------------------------------------ sharded steps

def unit_partial(plan: Plan, A, B, unit: int, rows=None) -> np.ndarray:
    """C_u = A_u . B_u over the unit's own slice of J (fp64)."""
    if plan.case not in (1, 3):
        raise PlanError("NEEDS_GATHER", f"case {plan.case}: gather an operand first")
    v = plan.unit_views(unit)
    return view_matmul(A, v["A"], B, v["B"], rows)


def unit_entries(plan: Plan, A, B, unit: int, ri, ci) -> np.ndarray:
    v = plan.unit_views(unit)
    return view_entries(A, v["A"], B, v["B"], ri, ci)


def partials(plan: Plan, A, B, units: Optional[Sequence[int]] = None) -> List[np.ndarray]:
    us = range(plan.n_units) if units is None else units
    return [unit_partial(plan, A, B, u) for u in us]


def sum_ranked(parts: Sequence[np.ndarray]) -> np.ndarray:
    """((P_0 + P_1) + P_2) + ... elementwise, in rank order, fp64."""
    lib = load_library()
    N = len(parts)
    stack = np.ascontiguousarray(np.stack([np.asarray(p, dtype=np.float64) for p in parts]))
    out = np.empty(parts[0].shape, dtype=np.float64)
    n = out.size
    rc = lib.orc_sum_ranked(stack.ctypes.data, n, N, n, out.ctypes.data)
    if rc:
        raise RuntimeError("orc_sum_ranked failed")
    return out


def group_sum(plan: Plan, parts: Sequence[np.ndarray], g: int) -> np.ndarray:
    N = plan.n_partials
    return sum_ranked([parts[g * N + y] for y in range(N)])


def allreduce(plan: Plan, parts: Sequence[np.ndarray]) -> List[np.ndarray]:
    """Per group, the completed block every rank of the group holds."""
    if plan.case != 3:
        raise PlanError("CASE", "nothing to reduce")
    return [group_sum(plan, parts, g) for g in range(plan.n_groups)]


def reduce_scatter(plan: Plan, parts: Sequence[np.ndarray]) -> Dict[Tuple[int, int], np.ndarray]:
    """(g, y) -> rows [y m/N, (y+1) m/N) of the completed block of group g."""
    if plan.case != 3:
        raise PlanError("CASE", "nothing to reduce")
    m = plan.c_local[0]
    N = plan.n_partials
    if m % N:
        raise PlanError("INDIVISIBLE", "rows do not split N ways")
    step = m // N
    out = {}
    for g in range(plan.n_groups):
        s = group_sum(plan, parts, g)
        for y in range(N):
            out[(g, y)] = s[y * step:(y + 1) * step].copy()
    return out


def gather(plan: Plan, blocks: Sequence[np.ndarray]) -> np.ndarray:
    """Place finished output blocks (one per group) at their coordinates."""
    m, n = plan.c_local
    out = np.zeros((plan.I, plan.K), dtype=np.float64)
    for g, blk in enumerate(blocks):
        bi, bk = divmod(g, plan.c_grid[1])
        out[bi * m:(bi + 1) * m, bk * n:(bk + 1) * n] = blk
    return out


def gather_scattered(plan: Plan, rs: Dict[Tuple[int, int], np.ndarray]) -> np.ndarray:
    n = plan.c_local[1]
    out = np.zeros((plan.I, plan.K), dtype=np.float64)
    for (g, y), blk in rs.items():
        r0, rows = plan.rs_rows(g, y)
        bk = g % plan.c_grid[1]
        out[r0:r0 + rows, bk * n:(bk + 1) * n] = blk
    return out


def gather_partials(plan: Plan, parts) -> np.ndarray:
    """Gathering unfinished partials is refused: they overlap in output
    coordinates and need addition, not concatenation."""
    if plan.case == 3 and plan.n_partials > 1:
        raise PlanError("UNREDUCED", "partials need addition, not concatenation")
    return gather(plan, parts)


def rank_outputs_allreduce(plan: Plan, parts) -> Dict[int, np.ndarray]:
    """Every rank's block after all-reduce (replicas are equal objects)."""
    sums = allreduce(plan, parts)
    return {r: sums[plan.rank_unit(r) // plan.n_partials] for r in range(plan.n_ranks)}


# --------------------------------------------------------------- elementwise

def gelu_tanh(x: np.ndarray) -> np.ndarray:
    lib = load_library()
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    if lib.orc_gelu_tanh_array(x.ctypes.data, y.ctypes.data, x.size):
        raise RuntimeError("orc_gelu_tanh_array failed")
    return y


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> bfloat16 bit patterns, round to nearest, ties to even."""
    lib = load_library()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    if lib.orc_round_bf16_array(x.ctypes.data, out.ctypes.data, x.size):
        raise RuntimeError("orc_round_bf16_array failed")
    return out


def mlp_hidden(plan1: Plan, X, W1, rows=None) -> np.ndarray:
    """First layer of the Megatron MLP: H_u = round_bf16(gelu(X W1_u)) for
    each column block u of W1 (GeLU applies per column block, since it is
    elementwise), concatenated into [rows, F] bfloat16 bit patterns."""
    assert plan1.case == 1
    hs = []
    for u in range(plan1.n_units):
        y = unit_partial(plan1, X, W1, u, rows)
        hs.append(round_bf16(gelu_tanh(y)))
    return np.concatenate(hs, axis=1) if len(hs) > 1 else hs[0]


def mlp_chain(plan1: Plan, plan2: Plan, X, W1, W2, rows=None):
    """Megatron MLP: column-split W1, GeLU on each column block, row-split W2.

    Returns (H_bits [rows, F] bfloat16 bit patterns, Z [rows, D] fp64) where
    H_u = round_bf16(gelu(X W1_u)) and Z = sum_u H_u W2_u in rank order.
    ``rows`` restricts the computation to a sample of output rows.
    """
    assert plan1.case == 1 and plan2.case == 3
    H = mlp_hidden(plan1, X, W1, rows)
    zs = []
    Hk = H.shape[1] // plan2.n_partials
    for u in range(plan2.n_units):
        v = plan2.unit_views(u)
        hv = (0, v["A"][1], H.shape[0], Hk)
        zs.append(view_matmul(H, hv, W2, v["B"]))
    return H, sum_ranked(zs)


# ------------------------------------------------- sequence-parallel tail

def layer_norm(x: np.ndarray, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """Row-wise layer norm in fp64: (x - mean) / sqrt(var + eps) * gamma +
    beta, with the biased (1/n) variance (Ba, Kiros & Hinton 2016; the pages
    apply layer norm per token between the reduce-scatter and the
    all-gather -- ana-alekseeva.com, "Sequence parallelism")."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    mean = x.sum(axis=-1, keepdims=True) / n
    d = x - mean
    var = (d * d).sum(axis=-1, keepdims=True) / n
    y = d / np.sqrt(var + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64)
    return y


def sp_tail(plan: Plan, parts, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """Reduce-scatter, layer norm of each owned row, all-gather: the global
    [I, K] result every rank holds afterwards."""
    rs = reduce_scatter(plan, parts)
    normed = {key: layer_norm(blk, gamma, beta, eps) for key, blk in rs.items()}
    return gather_scattered(plan, normed)


# ------------------------------------------------------------- resharding

def shard(X: np.ndarray, mesh, spec) -> Dict[int, np.ndarray]:
    """The distinct blocks of X under a spec, by block id."""
    from .planner import array_blocks

    return {b: X[r0:r0 + nr, c0:c0 + nc].copy() for b, (r0, c0, nr, nc) in
            array_blocks(mesh, spec, X.shape[0], X.shape[1]).items()}


def unshard(blocks: Dict[int, np.ndarray], mesh, spec, rows: int, cols: int) -> np.ndarray:
    from .planner import array_blocks

    out = np.zeros((rows, cols), dtype=next(iter(blocks.values())).dtype)
    for b, (r0, c0, nr, nc) in array_blocks(mesh, spec, rows, cols).items():
        out[r0:r0 + nr, c0:c0 + nc] = blocks[b]
    return out


def reshard(blocks: Dict[int, np.ndarray], mesh, frm, to, rows: int, cols: int) -> Dict[int, np.ndarray]:
    """Blocks under `to` from blocks under `frm` (AllToAll when the sharded
    dimension moves; AllGather when `to` is replicated)."""
    return shard(unshard(blocks, mesh, frm, rows, cols), mesh, to)


# ------------------------------------------------------------------- checks

def freivalds(A, a_view, B, b_view, C: np.ndarray, trials: int = 2, seed: int = 0,
              ints: bool = True) -> float:
    """Max over trials of |C v - A (B v)| / (|A| |B| |v|)-scaled residual.

    With integer-valued A, B, C and integer v, both sides are exact in fp64
    (magnitudes far below 2^53), so any nonzero residual is a wrong entry.
    """
    rng = np.random.default_rng(seed)
    n = b_view[3]
    worst = 0.0
    Cw = np.ascontiguousarray(C, dtype=np.float64)
    for _ in range(trials):
        v = rng.integers(-1000, 1001, size=n).astype(np.float64) if ints else rng.standard_normal(n)
        w = view_matvec(B, b_view, v)
        y = view_matvec(A, a_view, w)
        cv = view_matvec(Cw, (0, 0, Cw.shape[0], Cw.shape[1]), v)
        if ints:
            worst = max(worst, float(np.max(np.abs(cv - y))) if y.size else 0.0)
        else:
            scale = float(np.linalg.norm(y)) or 1.0
            worst = max(worst, float(np.linalg.norm(cv - y)) / scale)
    return worst


def rel_frobenius(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = float(np.linalg.norm(want))
    num = float(np.linalg.norm(got - want))
    return num / den if den else num
