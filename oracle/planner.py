"""Reference planner for A[I,J].B[J,K] -> C[I,K] on a named device mesh.

TEST INFRASTRUCTURE: part of the oracle. Written only from the pages'
rules; shares no code with the C++ planner of the HIP library.

Rules followed (page, section):
  * Notation, one axis per dimension at most, replication by unmentioned
    axes: lingze.zone "Cheetsheet ...", section "Notation"; learntpu.dev
    ch05, section "Notation" (table of subscripts and PartitionSpecs and the
    two rules under it).
  * The four cases: lingze.zone, sections "Case 1" .. "Case 4" and
    "Summary"; learntpu.dev ch05, section "The four cases of a sharded
    matmul".
  * Unreduced partials {U_Y} and the AllReduce / ReduceScatter choice:
    learntpu.dev ch05, "Notation" (last row of the table) and "The four
    collectives and their cost" (table); semiaifoundry.com "The mechanism".
  * Payload accounting of the 2x2 exchange: semiaifoundry.com,
    "Engineering example".

Readings where the pages are silent (each listed in the design notes):
  * ranks are numbered row-major over the mesh axes in declared order;
  * a dimension split over several axes is flattened with the first listed
    axis major;
  * case 4 is checked before the J-sharding cases; J sharded on different
    axis lists in A and B is an error (J_MISMATCH);
  * reduce-scatter splits the rows (I) of each output block, and the
    reduced axes become the minor axes of I's sharding;
  * the partial with reduce coordinate y owns row block y of its group.
"""
from __future__ import annotations

import ast
import math
import re
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

Spec = Tuple[Tuple[str, ...], Tuple[str, ...]]

ELEM_BYTES = {"bf16": 2, "f32": 4}


class PlanError(Exception):
    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


# ----------------------------------------------------------------- parsing

def _entry(e) -> Tuple[str, ...]:
    if e is None:
        return ()
    if isinstance(e, str):
        return (e,)
    if isinstance(e, tuple) and all(isinstance(s, str) for s in e):
        return tuple(e)
    raise PlanError("SPEC", f"bad spec entry {e!r}")


_SUB_RE = re.compile(r"^\s*([A-Za-z]+)(?:_([A-Za-z]+))?\s*$")


def parse_spec(text: str, ndim: int = 2) -> Spec:
    """Parse a partition spec for a 2-D array.

    Accepted forms: ``P('X','Y')``, ``P(('X','Y'), None)``, ``P(None, None)``,
    ``P()``, the bare entry list ``('X','Y'), None``, and the subscript
    notation ``A[I_X, J_Y]`` / ``I_XY, J`` (single-letter axis names).
    """
    t = text.strip()
    if t == "" or t == "None":
        return ((), ())
    m = re.match(r"^[A-Za-z0-9]*\[(.*)\]$", t)
    quoted = "'" in t or '"' in t
    if m or (not quoted and not t.startswith("P") and "None" not in t):
        body = m.group(1) if m else t
        parts = [p for p in body.split(",")]
        if len(parts) > ndim:
            raise PlanError("SPEC", f"too many dims in {text!r}")
        out: List[Tuple[str, ...]] = []
        for p in parts:
            mm = _SUB_RE.match(p)
            if not mm:
                raise PlanError("SPEC", f"bad subscript {p!r}")
            out.append(tuple(mm.group(2)) if mm.group(2) else ())
        while len(out) < ndim:
            out.append(())
        return (out[0], out[1])
    m = re.match(r"^P\s*\((.*)\)$", t, re.S)
    inner = m.group(1) if m else t
    if inner.strip() == "":
        entries: Sequence = ()
    else:
        try:
            val = ast.literal_eval("(" + inner + ",)")
        except Exception as exc:  # noqa: BLE001
            raise PlanError("SPEC", f"cannot parse {text!r}: {exc}") from None
        entries = val
    if len(entries) > ndim:
        raise PlanError("SPEC", f"too many dims in {text!r}")
    dims = [_entry(e) for e in entries]
    while len(dims) < ndim:
        dims.append(())
    return (dims[0], dims[1])


# --------------------------------------------------------------- the plan

@dataclass
class Plan:
    case: int
    mesh: Tuple[Tuple[str, int], ...]
    I: int
    J: int
    K: int
    a: Spec
    b: Spec
    in_dtype: str
    out_dtype: str
    a_local: Tuple[int, int]
    b_local: Tuple[int, int]
    c_local: Tuple[int, int]
    a_grid: Tuple[int, int]
    b_grid: Tuple[int, int]
    c_grid: Tuple[int, int]
    a_copies: int
    b_copies: int
    c_copies: int
    c_spec: Spec                 # spec of the local products (before any reduce)
    c_rs_spec: Optional[Spec]    # case 3: spec after reduce-scatter
    unreduced: Tuple[str, ...]   # case 3: axes still to be summed ({U_...})
    n_partials: int              # N
    n_groups: int                # G (distinct output blocks)
    gather_operand: Optional[str]  # case 2 / 4: "A" or "B"
    gather_axes: Tuple[str, ...]

    # ---- mesh helpers
    @property
    def sizes(self) -> Dict[str, int]:
        return dict(self.mesh)

    @property
    def n_ranks(self) -> int:
        return math.prod(s for _, s in self.mesh)

    @property
    def n_units(self) -> int:
        return self.n_groups * self.n_partials

    def coords(self, rank: int) -> Dict[str, int]:
        out = {}
        r = rank
        for name, size in reversed(self.mesh):
            out[name] = r % size
            r //= size
        return out

    def rank_of(self, coords: Dict[str, int]) -> int:
        r = 0
        for name, size in self.mesh:
            r = r * size + coords.get(name, 0)
        return r

    def block_index(self, axes: Tuple[str, ...], coords: Dict[str, int]) -> int:
        idx = 0
        for a in axes:
            idx = idx * self.sizes[a] + coords[a]
        return idx

    # ---- per-rank view
    def rank_blocks(self, rank: int) -> Dict[str, Tuple[int, int]]:
        c = self.coords(rank)
        return {
            "A": (self.block_index(self.a[0], c), self.block_index(self.a[1], c)),
            "B": (self.block_index(self.b[0], c), self.block_index(self.b[1], c)),
            "C": (self.block_index(self.a[0], c), self.block_index(self.b[1], c)),
        }

    def rank_unit(self, rank: int) -> int:
        if self.case not in (1, 3):
            raise PlanError("NEEDS_GATHER", f"case {self.case} has no local units")
        c = self.coords(rank)
        g = self.block_index(self.a[0], c) * self.c_grid[1] + self.block_index(self.b[1], c)
        y = self.block_index(self.unreduced, c) if self.case == 3 else 0
        return g * self.n_partials + y

    def unit_rank(self, unit: int) -> int:
        """Lowest rank computing this unit (replica axes at coordinate 0)."""
        for r in range(self.n_ranks):
            if self.rank_unit(r) == unit:
                return r
        raise PlanError("ARG", f"unit {unit} out of range")

    def unit_blocks(self, unit: int) -> Dict[str, Tuple[int, int]]:
        return self.rank_blocks(self.unit_rank(unit))

    def unit_views(self, unit: int):
        """(row0, col0, rows, cols) of A, B and C for a unit, in global coordinates."""
        bl = self.unit_blocks(unit)
        (am, ak), (bk, bn), (cm, cn) = self.a_local, self.b_local, self.c_local
        return {
            "A": (bl["A"][0] * am, bl["A"][1] * ak, am, ak),
            "B": (bl["B"][0] * bk, bl["B"][1] * bn, bk, bn),
            "C": (bl["C"][0] * cm, bl["C"][1] * cn, cm, cn),
        }

    def rs_rows(self, group: int, y: int) -> Tuple[int, int]:
        """Global (row0, rows) that reduce coordinate y of group g owns after RS."""
        m = self.c_local[0]
        if m % self.n_partials:
            raise PlanError("INDIVISIBLE", "rows of a block do not split N ways")
        gi = group // self.c_grid[1]
        step = m // self.n_partials
        return gi * m + y * step, step

    # ---- sizes and work
    def shard_bytes(self, which: str, dtype: Optional[str] = None) -> int:
        shape = {"A": self.a_local, "B": self.b_local, "C": self.c_local}[which]
        dt = dtype or (self.in_dtype if which in "AB" else self.out_dtype)
        return shape[0] * shape[1] * ELEM_BYTES[dt]

    def local_flops(self) -> int:
        m, k = self.a_local
        return 2 * m * k * self.b_local[1]

    def exchange_bytes(self) -> Dict[str, int]:
        """Payload each rank sends, counted once at the link boundary.

        Reduce-scatter: each rank passes on the N-1 row blocks it does not
        own; all-gather: each rank's owned block goes to the N-1 others
        (ring or direct alike).
        """
        if self.case != 3:
            return {"rs": 0, "ag": 0, "ar": 0}
        m, n = self.c_local
        N = self.n_partials
        blk = (m // N) * n * ELEM_BYTES[self.out_dtype]
        rs = (N - 1) * blk
        ag = (N - 1) * blk
        return {"rs": rs, "ag": ag, "ar": rs + ag}


def _validate_mesh(mesh) -> Tuple[Tuple[str, int], ...]:
    mesh = tuple((str(n), int(s)) for n, s in (mesh.items() if isinstance(mesh, dict) else mesh))
    if not mesh or len(mesh) > 4:
        raise PlanError("MESH", "1 to 4 axes")
    names = [n for n, _ in mesh]
    if len(set(names)) != len(names):
        raise PlanError("MESH", "duplicate axis names")
    if any(s < 1 for _, s in mesh):
        raise PlanError("MESH", "axis sizes must be >= 1")
    return mesh


def _validate_spec(spec: Spec, sizes: Dict[str, int], what: str) -> None:
    seen = []
    for dim in spec:
        for a in dim:
            if a not in sizes:
                raise PlanError("SPEC", f"{what}: unknown axis {a!r}")
            if a in seen:
                raise PlanError("AXIS_REUSED", f"{what}: axis {a!r} shards two dimensions")
            seen.append(a)


def _split(total: int, axes: Tuple[str, ...], sizes: Dict[str, int], what: str) -> Tuple[int, int]:
    parts = math.prod(sizes[a] for a in axes)
    if total % parts:
        raise PlanError("INDIVISIBLE", f"{what}: {total} does not split {parts} ways")
    return total // parts, parts


def plan(mesh, a, b, I: int, J: int, K: int, in_dtype: str = "bf16", out_dtype: str = "f32") -> Plan:
    mesh = _validate_mesh(mesh)
    sizes = dict(mesh)
    if isinstance(a, str):
        a = parse_spec(a)
    if isinstance(b, str):
        b = parse_spec(b)
    a = (tuple(a[0]), tuple(a[1]))
    b = (tuple(b[0]), tuple(b[1]))
    if min(I, J, K) < 1:
        raise PlanError("SHAPE", "dimensions must be >= 1")
    _validate_spec(a, sizes, "A")
    _validate_spec(b, sizes, "B")

    a_used = set(a[0]) | set(a[1])
    b_used = set(b[0]) | set(b[1])
    a_copies = math.prod(s for n, s in mesh if n not in a_used)
    b_copies = math.prod(s for n, s in mesh if n not in b_used)

    am, ga0 = _split(I, a[0], sizes, "A rows")
    ak, ga1 = _split(J, a[1], sizes, "A cols")
    bk, gb0 = _split(J, b[0], sizes, "B rows")
    bn, gb1 = _split(K, b[1], sizes, "B cols")

    shared_out = set(a[0]) & set(b[1])
    gather_operand = None
    gather_axes: Tuple[str, ...] = ()
    unreduced: Tuple[str, ...] = ()
    if shared_out:
        case = 4
        # fix: gather the smaller operand over the shared axes (tie -> A)
        a_bytes = I * J
        b_bytes = J * K
        gather_operand = "A" if a_bytes <= b_bytes else "B"
        src = a[0] if gather_operand == "A" else b[1]
        gather_axes = tuple(x for x in src if x in shared_out)
    elif a[1] and b[0]:
        if a[1] != b[0]:
            raise PlanError("J_MISMATCH", f"A shards J over {a[1]}, B over {b[0]}")
        case = 3
        unreduced = a[1]
    elif a[1] or b[0]:
        case = 2
        gather_operand = "A" if a[1] else "B"
        gather_axes = a[1] if a[1] else b[0]
    else:
        case = 1

    c_spec: Spec = (a[0], b[1])
    c_rs_spec = (a[0] + unreduced, b[1]) if case == 3 else None
    n_partials = math.prod(sizes[x] for x in unreduced) if case == 3 else 1
    n_groups = ga0 * gb1
    c_used = set(a[0]) | set(b[1]) | set(unreduced)
    c_copies = math.prod(s for n, s in mesh if n not in c_used)
    return Plan(
        case=case, mesh=mesh, I=I, J=J, K=K, a=a, b=b,
        in_dtype=in_dtype, out_dtype=out_dtype,
        a_local=(am, ak), b_local=(bk, bn), c_local=(am, bn),
        a_grid=(ga0, ga1), b_grid=(gb0, gb1), c_grid=(ga0, gb1),
        a_copies=a_copies, b_copies=b_copies, c_copies=c_copies,
        c_spec=c_spec, c_rs_spec=c_rs_spec, unreduced=unreduced,
        n_partials=n_partials, n_groups=n_groups,
        gather_operand=gather_operand, gather_axes=gather_axes,
    )


def array_blocks(mesh, spec, rows: int, cols: int):
    """Distinct blocks of one 2-D array under a spec: {block_id: (r0, c0,
    rows, cols)}, block_id = row_block * grid[1] + col_block (learntpu.dev
    ch05 sandbox: "A: 4 x 2 blocks of [2048, 14336]")."""
    mesh = _validate_mesh(mesh)
    sizes = dict(mesh)
    if isinstance(spec, str):
        spec = parse_spec(spec)
    spec = (tuple(spec[0]), tuple(spec[1]))
    _validate_spec(spec, sizes, "array")
    br, gr = _split(rows, spec[0], sizes, "rows")
    bc, gc = _split(cols, spec[1], sizes, "cols")
    return {i * gc + j: (i * br, j * bc, br, bc) for i in range(gr) for j in range(gc)}


def gathered(p: Plan) -> Plan:
    """The plan after the case-2 / case-4 fix: all-gather ``p.gather_operand``
    over ``p.gather_axes`` (lingze.zone "Case 2" and "Case 4"; learntpu.dev
    ch05, the four cases), i.e. drop those axes from that operand's spec and
    plan again."""
    if p.case not in (2, 4):
        raise PlanError("CASE", "nothing to gather")
    drop = set(p.gather_axes)

    def strip(spec: Spec) -> Spec:
        return (tuple(a for a in spec[0] if a not in drop), tuple(a for a in spec[1] if a not in drop))

    a = strip(p.a) if p.gather_operand == "A" else p.a
    b = strip(p.b) if p.gather_operand == "B" else p.b
    return plan(p.mesh, a, b, p.I, p.J, p.K, p.in_dtype, p.out_dtype)


def notation(name: str, spec: Spec, dims=("I", "J"), unreduced: Tuple[str, ...] = ()) -> str:
    """Subscript notation of the pages, e.g. A[I_X, J_Y]{U_Y}."""
    parts = []
    for d, axes in zip(dims, spec):
        parts.append(d + ("_" + "".join(axes) if axes else ""))
    s = f"{name}[{', '.join(parts)}]"
    if unreduced:
        s += "{U_" + "".join(unreduced) + "}"
    return s
