"""The oracle's pins must catch plausible slips in the oracle (CPU only).

Each mutant below plants one mistake in a copy of the oracle's source: a
dropped term, an operand read through the wrong index, a wrong sign, a
rounding step done in the wrong precision, a rule of the planner read the
wrong way. The mutated oracle is installed in this process, every test of
``test_oracle_pins.py`` and ``test_oracle_planner.py`` is run against it,
and at least one of them must fail. A mutant that every pin accepts is a
gap in the pins.

* C mutants are compiled from a patched ``oracle.c`` with the oracle's own
  build command and loaded in place of ``liboracle.so``. They are chosen so
  that every memory access stays inside the operands' buffers (a dropped
  leading dimension, not a transposed one), so a slip cannot crash the
  test process.
* Python mutants are executed from a patched ``reference.py`` or
  ``planner.py`` as modules of the ``oracle`` package, and their functions
  and classes replace the real ones for the duration of one run.

Every patch must match its source exactly once, so an edit of the oracle
that moves a mutated line fails here and asks for the list to be updated.
"""
import importlib.util
import os
import sys
import types

import pytest

import oracle.build as obuild
from oracle import planner as oplanner
from oracle import reference as oref

HERE = os.path.dirname(os.path.abspath(__file__))
PIN_FILES = ("test_oracle_pins.py", "test_oracle_planner.py")


# ------------------------------------------------------------- the mutants

C_MUTANTS = {
    "matmul: first product of each sum dropped":
        ("for (int64_t j = 0; j < J; ++j) {\n      double a", "for (int64_t j = 1; j < J; ++j) {\n      double a"),
    "matmul: A read without its leading dimension":
        ("double a = elem(A, akind, i * lda + j);", "double a = elem(A, akind, i + j);"),
    "matmul: float64 B read without its leading dimension":
        ("const double* b = (const double*)B + j * ldb;", "const double* b = (const double*)B + j;"),
    "matmul: sampled rows ignored":
        ("int64_t i = rows ? rows[t] : t;", "int64_t i = t;"),
    "matmul: float32 B multiplied in float32":
        ("c[k] += a * (double)b[k];", "c[k] += (double)((float)a * b[k]);"),
    "matmul: bfloat16 B bits used as a number":
        ("c[k] += a * bf16_bits_to_double(b[k]);", "c[k] += a * (double)b[k];"),
    "bfloat16 widened from the wrong bits":
        ("uint32_t bits = (uint32_t)h << 16;", "uint32_t bits = (uint32_t)h << 15;"),
    "entries: B column taken from the sample's row":
        ("elem(B, bkind, j * ldb + ci[t])", "elem(B, bkind, j * ldb + ci[t] / 2)"),
    "matvec: vector indexed by the row":
        ("s += elem(M, kind, i * ld + j) * v[j];", "s += elem(M, kind, i * ld + j) * v[j / 2];"),
    "rank-ordered sum: last partial dropped":
        ("for (int r = 1; r < N; ++r) s += P", "for (int r = 1; r < N - 1; ++r) s += P"),
    "rank-ordered sum: first partial dropped":
        ("double s = P[e];", "double s = 0.0 * P[e];"),
    "rank-ordered sum: partials subtracted":
        ("s += P[(int64_t)r * stride + e];", "s -= P[(int64_t)r * stride + e];"),
    "GeLU: cubic coefficient truncated":
        ("0.044715 * x * x * x", "0.0447 * x * x * x"),
    "GeLU: square instead of cube":
        ("0.044715 * x * x * x", "0.044715 * x * x"),
    "GeLU: sqrt(1/pi) instead of sqrt(2/pi)":
        ("sqrt(2.0 / 3.14159265358979323846)", "sqrt(1.0 / 3.14159265358979323846)"),
    "GeLU: factor one half dropped":
        ("return 0.5 * x * (1.0 + tanh(", "return x * (1.0 + tanh("),
    "bfloat16 rounding: nine significant bits":
        ("int qexp = e - 8;", "int qexp = e - 9;"),
    "bfloat16 rounding: ties away from zero":
        ("double r = nearbyint(ax / q) * q;", "double r = round(ax / q) * q;"),
    "bfloat16 rounding: truncation":
        ("double r = nearbyint(ax / q) * q;", "double r = trunc(ax / q) * q;"),
    "bfloat16 rounding: subnormals flushed to the normal spacing":
        ("if (qexp < -133) qexp = -133;", "if (qexp < -126) qexp = -126;"),
    "bfloat16 rounding: through float32 first":
        ("double ax = fabs(x);", "double ax = (double)(float)fabs(x);"),
    "bfloat16 rounding: sign dropped":
        ("uint16_t sign = signbit(x) ? 0x8000 : 0;", "uint16_t sign = 0;"),
    "bfloat16 rounding: largest finite value one step too small":
        ("double maxf = ldexp(255.0, 120);", "double maxf = ldexp(254.0, 120);"),
}

REF_MUTANTS = {
    "reduce-scatter: row blocks given to the wrong coordinate":
        ("out[(g, y)] = s[y * step:(y + 1) * step].copy()",
         "out[(g, y)] = s[(N - 1 - y) * step:(N - y) * step].copy()"),
    "group sum: partials taken group-minor":
        ("return sum_ranked([parts[g * N + y] for y in range(N)])",
         "return sum_ranked([parts[g + y * plan.n_groups] for y in range(N)])"),
    "gather: block row and column swapped":
        ("bi, bk = divmod(g, plan.c_grid[1])", "bk, bi = divmod(g, plan.c_grid[0])"),
    "scattered gather: every row block at its group's start":
        ("r0, rows = plan.rs_rows(g, y)", "r0, rows = plan.rs_rows(g, 0)"),
    "per-rank all-reduce output indexed by the rank's partial, not its group":
        ("return {r: sums[plan.rank_unit(r) // plan.n_partials] for r in range(plan.n_ranks)}",
         "return {r: sums[plan.rank_unit(r) % plan.n_partials] for r in range(plan.n_ranks)}"),
    "gather of partials accepted":
        ("if plan.case == 3 and plan.n_partials > 1:", "if False:"),
    "layer norm: unbiased variance":
        ("var = (d * d).sum(axis=-1, keepdims=True) / n", "var = (d * d).sum(axis=-1, keepdims=True) / (n - 1)"),
    "layer norm: epsilon outside the square root":
        ("y = d / np.sqrt(var + eps)", "y = d / (np.sqrt(var) + eps)"),
    "layer norm: shift and scale swapped":
        ("y = y + np.asarray(beta, dtype=np.float64)", "y = y + np.asarray(gamma, dtype=np.float64)"),
    "MLP chain: GeLU skipped":
        ("hs.append(round_bf16(gelu_tanh(y)))", "hs.append(round_bf16(y))"),
    "MLP chain: every unit reads H from column 0":
        ("hv = (0, v[\"A\"][1], H.shape[0], Hk)", "hv = (0, 0, H.shape[0], Hk)"),
    "reshard: source blocks read under the target spec":
        ("return shard(unshard(blocks, mesh, frm, rows, cols), mesh, to)",
         "return shard(unshard(blocks, mesh, to, rows, cols), mesh, to)"),
    "Freivalds: the check multiplies C by B v":
        ("cv = view_matvec(Cw, (0, 0, Cw.shape[0], Cw.shape[1]), v)",
         "cv = view_matvec(Cw, (0, 0, Cw.shape[0], Cw.shape[1]), v) * 0 + y"),
    "relative Frobenius error without the norm of the reference":
        ("return num / den if den else num", "return num"),
}

PLANNER_MUTANTS = {
    "ranks numbered column-major":
        ("for name, size in reversed(self.mesh):", "for name, size in self.mesh:"),
    "split dimension flattened with the last axis major":
        ("for a in axes:\n            idx = idx * self.sizes[a] + coords[a]",
         "for a in reversed(axes):\n            idx = idx * self.sizes[a] + coords[a]"),
    "case 4 never detected":
        ("if shared_out:\n        case = 4", "if False:\n        case = 4"),
    "mismatched J sharding accepted":
        ("if a[1] != b[0]:", "if False:"),
    "case 2 gathers the other operand":
        ("gather_operand = \"A\" if a[1] else \"B\"", "gather_operand = \"B\" if a[1] else \"A\""),
    "case 4 gathers the larger operand":
        ("gather_operand = \"A\" if a_bytes <= b_bytes else \"B\"",
         "gather_operand = \"B\" if a_bytes <= b_bytes else \"A\""),
    "axis reuse accepted":
        ("if a in seen:", "if False:"),
    "copies counted over the used axes":
        ("a_copies = math.prod(s for n, s in mesh if n not in a_used)",
         "a_copies = math.prod(s for n, s in mesh if n in a_used)"),
    "reduced axes made major in the scattered spec":
        ("c_rs_spec = (a[0] + unreduced, b[1]) if case == 3 else None",
         "c_rs_spec = (unreduced + a[0], b[1]) if case == 3 else None"),
    "groups counted over the operands' J grid":
        ("n_groups = ga0 * gb1", "n_groups = ga0 * ga1"),
    "unit B view starts at column 0":
        ("\"B\": (bl[\"B\"][0] * bk, bl[\"B\"][1] * bn, bk, bn),", "\"B\": (bl[\"B\"][0] * bk, 0, bk, bn),"),
    "unit A view starts at column 0":
        ("\"A\": (bl[\"A\"][0] * am, bl[\"A\"][1] * ak, am, ak),", "\"A\": (bl[\"A\"][0] * am, 0, am, ak),"),
    "reduce-scatter rows offset by group column":
        ("gi = group // self.c_grid[1]", "gi = group % max(self.c_grid[0], 1)"),
    "exchange bytes count the owned block too":
        ("rs = (N - 1) * blk", "rs = N * blk"),
    "multi-axis subscript read as one axis":
        ("out.append(tuple(mm.group(2)) if mm.group(2) else ())",
         "out.append((mm.group(2),) if mm.group(2) else ())"),
    "indivisible dimension rounded down":
        ("if total % parts:", "if False:"),
    "local FLOPs counted once per multiply-add pair":
        ("return 2 * m * k * self.b_local[1]", "return m * k * self.b_local[1]"),
}


# ---------------------------------------------------------------- machinery

def _patched(text, old, new, what):
    assert text.count(old) == 1, f"{what}: the mutated text must occur exactly once in the oracle source"
    return text.replace(old, new)


def _load_pin_module(name):
    path = os.path.join(HERE, name)
    spec = importlib.util.spec_from_file_location(f"_pins_{name[:-3]}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _expand(fn):
    """Calls of one test function: its parametrize marks expanded."""
    calls = [{}]
    for mark in getattr(fn, "pytestmark", []):
        if mark.name != "parametrize":
            continue
        names, values = mark.args[0], mark.args[1]
        names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
        new = []
        for base in calls:
            for v in values:
                v = v.values if hasattr(v, "values") and not isinstance(v, (tuple, list)) else v
                vals = v if len(names) > 1 else (v,)
                new.append({**base, **dict(zip(names, vals))})
        calls = new
    return calls


def _run_pins():
    """Run every pin; return the names of those that failed."""
    failed = []
    for f in PIN_FILES:
        mod = _load_pin_module(f)  # fresh, so `from oracle.x import y` sees the installed mutant
        for name in sorted(dir(mod)):
            fn = getattr(mod, name)
            if not (name.startswith("test_") and callable(fn)):
                continue
            for kwargs in _expand(fn):
                try:
                    fn(**kwargs)
                except (Exception, pytest.fail.Exception):  # noqa: BLE001 - any failure kills the mutant
                    failed.append(f"{f}::{name}{kwargs or ''}")
    return failed


class _Installed:
    """Replace module attributes for one run and put them back after."""

    def __init__(self):
        self.saved = []

    def set(self, obj, name, value):
        self.saved.append((obj, name, getattr(obj, name)))
        setattr(obj, name, value)

    def undo(self):
        for obj, name, value in reversed(self.saved):
            setattr(obj, name, value)
        self.saved.clear()


def _exec_module(src_path, text, real):
    name = f"oracle._mutant_{os.path.basename(src_path)[:-3]}"
    mod = types.ModuleType(name)
    mod.__file__ = src_path
    mod.__package__ = "oracle"
    sys.modules[name] = mod  # dataclasses look their module up while the class is made
    try:
        exec(compile(text, src_path, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    if "PlanError" in mod.__dict__:
        mod.PlanError = oplanner.PlanError  # the pins match errors by this class
    inst = _Installed()
    for key, val in mod.__dict__.items():
        if key.startswith("__") or key == "PlanError":
            continue
        if getattr(val, "__module__", None) == name:
            inst.set(real, key, val)
    return inst


@pytest.fixture(scope="module")
def c_source():
    with open(obuild.SRC) as f:
        return f.read()


def _run_c_mutant(tmp_path, text):
    src = tmp_path / "oracle.c"
    src.write_text(text)
    inst = _Installed()
    inst.set(obuild, "SRC", str(src))
    inst.set(obuild, "LIB", str(tmp_path / "liboracle.so"))
    try:
        obuild.build()
        inst.set(obuild, "_lib", None)
        obuild.load_library()
        return _run_pins()
    finally:
        inst.undo()


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins() == []


def test_unmutated_c_build_passes_every_pin(tmp_path, c_source):
    """The harness itself: the oracle rebuilt from an unchanged copy."""
    assert _run_c_mutant(tmp_path, c_source) == []


@pytest.mark.parametrize("what", sorted(C_MUTANTS))
def test_c_mutant_is_caught(what, tmp_path, c_source):
    old, new = C_MUTANTS[what]
    failed = _run_c_mutant(tmp_path, _patched(c_source, old, new, what))
    assert failed, f"no pin fails when the oracle has: {what}"


@pytest.mark.parametrize("what", sorted(REF_MUTANTS))
def test_reference_mutant_is_caught(what):
    old, new = REF_MUTANTS[what]
    with open(oref.__file__) as f:
        text = _patched(f.read(), old, new, what)
    inst = _exec_module(oref.__file__, text, oref)
    try:
        failed = _run_pins()
    finally:
        inst.undo()
    assert failed, f"no pin fails when the oracle has: {what}"


@pytest.mark.parametrize("what", sorted(PLANNER_MUTANTS))
def test_planner_mutant_is_caught(what):
    old, new = PLANNER_MUTANTS[what]
    with open(oplanner.__file__) as f:
        text = _patched(f.read(), old, new, what)
    inst = _exec_module(oplanner.__file__, text, oplanner)
    try:
        failed = _run_pins()
    finally:
        inst.undo()
    assert failed, f"no pin fails when the oracle has: {what}"
