"""Seeded synthetic operands for the sharded-matmul workloads.

This module holds shapes, meshes, partition specs, seeds and value
distributions only. It contains no step of the sharded-matmul arithmetic
(no products, sums, reductions or layouts of shards), so both the HIP path
(tests, bench) and the CPU oracle can draw identical bytes from it while
sharing nothing else.

Value recipes
-------------
* ``normal``: ``numpy.random.default_rng(seed).standard_normal(shape,
  dtype=float32) * sigma``, then rounded to bfloat16 with round-to-nearest-
  even (``torch.Tensor.to(torch.bfloat16)``).
* ``int``: ``default_rng(seed).integers(-4, 5, shape)``, i.e. the nine
  integers -4..4 with equal probability, stored as bfloat16 (exact: every
  integer of magnitude <= 256 is a bfloat16 value).

Dense, no structure and no sparsity, as the pages' workloads are plain
dense matrices (the learntpu.dev chapter's sharding sandbox: a tensor-
parallel down-projection; the Megatron MLP pair on the row-parallelism page
and in "The simple maths behind parallel training").
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

__all__ = ["Operand", "Workload", "WORKLOADS", "get", "make_operand", "int_variant"]


@dataclass(frozen=True)
class Operand:
    name: str
    shape: Tuple[int, int]
    spec: str            # partition spec text, JAX PartitionSpec form
    dist: str            # "normal" or "int"
    sigma: float
    seed: int


@dataclass(frozen=True)
class Workload:
    name: str
    mesh: Tuple[Tuple[str, int], ...]
    operands: Tuple[Operand, ...]
    note: str = ""
    extra: Dict[str, object] = field(default_factory=dict)

    def operand(self, name: str) -> Operand:
        for op in self.operands:
            if op.name == name:
                return op
        raise KeyError(name)


# Case-3 toy: J split over two logical ranks; integer values (exact in fp32).
TOY = Workload(
    name="toy_case3_64x128x64",
    mesh=(("X", 2),),
    operands=(
        Operand("A", (64, 128), "P(None, 'X')", "int", 1.0, 1001),
        Operand("B", (128, 64), "P('X', None)", "int", 1.0, 1002),
    ),
    note="A[I,J_X].B[J_X,K], N=2 partials [64,64]; all-reduce and reduce-scatter (row halves)",
)

# Case 1 (no communication): mesh {X:4,Y:2}, A[I_X,J].B[J,K_Y], I=J=K=4096.
CASE1 = Workload(
    name="case1_4096_x4y2",
    mesh=(("X", 4), ("Y", 2)),
    operands=(
        Operand("A", (4096, 4096), "P('X', None)", "normal", 1.0, 2001),
        Operand("B", (4096, 4096), "P(None, 'Y')", "normal", 1.0, 2002),
    ),
    note="8 local blocks C[1024,2048], then gathered to a replicated C[4096,4096]",
)

# Case 3 down-projection shard (the sandbox default): mesh {X:4,Y:2},
# A[I_X,J_Y] with I=8192, J=28672; B[J_Y,K] with K=8192.
DOWN_PROJ = Workload(
    name="case3_downproj_8192x28672x8192_x4y2",
    mesh=(("X", 4), ("Y", 2)),
    operands=(
        Operand("A", (8192, 28672), "P('X', 'Y')", "normal", 0.02, 3001),
        Operand("B", (28672, 8192), "P('Y', None)", "normal", 0.02, 3002),
    ),
    note="per-rank A shard [2048,14336], B shard [14336,8192]; two Y-partials "
         "[2048,8192] fp32 per X-group, reduce-scattered to [1024,8192] row blocks",
)

# Megatron column->row MLP chain on {T:4}.
MLP_CHAIN = Workload(
    name="megatron_mlp_4096x16384_t4",
    mesh=(("T", 4),),
    operands=(
        Operand("X", (4096, 4096), "P(None, None)", "normal", 1.0, 4001),
        Operand("W1", (4096, 16384), "P(None, 'T')", "normal", 0.02, 4002),
        Operand("W2", (16384, 4096), "P('T', None)", "normal", 0.02, 4003),
    ),
    note="column-sharded W1, GeLU(tanh), row-sharded W2; 4 fp32 partials "
         "[4096,4096] all-reduced; no gather between the layers",
)

# Skinny split-J (bandwidth bound): X[16,28672].A[28672,8192], J split 8 ways.
SKINNY = Workload(
    name="skinny_splitj_16x28672x8192_t8",
    mesh=(("T", 8),),
    operands=(
        Operand("X", (16, 28672), "P(None, 'T')", "normal", 1.0, 5001),
        Operand("A", (28672, 8192), "P('T', None)", "normal", 0.02, 5002),
    ),
    note="8 fp32 partials [16,8192], reduced in rank order",
)

WORKLOADS: Dict[str, Workload] = {
    "toy": TOY,
    "case1": CASE1,
    "downproj": DOWN_PROJ,
    "mlp": MLP_CHAIN,
    "skinny": SKINNY,
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def int_variant(w: Workload) -> Workload:
    """Same shapes and specs, values = integers -4..4, seeds + 500."""
    ops = tuple(Operand(o.name, o.shape, o.spec, "int", 1.0, o.seed + 500) for o in w.operands)
    return Workload(w.name + "_int", w.mesh, ops, w.note + " (integer values)", dict(w.extra))


def _normal_f32(shape, sigma: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def _int_f32(shape, seed: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def make_operand(op: Operand, shape=None):
    """Return the operand as a CPU torch.bfloat16 tensor (the stored bytes).

    ``shape`` overrides the operand's own shape (used for reduced-size
    parity cases that keep the value recipe and seed).
    """
    import torch

    shp = tuple(shape) if shape is not None else op.shape
    if op.dist == "normal":
        x = _normal_f32(shp, op.sigma, op.seed)
    elif op.dist == "int":
        x = _int_f32(shp, op.seed)
    else:
        raise ValueError(op.dist)
    return torch.from_numpy(x).to(torch.bfloat16)


def random_ints(shape, seed: int, lo: int = -4, hi: int = 4):
    """Integer-valued bfloat16 tensor of any shape (edge-case parity inputs)."""
    import torch

    return torch.from_numpy(_int_f32(shape, seed, lo, hi)).to(torch.bfloat16)


def random_normal(shape, seed: int, sigma: float = 1.0):
    """Normal bfloat16 tensor of any shape (edge-case parity inputs)."""
    import torch

    return torch.from_numpy(_normal_f32(shape, sigma, seed)).to(torch.bfloat16)


def mesh_dict(w: Workload) -> Dict[str, int]:
    return dict(w.mesh)


def mesh_names(w: Workload) -> List[str]:
    return [a for a, _ in w.mesh]
