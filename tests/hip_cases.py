"""Helpers shared by the GPU parity tests: device buffers, HIP-path calls
through the C-ABI binding, and comparisons with the oracle.

Comparison rules
  * integer-valued inputs: the GPU float32 result must equal the oracle's
    float64 value converted to float32, bit for bit (every partial sum is an
    integer below 2^24 in magnitude, so both sides are exact);
  * random bfloat16 inputs: relative Frobenius error <= 1e-3 against the
    float64 oracle (REL_TOL).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import local_shard_gemm_amd as sm
from oracle import reference as ref

REL_TOL = 1e-3
DEV = "cuda:0"
SENTINEL = float("nan")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(t: torch.Tensor) -> torch.Tensor:
    return t.to(DEV, non_blocking=False).contiguous()


def guarded(shape, dtype, pad=4096):
    """Device buffer with a sentinel-filled guard band after the payload.

    Returns (full, view): view is the first prod(shape) elements reshaped.
    """
    n = int(np.prod(shape))
    full = torch.full((n + pad,), SENTINEL if dtype.is_floating_point else 0, dtype=dtype, device=DEV)
    return full, full[:n].view(*shape)


def guard_intact(full: torch.Tensor, n: int) -> bool:
    tail = full[n:]
    return bool(torch.isnan(tail.float()).all().item())


def f32_bits_equal(gpu: np.ndarray, oracle64: np.ndarray) -> bool:
    want = oracle64.astype(np.float32)
    return gpu.shape == want.shape and np.array_equal(gpu.view(np.uint32), want.view(np.uint32))


def run_partials(plan, A_dev, B_dev, unit_begin=0, unit_count=None, stream=None):
    """Local products of a case-1/3 plan into a stacked fp32 (or bf16) buffer."""
    if unit_count is None:
        unit_count = plan.n_units - unit_begin
    m, n = plan.c_local
    dt = torch.float32 if plan.out_dtype == sm.SM_F32 else torch.bfloat16
    full, C = guarded((unit_count, m, n), dt)
    sm.sm_local_gemm(plan, sm.buf(A_dev), sm.buf(B_dev), sm.buf(C), sm.SM_EPI_STORE, unit_begin, unit_count,
                     stream)
    return full, C


def sample_rows(m: int, k: int, seed: int):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(m, size=min(k, m), replace=False).tolist())
    rows.update({0, m - 1})
    return sorted(rows)
