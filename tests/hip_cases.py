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


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |v| (8 significant bits)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, ex = np.frexp(a)
    return np.where(a > 0, np.ldexp(1.0, np.maximum(ex - 8, -133)), 2.0 ** -133)


def gelu_h_within_bound(h_gpu_bits, h_oracle_bits, abs_dot: np.ndarray, k: int) -> np.ndarray:
    """Elementwise check of bfloat16 GeLU outputs against the oracle.

    The GPU's float32 pre-activation differs from the exact one by at most
    k * 2^-24 * sum_j |x_j w_j| (a standard bound for recursive float32
    summation of k products, each exact); GeLU(tanh) has slope at most 1.13,
    and each side rounds once to bfloat16. So
      |H_gpu - H_oracle| <= 1.13 * k * 2^-24 * sum|x w| + ulp(max |H|).
    """
    hg = ref.bf16_bits_to_f64(np.asarray(h_gpu_bits))
    hw = ref.bf16_bits_to_f64(np.asarray(h_oracle_bits))
    bound = 1.13 * k * 2.0 ** -24 * abs_dot + bf16_ulp(np.maximum(np.abs(hg), np.abs(hw)))
    return np.abs(hg - hw) <= bound


def sample_rows(m: int, k: int, seed: int):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(m, size=min(k, m), replace=False).tolist())
    rows.update({0, m - 1})
    return sorted(rows)
