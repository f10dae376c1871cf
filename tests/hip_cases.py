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


# Probabilistic rounding-error bound for the GPU's float32 pre-activation
# (Higham & Mary, "A new approach to probabilistic rounding error analysis",
# SIAM J. Sci. Comput. 41 (2019), their inner-product bound): an inner
# product of k exact products accumulated in float32 (unit roundoff
# u = 2^-24), with rounding errors independent and of mean zero, is within
#   lambda * sqrt(k) * u * sum_j |x_j w_j|
# of the exact value with probability at least 1 - 2k exp(-lambda^2 / 2).
# lambda = 8 puts that failure probability below 1e-10 per element at
# k = 4096 (below 0.01 over all 67 M elements of the MLP's H). The
# deterministic worst case is k u sum|x w|, sqrt(k) / lambda = 8 times
# looser at k = 4096.
GELU_LAMBDA = 8.0


def gelu_h_within_bound(h_gpu_bits, h_oracle_bits, abs_dot: np.ndarray, k: int) -> np.ndarray:
    """Elementwise check of bfloat16 GeLU outputs against the oracle.

    The GPU's float32 pre-activation differs from the exact one by at most
    GELU_LAMBDA * sqrt(k) * 2^-24 * sum_j |x_j w_j| (see above); GeLU(tanh)
    has slope at most 1.13, the GPU's float32 GeLU adds a few float32 ulps
    (far below half a bfloat16 ulp), and each side rounds once to bfloat16.
    So
      |H_gpu - H_oracle| <= 1.13 * lambda * sqrt(k) * 2^-24 * sum|x w|
                            + ulp_bf16(max |H|).
    """
    hg = ref.bf16_bits_to_f64(np.asarray(h_gpu_bits))
    hw = ref.bf16_bits_to_f64(np.asarray(h_oracle_bits))
    bound = 1.13 * GELU_LAMBDA * np.sqrt(k) * 2.0 ** -24 * abs_dot + bf16_ulp(np.maximum(np.abs(hg), np.abs(hw)))
    return np.abs(hg - hw) <= bound


def h_ulp_stats(h_gpu_bits, h_oracle_bits) -> dict:
    """Differences of bfloat16 outputs in units of the bfloat16 spacing at
    the larger magnitude: fraction of elements that differ, the largest
    difference, and how many differ by more than one ulp."""
    hg = ref.bf16_bits_to_f64(np.asarray(h_gpu_bits))
    hw = ref.bf16_bits_to_f64(np.asarray(h_oracle_bits))
    ulps = np.abs(hg - hw) / bf16_ulp(np.maximum(np.abs(hg), np.abs(hw)))
    return {"differ": float((ulps > 0).mean()), "max_ulps": float(ulps.max()) if ulps.size else 0.0,
            "over_one_ulp": int((ulps > 1).sum()), "elements": int(ulps.size)}


# Whole-output check of a float product: Freivalds' residual
# |C v - A (B v)| / |A (B v)| for a Gaussian v estimates the relative
# Frobenius error of C (E|E v|^2 = |E|_F^2 for v ~ N(0, I)). float32
# accumulation of k exact bfloat16 products leaves that error near
# sqrt(k) * 2^-24 (about 1e-5 at k = 14336), while one output element wrong
# by its own magnitude in an m x n result moves the residual by about
# 1/sqrt(m n) (2.4e-4 for 4096 x 4096), a zeroed 16 x 16 block by 16 times
# that. 1e-4 separates the two.
FREIVALDS_FLOAT_TOL = 1e-4


def sample_rows(m: int, k: int, seed: int):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(m, size=min(k, m), replace=False).tolist())
    rows.update({0, m - 1})
    return sorted(rows)
