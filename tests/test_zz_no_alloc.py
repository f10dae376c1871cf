"""The no-allocation entry point, sm_local_gemm_reduce_noalloc, through the C
ABI: bit for bit the results of sm_local_gemm_reduce_ws (the entry point
whose kernels it shares, with the caller's workspace) on two calls in a
row, the second with a smaller input; the oracle pins the integer cases;
calls larger than the static scratch are refused before any launch."""
import pytest
import torch

import local_shard_gemm_amd as sm
import workloads as wl
from oracle import planner, reference as ref

from hip_cases import DEV, f32_bits_equal, guard_intact, guarded, say, to_dev

pytestmark = pytest.mark.gpu


def _both(p, A, B, mode, shape):
    """(no-allocation result, workspace result) of one call each."""
    ws = torch.zeros(sm.sm_gemm_reduce_workspace(p) // 4 + 64, dtype=torch.int32, device=DEV)
    fa, a = guarded(shape, torch.float32)
    sm.sm_local_gemm_reduce_noalloc(p, sm.buf(A), sm.buf(B), sm.buf(a), mode)
    b = torch.full(shape, float("nan"), device=DEV)
    sm.sm_local_gemm_reduce_ws(p, sm.buf(A), sm.buf(B), sm.buf(b), ws, mode)
    torch.cuda.synchronize()
    assert guard_intact(fa, a.numel())
    return a, b


def test_noalloc_two_calls_then_smaller():
    # 1: the skinny workload at full size (float), all-reduce
    w = wl.get("skinny")
    say("case: noalloc full skinny")
    X = to_dev(wl.make_operand(w.operand("X")))
    A = to_dev(wl.make_operand(w.operand("A")))
    p = sm.sm_plan(dict(w.mesh), w.operand("X").spec, w.operand("A").spec, 16, 28672, 8192)
    a, b = _both(p, X, A, sm.SM_ALLREDUCE, (16, 8192))
    assert torch.equal(a, b)
    del X, A
    # 2: a smaller input right after, integer-valued, reduce-scatter over two
    # groups; the scratch still holds the first call's partials and counters
    say("case: noalloc smaller")
    mesh, sa, sb, I, J, K = {"X": 2, "T": 4}, "P('X', 'T')", "P('T', None)", 2 * 24, 4 * 128, 512
    Ai, Bi = wl.random_ints((I, J), 901), wl.random_ints((J, K), 902)
    p2 = sm.sm_plan(mesh, sa, sb, I, J, K)
    q2 = planner.plan(mesh, sa, sb, I, J, K)
    a2, b2 = _both(p2, to_dev(Ai), to_dev(Bi), sm.SM_REDUCESCATTER, (I, K))
    assert torch.equal(a2, b2)
    parts = [ref.unit_partial(q2, Ai, Bi, u) for u in range(q2.n_units)]
    assert f32_bits_equal(a2.cpu().numpy(), ref.gather(q2, ref.allreduce(q2, parts)))
    # 3: smaller still, ragged K and N, one group, all-reduce
    say("case: noalloc ragged")
    mesh, sa, sb, I, J, K = {"T": 4}, "P(None, 'T')", "P('T', None)", 5, 4 * 100, 296
    Ai, Bi = wl.random_ints((I, J), 903), wl.random_ints((J, K), 904)
    p3 = sm.sm_plan(mesh, sa, sb, I, J, K)
    q3 = planner.plan(mesh, sa, sb, I, J, K)
    a3, b3 = _both(p3, to_dev(Ai), to_dev(Bi), sm.SM_ALLREDUCE, (I, K))
    assert torch.equal(a3, b3)
    parts = [ref.unit_partial(q3, Ai, Bi, u) for u in range(q3.n_units)]
    assert f32_bits_equal(a3.cpu().numpy(), ref.allreduce(q3, parts)[0])


def test_noalloc_refuses_calls_beyond_the_scratch_and_runs_taller_products():
    say("case: noalloc limits")
    # 8 partials of [64, 16400] float32 need 33.6 MB of partials: refused
    p = sm.sm_plan({"T": 8}, "P(None, 'T')", "P('T', None)", 64, 8 * 16, 16400)
    X = to_dev(wl.random_ints((64, 128), 911))
    A = to_dev(wl.random_ints((128, 16400), 912))
    out = torch.full((64, 16400), float("nan"), device=DEV)
    with pytest.raises(sm.ShardmmError) as ei:
        sm.sm_local_gemm_reduce_noalloc(p, sm.buf(X), sm.buf(A), sm.buf(out))
    assert ei.value.status == sm.SM_ERR_SHAPE and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all())
    # more than 64 rows with few tiles: the units' products on the scratch,
    # as sm_local_gemm_reduce_ws does them with its workspace
    p = sm.sm_plan({"Y": 2}, "P(None, 'Y')", "P('Y', None)", 128, 2 * 128, 256)
    X = to_dev(wl.random_normal((128, 256), 913))
    A = to_dev(wl.random_normal((256, 256), 914))
    a = torch.empty(128, 256, device=DEV)
    b = torch.empty(128, 256, device=DEV)
    ws = torch.empty(sm.sm_gemm_reduce_workspace(p) // 4, device=DEV)
    sm.sm_local_gemm_reduce_noalloc(p, sm.buf(X), sm.buf(A), sm.buf(a), sm.SM_REDUCESCATTER)
    sm.sm_local_gemm_reduce_ws(p, sm.buf(X), sm.buf(A), sm.buf(b), ws, sm.SM_REDUCESCATTER)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # partials beyond the scratch: the single launch, as sm_local_gemm_reduce
    p = sm.sm_plan({"T": 8}, "P(None, 'T')", "P('T', None)", 128, 8 * 64, 16384)  # 8 x 8 MiB of partials
    X = to_dev(wl.random_ints((128, 512), 915))
    A = to_dev(wl.random_ints((512, 16384), 916))
    a = torch.empty(128, 16384, device=DEV)
    b = torch.empty(128, 16384, device=DEV)
    sm.sm_local_gemm_reduce_noalloc(p, sm.buf(X), sm.buf(A), sm.buf(a))
    sm.sm_local_gemm_reduce(p, sm.buf(X), sm.buf(A), sm.buf(b))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_noalloc_medium_batch_on_the_scratch():
    """A 128-row batch on the skinny workload's weights (8 partials of
    [128, 8192] float32, 32 MiB: the whole scratch): bit for bit the
    workspace call, twice in a row."""
    w = wl.get("skinny")
    say("case: noalloc medium batch")
    X = to_dev(wl.make_operand(w.operand("X"), shape=(128, 28672)))
    A = to_dev(wl.make_operand(w.operand("A")))
    p = sm.sm_plan(dict(w.mesh), w.operand("X").spec, w.operand("A").spec, 128, 28672, 8192)
    for mode in (sm.SM_ALLREDUCE, sm.SM_REDUCESCATTER):
        a, b = _both(p, X, A, mode, (128, 8192))
        assert torch.equal(a, b)
