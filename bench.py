"""Benchmark of the sharded-matmul hot path on one MI355X.

One step = one pass of the whole path over the case-3 down-projection
workload (mesh {X:4, Y:2}, A[I_X, J_Y] . B[J_Y, K] with I = K = 8192,
J = 28672; the sharding sandbox default of learntpu.dev ch05):
  1. sm_plan (host),
  2. sm_local_gemm: the 8 logical ranks' local products
     [2048,14336] . [14336,8192] -> 8 fp32 partials, one launch,
  3. sm_reduce_partials(REDUCESCATTER): 4 groups x 2 partials -> row blocks
     [1024,8192] of the finished C, one launch.
Inputs are resident in HBM before the timed region. One JSON line on stdout.

The timed region is the K steps between two synchronisations (wall clock,
and HIP events on the stream the kernels run on). Each kernel's average
launch duration is then measured on its own: K launches queued back to back
between two HIP events on that stream. `--copy-calibration` runs a plain device copy of a known
size (for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters).
"""
from __future__ import annotations

import argparse
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "shard GEMM TFLOP/s (% bf16 MFMA peak) + partial-reduce GB/s (% HBM peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def setup(workload: str):
    import torch

    import local_shard_gemm_amd as sm
    import workloads as wl

    w = wl.get(workload)
    names = [o.name for o in w.operands]
    A = wl.make_operand(w.operand(names[0]))
    B = wl.make_operand(w.operand(names[1]))
    I, J = A.shape
    K = B.shape[1]
    dev = torch.device("cuda:0")
    p = sm.sm_plan(dict(w.mesh), w.operand(names[0]).spec, w.operand(names[1]).spec, I, J, K)
    Ad, Bd = A.to(dev), B.to(dev)
    m, n = p.c_local[0], p.c_local[1]
    P = torch.empty(p.n_units, m, n, dtype=torch.float32, device=dev)
    if p.kase == sm.SM_CASE3 and m % p.n_partials == 0:
        mode = sm.SM_REDUCESCATTER
        out = torch.empty(I, K, dtype=torch.float32, device=dev)
    else:
        mode = sm.SM_ALLREDUCE
        out = torch.empty(p.n_groups, m, n, dtype=torch.float32, device=dev)
    return dict(w=w, A=A, B=B, p=p, Ad=Ad, Bd=Bd, P=P, out=out, mode=mode, I=I, J=J, K=K)


def plan_time_us(ctx, reps: int = 2000) -> float:
    """Host time of one sm_plan call on the workload's mesh and specs (the
    binding's marshalling included), averaged over `reps` calls."""
    import local_shard_gemm_amd as sm

    w = ctx["w"]
    names = [o.name for o in w.operands]
    mesh, sa, sb = dict(w.mesh), w.operand(names[0]).spec, w.operand(names[1]).spec
    sm.sm_plan(mesh, sa, sb, ctx["I"], ctx["J"], ctx["K"])
    t0 = time.perf_counter()
    for _ in range(reps):
        sm.sm_plan(mesh, sa, sb, ctx["I"], ctx["J"], ctx["K"])
    return (time.perf_counter() - t0) / reps * 1e6


def cpu_baseline(ctx, rows: int):
    """The oracle (fp64 naive loops) on a bounded sample of the same step:
    the first `rows` output rows of the local products, taken unit by unit
    (unit 0's rows first), timed on the host cores."""
    import numpy as np

    from oracle import planner, reference as ref
    from oracle.build import load_library

    w = ctx["w"]
    names = [o.name for o in w.operands]
    q = planner.plan(dict(w.mesh), w.operand(names[0]).spec, w.operand(names[1]).spec, ctx["I"], ctx["J"], ctx["K"])
    m, n = q.c_local
    k = q.a_local[1]
    rows = min(rows, m * q.n_units)
    done, units = 0, 0
    t0 = time.perf_counter()
    while done < rows:
        take = min(m, rows - done)
        ref.unit_partial(q, ctx["A"], ctx["B"], units, rows=np.arange(take))
        done += take
        units += 1
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * n * k
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(load_library().orc_num_threads()),
            "kind": "oracle", "host": f"{model}, {os.cpu_count()} logical CPUs visible",
            "sample": f"{rows} output rows of the local products [{m},{k}]x[{k},{n}] of units 0..{units - 1} "
                      f"({flops / 1e9:.1f} GFLOP, fp64 naive loops, {dt:.1f} s)"}


def rate(bound: str, work: float, ms: float, cold_ms=None) -> dict:
    """Roofline entry for one launch: `work` is flops (bound "mfma") or
    bytes (bound "hbm") per launch, `ms` its average duration back to back
    on the same buffers. For an HBM-bound launch whose data would fit in
    the 256 MB Infinity Cache, `cold_ms` is the average over launches that
    rotate through copies of the buffers (no launch finds its data in the
    cache); that figure is then the HBM one (`avg_ms`, `achieved`) and the
    same-buffer rate is kept as `warm_*`."""
    if bound == "mfma":
        achieved, peak, unit = work / (ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
        return {"avg_ms": round(ms, 4), "bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "work": work}
    t = cold_ms if cold_ms else ms
    achieved = work / (t * 1e-3) / 1e9
    out = {"avg_ms": round(t, 4), "bound": bound, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
           "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4), "work": work,
           "cache": "rotating copies" if cold_ms else "footprint over 512 MiB"}
    if cold_ms:
        out.update({"warm_avg_ms": round(ms, 4), "warm_achieved": round(work / (ms * 1e-3) / 1e9, 1)})
    return out


def oracle_sample(entry: dict, fn, work: float, what: str) -> None:
    """Attach to a roofline entry the oracle's rate on a bounded sample of
    the same operation: fn() runs the oracle (fp64, the host's cores) on the
    sample and `work` is that sample's algorithmic flops or bytes, counted
    as for the GPU launch, so the two rates compare like for like."""
    runs, t0 = 0, time.perf_counter()
    while True:  # repeated until half a second has passed, for a stable rate
        fn()
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= 0.5:
            break
    v = work * runs / dt / (1e12 if entry["unit"] == "TFLOP/s" else 1e9)
    entry["oracle"] = {"value": float(f"{v:.4g}"), "unit": entry["unit"], "seconds": round(dt / runs, 4),
                       "runs": runs, "sample": what, "gpu_over_oracle": round(entry["achieved"] / v, 1)}


def measure_rows(back_to_back, cold, stream, with_oracle: bool) -> dict:
    """The other rows of the path on their own workloads, each launch timed
    back to back like the step's kernels:
      a4  Megatron MLP chain [4096,4096] . W1[4096,16384] (4 column blocks,
          GeLU(tanh) -> bf16 epilogue) . W2[16384,4096] (4 row blocks), then
          the all-reduce of the 4 fp32 partials;
      a6  case 1 on {X:4,Y:2} at 4096^3: 8 local blocks, then the gather of
          the 8 fp32 blocks into the global C;
      f1  case 2 A[I,J_X] . B[J,K] at 4096^3: all-gather A, then the case-1
          product of the gathered plan;
      f3  the sequence-parallel tail on the MLP's 4 partials: reduce-scatter,
          per-token layer norm (with gamma, beta), all-gather;
      f4  the all-to-all reshard A[I,J_X] -> A[I_X,J] of a bf16 [4096,4096];
      a7  the skinny split-J path with its fused reduce (measure_skinny).
    With `with_oracle`, every entry also carries the oracle's rate on a
    bounded sample of the same operation (oracle_sample)."""
    import numpy as np
    import torch

    import local_shard_gemm_amd as sm
    import workloads as wl

    if with_oracle:
        from oracle import planner, reference as ref
    dev = torch.device("cuda:0")
    rows = {}
    rng = np.random.default_rng(7)

    # a4 (+ f3 on the same partials)
    w = wl.get("mlp")
    Xc, W1c, W2c = (wl.make_operand(w.operand(n)) for n in ("X", "W1", "W2"))
    X, W1, W2 = Xc.to(dev), W1c.to(dev), W2c.to(dev)
    B_, D = X.shape
    F = W1.shape[1]
    p1 = sm.sm_plan(dict(w.mesh), w.operand("X").spec, w.operand("W1").spec, B_, D, F, out_dtype=sm.SM_BF16)
    p2 = sm.sm_plan(dict(w.mesh), "P(None, 'T')", w.operand("W2").spec, B_, F, D)
    H = torch.empty(B_, F, dtype=torch.bfloat16, device=dev)
    P = torch.empty(p2.n_units, B_, D, dtype=torch.float32, device=dev)
    Z = torch.empty(B_, D, dtype=torch.float32, device=dev)
    bx, bw1, bw2, bh, bp, bz = (sm.buf(t) for t in (X, W1, W2, H, P, Z))
    l1 = back_to_back(lambda: sm.sm_local_gemm(p1, bx, bw1, bh, sm.SM_EPI_GELU_TANH, 0, p1.n_units, stream),
                      clock_warm=True)
    l2 = back_to_back(lambda: sm.sm_local_gemm(p2, bh, bw2, bp, sm.SM_EPI_STORE, 0, p2.n_units, stream),
                      clock_warm=True)
    ar = back_to_back(lambda: sm.sm_reduce_partials(p2, bp, bz, sm.SM_ALLREDUCE, 0, p2.n_groups, stream))
    layer_flops = 2.0 * B_ * D * F
    red_bytes = (p2.n_partials + 1) * B_ * D * 4.0
    rows["a4_mlp_chain"] = {
        "workload": w.name,
        "layer1_gemm_gelu_bf16": rate("mfma", layer_flops, l1),
        "layer2_gemm": rate("mfma", layer_flops, l2),
        "allreduce": rate("hbm", red_bytes, ar,
                          cold(lambda i: (lambda q=(bp if i == 0 else sm.buf(P.clone())):
                                          sm.sm_reduce_partials(p2, q, bz, sm.SM_ALLREDUCE, 0, p2.n_groups, stream)),
                               red_bytes)),
        "chain_ms": round(l1 + l2 + ar, 4),
    }
    g = torch.randn(D, device=dev)
    bta = torch.randn(D, device=dev)
    sp = back_to_back(lambda: sm.sm_reduce_scatter_layernorm(p2, bp, bz, g, bta, 1e-5, 0, p2.n_groups, stream))
    sp_cold = cold(lambda i: (lambda q=(bp if i == 0 else sm.buf(P.clone())):
                              sm.sm_reduce_scatter_layernorm(p2, q, bz, g, bta, 1e-5, 0, p2.n_groups, stream)),
                   red_bytes)
    rows["f3_sp_tail"] = {"workload": w.name + ": reduce-scatter 4 x [4096,4096] -> layer norm -> all-gather",
                          **rate("hbm", red_bytes + 2 * D * 4.0, sp, sp_cold)}
    del X, W1, W2, H, P, Z, bx, bw1, bw2, bh, bp, bz
    if with_oracle:
        q1 = planner.plan(dict(w.mesh), w.operand("X").spec, w.operand("W1").spec, B_, D, F)
        q2 = planner.plan(dict(w.mesh), "P(None, 'T')", w.operand("W2").spec, B_, F, D)
        R = 256
        hr = {}
        oracle_sample(rows["a4_mlp_chain"]["layer1_gemm_gelu_bf16"],
                      lambda: hr.setdefault("H", ref.mlp_hidden(q1, Xc, W1c, rows=range(R))),
                      2.0 * R * D * F, f"{R} rows of round_bf16(gelu(X W1_u)), all 4 column blocks")
        Fk = F // q2.n_partials
        oracle_sample(rows["a4_mlp_chain"]["layer2_gemm"],
                      lambda: [ref.view_matmul(hr["H"], (0, u * Fk, R, Fk), W2c, q2.unit_views(u)["B"])
                               for u in range(q2.n_units)],
                      2.0 * R * D * F, f"{R} rows of the 4 partials H_u W2_u")
        R = 1024
        parts = [rng.standard_normal((R, D)).astype(np.float32).astype(np.float64) for _ in range(q2.n_partials)]
        gam, bet = np.asarray(g.cpu(), np.float64), np.asarray(bta.cpu(), np.float64)
        oracle_sample(rows["a4_mlp_chain"]["allreduce"], lambda: ref.sum_ranked(parts),
                      (q2.n_partials + 1) * R * D * 4.0, f"rank-ordered sum of {q2.n_partials} x [{R},{D}]")
        oracle_sample(rows["f3_sp_tail"], lambda: ref.layer_norm(ref.sum_ranked(parts), gam, bet, 1e-5),
                      (q2.n_partials + 1) * R * D * 4.0,
                      f"rank-ordered sum of {q2.n_partials} x [{R},{D}] then layer norm of each row")
        del parts, hr
    del Xc, W1c, W2c

    # a6
    w = wl.get("case1")
    Acpu, Bcpu = wl.make_operand(w.operand("A")), wl.make_operand(w.operand("B"))
    A, Bm = Acpu.to(dev), Bcpu.to(dev)
    I, J = A.shape
    K = Bm.shape[1]
    p = sm.sm_plan(dict(w.mesh), w.operand("A").spec, w.operand("B").spec, I, J, K)
    m, n = p.c_local
    Pc = torch.empty(p.n_units, m, n, dtype=torch.float32, device=dev)
    C = torch.empty(I, K, dtype=torch.float32, device=dev)
    ba, bb, bpc, bc = sm.buf(A), sm.buf(Bm), sm.buf(Pc), sm.buf(C)
    gm = back_to_back(lambda: sm.sm_local_gemm(p, ba, bb, bpc, sm.SM_EPI_STORE, 0, p.n_units, stream),
                      clock_warm=True)
    ga = back_to_back(lambda: sm.sm_gather_shards(p, sm.SM_WHAT_C_BLOCKS, bpc, bc, stream))
    ga_cold = cold(lambda i: (lambda q=(bpc if i == 0 else sm.buf(Pc.clone())):
                              sm.sm_gather_shards(p, sm.SM_WHAT_C_BLOCKS, q, bc, stream)), 2 * 4.0 * I * K)
    rows["a6_case1_gather"] = {"workload": w.name,
                               "gemm": rate("mfma", 2.0 * m * n * p.a_local[1] * p.n_units, gm),
                               "gather": rate("hbm", 2 * 4.0 * I * K, ga, ga_cold)}
    if with_oracle:
        q = planner.plan(dict(w.mesh), w.operand("A").spec, w.operand("B").spec, I, J, K)
        R = 512
        oracle_sample(rows["a6_case1_gather"]["gemm"], lambda: ref.unit_partial(q, Acpu, Bcpu, 0, rows=range(R)),
                      2.0 * R * n * q.a_local[1], f"{R} rows of unit 0's [{m},{q.a_local[1]}]x[{q.a_local[1]},{n}]")
        blks = [rng.standard_normal((m, n)) for _ in range(q.n_units)]
        oracle_sample(rows["a6_case1_gather"]["gather"], lambda: ref.gather(q, blks), 2 * 4.0 * I * K,
                      f"placing {q.n_units} blocks [{m},{n}] into [{I},{K}]")
        del blks

    # f1: case 2 at the same sizes, A held as 4 column blocks
    mesh = {"X": 4, "Y": 2}
    p = sm.sm_plan(mesh, "A[I, J_X]", "B[J, K]", I, J, K)
    gr, gc = p.a_grid
    blocks = torch.stack([A[i * (I // gr):(i + 1) * (I // gr), j * (J // gc):(j + 1) * (J // gc)]
                          for i in range(gr) for j in range(gc)]).contiguous()
    Ag = torch.empty(I, J, dtype=torch.bfloat16, device=dev)
    p_g = sm.sm_plan_gathered(p)
    Cg = torch.empty(p_g.n_units, p_g.c_local[0], p_g.c_local[1], dtype=torch.float32, device=dev)
    bbl, bag, bcg = sm.buf(blocks), sm.buf(Ag), sm.buf(Cg)
    gA = back_to_back(lambda: sm.sm_gather_shards(p, sm.SM_WHAT_A, bbl, bag, stream))
    gA_cold = cold(lambda i: (lambda q=(bbl if i == 0 else sm.buf(blocks.clone())):
                              sm.sm_gather_shards(p, sm.SM_WHAT_A, q, bag, stream)), 2 * 2.0 * I * J)
    gg = back_to_back(lambda: sm.sm_local_gemm(p_g, bag, bb, bcg, sm.SM_EPI_STORE, 0, p_g.n_units, stream),
                      clock_warm=True)
    rows["f1_case2_gather_then_gemm"] = {
        "workload": f"A[I,J_X] . B[J,K] on {{X:4,Y:2}}, I = J = K = {I}",
        "gather_A": rate("hbm", 2 * 2.0 * I * J, gA, gA_cold),
        "gemm": rate("mfma", 2.0 * p_g.c_local[0] * p_g.c_local[1] * p_g.a_local[1] * p_g.n_units, gg)}
    if with_oracle:
        qa = planner.plan(mesh, "A[I, J_X]", "B[J, K]", I, J, K)
        qg = planner.gathered(qa)
        a_blocks = ref.shard(ref.stored(Acpu)[0], mesh, "A[I, J_X]")
        oracle_sample(rows["f1_case2_gather_then_gemm"]["gather_A"],
                      lambda: ref.unshard(a_blocks, mesh, "A[I, J_X]", I, J), 2 * 2.0 * I * J,
                      f"assembling A [{I},{J}] from its {len(a_blocks)} column blocks")
        R = 512
        mg, ng = qg.c_local
        oracle_sample(rows["f1_case2_gather_then_gemm"]["gemm"],
                      lambda: ref.unit_partial(qg, Acpu, Bcpu, 0, rows=range(R)), 2.0 * R * ng * qg.a_local[1],
                      f"{R} rows of unit 0's [{mg},{qg.a_local[1]}]x[{qg.a_local[1]},{ng}]")

    # f4: all-to-all reshard of A's column blocks into row blocks
    dst = torch.empty(4, I // 4, J, dtype=torch.bfloat16, device=dev)
    mesh4 = sm.sm_mesh_init({"X": 4})
    frm, to = sm.sm_parse_spec(mesh4, "A[I, J_X]"), sm.sm_parse_spec(mesh4, "A[I_X, J]")
    blocks4 = torch.stack([A[:, j * (J // 4):(j + 1) * (J // 4)] for j in range(4)]).contiguous()
    b4, bd4 = sm.buf(blocks4), sm.buf(dst)
    rs = back_to_back(lambda: sm.sm_reshard(mesh4, frm, to, I, J, sm.SM_BF16, b4, bd4, stream))
    rs_cold = cold(lambda i: (lambda q=(b4 if i == 0 else sm.buf(blocks4.clone())):
                              sm.sm_reshard(mesh4, frm, to, I, J, sm.SM_BF16, q, bd4, stream)), 2 * 2.0 * I * J)
    rows["f4_alltoall_reshard"] = {"workload": f"bf16 [{I},{J}] A[I,J_X] -> A[I_X,J] on {{X:4}}",
                                   **rate("hbm", 2 * 2.0 * I * J, rs, rs_cold)}
    if with_oracle:
        src = ref.shard(ref.stored(Acpu)[0], {"X": 4}, "A[I, J_X]")
        oracle_sample(rows["f4_alltoall_reshard"],
                      lambda: ref.reshard(src, {"X": 4}, "A[I, J_X]", "A[I_X, J]", I, J), 2 * 2.0 * I * J,
                      f"the whole all-to-all of [{I},{J}]")
    rows["a7_skinny"] = measure_skinny(back_to_back, cold, stream, with_oracle)
    return rows


def measure_skinny(back_to_back, cold, stream, with_oracle: bool = False) -> dict:
    """Row a7 on the skinny workload (X[16,28672] . A[28672,8192], J split
    over {T:8}): the split-J kernel with the fused rank-ordered all-reduce
    of its 8 partials (sm_local_gemm_reduce_ws), and, for comparison, the
    split-J kernel alone plus sm_reduce_partials. HBM-bound: the
    algorithmic bytes are A, X and the output once (471.2 MB); the 8 fp32
    partials the kernel writes and re-reads through the workspace (8.4 MB)
    are not counted."""
    import torch

    import local_shard_gemm_amd as sm
    import workloads as wl

    dev = torch.device("cuda:0")
    w = wl.get("skinny")
    Xc, Ac = wl.make_operand(w.operand("X")), wl.make_operand(w.operand("A"))
    X, A = Xc.to(dev), Ac.to(dev)
    B_, J = X.shape
    K = A.shape[1]
    p = sm.sm_plan(dict(w.mesh), w.operand("X").spec, w.operand("A").spec, B_, J, K)
    ws = torch.zeros(sm.sm_gemm_reduce_workspace(p) // 4 + 1, dtype=torch.int32, device=dev)
    out = torch.empty(B_, K, dtype=torch.float32, device=dev)
    P = torch.empty(p.n_units, B_, K, dtype=torch.float32, device=dev)
    bx, ba, bo, bp = sm.buf(X), sm.buf(A), sm.buf(out), sm.buf(P)
    work = 2.0 * (B_ * J + J * K) + 4.0 * B_ * K
    extra = 2 * 4.0 * p.n_units * B_ * K

    def fused(q=ba):
        sm.sm_local_gemm_reduce_ws(p, bx, q, bo, ws, sm.SM_ALLREDUCE, 0, p.n_groups, stream)

    f = back_to_back(fused)
    f_cold = cold(lambda i: (lambda q=(ba if i == 0 else sm.buf(A.clone())): fused(q)), work)
    g = back_to_back(lambda: sm.sm_local_gemm(p, bx, ba, bp, sm.SM_EPI_STORE, 0, p.n_units, stream))
    r = back_to_back(lambda: sm.sm_reduce_partials(p, bp, bo, sm.SM_ALLREDUCE, 0, p.n_groups, stream))
    entry = rate("hbm", work, f, f_cold)
    entry["traffic"] = recorded_traffic("fused", w.name)
    if with_oracle:
        from oracle import planner, reference as ref

        q = planner.plan(dict(w.mesh), w.operand("X").spec, w.operand("A").spec, B_, J, K)
        oracle_sample(entry, lambda: ref.allreduce(q, ref.partials(q, Xc, Ac)), work,
                      f"the whole step: {q.n_units} partials X_u A_u and their rank-ordered sum")
    # a medium batch on the same weights: 128 rows, past the split-J kernel,
    # on the 128-row MFMA tile (8 partials [128,8192], HBM-bound on A)
    Mm = 128
    Xm_cpu = wl.make_operand(w.operand("X"), shape=(Mm, J))
    Xm = Xm_cpu.to(dev)
    pm = sm.sm_plan(dict(w.mesh), w.operand("X").spec, w.operand("A").spec, Mm, J, K)
    Pm = torch.empty(pm.n_units, Mm, K, dtype=torch.float32, device=dev)
    bxm, bpm = sm.buf(Xm), sm.buf(Pm)
    work_m = 2.0 * (Mm * J + J * K) + 4.0 * pm.n_units * Mm * K
    gmm = back_to_back(lambda q=ba: sm.sm_local_gemm(pm, bxm, q, bpm, sm.SM_EPI_STORE, 0, pm.n_units, stream),
                       clock_warm=True)
    gmm_cold = cold(lambda i: (lambda q=(ba if i == 0 else sm.buf(A.clone())):
                               sm.sm_local_gemm(pm, bxm, q, bpm, sm.SM_EPI_STORE, 0, pm.n_units, stream)), work_m)
    medium = rate("hbm", work_m, gmm, gmm_cold)
    medium["traffic"] = recorded_traffic("medium", w.name)
    if with_oracle:
        qm = planner.plan(dict(w.mesh), w.operand("X").spec, w.operand("A").spec, Mm, J, K)
        oracle_sample(medium, lambda: ref.partials(qm, Xm_cpu, Ac), work_m,
                      f"the whole launch: {qm.n_units} partials X_u A_u of [{Mm},{qm.a_local[1]}]x[{qm.a_local[1]},{K}]")
    medium["workload"] = f"X[{Mm},{J}] . A[{J},{K}] on {{T:{pm.n_partials}}}: {pm.n_units} partials [{Mm},{K}] fp32"
    # the medium batch's whole step with its sum (sm_local_gemm_reduce_ws:
    # the 8 units' products into the workspace, then their rank-ordered
    # sum); algorithmic bytes as for the skinny step: X, A and the output
    wsm = torch.empty(sm.sm_gemm_reduce_workspace(pm) // 4, dtype=torch.float32, device=dev)
    outm = torch.empty(Mm, K, dtype=torch.float32, device=dev)
    bom = sm.buf(outm)
    work_ms = 2.0 * (Mm * J + J * K) + 4.0 * Mm * K
    mstep = back_to_back(lambda: sm.sm_local_gemm_reduce_ws(pm, bxm, ba, bom, wsm, sm.SM_ALLREDUCE, 0, 1, stream),
                         clock_warm=True)
    mstep_cold = cold(lambda i: (lambda q=(ba if i == 0 else sm.buf(A.clone())):
                                 sm.sm_local_gemm_reduce_ws(pm, bxm, q, bom, wsm, sm.SM_ALLREDUCE, 0, 1, stream)),
                      work_ms)
    medium_step = rate("hbm", work_ms, mstep, mstep_cold)
    medium_step["workload"] = (f"X[{Mm},{J}] . A[{J},{K}], J split over {{T:{pm.n_partials}}}, all-reduce "
                               f"(products into the workspace, then the rank-ordered sum)")
    medium_step["partials_bytes_not_counted"] = 2 * 4.0 * pm.n_units * Mm * K
    if with_oracle:
        oracle_sample(medium_step, lambda: ref.allreduce(qm, ref.partials(qm, Xm_cpu, Ac)), work_ms,
                      f"the whole step: {qm.n_units} partials of [{Mm},{qm.a_local[1]}]x[{qm.a_local[1]},{K}] "
                      f"and their rank-ordered sum")
    return {"workload": f"{w.name}: X[{B_},{J}] . A[{J},{K}], J split over {{T:{p.n_partials}}}, all-reduce",
            "fused_gemm_reduce": {**entry, "partials_bytes_not_counted": extra},
            "split_j_gemm_then_reduce_ms": round(g + r, 4),
            "split_j_gemm_ms": round(g, 4), "reduce_ms": round(r, 4),
            "medium_batch_local_gemm": medium,
            "medium_batch_gemm_reduce": medium_step}


def source_digest(paths) -> str:
    """sha256 over the listed source files (repository-relative), in order."""
    import hashlib

    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(launch: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain-copy calibration), as recorded in a
    `traffic-record:` line of a counter summary under profiles/. Returns None
    when there is no record for this launch ("gemm", "reduce", "fused" or
    "medium") and workload, or when the kernel's sources changed after the
    counters were taken."""
    import glob

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("traffic-record:"):
                    continue
                kv = dict(tok.split("=", 1) for tok in line.split()[1:] if "=" in tok)
                if kv.get("launch") != launch or kv.get("workload") != workload:
                    continue
                try:
                    if source_digest(kv["sources"].split("+")) != kv.get("sha256"):
                        return None
                except OSError:
                    return None
                return float(kv["bytes"])
    return None


def copy_calibration(mib: int, reps: int) -> None:
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "reps": reps}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="downproj")
    ap.add_argument("--cpu-rows", type=int, default=6144, help="oracle sample size (output rows, unit by unit)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the measurements of the other rows")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every logical rank's shards are resident on a single "
              "MI355X; the library has no multi-GPU path to measure.", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return 0

    import torch

    import local_shard_gemm_amd as sm

    log(f"bench: setting up workload {args.workload}")
    ctx = setup(args.workload)
    p, P, out, mode = ctx["p"], ctx["P"], ctx["out"], ctx["mode"]
    a, b, c, o = sm.buf(ctx["Ad"]), sm.buf(ctx["Bd"]), sm.buf(P), sm.buf(out)
    stream = torch.cuda.current_stream()

    def gemm():
        sm.sm_local_gemm(p, a, b, c, sm.SM_EPI_STORE, 0, p.n_units, stream)

    def reduce():
        sm.sm_reduce_partials(p, c, o, mode, 0, p.n_groups, stream)

    def fused_call():
        sm.sm_local_gemm_reduce(p, a, b, o, mode, 0, p.n_groups, stream)

    def step():
        gemm()
        if p.kase == sm.SM_CASE3:
            reduce()

    def back_to_back(fn, reps, warm_ms=100.0, clock_warm=False):
        """Average duration of one launch: `reps` launches queued back to back
        on the kernels' stream between two HIP events.

        Kernels under 0.2 ms: a ~5 ms spin kernel goes first, so that all
        launches are queued before the GPU reaches them and host-side call
        overhead never shows between them; they are timed over 10x as many
        launches. Longer kernels, and matrix-core kernels of any length
        (clock_warm): about `warm_ms` of the same launches go first instead,
        so that the timed ones run at the clock the board settles at under
        this load (the first ~100 ms of back-to-back matrix-core launches run
        a few percent slower: a one-wave K = 4096 GEMM timed after the spin
        kernel read 8 % below its settled rate); short ones are then timed
        over at least 20 ms of launches."""
        def once(n, n_warm):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            if n_warm:
                for _ in range(n_warm):
                    fn()
            else:
                with torch.cuda.stream(stream):
                    torch.cuda._sleep(10_000_000)
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        fn()
        t = once(reps, 0)
        if t >= 0.2 or clock_warm:
            return once(max(reps, int(20.0 / t)), int(warm_ms / t) + 1)
        return once(10 * reps, 0)

    def single_launches(fn, reps):
        """(median, min) ms of `reps` launches, each between its own two HIP
        events on the kernels' stream (launches still queued back to back)."""
        evs = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        return ts[len(ts) // 2], ts[0]

    def cold(make_call, footprint: float):
        """Average launch duration without help from the 256 MB Infinity
        Cache, or None when one launch already moves 512 MiB or more (then
        the back-to-back figure is the cold one). Launches run back to back,
        cycling through R copies of the buffers with R x footprint >= 512
        MiB, so at least twice the cache's capacity of other data passes
        between two launches on one copy. make_call(i) returns the launch on
        copy i (copy 0: the original buffers)."""
        r = -(-(512 << 20) // int(footprint))
        if r <= 1:
            return None
        r = min(r, 64)
        calls = [make_call(i) for i in range(r)]
        it = itertools.cycle(calls)
        return back_to_back(lambda: next(it)(), r * max(1, -(-args.steps // r)))

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s0.record(stream)
    for _ in range(args.steps):
        step()
    s1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    ms_step_events = s0.elapsed_time(s1) / args.steps

    # Per-kernel launch durations, each kernel on its own.
    gemm_avg = back_to_back(gemm, args.steps)
    red_avg = back_to_back(reduce, args.steps) if p.kase == sm.SM_CASE3 else 0.0
    gemm_single = single_launches(gemm, args.steps)
    red_single = single_launches(reduce, args.steps) if p.kase == sm.SM_CASE3 else None
    plan_us = plan_time_us(ctx)

    m, n = p.c_local[0], p.c_local[1]
    kl = p.a_local[1]
    gemm_flops = 2.0 * m * n * kl * p.n_units
    N = p.n_partials
    # reduce: each group reads N fp32 partials and writes one fp32 block
    red_bytes = (N + 1) * m * n * 4.0 * p.n_groups if p.kase == sm.SM_CASE3 else 0.0
    gemm_tflops = gemm_flops / (gemm_avg * 1e-3) / 1e12
    red_gbps_warm = red_bytes / (red_avg * 1e-3) / 1e9 if red_bytes else 0.0
    # algorithmic HBM bytes of the local products: each distinct operand
    # block read once, each output written once
    # Without help from the Infinity Cache: on copies of the partials when one
    # launch moves less than 512 MiB (the down-projection's 805 MB does not).
    red_cold = None
    if p.kase == sm.SM_CASE3:
        red_cold = cold(lambda i: (lambda q=(c if i == 0 else sm.buf(P.clone())):
                                   sm.sm_reduce_partials(p, q, o, mode, 0, p.n_groups, stream)), red_bytes)
    red_t = red_cold if red_cold else red_avg
    red_gbps = red_bytes / (red_t * 1e-3) / 1e9 if red_bytes else 0.0
    a_bytes = 2.0 * ctx["I"] * ctx["J"]
    b_bytes = 2.0 * ctx["J"] * ctx["K"]
    gemm_bytes = a_bytes + b_bytes + 4.0 * m * n * p.n_units
    gemm_gbps = gemm_bytes / (gemm_avg * 1e-3) / 1e9
    skinny = m <= 16
    gemm_cold = None
    if skinny:  # the skinny product is HBM-bound
        gemm_cold = cold(lambda i: (lambda q=(b if i == 0 else sm.buf(ctx["Bd"].clone())):
                                    sm.sm_local_gemm(p, a, q, c, sm.SM_EPI_STORE, 0, p.n_units, stream)), gemm_bytes)

    # The fused kernel (local products and rank-ordered reduction in one
    # launch, no partial buffers) on the same inputs, timed the same way.
    fused = None
    if p.kase == sm.SM_CASE3 and m > 16:
        f_avg = back_to_back(fused_call, args.steps)
        fused = {"avg_ms": round(f_avg, 4),
                 "tflops": round(gemm_flops / (f_avg * 1e-3) / 1e12, 1),
                 "vs_gemm_plus_reduce": round((gemm_avg + red_avg) / f_avg, 3),
                 "traffic": recorded_traffic("fused", ctx["w"].name)}

    # Smaller launches of the same products: one logical rank's shard, and
    # one reduce group (for case 3: the N ranks whose partials are summed
    # together, the configuration as one group sees it), GEMM and reduce.
    subsets = None
    if p.n_units > 1 and not skinny:
        def sub_gemm(cnt):
            return lambda: sm.sm_local_gemm(p, a, b, c, sm.SM_EPI_STORE, 0, cnt, stream)
        per_unit = 2.0 * m * n * kl
        subsets = {"gemm_1_shard": rate("mfma", per_unit, back_to_back(sub_gemm(1), args.steps))}
        if p.kase == sm.SM_CASE3:
            subsets["gemm_1_group"] = rate("mfma", per_unit * N, back_to_back(sub_gemm(N), args.steps))
            red1 = lambda: sm.sm_reduce_partials(p, c, o, mode, 0, 1, stream)  # noqa: E731
            red1_cold = cold(lambda i: (lambda q=(c if i == 0 else sm.buf(P[:N].clone())):
                                        sm.sm_reduce_partials(p, q, o, mode, 0, 1, stream)), (N + 1) * m * n * 4.0)
            subsets["reduce_1_group"] = rate("hbm", (N + 1) * m * n * 4.0, back_to_back(red1, args.steps), red1_cold)

    rows = None
    if not args.no_rows:
        log("bench: the other rows of the path")
        rows = measure_rows(lambda fn, **kw: back_to_back(fn, args.steps, **kw), cold, stream,
                            not args.no_cpu_baseline)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"bench: oracle CPU baseline on {args.cpu_rows} rows")
        cpu = cpu_baseline(ctx, args.cpu_rows)
        cpu["gpu_gemm_over_oracle"] = round(gemm_tflops / cpu["value"], 1)

    # HBM bytes per launch from rocprofv3 counters (null when not recorded for
    # the kernel as it is now)
    gemm_traffic = recorded_traffic("gemm", ctx["w"].name)
    line = {
        "metric": METRIC,
        "value": round(gemm_flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ctx["w"].name,
            "mesh": "{X:4,Y:2}" if args.workload == "downproj" else str(dict(ctx["w"].mesh)),
            "global": f"A[{ctx['I']},{ctx['J']}] . B[{ctx['J']},{ctx['K']}]",
            "units": int(p.n_units),
            "local_gemm": f"[{m},{kl}]x[{kl},{n}] bf16 -> fp32",
            "reduce": ("reduce-scatter" if mode == sm.SM_REDUCESCATTER else "all-reduce")
                      + f" {p.n_groups} groups x {N} fp32 partials [{m},{n}]",
        },
        "ms_per_step_events": round(ms_step_events, 4),
        "sm_plan_us": round(plan_us, 2),
        "gemm": {"avg_ms": round(gemm_avg, 4),
                 "single_launch_median_ms": round(gemm_single[0], 4), "single_launch_min_ms": round(gemm_single[1], 4),
                 **({"cold_avg_ms": round(gemm_cold, 4),
                     "cold_gbps": round(gemm_bytes / (gemm_cold * 1e-3) / 1e9, 1)} if gemm_cold else {}),
                 "tflops": round(gemm_tflops, 1), "frac_of_peak": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                 "bytes": gemm_bytes, "gbps": round(gemm_gbps, 1)},
        "reduce": {"avg_ms": round(red_avg, 4), "bytes": red_bytes,
                   **({"single_launch_median_ms": round(red_single[0], 4),
                       "single_launch_min_ms": round(red_single[1], 4)} if red_single else {}),
                   "cold_avg_ms": round(red_cold, 4) if red_cold else None,
                   "gbps": round(red_gbps, 1), "frac_of_peak": round(red_gbps / PEAK_HBM_GBPS, 4),
                   "warm_gbps": round(red_gbps_warm, 1)},
        "roofline": ({"bound": "hbm", "achieved": round(gemm_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                      "frac": round(gemm_gbps / PEAK_HBM_GBPS, 4), "traffic": gemm_traffic} if skinny else
                     {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                      "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4), "traffic": gemm_traffic}),
        "roofline_reduce": {"bound": "hbm", "achieved": round(red_gbps, 1), "peak": PEAK_HBM_GBPS,
                            "unit": "GB/s", "frac": round(red_gbps / PEAK_HBM_GBPS, 4),
                            "traffic": recorded_traffic("reduce", ctx["w"].name)},
        # the launch the case-3 shard GEMM bar is graded on: one X-group, the
        # N ranks whose partials are summed together (learntpu.dev ch05,
        # sharding sandbox "Local matmul", here for both ranks of the group)
        "roofline_x_group": ({k: subsets["gemm_1_group"][k] for k in
                              ("bound", "achieved", "peak", "unit", "frac", "avg_ms", "work")}
                             if subsets and "gemm_1_group" in subsets else None),
        "fused_gemm_reduce": fused,
        "subsets": subsets,
        "rows": rows,
        "cpu_baseline": cpu,
        "context": "learntpu.dev sandbox, modelled (not measured) on Ironwood: 481 GFLOP local matmul "
                   "in 209 us per rank",
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
