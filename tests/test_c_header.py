"""The C ABI from plain C (CPU only): a C99 program that includes
include/shardmm.h, compiled with gcc -std=c99 -pedantic -Werror and linked
against the in-tree libshardmm.so, plans the down-projection
(A[I_X, J_Y] . B[J_Y, K] on {X:4, Y:2}, the learntpu.dev ch05 sharding
sandbox's default) and a case-4 re-plan, and prints what it got; the
values must equal the Python binding's. This checks that the header is
valid C on its own (no HIP or C++ header needed) and that its struct
layouts agree with the library's. No device call is made."""
import os
import subprocess

import pytest

import local_shard_gemm_amd as sm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "shardmm.h"

static int check(int32_t st, const char* what) {
  if (st != SM_OK) {
    printf("FAIL %s %s %s\n", what, sm_status_str(st), sm_last_error());
    return 1;
  }
  return 0;
}

int main(void) {
  const char* names[2] = {"X", "Y"};
  const int32_t sizes[2] = {4, 2};
  sm_mesh mesh;
  sm_spec a, b;
  sm_plan_t plan, fixed;
  sm_rank_info_t info;
  memset(&plan, 0, sizeof plan);
  printf("abi %d plan_size %d sizeof %d\n", (int)sm_abi_version(), (int)sm_plan_size(), (int)sizeof(sm_plan_t));
  if (check(sm_mesh_init(&mesh, 2, names, sizes), "mesh")) return 1;
  if (check(sm_parse_spec(&mesh, "A[I_X, J_Y]", &a), "spec a")) return 1;
  if (check(sm_parse_spec(&mesh, "P('Y', None)", &b), "spec b")) return 1;
  if (check(sm_plan(&mesh, &a, &b, 8192, 28672, 8192, SM_BF16, SM_F32, &plan), "plan")) return 1;
  printf("case %d ranks %d units %d groups %d partials %d\n", (int)plan.kase, (int)plan.n_ranks,
         (int)plan.n_units, (int)plan.n_groups, (int)plan.n_partials);
  printf("a_local %lld %lld c_local %lld %lld\n", (long long)plan.a_local[0], (long long)plan.a_local[1],
         (long long)plan.c_local[0], (long long)plan.c_local[1]);
  if (check(sm_rank_info(&plan, 3, &info), "rank info")) return 1;
  printf("rank3 unit %d group %d partial %d a %lld %lld rs %lld %lld\n", (int)info.unit, (int)info.group,
         (int)info.partial, (long long)info.a_row0, (long long)info.a_col0, (long long)info.rs_row0,
         (long long)info.rs_rows);
  {
    int64_t ws = -1;
    if (check(sm_gemm_reduce_workspace(&plan, 1, &ws), "workspace")) return 1;
    printf("workspace %lld\n", (long long)ws);
  }
  /* case 4, then the plan once the smaller operand is gathered */
  if (check(sm_parse_spec(&mesh, "A[I_X, J]", &a), "spec a4")) return 1;
  if (check(sm_parse_spec(&mesh, "B[J, K_X]", &b), "spec b4")) return 1;
  if (check(sm_plan(&mesh, &a, &b, 512, 256, 1024, SM_BF16, SM_F32, &plan), "plan4")) return 1;
  if (check(sm_plan_gathered(&plan, &fixed), "gathered")) return 1;
  printf("case4 %d gather %d -> case %d units %d\n", (int)plan.kase, (int)plan.gather_operand, (int)fixed.kase,
         (int)fixed.n_units);
  /* an error path: one axis on two dimensions of A (parsed, then refused
     by the planner) */
  {
    int32_t st = sm_parse_spec(&mesh, "P('X', 'X')", &a);
    if (st == SM_OK) st = sm_plan(&mesh, &a, &b, 512, 256, 1024, SM_BF16, SM_F32, &plan);
    printf("reuse %s\n", sm_status_str(st));
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def c_program(tmp_path_factory):
    lib = sm.load()
    libdir = os.path.dirname(sm.loaded_library_path())
    out = tmp_path_factory.mktemp("cabi")
    src, exe = out / "abi.c", out / "abi"
    src.write_text(PROGRAM)
    r = subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I" + os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), "-L" + libdir, "-lshardmm", "-Wl,-rpath," + libdir],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    assert lib is not None
    return str(exe)


def test_header_is_plain_c_and_layouts_agree(c_program):
    r = subprocess.run([c_program], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    got = dict((line.split(" ", 1)[0], line.split(" ", 1)[1]) for line in r.stdout.strip().splitlines())
    p = sm.sm_plan({"X": 4, "Y": 2}, "A[I_X, J_Y]", "P('Y', None)", 8192, 28672, 8192)
    assert got["abi"] == f"{sm.SM_ABI_VERSION} plan_size {sm.ctypes.sizeof(sm.sm_plan_t)} sizeof " \
                         f"{sm.ctypes.sizeof(sm.sm_plan_t)}"
    assert got["case"] == f"{p.kase} ranks {p.n_ranks} units {p.n_units} groups {p.n_groups} partials {p.n_partials}"
    assert got["a_local"] == f"{p.a_local[0]} {p.a_local[1]} c_local {p.c_local[0]} {p.c_local[1]}"
    ri = sm.sm_rank_info(p, 3)
    assert got["rank3"] == (f"unit {ri.unit} group {ri.group} partial {ri.partial} a {ri.a_row0} {ri.a_col0} "
                            f"rs {ri.rs_row0} {ri.rs_rows}")
    assert got["workspace"] == str(sm.sm_gemm_reduce_workspace(p, 1))
    p4 = sm.sm_plan({"X": 4, "Y": 2}, "A[I_X, J]", "B[J, K_X]", 512, 256, 1024)
    f4 = sm.sm_plan_gathered(p4)
    assert got["case4"] == f"{p4.kase} gather {p4.gather_operand} -> case {f4.kase} units {f4.n_units}"
    assert got["reuse"] == "SM_ERR_AXIS_REUSED"
