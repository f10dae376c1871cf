// Entry points built from the core kernels: the sequence-parallel tail
// (reduce-scatter + layer norm of the owned rows) and resharding between
// two partition specs (all-to-all, all-gather). Host-side validation first,
// as for the core calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"
#include "kernels.h"

using namespace shardmm;

extern "C" int32_t sm_reduce_scatter_layernorm(const sm_plan_t* plan, const sm_buf* partials, const sm_buf* out,
                                               const float* gamma, const float* beta, float eps, int32_t group_begin,
                                               int32_t group_count, void* stream) {
  clear_error();
  int32_t st = check_plan(plan);
  if (st) return st;
  const sm_plan_t& p = *plan;
  if (p.kase != SM_CASE3) return fail(SM_ERR_CASE, "only case-3 plans have partial sums to reduce");
  if (p.c_grid[1] != 1) return fail(SM_ERR_CASE, "layer norm needs whole rows: the output's K is sharded");
  if (p.out_dtype != SM_F32) return fail(SM_ERR_DTYPE, "partials are float32");
  if (!(eps >= 0.0f)) return fail(SM_ERR_ARG, "eps must be >= 0");
  if (group_count < 1 || group_begin < 0 || group_begin > p.n_groups - group_count)
    return fail(SM_ERR_ARG, "group range outside [0, n_groups)");
  if ((st = check_buf_basic(partials, "partials", SM_F32))) return st;
  if ((st = check_buf_basic(out, "out", SM_F32))) return st;
  if (partials->block_stride == 0)
    return fail(SM_ERR_UNREDUCED, "partials overlap in output coordinates; they must be stacked");
  const int64_t m = p.c_local[0], n = p.c_local[1];
  const int32_t N = p.n_partials;
  if (n > kLayerNormMaxCols) return fail(SM_ERR_SHAPE, "rows longer than 32768 elements");
  if (n % 4) return fail(SM_ERR_SHAPE, "row length must be a multiple of 4");
  if (m % N) return fail(SM_ERR_INDIVISIBLE, "rows of a block do not split N ways");
  if (reinterpret_cast<uintptr_t>(gamma) % 16 || reinterpret_cast<uintptr_t>(beta) % 16)
    return fail(SM_ERR_ALIGN, "gamma / beta not 16-byte aligned");
  if ((st = check_stacked(partials, m, n, "partials"))) return st;
  {
    BlockRef last{static_cast<i128>(group_count) * N * partials->block_stride - partials->block_stride, m, n};
    if ((st = check_extent(partials, last, "partials"))) return st;
  }
  const int64_t orows = m / N;
  if (out->block_stride == 0) {
    if (out->ld < p.K) return fail(SM_ERR_SHAPE, "out: global layout needs ld >= K");
  } else if ((st = check_stacked(out, orows, n, "out"))) {
    return st;
  }
  std::vector<RowJob> jobs;
  const float* P = static_cast<const float*>(partials->ptr);
  float* O = static_cast<float*>(out->ptr);
  for (int32_t g = group_begin; g < group_begin + group_count; ++g) {
    const int64_t bi = g / p.c_grid[1];
    const int64_t src0 = static_cast<int64_t>(g - group_begin) * N * partials->block_stride;
    for (int32_t y = 0; y < N; ++y) {
      BlockRef d{out->block_stride == 0 ? (static_cast<i128>(bi) * m + y * orows) * out->ld
                                        : (static_cast<i128>(g - group_begin) * N + y) * out->block_stride,
                 orows, n};
      if ((st = check_extent(out, d, "out"))) return st;
      RowJob J;
      std::memset(&J, 0, sizeof J);
      J.src = P + src0 + y * orows * partials->ld;
      J.dst = O + d.off();
      J.src_stride = partials->block_stride;
      J.lds = partials->ld;
      J.ldd = out->ld;
      J.rows = static_cast<int32_t>(orows);
      J.cols = static_cast<int32_t>(n);
      J.vec = 1;
      if (reinterpret_cast<uintptr_t>(J.src) % 16 || reinterpret_cast<uintptr_t>(J.dst) % 16)
        return fail(SM_ERR_ALIGN, "rows must start 16-byte aligned");
      jobs.push_back(J);
    }
  }
  if ((st = check_device_memory(partials->ptr, "partials")) || (st = check_device_memory(out->ptr, "out")) ||
      (gamma && (st = check_device_memory(gamma, "gamma"))) || (beta && (st = check_device_memory(beta, "beta"))))
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RowLaunch L;
  for (size_t first = 0; first < jobs.size(); first += kMaxJobsPerLaunch) {
    std::memset(&L, 0, sizeof L);
    const size_t cnt = std::min(jobs.size() - first, static_cast<size_t>(kMaxJobsPerLaunch));
    L.n_jobs = static_cast<int32_t>(cnt);
    L.n_sum = N;
    L.elem_bytes = 4;
    for (size_t i = 0; i < cnt; ++i) {
      L.jobs[i] = jobs[first + i];
      L.max_rows = std::max(L.max_rows, L.jobs[i].rows);
    }
    L.chunk = static_cast<int32_t>(n);
    L.n_chunks = 1;
    hipError_t e = launch_rows_layernorm(L, gamma, beta, eps, s);
    if (e != hipSuccess) return hip_fail(e, "sm_reduce_scatter_layernorm launch");
  }
  return SM_OK;
}

namespace {

struct Grid {
  int64_t gr, gc, br, bc;  // blocks per dim and block extents
};

int32_t spec_grid(const sm_mesh& mesh, const sm_spec& s, int64_t rows, int64_t cols, const char* what, Grid* g) {
  g->gr = axes_product(mesh, s.axes[0], s.n[0]);
  g->gc = axes_product(mesh, s.axes[1], s.n[1]);
  if (rows % g->gr || cols % g->gc) return fail(SM_ERR_INDIVISIBLE, std::string(what) + ": shape does not split evenly");
  g->br = rows / g->gr;
  g->bc = cols / g->gc;
  return SM_OK;
}

}  // namespace

extern "C" int32_t sm_reshard(const sm_mesh* mesh, const sm_spec* from, const sm_spec* to, int64_t rows, int64_t cols,
                              int32_t dtype, const sm_buf* src, const sm_buf* dst, void* stream) {
  clear_error();
  if (!mesh || !from || !to) return fail(SM_ERR_ARG, "NULL argument");
  if (mesh->n_axes < 1 || mesh->n_axes > SM_MAX_AXES) return fail(SM_ERR_MESH, "1 to 4 axes");
  for (int32_t a = 0; a < mesh->n_axes; ++a)
    if (mesh->sizes[a] < 1) return fail(SM_ERR_MESH, "axis sizes must be >= 1");
  int32_t st;
  if ((st = validate_spec(*mesh, *from, "from"))) return st;
  if ((st = validate_spec(*mesh, *to, "to"))) return st;
  if (rows < 1 || cols < 1 || rows > INT32_MAX || cols > INT32_MAX) return fail(SM_ERR_SHAPE, "bad shape");
  if (dtype != SM_BF16 && dtype != SM_F32) return fail(SM_ERR_DTYPE, "bfloat16 or float32");
  if ((st = check_buf_basic(src, "src", dtype))) return st;
  if ((st = check_buf_basic(dst, "dst", dtype))) return st;
  if (src->block_stride == 0 && dst->block_stride == 0) return fail(SM_ERR_ARG, "both layouts are global");
  Grid gs, gd;
  if ((st = spec_grid(*mesh, *from, rows, cols, "from", &gs))) return st;
  if ((st = spec_grid(*mesh, *to, rows, cols, "to", &gd))) return st;
  if (src->block_stride > 0 && (st = check_stacked(src, gs.br, gs.bc, "src"))) return st;
  if (dst->block_stride > 0 && (st = check_stacked(dst, gd.br, gd.bc, "dst"))) return st;
  if (src->block_stride == 0 && src->ld < cols) return fail(SM_ERR_SHAPE, "src: global layout needs ld >= cols");
  if (dst->block_stride == 0 && dst->ld < cols) return fail(SM_ERR_SHAPE, "dst: global layout needs ld >= cols");

  const int64_t esz = static_cast<int64_t>(dtype_size(dtype));
  // Offset (elements) of global element (r, c) inside a buffer laid out by grid g.
  auto where = [](const sm_buf* b, const Grid& g, int64_t r, int64_t c) -> i128 {
    if (b->block_stride == 0) return static_cast<i128>(r) * b->ld + c;
    const int64_t bi = r / g.br, bj = c / g.bc;
    return (static_cast<i128>(bi) * g.gc + bj) * b->block_stride + static_cast<i128>(r - bi * g.br) * b->ld +
           (c - bj * g.bc);
  };
  std::vector<RowJob> jobs;
  for (int64_t di = 0; di < gd.gr; ++di)
    for (int64_t dj = 0; dj < gd.gc; ++dj) {
      const int64_t r0 = di * gd.br, r1 = r0 + gd.br, c0 = dj * gd.bc, c1 = c0 + gd.bc;
      // every source block overlapping this target block
      for (int64_t si = r0 / gs.br; si * gs.br < r1; ++si)
        for (int64_t sj = c0 / gs.bc; sj * gs.bc < c1; ++sj) {
          const int64_t ir0 = std::max(r0, si * gs.br), ir1 = std::min(r1, (si + 1) * gs.br);
          const int64_t ic0 = std::max(c0, sj * gs.bc), ic1 = std::min(c1, (sj + 1) * gs.bc);
          BlockRef s{where(src, gs, ir0, ic0), ir1 - ir0, ic1 - ic0};
          BlockRef d{where(dst, gd, ir0, ic0), ir1 - ir0, ic1 - ic0};
          if ((st = check_extent(src, s, "src"))) return st;
          if ((st = check_extent(dst, d, "dst"))) return st;
          RowJob J;
          std::memset(&J, 0, sizeof J);
          J.src = static_cast<const char*>(src->ptr) + s.off() * esz;
          J.dst = static_cast<char*>(dst->ptr) + d.off() * esz;
          J.src_stride = 0;
          J.lds = src->ld;
          J.ldd = dst->ld;
          J.rows = static_cast<int32_t>(s.rows);
          J.cols = static_cast<int32_t>(s.cols);
          jobs.push_back(J);
        }
    }
  // Copy in source order: workgroups that run together then stream one
  // source region instead of reading from several blocks at once (measured
  // on the all-to-all A[I,J_X] -> A[I_X,J] of a bf16 [4096,4096]: 5.1 ->
  // 5.6 TB/s).
  std::stable_sort(jobs.begin(), jobs.end(),
                   [](const RowJob& a, const RowJob& b) { return a.src < b.src; });
  if ((st = check_device_memory(src->ptr, "src")) || (st = check_device_memory(dst->ptr, "dst"))) return st;
  return run_jobs(jobs, 1, static_cast<int32_t>(esz), static_cast<hipStream_t>(stream), "sm_reshard launch");
}
