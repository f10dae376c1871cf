// Device entry points of libshardmm: sm_local_gemm, sm_reduce_partials,
// sm_gather_shards. Every argument is validated on the host before the
// first HIP call, so a failed check leaves all outputs untouched and makes
// no device call at all.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"
#include "kernels.h"


namespace shardmm {

static const char* dtype_name(int32_t d) { return d == SM_BF16 ? "bfloat16" : d == SM_F32 ? "float32" : "unknown"; }

int32_t check_buf_basic(const sm_buf* b, const char* what, int32_t dtype) {
  if (!b) return fail(SM_ERR_ARG, std::string(what) + ": NULL sm_buf");
  if (!b->ptr) return fail(SM_ERR_ARG, std::string(what) + ": NULL pointer");
  if (b->dtype != dtype)
    return fail(SM_ERR_DTYPE, std::string(what) + ": buffer holds " + dtype_name(b->dtype) + " elements, the call " +
                                  "accesses it as " + dtype_name(dtype));
  if (reinterpret_cast<uintptr_t>(b->ptr) % 16)
    return fail(SM_ERR_ALIGN, std::string(what) + ": pointer not 16-byte aligned");
  const int64_t q = dtype == SM_BF16 ? 8 : 4;
  if (b->ld < 1) return fail(SM_ERR_SHAPE, std::string(what) + ": ld < 1");
  if (b->ld % q) return fail(SM_ERR_ALIGN, std::string(what) + ": ld not a multiple of " + std::to_string(q));
  if (b->block_stride < 0) return fail(SM_ERR_ARG, std::string(what) + ": negative block_stride");
  if (b->block_stride % q)
    return fail(SM_ERR_ALIGN, std::string(what) + ": block_stride not a multiple of " + std::to_string(q));
  if (b->elems < 1) return fail(SM_ERR_SHAPE, std::string(what) + ": elems < 1");
  return SM_OK;
}

// A block at `offset` spanning rows x cols must lie inside the buffer. The
// end is computed in 128 bits, so no caller-supplied size can wrap it.
int32_t check_extent(const sm_buf* b, const BlockRef& r, const char* what) {
  if (r.cols > b->ld) return fail(SM_ERR_SHAPE, std::string(what) + ": ld smaller than the block width");
  const __int128 last = static_cast<__int128>(r.offset) + static_cast<__int128>(r.rows - 1) * b->ld + r.cols;
  if (r.offset < 0 || r.rows < 1 || last > b->elems)
    return fail(SM_ERR_SHAPE, std::string(what) + ": block extends past the buffer (" + std::to_string(b->elems) +
                                  " elements)");
  return SM_OK;
}

// Stacked layout: blocks must not overlap (required of outputs, harmless
// for inputs but kept uniform).
int32_t check_stacked(const sm_buf* b, int64_t rows, int64_t cols, const char* what) {
  if (cols > b->ld) return fail(SM_ERR_SHAPE, std::string(what) + ": ld smaller than the block width");
  if (static_cast<__int128>(b->block_stride) < static_cast<__int128>(rows) * b->ld)
    return fail(SM_ERR_SHAPE, std::string(what) + ": block_stride smaller than rows * ld");
  return SM_OK;
}

int32_t hip_fail(hipError_t e, const char* where) {
  return fail(SM_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

// Memory a kernel will touch must be addressable by the GPU: device,
// managed, or HIP-allocated / registered host memory. A plain host pointer
// would fault the kernel, so it is refused here, after every other check
// and before any launch.
// The MFMA kernel reads B in 16-byte chunks; on a tile past column N the
// chunk that holds column N-1 also covers up to 7 columns after it. Those
// lie inside the row's leading dimension (ld is a multiple of 8), but on the
// view's last row they must also lie inside the buffer, else the launch
// takes the element-wise edge kernel (vec_ok = 0).
bool b_rows_padded(const sm_buf* B, const BlockRef& rb) {
  const i128 end = static_cast<i128>(rb.offset) + static_cast<i128>(rb.rows - 1) * B->ld + (rb.cols + 7) / 8 * 8;
  return end <= B->elems;
}

int32_t check_device_memory(const void* ptr, const char* what) {
  hipPointerAttribute_t attr;
  const hipError_t e = hipPointerGetAttributes(&attr, ptr);
  if (e == hipErrorInvalidValue) {
    (void)hipGetLastError();  // not sticky; keep it out of the launch checks
    return fail(SM_ERR_ARG, std::string(what) + ": not memory the GPU can address");
  }
  if (e != hipSuccess) return hip_fail(e, what);
  if (attr.type == hipMemoryTypeUnregistered || attr.devicePointer == nullptr)
    return fail(SM_ERR_ARG, std::string(what) + ": not memory the GPU can address");
  return SM_OK;
}

}  // namespace shardmm

using namespace shardmm;

extern "C" int32_t sm_local_gemm(const sm_plan_t* plan, const sm_buf* A, const sm_buf* B, const sm_buf* C,
                                 int32_t epilogue, int32_t unit_begin, int32_t unit_count, void* stream) {
  clear_error();
  int32_t st = check_plan(plan);
  if (st) return st;
  const sm_plan_t& p = *plan;
  if (p.kase == SM_CASE2 || p.kase == SM_CASE4)
    return fail(SM_ERR_NEEDS_GATHER, std::string("case ") + std::to_string(p.kase) + ": all-gather operand " +
                                         (p.gather_operand == 0 ? "A" : "B") + " first");
  if (p.kase != SM_CASE1 && p.kase != SM_CASE3) return fail(SM_ERR_ARG, "corrupt plan");
  if (epilogue != SM_EPI_STORE && epilogue != SM_EPI_GELU_TANH) return fail(SM_ERR_ARG, "unknown epilogue");
  if (epilogue == SM_EPI_GELU_TANH && p.kase == SM_CASE3)
    return fail(SM_ERR_CASE, "GeLU of an unreduced partial is not GeLU of the sum");
  if (p.in_dtype != SM_BF16) return fail(SM_ERR_DTYPE, "inputs must be bfloat16");
  if (unit_count < 1 || unit_begin < 0 || unit_begin > p.n_units - unit_count)
    return fail(SM_ERR_ARG, "unit range outside [0, n_units)");
  if ((st = check_buf_basic(A, "A", SM_BF16))) return st;
  if ((st = check_buf_basic(B, "B", SM_BF16))) return st;
  if ((st = check_buf_basic(C, "C", p.out_dtype))) return st;
  if (p.kase == SM_CASE3 && C->block_stride == 0)
    return fail(SM_ERR_UNREDUCED, "case-3 partials overlap in output coordinates; C must be stacked");

  const int64_t m = p.a_local[0], k = p.a_local[1], n = p.b_local[1];
  if (m > INT32_MAX / 2 || n > INT32_MAX / 2 || k > INT32_MAX / 2) return fail(SM_ERR_SHAPE, "local shape too large");
  if (((m + kTileM - 1) / kTileM) * ((n + kTileN - 1) / kTileN) * kMaxUnitsPerLaunch > INT32_MAX)
    return fail(SM_ERR_SHAPE, "too many output tiles for one launch grid");
  if (A->block_stride == 0 && A->ld < p.J) return fail(SM_ERR_SHAPE, "A: global layout needs ld >= J");
  if (B->block_stride == 0 && B->ld < p.K) return fail(SM_ERR_SHAPE, "B: global layout needs ld >= K");
  if (C->block_stride == 0 && C->ld < p.K) return fail(SM_ERR_SHAPE, "C: global layout needs ld >= K");
  if (A->block_stride > 0 && (st = check_stacked(A, m, k, "A"))) return st;
  if (B->block_stride > 0 && (st = check_stacked(B, k, n, "B"))) return st;
  if (C->block_stride > 0 && (st = check_stacked(C, m, n, "C"))) return st;

  struct Item {
    int32_t unit, b_id, a_row;
    GemmUnitPtrs ptrs;
  };
  std::vector<Item> items;
  items.reserve(unit_count);
  bool b_padded = true;
  const size_t csz = dtype_size(p.out_dtype);
  for (int32_t u = unit_begin; u < unit_begin + unit_count; ++u) {
    UnitView v;
    if ((st = unit_view(p, u, &v))) return st;
    BlockRef ra, rb, rc;
    ra.rows = m;
    ra.cols = k;
    rb.rows = k;
    rb.cols = n;
    rc.rows = m;
    rc.cols = n;
    const int32_t a_id = v.a_block[0] * p.a_grid[1] + v.a_block[1];
    const int32_t b_id = v.b_block[0] * p.b_grid[1] + v.b_block[1];
    ra.offset = A->block_stride ? static_cast<i128>(a_id) * A->block_stride : static_cast<i128>(v.a_row0) * A->ld + v.a_col0;
    rb.offset = B->block_stride ? static_cast<i128>(b_id) * B->block_stride : static_cast<i128>(v.b_row0) * B->ld + v.b_col0;
    rc.offset = C->block_stride ? static_cast<i128>(u - unit_begin) * C->block_stride
                                : static_cast<i128>(v.c_row0) * C->ld + v.c_col0;
    if ((st = check_extent(A, ra, "A"))) return st;
    if ((st = check_extent(B, rb, "B"))) return st;
    if ((st = check_extent(C, rc, "C"))) return st;
    Item it;
    it.unit = u;
    it.b_id = b_id;
    it.a_row = v.a_block[0];
    it.ptrs.a = static_cast<const uint16_t*>(A->ptr) + ra.off();
    it.ptrs.b = static_cast<const uint16_t*>(B->ptr) + rb.off();
    it.ptrs.c = static_cast<char*>(C->ptr) + rc.off() * static_cast<int64_t>(csz);
    if (!b_rows_padded(B, rb)) b_padded = false;
    items.push_back(it);
  }
  if ((st = check_device_memory(A->ptr, "A")) || (st = check_device_memory(B->ptr, "B")) ||
      (st = check_device_memory(C->ptr, "C")))
    return st;
  // Units sharing a B block go next to each other (their tiles stack into
  // one tall matrix in the kernel's tile order).
  std::stable_sort(items.begin(), items.end(), [](const Item& x, const Item& y) {
    return x.b_id != y.b_id ? x.b_id < y.b_id : x.a_row < y.a_row;
  });

  GemmLaunch L;
  std::memset(&L, 0, sizeof L);
  L.M = static_cast<int32_t>(m);
  L.N = static_cast<int32_t>(n);
  L.K = static_cast<int32_t>(k);
  L.tiles_m = static_cast<int32_t>((m + kTileM - 1) / kTileM);
  L.tiles_n = static_cast<int32_t>((n + kTileN - 1) / kTileN);
  L.lda = A->ld;
  L.ldb = B->ld;
  L.ldc = C->ld;
  L.epilogue = epilogue == SM_EPI_GELU_TANH ? kEpiGelu : kEpiStore;
  L.out_bf16 = p.out_dtype == SM_BF16 ? 1 : 0;
  L.split_rows = L.M;  // one plain block per unit
  L.split_stride = 0;
  L.vec_ok = 1;
  L.vec_c = 1;
  for (const Item& it : items) {
    if (reinterpret_cast<uintptr_t>(it.ptrs.a) % 16 || reinterpret_cast<uintptr_t>(it.ptrs.b) % 16) L.vec_ok = 0;
    if (reinterpret_cast<uintptr_t>(it.ptrs.c) % (L.out_bf16 ? 8 : 16)) L.vec_c = 0;
  }
  if (!b_padded) L.vec_ok = 0;
  const bool skinny = m <= kSkinnyMaxM;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (size_t first = 0; first < items.size(); first += kMaxUnitsPerLaunch) {
    const size_t cnt = std::min(items.size() - first, static_cast<size_t>(kMaxUnitsPerLaunch));
    L.n_units = static_cast<int32_t>(cnt);
    for (size_t i = 0; i < cnt; ++i) L.u[i] = items[first + i].ptrs;
    hipError_t e = skinny ? launch_gemm_skinny(L, s) : launch_gemm_mfma(L, s);
    if (e != hipSuccess) return hip_fail(e, "sm_local_gemm launch");
  }
  return SM_OK;
}

namespace shardmm {

// 16-byte vectors need aligned row starts in every source and the target.
void set_vec_flags(std::vector<RowJob>& jobs, int32_t elem_bytes) {
  const int64_t per = 16 / elem_bytes;
  for (RowJob& J : jobs) {
    const bool ok = reinterpret_cast<uintptr_t>(J.src) % 16 == 0 && reinterpret_cast<uintptr_t>(J.dst) % 16 == 0 &&
                    J.lds % per == 0 && J.ldd % per == 0 && J.src_stride % per == 0 && J.cols % per == 0;
    J.vec = ok ? 1 : 0;
  }
}

int32_t run_jobs(std::vector<RowJob>& jobs, int32_t n_sum, int32_t elem_bytes, hipStream_t s, const char* where) {
  set_vec_flags(jobs, elem_bytes);
  RowLaunch L;
  for (size_t first = 0; first < jobs.size(); first += kMaxJobsPerLaunch) {
    std::memset(&L, 0, sizeof L);
    const size_t cnt = std::min(jobs.size() - first, static_cast<size_t>(kMaxJobsPerLaunch));
    L.n_jobs = static_cast<int32_t>(cnt);
    L.n_sum = n_sum;
    L.elem_bytes = elem_bytes;
    L.max_rows = 0;
    int32_t max_cols = 0;
    for (size_t i = 0; i < cnt; ++i) {
      L.jobs[i] = jobs[first + i];
      L.max_rows = std::max(L.max_rows, L.jobs[i].rows);
      max_cols = std::max(max_cols, L.jobs[i].cols);
    }
    // Few rows: split rows into column chunks (>= 1024 columns each) so that
    // the launch has enough workgroups to keep HBM busy.
    const int64_t base = static_cast<int64_t>(cnt) * L.max_rows;
    int64_t n_chunks = 1;
    if (base < 2048) n_chunks = std::min<int64_t>((2048 + base - 1) / base, (max_cols + 1023) / 1024);
    n_chunks = std::max<int64_t>(n_chunks, 1);
    int64_t chunk = (max_cols + n_chunks - 1) / n_chunks;
    chunk = (chunk + 7) / 8 * 8;
    L.chunk = static_cast<int32_t>(chunk);
    L.n_chunks = static_cast<int32_t>((max_cols + chunk - 1) / chunk);
    if (static_cast<int64_t>(L.max_rows) * L.n_chunks > INT32_MAX) return fail(SM_ERR_SHAPE, "too many rows");
    // Copies of short rows: 16 KiB of rows per workgroup.
    const int64_t row_bytes = static_cast<int64_t>(max_cols) * elem_bytes;
    L.tile_rows = 1;
    if (n_sum == 1 && L.n_chunks == 1 && row_bytes <= 4096)
      L.tile_rows = static_cast<int32_t>(std::min<int64_t>(16384 / row_bytes, L.max_rows));
    hipError_t e = launch_rows(L, s);
    if (e != hipSuccess) return hip_fail(e, where);
  }
  return SM_OK;
}

}  // namespace shardmm

extern "C" int32_t sm_reduce_partials(const sm_plan_t* plan, const sm_buf* partials, const sm_buf* out,
                                      int32_t mode, int32_t group_begin, int32_t group_count, void* stream) {
  clear_error();
  int32_t st = check_plan(plan);
  if (st) return st;
  const sm_plan_t& p = *plan;
  if (p.kase != SM_CASE3) return fail(SM_ERR_CASE, "only case-3 plans have partial sums to reduce");
  if (mode != SM_ALLREDUCE && mode != SM_REDUCESCATTER) return fail(SM_ERR_ARG, "unknown reduce mode");
  if (p.out_dtype != SM_F32) return fail(SM_ERR_DTYPE, "partials are float32");
  if (group_count < 1 || group_begin < 0 || group_begin > p.n_groups - group_count)
    return fail(SM_ERR_ARG, "group range outside [0, n_groups)");
  if ((st = check_buf_basic(partials, "partials", SM_F32))) return st;
  if ((st = check_buf_basic(out, "out", SM_F32))) return st;
  if (partials->block_stride == 0)
    return fail(SM_ERR_UNREDUCED, "partials overlap in output coordinates; they must be stacked");
  const int64_t m = p.c_local[0], n = p.c_local[1];
  const int32_t N = p.n_partials;
  if (m > INT32_MAX || n > INT32_MAX) return fail(SM_ERR_SHAPE, "block too large");
  if ((st = check_stacked(partials, m, n, "partials"))) return st;
  {
    BlockRef last{static_cast<i128>(group_count) * N * partials->block_stride - partials->block_stride, m, n};
    if ((st = check_extent(partials, last, "partials"))) return st;
  }
  const bool rs = mode == SM_REDUCESCATTER;
  if (rs && m % N) return fail(SM_ERR_INDIVISIBLE, "rows of a block do not split N ways");
  const int64_t orows = rs ? m / N : m;
  if (out->block_stride == 0) {
    if (out->ld < p.K) return fail(SM_ERR_SHAPE, "out: global layout needs ld >= K");
  } else if ((st = check_stacked(out, orows, n, "out"))) {
    return st;
  }

  std::vector<RowJob> jobs;
  const float* P = static_cast<const float*>(partials->ptr);
  float* O = static_cast<float*>(out->ptr);
  for (int32_t g = group_begin; g < group_begin + group_count; ++g) {
    const int64_t bi = g / p.c_grid[1], bk = g % p.c_grid[1];
    const int64_t src0 = static_cast<int64_t>(g - group_begin) * N * partials->block_stride;
    const int32_t nblk = rs ? N : 1;
    for (int32_t y = 0; y < nblk; ++y) {
      BlockRef d;
      d.rows = orows;
      d.cols = n;
      if (out->block_stride == 0)
        d.offset = (static_cast<i128>(bi) * m + y * orows) * out->ld + bk * n;
      else
        d.offset = (static_cast<i128>(g - group_begin) * nblk + y) * out->block_stride;
      if ((st = check_extent(out, d, "out"))) return st;
      RowJob J;
      J.src = P + src0 + y * orows * partials->ld;
      J.dst = O + d.off();
      J.src_stride = partials->block_stride;
      J.lds = partials->ld;
      J.ldd = out->ld;
      J.rows = static_cast<int32_t>(orows);
      J.cols = static_cast<int32_t>(n);
      jobs.push_back(J);
    }
  }
  if ((st = check_device_memory(partials->ptr, "partials")) || (st = check_device_memory(out->ptr, "out"))) return st;
  return run_jobs(jobs, N, 4, static_cast<hipStream_t>(stream), "sm_reduce_partials launch");
}

extern "C" int32_t sm_gather_shards(const sm_plan_t* plan, int32_t what, const sm_buf* shards, const sm_buf* out,
                                    void* stream) {
  clear_error();
  int32_t st = check_plan(plan);
  if (st) return st;
  const sm_plan_t& p = *plan;
  if (what == SM_WHAT_C_PARTIAL)
    return fail(SM_ERR_UNREDUCED, "concatenating unreduced partials does not add them; reduce first");
  if (what < SM_WHAT_A || what > SM_WHAT_C_SCATTERED) return fail(SM_ERR_ARG, "unknown sm_what");
  if ((what == SM_WHAT_C_BLOCKS) && p.kase != SM_CASE1 && p.kase != SM_CASE3)
    return fail(SM_ERR_CASE, "no local output blocks in a case-2/4 plan");
  if (what == SM_WHAT_C_SCATTERED && p.kase != SM_CASE3)
    return fail(SM_ERR_CASE, "reduce-scatter blocks exist only for case 3");

  int32_t dtype;
  int64_t rows, cols, grid_r, grid_c, gwidth;
  switch (what) {
    case SM_WHAT_A:
      dtype = p.in_dtype;
      rows = p.a_local[0];
      cols = p.a_local[1];
      grid_r = p.a_grid[0];
      grid_c = p.a_grid[1];
      gwidth = p.J;
      break;
    case SM_WHAT_B:
      dtype = p.in_dtype;
      rows = p.b_local[0];
      cols = p.b_local[1];
      grid_r = p.b_grid[0];
      grid_c = p.b_grid[1];
      gwidth = p.K;
      break;
    case SM_WHAT_C_BLOCKS:
      dtype = p.out_dtype;
      rows = p.c_local[0];
      cols = p.c_local[1];
      grid_r = p.c_grid[0];
      grid_c = p.c_grid[1];
      gwidth = p.K;
      break;
    default:  // SM_WHAT_C_SCATTERED
      if (p.c_local[0] % p.n_partials) return fail(SM_ERR_INDIVISIBLE, "rows of a block do not split N ways");
      dtype = p.out_dtype;
      rows = p.c_local[0] / p.n_partials;
      cols = p.c_local[1];
      grid_r = static_cast<int64_t>(p.c_grid[0]) * p.n_partials;
      grid_c = p.c_grid[1];
      gwidth = p.K;
      break;
  }
  if (rows > INT32_MAX || cols > INT32_MAX) return fail(SM_ERR_SHAPE, "block too large");
  if ((st = check_buf_basic(shards, "shards", dtype))) return st;
  if ((st = check_buf_basic(out, "out", dtype))) return st;
  if (shards->block_stride == 0) return fail(SM_ERR_ARG, "shards must use the stacked layout");
  if (out->block_stride != 0) return fail(SM_ERR_ARG, "out must use the global layout");
  if (out->ld < gwidth) return fail(SM_ERR_SHAPE, "out: ld smaller than the global width");
  if ((st = check_stacked(shards, rows, cols, "shards"))) return st;

  // Stacked order of blocks: for C_SCATTERED the (group, y) index, which is
  // the row-block index (bi * N + y) when the grid has one block column;
  // in general block id = (g * N + y) with g = bi * grid_c + bk.
  std::vector<RowJob> jobs;
  const size_t esz = dtype_size(dtype);
  for (int64_t id = 0; id < grid_r * grid_c; ++id) {
    int64_t r0, c0;
    if (what == SM_WHAT_C_SCATTERED) {
      const int64_t g = id / p.n_partials, y = id % p.n_partials;
      r0 = (g / p.c_grid[1]) * p.c_local[0] + y * rows;
      c0 = (g % p.c_grid[1]) * cols;
    } else {
      r0 = (id / grid_c) * rows;
      c0 = (id % grid_c) * cols;
    }
    BlockRef s{static_cast<i128>(id) * shards->block_stride, rows, cols};
    BlockRef d{static_cast<i128>(r0) * out->ld + c0, rows, cols};
    if ((st = check_extent(shards, s, "shards"))) return st;
    if ((st = check_extent(out, d, "out"))) return st;
    RowJob J;
    J.src = static_cast<const char*>(shards->ptr) + s.off() * static_cast<int64_t>(esz);
    J.dst = static_cast<char*>(out->ptr) + d.off() * static_cast<int64_t>(esz);
    J.src_stride = 0;
    J.lds = shards->ld;
    J.ldd = out->ld;
    J.rows = static_cast<int32_t>(rows);
    J.cols = static_cast<int32_t>(cols);
    jobs.push_back(J);
  }
  if ((st = check_device_memory(shards->ptr, "shards")) || (st = check_device_memory(out->ptr, "out"))) return st;
  return run_jobs(jobs, 1, static_cast<int32_t>(esz), static_cast<hipStream_t>(stream), "sm_gather_shards launch");
}

namespace shardmm {

ReduceWorkspace reduce_workspace(const sm_plan_t& p, int64_t groups) {
  ReduceWorkspace w{};
  const int64_t m = p.c_local[0], n = p.c_local[1];
  w.ldp = (n + 3) / 4 * 4;
  if (m > kSkinnyMaxM) {
    // One launch over the group's whole J has groups x tiles-per-block
    // workgroups; when that leaves CUs idle, the N units' products in
    // parallel and a rank-ordered sum (two launches) are several times
    // faster (a 128-row batch on [28672, 8192] split over 8 ranks: 455 us
    // against 105 us).
    const int64_t bm = m <= 128 ? 128 : kTileM;
    const int64_t tiles = groups * ((m + bm - 1) / bm) * ((n + kTileN - 1) / kTileN);
    if (p.n_partials > 1 && tiles < kFewTiles) {
      w.two_pass = 1;
      w.part_bytes = groups * p.n_partials * m * w.ldp * 4;
    }
    return w;
  }
  w.n_colblk = static_cast<int32_t>((n + kSkinnyCols - 1) / kSkinnyCols);
  w.counter_bytes = (groups * w.n_colblk * 4 + 255) / 256 * 256;
  w.part_bytes = groups * p.n_partials * m * w.ldp * 4;
  return w;
}

// Local products of a case-3 plan and their rank-ordered reduction, for
// sm_local_gemm_reduce (no scratch), sm_local_gemm_reduce_ws (the caller's
// workspace) and the no-allocation entry point (the library's static
// scratch). Products of more than 64 rows: one tile-kernel launch per batch
// of groups, K = the group's whole J, no scratch; or, when that launch would
// have few tiles and the scratch holds the partials, the units' products into
// the scratch (one tile-kernel launch) and their rank-ordered sum (one row
// launch). Skinny products: the split-J kernel with the fused reduction,
// whose counters and partials live in the scratch `sc` describes.
int32_t gemm_reduce_impl(const sm_plan_t* plan, const sm_buf* A, const sm_buf* B, const sm_buf* out, int32_t mode,
                         int32_t group_begin, int32_t group_count, const ReduceScratch& sc, void* stream,
                         const char* where) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t st = check_plan(plan);
  if (st) return st;
  const sm_plan_t& p = *plan;
  if (p.kase == SM_CASE2 || p.kase == SM_CASE4)
    return fail(SM_ERR_NEEDS_GATHER, "all-gather the J-sharded operand first (sm_plan_gathered)");
  if (p.kase != SM_CASE3) return fail(SM_ERR_CASE, "only case-3 plans have partial sums to reduce");
  if (mode != SM_ALLREDUCE && mode != SM_REDUCESCATTER) return fail(SM_ERR_ARG, "unknown reduce mode");
  if (p.in_dtype != SM_BF16 || p.out_dtype != SM_F32) return fail(SM_ERR_DTYPE, "bfloat16 inputs, float32 output");
  if (group_count < 1 || group_begin < 0 || group_begin > p.n_groups - group_count)
    return fail(SM_ERR_ARG, "group range outside [0, n_groups)");
  if ((st = check_buf_basic(A, "A", SM_BF16))) return st;
  if ((st = check_buf_basic(B, "B", SM_BF16))) return st;
  if ((st = check_buf_basic(out, "out", SM_F32))) return st;
  if (A->block_stride != 0 || B->block_stride != 0)
    return fail(SM_ERR_ARG, "the fused path reads A and B in the global layout (block_stride 0)");
  if (A->ld < p.J) return fail(SM_ERR_SHAPE, "A: global layout needs ld >= J");
  if (B->ld < p.K) return fail(SM_ERR_SHAPE, "B: global layout needs ld >= K");
  const int64_t m = p.c_local[0], n = p.c_local[1], kfull = p.J;
  const int32_t N = p.n_partials;
  const bool skinny = m <= kSkinnyMaxM;
  if (skinny && sc.kind == ReduceScratch::kNone)
    return fail(SM_ERR_SHAPE, "local products of at most 64 rows reduce through a workspace "
                              "(sm_local_gemm_reduce_ws)");
  if (m > INT32_MAX / 2 || n > INT32_MAX / 2 || kfull > INT32_MAX / 2) return fail(SM_ERR_SHAPE, "shape too large");
  if (((m + kTileM - 1) / kTileM) * ((n + kTileN - 1) / kTileN) * kMaxUnitsPerLaunch > INT32_MAX)
    return fail(SM_ERR_SHAPE, "too many output tiles for one launch grid");
  if (skinny && N > kMaxUnitsPerLaunch)
    return fail(SM_ERR_SHAPE, "the fused split-J reduction takes at most 64 partials per group");
  const bool rs = mode == SM_REDUCESCATTER;
  if (rs && m % N) return fail(SM_ERR_INDIVISIBLE, "rows of a block do not split N ways");
  const int64_t orows = rs ? m / N : m;
  if (out->block_stride == 0) {
    if (out->ld < p.K) return fail(SM_ERR_SHAPE, "out: global layout needs ld >= K");
  } else if ((st = check_stacked(out, orows, n, "out"))) {
    return st;
  }
  ReduceWorkspace W{};
  uint32_t* counters = nullptr;
  float* parts = nullptr;
  if (skinny) {
    W = reduce_workspace(p, group_count);
    if (sc.kind == ReduceScratch::kCaller) {
      if (!sc.ws) return fail(SM_ERR_ARG, "NULL workspace");
      if (reinterpret_cast<uintptr_t>(sc.ws) % 256) return fail(SM_ERR_ALIGN, "workspace not 256-byte aligned");
      if (sc.ws_bytes < W.counter_bytes + W.part_bytes)
        return fail(SM_ERR_SHAPE, "workspace of " + std::to_string(sc.ws_bytes) + " bytes, the call needs " +
                                      std::to_string(W.counter_bytes + W.part_bytes));
      counters = static_cast<uint32_t*>(sc.ws);
      parts = reinterpret_cast<float*>(static_cast<char*>(sc.ws) + W.counter_bytes);
    } else if (sc.kind == ReduceScratch::kFixed) {
      if (W.counter_bytes > sc.counter_cap || W.part_bytes > sc.part_cap)
        return fail(SM_ERR_SHAPE, "the call needs " + std::to_string(W.counter_bytes) + " bytes of counters and " +
                                      std::to_string(W.part_bytes) + " bytes of partials; the static scratch holds " +
                                      std::to_string(sc.counter_cap) + " and " + std::to_string(sc.part_cap) +
                                      " (use sm_local_gemm_reduce_ws)");
      counters = sc.counters;
      parts = sc.parts;
    }
  }
  // Products whose one launch over the whole J would leave CUs idle run as
  // the N units' products into the scratch, then their rank-ordered sum,
  // whenever a scratch that holds the partials is at hand (it is optional
  // for them: without one, the single launch).
  bool two_pass = false;
  if (!skinny && sc.kind != ReduceScratch::kNone) {
    W = reduce_workspace(p, group_count);
    if (W.two_pass && sc.kind == ReduceScratch::kCaller && sc.ws) {
      if (reinterpret_cast<uintptr_t>(sc.ws) % 256) return fail(SM_ERR_ALIGN, "workspace not 256-byte aligned");
      if (sc.ws_bytes >= W.part_bytes) {
        parts = static_cast<float*>(sc.ws);
        two_pass = true;
      }
    } else if (W.two_pass && sc.kind == ReduceScratch::kFixed && W.part_bytes <= sc.part_cap) {
      parts = sc.parts;
      two_pass = true;
    }
  }
  const int64_t kl = p.a_local[1];

  GemmLaunch L;
  std::memset(&L, 0, sizeof L);
  L.M = static_cast<int32_t>(m);
  L.N = static_cast<int32_t>(n);
  L.K = static_cast<int32_t>(skinny || two_pass ? kl : kfull);
  L.tiles_m = static_cast<int32_t>((m + kTileM - 1) / kTileM);
  L.tiles_n = static_cast<int32_t>((n + kTileN - 1) / kTileN);
  L.lda = A->ld;
  L.ldb = B->ld;
  L.ldc = two_pass ? W.ldp : out->ld;
  L.epilogue = kEpiStore;
  L.out_bf16 = 0;
  const bool split = rs && out->block_stride != 0;
  L.split_rows = split && !two_pass ? static_cast<int32_t>(orows) : L.M;
  L.split_stride = split && !two_pass ? out->block_stride : 0;
  L.vec_ok = 1;
  L.vec_c = 1;

  struct Item {
    int32_t b_id, a_row;
    GemmUnitPtrs ptrs;
  };
  std::vector<Item> items;
  std::vector<float*> group_out;
  bool out_vec = n % 4 == 0 && out->ld % 4 == 0 && L.split_stride % 4 == 0;
  for (int32_t g = group_begin; g < group_begin + group_count; ++g) {
    // Rank order y = 0..N-1 covers J contiguously in both operands.
    UnitView v;
    if ((st = unit_view(p, g * N, &v))) return st;
    if (v.a_col0 != 0 || v.b_row0 != 0) return fail(SM_ERR_ARG, "J slices are not contiguous from 0");
    BlockRef ra{static_cast<i128>(v.a_row0) * A->ld, m, kfull};
    BlockRef rb{v.b_col0, kfull, n};
    if ((st = check_extent(A, ra, "A"))) return st;
    if ((st = check_extent(B, rb, "B"))) return st;
    int64_t coff;
    if (out->block_stride == 0) {
      BlockRef rc{static_cast<i128>(v.c_row0) * out->ld + v.c_col0, m, n};
      if ((st = check_extent(out, rc, "out"))) return st;
      coff = rc.off();
    } else {
      const int32_t nblk = rs ? N : 1;
      const i128 c0 = static_cast<i128>(g - group_begin) * nblk * out->block_stride;
      for (int32_t y = 0; y < nblk; ++y) {
        BlockRef rc{c0 + static_cast<i128>(y) * out->block_stride, orows, n};
        if ((st = check_extent(out, rc, "out"))) return st;
      }
      coff = static_cast<int64_t>(c0);  // bounded by the checks above
    }
    float* c = static_cast<float*>(out->ptr) + coff;
    if (reinterpret_cast<uintptr_t>(c) % 16) {
      L.vec_c = 0;  // float32 partial sums
      out_vec = false;
    }
    if (!b_rows_padded(B, rb)) L.vec_ok = 0;
    if (skinny || two_pass) {
      // the N units of the group, each on its own J slice: A view
      // [m, k_local] at column y * k_local, B view [k_local, n] at row
      // y * k_local; the tile kernel (two_pass) stores unit y's product at
      // its place in the stacked partials
      group_out.push_back(c);
      for (int32_t y = 0; y < N; ++y) {
        Item it;
        it.b_id = y * p.b_grid[1] + v.b_block[1];
        it.a_row = v.a_block[0];
        it.ptrs.a = static_cast<const uint16_t*>(A->ptr) + ra.off() + y * kl;
        it.ptrs.b = static_cast<const uint16_t*>(B->ptr) + rb.off() + static_cast<int64_t>(y) * kl * B->ld;
        it.ptrs.c = two_pass ? parts + ((static_cast<int64_t>(g - group_begin) * N + y) * m * W.ldp) : nullptr;
        if (reinterpret_cast<uintptr_t>(it.ptrs.a) % 16 || reinterpret_cast<uintptr_t>(it.ptrs.b) % 16) L.vec_ok = 0;
        items.push_back(it);
      }
    } else {
      Item it;
      it.b_id = v.b_block[1];
      it.a_row = v.a_block[0];
      it.ptrs.a = static_cast<const uint16_t*>(A->ptr) + ra.off();
      it.ptrs.b = static_cast<const uint16_t*>(B->ptr) + rb.off();
      it.ptrs.c = c;
      if (reinterpret_cast<uintptr_t>(it.ptrs.a) % 16 || reinterpret_cast<uintptr_t>(it.ptrs.b) % 16) L.vec_ok = 0;
      items.push_back(it);
    }
  }
  if ((st = check_device_memory(A->ptr, "A")) || (st = check_device_memory(B->ptr, "B")) ||
      (st = check_device_memory(out->ptr, "out")))
    return st;
  if ((skinny || two_pass) && sc.kind == ReduceScratch::kCaller && (st = check_device_memory(sc.ws, "workspace")))
    return st;
  if (sc.kind == ReduceScratch::kValidate) return SM_OK;

  if (skinny) {
    SkinnyReduce R;
    std::memset(&R, 0, sizeof R);
    R.part_stride = m * W.ldp;
    R.ldp = W.ldp;
    R.n_colblk = W.n_colblk;
    R.n_partials = N;
    R.split_rows = L.split_rows;
    R.split_stride = L.split_stride;
    R.ldo = out->ld;
    R.vec_out = out_vec ? 1 : 0;
    const int32_t groups_per_launch = kMaxUnitsPerLaunch / N;
    for (int32_t g0 = 0; g0 < group_count; g0 += groups_per_launch) {
      const int32_t gc = std::min(groups_per_launch, group_count - g0);
      L.n_units = gc * N;
      for (int32_t i = 0; i < gc * N; ++i) L.u[i] = items[static_cast<size_t>(g0) * N + i].ptrs;
      for (int32_t i = 0; i < gc; ++i) R.out[i] = group_out[g0 + i];
      R.part = parts + static_cast<int64_t>(g0) * N * R.part_stride;
      R.counters = counters + static_cast<int64_t>(g0) * W.n_colblk;
      hipError_t e = launch_gemm_skinny_reduce(L, R, s);
      if (e != hipSuccess) return hip_fail(e, where);
    }
    return SM_OK;
  }

  std::stable_sort(items.begin(), items.end(), [](const Item& x, const Item& y) {
    return x.b_id != y.b_id ? x.b_id < y.b_id : x.a_row < y.a_row;
  });
  for (size_t first = 0; first < items.size(); first += kMaxUnitsPerLaunch) {
    const size_t cnt = std::min(items.size() - first, static_cast<size_t>(kMaxUnitsPerLaunch));
    L.n_units = static_cast<int32_t>(cnt);
    for (size_t i = 0; i < cnt; ++i) L.u[i] = items[first + i].ptrs;
    hipError_t e = launch_gemm_mfma(L, s);
    if (e != hipSuccess) return hip_fail(e, where);
  }
  if (!two_pass) return SM_OK;
  // the rank-ordered sums of the partials, as sm_reduce_partials does them
  std::vector<RowJob> jobs;
  const int32_t nblk = rs ? N : 1;
  for (int32_t gi = 0; gi < group_count; ++gi) {
    const float* src = parts + static_cast<int64_t>(gi) * N * m * W.ldp;
    for (int32_t y = 0; y < nblk; ++y) {
      RowJob J;
      J.src = src + static_cast<int64_t>(y) * orows * W.ldp;
      J.dst = group_out[gi] + (out->block_stride ? y * out->block_stride : static_cast<int64_t>(y) * orows * out->ld);
      J.src_stride = m * W.ldp;
      J.lds = W.ldp;
      J.ldd = out->ld;
      J.rows = static_cast<int32_t>(orows);
      J.cols = static_cast<int32_t>(n);
      jobs.push_back(J);
    }
  }
  return run_jobs(jobs, N, 4, s, where);
}

}  // namespace shardmm

extern "C" int32_t sm_local_gemm_reduce(const sm_plan_t* plan, const sm_buf* A, const sm_buf* B, const sm_buf* out,
                                        int32_t mode, int32_t group_begin, int32_t group_count, void* stream) {
  clear_error();
  return gemm_reduce_impl(plan, A, B, out, mode, group_begin, group_count, ReduceScratch{}, stream,
                          "sm_local_gemm_reduce launch");
}

extern "C" int32_t sm_gemm_reduce_workspace(const sm_plan_t* plan, int32_t group_count, int64_t* bytes) {
  clear_error();
  int32_t st = check_plan(plan);
  if (st) return st;
  if (!bytes) return fail(SM_ERR_ARG, "NULL bytes");
  if (plan->kase != SM_CASE3) return fail(SM_ERR_CASE, "only case-3 plans have partial sums to reduce");
  if (group_count < 1 || group_count > plan->n_groups) return fail(SM_ERR_ARG, "group_count outside [1, n_groups]");
  const ReduceWorkspace w = reduce_workspace(*plan, group_count);
  *bytes = w.counter_bytes + w.part_bytes;
  return SM_OK;
}

extern "C" int32_t sm_local_gemm_reduce_ws(const sm_plan_t* plan, const sm_buf* A, const sm_buf* B,
                                           const sm_buf* out, int32_t mode, int32_t group_begin,
                                           int32_t group_count, void* workspace, int64_t workspace_bytes,
                                           void* stream) {
  clear_error();
  ReduceScratch sc;
  sc.kind = ReduceScratch::kCaller;
  sc.ws = workspace;
  sc.ws_bytes = workspace_bytes;
  return gemm_reduce_impl(plan, A, B, out, mode, group_begin, group_count, sc, stream,
                          "sm_local_gemm_reduce_ws launch");
}
