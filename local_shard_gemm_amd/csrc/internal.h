// Internal declarations shared by the library's translation units.
#pragma once

#include <cstdint>
#include <string>

#include "shardmm.h"

namespace shardmm {

constexpr uint32_t kPlanMagic = 0x5348414Du;  // "SHAM"
constexpr int64_t kMaxRanks = int64_t(1) << 20;  // logical ranks per mesh

// Record a failure and return its status (thread-local text for sm_last_error).
int32_t fail(int32_t status, const std::string& msg);
void clear_error();

// Flattened block index of `coords` over an ordered axis list (first = major).
int32_t block_of(const sm_mesh& mesh, const int32_t* axes, int32_t n, const int32_t* coords);
int32_t axes_product(const sm_mesh& mesh, const int32_t* axes, int32_t n);
void rank_coords(const sm_mesh& mesh, int32_t rank, int32_t* coords);

// Global coordinates of one unit's operand and output views.
struct UnitView {
  int32_t a_block[2], b_block[2], c_block[2];
  int64_t a_row0, a_col0, b_row0, b_col0, c_row0, c_col0;
  int32_t group, partial;
};
int32_t unit_view(const sm_plan_t& p, int32_t unit, UnitView* out);

int32_t check_plan(const sm_plan_t* p);

// Axis indices in range and no axis on two dims (SM_ERR_SPEC / SM_ERR_AXIS_REUSED).
int32_t validate_spec(const sm_mesh& mesh, const sm_spec& s, const char* what);

size_t dtype_size(int32_t dt);

// ---- buffer checks and row-job launches shared by the device entry points

// One logical block of a buffer: element offset of its (0,0) and its extent.
// Offsets are computed in 128 bits from caller-supplied sizes, so that no
// product can wrap before check_extent bounds it by the buffer's elems;
// off() narrows it once the check has passed.
typedef __int128 i128;
struct BlockRef {
  i128 offset;
  int64_t rows, cols;
  int64_t off() const { return static_cast<int64_t>(offset); }
};
// Pointer, alignment, ld, block_stride and elems of one sm_buf.
int32_t check_buf_basic(const sm_buf* b, const char* what, int32_t dtype);
// The block lies inside the buffer.
int32_t check_extent(const sm_buf* b, const BlockRef& r, const char* what);
// The GPU can address the memory at ptr (device, managed or HIP host memory).
int32_t check_device_memory(const void* ptr, const char* what);
// Stacked blocks of rows x cols do not overlap.
int32_t check_stacked(const sm_buf* b, int64_t rows, int64_t cols, const char* what);

// ---- the fused local products + reduction (case 3)

// Workspace of sm_local_gemm_reduce_ws. Skinny products (fused split-J
// reduction): arrival counters (one 32-bit word per group and column block,
// rounded up to 256 bytes), then the groups' N partials, each [M, ldp]
// float32. Products whose one-launch grid would have fewer tiles than the
// GPU has CUs (two_pass): the N partials only, written by the tile kernel
// and summed in rank order by the row kernel.
struct ReduceWorkspace {
  int64_t counter_bytes, part_bytes, ldp;
  int32_t n_colblk;
  int32_t two_pass;
};
// Tiles below which a one-launch fused product over the whole J leaves CUs
// idle (the MI355X has 256).
constexpr int64_t kFewTiles = 256;
// Workspace layout of a fused reduction over `groups` groups.
ReduceWorkspace reduce_workspace(const sm_plan_t& p, int64_t groups);
// Where a fused reduction keeps its counters and partials (skinny products),
// or its partials (few-tile taller products).
struct ReduceScratch {
  enum Kind : int32_t {
    kNone = 0,      // none (sm_local_gemm_reduce): skinny products are refused, taller ones run as one launch
    kCaller = 1,    // the caller's workspace `ws`, split as documented for sm_local_gemm_reduce_ws
    kFixed = 2,     // fixed regions (the static scratch): counters, then partials, each with a capacity
    kValidate = 3,  // run every host check, launch nothing
  };
  int32_t kind = kNone;
  void* ws = nullptr;
  int64_t ws_bytes = 0;
  uint32_t* counters = nullptr;
  int64_t counter_cap = 0;
  float* parts = nullptr;
  int64_t part_cap = 0;
};
// sm_local_gemm_reduce and its scratch variants: every check on the host,
// then the launches on `stream` (a hipStream_t).
int32_t gemm_reduce_impl(const sm_plan_t* plan, const sm_buf* A, const sm_buf* B, const sm_buf* out, int32_t mode,
                         int32_t group_begin, int32_t group_count, const ReduceScratch& sc, void* stream,
                         const char* where);

}  // namespace shardmm
