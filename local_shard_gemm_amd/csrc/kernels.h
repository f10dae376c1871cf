// Launch descriptors of libshardmm's device kernels. Everything here is
// passed by value as kernel arguments (no device-side tables, no workspace).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

namespace shardmm {

constexpr int kMaxUnitsPerLaunch = 64;
constexpr int kMaxJobsPerLaunch = 32;

// One local product: pointers already offset to the unit's views.
struct GemmUnitPtrs {
  const uint16_t* a;  // [M, K] bfloat16, leading dim lda
  const uint16_t* b;  // [K, N] bfloat16, leading dim ldb
  void* c;            // [M, N] float32 or bfloat16, leading dim ldc
};

enum : int32_t { kEpiStore = 0, kEpiGelu = 1 };

struct GemmLaunch {
  int32_t M, N, K;           // local shape shared by all units of the launch
  int32_t tiles_m, tiles_n;  // MFMA kernel only
  int32_t n_units;
  int64_t lda, ldb, ldc;
  int32_t epilogue;          // kEpiStore / kEpiGelu
  int32_t out_bf16;          // 1: store bfloat16 (RNE), 0: float32
  int32_t vec_ok;            // 1: every A/B view starts 16-byte aligned
  int32_t vec_c;             // 1: every C view starts on 4 elements (8 bytes bf16, 16 float32): vector stores
  // Output rows in blocks: row r goes to c + (r / split_rows) * split_stride
  // + (r % split_rows) * ldc (split_rows >= M: one plain [M, N] block).
  int32_t split_rows;
  int64_t split_stride;
  GemmUnitPtrs u[kMaxUnitsPerLaunch];  // in scheduling order
};

// Rank-order sum / copy of row blocks: dst[r, c] = sum_{y<N} src_y[r, c]
// with src_y = src + y * src_stride (elements).
struct RowJob {
  const void* src;
  void* dst;
  int64_t src_stride;
  int64_t lds, ldd;
  int32_t rows, cols;
  int32_t vec;  // 1: src, dst, lds, ldd and src_stride allow 16-byte vectors
};

struct RowLaunch {
  int32_t n_jobs;
  int32_t n_sum;       // N (1 = plain copy)
  int32_t elem_bytes;  // 4 (float32 sum / copy) or 2 (bfloat16 copy)
  int32_t max_rows;
  int32_t chunk;      // columns per workgroup (a multiple of 8)
  int32_t n_chunks;   // column chunks per row
  int32_t tile_rows;  // copies (n_sum 1) of short rows: rows per workgroup (1 = one row each)
  RowJob jobs[kMaxJobsPerLaunch];
};

// Rank-ordered reduction fused into the skinny split-J kernel. Every
// workgroup (one unit, one block of 256 output columns) writes its unit's
// partial block into the workspace and counts itself in at the counter of
// its (group, column block); the workgroup that arrives last sums the
// group's N partials in rank order and writes the finished rows. Units of a
// launch are ordered group-major (unit = group * N + y).
struct SkinnyReduce {
  float* part;            // partial of launch unit i at part + i * part_stride
  int64_t part_stride;    // elements between two units' partials
  int64_t ldp;            // leading dimension of a partial
  uint32_t* counters;     // [groups of the launch][n_colblk], zero on entry, left zero
  int32_t n_colblk;       // column blocks per unit (grid x)
  int32_t n_partials;     // N
  int32_t split_rows;     // output row r -> out + (r / split_rows) * split_stride + (r % split_rows) * ldo
  int32_t vec_out;        // 1: 16-byte vectors for every partial and output row
  int64_t split_stride;
  int64_t ldo;
  float* out[kMaxUnitsPerLaunch];  // finished block of launch group g
};

hipError_t launch_gemm_mfma(const GemmLaunch& L, hipStream_t s);
hipError_t launch_gemm_skinny(const GemmLaunch& L, hipStream_t s);
// The skinny kernel with the fused reduction (float32 store epilogue only).
hipError_t launch_gemm_skinny_reduce(const GemmLaunch& L, const SkinnyReduce& R, hipStream_t s);
// Zero `n` 32-bit words (a fill kernel, so that the call can sit in a
// captured graph).
hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t s);
hipError_t launch_rows(const RowLaunch& L, hipStream_t s);
// Host side: launch row jobs (rank-ordered sums when n_sum > 1, copies when
// n_sum == 1) in batches of kMaxJobsPerLaunch; returns an sm_status.
int32_t run_jobs(std::vector<RowJob>& jobs, int32_t n_sum, int32_t elem_bytes, hipStream_t s, const char* where);
// SM_ERR_HIP with the runtime's text.
int32_t hip_fail(hipError_t e, const char* where);
// Rank-ordered reduce of whole rows followed by a layer norm of each row
// (float32 only, 16-byte vectors, rows of at most 32768 elements).
hipError_t launch_rows_layernorm(const RowLaunch& L, const float* gamma, const float* beta, float eps,
                                 hipStream_t s);
constexpr int kLayerNormMaxCols = 32768;

// Tile sizes of the MFMA kernel (host side uses them for the grid).
constexpr int kTileM = 256, kTileN = 256, kTileK = 64;
// Rows handled by the skinny split-J kernel, and its output columns per
// workgroup.
constexpr int kSkinnyMaxM = 64;
constexpr int kSkinnyCols = 256;

}  // namespace shardmm
