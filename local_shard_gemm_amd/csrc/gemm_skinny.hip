// Split-J kernel for skinny local products (M <= 64 rows): each rank's
// partial P_u = X_u . A_u with X_u [M, K] small and A_u [K, N] streamed
// once from HBM. Used for the row-parallel step Z_i = X_i A_i with a small
// batch (mbrenndoerfer.com "Row Parallelism": Z_i = X_i A_i; the partials
// have the full output shape and are summed afterwards).
//
// Design (gfx950): the work is bound by HBM reads of A_u, so the kernel is
// shaped for the access pattern HBM streams best, not for matrix-core
// throughput (measured on the [28672, 8192] bf16 stream: workgroups that own
// 256 columns and read 512 contiguous bytes per row per 32 lanes reach
// 6.4-6.6 TB/s; 128-column workgroups stay at 5.9 TB/s).
//  * One workgroup = 4 waves = one unit and 256 output columns; the unit's
//    K range is split into 4 contiguous slices, one per wave.
//  * A wave walks its slice 16 rows at a time. Lane (h = lane/32, j =
//    lane%32) loads the 8x8 block rows k0+8h..+8, columns n0+8j..+8 of A_u
//    (32 lanes read 512 contiguous bytes of a row), transposes it in
//    registers, and issues 8 v_mfma_f32_32x32x16_bf16. Their B operand is
//    exactly that layout (lane l: column l%32, k-group l/32): MFMA c covers
//    the strided column set {n0 + 8j + c : j = 0..31}. X_u's fragment (row
//    lane%32, 8 consecutive k) is a 16-byte load that stays in L2.
//  * Rows come in blocks of 32 (the MFMA's rows): RB = 1 block for M <= 32,
//    2 for M <= 64, 8 MFMAs per block and step. Rows past M read as zero.
//    At M = 16 half of the matrix-core work is padding; at M = 64 the
//    matrix cores are still far from limiting (16 MFMAs per 8 KiB of A per
//    wave), so the kernel stays bound by HBM.
//  * The next step's 8 loads are in flight while a step's MFMAs run.
//  * The 4 wave partials are added in LDS in wave order (a fixed order, so
//    the result is deterministic), 32 rows per pass, and stored once.
//  * Fused reduction (sm_local_gemm_reduce_ws): the sum over the N ranks'
//    partials, Y = sum_i X_i A_i, runs in the same launch. Each workgroup
//    stores its partial block into the caller's workspace and counts itself
//    in at its (group, column block) counter; the workgroup that arrives
//    last adds the N partials of that block in rank order and writes the
//    finished rows, then returns the counter to zero. Arrival order never
//    changes the result: the sum is always ((P_0 + P_1) + ...) + P_{N-1}.
#include "device_math.h"
#include "kernels.h"

#include <algorithm>

namespace shardmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WAVES = 4;
constexpr int NT = 64 * WAVES;
constexpr int COLS = 256;  // output columns per workgroup
constexpr int KSTEP = 16;  // rows of A per MFMA step
// Output rows per reduction pass: one MFMA row block (32), or 16 when M <=
// 16, which halves the reduction buffer (64 KiB: two workgroups fit a CU).

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// A_u is read exactly once: non-temporal loads (plain loads of the same
// stream run at about half the rate).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 load16_guarded(const uint16_t* base, int64_t ld, int row, int col,
                                               int rows, int cols, bool vec) {
  if (row >= rows || col >= cols) return make_uint4(0u, 0u, 0u, 0u);
  const uint16_t* p = base + static_cast<int64_t>(row) * ld + col;
  if (vec && col + 8 <= cols) return load16(p);
  uint32_t e[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) e[k] = (col + k < cols) ? p[k] : 0u;
  return make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
}

__device__ __forceinline__ uint32_t word(const uint4& v, int d) {
  return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

__device__ __forceinline__ void transpose8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = j >> 1;
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    out[j] = make_uint4(__builtin_amdgcn_perm(word(in[1], d), word(in[0], d), sel),
                        __builtin_amdgcn_perm(word(in[3], d), word(in[2], d), sel),
                        __builtin_amdgcn_perm(word(in[5], d), word(in[4], d), sel),
                        __builtin_amdgcn_perm(word(in[7], d), word(in[6], d), sel));
  }
}


template <int RB>
struct StepRegs {
  uint4 x[RB];  // X fragments, one per 32-row block
  uint4 a[8];   // 8 rows x 8 columns of A
};

template <bool EDGE, int RB>
__device__ __forceinline__ void load_step(StepRegs<RB>& r, const uint16_t* X, int64_t ldx, const uint16_t* A,
                                          int64_t lda, int M, int K, int N, int k0, int n0, int h, int j,
                                          bool vec) {
  const int kx = k0 + 8 * h;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int row = 32 * b + j;
    if (EDGE || row >= M)
      r.x[b] = load16_guarded(X, ldx, row, kx, M, K, vec);
    else
      r.x[b] = load16(X + static_cast<int64_t>(row) * ldx + kx);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (EDGE)
      r.a[i] = load16_guarded(A, lda, kx + i, n0 + 8 * j, K, N, vec);
    else
      r.a[i] = load16_stream(A + static_cast<int64_t>(kx + i) * lda + n0 + 8 * j);
  }
}

// The workgroup that arrives last at its (group, column block) counter
// sums the group's N partials of that block in rank order, ((P_0 + P_1) +
// P_2) + ..., and writes the finished rows (split into the reduce-scatter
// owners' blocks when split_rows < M). Partials of other workgroups were
// written before their release fences; the caller issued the acquire.
__device__ __forceinline__ void finish_block(const SkinnyReduce& R, int group, int M, int N, int n0) {
  const int tid = threadIdx.x;
  const int nsum = R.n_partials;
  const float* base = R.part + static_cast<int64_t>(group) * nsum * R.part_stride;
  float* out = R.out[group];
  const int cols = min(COLS, N - n0);
  auto dst_of = [&](int row) -> float* {
    return out + (row / R.split_rows) * R.split_stride + static_cast<int64_t>(row % R.split_rows) * R.ldo;
  };
  if (R.vec_out) {
    // cols is a multiple of 4: N is, and n0 is a multiple of 256
    const int c4n = cols >> 2;
    const int total = M * c4n;
    constexpr int U = 4, YB = 8;  // one round of loads for 16 rows
    for (int q0 = tid; q0 < total; q0 += NT * U) {
      float4 acc[U];
      for (int y0 = 0; y0 < nsum; y0 += YB) {
        float4 v[YB][U];
#pragma unroll
        for (int i = 0; i < YB; ++i)
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int q = q0 + u * NT;
            if (y0 + i < nsum && q < total) {
              const int row = q / c4n, c = n0 + 4 * (q - row * c4n);
              v[i][u] = *reinterpret_cast<const float4*>(base + (y0 + i) * R.part_stride + row * R.ldp + c);
            }
          }
#pragma unroll
        for (int i = 0; i < YB; ++i)
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (y0 + i >= nsum) continue;
            if (y0 + i == 0) {
              acc[u] = v[i][u];
            } else {
              acc[u].x += v[i][u].x;
              acc[u].y += v[i][u].y;
              acc[u].z += v[i][u].z;
              acc[u].w += v[i][u].w;
            }
          }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u * NT;
        if (q < total) {
          const int row = q / c4n, c = n0 + 4 * (q - row * c4n);
          *reinterpret_cast<float4*>(dst_of(row) + c) = acc[u];
        }
      }
    }
  } else {
    for (int q = tid; q < M * cols; q += NT) {
      const int row = q / cols, c = n0 + (q - row * cols);
      const float* p = base + row * R.ldp + c;
      float sum = p[0];
      for (int y = 1; y < nsum; ++y) sum += p[y * R.part_stride];
      dst_of(row)[c] = sum;
    }
  }
}

template <bool EDGE, bool OUT_BF16, bool GELU, int RB, int PROWS, bool FUSED>
__global__ __launch_bounds__(NT) void gemm_skinny_kernel(const GemmLaunch L, const SkinnyReduce R) {
  __shared__ float red[WAVES][PROWS][COLS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, j = lane & 31;
  const int n0 = blockIdx.x * COLS;
  const GemmUnitPtrs U = L.u[blockIdx.y];
  const int M = L.M, N = L.N, K = L.K;

  // This wave's slice of whole 16-row steps.
  const int steps = (K + KSTEP - 1) / KSTEP;
  const int s_begin = (steps * wave) / WAVES;
  const int s_end = (steps * (wave + 1)) / WAVES;

  f32x16 acc[RB][8];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[b][c][v] = 0.f;

  // One set of load registers: once a step's block has been transposed into
  // the MFMA operands, the load registers take the next step's loads while
  // the MFMAs run.
  StepRegs<RB> r;
  if (s_begin < s_end) load_step<EDGE>(r, U.a, L.lda, U.b, L.ldb, M, K, N, s_begin * KSTEP, n0, h, j, L.vec_ok);
  for (int s = s_begin; s < s_end; ++s) {
    uint4 t[8];
    transpose8(r.a, t);
    bf16x8 xf[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) xf[b] = __builtin_bit_cast(bf16x8, r.x[b]);
    if (s + 1 < s_end) load_step<EDGE>(r, U.a, L.lda, U.b, L.ldb, M, K, N, (s + 1) * KSTEP, n0, h, j, L.vec_ok);
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[b][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[b], __builtin_bit_cast(bf16x8, t[c]), acc[b][c], 0, 0, 0);
  }

  // Output of MFMA (b, c), register v: row 32b + 8(v/4) + 4h + v%4, column
  // n0 + 8j + c. One reduction pass per row block, rows past M skipped.
  // Fused: the unit's partial goes to the workspace instead of the output.
  float* part = nullptr;
  if constexpr (FUSED) part = R.part + blockIdx.y * R.part_stride;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int rows = min(PROWS, M - 32 * b);
    if (b > 0) __syncthreads();  // the previous pass has read red
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < rows) red[wave][m][8 * j + c] = acc[b][c][v];
      }
    __syncthreads();
    for (int o = tid; o < rows * COLS; o += NT) {
      const int m = o / COLS, col = o % COLS;
      float sum = red[0][m][col];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][m][col];
      const int n = n0 + col;
      if (n < N) {
        if constexpr (FUSED) {
          // agent-scope stores write through to where every XCD reads
          // them, so the release below has no dirty partial lines to flush
          __hip_atomic_store(part + static_cast<int64_t>(32 * b + m) * R.ldp + n, sum, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        } else {
          if (GELU) sum = gelu_tanh_f32(sum);
          const int64_t off = static_cast<int64_t>(32 * b + m) * L.ldc + n;
          if (OUT_BF16)
            static_cast<uint16_t*>(U.c)[off] = bf16_rne(sum);
          else
            static_cast<float*>(U.c)[off] = sum;
        }
      }
    }
  }

  if constexpr (FUSED) {
    // Arrival: every wave's partial stores complete before the workgroup
    // barrier, and one thread counts the workgroup in with a vector atomic
    // that releases at device scope, so the whole workgroup's stores are
    // visible before the count. The last of the
    // N arrivals acquires (every thread) and finishes the block. No
    // workgroup ever waits for another. One device-scope release (an L2
    // write-back) per workgroup, not one per wave: on the [16, 28672] x
    // [28672, 8192] split over 8 ranks the launch took 94 us with one per
    // wave and 77 us like this (split-J kernel + separate reduce: 75 us).
    __shared__ int s_last;
    const int group = blockIdx.y / R.n_partials;
    uint32_t* counter = R.counters + group * R.n_colblk + blockIdx.x;
    // Each wave waits until its own device-scope partial stores have
    // completed. The device-scope release below waits only for the
    // releasing wave's memory operations, and a CU keeps a separate request
    // queue per L2 channel, so another wave's stores still in flight could
    // otherwise reach their channels after the count. (The "memory" clobber
    // keeps the compiler from moving the stores below the wait.)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (tid == 0) {
      const uint32_t before = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      const int last = before == static_cast<uint32_t>(R.n_partials - 1);
      // every arrival of this launch has happened: the counter goes back to
      // zero for the next call
      if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    finish_block(R, group, M, N, n0);
  }
}

__global__ __launch_bounds__(NT) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(NT) + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * NT)
    p[i] = 0u;
}

template <bool OUT_BF16, bool GELU, int RB, int PROWS, bool FUSED>
hipError_t launch_rb(const GemmLaunch& L, const SkinnyReduce& R, hipStream_t s) {
  const bool edge = (L.N % COLS) != 0 || (L.K % KSTEP) != 0 || !L.vec_ok;
  dim3 grid((L.N + COLS - 1) / COLS, L.n_units);
  if (edge)
    hipLaunchKernelGGL((gemm_skinny_kernel<true, OUT_BF16, GELU, RB, PROWS, FUSED>), grid, dim3(NT), 0, s, L, R);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<false, OUT_BF16, GELU, RB, PROWS, FUSED>), grid, dim3(NT), 0, s, L, R);
  return hipGetLastError();
}

template <bool OUT_BF16, bool GELU, bool FUSED>
hipError_t launch_variant(const GemmLaunch& L, const SkinnyReduce& R, hipStream_t s) {
  if (L.M <= 16) return launch_rb<OUT_BF16, GELU, 1, 16, FUSED>(L, R, s);
  if (L.M <= 32) return launch_rb<OUT_BF16, GELU, 1, 32, FUSED>(L, R, s);
  return launch_rb<OUT_BF16, GELU, 2, 32, FUSED>(L, R, s);
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmLaunch& L, hipStream_t s) {
  SkinnyReduce none{};
  if (L.out_bf16)
    return L.epilogue == kEpiGelu ? launch_variant<true, true, false>(L, none, s)
                                  : launch_variant<true, false, false>(L, none, s);
  return L.epilogue == kEpiGelu ? launch_variant<false, true, false>(L, none, s)
                                : launch_variant<false, false, false>(L, none, s);
}

hipError_t launch_gemm_skinny_reduce(const GemmLaunch& L, const SkinnyReduce& R, hipStream_t s) {
  return launch_variant<false, false, true>(L, R, s);
}

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t s) {
  const int64_t blocks = std::min<int64_t>((n + NT - 1) / NT, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>(std::max<int64_t>(blocks, 1))), dim3(NT), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace shardmm
