// Streaming row kernel behind sm_reduce_partials and sm_gather_shards.
//
//  * Reduce (n_sum = N >= 2, float32): dst[r, c] = (((P_0 + P_1) + P_2) ...)
//    [r, c], the partials added in rank order -- the addition of
//    contributions with matching output coordinates that finishes a case-3
//    product (semiaifoundry.com "The mechanism", step 4; learntpu.dev ch05,
//    AllReduce / ReduceScatter rows of the collectives table). With all
//    ranks on one GPU the "collective" is this HBM-bound pass.
//  * Copy (n_sum = 1): all-gather of finished blocks into the global layout.
//
// Design (gfx950): pure streaming. Each workgroup owns one row (or one
// column chunk of a row, when a launch has few rows) of one job; its 256
// threads walk it in 16-byte vectors, four vectors per thread
// per iteration, and issue every partial's loads before the rank-ordered
// adds so that 4 x N loads per thread are in flight. Loads are
// non-temporal (nothing is re-read, so the data should not displace L2);
// stores are plain, which the HBM writes back at a higher rate.
#include "kernels.h"

namespace shardmm {
namespace {

constexpr int NT = 256;
constexpr int UNROLL = 4;

__device__ __forceinline__ float4 ldnt(const float4* p) {
  float4 v;
  v.x = __builtin_nontemporal_load(&p->x);
  v.y = __builtin_nontemporal_load(&p->y);
  v.z = __builtin_nontemporal_load(&p->z);
  v.w = __builtin_nontemporal_load(&p->w);
  return v;
}

__device__ __forceinline__ void stnt(float4* p, const float4& v) {
  __builtin_nontemporal_store(v.x, &p->x);
  __builtin_nontemporal_store(v.y, &p->y);
  __builtin_nontemporal_store(v.z, &p->z);
  __builtin_nontemporal_store(v.w, &p->w);
}

__device__ __forceinline__ void add4(float4& a, const float4& b) {
  a.x += b.x;
  a.y += b.y;
  a.z += b.z;
  a.w += b.w;
}

__device__ __forceinline__ float4 ld4(const float4* p) { return *p; }
__device__ __forceinline__ void st4(float4* p, const float4& v) { *p = v; }

// Rank-ordered sum of NS partials (NS > 0 fixed at compile time, or the
// runtime count when NS == 0) for one row, float4 path. Sums use
// non-temporal loads (+40 % over plain ones) and plain stores; a plain copy
// (NS == 1) measured 5 % faster with plain loads on 8 KiB rows.
template <int NS>
__device__ __forceinline__ void sum_row_vec(const RowJob& J, int n_sum, int row) {
  constexpr bool kNT = NS != 1;
  const int nsum = NS > 0 ? NS : n_sum;
  const float* src = static_cast<const float*>(J.src) + static_cast<int64_t>(row) * J.lds;
  float* dst = static_cast<float*>(J.dst) + static_cast<int64_t>(row) * J.ldd;
  const int n4 = J.cols >> 2;
  for (int base = threadIdx.x; base < n4; base += NT * UNROLL) {
    float4 acc[UNROLL];
    if (NS > 0) {
      float4 v[NS > 0 ? NS : 1][UNROLL];
#pragma unroll
      for (int y = 0; y < (NS > 0 ? NS : 1); ++y)
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int c4 = base + u * NT;
          if (c4 < n4) {
            const float4* q = reinterpret_cast<const float4*>(src + y * J.src_stride) + c4;
            v[y][u] = kNT ? ldnt(q) : ld4(q);
          }
        }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        acc[u] = v[0][u];
#pragma unroll
        for (int y = 1; y < (NS > 0 ? NS : 1); ++y) add4(acc[u], v[y][u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int c4 = base + u * NT;
        if (c4 < n4) acc[u] = ldnt(reinterpret_cast<const float4*>(src) + c4);
      }
      for (int y = 1; y < nsum; ++y) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int c4 = base + u * NT;
          if (c4 < n4) add4(acc[u], ldnt(reinterpret_cast<const float4*>(src + y * J.src_stride) + c4));
        }
      }
    }
    // plain stores for sums and copies alike: on the down-projection's
    // reduce-scatter (805 MB) they ran at 6.68 TB/s against 6.36 with
    // non-temporal stores (a lab stream of 2 non-temporal reads + 1 write:
    // 6.81 vs 6.12 TB/s; a plain write stream alone: 6.97 vs 5.85 TB/s)
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int c4 = base + u * NT;
      if (c4 < n4) st4(reinterpret_cast<float4*>(dst) + c4, acc[u]);
    }
  }
}

__device__ __forceinline__ void sum_row_scalar(const RowJob& J, int n_sum, int row) {
  const float* src = static_cast<const float*>(J.src) + static_cast<int64_t>(row) * J.lds;
  float* dst = static_cast<float*>(J.dst) + static_cast<int64_t>(row) * J.ldd;
  for (int c = threadIdx.x; c < J.cols; c += NT) {
    float s = src[c];
    for (int y = 1; y < n_sum; ++y) s += src[y * J.src_stride + c];
    dst[c] = s;
  }
}

__device__ __forceinline__ void copy_row_16(const RowJob& J, int row) {
  // 16-bit elements; 8 per 16-byte vector (alignment checked by the host).
  const uint16_t* src = static_cast<const uint16_t*>(J.src) + static_cast<int64_t>(row) * J.lds;
  uint16_t* dst = static_cast<uint16_t*>(J.dst) + static_cast<int64_t>(row) * J.ldd;
  const int n8 = J.cols >> 3;
  for (int c = threadIdx.x; c < n8; c += NT)
    reinterpret_cast<uint4*>(dst)[c] = reinterpret_cast<const uint4*>(src)[c];
}

__device__ __forceinline__ void copy_row_16_scalar(const RowJob& J, int row) {
  const uint16_t* src = static_cast<const uint16_t*>(J.src) + static_cast<int64_t>(row) * J.lds;
  uint16_t* dst = static_cast<uint16_t*>(J.dst) + static_cast<int64_t>(row) * J.ldd;
  for (int c = threadIdx.x; c < J.cols; c += NT) dst[c] = src[c];
}

// Workgroup -> (job, row, column chunk). Jobs with few rows are split into
// column chunks so that small reductions still spread over many CUs.
__device__ __forceinline__ bool job_slice(const RowLaunch& L, RowJob& J, int& row) {
  J = L.jobs[blockIdx.y];
  row = blockIdx.x / L.n_chunks;
  const int c0 = (blockIdx.x - row * L.n_chunks) * L.chunk;
  if (row >= J.rows || c0 >= J.cols) return false;
  const int64_t off = static_cast<int64_t>(c0) * L.elem_bytes;
  J.src = static_cast<const char*>(J.src) + off;
  J.dst = static_cast<char*>(J.dst) + off;
  J.cols = min(J.cols - c0, L.chunk);
  return true;
}

template <int NS>
__global__ __launch_bounds__(NT) void rows_f32_kernel(const RowLaunch L) {
  RowJob J;
  int row;
  if (!job_slice(L, J, row)) return;
  if (J.vec)
    sum_row_vec<NS>(J, L.n_sum, row);
  else
    sum_row_scalar(J, L.n_sum, row);
}

__global__ __launch_bounds__(NT) void rows_b16_copy_kernel(const RowLaunch L) {
  RowJob J;
  int row;
  if (!job_slice(L, J, row)) return;
  if (J.vec)
    copy_row_16(J, row);
  else
    copy_row_16_scalar(J, row);
}

// Copy of short rows (at most 4 KiB each): one workgroup per tile of
// L.tile_rows consecutive rows of a job, walked as one flat sequence of
// 16-byte vectors; each thread issues all of its CU loads (non-temporal)
// before its stores. With one 2 KiB row per workgroup half the threads
// idle and the launch needs 8x as many workgroups: a bf16 gather of
// [4096,1024] column blocks measured 11.9 us against 12.8 us, from HBM.
constexpr int CU = 8;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <int ESZ>
__global__ __launch_bounds__(NT) void rows_copy_tiled_kernel(const RowLaunch L) {
  const RowJob J = L.jobs[blockIdx.y];
  const int r0 = blockIdx.x * L.tile_rows;
  if (r0 >= J.rows) return;
  const int rows = min(L.tile_rows, J.rows - r0);
  const char* src = static_cast<const char*>(J.src) + static_cast<int64_t>(r0) * J.lds * ESZ;
  char* dst = static_cast<char*>(J.dst) + static_cast<int64_t>(r0) * J.ldd * ESZ;
  if (!J.vec) {
    for (int r = 0; r < rows; ++r)
      for (int c = threadIdx.x; c < J.cols; c += NT) {
        const int64_t so = (static_cast<int64_t>(r) * J.lds + c) * ESZ, d = (static_cast<int64_t>(r) * J.ldd + c) * ESZ;
        if (ESZ == 2)
          *reinterpret_cast<uint16_t*>(dst + d) = *reinterpret_cast<const uint16_t*>(src + so);
        else
          *reinterpret_cast<uint32_t*>(dst + d) = *reinterpret_cast<const uint32_t*>(src + so);
      }
    return;
  }
  const int nv = J.cols * ESZ / 16;  // vectors per row
  const int total = rows * nv;
  for (int base = 0; base < total; base += NT * CU) {
    u32x4_t v[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int i = base + threadIdx.x + u * NT;
      if (i < total) {
        const int r = i / nv, c = i - r * nv;
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + static_cast<int64_t>(r) * J.lds * ESZ) + c);
      }
    }
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int i = base + threadIdx.x + u * NT;
      if (i < total) {
        const int r = i / nv, c = i - r * nv;
        __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(dst + static_cast<int64_t>(r) * J.ldd * ESZ) + c);
      }
    }
  }
}

// Sum of one float per thread over the workgroup, in a fixed order (wave
// butterflies, then the 4 wave totals in wave order): deterministic.
__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) t += red[w];
  return t;
}

// Rank-ordered sum of the partials of one row, then layer norm of the row:
// y = (x - mean) / sqrt(var + eps) * gamma + beta (biased variance). The
// whole row stays in registers: V float4 per thread (n <= 1024 V).
template <int NS, int V>
__global__ __launch_bounds__(NT) void rows_layernorm_kernel(const RowLaunch L, const float* __restrict__ gamma,
                                                            const float* __restrict__ beta, float eps) {
  __shared__ float red[NT / 64];
  const RowJob& J = L.jobs[blockIdx.y];
  const int row = blockIdx.x;
  if (row >= J.rows) return;
  const int nsum = NS > 0 ? NS : L.n_sum;
  const float* src = static_cast<const float*>(J.src) + static_cast<int64_t>(row) * J.lds;
  float* dst = static_cast<float*>(J.dst) + static_cast<int64_t>(row) * J.ldd;
  const int n4 = J.cols >> 2;
  float4 v[V];
  float s = 0.f;
  // Few partials and short rows (NS * V <= 16 vectors per thread): every
  // load of the row is issued before the rank-ordered adds, so they are all
  // in flight together. Otherwise partials are added as they arrive.
  constexpr bool kAllFirst = NS > 0 && NS * V <= 16;
  if constexpr (kAllFirst) {
    float4 t[kAllFirst ? NS : 1][V];
#pragma unroll
    for (int y = 0; y < NS; ++y)
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int c4 = threadIdx.x + i * NT;
        t[y][i] = c4 < n4 ? ldnt(reinterpret_cast<const float4*>(src + y * J.src_stride) + c4)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int i = 0; i < V; ++i) {
      v[i] = t[0][i];
#pragma unroll
      for (int y = 1; y < NS; ++y) add4(v[i], t[y][i]);
      s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int c4 = threadIdx.x + i * NT;
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c4 < n4) {
        v[i] = ldnt(reinterpret_cast<const float4*>(src) + c4);
        for (int y = 1; y < nsum; ++y) add4(v[i], ldnt(reinterpret_cast<const float4*>(src + y * J.src_stride) + c4));
        s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
      }
    }
  }
  const float inv_n = 1.0f / static_cast<float>(J.cols);
  const float mean = block_sum(s, red) * inv_n;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int c4 = threadIdx.x + i * NT;
    if (c4 < n4) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      q += (a * a + b * b) + (c * c + d * d);
    }
  }
  const float var = block_sum(q, red) * inv_n;
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int c4 = threadIdx.x + i * NT;
    if (c4 < n4) {
      float4 g = make_float4(1.f, 1.f, 1.f, 1.f), b = make_float4(0.f, 0.f, 0.f, 0.f);
      if (gamma) g = reinterpret_cast<const float4*>(gamma)[c4];
      if (beta) b = reinterpret_cast<const float4*>(beta)[c4];
      float4 o;
      o.x = (v[i].x - mean) * rstd * g.x + b.x;
      o.y = (v[i].y - mean) * rstd * g.y + b.y;
      o.z = (v[i].z - mean) * rstd * g.z + b.z;
      o.w = (v[i].w - mean) * rstd * g.w + b.w;
      stnt(reinterpret_cast<float4*>(dst) + c4, o);
    }
  }
}

template <int V>
void launch_ln_v(const RowLaunch& L, const float* gamma, const float* beta, float eps, hipStream_t s) {
  dim3 grid(L.max_rows, L.n_jobs);
  switch (L.n_sum) {
    case 1: hipLaunchKernelGGL((rows_layernorm_kernel<1, V>), grid, dim3(NT), 0, s, L, gamma, beta, eps); break;
    case 2: hipLaunchKernelGGL((rows_layernorm_kernel<2, V>), grid, dim3(NT), 0, s, L, gamma, beta, eps); break;
    case 4: hipLaunchKernelGGL((rows_layernorm_kernel<4, V>), grid, dim3(NT), 0, s, L, gamma, beta, eps); break;
    case 8: hipLaunchKernelGGL((rows_layernorm_kernel<8, V>), grid, dim3(NT), 0, s, L, gamma, beta, eps); break;
    default: hipLaunchKernelGGL((rows_layernorm_kernel<0, V>), grid, dim3(NT), 0, s, L, gamma, beta, eps); break;
  }
}

}  // namespace

hipError_t launch_rows_layernorm(const RowLaunch& L, const float* gamma, const float* beta, float eps,
                                 hipStream_t s) {
  if (L.n_jobs <= 0 || L.max_rows <= 0) return hipSuccess;
  int max_cols = 0;
  for (int i = 0; i < L.n_jobs; ++i) max_cols = max(max_cols, L.jobs[i].cols);
  const int per = (max_cols / 4 + NT - 1) / NT;  // float4 per thread
  if (per <= 1) launch_ln_v<1>(L, gamma, beta, eps, s);
  else if (per <= 2) launch_ln_v<2>(L, gamma, beta, eps, s);
  else if (per <= 4) launch_ln_v<4>(L, gamma, beta, eps, s);
  else if (per <= 8) launch_ln_v<8>(L, gamma, beta, eps, s);
  else if (per <= 16) launch_ln_v<16>(L, gamma, beta, eps, s);
  else if (per <= 32) launch_ln_v<32>(L, gamma, beta, eps, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_rows(const RowLaunch& L, hipStream_t s) {
  if (L.n_jobs <= 0 || L.max_rows <= 0 || L.n_chunks <= 0) return hipSuccess;
  if (L.n_sum == 1 && L.tile_rows > 1 && L.n_chunks == 1) {
    dim3 grid((L.max_rows + L.tile_rows - 1) / L.tile_rows, L.n_jobs);
    if (L.elem_bytes == 2)
      hipLaunchKernelGGL(rows_copy_tiled_kernel<2>, grid, dim3(NT), 0, s, L);
    else
      hipLaunchKernelGGL(rows_copy_tiled_kernel<4>, grid, dim3(NT), 0, s, L);
    return hipGetLastError();
  }
  dim3 grid(L.max_rows * L.n_chunks, L.n_jobs);
  if (L.elem_bytes == 2) {
    hipLaunchKernelGGL(rows_b16_copy_kernel, grid, dim3(NT), 0, s, L);
  } else {
    switch (L.n_sum) {
      case 1: hipLaunchKernelGGL(rows_f32_kernel<1>, grid, dim3(NT), 0, s, L); break;
      case 2: hipLaunchKernelGGL(rows_f32_kernel<2>, grid, dim3(NT), 0, s, L); break;
      case 4: hipLaunchKernelGGL(rows_f32_kernel<4>, grid, dim3(NT), 0, s, L); break;
      case 8: hipLaunchKernelGGL(rows_f32_kernel<8>, grid, dim3(NT), 0, s, L); break;
      default: hipLaunchKernelGGL(rows_f32_kernel<0>, grid, dim3(NT), 0, s, L); break;
    }
  }
  return hipGetLastError();
}

}  // namespace shardmm
