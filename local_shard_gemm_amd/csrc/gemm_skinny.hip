// Split-J kernel for skinny local products (M <= 16 rows): each rank's
// partial P_u = X_u . A_u with X_u [M, K] small and A_u [K, N] streamed
// once from HBM. Used for the row-parallel step Z_i = X_i A_i with a small
// batch (mbrenndoerfer.com "Row Parallelism": Z_i = X_i A_i; the partials
// have the full output shape and are summed afterwards).
//
// Design (gfx950): the work is bound by HBM reads of A_u, so the kernel is
// shaped for bytes in flight, not for matrix-core throughput.
//  * One workgroup = 8 waves = one unit and 128 output columns; the unit's
//    K range is split into 8 contiguous slices, one per wave.
//  * A wave walks its slice 32 rows at a time. Lane (g = lane/16, j =
//    lane%16) loads the 8x8 block rows k0+8g..+8, columns n0+8j..+8 of A_u
//    (16 lanes read 256 contiguous bytes of a row), transposes it in
//    registers, and issues 8 v_mfma_f32_16x16x32_bf16: MFMA c covers the
//    strided column set {n0 + 8j + c : j = 0..15}. X_u's fragment (row
//    lane%16, 8 consecutive k) is a 16-byte load that stays in L2.
//  * The next step's 8 loads are in flight while a step's MFMAs run; at
//    most 128 VGPRs, so two workgroups (16 waves) share a CU.
//  * The 8 wave partials are added in LDS in wave order (a fixed order, so
//    the result is deterministic) and stored once.
#include "kernels.h"

namespace shardmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = 8;
constexpr int NT = 64 * WAVES;
constexpr int COLS = 128;  // output columns per workgroup
constexpr int KSTEP = 32;  // rows of A per MFMA step

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// A_u is read exactly once: non-temporal loads (measured on this access
// pattern: 5.4 -> 6.2 TB/s).
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

// GeLU, tanh form: 0.5 x (1 + tanh(z)), z = sqrt(2/pi) (x + 0.044715 x^3),
// evaluated as x / (1 + exp(-2 z)) -- the same function (1 + tanh(z) =
// 2 / (1 + exp(-2z))) without the float32 cancellation of 1 + tanh(z) for
// negative z.
__device__ __forceinline__ float gelu_tanh_f32(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  const float z = k0 * (x + k1 * x * x * x);
  return x / (1.0f + expf(-2.0f * z));
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

struct StepRegs {
  uint4 x;      // X fragment
  uint4 a[8];   // 8 rows x 8 columns of A
};

template <bool EDGE>
__device__ __forceinline__ void load_step(StepRegs& r, const uint16_t* X, int64_t ldx, const uint16_t* A,
                                          int64_t lda, int M, int K, int N, int k0, int n0, int g, int j,
                                          bool vec) {
  const int kx = k0 + 8 * g;
  if (EDGE || j >= M)
    r.x = load16_guarded(X, ldx, j, kx, M, K, vec);
  else
    r.x = load16(X + static_cast<int64_t>(j) * ldx + kx);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (EDGE)
      r.a[i] = load16_guarded(A, lda, kx + i, n0 + 8 * j, K, N, vec);
    else
      r.a[i] = load16_stream(A + static_cast<int64_t>(kx + i) * lda + n0 + 8 * j);
  }
}

template <bool EDGE, bool OUT_BF16, bool GELU>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 4))) void gemm_skinny_kernel(const GemmLaunch L) {
  __shared__ float red[WAVES][16][COLS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int n0 = blockIdx.x * COLS;
  const GemmUnitPtrs U = L.u[blockIdx.y];
  const int M = L.M, N = L.N, K = L.K;

  // This wave's slice of whole 32-row steps.
  const int steps = (K + KSTEP - 1) / KSTEP;
  const int s_begin = (steps * wave) / WAVES;
  const int s_end = (steps * (wave + 1)) / WAVES;

  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One set of load registers: once a step's block has been transposed into
  // the MFMA operands, the load registers take the next step's loads while
  // the 8 MFMAs run.
  StepRegs r;
  if (s_begin < s_end) load_step<EDGE>(r, U.a, L.lda, U.b, L.ldb, M, K, N, s_begin * KSTEP, n0, g, j, L.vec_ok);
  for (int s = s_begin; s < s_end; ++s) {
    uint4 t[8];
    transpose8(r.a, t);
    const bf16x8 xf = __builtin_bit_cast(bf16x8, r.x);
    if (s + 1 < s_end) load_step<EDGE>(r, U.a, L.lda, U.b, L.ldb, M, K, N, (s + 1) * KSTEP, n0, g, j, L.vec_ok);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf, __builtin_bit_cast(bf16x8, t[c]), acc[c], 0, 0, 0);
  }

  // Output of MFMA c, register v: row 4g + v, column n0 + 8j + c.
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * g + v][8 * j + c] = acc[c][v];
  __syncthreads();

  for (int o = tid; o < 16 * COLS; o += NT) {
    const int m = o / COLS, col = o % COLS;
    float sum = red[0][m][col];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[w][m][col];
    const int n = n0 + col;
    if (m < M && n < N) {
      if (GELU) sum = gelu_tanh_f32(sum);
      const int64_t off = static_cast<int64_t>(m) * L.ldc + n;
      if (OUT_BF16)
        static_cast<uint16_t*>(U.c)[off] = bf16_rne(sum);
      else
        static_cast<float*>(U.c)[off] = sum;
    }
  }
}

template <bool OUT_BF16, bool GELU>
hipError_t launch_variant(const GemmLaunch& L, hipStream_t s) {
  const bool edge = (L.N % COLS) != 0 || (L.K % KSTEP) != 0 || !L.vec_ok;
  dim3 grid((L.N + COLS - 1) / COLS, L.n_units);
  if (edge)
    hipLaunchKernelGGL((gemm_skinny_kernel<true, OUT_BF16, GELU>), grid, dim3(NT), 0, s, L);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<false, OUT_BF16, GELU>), grid, dim3(NT), 0, s, L);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmLaunch& L, hipStream_t s) {
  if (L.out_bf16)
    return L.epilogue == kEpiGelu ? launch_variant<true, true>(L, s) : launch_variant<true, false>(L, s);
  return L.epilogue == kEpiGelu ? launch_variant<false, true>(L, s) : launch_variant<false, false>(L, s);
}

}  // namespace shardmm
