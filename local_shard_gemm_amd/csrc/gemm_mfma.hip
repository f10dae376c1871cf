// Batched bfloat16 GEMM for gfx950 matrix cores: C_u = A_u . B_u for a
// batch of units (one logical rank's local product each), fp32 accumulate.
//
// The local matmul each rank runs after sharding (learntpu.dev ch05,
// sharding sandbox "Local matmul"; lingze.zone "Case 1" and "Case 3").
//
// Design (gfx950, wave64):
//  * 256x256 output tile per workgroup of 4 waves (2x2); each wave owns a
//    128x128 sub-tile = 4x4 MFMA blocks of v_mfma_f32_32x32x16_bf16, i.e.
//    256 fp32 accumulators per lane.
//  * K advances 64 at a time through two LDS buffers (2 x 64 KiB): the
//    next slice is fetched from HBM into registers while the current one
//    feeds the matrix cores, then written to the other buffer; one barrier
//    per slice.
//  * A is row-major [M,K] (K contiguous): 16-byte chunks go to LDS as is.
//    B is row-major [K,N] (N contiguous) but the MFMA wants 8 consecutive
//    k per lane: each thread loads an 8(k) x 8(n) block and transposes it
//    in registers (v_perm_b32) before the 16-byte LDS stores.
//  * LDS rows are 64 bf16 = 8 chunks of 16 bytes; chunk c of row r is stored
//    at c ^ ((r ^ r>>3) & 7), which keeps both the row-wise stores and the
//    MFMA fragment reads (8 consecutive rows, same chunk) free of bank
//    conflicts.
//  * Tile order: groups of 16 tile rows, column-major inside a group, and
//    inside every full chunk of 256 workgroups an XCD-aware permutation
//    that gives each of the 8 XCDs (workgroup id mod 8) a 4x8 block of
//    tiles, so the 32 CUs of an XCD share A rows and B columns in their L2
//    and the 8 XCDs together cover a 16x16 block through the MALL.
//  * Units that share a B block are listed next to each other by the host,
//    so their tiles stack into one tall virtual matrix.
#include "kernels.h"

namespace shardmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = kTileM, BN = kTileN, BK = kTileK;
constexpr int NT = 256;
constexpr int CH = BK / 8;  // 16-byte chunks per LDS row

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Eight consecutive elements of row `row` from column `col` of a rows x cols
// view; zero outside the view (edge tiles and ragged K).
// vec: the view is 16-byte aligned, so whole chunks may use one vector load.
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

// 8x8 transpose of 16-bit elements held as 8 rows of 16 bytes.
// out[j] holds column j: element i of out[j] = element j of in[i].
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

// float -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Workgroup id -> (virtual tile row, tile column). A bijection on [0, T).
__device__ __forceinline__ void tile_of(int w, int T, int VR, int VC, int* vr, int* vc) {
  int t = w;
  const int chunk = w >> 8;
  if ((chunk + 1) * 256 <= T) {
    const int xcd = w & 7, q = (w & 255) >> 3;
    const int r16 = (xcd & 3) * 4 + (q & 3);
    const int c16 = (xcd >> 2) * 8 + (q >> 2);
    t = (chunk << 8) + c16 * 16 + r16;
  }
  constexpr int GM = 16;
  const int group = t / (GM * VC);
  const int first = group * GM;
  const int rows = min(GM, VR - first);
  const int idx = t - group * GM * VC;
  *vr = first + idx % rows;
  *vc = idx / rows;
}

template <bool OUT_BF16, bool GELU, bool EDGE>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], void* C, int64_t ldc, int row0,
                                           int col0, int M, int N) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int rsub = 4 * (lane >> 5), csub = lane & 31;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = row0 + wm * 128 + mi * 32 + 8 * (v >> 2) + rsub + (v & 3);
        const int c = col0 + wn * 128 + ni * 32 + csub;
        if (EDGE && (r >= M || c >= N)) continue;
        float x = acc[mi][ni][v];
        if (GELU) x = gelu_tanh_f32(x);
        const int64_t off = static_cast<int64_t>(r) * ldc + c;
        if (OUT_BF16)
          static_cast<uint16_t*>(C)[off] = bf16_rne(x);
        else
          static_cast<float*>(C)[off] = x;
      }
}

template <bool EDGE, bool OUT_BF16, bool GELU>
__device__ __forceinline__ void run_tile(const GemmLaunch& L, const uint16_t* __restrict__ A,
                                         const uint16_t* __restrict__ B, void* C, int row0, int col0,
                                         uint4* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int M = L.M, N = L.N, K = L.K;
  const int64_t lda = L.lda, ldb = L.ldb;
  const int a_c = tid & 7, a_r = tid >> 3;   // A: chunk 0..7, row 0..31 (+32 i)
  const int b_n = tid & 31, b_k = tid >> 5;  // B: n chunk 0..31, k group 0..7
  const uint16_t* a_base = A + static_cast<int64_t>(row0 + a_r) * lda + 8 * a_c;
  const uint16_t* b_base = B + static_cast<int64_t>(8 * b_k) * ldb + col0 + 8 * b_n;

  uint4 ra[8], rb[8];
  f32x16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  const int nk = (K + BK - 1) / BK;

  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (EDGE)
        ra[i] = load16_guarded(A, lda, row0 + a_r + 32 * i, k0 + 8 * a_c, M, K, L.vec_ok);
      else
        ra[i] = load16(a_base + static_cast<int64_t>(32 * i) * lda + k0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (EDGE)
        rb[i] = load16_guarded(B, ldb, k0 + 8 * b_k + i, col0 + 8 * b_n, K, N, L.vec_ok);
      else
        rb[i] = load16(b_base + static_cast<int64_t>(k0 + i) * ldb);
    }
  };
  auto sstore = [&](int buf) {
    uint4* la = lds + buf * (2 * BM * CH);
    uint4* lb = la + BM * CH;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = a_r + 32 * i;
      la[r * CH + (a_c ^ swz(r))] = ra[i];
    }
    uint4 tb[8];
    transpose8(rb, tb);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = 8 * b_n + j;
      lb[n * CH + (b_k ^ swz(n))] = tb[j];
    }
  };
  auto compute = [&](int buf) {
    const uint4* la = lds + buf * (2 * BM * CH);
    const uint4* lb = la + BM * CH;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int ch = 2 * s + (lane >> 5);
      bf16x8 af[4], bfv[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 128 + mi * 32 + (lane & 31);
        af[mi] = __builtin_bit_cast(bf16x8, la[r * CH + (ch ^ swz(r))]);
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int n = wn * 128 + ni * 32 + (lane & 31);
        bfv[ni] = __builtin_bit_cast(bf16x8, lb[n * CH + (ch ^ swz(n))]);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfv[ni], acc[mi][ni], 0, 0, 0);
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    compute(cur);
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  store_tile<OUT_BF16, GELU, EDGE>(acc, C, L.ldc, row0, col0, M, N);
}

// Interior tiles: every tile of the launch is a full BM x BN tile and K is a
// multiple of BK, so no load or store needs a bounds check.
template <bool OUT_BF16, bool GELU>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_mfma_kernel(const GemmLaunch L) {
  __shared__ uint4 lds[2 * 2 * BM * CH];
  const int full_m = L.M / BM, full_n = L.N / BN;
  const int VR = L.n_units * full_m;
  const int T = VR * full_n;
  int vr, vc;
  tile_of(blockIdx.x, T, VR, full_n, &vr, &vc);
  const int unit = vr / full_m;
  const int row0 = (vr - unit * full_m) * BM;
  const int col0 = vc * BN;
  const GemmUnitPtrs U = L.u[unit];
  run_tile<false, OUT_BF16, GELU>(L, U.a, U.b, U.c, row0, col0, lds);
}

// Edge tiles: the last tile row (M % BM), the last tile column (N % BN), or
// every tile when K % BK != 0 or a view is not 16-byte aligned. Loads
// outside the views read as zero and stores outside them are skipped.
// blockIdx.y = unit.
template <bool OUT_BF16, bool GELU>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_mfma_edge_kernel(const GemmLaunch L) {
  __shared__ uint4 lds[2 * 2 * BM * CH];
  const int unit = blockIdx.y;
  int tm, tn;
  if ((L.K % BK) || !L.vec_ok) {
    tm = blockIdx.x / L.tiles_n;
    tn = blockIdx.x % L.tiles_n;
  } else {
    const int e_rows = (L.M % BM) ? 1 : 0;
    const int t = blockIdx.x;
    if (t < e_rows * L.tiles_n) {
      tm = L.tiles_m - 1;
      tn = t;
    } else {
      tm = t - e_rows * L.tiles_n;
      tn = L.tiles_n - 1;
    }
  }
  const GemmUnitPtrs U = L.u[unit];
  run_tile<true, OUT_BF16, GELU>(L, U.a, U.b, U.c, tm * BM, tn * BN, lds);
}

template <bool OUT_BF16, bool GELU>
hipError_t launch_variant(const GemmLaunch& L, hipStream_t s) {
  const int full_m = L.M / BM, full_n = L.N / BN;
  const bool k_ragged = (L.K % BK) != 0 || !L.vec_ok;
  if (!k_ragged && full_m > 0 && full_n > 0) {
    const int T = L.n_units * full_m * full_n;
    hipLaunchKernelGGL((gemm_bf16_mfma_kernel<OUT_BF16, GELU>), dim3(T), dim3(NT), 0, s, L);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int n_edge;
  if (k_ragged) {
    n_edge = L.tiles_m * L.tiles_n;
  } else {
    const int e_rows = (L.M % BM) ? 1 : 0, e_cols = (L.N % BN) ? 1 : 0;
    n_edge = e_rows * L.tiles_n + e_cols * (L.tiles_m - e_rows);
  }
  if (n_edge > 0) {
    hipLaunchKernelGGL((gemm_bf16_mfma_edge_kernel<OUT_BF16, GELU>), dim3(n_edge, L.n_units), dim3(NT), 0, s, L);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemm_mfma(const GemmLaunch& L, hipStream_t s) {
  if (L.out_bf16)
    return L.epilogue == kEpiGelu ? launch_variant<true, true>(L, s) : launch_variant<true, false>(L, s);
  return L.epilogue == kEpiGelu ? launch_variant<false, true>(L, s) : launch_variant<false, false>(L, s);
}

}  // namespace shardmm
