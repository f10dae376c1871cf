// Batched bfloat16 GEMM for gfx950 matrix cores: C_u = A_u . B_u for a
// batch of units (one logical rank's local product each), fp32 accumulate.
//
// The local matmul each rank runs after sharding (learntpu.dev ch05,
// sharding sandbox "Local matmul"; lingze.zone "Case 1" and "Case 3").
//
// Two kernels share the 256x256 output tile per workgroup of 4 waves (2x2),
// each wave owning a 128x128 sub-tile (256 fp32 accumulators per lane):
//  * gemm_bf16_mfma_kernel (every tile when the views are 16-byte aligned):
//    8x8 blocks of v_mfma_f32_16x16x32_bf16, direct HBM -> LDS buffer loads,
//    transposing LDS reads, a 5-stage LDS ring and two register fragment
//    sets; described above run_tile_lds.
//  * gemm_bf16_mfma_edge_kernel (unaligned views): 4x4 blocks of
//    v_mfma_f32_32x32x16_bf16, guarded loads through registers, described
//    here.
//
// Edge-tile design:
//  * K advances 64 at a time through two LDS buffers (2 x 64 KiB): the
//    next slice is fetched into registers while the current one feeds the
//    matrix cores, then written to the other buffer; one barrier per slice.
//  * A is row-major [M,K] (K contiguous): 16-byte chunks go to LDS as is.
//    B is row-major [K,N] (N contiguous) but the MFMA wants 8 consecutive
//    k per lane: each thread loads an 8(k) x 8(n) block and transposes it
//    in registers (v_perm_b32) before the 16-byte LDS stores.
//  * LDS rows are 64 bf16 = 8 chunks of 16 bytes; chunk c of row r is stored
//    at c ^ ((r ^ r>>3) & 7), which keeps both the row-wise stores and the
//    MFMA fragment reads (8 consecutive rows, same chunk) free of bank
//    conflicts.
//
// Both kernels:
//  * Tile order: groups of 16 tile rows, column-major inside a group, and
//    inside every full chunk of 256 workgroups an XCD-aware permutation
//    that gives each of the 8 XCDs (workgroup id mod 8) a 4x8 block of
//    tiles, so the 32 CUs of an XCD share A rows and B columns in their L2
//    and the 8 XCDs together cover a 16x16 block through the MALL.
//  * Units that share a B block are listed next to each other by the host,
//    so their tiles stack into one tall virtual matrix.
#include "device_math.h"
#include "kernels.h"
#include "mfma16.h"

#include <type_traits>

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


// Workgroup id -> (virtual tile row, tile column). A bijection on [0, T).
// Each run of 256 workgroups (one wave of tiles, one per CU) covers a 16x16
// block of tiles, each XCD a 4x8 part of it. Groups of 16 tile rows walk
// their columns in alternating directions, so every wave shares the A or
// the B panels of the wave before it while those may still sit in the
// Infinity Cache: +0.5-1 % on multi-wave launches, same-box A/B.
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
  *vc = (group & 1) ? VC - 1 - idx / rows : idx / rows;
}

// One 32x32 block of v_mfma_f32_32x32x16_bf16. TRANS puts the B fragment
// first, so the block accumulates C^T (see store_tile).
template <bool TRANS>
__device__ __forceinline__ f32x16 mfma_block(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return TRANS ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0)
               : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Epilogue of a 256x256 tile (wave (wm, wn) owns a 128x128 sub-tile of
// 4x4 blocks of 32x32).
//  * float32 output: blocks accumulate C, register v of lane l holding
//    C[.. + 8(v/4) + 4(l/32) + v%4][.. + l%32]; each store instruction
//    writes two full 128-byte row segments (32 lanes x 4 bytes per row).
//  * bfloat16 output: blocks accumulate C^T (mfma_block<true>), register
//    4g + e of lane l holding C[.. + l%32][.. + 8g + 4(l/32) + e]: four
//    consecutive columns of one row, one 8-byte store when every C view is
//    8-byte aligned (L.vec_c) -- a quarter of the store instructions of
//    element-wise 2-byte stores.
template <bool OUT_BF16, bool GELU, bool EDGE>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], void* C, const GemmLaunch& L, int row0,
                                           int col0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int M = L.M, N = L.N;
  const int64_t ldc = L.ldc;
  const bool split = L.split_rows < M;
  auto row_off = [&](int r) -> int64_t {
    return split ? (r / L.split_rows) * L.split_stride + static_cast<int64_t>(r % L.split_rows) * ldc
                 : static_cast<int64_t>(r) * ldc;
  };
  if constexpr (!OUT_BF16) {
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
          static_cast<float*>(C)[row_off(r) + c] = x;
        }
  } else {
    const int rl = lane & 31, cq = 4 * (lane >> 5);
    const bool vec = L.vec_c != 0;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int r = row0 + wm * 128 + mi * 32 + rl;
      if (EDGE && r >= M) continue;
      const int64_t roff = row_off(r);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = col0 + wn * 128 + ni * 32 + 8 * g + cq;
          uint32_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = acc[mi][ni][4 * g + e];
            if (GELU) x = gelu_tanh_f32(x);
            h[e] = bf16_rne(x);
          }
          uint16_t* dst = static_cast<uint16_t*>(C) + roff + c;
          if (vec && (!EDGE || c + 3 < N)) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (!EDGE || c + e < N) dst[e] = static_cast<uint16_t>(h[e]);
          }
        }
    }
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
          acc[mi][ni] = mfma_block<OUT_BF16>(af[mi], bfv[ni], acc[mi][ni]);
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

  store_tile<OUT_BF16, GELU, EDGE>(acc, C, L, row0, col0);
}

// ---------------------------------------------------------------------------
// Interior tiles: direct HBM -> LDS pipeline, v_mfma_f32_16x16x32_bf16.
//
//  * Both operands travel global -> LDS with buffer_load_dwordx4 ... lds (16
//    bytes per lane, landing at M0 + 16 * lane): no staging registers, no
//    LDS stores, no register transpose. Each lane's byte offset inside the
//    tile is fixed; the k advance moves the buffer resource's base (scalar
//    arithmetic), so a load costs no vector instructions.
//  * K advances 32 at a time through a ring of 5 LDS stages of 32 KiB (A
//    256x32, B 32x256; 160 KiB, the whole LDS); loads run 4 stages ahead of
//    the stage whose MFMAs run (a stage's buffer is refilled as soon as its
//    fragments are in registers).
//  * Each wave's 128x128 sub-tile is 8x8 blocks of 16x16; one stage is one
//    k32 step of 64 MFMAs on 8 A and 8 B fragments. The 16x16x32 shape moves
//    half the accumulator data per flop of the 32x32x16 one, and under the
//    board's power limit on random data it holds a higher clock for the
//    same work.
//  * Blocks accumulate C^T (the B fragment goes in the first operand): lane
//    l holds C[16 mi + l%16][16 ni + 4(l/16) + e], e < 4, four consecutive
//    columns of one row.
//  * A stage: row r holds 32 k (64 bytes = 4 chunks); chunk c of row r sits
//    at c ^ a_swz(r), a_swz(r) = (row bit 2) << 1. An A fragment is one
//    16-byte LDS read per lane (8 k of row l%16, chunk l/16).
//  * Choosing the swizzle: a 16-byte LDS read serves 16 lanes a cycle, and
//    the conflict counters show the 16 are not 16 consecutive lanes: the
//    former swizzle (r >> 2) & 3 and a bit-swapped one both read at half
//    rate here, while the 32x32 layout's pattern and a contiguous 1 KiB
//    read run at the 4-cycle minimum. Modelling the lanes served together
//    as the cosets of a 4-dimensional XOR subspace of lane-index bits, 32
//    subspaces fit those four measurements. A row-major layout maps lane
//    bits to the 16 slots of a 256-byte window linearly, with a 2-dimensional
//    kernel, and reads without conflicts iff that kernel meets none of the
//    32; a_swz's kernel (lanes 0, 8, 36, 44) is one that does. A fragment
//    order (block-contiguous 1 KiB reads) also avoids the conflicts, but
//    its DMA touches 16 rows per 16 lanes and starved the pipeline.
//  * B stage: row k holds 256 n (512 bytes = 32 chunks); chunk c of row k
//    sits at c ^ b_swz(k), b_swz(k) = ((k & 3) << 2) | (((k >> 3) & 1) << 1).
//    B stays N-contiguous in LDS; the MFMA's k-packed fragment is read with
//    ds_read_b64_tr_b16, which (per 16-lane group) takes lane 4r+q's 4
//    consecutive elements as row r, columns 4q..4q+3 of a 4x16 tile and
//    returns column j to lane j. Two such reads give a lane the 8 k values
//    of its column. The (k & 3) term spreads the 4 rows of one group over
//    the banks; the k-bit-3 term moves the group reading k 8..15 to the
//    other 32-byte halves, so the two groups served together fill a
//    256-byte window (without it they collide, also at half rate).
//  * Two fragment sets: stage kt+1's 24 fragment reads ride on every other
//    MFMA of the first 48 of stage kt, which leaves each read at least 17
//    MFMAs to land; the fragment registers a read overwrites were last used
//    at least 15 MFMAs earlier.
// ---------------------------------------------------------------------------
constexpr int BK2 = 32;
constexpr int B_STAGE = BK2 * BN * 2;  // bytes

// Geometry of the pipeline kernel for MB row blocks of 16 per wave: MB = 8,
// the 256x256 tile above; MB = 4, a 128x256 tile for local products of at
// most 128 rows (a batch of 65..128 tokens, whose 256-row tiles would be
// half padding: with 128-row tiles the matrix cores do only the useful work
// and the launch stays bound by its single pass over B).
template <int MB>
struct Tile {
  static_assert(MB == 8 || MB == 4, "row blocks per wave");
  static constexpr int BMT = 32 * MB;           // tile rows (2 waves x MB blocks of 16)
  static constexpr int A_ST = BMT * BK2 * 2;    // A bytes per stage
  static constexpr int ST = A_ST + B_STAGE;     // stage bytes
  static constexpr int NST = MB == 8 ? 5 : 6;   // ring stages (160 KiB / 144 KiB)
  static constexpr int NA = MB / 2;             // A DMA items per wave and stage
  static constexpr int NDMA = NA + 4;           // DMA items per wave and stage
  static constexpr int NMF = 8 * MB;            // MFMAs per wave and stage
  static constexpr int NRD = MB + 16;           // fragment reads per wave and stage
  // Cache policy of the B loads: the 128-row tile serves local products of
  // at most 128 rows, one row tile per unit, so every B element is read
  // once per unit and streams past the caches (non-temporal: a 128-row batch
  // on [3584, 8192] x 8 B blocks ran 88 -> 86 us, 65 rows 86 -> 80 us, bit
  // for bit the same). The 256-row tile's B panels are re-read by the unit's
  // other row tiles and keep the default policy.
  static constexpr int B_AUX = MB == 4 ? 2 : 0;
  // Fragment read issued after MFMA idx of a stage (-1: none). Item i < MB:
  // A fragment i; item MB + 2 ni + t: read t of B fragment ni. Every read
  // overwrites registers last used at least 15 MFMAs earlier (a fragment of
  // the other set, last read by the previous stage's MFMAs).
  static constexpr int read_at(int idx) {
    if (MB == 8) return (idx < 48 && (idx & 1) == 0) ? idx >> 1 : -1;
    // MB = 4 (32 MFMAs, A fragment i last used at 8i + 7, B fragment ni at
    // 24 + ni): A0, A1 first, A2 at 6, A3 at 14, the B reads from 7 on
    constexpr int t[32] = {0, 1, -1, -1, -1, -1, 2, 4, 5, 6, 7, 8, 9, 10, 3, 11,
                           12, 13, 14, 15, 16, 17, 18, 19, -1, -1, -1, -1, -1, -1, -1, -1};
    return t[idx];
  }
  // DMA item issued after MFMA idx (-1: none): MB = 8 on 8j + 5, MB = 4 on 5j + 3.
  static constexpr int dma_at(int idx) {
    if (MB == 8) return (idx & 7) == 5 ? idx >> 3 : -1;
    return (idx % 5 == 3 && idx / 5 < NDMA) ? idx / 5 : -1;
  }
};

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint4 lds_u4;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef mfma_f32x4 f32x4;

__device__ __forceinline__ int b_swz(int k) { return ((k & 3) << 2) | (((k >> 3) & 1) << 1); }
// A chunk swizzle: chunk bit 1 flips with row bit 2.
__device__ __forceinline__ int a_swz(int r) { return ((r >> 2) & 1) << 1; }
// bfloat16 epilogue image: chunk swizzle of row r (16-byte chunks, 32 a row).
__device__ __forceinline__ int e_swz(int r) { return (r ^ ((r & 1) << 2)) & 31; }

// One 16x16 block, accumulating C^T in place (the B fragment is the first
// operand); the instruction and its hazard rules are in mfma16.h. Here:
//  * every accumulator is written once per 64 MFMAs;
//  * fragment registers are rewritten only by LDS reads issued at least 15
//    MFMAs after their last use, and each stage starts by waiting for every
//    LDS read (lgkmcnt 0);
//  * acc_fence() follows the zero fill, ahead of the prologue's loads, and
//    acc_drain() follows the last MFMA (before the K tail and before the
//    epilogue).
__device__ __forceinline__ void mfma16(const bf16x8& a, const bf16x8& b, f32x4& c) { mfma16x16x32(b, a, c); }

// s_waitcnt vmcnt(vm) lgkmcnt(lg) (expcnt unconstrained).
template <int vm, int lg>
__device__ __forceinline__ void wait_cnt() {
  static_assert(vm >= 0 && vm < 64 && lg >= 0 && lg < 16, "waitcnt range");
  __builtin_amdgcn_s_waitcnt((vm & 0xF) | ((vm >> 4) << 14) | 0x70 | (lg << 8));
}

template <int MB>
struct Frags {
  bf16x8 a[MB];
  bf16x8 b[8];
};

// A wave-uniform pointer moved into scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Element offset of the tile's first row in C (its output block when the
// rows are split).
__device__ __forceinline__ int64_t tile_row_base(const GemmLaunch& L, int row0) {
  if (L.split_rows < L.M) {
    const int blk = row0 / L.split_rows;
    return blk * L.split_stride + static_cast<int64_t>(row0 - blk * L.split_rows) * L.ldc;
  }
  return static_cast<int64_t>(row0) * L.ldc;
}

// Epilogue of an interior tile straight from the registers. The tile lies
// inside one output block (the host sends launches whose row split would cut
// a tile to the edge kernel), so every store address is a wave-uniform row
// base plus a per-lane offset fixed for the whole tile. Per block a lane
// stores its 4 consecutive columns: one 16-byte (float32) or 8-byte
// (bfloat16) store when the C views start on 4 elements (L.vec_c), else
// element by element.
// The 16-byte float32 stores carry the cache policy "nt sc0 sc1" (streaming,
// system scope): all tiles of a wave store at once, 64 MB per 256 tiles,
// and left in the L2 as dirty lines that burst slows the loads of the next
// wave of tiles. Measured against plain stores, same data and box: +12 % on
// four waves of K = 4096 tiles, +2.5 % on eight waves of K = 14336, +3 % on
// one wave; HBM write bytes unchanged. "nt" alone wrote half lines (1.46x
// the bytes) and lost on single waves. The 128-row tile (products of at most
// 128 rows: one wave of small partial blocks, which a rank-ordered sum reads
// right after) stores plainly: a 128-row batch on 8 [3584, 8192] blocks
// 89.9 -> 88.2 us alone and 100.6 -> 97.0 us with the sum that follows, 65
// and 96 rows within 1 %, bit for bit the same.
// GUARD: a ragged tile (past row M or column N of the view); only elements
// inside the view are stored.
template <bool OUT_BF16, bool GELU, bool GUARD, int MB>
__device__ __forceinline__ void store_tile_interior(const f32x4 (&acc)[MB][8], void* C, const GemmLaunch& L,
                                                    int row0, int col0, int wave) {
  const int lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int WR = 16 * MB;  // rows of a wave's sub-tile
  // rows / columns of this wave's sub-tile still inside the view
  const int rmax = GUARD ? L.M - row0 - wm * WR : WR, cmax = GUARD ? L.N - col0 - wn * 128 : 128;
  const int64_t ldc = L.ldc;
  const int64_t base = tile_row_base(L, row0) + static_cast<int64_t>(wm * WR) * ldc + col0 + wn * 128;
  const int lr = lane & 15, lc = 4 * (lane >> 4);
  const int voff = lr * static_cast<int>(ldc) + lc;
  const bool vec = L.vec_c != 0;
#pragma unroll
  for (int mi = 0; mi < MB; ++mi) {
    if (GUARD && mi * 16 + lr >= rmax) continue;
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) {
      const int cl = ni * 16 + lc;  // first of this lane's 4 columns
      if (GUARD && cl >= cmax) continue;
      const f32x4 v = acc_take(acc[mi][ni]);
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = v[e];
        if (GELU) x[e] = gelu_tanh_f32(x[e]);
      }
      const bool whole = vec && (!GUARD || cl + 3 < cmax);
      if constexpr (!OUT_BF16) {
        float* dst = static_cast<float*>(C) + base + static_cast<int64_t>(mi * 16) * ldc + voff + ni * 16;
        if (whole) {
          const f32x4 val = f32x4{x[0], x[1], x[2], x[3]};
          if constexpr (MB == 4)
            *reinterpret_cast<f32x4*>(dst) = val;
          else
            asm volatile("global_store_dwordx4 %0, %1, off nt sc0 sc1" ::"v"(dst), "v"(val) : "memory");
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!GUARD || cl + e < cmax) dst[e] = x[e];
        }
      } else {
        uint16_t* dst = static_cast<uint16_t*>(C) + base + static_cast<int64_t>(mi * 16) * ldc + voff + ni * 16;
        const uint32_t p01 = bf16x2_rne(x[0], x[1]), p23 = bf16x2_rne(x[2], x[3]);
        if (whole) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(p01, p23);
        } else {
          const uint16_t h[4] = {static_cast<uint16_t>(p01), static_cast<uint16_t>(p01 >> 16),
                                 static_cast<uint16_t>(p23), static_cast<uint16_t>(p23 >> 16)};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!GUARD || cl + e < cmax) dst[e] = h[e];
        }
      }
    }
  }
}

// bfloat16 epilogue of a full interior tile through LDS (the ring is free
// once the K loop is done): every wave writes its 128x128 sub-tile (after
// GeLU, rounded) into a row-major 256x256 bfloat16 image (128 KiB; 16-byte
// chunk c of row r at c ^ e_swz(r): 16 consecutive rows take distinct
// chunks for the 8-byte writes, and rows 2i, 2i+1, read in the same cycles,
// differ in chunk bit 2 for the 16-byte reads), then
// the workgroup stores whole rows: each store instruction writes two rows of
// 512 contiguous bytes. Stored straight from the registers, each instruction
// writes 32 bytes to each of 16 rows, and such partial lines doubled the HBM
// write traffic.
template <bool GELU, int MB>
__device__ __forceinline__ void store_tile_bf16_staged(const f32x4 (&acc)[MB][8], uint16_t* ct, int64_t ldc, int wave,
                                                       lds_char* smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int WR = 16 * MB;  // rows of a wave's sub-tile
  wait_cnt<0, 0>();
  __builtin_amdgcn_s_barrier();  // every wave is done with the ring
  asm volatile("" ::: "memory");
#pragma unroll
  for (int mi = 0; mi < MB; ++mi) {
    const int r = wm * WR + mi * 16 + (lane & 15);
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) {
      const int c = wn * 128 + ni * 16 + 4 * (lane >> 4);
      const f32x4 v = acc_take(acc[mi][ni]);
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = v[e];
        if (GELU) x[e] = gelu_tanh_f32(x[e]);
      }
      *(lds_u32x2*)(smem + r * 512 + (((c >> 3) ^ e_swz(r)) << 4) + ((c >> 2) & 1) * 8) =
          u32x2{bf16x2_rne(x[0], x[1]), bf16x2_rne(x[2], x[3])};
    }
  }
  wait_cnt<0, 0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll 4
  for (int it = 0; it < 32 * 2 * WR / NT; ++it) {  // 2 WR rows of 32 chunks
    const int q = tid + NT * it;
    const int r = q >> 5, ch = q & 31;
    const u32x4 v = *(lds_u32x4*)(smem + r * 512 + ((ch ^ e_swz(r)) << 4));
    *reinterpret_cast<u32x4*>(ct + static_cast<int64_t>(r) * ldc + ch * 8) = v;
  }
}

// ragged: the tile runs past row M or column N of the view. Its lanes that
// would load rows of A at or past M load row M-1 instead, and those that
// would load columns of B at or past N load the chunk holding column N-1:
// every load stays inside the views (no bounds on the loop's loads), and
// the duplicated data only reaches outputs past row M or column N, which
// are not stored.
// `wait_cnt<NDMA * n, LG>` for a count n known only at run time (n < 6).
template <int NDMA, int LG>
__device__ __forceinline__ void wait_stages(int n) {
  switch (n) {
    case 0: wait_cnt<0, LG>(); break;
    case 1: wait_cnt<NDMA, LG>(); break;
    case 2: wait_cnt<2 * NDMA, LG>(); break;
    case 3: wait_cnt<3 * NDMA, LG>(); break;
    case 4: wait_cnt<4 * NDMA, LG>(); break;
    default: wait_cnt<5 * NDMA, LG>(); break;
  }
}

template <bool OUT_BF16, bool GELU, int MB>
__device__ __forceinline__ void run_tile_lds(const GemmLaunch& L, const uint16_t* __restrict__ A,
                                             const uint16_t* __restrict__ B, void* C, int row0, int col0,
                                             bool ragged, lds_char* smem) {
  using T = Tile<MB>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t lda = L.lda, ldb = L.ldb;

  // ---- loader: per wave and stage NA A items (rows (NA w + i) * 16 +
  // lane/4, 64 bytes each) and 4 B items (rows (4w+i)*2 + lane/32, 512
  // bytes each), 1 KiB per instruction, through buffer loads whose per-lane
  // offsets stay fixed; the k advance moves the resource base.
  int va[T::NA], vb[4];
#pragma unroll
  for (int i = 0; i < T::NA; ++i) {
    const int ra = (T::NA * wave + i) * 16 + (lane >> 2);
    const int ca = (lane & 3) ^ a_swz(ra);
    const int ra_src = ragged ? min(ra, L.M - 1 - row0) : ra;
    va[i] = static_cast<int>((static_cast<int64_t>(ra_src) * lda + 8 * ca) * 2);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rb = (4 * wave + i) * 2 + (lane >> 5);
    const int cb = (lane & 31) ^ b_swz(rb);
    const int cb_src = ragged ? min(8 * cb, ((L.N - 1) & ~7) - col0) : 8 * cb;
    vb[i] = static_cast<int>((static_cast<int64_t>(rb) * ldb + cb_src) * 2);
  }
  // Tile bases in scalar registers: the buffer resources built from them
  // each stage must be wave-uniform registers, and a base the compiler kept
  // in vector registers would turn every load into a per-lane loop.
  const char* a_tile = uniform_ptr(reinterpret_cast<const char*>(A + static_cast<int64_t>(row0) * lda));
  const char* b_tile = uniform_ptr(reinterpret_cast<const char*>(B + col0));
  const int64_t a_step = BK2 * 2, b_step = static_cast<int64_t>(BK2) * ldb * 2;

  // ---- fragment offsets inside a stage buffer.
  // A block mi: row wm*16MB + 16 mi + l%16, chunk l/16. The swizzle reads
  // row bit 2, which comes from the lane alone, so block mi sits 1 KiB
  // after block 0.
  const int ar = wm * 16 * MB + (lane & 15);
  const int a_off = ar * (BK2 * 2) + (((lane >> 4) ^ a_swz(ar)) << 4);
  // B block ni: columns wn*128 + 16 ni + 4q (q = l%4) of rows 8g + rr
  // (g = l/16, rr = (l/4)%4) for the first read and 4 rows further for the
  // second; both rows have the same swizzle, so the second read sits 2 KiB
  // after the first.
  int b_off[8];
  {
    const int kr = 8 * (lane >> 4) + ((lane >> 2) & 3);
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) {
      const int col = wn * 128 + ni * 16 + 4 * (lane & 3);
      b_off[ni] = T::A_ST + kr * (BN * 2) + (((col >> 3) ^ b_swz(kr)) << 4) + ((col >> 2) & 1) * 8;
    }
  }
  auto read_item = [&](Frags<MB>& F, int sb, int item) __attribute__((always_inline)) {
    lds_char* st = smem + sb;
    if (item < MB) {
      F.a[item] = __builtin_bit_cast(bf16x8, *(lds_u4*)(st + a_off + item * 1024));
    } else {
      const int ni = (item - MB) >> 1, t = (item - MB) & 1;
      const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(st + b_off[ni] + t * 2048));
      if (t == 0)
        F.b[ni] = __builtin_shufflevector(v, F.b[ni].hi, 0, 1, 2, 3, 4, 5, 6, 7);
      else
        F.b[ni] = __builtin_shufflevector(F.b[ni].lo, v, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  // DMA item of stage kt_load into the stage buffer at byte offset sb.
  auto dma_item = [&](int kt_load, int sb, int item) __attribute__((always_inline)) {
    if (item < T::NA) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a_tile + kt_load * a_step), (short)0, 0x7fffffff, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(smem + sb + (T::NA * wave + item) * 1024), 16, va[item],
                                               0, 0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(b_tile + kt_load * b_step), (short)0, 0x7fffffff, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_void*)(smem + sb + T::A_ST + (4 * wave + item - T::NA) * 1024), 16, vb[item - T::NA], 0, 0,
          T::B_AUX);
    }
  };

  f32x4 acc[MB][8];
#pragma unroll
  for (int mi = 0; mi < MB; ++mi)
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  acc_fence(acc);

  // One stage: NMF MFMAs on `cur`; the NRD fragment reads of the next stage
  // (if rd) and the NDMA DMA items of stage kt_load (if ld) ride on the
  // MFMAs that Tile<MB>::read_at / dma_at name. For the 256-row tile (64
  // MFMAs) the reads sit on every other MFMA from 0 to 46 and the DMA on
  // MFMAs 8j+5: spread this way the stage ran 6 % faster than with the
  // reads on MFMAs 0..23 and the DMA after them, and bunching the DMA early
  // in the stage was 5-12 % slower.
  // The lambdas are forced inline: inlined later, the LDS reads lost the
  // alias information that tells the compiler they do not touch the
  // in-flight LDS loads, and it waited for every load (vmcnt 0) before
  // them.
  auto stage = [&](const Frags<MB>& cur, Frags<MB>& nxt, bool rd, int sb_rd, bool ld, int kt_load, int sb_ld)
                   __attribute__((always_inline)) {
#pragma unroll
    for (int idx = 0; idx < T::NMF; ++idx) {
      const int mi = idx >> 3, ni = idx & 7;
      mfma16(cur.a[mi], cur.b[ni], acc[mi][ni]);
      if (T::read_at(idx) >= 0 && rd) read_item(nxt, sb_rd, T::read_at(idx));
      if (T::dma_at(idx) >= 0 && ld) dma_item(kt_load, sb_ld, T::dma_at(idx));
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = L.K / BK2;
  constexpr int NST = T::NST;
  constexpr int RING = NST * T::ST;
  Frags<MB> F[2];
  // prologue: stages 0..NST-1 in flight, then stage 0's fragments
#pragma unroll
  for (int p = 0; p < NST; ++p)
    if (p < nk) {
#pragma unroll
      for (int it = 0; it < T::NDMA; ++it) dma_item(p, p * T::ST, it);
    }
  wait_stages<T::NDMA, 15>(min(nk, NST) - 1);  // stage 0 landed
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < T::NRD; ++i) read_item(F[0], 0, i);
  }

  int sb_cur = 0;        // buffer of stage kt
  int sb_rd = T::ST;     // buffer of stage kt+1
  // Iteration kt: the MFMAs of stage kt on F[kt % 2]; stage kt+1's
  // fragments into the other set; stage kt+NST into stage kt's buffer. That
  // buffer is free: its fragments were read in iteration kt-1, and every
  // wave waited for its reads (lgkmcnt 0) before this iteration's barrier.
  // Loads run NST-1 stages ahead.
  auto iter = [&](auto parity_c, int kt, bool steady) __attribute__((always_inline)) {
    constexpr int P = decltype(parity_c)::value;  // kt % 2
    const bool rd = steady || kt + 1 < nk;
    const bool ld = steady || kt + NST < nk;
    __builtin_amdgcn_sched_barrier(0);
    // stage kt+1 landed; stages kt+2 .. kt+NST-1 may still be in flight
    if (steady)
      wait_cnt<(NST - 2) * T::NDMA, 0>();
    else
      wait_stages<T::NDMA, 0>(max(0, min(nk - 1, kt + NST - 1) - (kt + 1)));
    asm volatile("" ::: "memory");
    if (rd) __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    stage(F[P], F[P ^ 1], rd, sb_rd, ld, kt + NST, sb_cur);
    sb_cur = sb_rd;
    sb_rd = sb_rd + T::ST == RING ? 0 : sb_rd + T::ST;
  };

  int kt = 0;
  for (; kt + 1 + NST < nk; kt += 2) {
    iter(std::integral_constant<int, 0>{}, kt, true);
    iter(std::integral_constant<int, 1>{}, kt + 1, true);
  }
  for (; kt < nk; kt += 2) {
    iter(std::integral_constant<int, 0>{}, kt, false);
    if (kt + 1 < nk) iter(std::integral_constant<int, 1>{}, kt + 1, false);
  }

  acc_drain(acc);

  // K tail (K % 32 columns of A, rows of B): one more stage, loaded through
  // registers with every element at or past K (and past the view's rows of
  // A or columns of B) read as zero, and written into ring buffer 0 in the
  // layout the buffer loads produce; then its MFMAs.
  const int k_tail = L.K - nk * BK2;
  if (k_tail > 0) {
    wait_cnt<0, 0>();
    __builtin_amdgcn_s_barrier();  // every wave is done with the ring
    asm volatile("" ::: "memory");
    const int kb = nk * BK2;
#pragma unroll
    for (int j = 0; j < T::BMT * 4 / NT; ++j) {
      const int q = tid + NT * j;  // A: BMT rows x 4 chunks of 8 k
      const int r = q >> 2, c = q & 3;
      const int row = row0 + min(r, L.M - 1 - row0);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k0 = kb + 8 * c + 2 * e;
        const uint16_t* pa = A + static_cast<int64_t>(row) * lda + k0;
        const uint32_t lo = k0 < L.K ? pa[0] : 0u, hi = k0 + 1 < L.K ? pa[1] : 0u;
        w[e] = lo | (hi << 16);
      }
      *(lds_u32x4*)(smem + r * (BK2 * 2) + ((c ^ a_swz(r)) << 4)) = u32x4{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = tid + NT * j;  // B: 32 rows (k) x 32 chunks of 8 columns
      const int rb = q >> 5, cb = q & 31;
      const int k = kb + rb;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n0 = col0 + 8 * cb + 2 * e;
        const uint16_t* pb = B + static_cast<int64_t>(k) * ldb + n0;
        const uint32_t lo = (k < L.K && n0 < L.N) ? pb[0] : 0u, hi = (k < L.K && n0 + 1 < L.N) ? pb[1] : 0u;
        w[e] = lo | (hi << 16);
      }
      *(lds_u32x4*)(smem + T::A_ST + rb * (BN * 2) + ((cb ^ b_swz(rb)) << 4)) = u32x4{w[0], w[1], w[2], w[3]};
    }
    wait_cnt<0, 0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < T::NRD; ++i) read_item(F[0], 0, i);
    wait_cnt<0, 0>();
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) mfma16(F[0].a[mi], F[0].b[ni], acc[mi][ni]);
    acc_drain(acc);
  }

  if (ragged) {
    store_tile_interior<OUT_BF16, GELU, true, MB>(acc, C, L, row0, col0, wave);
  } else if constexpr (OUT_BF16) {
    // whole rows through LDS when the tile's rows start on 16 bytes (the
    // view's start; ldc is a multiple of 8 and col0 of 256)
    uint16_t* ct = static_cast<uint16_t*>(C) + tile_row_base(L, row0) + col0;
    if ((reinterpret_cast<uintptr_t>(ct) & 15) == 0)
      store_tile_bf16_staged<GELU, MB>(acc, ct, L.ldc, wave, smem);
    else
      store_tile_interior<OUT_BF16, GELU, false, MB>(acc, C, L, row0, col0, wave);
  } else {
    store_tile_interior<OUT_BF16, GELU, false, MB>(acc, C, L, row0, col0, wave);
  }
}

// Every tile of every unit: full tiles, and ragged ones (the last tile row
// past M, the last tile column past N), whose loads are clamped into the
// views and whose stores are guarded; a K that is not a multiple of 32 ends
// with a zero-filled tail stage. Every view is 16-byte aligned
// (all_tiles_edge false).
// L.tiles_m counts tiles of Tile<MB>::BMT rows.
template <bool OUT_BF16, bool GELU, int MB>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_mfma_kernel(const GemmLaunch L) {
  constexpr int BMT = Tile<MB>::BMT;
  __shared__ __attribute__((aligned(1024))) char smem[Tile<MB>::NST * Tile<MB>::ST];
  const int VR = L.n_units * L.tiles_m;
  const int T = VR * L.tiles_n;
  int vr, vc;
  tile_of(blockIdx.x, T, VR, L.tiles_n, &vr, &vc);
  const int unit = vr / L.tiles_m;
  const int row0 = (vr - unit * L.tiles_m) * BMT;
  const int col0 = vc * BN;
  const bool ragged = row0 + BMT > L.M || col0 + BN > L.N;
  const GemmUnitPtrs U = L.u[unit];
  run_tile_lds<OUT_BF16, GELU, MB>(L, U.a, U.b, U.c, row0, col0, ragged, (lds_char*)smem);
}

// The MFMA kernel takes every tile unless a view is not 16-byte aligned (or
// the last row of a B view leaves no room for a 16-byte chunk past column
// N, which the host folds into vec_ok), a lane's byte offset inside a tile's buffer
// resource (up to BMT-1 rows of A, 31 rows of B) or a lane's element offset
// inside an output tile (31 rows of C) would not fit in 31 bits, or a row
// split of the output does not fall on tile boundaries. Then every tile goes
// to the edge kernel.
__host__ __device__ __forceinline__ bool all_tiles_edge(const GemmLaunch& L, int bmt) {
  constexpr int64_t kMaxOffset = int64_t{1} << 31;
  return !L.vec_ok || (static_cast<int64_t>(bmt - 1) * L.lda + BK2) * 2 >= kMaxOffset ||
         (static_cast<int64_t>(BK2 - 1) * L.ldb + BN) * 2 >= kMaxOffset || L.ldc * 32 >= kMaxOffset ||
         (L.split_rows < L.M && L.split_rows % bmt != 0);
}

// Edge kernel: every tile of the launch (all_tiles_edge). Loads outside the
// views read as zero and stores outside them are skipped. blockIdx.y = unit.
template <bool OUT_BF16, bool GELU>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_mfma_edge_kernel(const GemmLaunch L) {
  __shared__ uint4 lds[2 * 2 * BM * CH];
  const int unit = blockIdx.y;
  const int tm = blockIdx.x / L.tiles_n;
  const int tn = blockIdx.x % L.tiles_n;
  const GemmUnitPtrs U = L.u[unit];
  run_tile<true, OUT_BF16, GELU>(L, U.a, U.b, U.c, tm * BM, tn * BN, lds);
}

// Local products of at most 128 rows take the 128-row tile (Tile<4>),
// taller ones the 256-row tile (Tile<8>).
template <bool OUT_BF16, bool GELU>
hipError_t launch_variant(const GemmLaunch& L, hipStream_t s) {
  if (L.M <= Tile<4>::BMT && !all_tiles_edge(L, Tile<4>::BMT)) {
    GemmLaunch L4 = L;
    L4.tiles_m = (L.M + Tile<4>::BMT - 1) / Tile<4>::BMT;
    const int T = L4.n_units * L4.tiles_m * L4.tiles_n;
    hipLaunchKernelGGL((gemm_bf16_mfma_kernel<OUT_BF16, GELU, 4>), dim3(T), dim3(NT), 0, s, L4);
  } else if (L.M > Tile<4>::BMT && !all_tiles_edge(L, Tile<8>::BMT)) {
    const int T = L.n_units * L.tiles_m * L.tiles_n;
    hipLaunchKernelGGL((gemm_bf16_mfma_kernel<OUT_BF16, GELU, 8>), dim3(T), dim3(NT), 0, s, L);
  } else {
    hipLaunchKernelGGL((gemm_bf16_mfma_edge_kernel<OUT_BF16, GELU>), dim3(L.tiles_m * L.tiles_n, L.n_units), dim3(NT),
                       0, s, L);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma(const GemmLaunch& L, hipStream_t s) {
  if (L.out_bf16)
    return L.epilogue == kEpiGelu ? launch_variant<true, true>(L, s) : launch_variant<true, false>(L, s);
  return L.epilogue == kEpiGelu ? launch_variant<false, true>(L, s) : launch_variant<false, false>(L, s);
}

}  // namespace shardmm
