// v_mfma_f32_16x16x32_bf16 as an instruction, and the rules that replace
// the hazard padding the compiler gives its own MFMAs.
//
// Why an instruction: with the compiler's MFMA for this shape, kernels that
// keep 256 accumulators split them between the AGPR and VGPR files and copy
// them around every MFMA (or spill). The "+a" tie keeps each accumulator in
// one AGPR quad, updated in place.
//
// The compiler sees no MFMA, so the kernels keep to these rules:
//  * an accumulator is not the target of two MFMAs closer than 8 apart;
//  * operands come from loads, not from VALU instructions, and operand
//    registers are rewritten only by loads issued well after their last
//    MFMA (the kernel documents the distance); before MFMAs read loaded
//    data the kernel waits for it (waitcnt);
//  * acc_fence() after the zero fill keeps the fill ahead of the first MFMA
//    (the kernels put loads and barriers in between);
//  * acc_drain() pads 24 wait states after the last MFMA (more than the
//    8-pass MFMA's write-to-read distance) and then claims every
//    accumulator, so no compiler-placed read of one (a spill, a store)
//    comes before the padding.
#pragma once

namespace shardmm {

typedef __bf16 mfma_bf16x8 __attribute__((ext_vector_type(8)));
typedef float mfma_f32x4 __attribute__((ext_vector_type(4)));

// c += a_op . b_op for a 16x16 block, 32 k (lane l: a_op row l%16, b_op
// column l%16, both k 8(l/16)..+8; c rows 4(l/16)..+4 of column l%16).
__device__ __forceinline__ void mfma16x16x32(const mfma_bf16x8& a_op, const mfma_bf16x8& b_op, mfma_f32x4& c) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a_op), "v"(b_op));
}

template <int R>
__device__ __forceinline__ void acc_fence(mfma_f32x4 (&acc)[R][8]) {
#pragma unroll
  for (int mi = 0; mi < R; ++mi)
    asm volatile("" : "+a"(acc[mi][0]), "+a"(acc[mi][1]), "+a"(acc[mi][2]), "+a"(acc[mi][3]), "+a"(acc[mi][4]),
                 "+a"(acc[mi][5]), "+a"(acc[mi][6]), "+a"(acc[mi][7]));
}

template <int R>
__device__ __forceinline__ void acc_drain(mfma_f32x4 (&acc)[R][8]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  acc_fence(acc);
}

// One block's accumulators moved to VGPRs where they are used (left to
// itself the compiler copies all of them out of the AGPRs at once and
// spills).
__device__ __forceinline__ mfma_f32x4 acc_take(const mfma_f32x4& a) {
  mfma_f32x4 v;
  asm volatile("" : "=v"(v) : "0"(a));
  return v;
}

}  // namespace shardmm
