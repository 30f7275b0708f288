// gfx950 matrix-core operand types and the 16x16x32 MFMA lane layout used by
// the attention kernels.
//
// v_mfma_f32_16x16x32_{bf16,f16}: D[16x16] += A[16x32] * B[32x16] per wavefront.
//   A: lane l holds row (l % 16), k = 8 * (l / 16) + e for e = 0..7
//   B: lane l holds col (l % 16), k = 8 * (l / 16) + e
//   C/D (4 fp32 per lane): lane l holds col (l % 16), rows 4 * (l / 16) + i
// The contraction index k may be any permutation of the 32 physical indices
// as long as A and B use the same one; the kernels use that freedom to keep
// each lane's data contiguous in memory.
#pragma once

#include <hip/hip_runtime.h>

namespace vc {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// ds_read_b64_tr_b16 (gfx950): inside each group of 16 lanes, lane j supplies the
// address of 4 consecutive 16-bit elements M[j][0..3]; lane i receives
// M[4 e + i / 4][i % 4] for e = 0..3.  Pointing lane j at row (r0 + j / 4),
// column (c0 + 4 * (j % 4)) of a row-major tile therefore hands lane i the
// column c0 + i of rows r0 .. r0 + 3: a transposed 4 x 16 read.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace vc
