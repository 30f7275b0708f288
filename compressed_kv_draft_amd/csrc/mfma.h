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

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace vc
