// MFMA helpers for gfx950 (wave64).
//
// v_mfma_f32_16x16x4_f32 lane layout (checked on the device): with l the lane, li = l % 16
// and gq = l / 16,
//   A (16 x 4):  lane l supplies A[li][gq]
//   B (4 x 16):  lane l supplies B[gq][li]
//   D (16 x 16): lane l holds D[4 * gq + r][li] in accumulator element r (r < 4)
// A K = 16 slice is consumed in four steps s = 0..3.  Every product here uses the
// permuted contraction index k(s, gq) = 4 * gq + s inside each 16-slice: it is a bijection,
// so the sum is unchanged, and it lets a D-layout accumulator tile serve directly as the
// B operand of the next product (its element r is then exactly the value for step s = r).
#pragma once

#include <hip/hip_runtime.h>

namespace vla {

typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4_t mfma_f32_16x16x4(float a, float b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4_t f4_zero() { return f4_t{0.f, 0.f, 0.f, 0.f}; }

}  // namespace vla
