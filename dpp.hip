#include <hip/hip_runtime.h>
#include <utility>
template <int J> __device__ __forceinline__ float rbc(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + J, 0xf, 0xf, false));
}
template <int J> __device__ __forceinline__ void step(float (&x)[16]) {
  const float nt = x[J] * -0.5f;
#pragma unroll
  for (int r = J + 1; r < 16; ++r) x[r] = fmaf(rbc<J>(x[r]), nt, x[r]);
}
template <int... J> __device__ __forceinline__ void all(float (&x)[16], std::integer_sequence<int, J...>) { (step<J>(x), ...); }
__global__ void k(const float *in, float *out) {
  const int lane = threadIdx.x & 63;
  float x[16];
  for (int r = 0; r < 16; ++r) x[r] = in[lane * 16 + r];
  all(x, std::make_integer_sequence<int, 15>{});
  for (int r = 0; r < 16; ++r) out[lane * 16 + r] = x[r];
}
