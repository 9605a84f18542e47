// Device helpers shared by the VLA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vla {

constexpr int kWave = 64;

// ---- input / output element conversion ------------------------------------------------
// bf16 is stored as its raw 16-bit pattern; widening to fp32 is exact.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet bit forced).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((x >> 16) | 0x0040u);
  x += 0x7fffu + ((x >> 16) & 1u);
  return static_cast<uint16_t>(x >> 16);
}

template <typename T> struct io;

template <> struct io<float> {
  static constexpr int kVec = 4;  // elements per 16-byte load
  using vec_t = float4;
  __device__ __forceinline__ static void unpack(const vec_t &r, float *o) {
    o[0] = r.x; o[1] = r.y; o[2] = r.z; o[3] = r.w;
  }
  __device__ __forceinline__ static float store_cvt(float x) { return x; }
};

template <> struct io<bf16_t> {
  static constexpr int kVec = 8;
  using vec_t = uint4;
  __device__ __forceinline__ static void unpack(const vec_t &r, float *o) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// The backward's per-token record, fp32: z = A_{t-1} u, ahat, r = v - S_{t-1} khat, o (d values
// each), then delta = 1 + u . z, ||A_t khat||, 1/||k||, den and spare slots (khat = k / ||k|| and
// phi(q) are formed again from the inputs where they are needed); and the state (S, A) after
// every kBwCk-th token and after each segment's last token.  Written by the backward's replay,
// or by the chunked forward's passes for the backward.
constexpr int kBwScalars = 8;
constexpr int kBwCk = 64;
template <int D>
struct BwRec {
  static constexpr int Z = 0, AH = D, R = 2 * D, O = 3 * D, SC = 4 * D;  // field offsets
  static constexpr int F = 4 * D + kBwScalars;  // floats per token record
};

// ELU(x) + 1 with alpha = 1.
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// ---- cross-lane sums ------------------------------------------------------------------
// Every step pairs lanes symmetrically (a + b on one side, b + a on the other), so all
// participating lanes finish with bitwise-identical sums.
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_half_mirror(float x) {  // lane i <-> 7 - i within 8
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_mirror(float x) {  // lane i <-> 15 - i within 16
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
}

__device__ __forceinline__ float pair_sum(float x) { return x + dpp_xor1(x); }

// Sum over each 16-lane row; every lane of the row ends with bitwise the same sum.
__device__ __forceinline__ float row_sum16(float x) {
  x = x + dpp_xor1(x);
  x = x + dpp_xor2(x);
  x = x + dpp_half_mirror(x);
  return x + dpp_mirror(x);
}

// row_sum16 of N independent values, stage by stage across the values, so that each DPP
// move has other work between it and the addition that produced its operand (no wait states
// between the stages of one chain); every value's sum is bitwise row_sum16's.
template <int N>
__device__ __forceinline__ void row_sum16_n(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = x[i] + dpp_xor1(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = x[i] + dpp_xor2(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = x[i] + dpp_half_mirror(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = x[i] + dpp_mirror(x[i]);
}

// y summed over the four 16-lane rows of the wave (lanes l, l ^ 16, l ^ 32, l ^ 48), in every
// lane: two gfx950 row swaps on the VALU (v_permlane16_swap_b32, v_permlane32_swap_b32; with
// both operands y, the two results of a swap add up to y plus its partner row's y), where
// __shfl_xor would go through the LDS crossbar (ds_bpermute) and wait for it.
__device__ __forceinline__ float sum_rows4(float y) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over all 64 lanes of the wave (the whole wave must be active), broadcast to every lane.
// After the row sums, rows 1 and 3 add the last lane of rows 0 and 2 (DPP row_bcast:15), row 3
// then adds lane 31 (row_bcast:31), and lane 63's total is read out: all on the VALU, no LDS
// permute, in a fixed order ((r2 + r3) + (r0 + r1)).
__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  x = x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));
  x = x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xC, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

}  // namespace vla
