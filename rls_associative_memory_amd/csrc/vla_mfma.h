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
#include <stdint.h>

namespace vla {

typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4_t mfma_f32_16x16x4(float a, float b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4_t f4_zero() { return f4_t{0.f, 0.f, 0.f, 0.f}; }

// ---- bf16 matrix cores with fp32 operands split into bf16 terms ------------------------
// v_mfma_f32_16x16x32_bf16 (checked on the device): A lane l supplies A[li][8 gq + e], B lane l
// supplies B[8 gq + e][li] (e < 8); D as above.  The products below use a permuted
// contraction index: element e < 4 of a lane is k = 32 s + 4 gq + e and element e >= 4 is
// k = 32 s + 16 + 4 gq + (e - 4), so that the four accumulator values of two D-layout tiles
// form one operand.  A raw bf16 input is exact in one term; an fp32 value x is split as
// x = h + m + l (three terms, about 24 significant bits) or x = h + l (two terms, about 16).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f4_t mfma_bf16(const bf16x8_t &a, const bf16x8_t &b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct Split3 {
  bf16x8_t t[3];
};

__device__ __forceinline__ Split3 split3(const float (&x)[8]) {
  Split3 s;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(x[e]);
    const float r1 = x[e] - static_cast<float>(h);
    const __bf16 m = static_cast<__bf16>(r1);
    const float r2 = r1 - static_cast<float>(m);
    s.t[0][e] = h;
    s.t[1][e] = m;
    s.t[2][e] = static_cast<__bf16>(r2);
  }
  return s;
}

// exact A operand x split B operand
__device__ __forceinline__ f4_t mm_xs(const bf16x8_t &a, const bf16x8_t (&b)[3], f4_t c) {
  c = mfma_bf16(a, b[2], c);
  c = mfma_bf16(a, b[1], c);
  return mfma_bf16(a, b[0], c);
}
// split A operand x exact B operand
__device__ __forceinline__ f4_t mm_sx(const bf16x8_t (&a)[3], const bf16x8_t &b, f4_t c) {
  c = mfma_bf16(a[2], b, c);
  c = mfma_bf16(a[1], b, c);
  return mfma_bf16(a[0], b, c);
}
// split x split (term pairs a + b <= 2)
__device__ __forceinline__ f4_t mm_ss(const bf16x8_t (&a)[3], const bf16x8_t (&b)[3], f4_t c) {
  c = mfma_bf16(a[1], b[1], c);
  c = mfma_bf16(a[0], b[2], c);
  c = mfma_bf16(a[2], b[0], c);
  c = mfma_bf16(a[0], b[1], c);
  c = mfma_bf16(a[1], b[0], c);
  return mfma_bf16(a[0], b[0], c);
}

__device__ __forceinline__ bf16x8_t ld_bf8(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(p));
}
__device__ __forceinline__ bf16x8_t ld_bf4x2(const uint16_t *p0, const uint16_t *p1) {
  const uint2 a = *reinterpret_cast<const uint2 *>(p0);
  const uint2 b = *reinterpret_cast<const uint2 *>(p1);
  return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}
__device__ __forceinline__ void ld_split(bf16x8_t (&dst)[3], const uint16_t *base, int term_stride) {
#pragma unroll
  for (int t = 0; t < 3; ++t) dst[t] = ld_bf8(base + t * term_stride);
}
__device__ __forceinline__ uint16_t bf_bits(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }
__device__ __forceinline__ float bf_val(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// ---- transposing LDS load (ds_read_b64_tr_b16) --------------------------------------------
// In each group of 16 lanes, lane j supplies the address of four 16-bit elements and lane i
// receives element i % 4 of lane 4 e + i / 4 (e = 0..3), as checked on the device.  So when
// lane j of the group addresses &M[r0 + j / 4][c0 + 4 (j % 4)] of a row-major 16-bit matrix
// M, lane i receives M[r0 + e][c0 + i], e = 0..3: four consecutive rows of its column.
typedef short s4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ld_tr4(const uint16_t *p) {
  typedef s4_t __attribute__((address_space(3))) *lds_s4_ptr;  // p points into LDS
  const s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(p));
  return __builtin_bit_cast(uint2, v);
}
// Two transposed 4 x 16 blocks as one bf16 operand: lane i gets M[r0 + e][c0 + i] (e < 4) and
// M[r1 + e][c0 + i]; `li` is the lane's index in its group of 16.
__device__ __forceinline__ bf16x8_t ld_tr4x2(const uint16_t *m, int ld, int r0, int r1, int c0, int li) {
  const int dr = li >> 2, dc = 4 * (li & 3);
  const uint2 a = ld_tr4(m + (r0 + dr) * ld + c0 + dc);
  const uint2 b = ld_tr4(m + (r1 + dr) * ld + c0 + dc);
  return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}

// The first block of ld_tr4x2 (lane i gets M[r0 + e][c0 + i]) and zeros for the second.
__device__ __forceinline__ bf16x8_t ld_tr4z(const uint16_t *m, int ld, int r0, int c0, int li) {
  const int dr = li >> 2, dc = 4 * (li & 3);
  const uint2 a = ld_tr4(m + (r0 + dr) * ld + c0 + dc);
  return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, 0u, 0u));
}

// N terms of a row-major matrix (term stride in elements), each read as ld_tr4x2
template <int N>
__device__ __forceinline__ void ld_tr_n(bf16x8_t (&dst)[N], const uint16_t *m, int term_stride, int ld,
                                        int r0, int r1, int c0, int li) {
#pragma unroll
  for (int t = 0; t < N; ++t) dst[t] = ld_tr4x2(m + t * term_stride, ld, r0, r1, c0, li);
}

// ---- packed splits: two fp32 values at a time through v_cvt_pk_bf16_f32 -----------------
// pk_bf16(a, b) rounds both to bf16 (nearest even), a in the low half.  A term's value is
// recovered by placing its half in the high bits of an fp32 word, so a residual costs a
// shift or a mask and a subtraction; one split of two values into N terms is N conversions.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ float pk_lo_val(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float pk_hi_val(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
// a = sum_i lo(t[i]), b = sum_i hi(t[i]), each to about 8 N significant bits
template <int N>
__device__ __forceinline__ void split_pk(float a, float b, uint32_t (&t)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    t[i] = pk_bf16(a, b);
    if (i + 1 < N) {
      a -= pk_lo_val(t[i]);
      b -= pk_hi_val(t[i]);
    }
  }
}

// Split one fp32 value into its three bf16 terms (bit patterns).
__device__ __forceinline__ void split1(float x, uint16_t &h, uint16_t &m, uint16_t &l) {
  const __bf16 bh = static_cast<__bf16>(x);
  const float r1 = x - static_cast<float>(bh);
  const __bf16 bm = static_cast<__bf16>(r1);
  const float r2 = r1 - static_cast<float>(bm);
  h = bf_bits(bh);
  m = bf_bits(bm);
  l = bf_bits(static_cast<__bf16>(r2));
}

// v where ok, else zeros (component-wise, so the value stays in registers)
__device__ __forceinline__ uint4 keep_if(bool ok, const uint4 &v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

// ---- N-term split (N = 2 or 3), generic over the number of terms ----------------------
template <int N>
__device__ __forceinline__ void split_n(float x, uint16_t (&out)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const __bf16 b = static_cast<__bf16>(x);
    out[i] = bf_bits(b);
    x -= static_cast<float>(b);
  }
}
template <int N>
__device__ __forceinline__ void split_n8(const float (&x)[8], bf16x8_t (&t)[N]) {
  uint32_t w[4][N];
#pragma unroll
  for (int e = 0; e < 4; ++e) split_pk<N>(x[2 * e], x[2 * e + 1], w[e]);
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0][i], w[1][i], w[2][i], w[3][i]));
}
template <int N>
__device__ __forceinline__ void ld_split_n(bf16x8_t (&dst)[N], const uint16_t *base, int term_stride) {
#pragma unroll
  for (int t = 0; t < N; ++t) dst[t] = ld_bf8(base + t * term_stride);
}
// exact x N-term (smallest terms first)
template <int N>
__device__ __forceinline__ f4_t mmn_xs(const bf16x8_t &a, const bf16x8_t (&b)[N], f4_t c) {
#pragma unroll
  for (int i = N - 1; i >= 0; --i) c = mfma_bf16(a, b[i], c);
  return c;
}
template <int N>
__device__ __forceinline__ f4_t mmn_sx(const bf16x8_t (&a)[N], const bf16x8_t &b, f4_t c) {
#pragma unroll
  for (int i = N - 1; i >= 0; --i) c = mfma_bf16(a[i], b, c);
  return c;
}
// N-term x N-term: the term pairs (i, j) with i + j < N, smallest first
template <int N>
__device__ __forceinline__ f4_t mmn_ss(const bf16x8_t (&a)[N], const bf16x8_t (&b)[N], f4_t c) {
#pragma unroll
  for (int s = N - 1; s >= 0; --s)
#pragma unroll
    for (int i = 0; i <= s; ++i) c = mfma_bf16(a[i], b[s - i], c);
  return c;
}

// ---- two-term split ----------------------------------------------------------------------
struct Split2 {
  bf16x8_t h, l;
};

__device__ __forceinline__ void split2_1(float x, uint16_t &h, uint16_t &l) {
  const __bf16 bh = static_cast<__bf16>(x);
  h = bf_bits(bh);
  l = bf_bits(static_cast<__bf16>(x - static_cast<float>(bh)));
}

__device__ __forceinline__ Split2 split2(const float (&x)[8]) {
  uint32_t w[4][2];
#pragma unroll
  for (int e = 0; e < 4; ++e) split_pk<2>(x[2 * e], x[2 * e + 1], w[e]);
  return Split2{__builtin_bit_cast(bf16x8_t, make_uint4(w[0][0], w[1][0], w[2][0], w[3][0])),
                __builtin_bit_cast(bf16x8_t, make_uint4(w[0][1], w[1][1], w[2][1], w[3][1]))};
}
// Four values (an accumulator tile) split into the first half of two-term operands; the
// second half is zero.
__device__ __forceinline__ Split2 split2_4z(const f4_t &v) {
  uint32_t a[2], b[2];
  split_pk<2>(v[0], v[1], a);
  split_pk<2>(v[2], v[3], b);
  return Split2{__builtin_bit_cast(bf16x8_t, make_uint4(a[0], b[0], 0u, 0u)),
                __builtin_bit_cast(bf16x8_t, make_uint4(a[1], b[1], 0u, 0u))};
}

// exact x two-term
__device__ __forceinline__ f4_t mm2_xs(const bf16x8_t &a, const Split2 &b, f4_t c) {
  c = mfma_bf16(a, b.l, c);
  return mfma_bf16(a, b.h, c);
}
// two-term x two-term (the l * l term, about 2^-16 relative, is dropped)
__device__ __forceinline__ f4_t mm2_ss(const Split2 &a, const Split2 &b, f4_t c) {
  c = mfma_bf16(a.l, b.h, c);
  c = mfma_bf16(a.h, b.l, c);
  return mfma_bf16(a.h, b.h, c);
}
// ---- K = 16 products (v_mfma_f32_16x16x16_bf16, checked on the device): lane l supplies
// A[li][4 gq + e] and B[4 gq + e][li] (e < 4, two VGPRs each), D as above.  A D-layout tile is
// then directly the B operand of the next product over its 16 rows.
__device__ __forceinline__ f4_t mfma_bf16_k16(const uint2 &a, const uint2 &b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, a), __builtin_bit_cast(s4_t, b),
                                                   c, 0, 0, 0);
}
struct Split2h {
  uint2 h, l;
};
// an accumulator tile (4 values) as a two-term K = 16 operand
__device__ __forceinline__ Split2h split2_4h(const f4_t &v) {
  uint32_t a[2], b[2];
  split_pk<2>(v[0], v[1], a);
  split_pk<2>(v[2], v[3], b);
  return Split2h{make_uint2(a[0], b[0]), make_uint2(a[1], b[1])};
}
// four bf16 per term at p (term stride in elements)
__device__ __forceinline__ Split2h ld2_4h(const uint16_t *p, int term_stride) {
  return Split2h{*reinterpret_cast<const uint2 *>(p), *reinterpret_cast<const uint2 *>(p + term_stride)};
}
// A 16 x 16 tile stored transposed (Tt[col][row], row stride ld) as the two-term K = 16 A
// operand of lane (gq, li): M[li][4 gq + e] = Tt[4 gq + e][li], read with the transposing load.
__device__ __forceinline__ Split2h ld2_tr4h(const uint16_t *tt, int ld, int term_stride, int gq, int li) {
  const uint16_t *p = tt + (4 * gq + (li >> 2)) * ld + 4 * (li & 3);
  return Split2h{ld_tr4(p), ld_tr4(p + term_stride)};
}
// two-term x two-term over K = 16 (the l * l term dropped)
__device__ __forceinline__ f4_t mm2h_ss(const Split2h &a, const Split2h &b, f4_t c) {
  c = mfma_bf16_k16(a.l, b.h, c);
  c = mfma_bf16_k16(a.h, b.l, c);
  return mfma_bf16_k16(a.h, b.h, c);
}

// four bf16 at p0 and four at p1, or zeros for the second half
__device__ __forceinline__ bf16x8_t ld_bf4z(const uint16_t *p0) {
  const uint2 a = *reinterpret_cast<const uint2 *>(p0);
  return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, 0u, 0u));
}
__device__ __forceinline__ Split2 ld2_4x2(const uint16_t *p0, const uint16_t *p1, int term_stride) {
  return Split2{ld_bf4x2(p0, p1), ld_bf4x2(p0 + term_stride, p1 + term_stride)};
}
__device__ __forceinline__ Split2 ld2_4z(const uint16_t *p0, int term_stride) {
  return Split2{ld_bf4z(p0), ld_bf4z(p0 + term_stride)};
}


}  // namespace vla
