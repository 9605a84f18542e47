// Decode step (T = 1): one token per stream, each stream's rows spread over workgroups.
//
// A decode call reads the carried state (S and A, d x d fp32 each) and writes it back.  With
// one workgroup per stream most of the chip idles while a few CUs wait on two d x d loads.
// Here workgroup (s, rt) owns rows 16 rt .. 16 rt + 15 of A and S of stream s.  It stages the
// whole (symmetrised) A of the stream in LDS, computes the stream-wide vectors redundantly
// with the other workgroups of the stream, and updates and writes only its own rows
// (VLA summary §2.3 steps 1-3 and the ratio readout, for one token):
//   z = A u,  delta = 1 + u.z,  A'[i][:] = A[i][:] - z_i z^T / delta
//   A' khat = (A k - z (z.k) / delta) / ||k||,  ahat = A' khat / ||A' khat||
//   S'[i][:] = S[i][:] + (v_i - S[i][:] . khat) ahat^T
//   n' = n + phi(k),  o_i = S'[i][:] . phi(q) / (n'.phi(q) + eps)
// Every workgroup of a stream computes delta and z identically and z_i z_j = z_j z_i, so
// the rows written by different workgroups keep A exactly symmetric.

#include "vla_common.h"
#include "vla_internal.h"

namespace vla {

template <typename TIn>
__device__ __forceinline__ float ld_in(const TIn *p, int64_t i);
template <>
__device__ __forceinline__ float ld_in<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_in<bf16_t>(const bf16_t *p, int64_t i) {
  return bf16_to_f32(p[i].bits);
}
template <typename TIn>
__device__ __forceinline__ void st_out(TIn *p, int64_t i, float x);
template <>
__device__ __forceinline__ void st_out<float>(float *p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void st_out<bf16_t>(bf16_t *p, int64_t i, float x) {
  p[i].bits = f32_to_bf16(x);
}

__device__ __forceinline__ float dec_wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float dec_sum16(float x) {  // over the 16 lanes of an aligned group
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D, typename TIn>
__global__ void __launch_bounds__(256)
vla_decode_kernel(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
                  const TIn *__restrict__ u, TIn *__restrict__ out, float *__restrict__ S_final,
                  float *__restrict__ A_final, const float *__restrict__ S0,
                  const float *__restrict__ A0, const float *__restrict__ n0,
                  float *__restrict__ n_final, float lambda0, float eps) {
  constexpr int NT = 256, LDA = D + 1, NM = D / 16;
  __shared__ float As[D][LDA];
  __shared__ float sU[D], sK[D], sQ[D], sZ[D], sG[D], sY[D], sN[D];
  __shared__ float red[5];  // ||k||^2, u.z, z.k, n'.phi(q), ||y||^2
  const int64_t s = blockIdx.x;
  const int rt = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tok = s * D;  // this stream's token (T = 1)

  // token vectors and n' = n + phi(k)
  if (tid < D) {
    sU[tid] = ld_in(u, tok + tid);
    const float kk = ld_in(k, tok + tid);
    sK[tid] = kk;
    sQ[tid] = phi(ld_in(q, tok + tid));
    sN[tid] = (n0 != nullptr ? n0[s * D + tid] : 0.f) + phi(kk);
  }
  // A, or I / lambda0
  if (A0 != nullptr) {
    const float *a = A0 + s * D * D;
    for (int e = tid; e < D * D; e += NT) As[e / D][e % D] = a[e];
  } else {
    const float il = 1.0f / lambda0;
    for (int e = tid; e < D * D; e += NT) As[e / D][e % D] = (e / D == e % D) ? il : 0.f;
  }
  // this workgroup's rows of S (row i = tid / 16, columns j = tid % 16 + 16 m)
  const int i = tid >> 4, pj = tid & 15, row = 16 * rt + i;
  float Srow[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) Srow[m] = S0 != nullptr ? S0[s * D * D + row * D + pj + 16 * m] : 0.f;
  const float vi = ld_in(v, tok + row);
  __syncthreads();
  if (A0 != nullptr) {  // (A0 + A0^T) / 2, each pair once
    for (int e = tid; e < D * D; e += NT) {
      const int r = e / D, c = e % D;
      if (r < c) {
        const float a = 0.5f * (As[r][c] + As[c][r]);
        As[r][c] = a;
        As[c][r] = a;
      }
    }
    __syncthreads();
  }
  // z = A u and g = A k
  if (tid < 2 * D) {
    const int r = tid < D ? tid : tid - D;
    const float *x = tid < D ? sU : sK;
    float acc = 0.f;
#pragma unroll 8
    for (int j = 0; j < D; ++j) acc = fmaf(As[r][j], x[j], acc);
    (tid < D ? sZ : sG)[r] = acc;
  }
  __syncthreads();
  if (wave == 0) {
    float kk = 0.f, uz = 0.f, zk = 0.f, nq = 0.f;
    for (int t = lane; t < D; t += 64) {
      kk = fmaf(sK[t], sK[t], kk);
      uz = fmaf(sU[t], sZ[t], uz);
      zk = fmaf(sZ[t], sK[t], zk);
      nq = fmaf(sN[t], sQ[t], nq);
    }
    kk = dec_wave_sum(kk); uz = dec_wave_sum(uz); zk = dec_wave_sum(zk); nq = dec_wave_sum(nq);
    if (lane == 0) { red[0] = kk; red[1] = uz; red[2] = zk; red[3] = nq; }
  }
  __syncthreads();
  const float delta = 1.0f + red[1];
  const float rk = red[0] > 0.f ? rsqrtf(red[0]) : 0.f;  // 1 / ||k||, 0 for a zero key
  const float czk = red[2] / delta;
  if (tid < D) sY[tid] = (sG[tid] - sZ[tid] * czk) * rk;  // A' khat
  __syncthreads();
  if (wave == 0) {
    float yy = 0.f;
    for (int t = lane; t < D; t += 64) yy = fmaf(sY[t], sY[t], yy);
    yy = dec_wave_sum(yy);
    if (lane == 0) red[4] = yy;
  }
  __syncthreads();
  const float ry = red[4] > 0.f ? rsqrtf(red[4]) : 0.f;  // ahat = y * ry, 0 for a zero gain
  // rows: A' and S', the readout
  float sk = 0.f;
#pragma unroll
  for (int m = 0; m < NM; ++m) sk = fmaf(Srow[m], sK[pj + 16 * m], sk);
  const float r_i = vi - dec_sum16(sk) * rk;
  float num = 0.f;
  const float zi = sZ[row];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int j = pj + 16 * m;
    const float sn = fmaf(r_i, sY[j] * ry, Srow[m]);
    num = fmaf(sn, sQ[j], num);
    if (S_final != nullptr) S_final[s * D * D + row * D + j] = sn;
    if (A_final != nullptr) A_final[s * D * D + row * D + j] = As[row][j] - zi * sZ[j] / delta;
  }
  num = dec_sum16(num);
  if (pj == 0) st_out(out, tok + row, num / (red[3] + eps));
  if (rt == 0 && n_final != nullptr && tid < D) n_final[s * D + tid] = sN[tid];
}

template <int D, typename TIn>
static hipError_t launch_decode_t(const Problem &p, const void *q, const void *k, const void *v,
                                  const void *u, void *out, const StateIO &st, hipStream_t stream) {
  VLA_LAUNCH("vla_decode_kernel", (vla_decode_kernel<D, TIn>),
             dim3(static_cast<unsigned>(p.streams), D / 16), dim3(256), 0, stream,
             static_cast<const TIn *>(q), static_cast<const TIn *>(k), static_cast<const TIn *>(v),
             static_cast<const TIn *>(u), static_cast<TIn *>(out), st.S_final, st.A_final, st.S0,
             st.A0, st.n0, st.n_final, p.lambda0, p.eps);
  return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_decode_dt(const Problem &p, const void *q, const void *k, const void *v,
                                   const void *u, void *out, const StateIO &st, hipStream_t stream) {
  switch (p.d) {
    case 32: return launch_decode_t<32, TIn>(p, q, k, v, u, out, st, stream);
    case 64: return launch_decode_t<64, TIn>(p, q, k, v, u, out, st, stream);
    case 96: return launch_decode_t<96, TIn>(p, q, k, v, u, out, st, stream);
    case 128: return launch_decode_t<128, TIn>(p, q, k, v, u, out, st, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const Problem &p, const void *q, const void *k, const void *v,
                         const void *u, void *out, const StateIO &st, hipStream_t stream) {
  if (p.T != 1) return hipErrorInvalidValue;
  if (p.dtype == Dtype::F32) return launch_decode_dt<float>(p, q, k, v, u, out, st, stream);
  return launch_decode_dt<bf16_t>(p, q, k, v, u, out, st, stream);
}

}  // namespace vla
