// Decode step (T = 1): one token per stream, the stream's state held in registers.
//
// A decode call reads the carried state (S and A, d x d fp32 each), advances it by one token
// and writes it back: per stream 16 d^2 bytes of HBM traffic for ~12 d^2 flops, so the call
// is bound by HBM bandwidth once there are enough streams, and by latency below that.  One
// workgroup of 512 threads (two waves per SIMD) takes one stream and touches each state
// element once: thread (i, p) = (tid / 16, tid % 16) owns rows i + 32 a (a < d / 32) and, in
// each, the column pairs 2 p + 32 b, 2 p + 32 b + 1 (b < d / 32), so that the 16 threads of a
// row read and write 128 contiguous bytes per instruction and a row's sums are 16-lane
// DPP sums.
// Per stream (VLA summary §2.3 steps 1-3 and the ratio readout, for one token):
//   z = A u,  g = A k,  delta = 1 + u.z,  A'[r][c] = A[r][c] - z_r z_c / delta
//   y = A' khat = (g - z (z.k) / delta) / ||k||,  ahat = y / ||y||
//   S'[r][:] = S[r][:] + (v_r - S[r][:] . khat) ahat^T
//   n' = n + phi(k),  o_r = S'[r][:] . phi(q) / (n'.phi(q) + eps)
// A carried A0 is used as (A0 + A0^T) / 2: the transposed element comes from a copy of A0
// in LDS.  Both halves of a pair add the same two numbers, and every lane holds bitwise the
// same z (symmetric DPP sums), so A' is exactly symmetric.

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

__device__ __forceinline__ float dec_wave_sum(float x) { return wave_sum(x); }
// over the 16 lanes of an aligned group (DPP; every lane of the group gets the same bits)
__device__ __forceinline__ float dec_sum16(float x) { return row_sum16(x); }

template <int D, typename TIn>
__global__ void __launch_bounds__(512)
vla_decode_kernel(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
                  const TIn *__restrict__ u, TIn *__restrict__ out, float *__restrict__ S_final,
                  float *__restrict__ A_final, const float *__restrict__ S0,
                  const float *__restrict__ A0, const float *__restrict__ n0,
                  float *__restrict__ n_final, float lambda0, float eps, int raw_gain) {
  constexpr int NT = 512, RG = NT / 16, R = D / RG, NB = D / 32, LDA = D + 1;
  static_assert(D % 32 == 0, "column pairs of 16 lanes cover whole 32-column blocks");
  __shared__ float As[D][LDA];
  __shared__ float sU[D], sK[D], sQ[D], sZ[D], sG[D], sY[D], sN[D];
  __shared__ float red[5];  // ||k||^2, u.z, z.k, n'.phi(q), ||y||^2
  const int64_t s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, i = tid >> 4, pj = tid & 15;
  const int64_t tok = s * D, base = s * D * D;  // this stream's token (T = 1) and state
  auto col = [&](int b, int e) { return 2 * pj + 32 * b + e; };

  // state loads first (the longest latency), then the token vectors
  float2 Ar[R][NB], Sr[R][NB];
  if (A0 != nullptr) {
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        Ar[a][b] = *reinterpret_cast<const float2 *>(A0 + base + (i + RG * a) * D + col(b, 0));
  }
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
      Sr[a][b] = S0 != nullptr
                     ? *reinterpret_cast<const float2 *>(S0 + base + (i + RG * a) * D + col(b, 0))
                     : make_float2(0.f, 0.f);
  float vr[R];
#pragma unroll
  for (int a = 0; a < R; ++a) vr[a] = ld_in(v, tok + i + RG * a);
  if (tid < D) {
    sU[tid] = ld_in(u, tok + tid);
    const float kk = ld_in(k, tok + tid);
    sK[tid] = kk;
    sQ[tid] = phi(ld_in(q, tok + tid));
    sN[tid] = (n0 != nullptr ? n0[s * D + tid] : 0.f) + phi(kk);
  }
  if (A0 != nullptr) {  // A <- (A0 + A0^T) / 2 through a copy in LDS
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        As[i + RG * a][col(b, 0)] = Ar[a][b].x;
        As[i + RG * a][col(b, 1)] = Ar[a][b].y;
      }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        Ar[a][b].x = 0.5f * (Ar[a][b].x + As[col(b, 0)][i + RG * a]);
        Ar[a][b].y = 0.5f * (Ar[a][b].y + As[col(b, 1)][i + RG * a]);
      }
  } else {
    const float il = 1.0f / lambda0;
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        Ar[a][b].x = (i + RG * a == col(b, 0)) ? il : 0.f;
        Ar[a][b].y = (i + RG * a == col(b, 1)) ? il : 0.f;
      }
  }
  __syncthreads();  // token vectors visible
  // row sums: z = A u, g = A k, S k (all lanes of a row end with the same value)
  float z[R], g[R], sk[R];
#pragma unroll
  for (int a = 0; a < R; ++a) {
    float za = 0.f, ga = 0.f, sa = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c0 = col(b, 0), c1 = col(b, 1);
      za = fmaf(Ar[a][b].y, sU[c1], fmaf(Ar[a][b].x, sU[c0], za));
      ga = fmaf(Ar[a][b].y, sK[c1], fmaf(Ar[a][b].x, sK[c0], ga));
      sa = fmaf(Sr[a][b].y, sK[c1], fmaf(Sr[a][b].x, sK[c0], sa));
    }
    z[a] = dec_sum16(za);
    g[a] = dec_sum16(ga);
    sk[a] = dec_sum16(sa);
  }
  if (pj == 0) {
#pragma unroll
    for (int a = 0; a < R; ++a) {
      sZ[i + RG * a] = z[a];
      sG[i + RG * a] = g[a];
    }
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
  // ahat = y * ry: the unit gain (0 for a zero y), or the raw gain y for the ablation
  const float ry = raw_gain ? 1.0f : (red[4] > 0.f ? rsqrtf(red[4]) : 0.f);
  const float rden = 1.0f / (red[3] + eps);
  // rows: A' and S', the readout
#pragma unroll
  for (int a = 0; a < R; ++a) {
    const int r = i + RG * a;
    const float ra = vr[a] - sk[a] * rk;
    float num = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c0 = col(b, 0), c1 = col(b, 1);
      float2 sn, an;
      sn.x = fmaf(ra, sY[c0] * ry, Sr[a][b].x);
      sn.y = fmaf(ra, sY[c1] * ry, Sr[a][b].y);
      num = fmaf(sn.y, sQ[c1], fmaf(sn.x, sQ[c0], num));
      an.x = Ar[a][b].x - z[a] * sZ[c0] / delta;
      an.y = Ar[a][b].y - z[a] * sZ[c1] / delta;
      if (S_final != nullptr) *reinterpret_cast<float2 *>(S_final + base + r * D + c0) = sn;
      if (A_final != nullptr) *reinterpret_cast<float2 *>(A_final + base + r * D + c0) = an;
    }
    num = dec_sum16(num);
    if (pj == 0) st_out(out, tok + r, num * rden);
  }
  if (n_final != nullptr && tid < D) n_final[s * D + tid] = sN[tid];
}

template <int D, typename TIn>
static hipError_t launch_decode_t(const Problem &p, const void *q, const void *k, const void *v,
                                  const void *u, void *out, const StateIO &st, hipStream_t stream) {
  if (p.streams > 0x7fffffff) return hipErrorInvalidValue;
  VLA_LAUNCH("vla_decode_kernel", (vla_decode_kernel<D, TIn>),
             dim3(static_cast<unsigned>(p.streams)), dim3(512), 0, stream,
             static_cast<const TIn *>(q), static_cast<const TIn *>(k), static_cast<const TIn *>(v),
             static_cast<const TIn *>(u), static_cast<TIn *>(out), st.S_final, st.A_final, st.S0,
             st.A0, st.n0, st.n_final, p.lambda0, p.eps, p.raw_gain ? 1 : 0);
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
