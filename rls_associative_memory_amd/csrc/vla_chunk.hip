// Chunked, time-segment-parallel VLA forward.
//
// "VLA summary" = the gist.science technical summary of "Variational Linear Attention:
// Stable Associative Memory for Long-Context Transformers".  The recurrence is that of
// §2.3 (steps 1-3 and the ELU+1 ratio readout); the summary names a parallel scan form
// (§2.4) without detail.  This file parallelises the recurrence over time with two facts
// that follow from §2.2-§2.3:
//   * A_t = (lambda0 I + sum_{s<=t} u_s u_s^T)^{-1} is a function of a prefix sum, so the
//     inverse penalty at the start of any segment is the inverse of lambda0 I plus the
//     Gram matrix of all earlier u (Sherman-Morrison, §2.2, maintains exactly this).
//   * S_t = S_{t-1}(I - khat ahat^T) + v ahat^T is affine in S_{t-1}, so a segment maps
//     its start state as S_end = S_start Pi + B, and the maps compose.
// Within a segment the S recurrence runs in chunks of C tokens in the WY / UT form
//   R = Vx - Kh X^T,  E = (I + tril-1(Kh ahat^T))^{-1} R,  X <- X + E^T ahat,
//   Num = Fq X_start^T + tril0(Fq ahat^T) E,
// whose rows e_j = v_j - S_{j-1} khat_j are exactly the sequential residuals.
//
// Passes (launched in order on one stream; every pass is parallel over (stream, segment)):
//   k_gram     Gram_p = U_p^T U_p (MFMA) and sum phi(k) per segment
//   k_prefix   exclusive prefix over segments in fp64: M_p = lambda0 I + sum_{p'<p} Gram
//   k_inv      A at each segment start = M_p^{-1} (in-place Gauss-Jordan, SPD, fp32)
//   k_aside    Sherman-Morrison token by token inside each segment (VGPR-resident A, one
//              wave per segment for d <= 96): gating vectors ahat_t, 1/||k_t|| and the
//              readout denominator n_t . phi(q_t) + eps
//   k_swy MAP  per segment, the affine map (Pi_p, B_p) as a 2d-row state in WY form (MFMA)
//   k_sprefix  S at every segment start: S_{p+1} = S_p Pi_p + B_p (MFMA)
//   k_swy FIN  per segment, the WY form again from the true start state: outputs, S_T
//
// MFMA (v_mfma_f32_16x16x4_f32) is used for the dense contractions only: the Gram, the
// chunk products of the WY form and the segment-map composition.

#include <algorithm>

#include "vla_common.h"
#include "vla_internal.h"
#include "vla_mfma.h"

namespace vla {

// ------------------------------------------------------------------------------------
// Plan and workspace layout
// ------------------------------------------------------------------------------------
struct ChunkPlan {
  int D = 0, C = 0;
  int64_t S = 0, T = 0, L = 0, P = 0;
  size_t off_m = 0, off_nk = 0, off_alpha = 0, off_rkden = 0, off_pib = 0, off_s0 = 0;
  size_t total = 0;
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static ChunkPlan make_plan(const Problem &p, int C) {
  ChunkPlan pl;
  pl.D = p.d;
  pl.C = C;
  pl.S = p.streams;
  pl.T = p.T;
  // Segment length: a power of two (>= 256, a multiple of C) sized so that all streams
  // together give about 2048 segments, capped so that P stays small enough to scan.
  const int64_t target = (p.streams * p.T + 2047) / 2048;
  int64_t L = 256;
  while (L < target && L < 8192) L *= 2;
  while ((p.T + L - 1) / L > 65535) L *= 2;
  if (L >= p.T) L = ((p.T + C - 1) / C) * C;
  pl.L = L;
  pl.P = (p.T + L - 1) / L;
  const size_t D = static_cast<size_t>(p.d);
  const size_t S = static_cast<size_t>(pl.S), P = static_cast<size_t>(pl.P);
  size_t off = 0;
  pl.off_m = off;     off = align256(off + S * P * D * D * 4);
  pl.off_nk = off;    off = align256(off + S * P * D * 4);
  pl.off_alpha = off; off = align256(off + S * static_cast<size_t>(pl.T) * D * 4);
  pl.off_rkden = off; off = align256(off + S * static_cast<size_t>(pl.T) * 2 * 4);
  pl.off_pib = off;   off = align256(off + S * P * 2 * D * D * 4);
  pl.off_s0 = off;    off = align256(off + S * P * D * D * 4);
  pl.total = off;
  return pl;
}

int chunk_default(const Problem &p) { return p.d > 96 ? 32 : 64; }

bool chunk_supported(const Problem &p, int chunk) {
  if (chunk != 16 && chunk != 32 && chunk != 64) return false;
  if (p.d > 96 && chunk > 32) return false;  // LDS budget of the WY kernel
  return p.d == 32 || p.d == 64 || p.d == 96 || p.d == 128;
}

size_t chunk_workspace_bytes(const Problem &p, int chunk) { return make_plan(p, chunk).total; }

// ------------------------------------------------------------------------------------
// Input staging helper: 16-byte vector of the input type -> fp32
// ------------------------------------------------------------------------------------
template <typename TIn>
__device__ __forceinline__ float load_elem(const TIn *p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<bf16_t>(const bf16_t *p, int64_t i) {
  return bf16_to_f32(p[i].bits);
}

template <typename TIn>
__device__ __forceinline__ void store_elem(TIn *p, int64_t i, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float *p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_elem<bf16_t>(bf16_t *p, int64_t i, float x) {
  p[i].bits = f32_to_bf16(x);
}

// ------------------------------------------------------------------------------------
// k_gram: Gram_p = sum_{t in segment p} u_t u_t^T, nk_p = sum phi(k_t)   (segments 0..P-2)
// ------------------------------------------------------------------------------------
template <int D, typename TIn>
__global__ void __launch_bounds__(256)
k_gram(const TIn *__restrict__ u, const TIn *__restrict__ k, float *__restrict__ M,
       float *__restrict__ nk, int64_t T, int64_t L, int64_t P) {
  constexpr int NT16 = D / 16;
  constexpr int NTILE = NT16 * (NT16 + 1) / 2;
  constexpr int TPW = (NTILE + 3) / 4;
  constexpr int TB = 64;
  constexpr int LDU = D + 4;
  __shared__ float sU[TB][LDU];

  const int64_t s = blockIdx.x;
  const int64_t p = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, gq = lane >> 4;
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const TIn *us = u + s * T * D;
  const TIn *ks = k + s * T * D;

  int ti_i[TPW], ti_j[TPW];
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    int t = wave + 4 * m, it = 0;
    while (t > it) { t -= it + 1; ++it; }
    ti_i[m] = it;
    ti_j[m] = t;
  }
  f4_t acc[TPW];
#pragma unroll
  for (int m = 0; m < TPW; ++m) acc[m] = f4_zero();
  float nka = 0.f;

  for (int64_t t0 = tb; t0 < te; t0 += TB) {
    const int nt = static_cast<int>(std::min<int64_t>(TB, te - t0));
    __syncthreads();
    for (int e = tid; e < TB * D; e += 256) {
      const int j = e / D, c = e % D;
      sU[j][c] = j < nt ? load_elem(us, (t0 + j) * D + c) : 0.f;
    }
    if (tid < D)
      for (int j = 0; j < nt; ++j) nka += phi(load_elem(ks, (t0 + j) * D + tid));
    __syncthreads();
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      if (wave + 4 * m < NTILE) {
        const int ci = 16 * ti_i[m] + li, cj = 16 * ti_j[m] + li;
#pragma unroll
        for (int kt = 0; kt < TB / 16; ++kt)
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const int tok = 16 * kt + 4 * gq + st;
            acc[m] = mfma_f32_16x16x4(sU[tok][ci], sU[tok][cj], acc[m]);
          }
      }
    }
  }
  float *Ms = M + (s * P + p) * D * D;
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    if (wave + 4 * m < NTILE) {
      const int it = ti_i[m], jt = ti_j[m];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * it + 4 * gq + r, j = 16 * jt + li;
        Ms[i * D + j] = acc[m][r];
        if (it != jt) Ms[j * D + i] = acc[m][r];
      }
    }
  }
  if (tid < D) nk[(s * P + p) * D + tid] = nka;
}

// ------------------------------------------------------------------------------------
// k_prefix: M_p <- lambda0 I + sum_{p' < p} Gram_p' (fp64 sums), nk_p <- sum_{p'<p} nk_p'
// ------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
k_prefix(float *__restrict__ M, float *__restrict__ nk, int64_t P, float lambda0) {
  const int64_t s = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  if (e < D * D) {
    const double diag = (e / D) == (e % D) ? static_cast<double>(lambda0) : 0.0;
    float *base = M + s * P * D * D + e;
    double acc = 0.0;
    for (int64_t p = 0; p < P; ++p) {
      const float g = (p + 1 < P) ? base[p * D * D] : 0.f;
      base[p * D * D] = static_cast<float>(acc + diag);
      acc += g;
    }
  }
  if (blockIdx.y == 0 && threadIdx.x < D) {
    float *base = nk + s * P * D + threadIdx.x;
    double acc = 0.0;
    for (int64_t p = 0; p < P; ++p) {
      const float g = (p + 1 < P) ? base[p * D] : 0.f;
      base[p * D] = static_cast<float>(acc);
      acc += g;
    }
  }
}

// ------------------------------------------------------------------------------------
// k_inv: M_p <- M_p^{-1} in place (Gauss-Jordan without pivoting; M_p is SPD), symmetrised
// ------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) k_inv(float *__restrict__ M, int64_t P) {
  __shared__ float a[D][D + 1];
  __shared__ float rowk[D], colk[D];
  const int64_t s = blockIdx.x, p = blockIdx.y;
  const int tid = threadIdx.x;
  float *base = M + (s * P + p) * D * D;
  for (int e = tid; e < D * D; e += 256) a[e / D][e % D] = base[e];
  for (int kk = 0; kk < D; ++kk) {
    __syncthreads();
    if (tid < D) {
      rowk[tid] = a[kk][tid];
      colk[tid] = a[tid][kk];
    }
    __syncthreads();
    const float piv = 1.0f / rowk[kk];
    for (int e = tid; e < D * D; e += 256) {
      const int i = e / D, j = e % D;
      if (i == kk)
        a[i][j] = (j == kk) ? piv : rowk[j] * piv;
      else if (j == kk)
        a[i][j] = -colk[i] * piv;
      else
        a[i][j] = fmaf(-colk[i] * piv, rowk[j], a[i][j]);
    }
  }
  __syncthreads();
  for (int e = tid; e < D * D; e += 256) {
    const int i = e / D, j = e % D;
    base[e] = 0.5f * (a[i][j] + a[j][i]);
  }
}

// ------------------------------------------------------------------------------------
// k_aside: per segment, Sherman-Morrison token by token from the segment-start A.
// Unit = the lanes that own one segment's A (one wave for d <= 96, two for d = 128).
// Lane l of a unit owns rows g + j*HALF (g = l >> 1) and column half h = l & 1.
// ------------------------------------------------------------------------------------
template <int D>
struct AsideCfg {
  static constexpr int NWA = (D > 96) ? 2 : 1;
  static constexpr int UPB = (D > 96) ? 1 : 4;
  static constexpr int NT = NWA * UPB * kWave;
  static constexpr int LA = NWA * kWave;
  static constexpr int HALF = LA / 2;
  static constexpr int CW = D / 2;
  static constexpr int RPL = D / HALF;
  static constexpr int CT = 16;
  static constexpr int NF = (D + LA - 1) / LA;  // normaliser features per lane
};

template <int NWA>
__device__ __forceinline__ void unit_sync() {
  if constexpr (NWA == 1) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

template <int D, typename TIn>
__global__ void __launch_bounds__(AsideCfg<D>::NT)
k_aside(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ u,
        const float *__restrict__ A0, const float *__restrict__ nk0, float *__restrict__ alpha,
        float *__restrict__ rkden, float *__restrict__ A_final, int64_t S, int64_t T,
        int64_t L, int64_t P, float eps) {
  using C = AsideCfg<D>;
  __shared__ __attribute__((aligned(16))) float sU[C::UPB][C::CT][D];
  __shared__ __attribute__((aligned(16))) float sK[C::UPB][C::CT][D];
  __shared__ __attribute__((aligned(16))) float sQ[C::UPB][C::CT][D];  // phi(q)
  __shared__ __attribute__((aligned(16))) float sW[C::UPB][D];
  __shared__ float sRed[2][C::NWA][2];
  __shared__ float sDen[C::NWA][C::CT];

  const int tid = threadIdx.x;
  const int unit_in_blk = tid / C::LA;
  const int lu = tid % C::LA;  // lane within the unit
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * C::UPB + unit_in_blk;
  if (unit >= S * P) return;  // whole unit (a single wave when UPB > 1) leaves together
  const int64_t s = unit / P, p = unit % P;
  const int h = lu & 1, g = lu >> 1, c0 = h * C::CW;
  const int wside = lu / kWave;
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const TIn *qs = q + s * T * D;
  const TIn *ks = k + s * T * D;
  const TIn *us = u + s * T * D;
  float *al = alpha + s * T * D;
  float *rd = rkden + s * T * 2;
  float(*U)[D] = sU[unit_in_blk];
  float(*K)[D] = sK[unit_in_blk];
  float(*Q)[D] = sQ[unit_in_blk];
  float *W = sW[unit_in_blk];

  float Mr[C::RPL][C::CW];
  const float *a0 = A0 + (s * P + p) * D * D;
#pragma unroll
  for (int r = 0; r < C::RPL; ++r) {
    const int row = g + r * C::HALF;
#pragma unroll
    for (int m = 0; m < C::CW / 4; ++m) {
      const float4 x = *reinterpret_cast<const float4 *>(&a0[row * D + c0 + 4 * m]);
      Mr[r][4 * m] = x.x; Mr[r][4 * m + 1] = x.y; Mr[r][4 * m + 2] = x.z; Mr[r][4 * m + 3] = x.w;
    }
  }
  float nrun[C::NF];
#pragma unroll
  for (int f = 0; f < C::NF; ++f) {
    const int feat = lu + f * C::LA;
    nrun[f] = feat < D ? nk0[(s * P + p) * D + feat] : 0.f;
  }

  for (int64_t t0 = tb; t0 < te; t0 += C::CT) {
    const int nt = static_cast<int>(std::min<int64_t>(C::CT, te - t0));
    unit_sync<C::NWA>();
    for (int e = lu; e < C::CT * D; e += C::LA) {
      const int j = e / D, c = e % D;
      const bool ok = j < nt;
      U[j][c] = ok ? load_elem(us, (t0 + j) * D + c) : 0.f;
      K[j][c] = ok ? load_elem(ks, (t0 + j) * D + c) : 0.f;
      Q[j][c] = ok ? phi(load_elem(qs, (t0 + j) * D + c)) : 0.f;
    }
    unit_sync<C::NWA>();
    // Readout denominators of the tile: n_t = n_{t-1} + phi(k_t), den_t = n_t . phi(q_t) + eps.
    {
      float part[C::CT];
#pragma unroll
      for (int j = 0; j < C::CT; ++j) {
        part[j] = 0.f;
        if (j < nt) {
#pragma unroll
          for (int f = 0; f < C::NF; ++f) {
            const int feat = lu + f * C::LA;
            if (feat < D) {
              nrun[f] += phi(K[j][feat]);
              part[j] = fmaf(nrun[f], Q[j][feat], part[j]);
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < C::CT; ++j) part[j] = wave_sum(part[j]);
      if constexpr (C::NWA > 1) {
        if ((lu & (kWave - 1)) == 0)
#pragma unroll
          for (int j = 0; j < C::CT; ++j) sDen[wside][j] = part[j];
        __syncthreads();
        if (lu == 0)
          for (int j = 0; j < nt; ++j) {
            float dsum = 0.f;
#pragma unroll
            for (int w = 0; w < C::NWA; ++w) dsum += sDen[w][j];
            rd[(t0 + j) * 2 + 1] = dsum + eps;
          }
      } else {
        if (lu == 0)
          for (int j = 0; j < nt; ++j) rd[(t0 + j) * 2 + 1] = part[j] + eps;
      }
    }
    // Sherman-Morrison token by token.
    for (int j = 0; j < nt; ++j) {
      float z[C::RPL], a[C::RPL];
#pragma unroll
      for (int r = 0; r < C::RPL; ++r) { z[r] = 0.f; a[r] = 0.f; }
      float kk = 0.f;
#pragma unroll
      for (int m = 0; m < C::CW / 4; ++m) {
        const float4 u4 = *reinterpret_cast<const float4 *>(&U[j][c0 + 4 * m]);
        const float4 k4 = *reinterpret_cast<const float4 *>(&K[j][c0 + 4 * m]);
        kk = fmaf(k4.x, k4.x, kk); kk = fmaf(k4.y, k4.y, kk);
        kk = fmaf(k4.z, k4.z, kk); kk = fmaf(k4.w, k4.w, kk);
#pragma unroll
        for (int r = 0; r < C::RPL; ++r) {
          z[r] = fmaf(Mr[r][4 * m + 0], u4.x, z[r]);
          a[r] = fmaf(Mr[r][4 * m + 0], k4.x, a[r]);
          z[r] = fmaf(Mr[r][4 * m + 1], u4.y, z[r]);
          a[r] = fmaf(Mr[r][4 * m + 1], k4.y, a[r]);
          z[r] = fmaf(Mr[r][4 * m + 2], u4.z, z[r]);
          a[r] = fmaf(Mr[r][4 * m + 2], k4.z, a[r]);
          z[r] = fmaf(Mr[r][4 * m + 3], u4.w, z[r]);
          a[r] = fmaf(Mr[r][4 * m + 3], k4.w, a[r]);
        }
      }
      kk = pair_sum(kk);
      const float rk = kk > 0.f ? rsqrtf(kk) : 0.f;
      float sd = 0.f, sg = 0.f;
#pragma unroll
      for (int r = 0; r < C::RPL; ++r) {
        const int row = g + r * C::HALF;
        z[r] = pair_sum(z[r]);
        a[r] = pair_sum(a[r]) * rk;
        sd = fmaf(U[j][row], z[r], sd);
        sg = fmaf(K[j][row] * rk, z[r], sg);
      }
      if (h) { sd = 0.f; sg = 0.f; }
      sd = wave_sum(sd);
      sg = wave_sum(sg);
      if constexpr (C::NWA > 1) {
        if ((lu & (kWave - 1)) == 0) { sRed[0][wside][0] = sd; sRed[0][wside][1] = sg; }
        __syncthreads();
        sd = 0.f; sg = 0.f;
#pragma unroll
        for (int w = 0; w < C::NWA; ++w) { sd += sRed[0][w][0]; sg += sRed[0][w][1]; }
      }
      const float delta = 1.0f + sd;
      const float cz = sg / delta;
      float y[C::RPL];
      float sy = 0.f;
#pragma unroll
      for (int r = 0; r < C::RPL; ++r) {
        y[r] = fmaf(-cz, z[r], a[r]);
        sy = fmaf(y[r], y[r], sy);
      }
      if (h) sy = 0.f;
      sy = wave_sum(sy);
      if constexpr (C::NWA > 1) {
        if ((lu & (kWave - 1)) == 0) sRed[1][wside][0] = sy;
        __syncthreads();
        sy = 0.f;
#pragma unroll
        for (int w = 0; w < C::NWA; ++w) sy += sRed[1][w][0];
      }
      const float inv = sy > 0.f ? rsqrtf(sy) : 0.f;
      const float rdl = rsqrtf(delta);
      const int64_t t = t0 + j;
      float w[C::RPL];
#pragma unroll
      for (int r = 0; r < C::RPL; ++r) {
        const int row = g + r * C::HALF;
        w[r] = z[r] * rdl;
        if (h == 0) {
          W[row] = w[r];
          al[t * D + row] = y[r] * inv;
        }
      }
      if (lu == 0) rd[t * 2] = rk;
      unit_sync<C::NWA>();
#pragma unroll
      for (int m = 0; m < C::CW / 4; ++m) {
        const float4 w4 = *reinterpret_cast<const float4 *>(&W[c0 + 4 * m]);
#pragma unroll
        for (int r = 0; r < C::RPL; ++r) {
          Mr[r][4 * m + 0] = fmaf(-w[r], w4.x, Mr[r][4 * m + 0]);
          Mr[r][4 * m + 1] = fmaf(-w[r], w4.y, Mr[r][4 * m + 1]);
          Mr[r][4 * m + 2] = fmaf(-w[r], w4.z, Mr[r][4 * m + 2]);
          Mr[r][4 * m + 3] = fmaf(-w[r], w4.w, Mr[r][4 * m + 3]);
        }
      }
      if constexpr (C::NWA > 1) __syncthreads();  // W is rewritten by the next token
    }
  }
  if (A_final != nullptr && p == P - 1) {
    float *dst = A_final + s * D * D;
#pragma unroll
    for (int r = 0; r < C::RPL; ++r) {
      const int row = g + r * C::HALF;
#pragma unroll
      for (int m = 0; m < C::CW / 4; ++m)
        *reinterpret_cast<float4 *>(&dst[row * D + c0 + 4 * m]) =
            make_float4(Mr[r][4 * m], Mr[r][4 * m + 1], Mr[r][4 * m + 2], Mr[r][4 * m + 3]);
    }
  }
}

// ------------------------------------------------------------------------------------
// k_swy: the S recurrence of one segment in WY form, one 16-row slice of the state per wave.
//   FINAL: state S (d rows) from the true segment start; writes outputs and S_T.
//   MAP:   state [Pi; B] (2d rows) from [I; 0]; writes the segment map.
// The state is held transposed (X^T, d x 16 per wave) in MFMA accumulators.
// ------------------------------------------------------------------------------------
template <int D, int CH, bool FINAL>
struct SwyCfg {
  static constexpr int ROWS = FINAL ? D : 2 * D;
  static constexpr int NWV = ROWS / 16;
  static constexpr int NT = NWV * kWave;
  static constexpr int NCT = CH / 16;   // 16-token tiles per chunk
  static constexpr int NFT = D / 16;    // 16-feature tiles
  static constexpr int NKT = NCT * (NCT + 1) / 2;
  static constexpr int LC = CH + 4;     // row stride of [feature][token] arrays
  static constexpr int LD = D + 4;      // row stride of [token][feature] arrays
};

template <int D, int CH, bool FINAL, typename TIn>
__global__ void __launch_bounds__((SwyCfg<D, CH, FINAL>::NT))
k_swy(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
      const float *__restrict__ alpha, const float *__restrict__ rkden,
      const float *__restrict__ s0, float *__restrict__ pib, TIn *__restrict__ out,
      float *__restrict__ S_final, int64_t T, int64_t L, int64_t P) {
  using C = SwyCfg<D, CH, FINAL>;
  __shared__ float KhT[D][C::LC];                 // khat^T
  __shared__ float AlT[D][C::LC];                 // ahat^T
  __shared__ float FqT[FINAL ? D : 1][C::LC];     // phi(q)^T
  __shared__ float Al[CH][C::LD];                 // ahat
  __shared__ float KaT[CH][C::LC];                // (strict lower of Kh ahat^T)^T
  __shared__ float QaT[FINAL ? CH : 1][C::LC];    // (lower of Fq ahat^T)^T
  __shared__ float InvT[C::NCT][16][20];          // diagonal-block inverses, transposed
  __shared__ float sDen[CH];

  const int64_t s = blockIdx.x, p = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, gq = lane >> 4;
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const TIn *ks = k + s * T * D;
  const TIn *vs = v + s * T * D;
  const TIn *qs = q + s * T * D;
  const float *als = alpha + s * T * D;
  const float *rds = rkden + s * T * 2;

  // This wave's 16 state rows.  MAP: waves [0, D/16) hold Pi rows, the rest B rows.
  const bool pi_rows = !FINAL && wave < D / 16;
  const int rowbase = 16 * (FINAL ? wave : (pi_rows ? wave : wave - D / 16));
  const bool has_v = FINAL || !pi_rows;

  f4_t X[C::NFT];
  if constexpr (FINAL) {
    const float *st = s0 + (s * P + p) * D * D;
#pragma unroll
    for (int ft = 0; ft < C::NFT; ++ft) {
      const float4 x = *reinterpret_cast<const float4 *>(&st[(rowbase + li) * D + 16 * ft + 4 * gq]);
      X[ft] = f4_t{x.x, x.y, x.z, x.w};
    }
  } else {
#pragma unroll
    for (int ft = 0; ft < C::NFT; ++ft)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        X[ft][r] = (pi_rows && rowbase + li == 16 * ft + 4 * gq + r) ? 1.f : 0.f;
  }

  for (int64_t c0 = tb; c0 < te; c0 += CH) {
    const int m = static_cast<int>(std::min<int64_t>(CH, te - c0));
    __syncthreads();
    // ---- stage the chunk ------------------------------------------------------------
    for (int e = tid; e < CH * D; e += C::NT) {
      const int c = e / D, f = e % D;
      const bool ok = c < m;
      const int64_t t = c0 + c;
      const float kh = ok ? load_elem(ks, t * D + f) * rds[t * 2] : 0.f;
      const float a = ok ? als[t * D + f] : 0.f;
      KhT[f][c] = kh;
      AlT[f][c] = a;
      Al[c][f] = a;
      if constexpr (FINAL) FqT[f][c] = ok ? phi(load_elem(qs, t * D + f)) : 0.f;
    }
    if constexpr (FINAL)
      for (int c = tid; c < CH; c += C::NT) sDen[c] = c < m ? rds[(c0 + c) * 2 + 1] : 1.f;
    __syncthreads();
    // ---- shared chunk products: Ka = strict-lower(Kh ahat^T), Qa = lower(Fq ahat^T) --
    for (int job = wave; job < (FINAL ? 2 : 1) * C::NKT; job += C::NWV) {
      const bool isq = job >= C::NKT;
      int t = isq ? job - C::NKT : job, ct = 0;
      while (t > ct) { t -= ct + 1; ++ct; }
      const int ct2 = t;
      f4_t acc = f4_zero();
#pragma unroll
      for (int kt = 0; kt < C::NFT; ++kt)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int f = 16 * kt + 4 * gq + st;
          const float aop = isq ? FqT[FINAL ? f : 0][16 * ct + li] : KhT[f][16 * ct + li];
          acc = mfma_f32_16x16x4(aop, AlT[f][16 * ct2 + li], acc);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * gq + r;
        float val = acc[r];
        if (ct == ct2 && (isq ? (li > i) : (li >= i))) val = 0.f;
        if (isq) {
          if constexpr (FINAL) QaT[16 * ct2 + li][16 * ct + i] = val;
        } else {
          KaT[16 * ct2 + li][16 * ct + i] = val;
        }
      }
    }
    __syncthreads();
    // ---- inverses of the unit-lower diagonal blocks of I + Ka -------------------------
    if (wave == 0 && lane < 16 * C::NCT) {
      const int b = lane >> 4, j = li;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int i2 = 0; i2 < i; ++i2) acc = fmaf(-KaT[16 * b + i2][16 * b + i], x[i2], acc);
        x[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) InvT[b][j][i] = x[i];
    }
    __syncthreads();
    // ---- this wave's rows -------------------------------------------------------------
    f4_t E[C::NCT];
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) {
      f4_t acc = f4_zero();
#pragma unroll
      for (int kt = 0; kt < C::NFT; ++kt)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          acc = mfma_f32_16x16x4(-KhT[16 * kt + 4 * gq + st][16 * ct + li], X[kt][st], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * ct + 4 * gq + r;
        if (has_v && c < m) acc[r] += load_elem(vs, (c0 + c) * D + rowbase + li);
      }
      E[ct] = acc;  // R for now
    }
    f4_t N[FINAL ? C::NCT : 1];
    if constexpr (FINAL) {
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct) {
        f4_t acc = f4_zero();
#pragma unroll
        for (int kt = 0; kt < C::NFT; ++kt)
#pragma unroll
          for (int st = 0; st < 4; ++st)
            acc = mfma_f32_16x16x4(FqT[16 * kt + 4 * gq + st][16 * ct + li], X[kt][st], acc);
        N[ct] = acc;
      }
    }
    // E = (I + Ka)^{-1} R by block forward substitution.
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) {
      f4_t acc = E[ct];
#pragma unroll
      for (int ct2 = 0; ct2 < ct; ++ct2)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          acc = mfma_f32_16x16x4(-KaT[16 * ct2 + 4 * gq + st][16 * ct + li], E[ct2][st], acc);
      f4_t e = f4_zero();
#pragma unroll
      for (int st = 0; st < 4; ++st) e = mfma_f32_16x16x4(InvT[ct][4 * gq + st][li], acc[st], e);
      E[ct] = e;
    }
    if constexpr (FINAL) {
      TIn *os = out + s * T * D;
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct) {
        f4_t acc = N[ct];
#pragma unroll
        for (int ct2 = 0; ct2 <= ct; ++ct2)
#pragma unroll
          for (int st = 0; st < 4; ++st)
            acc = mfma_f32_16x16x4(QaT[16 * ct2 + 4 * gq + st][16 * ct + li], E[ct2][st], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 16 * ct + 4 * gq + r;
          if (c < m) store_elem(os, (c0 + c) * D + rowbase + li, acc[r] / sDen[c]);
        }
      }
    }
    // X^T += ahat^T E.
#pragma unroll
    for (int ft = 0; ft < C::NFT; ++ft) {
      f4_t acc = X[ft];
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          acc = mfma_f32_16x16x4(Al[16 * ct + 4 * gq + st][16 * ft + li], E[ct][st], acc);
      X[ft] = acc;
    }
  }

  float *dst = nullptr;
  if constexpr (FINAL) {
    if (S_final != nullptr && p == P - 1) dst = S_final + s * D * D;
  } else {
    dst = pib + ((s * P + p) * 2 + (pi_rows ? 0 : 1)) * D * D;
  }
  if (dst != nullptr) {
#pragma unroll
    for (int ft = 0; ft < C::NFT; ++ft)
      *reinterpret_cast<float4 *>(&dst[(rowbase + li) * D + 16 * ft + 4 * gq]) =
          make_float4(X[ft][0], X[ft][1], X[ft][2], X[ft][3]);
  }
}

// ------------------------------------------------------------------------------------
// k_sprefix: S_0 = 0, S_{p+1} = S_p Pi_p + B_p; one wave per (stream, 16-row slice).
// ------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(64)
k_sprefix(const float *__restrict__ pib, float *__restrict__ s0, int64_t P) {
  constexpr int NFT = D / 16;
  const int64_t s = blockIdx.x;
  const int rowbase = 16 * blockIdx.y;
  const int lane = threadIdx.x, li = lane & 15, gq = lane >> 4;
  f4_t X[NFT];
#pragma unroll
  for (int ft = 0; ft < NFT; ++ft) X[ft] = f4_zero();
  float *out0 = s0 + s * P * D * D;
#pragma unroll
  for (int ft = 0; ft < NFT; ++ft)
    *reinterpret_cast<float4 *>(&out0[(rowbase + li) * D + 16 * ft + 4 * gq]) = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t p = 0; p + 1 < P; ++p) {
    const float *Pi = pib + (s * P + p) * 2 * D * D;
    const float *Bm = Pi + D * D;
    f4_t Y[NFT];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
      const float4 b = *reinterpret_cast<const float4 *>(&Bm[(rowbase + li) * D + 16 * ft + 4 * gq]);
      f4_t acc = f4_t{b.x, b.y, b.z, b.w};
#pragma unroll
      for (int kt = 0; kt < NFT; ++kt)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          acc = mfma_f32_16x16x4(Pi[(16 * kt + 4 * gq + st) * D + 16 * ft + li], X[kt][st], acc);
      Y[ft] = acc;
    }
    float *o = s0 + (s * P + p + 1) * D * D;
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
      X[ft] = Y[ft];
      *reinterpret_cast<float4 *>(&o[(rowbase + li) * D + 16 * ft + 4 * gq]) =
          make_float4(X[ft][0], X[ft][1], X[ft][2], X[ft][3]);
    }
  }
}

// ------------------------------------------------------------------------------------
// Host launch
// ------------------------------------------------------------------------------------
template <int D, int CH, typename TIn>
static hipError_t launch_chunk_t(const Problem &pr, const ChunkPlan &pl, const void *q,
                                 const void *k, const void *v, const void *u, void *out,
                                 float *S_final, float *A_final, char *ws, hipStream_t st) {
  const TIn *qq = static_cast<const TIn *>(q);
  const TIn *kk = static_cast<const TIn *>(k);
  const TIn *vv = static_cast<const TIn *>(v);
  const TIn *uu = static_cast<const TIn *>(u);
  TIn *oo = static_cast<TIn *>(out);
  float *Mw = reinterpret_cast<float *>(ws + pl.off_m);
  float *nkw = reinterpret_cast<float *>(ws + pl.off_nk);
  float *alw = reinterpret_cast<float *>(ws + pl.off_alpha);
  float *rdw = reinterpret_cast<float *>(ws + pl.off_rkden);
  float *pbw = reinterpret_cast<float *>(ws + pl.off_pib);
  float *s0w = reinterpret_cast<float *>(ws + pl.off_s0);
  const unsigned S = static_cast<unsigned>(pl.S), P = static_cast<unsigned>(pl.P);

  if (P > 1) {
    VLA_LAUNCH("k_gram", (k_gram<D, TIn>), dim3(S, P - 1), dim3(256), 0, st, uu, kk, Mw, nkw,
                       pl.T, pl.L, pl.P);
  }
  VLA_LAUNCH("k_prefix", (k_prefix<D>), dim3(S, (D * D + 255) / 256), dim3(256), 0, st, Mw, nkw,
                     pl.P, pr.lambda0);
  VLA_LAUNCH("k_inv", (k_inv<D>), dim3(S, P), dim3(256), 0, st, Mw, pl.P);
  {
    using AC = AsideCfg<D>;
    const int64_t units = pl.S * pl.P;
    const unsigned blocks = static_cast<unsigned>((units + AC::UPB - 1) / AC::UPB);
    VLA_LAUNCH("k_aside", (k_aside<D, TIn>), dim3(blocks), dim3(AC::NT), 0, st, qq, kk, uu, Mw,
                       nkw, alw, rdw, A_final, pl.S, pl.T, pl.L, pl.P, pr.eps);
  }
  if (P > 1) {
    VLA_LAUNCH("k_swy_map", (k_swy<D, CH, false, TIn>), dim3(S, P - 1),
                       dim3(SwyCfg<D, CH, false>::NT), 0, st, qq, kk, vv, alw, rdw, s0w, pbw,
                       oo, S_final, pl.T, pl.L, pl.P);
  }
  VLA_LAUNCH("k_sprefix", (k_sprefix<D>), dim3(S, D / 16), dim3(64), 0, st, pbw, s0w, pl.P);
  VLA_LAUNCH("k_swy_final", (k_swy<D, CH, true, TIn>), dim3(S, P), dim3(SwyCfg<D, CH, true>::NT), 0,
                     st, qq, kk, vv, alw, rdw, s0w, pbw, oo, S_final, pl.T, pl.L, pl.P);
  return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_chunk_dt(const Problem &pr, const ChunkPlan &pl, const void *q,
                                  const void *k, const void *v, const void *u, void *out,
                                  float *S_final, float *A_final, char *ws, hipStream_t st) {
#define VLA_CASE(DD, CC)                                                                      \
  if (pr.d == DD && pl.C == CC)                                                              \
    return launch_chunk_t<DD, CC, TIn>(pr, pl, q, k, v, u, out, S_final, A_final, ws, st);
  VLA_CASE(32, 16) VLA_CASE(32, 32) VLA_CASE(32, 64)
  VLA_CASE(64, 16) VLA_CASE(64, 32) VLA_CASE(64, 64)
  VLA_CASE(96, 16) VLA_CASE(96, 32) VLA_CASE(96, 64)
  VLA_CASE(128, 16) VLA_CASE(128, 32)
#undef VLA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_chunk(const Problem &p, int chunk, const void *q, const void *k,
                        const void *v, const void *u, void *out, float *S_final,
                        float *A_final, void *ws, hipStream_t stream) {
  if (!chunk_supported(p, chunk)) return hipErrorInvalidValue;
  const ChunkPlan pl = make_plan(p, chunk);
  char *w = static_cast<char *>(ws);
  if (p.dtype == Dtype::F32)
    return launch_chunk_dt<float>(p, pl, q, k, v, u, out, S_final, A_final, w, stream);
  return launch_chunk_dt<bf16_t>(p, pl, q, k, v, u, out, S_final, A_final, w, stream);
}

}  // namespace vla
