// Backward of the VLA recurrence (gradients of q, k, v, u and lambda0), gfx950.
//
// Forward per token (VLA summary §2.3 steps 1-3 and the ELU+1 ratio readout):
//   khat = k / ||k||, z = A u, delta = 1 + u.z, A' = A - z z^T / delta,
//   y = A' khat, ahat = y / ||y||, r = v - S khat, S' = S + r ahat^T,
//   n' = n + phi(k), o = S' phi(q) / (n'.phi(q) + eps)
// Reverse of one token, with the upstream gradients dS, dA (of the state after the token),
// dn and do:
//   dnum = do / den, dden = -(do.o) / den, dS += dnum phi(q)^T, dphi(q) = S'^T dnum + dden n',
//   dn += dden phi(q), dphi(k) = dn,
//   dr = dS ahat, dahat = dS^T r, dv = dr, dS -= dr khat^T, dkhat = -S^T dr (S before),
//   dy = (dahat - ahat (ahat.dahat)) / ||y||, dA += dy khat^T, dkhat += A' dy,
//   dz = -(dA + dA^T) z / delta + ddelta u, ddelta = z^T dA z / delta^2, du = ddelta z,
//   dA += dz u^T, du += A^T dz (A before; A is symmetric), dk += (dkhat - khat (khat.dkhat)) / ||k||
// dlambda0 uses the closed form A_t = (lambda0 I + sum_{s<=t} u_s u_s^T)^{-1} (Sherman-Morrison
// tracks it exactly, VLA summary §2.2), so dA_t / dlambda0 = -A_t^2 and lambda0 reaches the
// loss through y_t = A_t khat_t and the cotangent of A_T only:
//   dlambda0 = -sum_t (A_t dy_t) . y_t - <dA_T, A_T^2>
// Each term is weighted by A_t^2, which shrinks along the sequence; the equal quantity
// -tr(dA_0) / lambda0^2 of the reverse sweep is a small difference of large fp32 terms.
//
// One workgroup of 512 threads per stream.  Thread (i, p) = (tid / 16, tid % 16) holds rows
// i + 32 a and column pairs 2 p + 32 b of S, A, dS and dA in registers (the layout of the
// decode kernel), so row sums are 16-lane shuffles and column sums go through one LDS pass
// over the eight waves in a fixed order (deterministic).  A forward replay writes each
// token's vectors (khat, z, ahat, r, phi(q), o and four scalars) and the state after every
// 32nd token to the workspace; the reverse sweep undoes the rank-1 updates token by token
// (S -= r ahat^T, A += z z^T / delta) and reloads the exact state at every checkpoint, so
// rounding cannot drift over more than 32 steps.

#include "vla_common.h"
#include "vla_internal.h"

namespace vla {
namespace {

constexpr int BW_NT = 512;
constexpr int BW_CK = 32;  // tokens between state checkpoints
constexpr int BW_NS = 8;   // scalar slots per token record

template <int D>
struct BwCfg {
  static constexpr int RG = 32, R = D / RG, NB = D / 32, NW = BW_NT / kWave;
  static constexpr int REC = 6 * D + BW_NS;  // khat, z, ahat, r, phi(q), o, scalars
};

// Sum over each 16-lane row (DPP, no LDS round trip); every lane of the row gets the sum.
__device__ __forceinline__ float bw_sum16(float x) { return row_sum16(x); }
__device__ __forceinline__ float bw_wave_sum(float x) { return wave_sum(x); }
__device__ __forceinline__ float bw_cv(float x) { return x; }
__device__ __forceinline__ float bw_cv(bf16_t x) { return bf16_to_f32(x.bits); }
__device__ __forceinline__ float dphi(float x) { return x > 0.f ? 1.f : __expf(x); }

template <int D>
struct BwShared {
  float kr[D], u[D], v[D], fq[D], fk[D], n[D];  // raw k, u, v; phi(q), phi(k); normaliser
  float z[D], g[D], sk[D], y[D];                // forward vectors
  float kh[D], ah[D], r[D], o[D], dout[D], dnum[D], dah[D], dy[D], dkh[D], dz[D];
  float dr[D], ady[D], daz[D], datz[D], adz[D], dn[D];
  float part[2][BwCfg<D>::NW][D];
  float red[8];
  float sc[BW_NS];
};

template <int D, typename TIn>
__global__ void __launch_bounds__(BW_NT)
vla_backward_kernel(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
                    const TIn *__restrict__ u, const TIn *__restrict__ dout,
                    const float *__restrict__ dS_T, const float *__restrict__ dA_T,
                    const float *__restrict__ dn_T, float *__restrict__ dq, float *__restrict__ dk,
                    float *__restrict__ dv, float *__restrict__ du, float *__restrict__ dlambda0,
                    float *__restrict__ ws, int64_t T, float lambda0, float eps) {
  using C = BwCfg<D>;
  constexpr int R = C::R, NB = C::NB;
  __shared__ BwShared<D> sh;
  const int64_t s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = tid >> 4, pj = tid & 15;
  const int64_t NC = (T + BW_CK - 1) / BW_CK;
  float *rec0 = ws + s * (T * C::REC + NC * 2 * D * D);  // this stream's records
  float *ck0 = rec0 + T * C::REC;                        // then its checkpoints
  auto row = [&](int a) { return i + C::RG * a; };
  auto col = [&](int b, int e) { return 2 * pj + 32 * b + e; };
  // column sums over this thread's rows -> sh.part[slot][wave][c] (lanes 0..15 of a wave)
  auto col_part = [&](int slot, const float (&p)[NB][2]) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float x = p[b][e];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        if (lane < 16) sh.part[slot][w][col(b, e)] = x;
      }
  };
  auto col_total = [&](int slot, int c) {
    float x = 0.f;
#pragma unroll
    for (int ww = 0; ww < C::NW; ++ww) x += sh.part[slot][ww][c];
    return x;
  };

  float S[R][NB][2], A[R][NB][2];
  const float il = 1.0f / lambda0;
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        S[a][b][e] = 0.f;
        A[a][b][e] = row(a) == col(b, e) ? il : 0.f;
      }
  if (tid < D) sh.n[tid] = 0.f;

  // ---------------- forward replay: records and checkpoints ----------------
  // Token t + 1's inputs are loaded (raw, into registers) while token t is processed.
  TIn nk{}, nu{}, nv{}, nq{};
  if (tid < D) {
    const int64_t tok0 = s * T * D;
    nk = k[tok0 + tid]; nu = u[tok0 + tid]; nv = v[tok0 + tid]; nq = q[tok0 + tid];
  }
  for (int64_t t = 0; t < T; ++t) {
    const int64_t tok = (s * T + t) * D;
    if (tid < D) {
      const float kk = bw_cv(nk);
      sh.kr[tid] = kk;
      sh.u[tid] = bw_cv(nu);
      sh.v[tid] = bw_cv(nv);
      sh.fq[tid] = phi(bw_cv(nq));
      sh.fk[tid] = phi(kk);
      if (t + 1 < T) {
        nk = k[tok + D + tid]; nu = u[tok + D + tid]; nv = v[tok + D + tid]; nq = q[tok + D + tid];
      }
    }
    __syncthreads();
    float z[R], sk[R];
#pragma unroll
    for (int a = 0; a < R; ++a) {
      float zp = 0.f, gp = 0.f, sp = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int c = col(b, e);
          zp = fmaf(A[a][b][e], sh.u[c], zp);
          gp = fmaf(A[a][b][e], sh.kr[c], gp);
          sp = fmaf(S[a][b][e], sh.kr[c], sp);
        }
      z[a] = bw_sum16(zp);
      const float g = bw_sum16(gp);
      sk[a] = bw_sum16(sp);
      if (pj == 0) {
        sh.z[row(a)] = z[a];
        sh.g[row(a)] = g;
        sh.sk[row(a)] = sk[a];
      }
    }
    __syncthreads();
    if (w == 0) {
      float kk = 0.f, uz = 0.f, zk = 0.f, nq = 0.f;
      for (int c = lane; c < D; c += kWave) {
        kk = fmaf(sh.kr[c], sh.kr[c], kk);
        uz = fmaf(sh.u[c], sh.z[c], uz);
        zk = fmaf(sh.z[c], sh.kr[c], zk);
        nq = fmaf(sh.n[c] + sh.fk[c], sh.fq[c], nq);
      }
      kk = bw_wave_sum(kk); uz = bw_wave_sum(uz); zk = bw_wave_sum(zk); nq = bw_wave_sum(nq);
      if (lane == 0) { sh.red[0] = kk; sh.red[1] = uz; sh.red[2] = zk; sh.red[3] = nq; }
    }
    __syncthreads();
    const float delta = 1.0f + sh.red[1];
    const float rk = sh.red[0] > 0.f ? rsqrtf(sh.red[0]) : 0.f;
    const float czk = sh.red[2] / delta;
    const float den = sh.red[3] + eps;
    if (tid < D) {
      sh.y[tid] = (sh.g[tid] - sh.z[tid] * czk) * rk;
      sh.n[tid] += sh.fk[tid];
    }
    __syncthreads();
    if (w == 0) {
      float yy = 0.f;
      for (int c = lane; c < D; c += kWave) yy = fmaf(sh.y[c], sh.y[c], yy);
      yy = bw_wave_sum(yy);
      if (lane == 0) sh.red[4] = yy;
    }
    __syncthreads();
    const float ry = sh.red[4] > 0.f ? rsqrtf(sh.red[4]) : 0.f;
    float *rec = rec0 + t * C::REC;
#pragma unroll
    for (int a = 0; a < R; ++a) {
      const float ra = sh.v[row(a)] - sk[a] * rk;
      float np = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int c = col(b, e);
          A[a][b][e] -= z[a] * sh.z[c] / delta;
          S[a][b][e] = fmaf(ra, sh.y[c] * ry, S[a][b][e]);
          np = fmaf(S[a][b][e], sh.fq[c], np);
        }
      const float num = bw_sum16(np);
      if (pj == 0) {
        rec[3 * D + row(a)] = ra;          // r
        rec[5 * D + row(a)] = num / den;   // o
      }
    }
    if (tid < D) {
      rec[tid] = sh.kr[tid] * rk;          // khat
      rec[D + tid] = sh.z[tid];            // z
      rec[2 * D + tid] = sh.y[tid] * ry;   // ahat
      rec[4 * D + tid] = sh.fq[tid];       // phi(q)
    }
    if (tid == 0) {
      rec[6 * D + 0] = delta;
      rec[6 * D + 1] = sh.red[4] > 0.f ? sqrtf(sh.red[4]) : 0.f;  // ||y||
      rec[6 * D + 2] = rk;
      rec[6 * D + 3] = den;
    }
    if (t % BW_CK == BW_CK - 1 || t == T - 1) {
      float *ck = ck0 + (t / BW_CK) * 2 * D * D;
#pragma unroll
      for (int a = 0; a < R; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          *reinterpret_cast<float2 *>(ck + row(a) * D + col(b, 0)) = make_float2(S[a][b][0], S[a][b][1]);
          *reinterpret_cast<float2 *>(ck + D * D + row(a) * D + col(b, 0)) =
              make_float2(A[a][b][0], A[a][b][1]);
        }
    }
    __syncthreads();  // records and checkpoints are re-read by this workgroup's threads
  }
  __threadfence_block();

  // ---------------- reverse sweep ----------------
  float dS[R][NB][2], dA[R][NB][2];
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t off = s * D * D + row(a) * D + col(b, e);
        dS[a][b][e] = dS_T != nullptr ? dS_T[off] : 0.f;
        dA[a][b][e] = dA_T != nullptr ? dA_T[off] : 0.f;
      }
  if (tid < D) sh.dn[tid] = dn_T != nullptr ? dn_T[s * D + tid] : 0.f;
  double dlam = 0.0;  // -dL/dlambda0 accumulated by thread 0
  if (dlambda0 != nullptr && dA_T != nullptr) {
    // <dA_T, A_T^2> with A_T staged in LDS (A is symmetric: (A^2)[r][c] = sum_m A[r][m] A[c][m])
    __shared__ float As[D][D + 1];
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) As[row(a)][col(b, e)] = A[a][b][e];
    __syncthreads();
    float x = 0.f;
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float p2 = 0.f;
          for (int m = 0; m < D; ++m) p2 = fmaf(As[row(a)][m], As[col(b, e)][m], p2);
          x = fmaf(dA[a][b][e], p2, x);
        }
    x = bw_wave_sum(x);
    if (lane == 0) sh.red[w] = x;
    __syncthreads();
    if (tid == 0)
      for (int ww = 0; ww < C::NW; ++ww) dlam += static_cast<double>(sh.red[ww]);
    __syncthreads();
  }
  // Token t - 1's record and inputs are loaded (into registers) while token t is processed.
  float pr[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, psc = 0.f;
  TIn pk{}, pu{}, pdo{}, pq{};
  auto load_rev = [&](int64_t t) {
    const float *rec = rec0 + t * C::REC;
    const int64_t tok = (s * T + t) * D;
    if (tid < D) {
#pragma unroll
      for (int f = 0; f < 6; ++f) pr[f] = rec[f * D + tid];
      pk = k[tok + tid]; pu = u[tok + tid]; pdo = dout[tok + tid]; pq = q[tok + tid];
    }
    if (tid < BW_NS) psc = rec[6 * D + tid];
  };
  load_rev(T - 1);
  for (int64_t t = T - 1; t >= 0; --t) {
    const int64_t tok = (s * T + t) * D;
    if (t % BW_CK == BW_CK - 1 && t != T - 1) {  // exact state after token t
      const float *ck = ck0 + (t / BW_CK) * 2 * D * D;
#pragma unroll
      for (int a = 0; a < R; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float2 sv = *reinterpret_cast<const float2 *>(ck + row(a) * D + col(b, 0));
          const float2 av = *reinterpret_cast<const float2 *>(ck + D * D + row(a) * D + col(b, 0));
          S[a][b][0] = sv.x; S[a][b][1] = sv.y;
          A[a][b][0] = av.x; A[a][b][1] = av.y;
        }
    }
    float qt = 0.f;  // raw q of token t (for dq)
    if (tid < D) {
      sh.kh[tid] = pr[0];
      sh.z[tid] = pr[1];
      sh.ah[tid] = pr[2];
      sh.r[tid] = pr[3];
      sh.fq[tid] = pr[4];
      sh.o[tid] = pr[5];
      sh.kr[tid] = bw_cv(pk);
      sh.u[tid] = bw_cv(pu);
      sh.dout[tid] = bw_cv(pdo);
      qt = bw_cv(pq);
    }
    if (tid < BW_NS) sh.sc[tid] = psc;
    if (t > 0) load_rev(t - 1);
    __syncthreads();
    if (w == 0) {
      float x = 0.f;
      for (int c = lane; c < D; c += kWave) x = fmaf(sh.dout[c], sh.o[c], x);
      x = bw_wave_sum(x);
      if (lane == 0) sh.red[0] = x;
    }
    __syncthreads();
    const float delta = sh.sc[0], ynorm = sh.sc[1], rk = sh.sc[2], den = sh.sc[3];
    const float dden = -sh.red[0] / den;
    if (tid < D) sh.dnum[tid] = sh.dout[tid] / den;
    __syncthreads();
    // dS += dnum phi(q)^T; column sums S^T dnum and dS^T r; row sums dS ahat
    {
      float p1[NB][2], p2[NB][2];
#pragma unroll
      for (int b = 0; b < NB; ++b) p1[b][0] = p1[b][1] = p2[b][0] = p2[b][1] = 0.f;
#pragma unroll
      for (int a = 0; a < R; ++a) {
        const float dn_r = sh.dnum[row(a)], r_r = sh.r[row(a)];
        float rp = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int c = col(b, e);
            dS[a][b][e] = fmaf(dn_r, sh.fq[c], dS[a][b][e]);
            p1[b][e] = fmaf(S[a][b][e], dn_r, p1[b][e]);
            p2[b][e] = fmaf(dS[a][b][e], r_r, p2[b][e]);
            rp = fmaf(dS[a][b][e], sh.ah[c], rp);
          }
        const float dr = bw_sum16(rp);
        if (pj == 0) sh.dr[row(a)] = dr;
      }
      col_part(0, p1);
      col_part(1, p2);
    }
    __syncthreads();
    float dk_acc = 0.f, du_acc = 0.f;
    if (tid < D) {
      const float fqc = sh.fq[tid];
      const float dphiq = col_total(0, tid) + dden * sh.n[tid];
      dq[tok + tid] = dphiq * dphi(qt);
      sh.dah[tid] = col_total(1, tid);
      const float dnt = sh.dn[tid] + dden * fqc;  // gradient of n after token t
      sh.dn[tid] = dnt;
      dk_acc = dnt * dphi(sh.kr[tid]);
      dv[tok + tid] = sh.dr[tid];
    }
    __syncthreads();
    if (w == 0) {
      float x = 0.f;
      for (int c = lane; c < D; c += kWave) x = fmaf(sh.ah[c], sh.dah[c], x);
      x = bw_wave_sum(x);
      if (lane == 0) sh.red[1] = x;
    }
    __syncthreads();
    if (tid < D) sh.dy[tid] = ynorm > 0.f ? (sh.dah[tid] - sh.ah[tid] * sh.red[1]) / ynorm : 0.f;
    // S before the token, and dS -= dr khat^T
#pragma unroll
    for (int a = 0; a < R; ++a) {
      const float r_r = sh.r[row(a)], dr_r = sh.dr[row(a)];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int c = col(b, e);
          S[a][b][e] = fmaf(-r_r, sh.ah[c], S[a][b][e]);
          dS[a][b][e] = fmaf(-dr_r, sh.kh[c], dS[a][b][e]);
        }
    }
    __syncthreads();
    // dA += dy khat^T; row sums A dy and dA z; column sums S^T dr (S before) and dA^T z
    {
      float p1[NB][2], p2[NB][2];
#pragma unroll
      for (int b = 0; b < NB; ++b) p1[b][0] = p1[b][1] = p2[b][0] = p2[b][1] = 0.f;
#pragma unroll
      for (int a = 0; a < R; ++a) {
        const float dy_r = sh.dy[row(a)], dr_r = sh.dr[row(a)], z_r = sh.z[row(a)];
        float ap = 0.f, zp = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int c = col(b, e);
            dA[a][b][e] = fmaf(dy_r, sh.kh[c], dA[a][b][e]);
            ap = fmaf(A[a][b][e], sh.dy[c], ap);
            zp = fmaf(dA[a][b][e], sh.z[c], zp);
            p1[b][e] = fmaf(S[a][b][e], dr_r, p1[b][e]);
            p2[b][e] = fmaf(dA[a][b][e], z_r, p2[b][e]);
          }
        const float ady = bw_sum16(ap), daz = bw_sum16(zp);
        if (pj == 0) {
          sh.ady[row(a)] = ady;
          sh.daz[row(a)] = daz;
        }
      }
      col_part(0, p1);
      col_part(1, p2);
    }
    __syncthreads();
    if (tid < D) {
      sh.dkh[tid] = sh.ady[tid] - col_total(0, tid);
      sh.datz[tid] = col_total(1, tid);
    }
    __syncthreads();
    if (w == 0) {
      float zz = 0.f, kd = 0.f, ly = 0.f;
      for (int c = lane; c < D; c += kWave) {
        zz = fmaf(sh.z[c], sh.daz[c], zz);
        kd = fmaf(sh.kh[c], sh.dkh[c], kd);
        ly = fmaf(sh.ady[c], sh.ah[c], ly);  // (A_t dy) . ahat; y = ahat ||y||
      }
      zz = bw_wave_sum(zz);
      kd = bw_wave_sum(kd);
      ly = bw_wave_sum(ly);
      if (lane == 0) {
        sh.red[2] = zz;
        sh.red[3] = kd;
        dlam += static_cast<double>(ly) * ynorm;
      }
    }
    __syncthreads();
    const float ddelta = sh.red[2] / (delta * delta);
    if (tid < D) {
      sh.dz[tid] = -(sh.daz[tid] + sh.datz[tid]) / delta + ddelta * sh.u[tid];
      du_acc = ddelta * sh.z[tid];
      dk_acc += (sh.dkh[tid] - sh.kh[tid] * sh.red[3]) * rk;
    }
    __syncthreads();
    // A before the token; dA += dz u^T; row sums A dz (A before, symmetric)
#pragma unroll
    for (int a = 0; a < R; ++a) {
      const float z_r = sh.z[row(a)], dz_r = sh.dz[row(a)];
      float ap = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int c = col(b, e);
          A[a][b][e] += z_r * sh.z[c] / delta;
          dA[a][b][e] = fmaf(dz_r, sh.u[c], dA[a][b][e]);
          ap = fmaf(A[a][b][e], sh.dz[c], ap);
        }
      const float adz = bw_sum16(ap);
      if (pj == 0) sh.adz[row(a)] = adz;
    }
    __syncthreads();
    if (tid < D) {
      du[tok + tid] = du_acc + sh.adz[tid];
      dk[tok + tid] = dk_acc;
      sh.n[tid] -= phi(sh.kr[tid]);  // n before the token
    }
    __syncthreads();
  }
  if (dlambda0 != nullptr && tid == 0) dlambda0[s] = static_cast<float>(-dlam);
}

template <int D, typename TIn>
hipError_t launch_bw_t(const Problem &p, const BackwardIO &io, void *ws, hipStream_t st) {
  VLA_LAUNCH("vla_backward_kernel", (vla_backward_kernel<D, TIn>), dim3(static_cast<unsigned>(p.streams)),
             dim3(BW_NT), 0, st, static_cast<const TIn *>(io.q), static_cast<const TIn *>(io.k),
             static_cast<const TIn *>(io.v), static_cast<const TIn *>(io.u),
             static_cast<const TIn *>(io.dout), io.dS_T, io.dA_T, io.dn_T, io.dq, io.dk, io.dv, io.du,
             io.dlambda0, static_cast<float *>(ws), p.T, p.lambda0, p.eps);
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_bw_dt(const Problem &p, const BackwardIO &io, void *ws, hipStream_t st) {
  switch (p.d) {
    case 32: return launch_bw_t<32, TIn>(p, io, ws, st);
    case 64: return launch_bw_t<64, TIn>(p, io, ws, st);
    case 96: return launch_bw_t<96, TIn>(p, io, ws, st);
    case 128: return launch_bw_t<128, TIn>(p, io, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t backward_workspace_bytes(const Problem &p) {
  const int64_t NC = (p.T + BW_CK - 1) / BW_CK;
  const int64_t per = p.T * (6 * int64_t(p.d) + BW_NS) + NC * 2 * int64_t(p.d) * p.d;
  return static_cast<size_t>(p.streams * per) * sizeof(float);
}

hipError_t launch_backward(const Problem &p, const BackwardIO &io, void *ws, hipStream_t stream) {
  if (p.dtype == Dtype::F32) return launch_bw_dt<float>(p, io, ws, stream);
  return launch_bw_dt<bf16_t>(p, io, ws, stream);
}

}  // namespace vla
