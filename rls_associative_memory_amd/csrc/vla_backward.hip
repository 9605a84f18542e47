// Backward of the VLA recurrence (gradients of q, k, v, u and lambda0), gfx950.
//
// Forward per token (VLA summary §2.3 steps 1-3 and the ELU+1 ratio readout):
//   khat = k / ||k||, z = A u, delta = 1 + u.z, A' = A - z z^T / delta,
//   y = A' khat, ahat = y / ||y||, r = v - S khat, S' = S + r ahat^T,
//   n' = n + phi(k), o = S' phi(q) / (n'.phi(q) + eps)
// Reverse of one token, with the cotangents dS, dn of the state after the token and do:
//   dnum = do / den, dden = -(do.o) / den, dS += dnum phi(q)^T, dphi(q) = S'^T dnum + dden n',
//   dn += dden phi(q), dphi(k) = dn,
//   dr = dS ahat, dahat = dS^T r, dv = dr, dS -= dr khat^T, dkhat = -S^T dr (S before),
//   dy = (dahat - ahat (ahat.dahat)) / ||y||, w = A' dy, dkhat += w,
//   dk = (dkhat - khat (khat.dkhat)) / ||k|| + dn phi'(k).
// The inverse penalty needs no cotangent of its own.  Sherman-Morrison keeps
// A_t = (lambda0 I + sum_{s<=t} u_s u_s^T)^{-1} exactly (VLA summary §2.2), and A_t reaches the
// loss only through y_t = A_t khat_t and the final state.  With dA_t/dX = -A_t (dX) A_t for
// X = lambda0 I + sum u u^T, the cotangent of u_s and of lambda0 collapse to
//   du_s = -2 R_s u_s,    dlambda0 = -tr R_0,
//   R_s = sum_{t>=s} (w_t y_t^T + y_t w_t^T) / 2 + A_T sym(dA_T) A_T,   w_t = A_t dy_t,
// a suffix sum of rank-2 terms (the step-by-step adjoint of the Sherman-Morrison update gives
// the same values; only the symmetric part of a cotangent of A reaches u or lambda0).
//
// Time segments.  dS obeys dS_{t-1} = (dS_t + dnum_t phi(q_t)^T)(I - ahat_t khat_t^T), affine in
// dS_t with coefficients the forward fixes, so a segment maps the cotangent at its end E to the
// one at its start as  E Lmap + Bmap  (Lmap = the segment's forward map, transposed), and the
// maps compose; dn is a suffix sum and so is R.  Passes, every one parallel over (stream,
// segment) except the two scans:
//   (chunked forward passes, or k_bw_replay with one segment per stream: the per-token
//    vectors and the state at every 64th token and at every segment's last)
//   k_bw_dsmap    per segment from the end: (Lmap, Bmap) and the segment's sum of dden phi(q)
//   scan          dS and dn at every segment end (reverse order, so the forward scan applies)
//   k_bw_esweep   per segment from the end, the true dS: dr_t = dv_t token by token, and the
//                 S cotangent at every 32nd token
//   k_bw_cgrad    per segment, 32-token chunks from the end, on the fp32 matrix cores: dq, dk,
//                 du with R local to the segment, the segment's R sum and its trace
//   scan          R at every segment end (suffix sums, the final-state term first)
//   k_bw_fix      du_t -= 2 R_end u_t over each segment's tokens
//   k_bw_lambda   dlambda0 = -(tr of every segment's R sum + tr of the final-state term)
// With one segment per stream the pipeline is replay, sweep, chunked pass (R starting from the
// final-state term) and lambda.
//
// Layout of the per-token kernels: one workgroup of 512 threads per segment.  Thread (i, p) =
// (tid / 16, tid % 16) holds rows i + 32 a and column pairs 2 p + 32 b of each d x d matrix in
// registers, so row sums are 16-lane shuffles and column sums go through one LDS pass over the
// eight waves in a fixed order (deterministic).

#include <algorithm>

#include "vla_common.h"
#include "vla_internal.h"
#include "vla_mfma.h"

namespace vla {
namespace {

constexpr int BW_NT = 512;
constexpr int BW_NW = BW_NT / kWave;
constexpr int BW_CK = kBwCk;       // tokens between state checkpoints
constexpr int BW_NS = kBwScalars;  // scalar slots per token record
constexpr int BW_CC = 32;          // tokens per chunk of the chunked gradient pass

template <int D>
struct BwCfg {
  static constexpr int R = D / 32, NB = D / 32;
  static constexpr int REC = BwRec<D>::F;  // z, ahat, r, o, scalars
};

__device__ __forceinline__ float bw_cv(float x) { return x; }
__device__ __forceinline__ float bw_cv(bf16_t x) { return bf16_to_f32(x.bits); }
__device__ __forceinline__ float dphi(float x) { return x > 0.f ? 1.f : __expf(x); }

// Sum over the block's d-vector x . y of LDS arrays, computed redundantly by every wave (no
// barrier, the same value in every lane of every wave).
template <int D>
__device__ __forceinline__ float bw_dot(const float *x, const float *y, int lane) {
  float a = 0.f;
#pragma unroll
  for (int c = lane; c < D; c += kWave) a = fmaf(x[c], y[c], a);
  return wave_sum(a);
}

// ---------------------------------------------------------------------------------------------
// k_bw_replay: the forward over segment p from its start state (S0seg, A0seg, n0seg at
// [stream][P]; NULL = the fixed start S = 0, A = I / lambda0, n = 0).  Writes each token's
// record (z, ahat, r, o, delta, ||y||, 1/||k||, den) and the state (S, A) after
// every 64th token and after the segment's last token, and n after the segment.
// ---------------------------------------------------------------------------------------------
template <int D>
struct BwRepShared {
  float kr[D], u[D], v[D], fq[D], fk[D], n[D];
  float z[D], g[D], sk[D], y[D];
  float yy[BW_NW];
};

template <int D, typename TIn>
__global__ void __launch_bounds__(BW_NT)
k_bw_replay(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
            const TIn *__restrict__ u, const float *__restrict__ S0seg,
            const float *__restrict__ A0seg, const float *__restrict__ n0seg,
            float *__restrict__ recs, float *__restrict__ cks, float *__restrict__ n_end,
            int64_t T, int64_t L, int64_t P, float lambda0, float eps) {
  using C = BwCfg<D>;
  constexpr int R = C::R, NB = C::NB;
  __shared__ BwRepShared<D> sh;
  const int64_t s = blockIdx.x, p = blockIdx.y;
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = tid >> 4, pj = tid & 15;
  const int64_t NC = (T + BW_CK - 1) / BW_CK;
  float *rec0 = recs + s * T * C::REC;
  float *ck0 = cks + s * NC * 2 * D * D;
  auto row = [&](int a) { return i + 32 * a; };
  auto col = [&](int b, int e) { return 2 * pj + 32 * b + e; };

  float S[R][NB][2], A[R][NB][2];
  if (S0seg != nullptr) {
    const float *s0 = S0seg + (s * P + p) * D * D, *a0 = A0seg + (s * P + p) * D * D;
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float2 sv = *reinterpret_cast<const float2 *>(s0 + row(a) * D + col(b, 0));
        const float2 av = *reinterpret_cast<const float2 *>(a0 + row(a) * D + col(b, 0));
        S[a][b][0] = sv.x; S[a][b][1] = sv.y;
        A[a][b][0] = av.x; A[a][b][1] = av.y;
      }
  } else {
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
  }
  if (tid < D) sh.n[tid] = n0seg != nullptr ? n0seg[(s * P + p) * D + tid] : 0.f;

  // Token t + 1's inputs are loaded (raw, into registers) while token t is processed.
  TIn nk{}, nu{}, nv{}, nq{};
  if (tid < D) {
    const int64_t tok0 = (s * T + tb) * D;
    nk = k[tok0 + tid]; nu = u[tok0 + tid]; nv = v[tok0 + tid]; nq = q[tok0 + tid];
  }
  for (int64_t t = tb; t < te; ++t) {
    const int64_t tok = (s * T + t) * D;
    if (tid < D) {
      const float kk = bw_cv(nk);
      sh.kr[tid] = kk;
      sh.u[tid] = bw_cv(nu);
      sh.v[tid] = bw_cv(nv);
      sh.fq[tid] = phi(bw_cv(nq));
      sh.fk[tid] = phi(kk);
      if (t + 1 < te) {
        nk = k[tok + D + tid]; nu = u[tok + D + tid]; nv = v[tok + D + tid]; nq = q[tok + D + tid];
      }
    }
    __syncthreads();
    float z[R], sk[R];
    {
      float rs[3 * R];  // row sums of A u, A k, S k for every row of this thread
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
        rs[3 * a] = zp;
        rs[3 * a + 1] = gp;
        rs[3 * a + 2] = sp;
      }
      row_sum16_n(rs);
#pragma unroll
      for (int a = 0; a < R; ++a) {
        z[a] = rs[3 * a];
        sk[a] = rs[3 * a + 2];
      }
      if (pj == 0)
#pragma unroll
        for (int a = 0; a < R; ++a) {
          sh.z[row(a)] = rs[3 * a];
          sh.g[row(a)] = rs[3 * a + 1];
          sh.sk[row(a)] = rs[3 * a + 2];
        }
    }
    __syncthreads();
    // every wave forms the token's scalars itself (no further barrier)
    const float kk = bw_dot<D>(sh.kr, sh.kr, lane);
    const float uz = bw_dot<D>(sh.u, sh.z, lane);
    const float zk = bw_dot<D>(sh.z, sh.kr, lane);
    float nq = 0.f;
    for (int c = lane; c < D; c += kWave) nq = fmaf(sh.n[c] + sh.fk[c], sh.fq[c], nq);
    nq = wave_sum(nq);
    const float delta = 1.0f + uz;
    const float rk = kk > 0.f ? rsqrtf(kk) : 0.f;
    const float czk = zk / delta;
    const float den = nq + eps;
    // y = A' khat for this thread's rows, ||y||^2 from row-owner partial sums
    float yr[R];
    float yyp = 0.f;
#pragma unroll
    for (int a = 0; a < R; ++a) {
      yr[a] = (sh.g[row(a)] - z[a] * czk) * rk;
      if (pj == 0) yyp = fmaf(yr[a], yr[a], yyp);
    }
    yyp = wave_sum(yyp);
    if (lane == 0) sh.yy[w] = yyp;
    if (pj == 0)
#pragma unroll
      for (int a = 0; a < R; ++a) sh.y[row(a)] = yr[a];
    __syncthreads();
    float yy = 0.f;
#pragma unroll
    for (int ww = 0; ww < BW_NW; ++ww) yy += sh.yy[ww];
    const float ry = yy > 0.f ? rsqrtf(yy) : 0.f;
    float *rec = rec0 + t * C::REC;
    // A' = A - s s^T with s = z / sqrt(delta): one division per token, and entry (i, j) takes
    // the same product s_i s_j as entry (j, i), so A stays exactly symmetric
    const float rsd = 1.0f / sqrtf(delta);
    float sc[NB][2];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 2; ++e) sc[b][e] = sh.z[col(b, e)] * rsd;
    float ra[R], np[R];
#pragma unroll
    for (int a = 0; a < R; ++a) {
      ra[a] = sh.v[row(a)] - sk[a] * rk;
      const float sa = z[a] * rsd;
      np[a] = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int c = col(b, e);
          A[a][b][e] = fmaf(-sa, sc[b][e], A[a][b][e]);
          S[a][b][e] = fmaf(ra[a], sh.y[c] * ry, S[a][b][e]);
          np[a] = fmaf(S[a][b][e], sh.fq[c], np[a]);
        }
    }
    row_sum16_n(np);
    if (pj == 0) {
      const float rden = 1.0f / den;
#pragma unroll
      for (int a = 0; a < R; ++a) {
        rec[BwRec<D>::R + row(a)] = ra[a];
        rec[BwRec<D>::O + row(a)] = np[a] * rden;
      }
    }
    if (tid < D) {
      rec[BwRec<D>::Z + tid] = sh.z[tid];
      rec[BwRec<D>::AH + tid] = sh.y[tid] * ry;
      sh.n[tid] += sh.fk[tid];             // only this thread reads n[tid] until the barrier
    }
    if (tid == 0) {
      rec[BwRec<D>::SC + 0] = delta;
      rec[BwRec<D>::SC + 1] = yy > 0.f ? sqrtf(yy) : 0.f;  // ||y||
      rec[BwRec<D>::SC + 2] = rk;
      rec[BwRec<D>::SC + 3] = den;
    }
    if (t % BW_CK == BW_CK - 1 || t == te - 1) {
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
    __syncthreads();
  }
  if (tid < D) n_end[(s * P + p) * D + tid] = sh.n[tid];
}

// ---------------------------------------------------------------------------------------------
// k_bw_dsmap: segment p = blockIdx.y + 1 (the first segment's map is never needed) from its end
// with the cotangent E at the end left symbolic: E_start = E Lmap + Bmap.  Lmap, the product of
// (I - ahat_t khat_t^T) from the last token down, is the transpose of the forward's segment map
// Pi_p (the product of (I - khat_t ahat_t^T) in token order), which the chunked forward's map
// pass left in fpm ([stream][P][2][d][d], Pi_p first); Bmap is that recursion from 0 with the
// readout terms, token by token (rows independent).  Written to slot P - 1 - p of lb
// ([stream][P][2][d][d]: Lmap, Bmap) and nd ([stream][P][d]: the segment's sum of dden phi(q)),
// so that the forward scans, run over the slots, give the cotangents at every segment end.
// ---------------------------------------------------------------------------------------------
template <int D>
struct BwMapShared {
  float kh[2][D], ah[2][D], fq[2][D], dnum[2][D], x[2][D];
};

template <int D, typename TIn>
__global__ void __launch_bounds__(BW_NT)
k_bw_dsmap(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ dout,
           const float *__restrict__ recs, const float *__restrict__ fpm, float *__restrict__ lb,
           float *__restrict__ nd, int64_t T, int64_t L, int64_t P) {
  using C = BwCfg<D>;
  constexpr int R = C::R, NB = C::NB;
  __shared__ BwMapShared<D> sh;
  const int64_t s = blockIdx.x, p = blockIdx.y + 1;
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const int tid = threadIdx.x, lane = tid & 63, i = tid >> 4, pj = tid & 15;
  const float *rec0 = recs + s * T * C::REC;
  auto row = [&](int a) { return i + 32 * a; };
  auto col = [&](int b, int e) { return 2 * pj + 32 * b + e; };

  const int64_t slot = s * P + (P - 1 - p);
  {  // Lmap = Pi_p^T
    const float *pi = fpm + (s * P + p) * 2 * D * D;
    float *dst = lb + slot * 2 * D * D;
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        *reinterpret_cast<float2 *>(dst + row(a) * D + col(b, 0)) =
            make_float2(pi[col(b, 0) * D + row(a)], pi[col(b, 1) * D + row(a)]);
  }
  float Bm[R][NB][2];
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 2; ++e) Bm[a][b][e] = 0.f;
  float ndp = 0.f;  // thread f < d: sum of dden phi(q)_f

  // token t - 1's record is loaded while token t is processed
  float pa = 0.f, po = 0.f, prk = 0.f, pden = 1.f;
  TIn pdo{}, pkr{}, pq{};
  auto load = [&](int64_t t) {
    const float *rec = rec0 + t * C::REC;
    const int64_t tok = (s * T + t) * D;
    if (tid < D) {
      pa = rec[BwRec<D>::AH + tid];
      po = rec[BwRec<D>::O + tid];
      pdo = dout[tok + tid];
      pkr = k[tok + tid];
      pq = q[tok + tid];
    }
    prk = rec[BwRec<D>::SC + 2];
    pden = rec[BwRec<D>::SC + 3];
  };
  load(te - 1);
  for (int64_t t = te - 1; t >= tb; --t) {
    const int buf = static_cast<int>(t & 1);
    // Double-buffered staging: a thread writes this token's buffer only after the previous
    // token's barrier, past which nobody reads the buffer two tokens back.
    if (tid < D) {
      const float dd = bw_cv(pdo);
      sh.kh[buf][tid] = bw_cv(pkr) * prk;  // khat and phi(q) as the forward formed them
      sh.ah[buf][tid] = pa;
      sh.fq[buf][tid] = phi(bw_cv(pq));
      sh.dnum[buf][tid] = dd / pden;
      sh.x[buf][tid] = dd * po;
    }
    const float den = pden;
    if (t > tb) load(t - 1);
    __syncthreads();
    if (tid < (D + kWave - 1) / kWave * kWave) {  // the waves that hold n's features (uniform)
      float xo = 0.f;
      for (int c = lane; c < D; c += kWave) xo += sh.x[buf][c];
      xo = wave_sum(xo);
      if (tid < D) ndp = fmaf(-xo / den, sh.fq[buf][tid], ndp);
    }
    float bl[R];  // row sums of B ahat for every row of this thread
#pragma unroll
    for (int a = 0; a < R; ++a) {
      const float dn_r = sh.dnum[buf][row(a)];
      float bp = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int c = col(b, e);
          Bm[a][b][e] = fmaf(dn_r, sh.fq[buf][c], Bm[a][b][e]);
          bp = fmaf(Bm[a][b][e], sh.ah[buf][c], bp);
        }
      bl[a] = bp;
    }
    row_sum16_n(bl);
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) Bm[a][b][e] = fmaf(-bl[a], sh.kh[buf][col(b, e)], Bm[a][b][e]);
  }
  float *dst = lb + slot * 2 * D * D;
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
      *reinterpret_cast<float2 *>(dst + D * D + row(a) * D + col(b, 0)) = make_float2(Bm[a][b][0], Bm[a][b][1]);
  if (tid < D) nd[slot * D + tid] = ndp;
}

// ---------------------------------------------------------------------------------------------
// k_bw_esweep: the cotangent of S through segment p from its end (Ebuf at slot P - 1 - p; NULL =
// 0), token by token in reverse.  With X the cotangent arriving at token t from later tokens,
//   Shat = X + dnum_t phi(q_t)^T,   dr_t = Shat ahat_t (= dv_t),   X <- Shat - dr_t khat_t^T.
// The rows of X evolve independently, so row sums stay inside a 16-lane row (no exchange
// between waves).  Writes dv and, at the last token of every BW_CC-token chunk, X before that
// token's terms ([stream][ceil(T / BW_CC)][d][d]): the chunked pass forms every other
// gradient term of the chunk from it.
// ---------------------------------------------------------------------------------------------
template <int D>
struct BwSweepShared {
  float kh[2][D], ah[2][D], fq[2][D], dnum[2][D];
};

template <int D, typename TIn>
__global__ void __launch_bounds__(BW_NT)
k_bw_esweep(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ dout,
            const float *__restrict__ recs, const float *__restrict__ Ebuf, float *__restrict__ dv,
            float *__restrict__ Xc, int64_t T, int64_t L, int64_t P) {
  using C = BwCfg<D>;
  constexpr int R = C::R, NB = C::NB;
  __shared__ BwSweepShared<D> sh;
  const int64_t s = blockIdx.x, p = blockIdx.y;
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const int tid = threadIdx.x, i = tid >> 4, pj = tid & 15;
  const int64_t NX = (T + BW_CC - 1) / BW_CC;
  const float *rec0 = recs + s * T * C::REC;
  const int64_t slot = s * P + (P - 1 - p);
  auto row = [&](int a) { return i + 32 * a; };
  auto col = [&](int b, int e) { return 2 * pj + 32 * b + e; };

  float X[R][NB][2];
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float2 x = make_float2(0.f, 0.f);
      if (Ebuf != nullptr) x = *reinterpret_cast<const float2 *>(Ebuf + slot * D * D + row(a) * D + col(b, 0));
      X[a][b][0] = x.x;
      X[a][b][1] = x.y;
    }

  // token t - 1's record is loaded while token t is processed
  float pa = 0.f, prk = 0.f, pden = 1.f;
  TIn pdo{}, pkr{}, pq{};
  auto load = [&](int64_t t) {
    const float *rec = rec0 + t * C::REC;
    const int64_t tok = (s * T + t) * D;
    if (tid < D) {
      pa = rec[BwRec<D>::AH + tid];
      pdo = dout[tok + tid];
      pkr = k[tok + tid];
      pq = q[tok + tid];
    }
    prk = rec[BwRec<D>::SC + 2];
    pden = rec[BwRec<D>::SC + 3];
  };
  load(te - 1);
  for (int64_t t = te - 1; t >= tb; --t) {
    if (t % BW_CC == BW_CC - 1 || t == te - 1) {
      float *dst = Xc + (s * NX + t / BW_CC) * D * D;
#pragma unroll
      for (int a = 0; a < R; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          *reinterpret_cast<float2 *>(dst + row(a) * D + col(b, 0)) = make_float2(X[a][b][0], X[a][b][1]);
    }
    const int buf = static_cast<int>(t & 1);
    // double-buffered staging: this token's buffer was last read two tokens back, before the
    // previous token's barrier
    if (tid < D) {
      sh.kh[buf][tid] = bw_cv(pkr) * prk;  // khat and phi(q) as the forward formed them
      sh.ah[buf][tid] = pa;
      sh.fq[buf][tid] = phi(bw_cv(pq));
      sh.dnum[buf][tid] = bw_cv(pdo) / pden;
    }
    if (t > tb) load(t - 1);
    __syncthreads();
    float dr[R];
#pragma unroll
    for (int a = 0; a < R; ++a) {
      const float dn_r = sh.dnum[buf][row(a)];
      float x = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int c = col(b, e);
          X[a][b][e] = fmaf(dn_r, sh.fq[buf][c], X[a][b][e]);
          x = fmaf(X[a][b][e], sh.ah[buf][c], x);
        }
      dr[a] = x;
    }
    row_sum16_n(dr);
#pragma unroll
    for (int a = 0; a < R; ++a) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) X[a][b][e] = fmaf(-dr[a], sh.kh[buf][col(b, e)], X[a][b][e]);
      if (pj == 0) dv[(s * T + t) * D + row(a)] = dr[a];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// k_bw_cgrad: every gradient term but dv over segment p, in chunks of BW_CC tokens from the end,
// on the fp32 matrix cores.  Within a chunk [c0, c1) (rows: the chunk's tokens), with X the
// S cotangent at its last token (k_bw_esweep), dR the rows dr_t (= dv), Dn the rows
// dnum_t = do_t / den_t, Rr the residuals r_t, S0 and A0 the state before c0:
//   dAhat = Rr X + triu0(Rr Dn^T) Phi(q) - triu1(Rr dR^T) Khat          (dahat_t = Shat_t^T r_t)
//   dY    = (dAhat - ahat (ahat . dAhat)) / ||y||                        (row by row)
//   W     = dY A0 - tril0(dY Z^T) D^{-1} Z                               (w_t = A_t dy_t)
//   dKhat = W - dR S0 - tril(-1)(dR Rr^T) Ahat                           (- S_{t-1}^T dr_t + w_t)
//   dPhiq = Dn S0 + tril0(Dn Rr^T) Ahat + dden n_t                       (S_t^T dnum_t + dden n_t)
//   dU    = -2 U R1 - triu0(U Y^T) W - triu0(U W^T) Y                    (-2 R_s u_s, R local)
//   R0    = R1 + (W^T Y + Y^T W) / 2,    Y = diag(||y||) Ahat
// where S_t = S0 + sum_{i <= t} r_i ahat_i^T and A_t = A0 - sum_{i <= t} z_i z_i^T / delta_i
// (the forward's own updates), and dn_t, n_t are suffix sums over the chunk.  The state before
// c0 is the checkpoint before c0 when c0 is a multiple of BW_CK, else the checkpoint after
// c1 - 1 with the chunk's own updates undone (two more products).  Wave w owns features
// 16 w .. 16 w + 15 of every token-by-feature result, and the matching column tiles of S0, A0,
// X and R in registers (in the accumulator layout, which is the B-operand layout of the
// permuted contraction index).  Same outputs and buffers as the token-by-token sweep: dq, dk,
// du = -2 R u with R local to the segment (from Rinit, NULL = 0), the segment's R sum to Wbuf
// slot P - 1 - p when Wbuf is not NULL, and the sum of w . y to trw.
// ---------------------------------------------------------------------------------------------
// base[i] with a 32-bit byte offset from a uniform base (the offset goes into the load's
// register operand, with no 64-bit address arithmetic per element)
template <typename T>
__device__ __forceinline__ T &at32(T *base, uint32_t i) {
  return *reinterpret_cast<T *>(reinterpret_cast<char *>(base) + i * static_cast<uint32_t>(sizeof(T)));
}
template <typename T>
__device__ __forceinline__ const T &at32(const T *base, uint32_t i) {
  return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + i * static_cast<uint32_t>(sizeof(T)));
}

template <int D>
struct CgCfg {
  static constexpr int NW = D / 16;      // waves
  static constexpr int NT = NW * kWave;
  static constexpr int KB = D / 16;      // 16-feature blocks of a contraction over features
  static constexpr int LDT = D + 4;      // fp32 stride of token rows
  static constexpr int LDC = BW_CC + 4;  // fp32 stride of the chunk-by-chunk matrices
  static constexpr int G4 = D / 4;       // float4 groups per token row
};

template <int D>
struct CgShared {
  using C = CgCfg<D>;
  float Rr[BW_CC][C::LDT];  // residuals r; W once dAhat is formed
  float Dn[BW_CC][C::LDT];  // dnum
  float dR[BW_CC][C::LDT];  // dr
  float Fq[BW_CC][C::LDT];  // phi(q); dY once dAhat is formed
  float Kh[BW_CC][C::LDT];  // khat
  float Ah[BW_CC][C::LDT];  // ahat
  float Zr[BW_CC][C::LDT];  // z
  float Ur[BW_CC][C::LDT];  // u
  float M1[BW_CC][C::LDC];  // Rr Dn^T (upper, with the diagonal); U Y^T later
  float M2[BW_CC][C::LDC];  // Rr dR^T (strictly upper); U W^T later
  float M3[BW_CC][C::LDC];  // dY Z^T D^{-1} (lower, with the diagonal)
  float rd[BW_CC], yn[BW_CC], rk[BW_CC], den[BW_CC], dd[BW_CC];
  float dpo[BW_CC][C::G4];  // do . o over 4 features
  float part[3][C::NW][BW_CC];
  float dn[D], n[D];        // cotangent of n and n at the chunk's last token
};

template <int D, typename TIn>
__global__ void __launch_bounds__(CgCfg<D>::NT)
k_bw_cgrad(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ u,
           const TIn *__restrict__ dout, const float *__restrict__ recs,
           const float *__restrict__ cks, const float *__restrict__ n_end,
           const float *__restrict__ Xc, const float *__restrict__ dv,
           const float *__restrict__ ndbuf, const float *__restrict__ Rinit,
           float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ du,
           float *__restrict__ Wbuf, double *__restrict__ trw, int64_t T, int64_t L, int64_t P,
           float lambda0) {
  using C = CgCfg<D>;
  constexpr int NW = C::NW, KB = C::KB, NT = C::NT, G4 = C::G4, REC = BwRec<D>::F;
  __shared__ __attribute__((aligned(16))) CgShared<D> sh;
  const int64_t s = blockIdx.x, p = blockIdx.y;
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, gq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int f = 16 * w + li;  // this lane's feature in every token-by-feature result
  const int64_t NC = (T + BW_CK - 1) / BW_CK, NX = (T + BW_CC - 1) / BW_CC;
  const float *rec0 = recs + s * T * REC;
  const float *ck0 = cks + s * NC * 2 * D * D;
  const int64_t slot = s * P + (P - 1 - p);
  auto ld4 = [](const float *x) { return *reinterpret_cast<const f4_t *>(x); };
  // The chunk-by-chunk tile jobs go round the four SIMDs (a workgroup's waves sit on SIMD
  // w % 4), and among the waves of one SIMD in turn, so that every SIMD gets the same share.
  constexpr int NS = NW < 4 ? NW : 4;
  const int jsimd = w % NS, jn = (NW - jsimd + NS - 1) / NS;
  const int job0 = jsimd + NS * (w / NS), jstep = NS * jn;
  // acc + sgn * A B over the feature index for one 16 x 16 tile: A's row is arow (this lane's
  // token row in LDS, read 16 bytes at a time), B a register column tile in the accumulator
  // layout.  The next block's operand is read before this block's products, and nothing moves
  // across the blocks, so at most two blocks of operands are live.
  auto mm_rt = [&](f4_t acc, const float *arow, const f4_t (&bt)[KB], float sgn) {
    f4_t a = ld4(arow + 4 * gq);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f4_t an = a;
      if (kb + 1 < KB) an = ld4(arow + 16 * (kb + 1) + 4 * gq);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = mfma_f32_16x16x4(sgn * a[r], bt[kb][r], acc);
      a = an;
    }
    return acc;
  };
  // A B^T over the feature index for one tile: both operands token rows in LDS
  auto mm_rr = [&](const float *arow, const float *brow, float bs) {
    f4_t acc = f4_zero();
    f4_t a = ld4(arow + 4 * gq), b = ld4(brow + 4 * gq);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f4_t an = a, bn = b;
      if (kb + 1 < KB) {
        an = ld4(arow + 16 * (kb + 1) + 4 * gq);
        bn = ld4(brow + 16 * (kb + 1) + 4 * gq);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = mfma_f32_16x16x4(a[r], b[r] * bs, acc);
      a = an;
      b = bn;
    }
    return acc;
  };

  // R[16 kb + 4 gq + r][f] in Rt[kb][r]
  f4_t Rt[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      Rt[kb][r] = Rinit != nullptr ? Rinit[s * D * D + static_cast<uint32_t>((16 * kb + 4 * gq + r) * D + f)] : 0.f;
  if (tid < D) {
    sh.dn[tid] = ndbuf != nullptr ? ndbuf[slot * D + tid] : 0.f;
    sh.n[tid] = n_end[(s * P + p) * D + tid];
  }
  double trace = 0.0;  // thread 0

  for (int64_t c1 = te; c1 > tb;) {
    const int64_t c0 = std::max<int64_t>(tb, ((c1 - 1) / BW_CC) * BW_CC);
    const int m = static_cast<int>(c1 - c0);
    // Opaque per-chunk copies of the lane indices: the LDS and memory addresses derived from
    // them are formed again in each chunk instead of being hoisted out of the loop and held.
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, lane = tid & 63, li = lane & 15, gq = lane >> 4, f = 16 * w + li;
    // The state (S, A) the products start from: before c0 when c0 is a checkpoint boundary
    // (the fixed start at c0 = 0), else after c1 - 1, with the chunk's own rank-1 terms taken
    // back through the other triangle of the chunk matrices.
    const bool bef = (c0 % BW_CK) == 0;
    const bool init = bef && c0 == 0;
    const float *ck = ck0 + (bef ? (init ? 0 : (c0 - 1) / BW_CK) : (c1 - 1) / BW_CK) * 2 * D * D;
    // the chunk's rows: uniform bases, 32-bit offsets within the chunk
    const int64_t tok0 = (s * T + c0) * D;
    const float *rcb = rec0 + c0 * REC;
    const TIn *qb = q + tok0, *kb0 = k + tok0, *ub = u + tok0, *dob = dout + tok0;
    const float *dvb = dv + tok0;
    float *dqb = dq + tok0, *dkb = dk + tok0, *dub = du + tok0;
    // column tile of a d x d matrix in the accumulator layout: x[16 kb + 4 gq + r][f], or
    // dg times the identity where x is NULL
    // (32-bit byte offsets from the uniform base: no 64-bit address arithmetic per element)
    auto ld_tile = [&](const float *x, float dg, f4_t (&t)[KB]) {
      if (x != nullptr) {
        const char *xb = reinterpret_cast<const char *>(x);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            t[kb][r] = *reinterpret_cast<const float *>(
                xb + static_cast<uint32_t>(((16 * kb + 4 * gq + r) * D + f) * 4));
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) t[kb][r] = 16 * kb + 4 * gq + r == f ? dg : 0.f;
      }
    };
    __syncthreads();  // the previous chunk's readers are done
    // ---- stage the chunk's rows (rows past the chunk are zeros) ----
    for (int e = tid; e < BW_CC * G4; e += NT) {
      const int t = e / G4, c = 4 * (e % G4);
      f4_t rr = f4_zero(), dn = f4_zero(), dr = f4_zero(), fq = f4_zero(), kh = f4_zero(),
           ah = f4_zero(), zz = f4_zero(), uu = f4_zero();
      float po = 0.f;
      if (t < m) {
        const uint32_t rb = static_cast<uint32_t>(t * REC), o = static_cast<uint32_t>(t * D + c);
        const f4_t *rc4 = reinterpret_cast<const f4_t *>(rcb);
        const float rkt = at32(rcb, rb + BwRec<D>::SC + 2);
        const float rden = 1.0f / at32(rcb, rb + BwRec<D>::SC + 3);
        const f4_t oo = at32(rc4, (rb + BwRec<D>::O + c) / 4);
        zz = at32(rc4, (rb + BwRec<D>::Z + c) / 4);
        ah = at32(rc4, (rb + BwRec<D>::AH + c) / 4);
        rr = at32(rc4, (rb + BwRec<D>::R + c) / 4);
        dr = at32(reinterpret_cast<const f4_t *>(dvb), o / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float d = bw_cv(at32(dob, o + j));
          dn[j] = d * rden;
          po = fmaf(d, oo[j], po);
          uu[j] = bw_cv(at32(ub, o + j));
          kh[j] = bw_cv(at32(kb0, o + j)) * rkt;  // khat and phi(q) as the forward formed them
          fq[j] = phi(bw_cv(at32(qb, o + j)));
        }
      }
      *reinterpret_cast<f4_t *>(&sh.Rr[t][c]) = rr;
      *reinterpret_cast<f4_t *>(&sh.Dn[t][c]) = dn;
      *reinterpret_cast<f4_t *>(&sh.dR[t][c]) = dr;
      *reinterpret_cast<f4_t *>(&sh.Fq[t][c]) = fq;
      *reinterpret_cast<f4_t *>(&sh.Kh[t][c]) = kh;
      *reinterpret_cast<f4_t *>(&sh.Ah[t][c]) = ah;
      *reinterpret_cast<f4_t *>(&sh.Zr[t][c]) = zz;
      *reinterpret_cast<f4_t *>(&sh.Ur[t][c]) = uu;
      sh.dpo[t][c / 4] = po;
    }
    if (tid < BW_CC) {
      const int t = tid;
      const uint32_t rb = static_cast<uint32_t>((t < m ? t : 0) * REC) + BwRec<D>::SC;
      sh.rd[t] = t < m ? 1.0f / at32(rcb, rb) : 0.f;
      sh.yn[t] = t < m ? at32(rcb, rb + 1) : 0.f;
      sh.rk[t] = t < m ? at32(rcb, rb + 2) : 0.f;
      sh.den[t] = t < m ? at32(rcb, rb + 3) : 1.f;
    }
    f4_t Xt[KB];
    ld_tile(Xc + (s * NX + (c1 - 1) / BW_CC) * D * D, 0.f, Xt);
    __syncthreads();
    // dden_t = -(do_t . o_t) / den_t, the partial sums added in a fixed order
    if (tid < BW_CC) {
      float x = 0.f;
#pragma unroll
      for (int g = 0; g < G4; ++g) x += sh.dpo[tid][g];
      sh.dd[tid] = -x / sh.den[tid];
    }
    // ---- M1 = Rr Dn^T, M2 = Rr dR^T (all four tiles) ----
    for (int job = job0; job < 8; job += jstep) {
      const int mat = job >> 2, ti = (job >> 1) & 1, tj = job & 1;
      const float(*B)[C::LDT] = mat == 0 ? sh.Dn : sh.dR;
      const f4_t acc = mm_rr(&sh.Rr[16 * ti + li][0], &B[16 * tj + li][0], 1.f);
      float(*M)[C::LDC] = mat == 0 ? sh.M1 : sh.M2;
#pragma unroll
      for (int r = 0; r < 4; ++r) M[16 * ti + 4 * gq + r][16 * tj + li] = acc[r];
    }
    __syncthreads();
    // ---- dAhat = Rr X + triu0(M1) Phi(q) - triu1(M2) Khat; dN_t = sum_{j >= t} dden_j phi(q_j) ----
    f4_t dA[2], DN[2];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      f4_t acc = mm_rt(f4_zero(), &sh.Rr[16 * ti + li][0], Xt, 1.f), dacc = f4_zero();
      const int tr = 16 * ti + li;  // the A operand's row (token)
#pragma unroll
      for (int kb = ti; kb < 2; ++kb) {
        const f4_t a1 = ld4(&sh.M1[tr][16 * kb + 4 * gq]);
        const f4_t a2 = ld4(&sh.M2[tr][16 * kb + 4 * gq]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * kb + 4 * gq + r;
          const float fqj = sh.Fq[j][f];
          acc = mfma_f32_16x16x4(j >= tr ? a1[r] : 0.f, fqj, acc);
          acc = mfma_f32_16x16x4(j > tr ? -a2[r] : 0.f, sh.Kh[j][f], acc);
          dacc = mfma_f32_16x16x4(j >= tr ? sh.dd[j] : 0.f, fqj, dacc);
        }
      }
      dA[ti] = acc;
      DN[ti] = dacc;
    }
    {
      float x[8];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[4 * ti + r] = dA[ti][r] * sh.Ah[16 * ti + 4 * gq + r][f];
      row_sum16_n(x);
      if (li == 0)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
          for (int r = 0; r < 4; ++r) sh.part[0][w][16 * ti + 4 * gq + r] = x[4 * ti + r];
    }
    __syncthreads();
    // dY over the phi(q) rows (each wave's own columns; the other waves' reads of phi(q) and
    // of the partial sums are behind the barrier)
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ti + 4 * gq + r;
        float ad = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) ad += sh.part[0][ww][t];
        const float y = sh.yn[t];
        sh.Fq[t][f] = y > 0.f ? (dA[ti][r] - sh.Ah[t][f] * ad) / y : 0.f;
      }
    __syncthreads();
    // ---- M3 = dY Z^T D^{-1} (all four tiles) ----
    for (int job = job0; job < 4; job += jstep) {
      const int ti = job >> 1, tj = job & 1;
      const f4_t acc = mm_rr(&sh.Fq[16 * ti + li][0], &sh.Zr[16 * tj + li][0], 1.f);
      const float rdj = sh.rd[16 * tj + li];
#pragma unroll
      for (int r = 0; r < 4; ++r) sh.M3[16 * ti + 4 * gq + r][16 * tj + li] = acc[r] * rdj;
    }
    f4_t Mt[KB];  // A's column tile
    ld_tile(init ? nullptr : ck + D * D, 1.0f / lambda0, Mt);
    __syncthreads();
    // ---- W = dY A - (sum over i <= t | - sum over i > t) M3[t][i] z_i, over the residual rows ----
    f4_t Wv[2];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      f4_t acc = mm_rt(f4_zero(), &sh.Fq[16 * ti + li][0], Mt, 1.f);
      const int tr = 16 * ti + li;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (bef ? kb > ti : kb < ti) continue;  // whole tile masked (uniform)
        const f4_t av = ld4(&sh.M3[tr][16 * kb + 4 * gq]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * kb + 4 * gq + r;
          const float a = bef ? (j <= tr ? -av[r] : 0.f) : (j > tr ? av[r] : 0.f);
          acc = mfma_f32_16x16x4(a, sh.Zr[j][f], acc);
        }
      }
      Wv[ti] = acc;
    }
    ld_tile(init ? nullptr : ck, 0.f, Mt);  // S's column tile
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) sh.Rr[16 * ti + 4 * gq + r][f] = Wv[ti][r];
    // ---- dKhat = W - dR S -/+ (M2^T part) Ahat;  dPhiq = Dn S +/- (M1^T part) Ahat ----
    f4_t dK[2], dQ[2];
    // raw k of every token of the chunk at this lane's feature (for n_t and phi'(k))
    float kr[BW_CC];
#pragma unroll
    for (int j = 0; j < BW_CC; ++j) kr[j] = bw_cv(at32(kb0, static_cast<uint32_t>((j < m ? j : 0) * D + f)));
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      f4_t ak = mm_rt(Wv[ti], &sh.dR[16 * ti + li][0], Mt, -1.f);
      f4_t aq = mm_rt(f4_zero(), &sh.Dn[16 * ti + li][0], Mt, 1.f);
      const int tr = 16 * ti + li;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (bef ? kb > ti : kb < ti) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * kb + 4 * gq + r;
          const float ahj = sh.Ah[j][f];
          const float m2 = sh.M2[j][tr], m1 = sh.M1[j][tr];
          // before: S_{t-1} = S0 + sum_{j < t}, S_t = S0 + sum_{j <= t};
          // after:  S_{t-1} = Se - sum_{j >= t}, S_t = Se - sum_{j > t}
          ak = mfma_f32_16x16x4(bef ? (j < tr ? -m2 : 0.f) : (j >= tr ? m2 : 0.f), ahj, ak);
          aq = mfma_f32_16x16x4(bef ? (j <= tr ? m1 : 0.f) : (j > tr ? -m1 : 0.f), ahj, aq);
        }
      }
      dK[ti] = ak;
      dQ[ti] = aq;
    }
    {
      float x[16];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * ti + 4 * gq + r;
          x[4 * ti + r] = dK[ti][r] * sh.Kh[t][f];
          x[8 + 4 * ti + r] = Wv[ti][r] * sh.Ah[t][f];
        }
      row_sum16_n(x);
      if (li == 0)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sh.part[1][w][16 * ti + 4 * gq + r] = x[4 * ti + r];
            sh.part[2][w][16 * ti + 4 * gq + r] = x[8 + 4 * ti + r];
          }
    }
    __syncthreads();
    // ---- dq, dk ----
    const float dnf = sh.dn[f];
    // n_t token by token backwards from the chunk's last token, n_{t-1} = n_t - phi(k_t): the
    // exact inverse of the forward's additions where the forward added token by token (a
    // chunk sum subtracted at once would not be, and n_t for early tokens is a small
    // difference of large sums)
    float nv[2][4], kv[2][4], n_prev = sh.n[f];
#pragma unroll
    for (int j = BW_CC - 1; j >= 0; --j) {
      if (((j >> 2) & 3) == gq) {  // token j is this lane's output position (j >> 4, j & 3)
        nv[j >> 4][j & 3] = n_prev;
        kv[j >> 4][j & 3] = kr[j];
      }
      if (j < m) n_prev -= phi(kr[j]);
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ti + 4 * gq + r;
        if (t < m) {
          float kd = 0.f;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) kd += sh.part[1][ww][t];
          const uint32_t o = static_cast<uint32_t>(t * D + f);
          const float dnt = dnf + DN[ti][r];
          at32(dqb, o) = (dQ[ti][r] + sh.dd[t] * nv[ti][r]) * dphi(bw_cv(at32(qb, o)));
          at32(dkb, o) = (dK[ti][r] - sh.Kh[t][f] * kd) * sh.rk[t] + dnt * dphi(kv[ti][r]);
        }
      }
    if (tid == 0) {
      double tr = 0.0;
      for (int t = 0; t < m; ++t) {
        float wy = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) wy += sh.part[2][ww][t];
        tr += static_cast<double>(wy) * sh.yn[t];
      }
      trace += tr;
    }
    // dn carried to the previous chunk: lanes gq = 0 hold token 0's sum
    const float dn_prev = dnf + DN[0][0];
    // ---- M1 <- U Y^T, M2 <- U W^T (all four tiles) ----
    for (int job = job0; job < 8; job += jstep) {
      const int mat = job >> 2, ti = (job >> 1) & 1, tj = job & 1;
      const float ys = mat == 0 ? sh.yn[16 * tj + li] : 1.f;
      const float(*B)[C::LDT] = mat == 0 ? sh.Ah : sh.Rr;
      const f4_t acc = mm_rr(&sh.Ur[16 * ti + li][0], &B[16 * tj + li][0], ys);
      float(*M)[C::LDC] = mat == 0 ? sh.M1 : sh.M2;
#pragma unroll
      for (int r = 0; r < 4; ++r) M[16 * ti + 4 * gq + r][16 * tj + li] = acc[r];
    }
    __syncthreads();
    if (gq == 0) {
      sh.dn[f] = dn_prev;
      sh.n[f] = n_prev;
    }
    // ---- du = -2 U R - triu0(U Y^T) W - triu0(U W^T) Y ----
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      const f4_t a1 = mm_rt(f4_zero(), &sh.Ur[16 * ti + li][0], Rt, 1.f);
      f4_t a2 = f4_zero();
      const int tr = 16 * ti + li;
#pragma unroll
      for (int kb = ti; kb < 2; ++kb) {
        const f4_t m4 = ld4(&sh.M1[tr][16 * kb + 4 * gq]);
        const f4_t m5 = ld4(&sh.M2[tr][16 * kb + 4 * gq]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * kb + 4 * gq + r;
          a2 = mfma_f32_16x16x4(j >= tr ? m4[r] : 0.f, sh.Rr[j][f], a2);
          a2 = mfma_f32_16x16x4(j >= tr ? m5[r] : 0.f, sh.Ah[j][f] * sh.yn[j], a2);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ti + 4 * gq + r;
        if (t < m) at32(dub, static_cast<uint32_t>(t * D + f)) = -2.0f * a1[r] - a2[r];
      }
    }
    // ---- R += (W^T Y + Y^T W) / 2 ----
    {
      float yh[8], yf[8], wf[8];
#pragma unroll
      for (int q8 = 0; q8 < 8; ++q8) {
        const int t = 16 * (q8 >> 2) + 4 * gq + (q8 & 3);
        yh[q8] = 0.5f * sh.yn[t];
        yf[q8] = sh.Ah[t][f] * yh[q8];
        wf[q8] = sh.Rr[t][f];
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float wa[8], aa[8];
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) {
          const int t = 16 * (q8 >> 2) + 4 * gq + (q8 & 3);
          wa[q8] = sh.Rr[t][16 * kb + li];
          aa[q8] = sh.Ah[t][16 * kb + li];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) {
          Rt[kb] = mfma_f32_16x16x4(wa[q8], yf[q8], Rt[kb]);
          Rt[kb] = mfma_f32_16x16x4(aa[q8] * yh[q8], wf[q8], Rt[kb]);
        }
      }
    }
    c1 = c0;
  }
  if (Wbuf != nullptr) {
    float *dst = Wbuf + slot * D * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rw = 16 * kb + 4 * gq + r;
        dst[rw * D + f] = Rt[kb][r] - (Rinit != nullptr ? Rinit[s * D * D + rw * D + f] : 0.f);
      }
  }
  if (tid == 0) trw[s * P + p] = trace;
}

// ---------------------------------------------------------------------------------------------
// k_bw_cgradb: k_bw_cgrad for bf16 inputs (d <= 96) with every product on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16), the fp32 operands as two bf16 terms (about 16 significant bits,
// the accuracy the chunked forward's records carry for bf16 inputs; u is exact in one term).
// The token rows are staged as their two terms; the chunk-by-chunk matrices are stored as two
// terms too, already masked to the triangle each product takes (M1u = triu0(Rr Dn^T) and
// M2u = triu1(Rr dR^T) for dAhat and, with the state before the chunk, for dPhi(q) and dKhat;
// M1l, M2l the other triangles for the state after it).  W is staged as W' = diag(||y||) W, so
// that the products with Y = diag(||y||) Ahat take Ahat itself:
//   dU = -2 U R - triu0(U Ahat^T) W' - triu0(U W'^T) Ahat,   R += (W'^T Ahat + Ahat^T W') / 2.
// Operands over tokens are read with the transposing load (ds_read_b64_tr_b16).  Same inputs,
// outputs and buffers as k_bw_cgrad.
// ---------------------------------------------------------------------------------------------
template <int D>
struct CbCfg {
  static constexpr int NW = D / 16;
  static constexpr int NT = NW * kWave;
  static constexpr int KB = D / 16;
  static constexpr int LDB = D + 8;       // bf16 stride of token rows
  static constexpr int LDM = BW_CC + 8;   // bf16 stride of the chunk-by-chunk matrices
  static constexpr int G4 = D / 4;
  static constexpr int TS = BW_CC * LDB;  // term stride of a token matrix
  static constexpr int MS = BW_CC * LDM;  // term stride of a chunk-by-chunk matrix
};

template <int D>
struct CbShared {
  using C = CbCfg<D>;
  uint16_t Rr[2][BW_CC][C::LDB];  // residuals r; W' once dAhat is formed
  uint16_t Dn[2][BW_CC][C::LDB];  // dnum
  uint16_t dR[2][BW_CC][C::LDB];  // dr
  uint16_t Fq[2][BW_CC][C::LDB];  // phi(q); dY once dAhat is formed
  uint16_t Kh[2][BW_CC][C::LDB];  // khat
  uint16_t Ah[2][BW_CC][C::LDB];  // ahat
  uint16_t Zr[2][BW_CC][C::LDB];  // z
  uint16_t Ur[BW_CC][C::LDB];     // u (exact)
  uint16_t M1u[2][BW_CC][C::LDM], M1l[2][BW_CC][C::LDM];  // U Ahat^T, U W'^T later (in M1u, M2u)
  uint16_t M2u[2][BW_CC][C::LDM], M2l[2][BW_CC][C::LDM];
  uint16_t M3[2][BW_CC][C::LDM];
  float rd[BW_CC], yn[BW_CC], rk[BW_CC], den[BW_CC], dd[BW_CC];
  float dpo[BW_CC][C::G4];
  float part[3][C::NW][BW_CC];
  float dn[D], n[D];
  float Pk[BW_CC][D + 4];         // phi(k), formed once at staging
};

// two terms of a token-major (or chunk-by-chunk) matrix read over its rows r0.. and r1.. at
// column c0 + li, as an operand over the row index
__device__ __forceinline__ Split2 ld2_tr(const uint16_t *m, int ts, int ld, int r0, int r1, int c0, int li) {
  return Split2{ld_tr4x2(m, ld, r0, r1, c0, li), ld_tr4x2(m + ts, ld, r0, r1, c0, li)};
}

// ---------------------------------------------------------------------------------------------
// k_bw_xsweepb: the S-cotangent sweep of k_bw_esweep for bf16 inputs (d <= 96) in chunks of
// BW_CC tokens on the bf16 matrix cores (two-term operands).  Within a chunk, with X the
// cotangent at its last token (before that token's terms) and the rows dr_t, the token chain
//   Shat_t = X + sum_{j >= t} dnum_j phi_j^T - sum_{j > t} dr_j khat_j^T,  dr_t = Shat_t ahat_t
// is the unit upper-triangular system
//   (I + triu1(Ahat Khat^T)) dR = Ahat X^T + triu0(Ahat Phi^T) Dn,
// solved through the inverses of its two 16 x 16 diagonal blocks (each column by back
// substitution in one lane), and the cotangent before the chunk is, in transposed form,
//   X^T <- X^T + Phi^T Dn - Khat^T dR.
// Wave w keeps the column tile w of X^T (rows 16 w .. of X) in registers, in the accumulator
// layout that is also the B operand of Ahat X^T.  Writes dv and X at every chunk's last token
// (before its terms), as k_bw_esweep does.
// ---------------------------------------------------------------------------------------------
template <int D>
struct XsCfg {
  static constexpr int NW = D / 16, NT = NW * kWave, KB = D / 16, KS = KB / 2;
  static constexpr int LDB = D + 8;   // bf16 stride of token rows
  static constexpr int TS = BW_CC * LDB;
  static constexpr int LDM = BW_CC + 8;
  static constexpr int MS = BW_CC * LDM;
  static constexpr int LDH = 24;      // bf16 stride of the 16 x 16 blocks
  static constexpr int HS = 16 * LDH;
  static constexpr int G4 = D / 4;
};

template <int D>
struct XsShared {
  using C = XsCfg<D>;
  uint16_t Ah[2][BW_CC][C::LDB], Kh[2][BW_CC][C::LDB], Fq[2][BW_CC][C::LDB], Dn[2][BW_CC][C::LDB];
  uint16_t Ma[2][BW_CC][C::LDM];        // triu0(Ahat Phi^T)
  uint16_t Mk[2][16][C::LDH];           // the (0, 1) block of Ahat Khat^T
  uint16_t Iv[2][2][16][C::LDH];        // (I + N_bb)^{-1} of the two diagonal blocks
  float Nd[2][16][17];                  // N_bb = strictly upper part of the diagonal blocks
  float dpo[BW_CC][C::G4];              // the map: do . o over 4 features
  float dd[BW_CC];                      // the map: dden
};

template <int D, bool MAP>
__global__ void __launch_bounds__(XsCfg<D>::NT)
k_bw_xsweepb(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
             const bf16_t *__restrict__ dout, const float *__restrict__ recs,
             const float *__restrict__ Ebuf, float *__restrict__ dv, float *__restrict__ Xc,
             const float *__restrict__ fpm, float *__restrict__ lb, float *__restrict__ nd,
             int64_t T, int64_t L, int64_t P) {
  using C = XsCfg<D>;
  constexpr int NW = C::NW, NT = C::NT, KB = C::KB, KS = C::KS, G4 = C::G4, REC = BwRec<D>::F;
  constexpr int TS = C::TS, MS = C::MS, HS = C::HS, LDB = C::LDB;
  static_assert(KB % 2 == 0, "feature blocks go in pairs");
  __shared__ __attribute__((aligned(16))) XsShared<D> sh;
  const int64_t s = blockIdx.x, p = MAP ? blockIdx.y + 1 : blockIdx.y;
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int64_t NX = (T + BW_CC - 1) / BW_CC;
  const float *rec0 = recs + s * T * REC;
  const int64_t slot = s * P + (P - 1 - p);
  constexpr int NS = NW < 4 ? NW : 4;
  const int jsimd = w % NS, jn = (NW - jsimd + NS - 1) / NS;
  const int job0 = jsimd + NS * (w / NS), jstep = NS * jn;
  constexpr int LW = NW >= 4 ? 3 : NW - 1;  // the inverses: a wave with its SIMD to itself
  auto put2 = [](uint16_t *x, int ts, float v) {
    uint16_t t2[2];
    split_n<2>(v, t2);
    x[0] = t2[0];
    x[ts] = t2[1];
  };

  // X^T[16 kb + 4 gq + r][16 w + li] = X[16 w + li][16 kb + 4 gq + r] in Xt[kb][r]
  f4_t Xt[KB];
  {
    const int lane = threadIdx.x & 63, li = lane & 15, gq = lane >> 4;
    const float *e0 = !MAP && Ebuf != nullptr ? Ebuf + slot * D * D : nullptr;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      Xt[kb] = e0 != nullptr ? at32(reinterpret_cast<const f4_t *>(e0), static_cast<uint32_t>(((16 * w + li) * D + 16 * kb + 4 * gq) / 4))
                             : f4_zero();
  }

  // The chunk's inputs are loaded one chunk ahead into registers (two elements of 4 features
  // per thread: 32 tokens x d / 4 groups over d / 16 waves) and staged when the chunk starts.
  static_assert(BW_CC * G4 == 2 * NT, "two staging elements per thread");
  struct Pf {
    f4_t ah, oo;  // oo: o, for the map's dden
    uint2 kw, qw, dw;
    float rk, den;
  };
  float ndp = 0.f;  // MAP, lane (li, gq = 0) of wave w: feature 16 w + li of sum_t dden_t phi(q_t)
  Pf pf[2];
  auto fetch = [&](int64_t cs, int mm, int tid) {
    const int64_t tok = (s * T + cs) * D;
    const float *rc = rec0 + cs * REC;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int e = tid + it * NT, t = e / G4, c = 4 * (e % G4);
      const int tt = t < mm ? t : 0;  // rows past the chunk: a row of it, zeroed when staged
      const uint32_t rb = static_cast<uint32_t>(tt * REC), o = static_cast<uint32_t>(tt * D + c);
      pf[it].ah = at32(reinterpret_cast<const f4_t *>(rc), (rb + BwRec<D>::AH + c) / 4);
      if constexpr (MAP) pf[it].oo = at32(reinterpret_cast<const f4_t *>(rc), (rb + BwRec<D>::O + c) / 4);
      pf[it].kw = at32(reinterpret_cast<const uint2 *>(k + tok), o / 4);
      pf[it].qw = at32(reinterpret_cast<const uint2 *>(q + tok), o / 4);
      pf[it].dw = at32(reinterpret_cast<const uint2 *>(dout + tok), o / 4);
      pf[it].rk = at32(rc, rb + BwRec<D>::SC + 2);
      pf[it].den = at32(rc, rb + BwRec<D>::SC + 3);
    }
  };
  {
    const int64_t c0f = std::max<int64_t>(tb, ((te - 1) / BW_CC) * BW_CC);
    fetch(c0f, static_cast<int>(te - c0f), threadIdx.x);
  }

  for (int64_t c1 = te; c1 > tb;) {
    const int64_t c0 = std::max<int64_t>(tb, ((c1 - 1) / BW_CC) * BW_CC);
    const int m = static_cast<int>(c1 - c0);
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, lane = tid & 63, li = lane & 15, gq = lane >> 4;
    // X at the chunk's last token, before its terms
    if constexpr (!MAP) {
      f4_t *xc = reinterpret_cast<f4_t *>(Xc + (s * NX + (c1 - 1) / BW_CC) * D * D);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) at32(xc, static_cast<uint32_t>(((16 * w + li) * D + 16 * kb + 4 * gq) / 4)) = Xt[kb];
    }
    const int64_t tok0 = (s * T + c0) * D;
    __syncthreads();  // the previous chunk's readers are done
    // ---- stage ahat, khat, phi(q), dnum as two terms (rows past the chunk are zeros) ----
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int e = tid + it * NT, t = e / G4, c = 4 * (e % G4);
      f4_t ah = f4_zero(), kh = f4_zero(), fq = f4_zero(), dn = f4_zero();
      float po = 0.f;
      if (t < m) {
        const Pf &v = pf[it];
        ah = v.ah;
        const f4_t k4{pk_lo_val(v.kw.x), pk_hi_val(v.kw.x), pk_lo_val(v.kw.y), pk_hi_val(v.kw.y)};
        const f4_t q4{pk_lo_val(v.qw.x), pk_hi_val(v.qw.x), pk_lo_val(v.qw.y), pk_hi_val(v.qw.y)};
        const f4_t d4{pk_lo_val(v.dw.x), pk_hi_val(v.dw.x), pk_lo_val(v.dw.y), pk_hi_val(v.dw.y)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // khat, phi(q) and dnum as the forward and the sweep form them
          kh[j] = k4[j] * v.rk;
          fq[j] = phi(q4[j]);
          dn[j] = d4[j] / v.den;
          if constexpr (MAP) po = fmaf(d4[j], v.oo[j], po);
        }
      }
      if constexpr (MAP) {
        sh.dpo[t][c / 4] = po;
        if (c == 0) sh.dd[t] = t < m ? pf[it].den : 1.f;  // den, turned into dden below
      }
      auto stage2 = [&](uint16_t (*X)[BW_CC][LDB], const f4_t &x) {
        uint32_t a[2], b[2];
        split_pk<2>(x[0], x[1], a);
        split_pk<2>(x[2], x[3], b);
        *reinterpret_cast<uint2 *>(&X[0][t][c]) = make_uint2(a[0], b[0]);
        *reinterpret_cast<uint2 *>(&X[1][t][c]) = make_uint2(a[1], b[1]);
      };
      stage2(sh.Ah, ah);
      stage2(sh.Kh, kh);
      stage2(sh.Fq, fq);
      stage2(sh.Dn, dn);
    }
    if (c0 > tb) {  // the next chunk's inputs, in flight during this chunk's products
      const int64_t c0n = std::max<int64_t>(tb, ((c0 - 1) / BW_CC) * BW_CC);
      fetch(c0n, static_cast<int>(c0 - c0n), tid);
    }
    __syncthreads();
    if (MAP && w == LW && lane < BW_CC) {  // dden_t = -(do_t . o_t) / den_t, in a fixed order
      float x = 0.f;
#pragma unroll
      for (int g = 0; g < G4; ++g) x += sh.dpo[lane][g];
      sh.dd[lane] = -x / sh.dd[lane];
    }
    // ---- Ma = triu0(Ahat Phi^T); the diagonal blocks of Ahat Khat^T (strictly upper, fp32)
    // and its (0, 1) block (two terms) ----
    for (int job = job0; job < 6; job += jstep) {
      const int ti = job == 2 || job == 4 ? 1 : 0, tj = job == 0 || job == 3 ? 0 : 1;
      const uint16_t *asrc = &sh.Ah[0][16 * ti + li][0];
      const uint16_t *bsrc = job < 3 ? &sh.Fq[0][16 * tj + li][0] : &sh.Kh[0][16 * tj + li][0];
      f4_t acc = f4_zero();
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        acc = mm2_ss(ld2_4x2(asrc + 32 * s2 + 4 * gq, asrc + 32 * s2 + 16 + 4 * gq, TS),
                     ld2_4x2(bsrc + 32 * s2 + 4 * gq, bsrc + 32 * s2 + 16 + 4 * gq, TS), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int il = 4 * gq + r, jl = li;  // within the 16 x 16 tile
        if (job < 3) {
          put2(&sh.Ma[0][16 * ti + il][16 * tj + jl], MS, 16 * tj + jl >= 16 * ti + il ? acc[r] : 0.f);
          if (job == 2) put2(&sh.Ma[0][16 + il][jl], MS, 0.f);  // the (1, 0) block: below the diagonal
        } else if (job == 5) {
          put2(&sh.Mk[0][il][jl], HS, acc[r]);
        } else {
          sh.Nd[ti][il][jl] = jl > il ? acc[r] : 0.f;
        }
      }
    }
    __syncthreads();
    // ---- (I + N_bb)^{-1} for both diagonal blocks: lane (b, j) finds column j of block b by back
    // substitution (v_i = [i == j] - sum_{k > i} N[i][k] v_k, zero below the diagonal) ----
    if (w == LW && lane < 32) {
      const int bb = lane >> 4, j = lane & 15;
      float v[16];
#pragma unroll
      for (int i = 15; i >= 0; --i) {
        float x = i == j ? 1.f : 0.f;
#pragma unroll
        for (int kk = i + 1; kk < 16; ++kk) x = fmaf(-sh.Nd[bb][i][kk], v[kk], x);
        v[i] = x;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) put2(&sh.Iv[bb][0][i][j], HS, v[i]);
    }
    // ---- rhs = Ahat X^T + Ma Dn (this wave's 16 columns) ----
    const Split2 bdn = ld2_tr(&sh.Dn[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * w, li);
    f4_t rhs[2];
    {
      Split2 Bs[KS];
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
        const float x[8] = {Xt[2 * s2][0], Xt[2 * s2][1], Xt[2 * s2][2], Xt[2 * s2][3],
                            Xt[2 * s2 + 1][0], Xt[2 * s2 + 1][1], Xt[2 * s2 + 1][2], Xt[2 * s2 + 1][3]};
        Bs[s2] = split2(x);
      }
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const int tr = 16 * ti + li;
        const uint16_t *ar = &sh.Ah[0][tr][0];
        f4_t acc = f4_zero();
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
          acc = mm2_ss(ld2_4x2(ar + 32 * s2 + 4 * gq, ar + 32 * s2 + 16 + 4 * gq, TS), Bs[s2], acc);
        rhs[ti] = mm2_ss(ld2_4x2(&sh.Ma[0][tr][4 * gq], &sh.Ma[0][tr][16 + 4 * gq], MS), bdn, acc);
      }
    }
    if constexpr (MAP) {  // sum_t dden_t phi(q_t) at feature 16 w + li
      const Split2 fq = ld2_tr(&sh.Fq[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * w, li);
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f0 = bf_val(__builtin_bit_cast(uint16_t, fq.h[e])) + bf_val(__builtin_bit_cast(uint16_t, fq.l[e]));
        const float f1 = bf_val(__builtin_bit_cast(uint16_t, fq.h[4 + e])) + bf_val(__builtin_bit_cast(uint16_t, fq.l[4 + e]));
        x = fmaf(sh.dd[4 * gq + e], f0, fmaf(sh.dd[16 + 4 * gq + e], f1, x));
      }
      ndp += sum_rows4(x);
    }
    __syncthreads();  // the inverses
    // ---- dR_b = Iv_b rhs_b, dR_a = Iv_a (rhs_a - Mk dR_b) (K = 16 products) ----
    const f4_t dRb = mm2h_ss(ld2_4h(&sh.Iv[1][0][li][4 * gq], HS), split2_4h(rhs[1]), f4_zero());
    const f4_t cor = mm2h_ss(ld2_4h(&sh.Mk[0][li][4 * gq], HS), split2_4h(dRb), f4_zero());
    const f4_t dRa = mm2h_ss(ld2_4h(&sh.Iv[0][0][li][4 * gq], HS), split2_4h(rhs[0] - cor), f4_zero());
    if constexpr (!MAP) {
      float *dvb = dv + tok0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ta = 4 * gq + r, tbb = 16 + 4 * gq + r;
        if (ta < m) at32(dvb, static_cast<uint32_t>(ta * D + 16 * w + li)) = dRa[r];
        if (tbb < m) at32(dvb, static_cast<uint32_t>(tbb * D + 16 * w + li)) = dRb[r];
      }
    }
    // ---- X^T += Phi^T Dn - Khat^T dR ----
    {
      const float nx[8] = {-dRa[0], -dRa[1], -dRa[2], -dRa[3], -dRb[0], -dRb[1], -dRb[2], -dRb[3]};
      const Split2 bdr = split2(nx);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        Xt[kb] = mm2_ss(ld2_tr(&sh.Fq[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * kb, li), bdn, Xt[kb]);
        Xt[kb] = mm2_ss(ld2_tr(&sh.Kh[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * kb, li), bdr, Xt[kb]);
      }
    }
    c1 = c0;
  }
  if constexpr (MAP) {  // Lmap = Pi_p^T, Bmap = X, and the segment's sum of dden phi(q), at slot P - 1 - p
    const int lane = threadIdx.x & 63, li = lane & 15, gq = lane >> 4;
    float *dst = lb + slot * 2 * D * D;
    const float *pi = fpm + (s * P + p) * 2 * D * D;
    for (int idx = threadIdx.x; idx < D * D; idx += NT) dst[idx] = pi[(idx % D) * D + idx / D];
    f4_t *bm = reinterpret_cast<f4_t *>(dst + D * D);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) at32(bm, static_cast<uint32_t>(((16 * w + li) * D + 16 * kb + 4 * gq) / 4)) = Xt[kb];
    if (gq == 0) nd[slot * D + 16 * w + li] = ndp;
  }
}

template <int D>
__global__ void __launch_bounds__(CbCfg<D>::NT)
k_bw_cgradb(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k, const bf16_t *__restrict__ u,
            const bf16_t *__restrict__ dout, const float *__restrict__ recs,
            const float *__restrict__ cks, const float *__restrict__ n_end,
            const float *__restrict__ Xc, const float *__restrict__ dv,
            const float *__restrict__ ndbuf, const float *__restrict__ Rinit,
            float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ du,
            float *__restrict__ Wbuf, double *__restrict__ trw, int64_t T, int64_t L, int64_t P,
            float lambda0) {
  using C = CbCfg<D>;
  constexpr int NW = C::NW, KB = C::KB, NT = C::NT, G4 = C::G4, REC = BwRec<D>::F;
  constexpr int TS = C::TS, MS = C::MS, LDB = C::LDB, LDM = C::LDM, KS = KB / 2;
  static_assert(KB % 2 == 0, "feature blocks go in pairs");
  __shared__ __attribute__((aligned(16))) CbShared<D> sh;
  const int64_t s = blockIdx.x, p = blockIdx.y;
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int64_t NC = (T + BW_CK - 1) / BW_CK, NX = (T + BW_CC - 1) / BW_CC;
  const float *rec0 = recs + s * T * REC;
  const float *ck0 = cks + s * NC * 2 * D * D;
  const int64_t slot = s * P + (P - 1 - p);
  constexpr int NS = NW < 4 ? NW : 4;  // tile jobs round the SIMDs, as in k_bw_cgrad
  const int jsimd = w % NS, jn = (NW - jsimd + NS - 1) / NS;
  const int job0 = jsimd + NS * (w / NS), jstep = NS * jn;
  // per-token scalar work goes to a wave that has its SIMD to itself (wave 3 of six)
  constexpr int LW = NW >= 4 ? 3 : NW - 1;
  auto val2 = [](const uint16_t *x, int ts) { return bf_val(x[0]) + bf_val(x[ts]); };
  auto put2 = [](uint16_t *x, int ts, float v) {
    uint16_t t2[2];
    split_n<2>(v, t2);
    x[0] = t2[0];
    x[ts] = t2[1];
  };
  // a column tile in the accumulator layout as two-term operands over its rows, blocks of 32
  auto split_tile = [](const f4_t (&t)[KB], Split2 (&o)[KS]) {
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const float x[8] = {t[2 * s2][0], t[2 * s2][1], t[2 * s2][2], t[2 * s2][3],
                          t[2 * s2 + 1][0], t[2 * s2 + 1][1], t[2 * s2 + 1][2], t[2 * s2 + 1][3]};
      o[s2] = split2(x);
    }
  };

  f4_t Rt[KB];
  {
    const int gq = (threadIdx.x & 63) >> 4, f = 16 * w + (threadIdx.x & 15);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Rt[kb][r] = Rinit != nullptr ? Rinit[s * D * D + static_cast<uint32_t>((16 * kb + 4 * gq + r) * D + f)] : 0.f;
  }
  if (threadIdx.x < D) {
    sh.dn[threadIdx.x] = ndbuf != nullptr ? ndbuf[slot * D + threadIdx.x] : 0.f;
    sh.n[threadIdx.x] = n_end[(s * P + p) * D + threadIdx.x];
  }
  double trace = 0.0;  // wave LW, lane t < BW_CC: the sum of w . y over the tokens at chunk slot t

  for (int64_t c1 = te; c1 > tb;) {
    const int64_t c0 = std::max<int64_t>(tb, ((c1 - 1) / BW_CC) * BW_CC);
    const int m = static_cast<int>(c1 - c0);
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, lane = tid & 63, li = lane & 15, gq = lane >> 4, f = 16 * w + li;
    const bool bef = (c0 % BW_CK) == 0;
    const bool init = bef && c0 == 0;
    const float *ck = ck0 + (bef ? (init ? 0 : (c0 - 1) / BW_CK) : (c1 - 1) / BW_CK) * 2 * D * D;
    const int64_t tok0 = (s * T + c0) * D;
    const float *rcb = rec0 + c0 * REC;
    const bf16_t *qb = q + tok0, *kb0 = k + tok0, *ub = u + tok0, *dob = dout + tok0;
    const float *dvb = dv + tok0;
    float *dqb = dq + tok0, *dkb = dk + tok0, *dub = du + tok0;
    auto ld_tile = [&](const float *x, float dg, f4_t (&t)[KB]) {
      if (x != nullptr) {
        const char *xb = reinterpret_cast<const char *>(x);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            t[kb][r] = *reinterpret_cast<const float *>(
                xb + static_cast<uint32_t>(((16 * kb + 4 * gq + r) * D + f) * 4));
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) t[kb][r] = 16 * kb + 4 * gq + r == f ? dg : 0.f;
      }
    };
    __syncthreads();  // the previous chunk's readers are done
    // ---- stage the chunk's rows as two terms (rows past the chunk are zeros) ----
    for (int e = tid; e < BW_CC * G4; e += NT) {
      const int t = e / G4, c = 4 * (e % G4);
      f4_t rr = f4_zero(), dn = f4_zero(), dr = f4_zero(), fq = f4_zero(), kh = f4_zero(),
           ah = f4_zero(), zz = f4_zero();
      uint2 uu = make_uint2(0u, 0u);
      f4_t pk = f4_zero();
      float po = 0.f;
      if (t < m) {
        const uint32_t rb = static_cast<uint32_t>(t * REC), o = static_cast<uint32_t>(t * D + c);
        const f4_t *rc4 = reinterpret_cast<const f4_t *>(rcb);
        const float rkt = at32(rcb, rb + BwRec<D>::SC + 2);
        const float rden = 1.0f / at32(rcb, rb + BwRec<D>::SC + 3);
        const f4_t oo = at32(rc4, (rb + BwRec<D>::O + c) / 4);
        zz = at32(rc4, (rb + BwRec<D>::Z + c) / 4);
        ah = at32(rc4, (rb + BwRec<D>::AH + c) / 4);
        rr = at32(rc4, (rb + BwRec<D>::R + c) / 4);
        dr = at32(reinterpret_cast<const f4_t *>(dvb), o / 4);
        const uint2 dw = at32(reinterpret_cast<const uint2 *>(dob), o / 4);
        uu = at32(reinterpret_cast<const uint2 *>(ub), o / 4);
        const uint2 kw = at32(reinterpret_cast<const uint2 *>(kb0), o / 4);
        const uint2 qw = at32(reinterpret_cast<const uint2 *>(qb), o / 4);
        const f4_t k4{pk_lo_val(kw.x), pk_hi_val(kw.x), pk_lo_val(kw.y), pk_hi_val(kw.y)};
        const f4_t q4{pk_lo_val(qw.x), pk_hi_val(qw.x), pk_lo_val(qw.y), pk_hi_val(qw.y)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // khat and phi(q) as the forward formed them
          kh[j] = k4[j] * rkt;
          fq[j] = phi(q4[j]);
          pk[j] = phi(k4[j]);
        }
        const float dd4[4] = {pk_lo_val(dw.x), pk_hi_val(dw.x), pk_lo_val(dw.y), pk_hi_val(dw.y)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dn[j] = dd4[j] * rden;
          po = fmaf(dd4[j], oo[j], po);
        }
      }
      auto stage2 = [&](uint16_t (*X)[BW_CC][LDB], const f4_t &v) {
        uint32_t a[2], b[2];
        split_pk<2>(v[0], v[1], a);
        split_pk<2>(v[2], v[3], b);
        *reinterpret_cast<uint2 *>(&X[0][t][c]) = make_uint2(a[0], b[0]);
        *reinterpret_cast<uint2 *>(&X[1][t][c]) = make_uint2(a[1], b[1]);
      };
      stage2(sh.Rr, rr);
      stage2(sh.Dn, dn);
      stage2(sh.dR, dr);
      stage2(sh.Fq, fq);
      stage2(sh.Kh, kh);
      stage2(sh.Ah, ah);
      stage2(sh.Zr, zz);
      *reinterpret_cast<uint2 *>(&sh.Ur[t][c]) = uu;
      *reinterpret_cast<f4_t *>(&sh.Pk[t][c]) = pk;
      sh.dpo[t][c / 4] = po;
    }
    if (w == LW && lane < BW_CC) {
      const int t = lane;
      const uint32_t rb = static_cast<uint32_t>((t < m ? t : 0) * REC) + BwRec<D>::SC;
      sh.rd[t] = t < m ? 1.0f / at32(rcb, rb) : 0.f;
      sh.yn[t] = t < m ? at32(rcb, rb + 1) : 0.f;
      sh.rk[t] = t < m ? at32(rcb, rb + 2) : 0.f;
      sh.den[t] = t < m ? at32(rcb, rb + 3) : 1.f;
    }
    Split2 Bs[KS];  // the B-operand tile of the current products
    {
      f4_t Xt[KB];
      ld_tile(Xc + (s * NX + (c1 - 1) / BW_CC) * D * D, 0.f, Xt);
      split_tile(Xt, Bs);
    }
    __syncthreads();
    if (w == LW && lane < BW_CC) {
      float x = 0.f;
#pragma unroll
      for (int g = 0; g < G4; ++g) x += sh.dpo[lane][g];
      sh.dd[lane] = -x / sh.den[lane];
    }
    // ---- M1 = Rr Dn^T, M2 = Rr dR^T, stored masked: u = the upper part (with the diagonal
    // for M1, without for M2), l = the rest ----
    for (int job = job0; job < 8; job += jstep) {
      const int mat = job >> 2, ti = (job >> 1) & 1, tj = job & 1;
      const uint16_t *bsrc = mat == 0 ? &sh.Dn[0][16 * tj + li][0] : &sh.dR[0][16 * tj + li][0];
      const uint16_t *asrc = &sh.Rr[0][16 * ti + li][0];
      f4_t acc = f4_zero();
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        acc = mm2_ss(ld2_4x2(asrc + 32 * s2 + 4 * gq, asrc + 32 * s2 + 16 + 4 * gq, TS),
                     ld2_4x2(bsrc + 32 * s2 + 4 * gq, bsrc + 32 * s2 + 16 + 4 * gq, TS), acc);
      uint16_t(*Mu)[BW_CC][LDM] = mat == 0 ? sh.M1u : sh.M2u;
      uint16_t(*Ml)[BW_CC][LDM] = mat == 0 ? sh.M1l : sh.M2l;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + 4 * gq + r, j = 16 * tj + li;
        const bool up = mat == 0 ? j >= i : j > i;
        put2(&Mu[0][i][j], MS, up ? acc[r] : 0.f);
        put2(&Ml[0][i][j], MS, up ? 0.f : acc[r]);
      }
    }
    __syncthreads();
    // ---- dAhat = Rr X + M1u Phi(q) - M2u Khat;  dN_t = sum_{j >= t} dden_j phi(q_j) ----
    f4_t dA[2], DN[2];
    {
      const Split2 bq = ld2_tr(&sh.Fq[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * w, li);
      const Split2 bk = ld2_tr(&sh.Kh[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * w, li);
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const int tr = 16 * ti + li;
        const uint16_t *ar = &sh.Rr[0][tr][0];
        f4_t acc = f4_zero(), neg = f4_zero(), dacc = f4_zero();
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
          acc = mm2_ss(ld2_4x2(ar + 32 * s2 + 4 * gq, ar + 32 * s2 + 16 + 4 * gq, TS), Bs[s2], acc);
        acc = mm2_ss(ld2_4x2(&sh.M1u[0][tr][4 * gq], &sh.M1u[0][tr][16 + 4 * gq], MS), bq, acc);
        neg = mm2_ss(ld2_4x2(&sh.M2u[0][tr][4 * gq], &sh.M2u[0][tr][16 + 4 * gq], MS), bk, neg);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = e < 4 ? 4 * gq + e : 16 + 4 * gq + (e - 4);
          x[e] = j >= tr ? sh.dd[j] : 0.f;
        }
        dacc = mm2_ss(split2(x), bq, dacc);
        dA[ti] = acc - neg;
        DN[ti] = dacc;
      }
    }
    {
      float x[8];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[4 * ti + r] = dA[ti][r] * val2(&sh.Ah[0][16 * ti + 4 * gq + r][f], TS);
      row_sum16_n(x);
      if (li == 0)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
          for (int r = 0; r < 4; ++r) sh.part[0][w][16 * ti + 4 * gq + r] = x[4 * ti + r];
    }
    {
      f4_t At[KB];
      ld_tile(init ? nullptr : ck + D * D, 1.0f / lambda0, At);
      split_tile(At, Bs);
    }
    __syncthreads();
    // dY over the phi(q) rows (each wave its own columns; the reads of phi(q) and of the partial
    // sums are behind the barrier).  phi'(q) = min(phi(q), 1) at this lane's output positions
    // is kept first.
    float dpq[2][4];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ti + 4 * gq + r;
        float ad = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) ad += sh.part[0][ww][t];
        const float y = sh.yn[t];
        dpq[ti][r] = fminf(val2(&sh.Fq[0][t][f], TS), 1.0f);
        put2(&sh.Fq[0][t][f], TS, y > 0.f ? (dA[ti][r] - val2(&sh.Ah[0][t][f], TS) * ad) / y : 0.f);
      }
    __syncthreads();
    // ---- M3 = dY Z^T D^{-1}, masked: lower with the diagonal (state before the chunk), or
    // strictly upper (state after it) ----
    for (int job = job0; job < 4; job += jstep) {
      const int ti = job >> 1, tj = job & 1;
      const uint16_t *asrc = &sh.Fq[0][16 * ti + li][0], *bsrc = &sh.Zr[0][16 * tj + li][0];
      f4_t acc = f4_zero();
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        acc = mm2_ss(ld2_4x2(asrc + 32 * s2 + 4 * gq, asrc + 32 * s2 + 16 + 4 * gq, TS),
                     ld2_4x2(bsrc + 32 * s2 + 4 * gq, bsrc + 32 * s2 + 16 + 4 * gq, TS), acc);
      const int j = 16 * tj + li;
      const float rdj = sh.rd[j];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + 4 * gq + r;
        put2(&sh.M3[0][i][j], MS, (bef ? j <= i : j > i) ? acc[r] * rdj : 0.f);
      }
    }
    __syncthreads();
    // ---- W = dY A -/+ M3 Z;  W' = diag(||y||) W over the residual rows ----
    f4_t Wv[2];
    {
      const Split2 bz = ld2_tr(&sh.Zr[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * w, li);
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const int tr = 16 * ti + li;
        const uint16_t *ar = &sh.Fq[0][tr][0];
        f4_t acc = f4_zero(), m3 = f4_zero();
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
          acc = mm2_ss(ld2_4x2(ar + 32 * s2 + 4 * gq, ar + 32 * s2 + 16 + 4 * gq, TS), Bs[s2], acc);
        m3 = mm2_ss(ld2_4x2(&sh.M3[0][tr][4 * gq], &sh.M3[0][tr][16 + 4 * gq], MS), bz, m3);
        Wv[ti] = bef ? acc - m3 : acc + m3;
      }
    }
    {
      f4_t St[KB];
      ld_tile(init ? nullptr : ck, 0.f, St);
      split_tile(St, Bs);
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ti + 4 * gq + r;
        put2(&sh.Rr[0][t][f], TS, sh.yn[t] * Wv[ti][r]);
      }
    // ---- dKhat = W - dR S -/+ (M2 part)^T Ahat;  dPhi(q) = Dn S +/- (M1 part)^T Ahat ----
    f4_t dK[2], dQ[2];
    {
      const Split2 ba = ld2_tr(&sh.Ah[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * w, li);
      const uint16_t *m1 = bef ? &sh.M1u[0][0][0] : &sh.M1l[0][0][0];
      const uint16_t *m2 = bef ? &sh.M2u[0][0][0] : &sh.M2l[0][0][0];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const uint16_t *a1 = &sh.dR[0][16 * ti + li][0], *a2 = &sh.Dn[0][16 * ti + li][0];
        f4_t ak = f4_zero(), aq = f4_zero();
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
          ak = mm2_ss(ld2_4x2(a1 + 32 * s2 + 4 * gq, a1 + 32 * s2 + 16 + 4 * gq, TS), Bs[s2], ak);
          aq = mm2_ss(ld2_4x2(a2 + 32 * s2 + 4 * gq, a2 + 32 * s2 + 16 + 4 * gq, TS), Bs[s2], aq);
        }
        // (M^T)[t][i] = M[i][t]: the chunk matrix read over its rows at column t
        const f4_t t2 = mm2_ss(ld2_tr(m2, MS, LDM, 4 * gq, 16 + 4 * gq, 16 * ti, li), ba, f4_zero());
        const f4_t t1 = mm2_ss(ld2_tr(m1, MS, LDM, 4 * gq, 16 + 4 * gq, 16 * ti, li), ba, f4_zero());
        // before: S_{t-1} = S0 + sum_{i < t}, S_t = S0 + sum_{i <= t};
        // after:  S_{t-1} = Se - sum_{i >= t}, S_t = Se - sum_{i > t}
        dK[ti] = bef ? Wv[ti] - ak - t2 : Wv[ti] - ak + t2;
        dQ[ti] = bef ? aq + t1 : aq - t1;
      }
    }
    {
      float x[16];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * ti + 4 * gq + r;
          x[4 * ti + r] = dK[ti][r] * val2(&sh.Kh[0][t][f], TS);
          x[8 + 4 * ti + r] = Wv[ti][r] * val2(&sh.Ah[0][t][f], TS);
        }
      row_sum16_n(x);
      if (li == 0)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sh.part[1][w][16 * ti + 4 * gq + r] = x[4 * ti + r];
            sh.part[2][w][16 * ti + 4 * gq + r] = x[8 + 4 * ti + r];
          }
    }
    {
      f4_t Rc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) Rc[kb] = Rt[kb];
      split_tile(Rc, Bs);  // R before this chunk's terms, for du
    }
    __syncthreads();
    // ---- dq, dk ----
    const float dnf = sh.dn[f];
    float nv[2][4], kv[2][4], n_prev = sh.n[f];
#pragma unroll
    for (int j = BW_CC - 1; j >= 0; --j) {
      const float pkj = sh.Pk[j][f];  // 0 past the chunk
      if (((j >> 2) & 3) == gq) {
        nv[j >> 4][j & 3] = n_prev;
        kv[j >> 4][j & 3] = fminf(pkj, 1.0f);  // phi'(k) = min(phi(k), 1)
      }
      n_prev -= pkj;
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ti + 4 * gq + r;
        if (t < m) {
          float kd = 0.f;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) kd += sh.part[1][ww][t];
          const uint32_t o = static_cast<uint32_t>(t * D + f);
          const float dnt = dnf + DN[ti][r];
          at32(dqb, o) = (dQ[ti][r] + sh.dd[t] * nv[ti][r]) * dpq[ti][r];
          at32(dkb, o) = (dK[ti][r] - val2(&sh.Kh[0][t][f], TS) * kd) * sh.rk[t] + dnt * kv[ti][r];
        }
      }
    if (w == LW && lane < m) {
      float wy = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) wy += sh.part[2][ww][lane];
      trace += static_cast<double>(wy) * sh.yn[lane];
    }
    const float dn_prev = dnf + DN[0][0];
    // ---- M1u <- U Ahat^T, M2u <- U W'^T (upper with the diagonal) ----
    for (int job = job0; job < 8; job += jstep) {
      const int mat = job >> 2, ti = (job >> 1) & 1, tj = job & 1;
      const uint16_t *asrc = &sh.Ur[16 * ti + li][0];
      const uint16_t *bsrc = mat == 0 ? &sh.Ah[0][16 * tj + li][0] : &sh.Rr[0][16 * tj + li][0];
      f4_t acc = f4_zero();
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        acc = mm2_xs(ld_bf4x2(asrc + 32 * s2 + 4 * gq, asrc + 32 * s2 + 16 + 4 * gq),
                     ld2_4x2(bsrc + 32 * s2 + 4 * gq, bsrc + 32 * s2 + 16 + 4 * gq, TS), acc);
      uint16_t(*M)[BW_CC][LDM] = mat == 0 ? sh.M1u : sh.M2u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + 4 * gq + r, j = 16 * tj + li;
        put2(&M[0][i][j], MS, j >= i ? acc[r] : 0.f);
      }
    }
    __syncthreads();
    if (gq == 0) {
      sh.dn[f] = dn_prev;
      sh.n[f] = n_prev;
    }
    // ---- du = -2 U R - M1u W' - M2u Ahat ----
    {
      const Split2 bw = ld2_tr(&sh.Rr[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * w, li);
      const Split2 ba = ld2_tr(&sh.Ah[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * w, li);
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const int tr = 16 * ti + li;
        const uint16_t *ar = &sh.Ur[tr][0];
        f4_t a1 = f4_zero(), a2 = f4_zero();
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
          a1 = mm2_xs(ld_bf4x2(ar + 32 * s2 + 4 * gq, ar + 32 * s2 + 16 + 4 * gq), Bs[s2], a1);
        a2 = mm2_ss(ld2_4x2(&sh.M1u[0][tr][4 * gq], &sh.M1u[0][tr][16 + 4 * gq], MS), bw, a2);
        a2 = mm2_ss(ld2_4x2(&sh.M2u[0][tr][4 * gq], &sh.M2u[0][tr][16 + 4 * gq], MS), ba, a2);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * ti + 4 * gq + r;
          if (t < m) at32(dub, static_cast<uint32_t>(t * D + f)) = -2.0f * a1[r] - a2[r];
        }
      }
      // ---- R += (W'^T Ahat + Ahat^T W') / 2 ----
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const Split2 aw = ld2_tr(&sh.Rr[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * kb, li);
        const Split2 aa = ld2_tr(&sh.Ah[0][0][0], TS, LDB, 4 * gq, 16 + 4 * gq, 16 * kb, li);
        f4_t x = mm2_ss(aw, ba, f4_zero());
        x = mm2_ss(aa, bw, x);
#pragma unroll
        for (int r = 0; r < 4; ++r) Rt[kb][r] = fmaf(0.5f, x[r], Rt[kb][r]);
      }
    }
    c1 = c0;
  }
  const int gq = (threadIdx.x & 63) >> 4, f = 16 * w + (threadIdx.x & 15);
  if (Wbuf != nullptr) {
    float *dst = Wbuf + slot * D * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rw = 16 * kb + 4 * gq + r;
        dst[rw * D + f] = Rt[kb][r] - (Rinit != nullptr ? Rinit[s * D * D + rw * D + f] : 0.f);
      }
  }
  if (w == LW) {  // the 32 slot sums, pairwise in a fixed order
#pragma unroll
    for (int off = 1; off < BW_CC; off <<= 1) trace += __shfl_xor(trace, off);
    if ((threadIdx.x & 63) == 0) trw[s * P + p] = trace;
  }
}

// ---------------------------------------------------------------------------------------------
// k_bw_terminal: X = A_T sym(dA_T) A_T per stream (A_T = the state after the last token, from
// the replay's checkpoint), through the scratch matrix Y = sym(dA_T) A_T.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
k_bw_terminal(const float *__restrict__ cks, const float *__restrict__ dA_T,
              float *__restrict__ Y, float *__restrict__ X, int64_t T) {
  const int64_t s = blockIdx.x;
  const int64_t NC = (T + BW_CK - 1) / BW_CK;
  const float *AT = cks + s * NC * 2 * D * D + ((T - 1) / BW_CK) * 2 * D * D + D * D;
  const float *G = dA_T + s * D * D;
  float *Ys = Y + s * D * D, *Xs = X + s * D * D;
  for (int e = threadIdx.x; e < D * D; e += 256) {
    const int r = e / D, c = e % D;
    float acc = 0.f;
    for (int m = 0; m < D; ++m) acc = fmaf(0.5f * (G[r * D + m] + G[m * D + r]), AT[m * D + c], acc);
    Ys[e] = acc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < D * D; e += 256) {
    const int r = e / D, c = e % D;
    float acc = 0.f;
    for (int m = 0; m < D; ++m) acc = fmaf(AT[r * D + m], Ys[m * D + c], acc);
    Xs[e] = acc;
  }
}

// ---------------------------------------------------------------------------------------------
// k_bw_fix: du_t -= 2 R_end u_t over up to 256 tokens of segment p (R_end at Rend slot P - 1 - p)
// on the matrix cores: wave w forms features 16 w .. 16 w + 15 of (R_end u_t) for 16 tokens at a
// time, with R_end's rows 16 w .. as the B operand in registers (B[k][f] = R_end[f][k]) and the
// token rows of u read straight from memory as the A operand.  bf16 inputs: u exact in one bf16
// term, R_end in two (v_mfma_f32_16x16x32_bf16); fp32 inputs: fp32 products.
// ---------------------------------------------------------------------------------------------
template <int D, typename TIn>
__global__ void __launch_bounds__(D / 16 * kWave)
k_bw_fix(const TIn *__restrict__ u, const float *__restrict__ Rend, float *__restrict__ du,
         int64_t T, int64_t L, int64_t P) {
  constexpr int KB = D / 16;
  const int64_t s = blockIdx.x, p = blockIdx.y;
  const int64_t seg_end = std::min<int64_t>(T, p * L + L);
  const int64_t t_beg = p * L + static_cast<int64_t>(blockIdx.z) * 256;
  if (t_beg >= seg_end) return;  // the whole workgroup
  const int nt = static_cast<int>(std::min<int64_t>(256, seg_end - t_beg));
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63, li = lane & 15, gq = lane >> 4, f = 16 * w + li;
  const float *Rs = Rend + (s * P + (P - 1 - p)) * D * D;
  // Rt[kb][r] = R_end[f][16 kb + 4 gq + r]
  f4_t Rt[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) Rt[kb] = at32(reinterpret_cast<const f4_t *>(Rs), static_cast<uint32_t>((f * D + 16 * kb + 4 * gq) / 4));
  const TIn *ub = u + (s * T + t_beg) * D;
  float *db = du + (s * T + t_beg) * D;
  if constexpr (sizeof(TIn) == 2) {
    Split2 Bs[KB / 2];
#pragma unroll
    for (int s2 = 0; s2 < KB / 2; ++s2) {
      const float x[8] = {Rt[2 * s2][0], Rt[2 * s2][1], Rt[2 * s2][2], Rt[2 * s2][3],
                          Rt[2 * s2 + 1][0], Rt[2 * s2 + 1][1], Rt[2 * s2 + 1][2], Rt[2 * s2 + 1][3]};
      Bs[s2] = split2(x);
    }
    const uint2 *u2 = reinterpret_cast<const uint2 *>(ub);
    for (int t0 = 0; t0 < nt; t0 += 16) {
      const int tr = t0 + li < nt ? t0 + li : 0;  // rows past the block: any row, never stored
      f4_t acc = f4_zero();
#pragma unroll
      for (int s2 = 0; s2 < KB / 2; ++s2) {
        const uint2 a0 = at32(u2, static_cast<uint32_t>((tr * D + 32 * s2 + 4 * gq) / 4));
        const uint2 a1 = at32(u2, static_cast<uint32_t>((tr * D + 32 * s2 + 16 + 4 * gq) / 4));
        acc = mm2_xs(__builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, a1.x, a1.y)), Bs[s2], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * gq + r;
        if (t < nt) at32(db, static_cast<uint32_t>(t * D + f)) -= 2.0f * acc[r];
      }
    }
  } else {
    const f4_t *u4 = reinterpret_cast<const f4_t *>(ub);
    for (int t0 = 0; t0 < nt; t0 += 16) {
      const int tr = t0 + li < nt ? t0 + li : 0;
      f4_t acc = f4_zero();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const f4_t a = at32(u4, static_cast<uint32_t>((tr * D + 16 * kb + 4 * gq) / 4));
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mfma_f32_16x16x4(a[r], Rt[kb][r], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * gq + r;
        if (t < nt) at32(db, static_cast<uint32_t>(t * D + f)) -= 2.0f * acc[r];
      }
    }
  }
}

// dlambda0 = -(trace of the final-state term + every segment's sum of w . y)
template <int D>
__global__ void __launch_bounds__(64)
k_bw_lambda(const float *__restrict__ X, const double *__restrict__ trw, float *__restrict__ dlambda0,
            int64_t P) {
  const int64_t s = blockIdx.x;
  double acc = 0.0;
  for (int64_t j = threadIdx.x; j < P; j += 64) acc += trw[s * P + j];
  if (X != nullptr)
    for (int c = threadIdx.x; c < D; c += 64) acc += static_cast<double>(X[s * D * D + c * D + c]);
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (threadIdx.x == 0) dlambda0[s] = static_cast<float>(-acc);
}

// ---------------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------------
struct BwPlan {
  int64_t L = 0, P = 1;
  size_t off_chunk = 0, off_md = 0, off_rec = 0, off_ck = 0, off_xc = 0, off_nend = 0, off_x = 0,
         off_y = 0, off_trw = 0;
  size_t total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

BwPlan make_bw_plan(const Problem &p, int chunk) {
  BwPlan b;
  b.L = p.T;
  b.P = 1;
  size_t off = 0;
  if (chunk > 0) {
    chunk_segments(p, chunk, &b.L, &b.P);
    if (b.P > 1) {
      b.off_chunk = 0;
      off = align256(chunk_workspace_bytes(p, chunk, true));
      b.off_md = off;
      off = align256(off + static_cast<size_t>(p.streams * b.P) * p.d * p.d * sizeof(double));
    } else {
      b.L = p.T;
    }
  }
  const size_t S = static_cast<size_t>(p.streams), T = static_cast<size_t>(p.T);
  const size_t D = static_cast<size_t>(p.d), P = static_cast<size_t>(b.P);
  const size_t NC = (T + BW_CK - 1) / BW_CK;
  b.off_rec = off;  off = align256(off + S * T * (4 * D + BW_NS) * 4);
  b.off_ck = off;   off = align256(off + S * NC * 2 * D * D * 4);
  b.off_xc = off;   off = align256(off + S * ((T + BW_CC - 1) / BW_CC) * D * D * 4);
  b.off_nend = off; off = align256(off + S * P * D * 4);
  b.off_x = off;    off = align256(off + S * D * D * 4);
  b.off_y = off;    off = align256(off + S * D * D * 4);
  b.off_trw = off;  off = align256(off + S * P * 8);
  b.total = off;
  return b;
}

// The chunked gradient pass: on the bf16 matrix cores (two-term operands) for bf16 inputs at
// d <= 96, on the fp32 matrix cores otherwise (fp32 inputs, and d = 128, whose two-term LDS
// staging would not fit).
template <int D, typename TIn>
void launch_cgrad(const TIn *q, const TIn *k, const TIn *u, const TIn *dout, const float *rec,
                  const float *ck, const float *nend, const float *xc, const float *dv,
                  const float *ndbuf, const float *Rinit, float *dq, float *dk, float *du,
                  float *Wbuf, double *trw, const Problem &pr, const BwPlan &bp, hipStream_t st) {
  const unsigned S = static_cast<unsigned>(pr.streams), P = static_cast<unsigned>(bp.P);
  if constexpr (sizeof(TIn) == 2 && D <= 96)
    VLA_LAUNCH("k_bw_cgrad", (k_bw_cgradb<D>), dim3(S, P), dim3(CbCfg<D>::NT), 0, st, q, k, u, dout,
               rec, ck, nend, xc, dv, ndbuf, Rinit, dq, dk, du, Wbuf, trw, pr.T, bp.L, bp.P, pr.lambda0);
  else
    VLA_LAUNCH("k_bw_cgrad", (k_bw_cgrad<D, TIn>), dim3(S, P), dim3(CgCfg<D>::NT), 0, st, q, k, u,
               dout, rec, ck, nend, xc, dv, ndbuf, Rinit, dq, dk, du, Wbuf, trw, pr.T, bp.L, bp.P,
               pr.lambda0);
}

// The S-cotangent sweep: in 32-token chunks on the bf16 matrix cores for bf16 inputs at d <= 96,
// token by token otherwise.
template <int D, typename TIn>
void launch_sweep(const TIn *q, const TIn *k, const TIn *dout, const float *rec, const float *E,
                  float *dv, float *xc, const Problem &pr, const BwPlan &bp, unsigned P, hipStream_t st) {
  const unsigned S = static_cast<unsigned>(pr.streams);
  if constexpr (sizeof(TIn) == 2 && D <= 96)
    VLA_LAUNCH("k_bw_esweep", (k_bw_xsweepb<D, false>), dim3(S, P), dim3(XsCfg<D>::NT), 0, st, q, k,
               dout, rec, E, dv, xc, static_cast<const float *>(nullptr), static_cast<float *>(nullptr),
               static_cast<float *>(nullptr), pr.T, bp.L, bp.P);
  else
    VLA_LAUNCH("k_bw_esweep", (k_bw_esweep<D, TIn>), dim3(S, P), dim3(BW_NT), 0, st, q, k, dout, rec,
               E, dv, xc, pr.T, bp.L, bp.P);
}

template <int D, typename TIn>
hipError_t launch_bw_t(const Problem &pr, int chunk, const BackwardIO &io, void *ws, hipStream_t st) {
  const BwPlan bp = make_bw_plan(pr, chunk);
  char *base = static_cast<char *>(ws);
  float *rec = reinterpret_cast<float *>(base + bp.off_rec);
  float *ck = reinterpret_cast<float *>(base + bp.off_ck);
  float *nend = reinterpret_cast<float *>(base + bp.off_nend);
  float *X = io.dA_T != nullptr ? reinterpret_cast<float *>(base + bp.off_x) : nullptr;
  float *Y = reinterpret_cast<float *>(base + bp.off_y);
  double *trw = reinterpret_cast<double *>(base + bp.off_trw);
  float *xc = reinterpret_cast<float *>(base + bp.off_xc);
  const TIn *q = static_cast<const TIn *>(io.q), *k = static_cast<const TIn *>(io.k);
  const TIn *v = static_cast<const TIn *>(io.v), *u = static_cast<const TIn *>(io.u);
  const TIn *dout = static_cast<const TIn *>(io.dout);
  const unsigned S = static_cast<unsigned>(pr.streams), P = static_cast<unsigned>(bp.P);
  hipError_t err;

  ChunkStates cs;
  bool replay = true;
  if (bp.P > 1) {
    // segment-start A from an fp64 inversion: dlambda0 sums terms weighted by A_t^2, so an
    // fp32 inverse's error (about cond * 2^-24) would show in it
    double *Md = reinterpret_cast<double *>(base + bp.off_md);
    // the chunked forward's passes (A side, final pass) write the token records and the state
    // checkpoints themselves, so no token-by-token replay runs
    BwRecords r;
    r.rec = rec;
    r.ck = ck;
    r.n_end = nend;
    err = launch_chunk_records(pr, chunk, io.q, io.k, io.v, io.u, base + bp.off_chunk, Md, st, r, &cs);
    replay = false;
    if (err != hipSuccess) return err;
  }
  if (replay)
    VLA_LAUNCH("k_bw_replay", (k_bw_replay<D, TIn>), dim3(S, P), dim3(BW_NT), 0, st, q, k, v, u,
               static_cast<const float *>(cs.S_seg), static_cast<const float *>(cs.A_seg),
               static_cast<const float *>(cs.n_seg), rec, ck, nend, pr.T, bp.L, bp.P, pr.lambda0, pr.eps);
  if (X != nullptr)
    VLA_LAUNCH("k_bw_terminal", (k_bw_terminal<D>), dim3(S), dim3(256), 0, st,
               static_cast<const float *>(ck), io.dA_T, Y, X, pr.T);
  if (bp.P > 1) {
    // After the forward's final pass the segment-start buffers are free: the maps go into the
    // fp64 penalty buffer (the same bytes as two fp32 d x d matrices per segment), the end
    // cotangents of S where the start states were, the segment sums of dden phi(q) where the
    // normalisers were and the segment R sums where A was; the forward's own maps (Pi_p) are
    // read for the L part of the backward's.
    float *lb = reinterpret_cast<float *>(base + bp.off_md), *E = cs.S_seg, *nd = cs.n_seg, *W = cs.A_seg;
    if constexpr (sizeof(TIn) == 2 && D <= 96)  // the chunked sweep from a zero cotangent
      VLA_LAUNCH("k_bw_dsmap", (k_bw_xsweepb<D, true>), dim3(S, P - 1), dim3(XsCfg<D>::NT), 0, st, q, k,
                 dout, static_cast<const float *>(rec), static_cast<const float *>(nullptr),
                 static_cast<float *>(nullptr), static_cast<float *>(nullptr),
                 static_cast<const float *>(cs.pib), lb, nd, pr.T, bp.L, bp.P);
    else
      VLA_LAUNCH("k_bw_dsmap", (k_bw_dsmap<D, TIn>), dim3(S, P - 1), dim3(BW_NT), 0, st, q, k, dout,
                 static_cast<const float *>(rec), static_cast<const float *>(cs.pib), lb, nd, pr.T,
                 bp.L, bp.P);
    err = launch_affine_prefix(pr, lb, E, bp.P, io.dS_T, nd, io.dn_T, st);
    if (err != hipSuccess) return err;
    launch_sweep<D, TIn>(q, k, dout, rec, E, io.dv, xc, pr, bp, P, st);
    launch_cgrad<D, TIn>(q, k, u, dout, rec, ck, nend, xc, io.dv, nd, nullptr, io.dq, io.dk, io.du,
                         W, trw, pr, bp, st);
    err = launch_matrix_prefix(pr, W, bp.P, X, st);
    if (err != hipSuccess) return err;
    const unsigned nz = static_cast<unsigned>((bp.L + 255) / 256);
    VLA_LAUNCH("k_bw_fix", (k_bw_fix<D, TIn>), dim3(S, P, nz), dim3(D / 16 * kWave), 0, st, u,
               static_cast<const float *>(W), io.du, pr.T, bp.L, bp.P);
  } else {
    launch_sweep<D, TIn>(q, k, dout, rec, io.dS_T, io.dv, xc, pr, bp, 1u, st);
    launch_cgrad<D, TIn>(q, k, u, dout, rec, ck, nend, xc, io.dv, io.dn_T, X, io.dq, io.dk, io.du,
                         nullptr, trw, pr, bp, st);
  }
  if (io.dlambda0 != nullptr)
    VLA_LAUNCH("k_bw_lambda", (k_bw_lambda<D>), dim3(S), dim3(64), 0, st,
               static_cast<const float *>(X), static_cast<const double *>(trw), io.dlambda0, bp.P);
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_bw_dt(const Problem &p, int chunk, const BackwardIO &io, void *ws, hipStream_t st) {
  switch (p.d) {
    case 32: return launch_bw_t<32, TIn>(p, chunk, io, ws, st);
    case 64: return launch_bw_t<64, TIn>(p, chunk, io, ws, st);
    case 96: return launch_bw_t<96, TIn>(p, chunk, io, ws, st);
    case 128: return launch_bw_t<128, TIn>(p, chunk, io, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t backward_workspace_bytes(const Problem &p, int chunk) { return make_bw_plan(p, chunk).total; }

hipError_t launch_backward(const Problem &p, int chunk, const BackwardIO &io, void *ws,
                           hipStream_t stream) {
  if (chunk > 0 && !chunk_supported(p, chunk)) return hipErrorInvalidValue;
  if (p.dtype == Dtype::F32) return launch_bw_dt<float>(p, chunk, io, ws, stream);
  return launch_bw_dt<bf16_t>(p, chunk, io, ws, stream);
}

}  // namespace vla
