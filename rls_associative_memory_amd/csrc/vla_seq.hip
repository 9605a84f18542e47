// Sequential VLA forward: one workgroup per (batch, head) stream, token by token.
//
// Recurrence (VLA summary = gist.science technical summary of "Variational Linear
// Attention: Stable Associative Memory for Long-Context Transformers"):
//   z = A u, delta = 1 + u.z, A <- A - z z^T / delta          §2.3 step 1
//   ahat = A khat / ||A khat||                                 §2.3 step 2
//   S <- S + (v - S khat) ahat^T                               §2.3 step 3
//   o = S phi(q) / (n.phi(q) + eps), n <- n + phi(k)           §2.3 readout (ELU+1)
//
// Layout.  The workgroup has an A side and an S side, each of NWA waves (1 for d <= 96,
// 2 for d = 128).  On each side lane l owns rows g + j*(lanes/2) (g = l >> 1, j < RPL) and
// the column half h = l & 1 of those rows, so a row is split over a lane pair: a
// matrix-vector product is CW fused multiply-adds per row plus one DPP exchange.  A and S
// live in VGPRs for the whole sequence; the per-token vectors (z / sqrt(delta) and ahat)
// are broadcast through LDS.  The A side never depends on S, so the two sides run as a
// two-stage pipeline: in phase p the A side handles token p while the S side handles
// token p-1, with one workgroup barrier per phase (d <= 96).
//
// Tokens are staged CT at a time: 16-byte coalesced global loads of the next tile are
// issued into registers before the current tile is processed (register double
// buffering), then widened to fp32 in LDS together with phi(q), phi(k) and the running
// normaliser products n_t[c] * phi(q_t)[c].
//
// Symmetry of A is kept exactly: the downdate is A[r][c] -= w_r * w_c with
// w = z / sqrt(delta) computed identically for row and column use, and every
// cross-lane sum is symmetric so all lanes hold bitwise-equal scalars.

#include "vla_common.h"
#include "vla_internal.h"

namespace vla {

template <int D>
struct SeqCfg {
  static constexpr int NWA = (D > 96) ? 2 : 1;   // waves per side
  static constexpr int NW = 2 * NWA;
  static constexpr int NT = NW * kWave;
  static constexpr int LA = NWA * kWave;         // lanes per side
  static constexpr int HALF = LA / 2;            // row stride between a lane's rows
  static constexpr int CW = D / 2;               // columns per lane
  static constexpr int RPL = D / HALF;           // rows per lane
  static constexpr int CT = (D <= 64) ? 32 : 16; // tokens per tile
  static_assert(D % HALF == 0 && CW % 4 == 0, "unsupported d");
};

template <int D, typename TIn>
__global__ void __launch_bounds__(SeqCfg<D>::NT)
vla_seq_kernel(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
               const TIn *__restrict__ u, TIn *__restrict__ out, float *__restrict__ S_final,
               float *__restrict__ A_final, const float *__restrict__ S0,
               const float *__restrict__ A0, const float *__restrict__ n0,
               float *__restrict__ n_final, int64_t T, float lambda0, float eps, int raw_gain) {
  using C = SeqCfg<D>;
  using IO = io<TIn>;
  constexpr int VW = IO::kVec;
  constexpr int CHUNKS = C::CT * D / VW;                 // 16-byte chunks per array per tile
  constexpr int PF = (CHUNKS + C::NT - 1) / C::NT;       // chunks per thread per array

  __shared__ __attribute__((aligned(16))) float sU[C::CT][D];
  __shared__ __attribute__((aligned(16))) float sK[C::CT][D];
  __shared__ __attribute__((aligned(16))) float sV[C::CT][D];   // v, then o in place
  __shared__ __attribute__((aligned(16))) float sFQ[C::CT][D];  // phi(q)
  __shared__ __attribute__((aligned(16))) float sP[C::CT][D];   // phi(k), then n*phi(q)
  __shared__ __attribute__((aligned(16))) float sW[D];          // z / sqrt(delta)
  __shared__ __attribute__((aligned(16))) float sAl[2][D];      // ahat, two slots
  __shared__ float sAphi[2];                                    // ahat . phi(q)
  __shared__ float sRed[2][C::NWA][2];                          // cross-wave partials

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const bool is_a = wave < C::NWA;
  const int ls = is_a ? tid : tid - C::LA;  // lane index within the side
  const int h = ls & 1;
  const int g = ls >> 1;
  const int c0 = h * C::CW;
  const int wside = ls / kWave;              // wave index within the side

  const int64_t sid = blockIdx.x;
  const int64_t base = sid * T * D;
  const TIn *qs = q + base;
  const TIn *ks = k + base;
  const TIn *vs = v + base;
  const TIn *us = u + base;
  TIn *os = out + base;

  // Matrix state: A on the A side, S on the S side, same registers.  A carried A0 is
  // symmetrised as it is read ((A0 + A0^T) / 2), which keeps A exactly symmetric.
  float M[C::RPL][C::CW];
  const float inv_l0 = 1.0f / lambda0;
  const float *m0 = is_a ? A0 : S0;
  if (m0 != nullptr) {
    m0 += sid * D * D;
#pragma unroll
    for (int j = 0; j < C::RPL; ++j) {
      const int r = g + j * C::HALF;
#pragma unroll
      for (int c = 0; c < C::CW; ++c)
        M[j][c] = is_a ? 0.5f * (m0[r * D + c0 + c] + m0[(c0 + c) * D + r]) : m0[r * D + c0 + c];
    }
  } else {
#pragma unroll
    for (int j = 0; j < C::RPL; ++j) {
      const int r = g + j * C::HALF;
#pragma unroll
      for (int c = 0; c < C::CW; ++c) M[j][c] = (is_a && r == c0 + c) ? inv_l0 : 0.0f;
    }
  }
  // normaliser component tid (tid < D)
  float n_run = (n0 != nullptr && tid < D) ? n0[sid * D + tid] : 0.0f;

  typename IO::vec_t pf[4][PF];
  auto prefetch = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int ch = tid + i * C::NT;
      const int j = (ch * VW) / D;
      const int col = (ch * VW) % D;
      const bool ok = ch < CHUNKS && (t0 + j) < T;
      const int64_t off = (t0 + j) * D + col;
      typename IO::vec_t zero{};
      pf[0][i] = ok ? *reinterpret_cast<const typename IO::vec_t *>(qs + off) : zero;
      pf[1][i] = ok ? *reinterpret_cast<const typename IO::vec_t *>(ks + off) : zero;
      pf[2][i] = ok ? *reinterpret_cast<const typename IO::vec_t *>(vs + off) : zero;
      pf[3][i] = ok ? *reinterpret_cast<const typename IO::vec_t *>(us + off) : zero;
    }
  };

  const int64_t ntiles = (T + C::CT - 1) / C::CT;
  prefetch(0);
  for (int64_t tile = 0; tile < ntiles; ++tile) {
    const int64_t t0 = tile * C::CT;
    const int nt = static_cast<int>((T - t0) < C::CT ? (T - t0) : C::CT);

    // (1) widen the staged tile into LDS.
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int ch = tid + i * C::NT;
      if (ch < CHUNKS) {
        const int j = (ch * VW) / D;
        const int col = (ch * VW) % D;
        float fq[VW], fk[VW], fv[VW], fu[VW];
        IO::unpack(pf[0][i], fq);
        IO::unpack(pf[1][i], fk);
        IO::unpack(pf[2][i], fv);
        IO::unpack(pf[3][i], fu);
#pragma unroll
        for (int e = 0; e < VW; e += 4) {
          *reinterpret_cast<float4 *>(&sU[j][col + e]) = make_float4(fu[e], fu[e + 1], fu[e + 2], fu[e + 3]);
          *reinterpret_cast<float4 *>(&sK[j][col + e]) = make_float4(fk[e], fk[e + 1], fk[e + 2], fk[e + 3]);
          *reinterpret_cast<float4 *>(&sV[j][col + e]) = make_float4(fv[e], fv[e + 1], fv[e + 2], fv[e + 3]);
          *reinterpret_cast<float4 *>(&sFQ[j][col + e]) =
              make_float4(phi(fq[e]), phi(fq[e + 1]), phi(fq[e + 2]), phi(fq[e + 3]));
          *reinterpret_cast<float4 *>(&sP[j][col + e]) =
              make_float4(phi(fk[e]), phi(fk[e + 1]), phi(fk[e + 2]), phi(fk[e + 3]));
        }
      }
    }
    __syncthreads();

    // (2) next tile's global loads go in flight now.
    if (tile + 1 < ntiles) prefetch(t0 + C::CT);

    // (3) normaliser: n_t = n_{t-1} + phi(k_t); store n_t[c] * phi(q_t)[c].
    if (tid < D) {
      for (int j = 0; j < nt; ++j) {
        n_run += sP[j][tid];
        sP[j][tid] = n_run * sFQ[j][tid];
      }
    }
    __syncthreads();

    // (4) two-stage pipeline over the tile's tokens.
    for (int p = 0; p <= nt; ++p) {
      if (is_a) {
        if (p < nt) {
          const int j = p;
          const int slot = p & 1;
          float z[C::RPL], a[C::RPL];
#pragma unroll
          for (int r = 0; r < C::RPL; ++r) { z[r] = 0.f; a[r] = 0.f; }
          float kk = 0.f;
#pragma unroll
          for (int m = 0; m < C::CW / 4; ++m) {
            const float4 u4 = *reinterpret_cast<const float4 *>(&sU[j][c0 + 4 * m]);
            const float4 k4 = *reinterpret_cast<const float4 *>(&sK[j][c0 + 4 * m]);
            kk = fmaf(k4.x, k4.x, kk); kk = fmaf(k4.y, k4.y, kk);
            kk = fmaf(k4.z, k4.z, kk); kk = fmaf(k4.w, k4.w, kk);
#pragma unroll
            for (int r = 0; r < C::RPL; ++r) {
              z[r] = fmaf(M[r][4 * m + 0], u4.x, z[r]);
              a[r] = fmaf(M[r][4 * m + 0], k4.x, a[r]);
              z[r] = fmaf(M[r][4 * m + 1], u4.y, z[r]);
              a[r] = fmaf(M[r][4 * m + 1], k4.y, a[r]);
              z[r] = fmaf(M[r][4 * m + 2], u4.z, z[r]);
              a[r] = fmaf(M[r][4 * m + 2], k4.z, a[r]);
              z[r] = fmaf(M[r][4 * m + 3], u4.w, z[r]);
              a[r] = fmaf(M[r][4 * m + 3], k4.w, a[r]);
            }
          }
          kk = pair_sum(kk);
          const float rk = kk > 0.f ? rsqrtf(kk) : 0.f;
          float sd = 0.f, sg = 0.f;
#pragma unroll
          for (int r = 0; r < C::RPL; ++r) {
            const int row = g + r * C::HALF;
            z[r] = pair_sum(z[r]);
            a[r] = pair_sum(a[r]) * rk;           // A_{t-1} khat
            sd = fmaf(sU[j][row], z[r], sd);        // u . z
            sg = fmaf(sK[j][row] * rk, z[r], sg);   // khat . z
          }
          if (h) { sd = 0.f; sg = 0.f; }
          sd = wave_sum(sd);
          sg = wave_sum(sg);
          if constexpr (C::NWA > 1) {
            if ((ls & (kWave - 1)) == 0) { sRed[0][wside][0] = sd; sRed[0][wside][1] = sg; }
            __syncthreads();
            sd = 0.f; sg = 0.f;
#pragma unroll
            for (int w = 0; w < C::NWA; ++w) { sd += sRed[0][w][0]; sg += sRed[0][w][1]; }
          }
          const float delta = 1.0f + sd;
          const float cz = sg / delta;
          float y[C::RPL];
          float sy = 0.f, sq = 0.f;
#pragma unroll
          for (int r = 0; r < C::RPL; ++r) {
            const int row = g + r * C::HALF;
            y[r] = fmaf(-cz, z[r], a[r]);           // A_t khat = A_{t-1} khat - z (z.khat)/delta
            sy = fmaf(y[r], y[r], sy);
            sq = fmaf(y[r], sFQ[j][row], sq);
          }
          if (h) { sy = 0.f; sq = 0.f; }
          sy = wave_sum(sy);
          sq = wave_sum(sq);
          if constexpr (C::NWA > 1) {
            if ((ls & (kWave - 1)) == 0) { sRed[1][wside][0] = sy; sRed[1][wside][1] = sq; }
            __syncthreads();
            sy = 0.f; sq = 0.f;
#pragma unroll
            for (int w = 0; w < C::NWA; ++w) { sy += sRed[1][w][0]; sq += sRed[1][w][1]; }
          }
          // unit gain (the method) or, for the ablation, the raw gain A_t khat
          const float inv = raw_gain ? 1.0f : (sy > 0.f ? rsqrtf(sy) : 0.f);
          const float rd = rsqrtf(delta);
          float w[C::RPL];
#pragma unroll
          for (int r = 0; r < C::RPL; ++r) {
            const int row = g + r * C::HALF;
            w[r] = z[r] * rd;
            if (h == 0) {
              sW[row] = w[r];
              sAl[slot][row] = y[r] * inv;
            }
          }
          if (ls == 0) sAphi[slot] = sq * inv;
          if constexpr (C::NWA > 1) {
            __syncthreads();
          } else {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          }
#pragma unroll
          for (int m = 0; m < C::CW / 4; ++m) {
            const float4 w4 = *reinterpret_cast<const float4 *>(&sW[c0 + 4 * m]);
#pragma unroll
            for (int r = 0; r < C::RPL; ++r) {
              M[r][4 * m + 0] = fmaf(-w[r], w4.x, M[r][4 * m + 0]);
              M[r][4 * m + 1] = fmaf(-w[r], w4.y, M[r][4 * m + 1]);
              M[r][4 * m + 2] = fmaf(-w[r], w4.z, M[r][4 * m + 2]);
              M[r][4 * m + 3] = fmaf(-w[r], w4.w, M[r][4 * m + 3]);
            }
          }
        } else if constexpr (C::NWA > 1) {
          __syncthreads();
          __syncthreads();
          __syncthreads();
        }
      } else {
        if (p >= 1) {
          const int j = p - 1;
          const int slot = j & 1;
          float s[C::RPL], pq[C::RPL];
#pragma unroll
          for (int r = 0; r < C::RPL; ++r) { s[r] = 0.f; pq[r] = 0.f; }
          float kk = 0.f, dp = 0.f;
#pragma unroll
          for (int m = 0; m < C::CW / 4; ++m) {
            const float4 k4 = *reinterpret_cast<const float4 *>(&sK[j][c0 + 4 * m]);
            const float4 f4 = *reinterpret_cast<const float4 *>(&sFQ[j][c0 + 4 * m]);
            const float4 p4 = *reinterpret_cast<const float4 *>(&sP[j][c0 + 4 * m]);
            kk = fmaf(k4.x, k4.x, kk); kk = fmaf(k4.y, k4.y, kk);
            kk = fmaf(k4.z, k4.z, kk); kk = fmaf(k4.w, k4.w, kk);
            dp += (p4.x + p4.y) + (p4.z + p4.w);
#pragma unroll
            for (int r = 0; r < C::RPL; ++r) {
              s[r] = fmaf(M[r][4 * m + 0], k4.x, s[r]);
              pq[r] = fmaf(M[r][4 * m + 0], f4.x, pq[r]);
              s[r] = fmaf(M[r][4 * m + 1], k4.y, s[r]);
              pq[r] = fmaf(M[r][4 * m + 1], f4.y, pq[r]);
              s[r] = fmaf(M[r][4 * m + 2], k4.z, s[r]);
              pq[r] = fmaf(M[r][4 * m + 2], f4.z, pq[r]);
              s[r] = fmaf(M[r][4 * m + 3], k4.w, s[r]);
              pq[r] = fmaf(M[r][4 * m + 3], f4.w, pq[r]);
            }
          }
          kk = pair_sum(kk);
          dp = pair_sum(dp);
          const float rk = kk > 0.f ? rsqrtf(kk) : 0.f;
          const float rden = 1.0f / (dp + eps);
          const float aphi = sAphi[slot];
          float res[C::RPL];
#pragma unroll
          for (int r = 0; r < C::RPL; ++r) {
            const int row = g + r * C::HALF;
            s[r] = pair_sum(s[r]) * rk;          // S_{t-1} khat
            pq[r] = pair_sum(pq[r]);             // S_{t-1} phi(q)
            res[r] = sV[j][row] - s[r];          // v - S_{t-1} khat
            const float o = fmaf(res[r], aphi, pq[r]) * rden;  // S_t phi(q) / den
            if (h == 0) sV[j][row] = o;
          }
#pragma unroll
          for (int m = 0; m < C::CW / 4; ++m) {
            const float4 a4 = *reinterpret_cast<const float4 *>(&sAl[slot][c0 + 4 * m]);
#pragma unroll
            for (int r = 0; r < C::RPL; ++r) {
              M[r][4 * m + 0] = fmaf(res[r], a4.x, M[r][4 * m + 0]);
              M[r][4 * m + 1] = fmaf(res[r], a4.y, M[r][4 * m + 1]);
              M[r][4 * m + 2] = fmaf(res[r], a4.z, M[r][4 * m + 2]);
              M[r][4 * m + 3] = fmaf(res[r], a4.w, M[r][4 * m + 3]);
            }
          }
        }
        if constexpr (C::NWA > 1) {
          __syncthreads();
          __syncthreads();
          __syncthreads();
        }
      }
      __syncthreads();
    }

    // (5) outputs of the tile (in sV) to global memory, rounded once to the input dtype.
    {
      constexpr int OCH = C::CT * D / 4;  // float4 chunks
      for (int ch = tid; ch < OCH; ch += C::NT) {
        const int j = (ch * 4) / D;
        const int col = (ch * 4) % D;
        if (j < nt) {
          const float4 o4 = *reinterpret_cast<const float4 *>(&sV[j][col]);
          const int64_t off = (t0 + j) * D + col;
          if constexpr (sizeof(TIn) == 4) {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(os) + off) = o4;
          } else {
            const uint32_t lo = f32_to_bf16(o4.x) | (static_cast<uint32_t>(f32_to_bf16(o4.y)) << 16);
            const uint32_t hi = f32_to_bf16(o4.z) | (static_cast<uint32_t>(f32_to_bf16(o4.w)) << 16);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(os) + off) = make_uint2(lo, hi);
          }
        }
      }
    }
    __syncthreads();
  }

  // Final state.
  if (n_final != nullptr && tid < D) n_final[sid * D + tid] = n_run;
  float *dst = is_a ? A_final : S_final;
  if (dst != nullptr) {
    dst += sid * D * D;
#pragma unroll
    for (int r = 0; r < C::RPL; ++r) {
      const int row = g + r * C::HALF;
#pragma unroll
      for (int m = 0; m < C::CW / 4; ++m)
        *reinterpret_cast<float4 *>(&dst[row * D + c0 + 4 * m]) =
            make_float4(M[r][4 * m], M[r][4 * m + 1], M[r][4 * m + 2], M[r][4 * m + 3]);
    }
  }
}

template <int D, typename TIn>
static hipError_t launch_seq_t(const Problem &p, const void *q, const void *k, const void *v,
                               const void *u, void *out, const StateIO &st, hipStream_t stream) {
  using C = SeqCfg<D>;
  VLA_LAUNCH("vla_seq_kernel", (vla_seq_kernel<D, TIn>), dim3(static_cast<unsigned>(p.streams)),
                     dim3(C::NT), 0, stream, static_cast<const TIn *>(q),
                     static_cast<const TIn *>(k), static_cast<const TIn *>(v),
                     static_cast<const TIn *>(u), static_cast<TIn *>(out), st.S_final, st.A_final,
                     st.S0, st.A0, st.n0, st.n_final, p.T, p.lambda0, p.eps, p.raw_gain ? 1 : 0);
  return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_seq_dt(const Problem &p, const void *q, const void *k, const void *v,
                                const void *u, void *out, const StateIO &st, hipStream_t stream) {
  switch (p.d) {
    case 32: return launch_seq_t<32, TIn>(p, q, k, v, u, out, st, stream);
    case 64: return launch_seq_t<64, TIn>(p, q, k, v, u, out, st, stream);
    case 96: return launch_seq_t<96, TIn>(p, q, k, v, u, out, st, stream);
    case 128: return launch_seq_t<128, TIn>(p, q, k, v, u, out, st, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_seq(const Problem &p, const void *q, const void *k, const void *v,
                      const void *u, void *out, const StateIO &st, hipStream_t stream) {
  if (p.dtype == Dtype::F32) return launch_seq_dt<float>(p, q, k, v, u, out, st, stream);
  return launch_seq_dt<bf16_t>(p, q, k, v, u, out, st, stream);
}

}  // namespace vla
