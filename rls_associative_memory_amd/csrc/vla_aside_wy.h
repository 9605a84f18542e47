// A side of the chunked path on the bf16 matrix cores (bf16 inputs).
//
// Per segment (one workgroup of d/16 waves) the inverse penalty A starts from the
// segment-start inverse and advances 32 tokens at a time.  For a chunk with rows U, K
// (raw bf16 u_t, k_t) the Sherman-Morrison recursion of the VLA summary (§2.2, §2.3
// step 1) is equivalent to (Woodbury, with G = I + U A U^T = L D L^T, L unit lower):
//   Z  = L^{-1} (U A)        row j is z_j = A_{j-1} u_j,  D_jj = delta_j
//   Y  = K A - tril0(K Z^T) D^{-1} Z          row j is A_j k_j (gate before normalising)
//   A <- A - Z^T D^{-1} Z
// and ahat_j = Y_j / ||Y_j|| (§2.3 step 2; the key's norm cancels), written as its two bf16
// terms (hi, then the residual lo) in a row of 2d per token, which the S passes use as they are.
//
// Layout.  Wave w holds column tile w of A (16 columns, all rows) in MFMA accumulators.
// Because A is symmetric, those registers are also row tile w of A, i.e. exactly the
// A operand of A [U^T | K^T] for rows 16w..16w+15, so A never goes through LDS; each
// fp32 operand is split into NTERM bf16 terms right before use: two terms (hi + lo, about 16
// significant bits), or three (about 24 bits) where the steps cancel strongly: with u_t of
// norm ~ sqrt(d) and a small lambda0, A_t k_t is a difference of terms up to
// 1 + ||u||^2 / lambda0 times larger than itself while fewer than d directions have been
// seen.  Products with the raw bf16 inputs take one MFMA per term; products of two derived
// fp32 operands take the term pairs (i, j) with i + j < NTERM (the dropped ones are near
// 2^-8 NTERM relative), all accumulated in fp32 by v_mfma_f32_16x16x32_bf16.
#pragma once

#include "vla_common.h"
#include "vla_mfma.h"

namespace vla {

template <int D, int TERMS = 2>
struct AwyCfg {
  static constexpr int NW = D / 16;
  static constexpr int NT = NW * kWave;  // = 4 D
  static constexpr int C = 32;           // tokens per chunk
  static constexpr int NKS = D / 32;     // 32-wide feature slices (D = 32 -> 1)
  static constexpr int LDU = D + 8;      // padded bf16 row stride of token rows
  static constexpr int LDL = 40;         // padded bf16 row stride of the 32 x 32 matrices
  static constexpr int NTERM = TERMS;    // bf16 terms per fp32 operand (2 or 3)
  static_assert(D % 32 == 0, "feature dimension must be a multiple of 32");
};

template <int D, int TERMS>
struct AwyLds {
  using C = AwyCfg<D, TERMS>;
  uint16_t sU[C::C][C::LDU];
  uint16_t sK[C::C][C::LDU];
  uint16_t Zr[C::NTERM][C::C][C::LDU];          // row-major Z0 terms, later W terms
  uint16_t Zb[C::NTERM][C::C][C::LDU];          // row-major Z terms
  float G[C::C][C::C + 4];               // I + U A U^T (lower part used); then L^{-1}, row-major
  union {                                       // live in different phases of a chunk
    uint16_t LX[C::NTERM][C::C][C::LDL];        // X~ terms (B operand), after the factorisation
    float lw[4][16][20];                        // blocked LDL^T scratch, during it
  } __attribute__((aligned(16)));
  float rsd[C::C], rd[C::C];
  float nbuf[2][D] __attribute__((aligned(16)));  // sum of phi(k) before the chunk
  float dpart[C::NKS][C::C], apart[C::NKS][C::C], kpart[C::NKS][C::C];  // per-slice shares
  float norm[C::NW][C::C];                       // partial ||Y_c||^2 per wave
};

// Two workgroups share a CU only when each stays within 128 VGPRs and about 53 KB of LDS:
// a workgroup's waves are placed from the first SIMD on, so with six waves (d = 96) two of the
// SIMDs hold four waves of two workgroups and the other two hold two, and larger LDS requests
// leave room for one workgroup only (both measured on gfx950).  d = 64 and d = 96 with two-term
// operands are compiled for four waves per SIMD; with one workgroup per CU the scheduler keeps
// its choice.  NSEG = 2 runs the same segment of two streams (2 s' and 2 s' + 1 for
// blockIdx.x = s') in one workgroup of twice the waves, each half with its own LDS: at d = 96
// twelve waves, three on every SIMD of the CU.  Every stream has the same T, so the two halves
// run the same chunks and meet at every barrier.  On 32 x 131072 tokens at d = 96, in one
// launch, 2.36 -> 2.22 ms.
template <int D, int TERMS, int NSEG = 1>
constexpr int awy_waves_per_simd() {
  return NSEG == 2 ? 3 : (TERMS == 2 && (D == 64 || D == 96)) ? 4 : 1;
}

// With REC the kernel also writes its part of the backward's token records (z, ahat in fp32,
// delta, ||A khat||) and the A half of the state checkpoints (brec, bck: BwRec layout).
template <int D, int TERMS, bool REC = false, int NSEG = 1>
__global__ void __launch_bounds__((NSEG * AwyCfg<D, TERMS>::NT))
__attribute__((amdgpu_waves_per_eu(awy_waves_per_simd<D, TERMS, NSEG>())))
k_aside_wy(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
           const bf16_t *__restrict__ u, const float *__restrict__ A0,
           float *__restrict__ nk, uint16_t *__restrict__ ahat, float *__restrict__ rkden,
           float *__restrict__ A_final, int64_t T, int64_t L,
           int64_t P, float eps, float *__restrict__ brec, float *__restrict__ bck) {
  using C = AwyCfg<D, TERMS>;
  constexpr int NW = C::NW, NT = C::NT, CH = C::C, NTM = C::NTERM;
  constexpr int ZR_T = CH * C::LDU;       // term stride of Zr
  constexpr int LX_T = CH * C::LDL;       // term stride of LX
  // The chunk buffers, or (after the last chunk) A_T being symmetrised.
  union Shared {
    AwyLds<D, TERMS> sh;
    float sym[D][D + 1];
  };
  static_assert(NSEG == 1 || NSEG == 2, "one or two streams per workgroup");
  __shared__ __attribute__((aligned(16))) Shared shus[NSEG];
  // the workgroup's half (its stream), uniform over each wave
  const int half = NSEG == 1 ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / NT);
  Shared &shu = shus[half];
  AwyLds<D, TERMS> &sh = shu.sh;

  const int64_t s = static_cast<int64_t>(blockIdx.x) * NSEG + half, p = blockIdx.y;
  const int tid = static_cast<int>(threadIdx.x) - NT * half, lane = tid & 63, li = lane & 15, gq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const uint16_t *us = reinterpret_cast<const uint16_t *>(u) + s * T * D;
  const uint16_t *ks = reinterpret_cast<const uint16_t *>(k) + s * T * D;
  const uint16_t *qs = reinterpret_cast<const uint16_t *>(q) + s * T * D;
  uint16_t *al = ahat + s * T * 2 * D;
  float *rd = rkden + s * T * 2;
  constexpr int RF = BwRec<D>::F;
  float *brs = REC ? brec + s * T * RF : nullptr;
  float *bcs = REC ? bck + s * ((T + kBwCk - 1) / kBwCk) * 2 * D * D + D * D : nullptr;  // A halves

  // Column tile w of A: At[it][r] = A[16 it + 4 gq + r][16 w + li].
  f4_t At[NW];
  {
    const float *a0 = A0 + (s * P + p) * D * D;
#pragma unroll
    for (int it = 0; it < NW; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) At[it][r] = a0[(16 * it + 4 * gq + r) * D + 16 * w + li];
  }
  // Readout normaliser from the segment start (sum of phi(k) over the segment's tokens before
  // the chunk), double buffered in LDS: chunk number c reads nbuf[c & 1] and its update is
  // written to nbuf[(c & 1) ^ 1].  The denominators written here omit phi(q) . n_p, n_p the
  // normaliser at the segment start: the final pass adds it once the segment sums written at
  // the end (nk) have been scanned.
  for (int f = tid; f < D; f += NT) sh.nbuf[0][f] = 0.f;

  // Staging: thread tid loads token tid / (D/8), features (tid % (D/8)) * 8 of u and k (q is
  // read only by the denominator waves, straight from memory into registers).
  // Rows past the segment are read as row 0 and zeroed when staged (no select on a load
  // result, which would make the load wait at once); offsets are 32-bit from uniform bases.
  // Every chunk prefetches and stages a next chunk (past the segment's end: its first row,
  // staged as zeros and never read), so no load is left pending across the loop's back edge
  // and the loop head does not wait for the previous chunk's stores.
  uint4 pv[2];
  auto prefetch = [&](int64_t cs, int tid) {
    const int sc = tid / (D / 8), sf0 = (tid % (D / 8)) * 8;
    const uint32_t off = (cs + sc < te) ? static_cast<uint32_t>(sc * D + sf0) : 0u;
    const int64_t cb = (cs < te) ? cs : tb;  // a row of this segment
    pv[0] = *reinterpret_cast<const uint4 *>(us + cb * D + off);
    pv[1] = *reinterpret_cast<const uint4 *>(ks + cb * D + off);
  };
  // Rows of the chunk at cs, staged into LDS; rows past the segment become zeros.
  auto stage = [&](int64_t cs, int tid) {
    const int sc = tid / (D / 8), sf0 = (tid % (D / 8)) * 8;
    const bool ok = cs + sc < te;
    *reinterpret_cast<uint4 *>(&sh.sU[sc][sf0]) = keep_if(ok, pv[0]);
    *reinterpret_cast<uint4 *>(&sh.sK[sc][sf0]) = keep_if(ok, pv[1]);
  };
  prefetch(tb, tid);
  stage(tb, tid);
  // Z0, Z or W (this wave's 16 features x 32 tokens, features-as-rows accumulators) into LDS,
  // row-major by token: a B operand over features as it is, an A or B operand over tokens
  // through the transposing load.
  auto publish = [&](const f4_t (&zt)[2], uint16_t (*buf)[CH][C::LDU]) {
    const int lane = threadIdx.x & 63, li = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      uint32_t w01[NTM], w23[NTM];  // features (f, f + 1) and (f + 2, f + 3), by term
      split_pk<NTM>(zt[ct][0], zt[ct][1], w01);
      split_pk<NTM>(zt[ct][2], zt[ct][3], w23);
      const int c = 16 * ct + li, f = 16 * w + 4 * gq;
#pragma unroll
      for (int t = 0; t < NTM; ++t) {
        *reinterpret_cast<uint2 *>(&buf[t][c][f]) = make_uint2(w01[t], w23[t]);
      }
    }
  };

  for (int64_t c0 = tb; c0 < te; c0 += CH) {
    const int m = static_cast<int>(std::min<int64_t>(CH, te - c0));
    // Opaque per-chunk copies of the lane indices: the addresses derived from them are
    // recomputed each chunk rather than hoisted out of the loop and kept (or spilled).
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o - NT * half, lane = tid & 63, li = lane & 15, gq = lane >> 4;
    // The previous chunk's last readers are done and this chunk's rows (staged during the
    // previous chunk) are visible.  The next chunk's rows are loaded now and staged once
    // this chunk has read its own (after X~).
    __syncthreads();
    prefetch(c0 + CH, tid);
    // The denominator waves' q rows (tokens 16 it + li, their slice's features 4 gq.. and
    // 16 + 4 gq..): used mid-chunk, so one load latency is covered by the products before.
    uint2 qd[2][2];
    if (w >= 1 && w <= C::NKS) {
      const int fa = 32 * (w - 1) + 4 * gq;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int64_t row = (c0 + 16 * it + li < te) ? c0 + 16 * it + li : tb;  // a row of the segment
        qd[it][0] = *reinterpret_cast<const uint2 *>(qs + row * D + fa);
        qd[it][1] = *reinterpret_cast<const uint2 *>(qs + row * D + fa + 16);
      }
    }

    // ---- [Z0^T | P^T] = A [U^T | K^T] (rows 16w.., 32 tokens) ---------------------------
    f4_t Z0t[2], Pt[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) { Z0t[ct] = f4_zero(); Pt[ct] = f4_zero(); }
    // Token rows of U and K for feature slice ksl; the next slice's are loaded before this
    // slice's products so that one LDS latency hides behind the matrix cores.
    auto ld_uk = [&](int ksl, bf16x8_t (&o)[2][2]) {
      const int f0 = 32 * ksl + 4 * gq, f1 = 32 * ksl + 16 + 4 * gq;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        o[ct][0] = ld_bf4x2(&sh.sU[16 * ct + li][f0], &sh.sU[16 * ct + li][f1]);
        o[ct][1] = ld_bf4x2(&sh.sK[16 * ct + li][f0], &sh.sK[16 * ct + li][f1]);
      }
    };
    bf16x8_t uk[2][2][2];
    ld_uk(0, uk[0]);
#pragma unroll
    for (int ksl = 0; ksl < C::NKS; ++ksl) {
      if (ksl + 1 < C::NKS) ld_uk(ksl + 1, uk[(ksl + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this slice's products
      float x[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) { x[r] = At[2 * ksl][r]; x[4 + r] = At[2 * ksl + 1][r]; }
      bf16x8_t af[NTM];
      split_n8<NTM>(x, af);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        Z0t[ct] = mmn_sx<NTM>(af, uk[ksl & 1][ct][0], Z0t[ct]);
        Pt[ct] = mmn_sx<NTM>(af, uk[ksl & 1][ct][1], Pt[ct]);
      }
    }
    // ---- publish Z0 (for G and L^{-1} Z0) -------------------------------------------------
    publish(Z0t, sh.Zr);
    __syncthreads();
    // ---- G = I + U Z0^T on the lower 16-tiles (0,0), (1,0), (1,1) ----------------------
    for (int tile = w; tile < 4; tile += NW) {
      if (tile == 3) {  // upper tile (0,1): zeros, never read as G; later L^{-1}'s zero tile
#pragma unroll
        for (int r = 0; r < 4; ++r) sh.G[4 * gq + r][16 + li] = 0.f;
        continue;
      }
      const int it = (tile == 0) ? 0 : 1, jt = (tile == 2) ? 1 : 0;
      bf16x8_t a[C::NKS], b[C::NKS][NTM];  // all operands first: one LDS latency
#pragma unroll
      for (int ksl = 0; ksl < C::NKS; ++ksl) {
        a[ksl] = ld_bf8(&sh.sU[16 * it + li][32 * ksl + 8 * gq]);
        ld_split_n<NTM>(b[ksl], &sh.Zr[0][16 * jt + li][32 * ksl + 8 * gq], ZR_T);
      }
      __builtin_amdgcn_sched_barrier(0);
      f4_t g = f4_zero();
#pragma unroll
      for (int ksl = 0; ksl < C::NKS; ++ksl) g = mmn_xs<NTM>(a[ksl], b[ksl], g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * it + 4 * gq + r, j = 16 * jt + li;
        sh.G[i][j] = g[r] + (i == j ? 1.f : 0.f);
      }
    }
    __syncthreads();
    // ---- wave 0: G = L D L^T and L^{-1};  waves 1..D/32: readout denominators --------------
    if (w == 0) {
      // The factorisation is the chunk's critical path, and its wave shares a SIMD with a
      // denominator wave (of the other stream at d = 96): it issues first while it runs (the
      // wave's own priority; on 32 x 131072 tokens at d = 96 the A side 1.95-2.00 -> 1.87-1.89 ms
      // per launch).
      __builtin_amdgcn_s_setprio(3);
      // Blocked LDL^T of G in two 16-column panels.  In a panel, lanes hold rows (of G, or of
      // the Schur complement) restricted to the panel's 16 columns, lanes 32..47 hold the
      // columns of the panel block of L^{-1} (starting from the identity), and pivots go two
      // at a time, j and j + 1, broadcast from the row lanes through scalar registers
      // (v_readlane): with d0 = G[j][j], g = G[j + 1][j], every lane first applies pivot j to
      // its entry j + 1,  x[j + 1] -= (g / d0) x[j],  which makes lane r's x[j + 1] the column
      // j + 1 after pivot j (so d1 is lane j + 1's), then both pivots to the entries r > j + 1:
      //   x[r] -= (x[j] / d0) c0[r] + (x[j + 1] / d1) c1[r].
      // For a row this is the elimination (the rows below the panel end holding L21 D1); for
      // any other vector b it is the forward substitution b <- L^{-1} b.  Between the panels
      // two 16 x 16 products run on the fp32 matrix core (k = 4 gq + s):
      //   S22 = G22 - (L21 D1) D1^{-1} (L21 D1)^T,   N = L21 L11^{-1},
      // and panel 1 carries the columns of -N (lanes 32..47) and of I (lanes 48..63), which
      // leave it as the columns of L^{-1}_21 = -L22^{-1} N and of L22^{-1}.  L^{-1} is written
      // row-major over G as it is found (G11 after panel 0, G21 and G22 after panel 1); the
      // upper tile of G holds zeros from its construction, which is L^{-1}'s upper tile.
      auto bcast = [](float v, int src) {
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
      };
      auto ldl16 = [&](float (&x)[16], float &myd) {
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
          const int j = 2 * jb;
          const float d0 = bcast(x[j], j), g = bcast(x[j], j + 1);
          const float rd0 = __builtin_amdgcn_rcpf(d0);
          x[j + 1] = fmaf(-g * rd0, x[j], x[j + 1]);
          const float d1 = bcast(x[j + 1], j + 1);
          const float t1 = x[j] * rd0, t2 = x[j + 1] * __builtin_amdgcn_rcpf(d1);
          if (lane == j) myd = d0;
          if (lane == j + 1) myd = d1;
#pragma unroll
          for (int r = j + 2; r < 16; ++r)
            x[r] = fmaf(-t2, bcast(x[j + 1], r), fmaf(-t1, bcast(x[j], r), x[r]));
        }
      };
      auto wsync = []() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      };
      const bool lrl = lane >= 32 && lane < 48;  // L^{-1} column lanes
      const int mcol = lane - 32;
      float (*Wb)[20] = sh.lw[0];   // L21 D1, row-major
      float (*Sb)[20] = sh.lw[1];   // S22, row-major
      float (*L1)[20] = sh.lw[2];   // L11^{-1} transposed: L1[m][r] = L11^{-1}[r][m]
      float (*Nt)[20] = sh.lw[3];   // -N transposed: Nt[m][r] = -N[r][m]
      // ---- panel 0: rows 0..31 of G, columns 0..15 ----
      float x[16];
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const f4_t gv = *reinterpret_cast<const f4_t *>(&sh.G[lane & 31][4 * c4]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[4 * c4 + e] = lane < 32 ? gv[e] : ((lrl && 4 * c4 + e == mcol) ? 1.f : 0.f);
      }
      float myd0 = 1.f;
      ldl16(x, myd0);
      if (lane < 16) {
        sh.rd[lane] = __builtin_amdgcn_rcpf(myd0);
        sh.rsd[lane] = rsqrtf(myd0);
        if constexpr (REC)
          if (lane < m) brs[(c0 + lane) * RF + BwRec<D>::SC] = myd0;  // delta: the LDL^T pivot
      } else if (lane < 32) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
          *reinterpret_cast<f4_t *>(&Wb[lane - 16][4 * c4]) = f4_t{x[4 * c4], x[4 * c4 + 1], x[4 * c4 + 2], x[4 * c4 + 3]};
      } else if (lrl) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
          *reinterpret_cast<f4_t *>(&L1[mcol][4 * c4]) = f4_t{x[4 * c4], x[4 * c4 + 1], x[4 * c4 + 2], x[4 * c4 + 3]};
#pragma unroll
        for (int r = 0; r < 16; ++r) sh.G[r][mcol] = x[r];  // L^{-1}_11, row-major
      }
      wsync();
      // ---- S22 = G22 - W D1^{-1} W^T and N = (W D1^{-1}) L11^{-1}, W = L21 D1 ----
      {
        f4_t acc = f4_zero(), nacc = f4_zero();
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int pp = 4 * gq + s4;
          const float wv = Wb[li][pp];
          const float lv = wv * sh.rd[pp];
          acc = mfma_f32_16x16x4(lv, wv, acc);
          nacc = mfma_f32_16x16x4(lv, L1[li][pp], nacc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Sb[4 * gq + r][li] = sh.G[16 + 4 * gq + r][16 + li] - acc[r];
        *reinterpret_cast<f4_t *>(&Nt[li][4 * gq]) = f4_t{-nacc[0], -nacc[1], -nacc[2], -nacc[3]};
      }
      wsync();
      // ---- panel 1: rows of S22 in lanes 0..15, -N e_m in lanes 32..47, e_m in 48..63 ----
      float y[16];
      {
        const float *src = lane < 16 ? &Sb[lane][0] : &Nt[mcol & 15][0];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const f4_t sv = *reinterpret_cast<const f4_t *>(src + 4 * c4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            y[4 * c4 + e] = (lane < 16 || lrl) ? sv[e] : ((lane >= 48 && 4 * c4 + e == lane - 48) ? 1.f : 0.f);
        }
      }
      float myd1 = 1.f;
      ldl16(y, myd1);
      if (lane < 16) {
        sh.rd[16 + lane] = __builtin_amdgcn_rcpf(myd1);
        sh.rsd[16 + lane] = rsqrtf(myd1);
        if constexpr (REC)
          if (16 + lane < m) brs[(c0 + 16 + lane) * RF + BwRec<D>::SC] = myd1;
      } else if (lane >= 32) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sh.G[16 + r][mcol] = y[r];  // L^{-1}_21 | L^{-1}_22
      }
      __builtin_amdgcn_s_setprio(0);
    } else if (w <= C::NKS) {
      // Readout denominators, key norms and the normaliser update of the chunk, one 32-feature
      // slice per wave (slice w - 1), on the matrix cores of waves that are otherwise idle
      // here.  With M = phi(Q) phi(K)^T and n0 the sum of phi(k) before the chunk,
      //   den_c = phi(q_c) . n0 + sum_{i <= c} M[c][i] + eps,
      // each slice giving its share of both sums and of ||k_c||^2; the shares are added after
      // the barrier.  The slice's features of n advance by the column sums of phi(K).
      const int sl = w - 1;
      const int pc = static_cast<int>((c0 - tb) / CH) & 1;
      const float *n0 = sh.nbuf[pc];
      const int fa = 32 * sl + 4 * gq, fb = fa + 16;
      const f4_t na = *reinterpret_cast<const f4_t *>(&n0[fa]);
      const f4_t nb = *reinterpret_cast<const f4_t *>(&n0[fb]);
      Split2 aq[2], ak[2];
      float asum[2], ksq[2], ncol[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ncol[e] = 0.f;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const bf16x8_t qr = __builtin_bit_cast(bf16x8_t, make_uint4(qd[it][0].x, qd[it][0].y, qd[it][1].x, qd[it][1].y));
        const bf16x8_t kr = ld_bf4x2(&sh.sK[16 * it + li][fa], &sh.sK[16 * it + li][fb]);
        const bool valid = 16 * it + li < m;
        float qv[8], kv[8];
        asum[it] = 0.f;
        ksq[it] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qv[e] = phi(static_cast<float>(qr[e]));
          asum[it] = fmaf(qv[e], e < 4 ? na[e] : nb[e - 4], asum[it]);
          const float kf = static_cast<float>(kr[e]);
          ksq[it] = fmaf(kf, kf, ksq[it]);
          kv[e] = phi(kf);
          ncol[e] += valid ? kv[e] : 0.f;
        }
        aq[it] = split2(qv);
        ak[it] = split2(kv);
      }
      // M tiles over this slice: m00 = (0,0), m10 = (1,0), m11 = (1,1);
      // element r of a tile is M[16 it + 4 gq + r][16 jt + li]
      const f4_t m00 = mm2_ss(aq[0], ak[0], f4_zero());
      const f4_t m10 = mm2_ss(aq[1], ak[0], f4_zero());
      const f4_t m11 = mm2_ss(aq[1], ak[1], f4_zero());
      float rs0[4], rs1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * gq + r;
        rs0[r] = row_sum16(li <= i ? m00[r] : 0.f);
        rs1[r] = row_sum16(m10[r] + (li <= i ? m11[r] : 0.f));
      }
#pragma unroll
      for (int it = 0; it < 2; ++it) {  // token 16 it + li: sums over the four lane groups
        asum[it] = sum_rows4(asum[it]);
        ksq[it] = sum_rows4(ksq[it]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ncol[e] = row_sum16(ncol[e]);
      if (li == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sh.dpart[sl][4 * gq + r] = rs0[r];
          sh.dpart[sl][16 + 4 * gq + r] = rs1[r];
        }
        *reinterpret_cast<f4_t *>(&sh.nbuf[pc ^ 1][fa]) = na + f4_t{ncol[0], ncol[1], ncol[2], ncol[3]};
        *reinterpret_cast<f4_t *>(&sh.nbuf[pc ^ 1][fb]) = nb + f4_t{ncol[4], ncol[5], ncol[6], ncol[7]};
      }
      if (gq == 0) {
        sh.apart[sl][li] = asum[0];
        sh.apart[sl][16 + li] = asum[1];
        sh.kpart[sl][li] = ksq[0];
        sh.kpart[sl][16 + li] = ksq[1];
      }
    }
    __syncthreads();
    // the chunk's (1/||k||, den) from the slices' shares
    if (w == NW - 1 && lane < CH) {
      float den = eps, kk = 0.f;
#pragma unroll
      for (int sl = 0; sl < C::NKS; ++sl) {
        den += sh.dpart[sl][lane] + sh.apart[sl][lane];
        kk += sh.kpart[sl][lane];
      }
      const float rkv = kk > 0.f ? rsqrtf(kk) : 0.f;
      if (lane < m) *reinterpret_cast<float2 *>(&rd[(c0 + lane) * 2]) = make_float2(rkv, den);
      if constexpr (REC) sh.kpart[0][lane] = rkv;  // read back for ||A khat|| (kpart is free until the next chunk)
    }
    // ---- Z^T = Z0^T L^{-T} ---------------------------------------------------------------
    f4_t Zt[2];
    {
      bf16x8_t a[NTM];
      f4_t l[2][2];
      ld_tr_n<NTM>(a, &sh.Zr[0][0][0], ZR_T, C::LDU, 8 * gq, 8 * gq + 4, 16 * w, li);  // Z0^T
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        l[ct][0] = *reinterpret_cast<const f4_t *>(&sh.G[16 * ct + li][8 * gq]);
        l[ct][1] = *reinterpret_cast<const f4_t *>(&sh.G[16 * ct + li][8 * gq + 4]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        bf16x8_t b[NTM];
        const float lv[8] = {l[ct][0][0], l[ct][0][1], l[ct][0][2], l[ct][0][3],
                             l[ct][1][0], l[ct][1][1], l[ct][1][2], l[ct][1][3]};
        split_n8<NTM>(lv, b);
        Zt[ct] = mmn_ss<NTM>(a, b, f4_zero());
      }
    }
    if constexpr (REC) {  // z_t = A_{t-1} u_t: this wave's 16 features of each token
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int c = 16 * ct + li;
        if (c < m)
          *reinterpret_cast<float4 *>(&brs[(c0 + c) * RF + BwRec<D>::Z + 16 * w + 4 * gq]) =
              make_float4(Zt[ct][0], Zt[ct][1], Zt[ct][2], Zt[ct][3]);
      }
    }
    // ---- publish Z into the second buffer (for K Z^T and X~ Z) ----------------------------
    publish(Zt, sh.Zb);
    __syncthreads();
    // ---- X~ = tril0(K Z^T) D^{-1} on tiles (0,0), (1,0), (1,1); the (0,1) tile is zero --
    for (int tile = w; tile < 4; tile += NW) {
      if (tile == 3) {  // X~ is lower triangular: the (0,1) tile is zero
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * gq + r, j = 16 + li;
#pragma unroll
          for (int t = 0; t < NTM; ++t) sh.LX[t][i][j] = 0;
        }
        continue;
      }
      const int it = (tile == 0) ? 0 : 1, jt = (tile == 2) ? 1 : 0;
      bf16x8_t a[C::NKS], b[C::NKS][NTM];  // all operands first: one LDS latency
#pragma unroll
      for (int ksl = 0; ksl < C::NKS; ++ksl) {
        a[ksl] = ld_bf8(&sh.sK[16 * it + li][32 * ksl + 8 * gq]);
        ld_split_n<NTM>(b[ksl], &sh.Zb[0][16 * jt + li][32 * ksl + 8 * gq], ZR_T);
      }
      __builtin_amdgcn_sched_barrier(0);
      f4_t hacc = f4_zero();
#pragma unroll
      for (int ksl = 0; ksl < C::NKS; ++ksl) hacc = mmn_xs<NTM>(a[ksl], b[ksl], hacc);
      const int j = 16 * jt + li;
      const float rdj = sh.rd[j];
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const int i = 16 * it + 4 * gq + r;
        uint32_t tm[NTM];
        split_pk<NTM>((j <= i) ? hacc[r] * rdj : 0.f, (j <= i + 1) ? hacc[r + 1] * rdj : 0.f, tm);
#pragma unroll
        for (int t = 0; t < NTM; ++t) {
          sh.LX[t][i][j] = static_cast<uint16_t>(tm[t]);
          sh.LX[t][i + 1][j] = static_cast<uint16_t>(tm[t] >> 16);
        }
      }
    }
    __syncthreads();
    // the next chunk's rows (sU, sK are not read again in this chunk)
    stage(c0 + CH, tid);
    // ---- W = D^{-1/2} Z into the first buffer (Z0 is no longer read) ----------------------
    {
      f4_t Ws[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float sc2 = sh.rsd[16 * ct + li];
#pragma unroll
        for (int r = 0; r < 4; ++r) Ws[ct][r] = Zt[ct][r] * sc2;
      }
      publish(Ws, sh.Zr);
    }
    // ---- Y^T = P^T - Z^T X~^T, then the gates ----------------------------------------------
    f4_t Yt[2];
    bf16x8_t za[NTM], xb[2][NTM];
    ld_tr_n<NTM>(za, &sh.Zb[0][0][0], ZR_T, C::LDU, 8 * gq, 8 * gq + 4, 16 * w, li);  // Z^T
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) ld_split_n<NTM>(xb[ct], &sh.LX[0][16 * ct + li][8 * gq], LX_T);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const f4_t xz = mmn_ss<NTM>(za, xb[ct], f4_zero());
#pragma unroll
      for (int r = 0; r < 4; ++r) Yt[ct][r] = Pt[ct][r] - xz[r];
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) part = fmaf(Yt[ct][r], Yt[ct][r], part);
      part = sum_rows4(part);
      if (gq == 0) sh.norm[w][16 * ct + li] = part;
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int c = 16 * ct + li;
      float tot = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) tot += sh.norm[w2][c];
      const float inv = tot > 0.f ? rsqrtf(tot) : 0.f;
      if (c < m) {
        // ahat as its two bf16 terms, hi then lo, each token's row [term][d]: the S passes
        // take the terms as they are
        // (the fp32 value is rounded first, not contracted into the residuals of the split)
        float a4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a4[r] = Yt[ct][r] * inv;
          asm volatile("" : "+v"(a4[r]));
        }
        uint32_t w01[2], w23[2];
        split_pk<2>(a4[0], a4[1], w01);
        split_pk<2>(a4[2], a4[3], w23);
        uint16_t *row = &al[c0 * 2 * D + static_cast<uint32_t>(c * 2 * D + 16 * w + 4 * gq)];
        *reinterpret_cast<uint2 *>(row) = make_uint2(w01[0], w23[0]);
        *reinterpret_cast<uint2 *>(row + D) = make_uint2(w01[1], w23[1]);
        if constexpr (REC) {  // ahat in fp32, and ||A_t khat|| = ||Y_t|| / ||k_t||
          float *rr = &brs[(c0 + c) * RF];
          *reinterpret_cast<float4 *>(&rr[BwRec<D>::AH + 16 * w + 4 * gq]) = make_float4(a4[0], a4[1], a4[2], a4[3]);
          if (w == 0 && gq == 0) rr[BwRec<D>::SC + 1] = sqrtf(tot) * sh.kpart[0][c];
        }
      }
    }
    // ---- A <- A - W^T W on this wave's column tile ------------------------------------------
    {
      bf16x8_t b[NTM], a[2][NTM];
      ld_tr_n<NTM>(b, &sh.Zr[0][0][0], ZR_T, C::LDU, 8 * gq, 8 * gq + 4, 16 * w, li);
      ld_tr_n<NTM>(a[0], &sh.Zr[0][0][0], ZR_T, C::LDU, 8 * gq, 8 * gq + 4, 0, li);
#pragma unroll
      for (int it = 0; it < NW; ++it) {
        if (it + 1 < NW)  // next row tile's operand first
          ld_tr_n<NTM>(a[(it + 1) & 1], &sh.Zr[0][0][0], ZR_T, C::LDU, 8 * gq, 8 * gq + 4, 16 * (it + 1), li);
        __builtin_amdgcn_sched_barrier(0);
        const f4_t t4 = mmn_ss<NTM>(a[it & 1], b, f4_zero());
#pragma unroll
        for (int r = 0; r < 4; ++r) At[it][r] -= t4[r];
      }
    }
    if (REC && ((c0 + m) % kBwCk == 0 || c0 + m == te)) {  // A after a checkpoint token
      float *dst = bcs + ((c0 + m - 1) / kBwCk) * 2 * D * D;
#pragma unroll
      for (int it = 0; it < NW; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * it + 4 * gq + r) * D + 16 * w + li] = At[it][r];
    }
  }

  {
    // the segment's sum of phi(k) (chunk c writes nbuf[(c & 1) ^ 1]), before any reuse of the
    // LDS below
    __syncthreads();
    const int nch = static_cast<int>((te - tb + CH - 1) / CH);
    for (int f = tid; f < D; f += NT) nk[(s * P + p) * D + f] = sh.nbuf[nch & 1][f];
  }
  if (A_final != nullptr && p == P - 1) {
    // Symmetrise through LDS: A_T <- (A + A^T) / 2.
    __syncthreads();
    float(*sym)[D + 1] = shu.sym;
#pragma unroll
    for (int it = 0; it < NW; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) sym[16 * it + 4 * gq + r][16 * w + li] = At[it][r];
    __syncthreads();
    float *dst = A_final + s * D * D;
    for (int e = tid; e < D * D; e += NT) {
      const int i = e / D, j = e % D;
      dst[e] = 0.5f * (sym[i][j] + sym[j][i]);
    }
  }
}

}  // namespace vla
