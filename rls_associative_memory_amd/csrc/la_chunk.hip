// Linear-attention baseline on the same harness as the VLA path (gfx950, wave64).
//
// Standard linear attention with the ELU+1 feature map and the ratio readout the VLA method
// shares with it (VLA summary §2.1: the unconditional accumulation VLA replaces; §2.3,
// closing paragraph: the readout; §2.4 prices VLA at about five times its operations):
//   S_t = S_{t-1} + v_t phi(k_t)^T,  n_t = n_{t-1} + phi(k_t),
//   o_t = S_t phi(q_t) / (n_t . phi(q_t) + eps)
//
// Chunked form over C = 64 tokens from the state (S0, n0) at the chunk start, with rows of
// Fq, Fk, V the chunk's phi(q_t), phi(k_t), v_t and P = tril0(Fq Fk^T) (P[t][s] =
// phi(q_t).phi(k_s) for s <= t):
//   O = Fq S0^T + P V,   den_t = phi(q_t).n0 + sum_s P[t][s] + eps,   o_t = O_t / den_t
//   S_end^T = S0^T + Fk^T V,   n_end = n0 + sum_t phi(k_t)
// Time is split into segments of whole chunks so that a few long streams still fill the
// chip: the state at every segment start is an exclusive prefix sum of the segments'
// (Fk^T V, sum phi(k)), which needs no sequential pass over tokens.
//   k_la_seg     per (stream, segment but the last): Sum Fk^T V and Sum phi(k) over it
//   k_la_prefix  per stream: exclusive prefix over segments, in place
//   k_la_out     per (stream, segment): the chunk recurrence from the segment's start
//                state, writing o and, for the last segment, S_T and n_T
// Products run on v_mfma_f32_16x16x32_bf16 with every fp32 operand split into two bf16
// terms (h + l, about 16 significant bits; the l * l product is dropped); v is one exact
// term when the inputs are bf16.  The normaliser's column sums are taken from the staging
// registers (each thread sums its own rows of four columns, then a fixed-order sum over
// the 16 row groups in LDS), so no wave walks a column of LDS serially.  Wave w of a
// workgroup owns column block w (16 value indices i) of S^T and of O, so the state stays
// in its accumulators for the whole segment; only P, its row sums and the chunk's
// operands go through LDS.

#include "vla_common.h"
#include "vla_internal.h"
#include "vla_mfma.h"

namespace vla {
namespace {

constexpr int LC = 64;  // tokens per chunk

template <int D>
struct LaCfg {
  static constexpr int NW = D / 16;       // waves; wave w owns value block w
  static constexpr int NT = NW * kWave;
  static constexpr int LD = D + 8;        // bf16 row stride: row reads of 4 are conflict-free
  static constexpr int LDP = LC + 8;
  static constexpr int TS = LC * LD;      // term stride of Fq, Fk, V (elements)
  static constexpr int TSP = LC * LDP;    // term stride of P
  static constexpr int GPT = LC * D / 4 / NT;  // 4-element groups per thread and tensor
  static_assert(LC * D / 4 % NT == 0, "whole groups per thread");
  static constexpr int64_t SEG = int64_t(D) * D + D;  // floats per (stream, segment) record
};

template <int D>
struct LaShared {
  uint16_t fq[2][LC][LaCfg<D>::LD];   // phi(q) terms
  uint16_t fk[2][LC][LaCfg<D>::LD];   // phi(k) terms
  uint16_t vv[2][LC][LaCfg<D>::LD];   // v terms
  uint16_t pp[2][LC][LaCfg<D>::LDP];  // P terms, P[t][s]
  float rs[4][LC];                    // row sums of P per 16-key block
  float nq[LC];                       // phi(q_t) . n at the chunk start
  alignas(16) float n[2][D];          // normaliser at the chunk start, by chunk parity
  alignas(16) float part[16][D];      // phi(k) column sums of each staging row group
};

template <int D>
struct LaSegShared {  // the segment sums need only the keys and values
  uint16_t fk[2][LC][LaCfg<D>::LD];
  uint16_t vv[2][LC][LaCfg<D>::LD];
  alignas(16) float part[16][D];
};

// four raw input elements held between the load and the LDS write
template <typename TIn>
struct Raw4;
template <>
struct Raw4<float> {
  float4 r;
  __device__ __forceinline__ void load(const float *p) { r = *reinterpret_cast<const float4 *>(p); }
  __device__ __forceinline__ void zero() { r = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void get(float (&x)[4]) const {
    x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w;
  }
};
template <>
struct Raw4<bf16_t> {
  uint2 r;
  __device__ __forceinline__ void load(const bf16_t *p) { r = *reinterpret_cast<const uint2 *>(p); }
  __device__ __forceinline__ void zero() { r = make_uint2(0u, 0u); }
  __device__ __forceinline__ void get(float (&x)[4]) const {
    x[0] = __uint_as_float(r.x << 16);
    x[1] = __uint_as_float(r.x & 0xffff0000u);
    x[2] = __uint_as_float(r.y << 16);
    x[3] = __uint_as_float(r.y & 0xffff0000u);
  }
};

template <typename TIn>
__device__ __forceinline__ void la_store(TIn *p, float x);
template <>
__device__ __forceinline__ void la_store<float>(float *p, float x) { *p = x; }
template <>
__device__ __forceinline__ void la_store<bf16_t>(bf16_t *p, float x) { p->bits = f32_to_bf16(x); }

// four values as two bf16 terms at h (term stride ts)
__device__ __forceinline__ void put2(uint16_t *h, int ts, const float (&x)[4]) {
  uint32_t a[2], b[2];
  split_pk<2>(x[0], x[1], a);
  split_pk<2>(x[2], x[3], b);
  *reinterpret_cast<uint2 *>(h) = make_uint2(a[0], b[0]);
  *reinterpret_cast<uint2 *>(h + ts) = make_uint2(a[1], b[1]);
}

// four values that are exact in bf16 as their one term at h
__device__ __forceinline__ void put1(uint16_t *h, const float (&x)[4]) {
  *reinterpret_cast<uint2 *>(h) = make_uint2(pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3]));
}

// K = 32 operands of v_mfma_f32_16x16x32_bf16 made of two K = 16 operands: with the
// permuted contraction index of both instructions, elements 0-3 of a lane are k-block 2 m and
// elements 4-7 are k-block 2 m + 1, so a pair of blocks is one instruction at full rate.
struct Split2w {
  bf16x8_t h, l;
};
__device__ __forceinline__ bf16x8_t cat4(const uint2 &a, const uint2 &b) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}
__device__ __forceinline__ Split2w cat2(const Split2h &a, const Split2h &b) {
  return Split2w{cat4(a.h, b.h), cat4(a.l, b.l)};
}
__device__ __forceinline__ f4_t mm2w_ss(const Split2w &a, const Split2w &b, f4_t c) {
  c = mfma_bf16(a.l, b.h, c);
  c = mfma_bf16(a.h, b.l, c);
  return mfma_bf16(a.h, b.h, c);
}
// v as the B operand: exact (VX, one term) or split in two
template <bool VX>
__device__ __forceinline__ f4_t mm_v(const Split2w &a, const Split2w &b, f4_t c) {
  if constexpr (VX) {
    c = mfma_bf16(a.l, b.h, c);
    return mfma_bf16(a.h, b.h, c);
  } else {
    return mm2w_ss(a, b, c);
  }
}
__device__ __forceinline__ Split2h zero2h() { return Split2h{make_uint2(0u, 0u), make_uint2(0u, 0u)}; }

// Chunk operands: group g = tid + NT m covers elements 4 g .. 4 g + 3 of the chunk's
// LC x D block, row t = 4 g / D, columns j = 4 g % D.
template <int D, typename TIn, int NTEN>
struct ChunkLoader {
  using C = LaCfg<D>;
  Raw4<TIn> r[NTEN][C::GPT];
  __device__ __forceinline__ void fetch(const TIn *const (&src)[NTEN], int64_t row0, int64_t tok0,
                                        int64_t T, int tid) {
#pragma unroll
    for (int m = 0; m < C::GPT; ++m) {
      const int g = tid + C::NT * m, t = 4 * g / D, j = 4 * g % D;
      const bool ok = tok0 + t < T;
#pragma unroll
      for (int x = 0; x < NTEN; ++x) {
        if (ok)
          r[x][m].load(src[x] + (row0 + tok0 + t) * D + j);
        else
          r[x][m].zero();
      }
    }
  }
};

// P tile (tb, sb), tb >= sb, of the 10 lower blocks of a 64 x 64 chunk
__device__ __forceinline__ void tile_of(int n, int &tb, int &sb) {
  tb = n < 1 ? 0 : n < 3 ? 1 : n < 6 ? 2 : 3;
  sb = n - tb * (tb + 1) / 2;
}

// S^T[:, 16 w ..] += Fk^T V[:, 16 w ..] over the chunk in LDS; vt holds V's blocks of column
// block w as B operands.
template <int D, bool VX, class Sh>
__device__ __forceinline__ void state_update(f4_t (&ST)[LaCfg<D>::NW], const Sh &sh,
                                             const Split2h (&vt)[4], int gq, int li) {
  using C = LaCfg<D>;
#pragma unroll
  for (int m = 0; m < 2; ++m) {  // token blocks 2 m, 2 m + 1
    const Split2w b = cat2(vt[2 * m], vt[2 * m + 1]);
#pragma unroll
    for (int jb = 0; jb < C::NW; ++jb)
      ST[jb] = mm_v<VX>(cat2(ld2_tr4h(&sh.fk[0][32 * m][16 * jb], C::LD, C::TS, gq, li),
                             ld2_tr4h(&sh.fk[0][32 * m + 16][16 * jb], C::LD, C::TS, gq, li)),
                        b, ST[jb]);
  }
}

template <int D, bool VX, class Sh>
__device__ __forceinline__ void load_vt(Split2h (&vt)[4], const Sh &sh, int w, int gq, int li) {
  using C = LaCfg<D>;
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    const uint16_t *p = &sh.vv[0][16 * sb + 4 * gq + (li >> 2)][16 * w + 4 * (li & 3)];
    vt[sb].h = ld_tr4(p);
    vt[sb].l = VX ? make_uint2(0u, 0u) : ld_tr4(p + C::TS);
  }
}

// Staging thread tid holds rows tid / (D / 4) + 16 m (m < 4) of columns 4 (tid % (D / 4)) .. + 3.
template <int D>
__device__ __forceinline__ int stage_rg(int tid) { return tid / (D / 4); }
template <int D>
__device__ __forceinline__ int stage_col(int tid) { return 4 * (tid % (D / 4)); }

// ---- k_la_seg: per (stream, segment p < P - 1) the sums Fk^T V and phi(k) ----------------
template <int D, typename TIn>
__global__ void __launch_bounds__(LaCfg<D>::NT)
k_la_seg(const TIn *__restrict__ k, const TIn *__restrict__ v, float *__restrict__ ws, int64_t T,
         int P, int cps) {
  using C = LaCfg<D>;
  __shared__ LaSegShared<D> sh;
  const int64_t s = blockIdx.x;
  const int p = blockIdx.y;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave, li = lane & 15, gq = lane >> 4;
  const int64_t NC = (T + LC - 1) / LC;
  const int64_t c0 = int64_t(p) * cps, c1 = c0 + cps < NC ? c0 + cps : NC;
  const int64_t row0 = s * T;
  f4_t ST[C::NW];
#pragma unroll
  for (int jb = 0; jb < C::NW; ++jb) ST[jb] = f4_zero();
  constexpr bool VX = sizeof(TIn) == 2;
  float ncol[4] = {0.f, 0.f, 0.f, 0.f};  // phi(k) sums of this thread's rows and columns
  ChunkLoader<D, TIn, 2> ld;
  const TIn *const src[2] = {k, v};
  ld.fetch(src, row0, c0 * LC, T, tid);
  for (int64_t c = c0; c < c1; ++c) {
#pragma unroll
    for (int m = 0; m < C::GPT; ++m) {
      const int g = tid + C::NT * m, t = 4 * g / D, j = 4 * g % D;
      const bool ok = c * LC + t < T;
      float xk[4], xv[4];
      ld.r[0][m].get(xk);
      ld.r[1][m].get(xv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xk[e] = ok ? phi(xk[e]) : 0.f;
        ncol[e] += xk[e];
      }
      put2(&sh.fk[0][t][j], C::TS, xk);
      if constexpr (VX)
        put1(&sh.vv[0][t][j], xv);
      else
        put2(&sh.vv[0][t][j], C::TS, xv);
    }
    if (c + 1 < c1) ld.fetch(src, row0, (c + 1) * LC, T, tid);
    __syncthreads();
    Split2h vt[4];
    load_vt<D, VX>(vt, sh, w, gq, li);
    state_update<D, VX>(ST, sh, vt, gq, li);
    __syncthreads();
  }
  *reinterpret_cast<float4 *>(&sh.part[stage_rg<D>(tid)][stage_col<D>(tid)]) =
      make_float4(ncol[0], ncol[1], ncol[2], ncol[3]);
  __syncthreads();
  float *rec = ws + (s * P + p) * C::SEG;
#pragma unroll
  for (int jb = 0; jb < C::NW; ++jb)
#pragma unroll
    for (int r = 0; r < 4; ++r) rec[(16 * jb + 4 * gq + r) * D + 16 * w + li] = ST[jb][r];
  if (tid < D) {
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) a += sh.part[g][tid];
    rec[D * D + tid] = a;
  }
}

// ---- k_la_prefix: exclusive prefix over segments, in place --------------------------------
template <int D>
__global__ void __launch_bounds__(256) k_la_prefix(float *__restrict__ ws, int P) {
  using C = LaCfg<D>;
  const int64_t s = blockIdx.x;
  const int64_t e = int64_t(blockIdx.y) * 256 + threadIdx.x;
  if (e >= C::SEG) return;
  float *base = ws + s * P * C::SEG + e;
  float run = 0.f;
  for (int p = 0; p < P; ++p) {
    const float x = p + 1 < P ? base[p * C::SEG] : 0.f;  // the last segment's sum is not needed
    base[p * C::SEG] = run;
    run += x;
  }
}

// ---- k_la_out: the chunk recurrence of one segment ----------------------------------------
template <int D, typename TIn>
__global__ void __launch_bounds__(LaCfg<D>::NT)
k_la_out(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
         TIn *__restrict__ out, const float *__restrict__ ws, float *__restrict__ S_final,
         float *__restrict__ n_final, int64_t T, int P, int cps, float eps) {
  using C = LaCfg<D>;
  __shared__ LaShared<D> sh;
  const int64_t s = blockIdx.x;
  const int p = blockIdx.y;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave, li = lane & 15, gq = lane >> 4;
  const int64_t NC = (T + LC - 1) / LC;
  const int64_t c0 = int64_t(p) * cps, c1 = c0 + cps < NC ? c0 + cps : NC;
  const int64_t row0 = s * T;
  const float *rec = ws + (s * P + p) * C::SEG;
  f4_t ST[C::NW];
#pragma unroll
  for (int jb = 0; jb < C::NW; ++jb)
#pragma unroll
    for (int r = 0; r < 4; ++r) ST[jb][r] = rec[(16 * jb + 4 * gq + r) * D + 16 * w + li];
  constexpr bool VX = sizeof(TIn) == 2;
  for (int j = tid; j < D; j += C::NT) sh.n[0][j] = rec[D * D + j];
  ChunkLoader<D, TIn, 3> ld;
  const TIn *const src[3] = {q, k, v};
  ld.fetch(src, row0, c0 * LC, T, tid);
  for (int64_t c = c0; c < c1; ++c) {
    // (1) the chunk's operands into LDS as two-term bf16, and this thread's phi(k) column sums
    const int cur = static_cast<int>((c - c0) & 1);
    float csum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < C::GPT; ++m) {
      const int g = tid + C::NT * m, t = 4 * g / D, j = 4 * g % D;
      const bool ok = c * LC + t < T;
      float xq[4], xk[4], xv[4];
      ld.r[0][m].get(xq);
      ld.r[1][m].get(xk);
      ld.r[2][m].get(xv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xq[e] = ok ? phi(xq[e]) : 0.f;
        xk[e] = ok ? phi(xk[e]) : 0.f;
        csum[e] += xk[e];
      }
      put2(&sh.fq[0][t][j], C::TS, xq);
      put2(&sh.fk[0][t][j], C::TS, xk);
      if constexpr (VX)
        put1(&sh.vv[0][t][j], xv);
      else
        put2(&sh.vv[0][t][j], C::TS, xv);
    }
    *reinterpret_cast<float4 *>(&sh.part[stage_rg<D>(tid)][stage_col<D>(tid)]) =
        make_float4(csum[0], csum[1], csum[2], csum[3]);
    if (c + 1 < c1) ld.fetch(src, row0, (c + 1) * LC, T, tid);
    __syncthreads();
    // (2) P = tril0(Fq Fk^T) by tiles, computed transposed so that a lane holds four keys of
    // one query row: P^T tile = Fk_sb Fq_tb^T, lane (gq, li) gets P[16 tb + li][16 sb + 4 gq + r]
    {
      constexpr int MT = (10 + C::NW - 1) / C::NW;  // tiles per wave, at most
      const int nt = (10 - w + C::NW - 1) / C::NW;  // this wave's tiles w, w + NW, ...
      int tb[MT], sb[MT];
      f4_t acc[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        tile_of(i < nt ? w + C::NW * i : 0, tb[i], sb[i]);
        acc[i] = f4_zero();
      }
#pragma unroll
      for (int kb = 0; kb < C::NW; kb += 2)
#pragma unroll
        for (int i = 0; i < MT; ++i)
          if (i < nt) {
            const uint16_t *fk = &sh.fk[0][16 * sb[i] + li][16 * kb + 4 * gq];
            const uint16_t *fq = &sh.fq[0][16 * tb[i] + li][16 * kb + 4 * gq];
            acc[i] = mm2w_ss(cat2(ld2_4h(fk, C::TS), ld2_4h(fk + 16, C::TS)),
                             cat2(ld2_4h(fq, C::TS), ld2_4h(fq + 16, C::TS)), acc[i]);
          }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (i >= nt) break;
        if (sb[i] == tb[i]) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * gq + r > li) acc[i][r] = 0.f;  // key after query
        }
        float part = acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (gq == 0) sh.rs[sb[i]][16 * tb[i] + li] = part;
        const Split2h sp = split2_4h(acc[i]);
        *reinterpret_cast<uint2 *>(&sh.pp[0][16 * tb[i] + li][16 * sb[i] + 4 * gq]) = sp.h;
        *reinterpret_cast<uint2 *>(&sh.pp[1][16 * tb[i] + li][16 * sb[i] + 4 * gq]) = sp.l;
      }
    }
    if (w == C::NW - 1) {
      // phi(q_t) . n at the chunk start, lane t
      float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < D; j += 4) {
        const uint2 h = *reinterpret_cast<const uint2 *>(&sh.fq[0][lane][j]);
        const uint2 l = *reinterpret_cast<const uint2 *>(&sh.fq[1][lane][j]);
        const float4 nn = *reinterpret_cast<const float4 *>(&sh.n[cur][j]);
        a[0] = fmaf(pk_lo_val(h.x) + pk_lo_val(l.x), nn.x, a[0]);
        a[1] = fmaf(pk_hi_val(h.x) + pk_hi_val(l.x), nn.y, a[1]);
        a[2] = fmaf(pk_lo_val(h.y) + pk_lo_val(l.y), nn.z, a[2]);
        a[3] = fmaf(pk_hi_val(h.y) + pk_hi_val(l.y), nn.w, a[3]);
      }
      sh.nq[lane] = (a[0] + a[1]) + (a[2] + a[3]);
    } else if (w == C::NW - 2) {
      // n at the next chunk start: n + the 16 row groups' column sums, in a fixed order
      for (int j = lane; j < D; j += kWave) {
        float b = sh.n[cur][j];
#pragma unroll
        for (int g = 0; g < 16; ++g) b += sh.part[g][j];
        sh.n[cur ^ 1][j] = b;
      }
    }
    __syncthreads();
    // (3) O[:, 16 w ..] = Fq S^T + P V, divided by the denominators
    Split2h vt[4];
    load_vt<D, VX>(vt, sh, w, gq, li);
    f4_t acc[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[tb] = f4_zero();
#pragma unroll
    for (int jb = 0; jb < C::NW; jb += 2) {  // key blocks jb, jb + 1
      const Split2w b = cat2(split2_4h(ST[jb]), split2_4h(ST[jb + 1]));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const uint16_t *fq = &sh.fq[0][16 * tb + li][16 * jb + 4 * gq];
        acc[tb] = mm2w_ss(cat2(ld2_4h(fq, C::TS), ld2_4h(fq + 16, C::TS)), b, acc[tb]);
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {  // token blocks 2 m, 2 m + 1 (P is zero above the diagonal)
      const Split2w b = cat2(vt[2 * m], vt[2 * m + 1]);
#pragma unroll
      for (int tb = 2 * m; tb < 4; ++tb) {
        const uint16_t *pr = &sh.pp[0][16 * tb + li][32 * m + 4 * gq];
        const Split2h lo = ld2_4h(pr, C::TSP);
        const Split2h hi = tb > 2 * m ? ld2_4h(pr + 16, C::TSP) : zero2h();
        acc[tb] = mm_v<VX>(cat2(lo, hi), b, acc[tb]);
      }
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tb + 4 * gq + r;
        const int64_t tok = c * LC + t;
        float den = sh.nq[t] + eps;
        for (int sb = 0; sb <= tb; ++sb) den += sh.rs[sb][t];
        if (tok < T) la_store<TIn>(out + (row0 + tok) * D + 16 * w + li, acc[tb][r] / den);
      }
    }
    // (4) S^T += Fk^T V
    state_update<D, VX>(ST, sh, vt, gq, li);
    __syncthreads();  // the next chunk rewrites every LDS operand
  }
  __syncthreads();  // sh.n complete even for a segment without chunks
  const int fin = static_cast<int>((c1 - c0) & 1);
  if (p == P - 1) {
    // S[i][j] = S^T[j][i]: lane (gq, li) holds S[16 w + li][16 jb + 4 gq + r], r < 4
    if (S_final != nullptr) {
#pragma unroll
      for (int jb = 0; jb < C::NW; ++jb)
        *reinterpret_cast<float4 *>(S_final + s * D * D + (16 * w + li) * D + 16 * jb + 4 * gq) =
            make_float4(ST[jb][0], ST[jb][1], ST[jb][2], ST[jb][3]);
    }
    if (n_final != nullptr)
      for (int j = tid; j < D; j += C::NT) n_final[s * D + j] = sh.n[fin][j];
  }
}

struct LaPlan {
  int P, cps;
};

// Segments: enough (stream, segment) workgroups for two per CU, whole chunks each.
LaPlan la_plan(const Problem &p) {
  const int64_t NC = (p.T + LC - 1) / LC;
  int64_t P = (512 + p.streams - 1) / p.streams;
  if (P > NC) P = NC;
  if (P < 1) P = 1;
  const int64_t cps = (NC + P - 1) / P;
  P = (NC + cps - 1) / cps;
  return LaPlan{static_cast<int>(P), static_cast<int>(cps)};
}

template <int D, typename TIn>
hipError_t launch_la_t(const Problem &p, const void *q, const void *k, const void *v, void *out,
                       float *S_final, float *n_final, void *ws, hipStream_t st) {
  using C = LaCfg<D>;
  const LaPlan pl = la_plan(p);
  const unsigned S = static_cast<unsigned>(p.streams);
  float *w = static_cast<float *>(ws);
  if (pl.P > 1)
    VLA_LAUNCH("k_la_seg", (k_la_seg<D, TIn>), dim3(S, pl.P - 1), dim3(C::NT), 0, st,
               static_cast<const TIn *>(k), static_cast<const TIn *>(v), w, p.T, pl.P, pl.cps);
  VLA_LAUNCH("k_la_prefix", (k_la_prefix<D>), dim3(S, (C::SEG + 255) / 256), dim3(256), 0, st, w,
             pl.P);
  VLA_LAUNCH("k_la_out", (k_la_out<D, TIn>), dim3(S, pl.P), dim3(C::NT), 0, st,
             static_cast<const TIn *>(q), static_cast<const TIn *>(k), static_cast<const TIn *>(v),
             static_cast<TIn *>(out), w, S_final, n_final, p.T, pl.P, pl.cps, p.eps);
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_la_dt(const Problem &p, const void *q, const void *k, const void *v, void *out,
                        float *S_final, float *n_final, void *ws, hipStream_t st) {
  switch (p.d) {
    case 32: return launch_la_t<32, TIn>(p, q, k, v, out, S_final, n_final, ws, st);
    case 64: return launch_la_t<64, TIn>(p, q, k, v, out, S_final, n_final, ws, st);
    case 96: return launch_la_t<96, TIn>(p, q, k, v, out, S_final, n_final, ws, st);
    case 128: return launch_la_t<128, TIn>(p, q, k, v, out, S_final, n_final, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t la_workspace_bytes(const Problem &p) {
  const LaPlan pl = la_plan(p);
  return static_cast<size_t>(p.streams) * pl.P * (static_cast<size_t>(p.d) * p.d + p.d) * sizeof(float);
}

hipError_t launch_la(const Problem &p, const void *q, const void *k, const void *v, void *out,
                     float *S_final, float *n_final, void *ws, hipStream_t stream) {
  if (p.dtype == Dtype::F32) return launch_la_dt<float>(p, q, k, v, out, S_final, n_final, ws, stream);
  return launch_la_dt<bf16_t>(p, q, k, v, out, S_final, n_final, ws, stream);
}

}  // namespace vla
