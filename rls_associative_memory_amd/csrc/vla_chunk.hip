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
// Passes (launched in order on one stream; every pass is parallel over (stream, segment);
// large calls run their streams as two groups, each in this order on its own HIP stream):
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
#include <mutex>
#include <type_traits>
#include <vector>

#include "vla_common.h"
#include "vla_internal.h"
#include "vla_mfma.h"
#include "vla_aside_wy.h"
#include "vla_swy_bf16.h"

namespace vla {

// ------------------------------------------------------------------------------------
// Plan and workspace layout
// ------------------------------------------------------------------------------------
struct ChunkPlan {
  int D = 0, C = 0;
  int64_t S = 0, T = 0, L = 0, P = 0;
  size_t off_m = 0, off_nk = 0, off_alpha = 0, off_rkden = 0, off_pib = 0, off_s0 = 0, off_minv = 0;
  size_t off_tiles = 0;  // valid when tiles: the S passes' shared tiles
  bool tiles = false;
  size_t total = 0;
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// records: the plan of the backward's chunked forward, whose S passes do not share tiles (its
// final pass writes the token records and is bound by those stores: loading the tiles,
// 403 MB at 32 x 131072 tokens, took it from 2.65 to 2.76 ms, forming them costs less).
static ChunkPlan make_plan(const Problem &p, int C, bool records = false) {
  ChunkPlan pl;
  pl.D = p.d;
  pl.C = C;
  pl.S = p.streams;
  pl.T = p.T;
  // Segment length: a power of two (a multiple of C) sized so that all streams together give
  // about 2048 segments, capped so that P stays small enough to scan.  At least 256 tokens for
  // bf16 inputs, whose A side runs two six-wave workgroups per CU (more, shorter segments only
  // add rounds and segment passes); at least 64 for fp32 inputs, whose A side is one wave per
  // segment with every segment resident at once, so shorter segments shorten the chain
  // (on 256 streams of 512 tokens at d = 32, 64-token segments take about 40 % less time than
  // 256-token ones).
  const int64_t target = (p.streams * p.T + 2047) / 2048;
  int64_t L = (p.dtype == Dtype::F32) ? 64 : 256;
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
  pl.off_minv = off;  off = align256(off + S * D * D * 4);  // A0^{-1} of a carried state
  pl.tiles = !records && swb_shares_tiles(p.dtype == Dtype::F32, pl.P, C);
  if (pl.tiles) {  // the S passes' shared tiles, last (a plan without them is a prefix)
    pl.off_tiles = off;
    off = align256(off + S * static_cast<size_t>(swb_tile_blocks(pl.T)) * kSwbTileBlock * 2);
  }
  pl.total = off;
  return pl;
}

int chunk_default(const Problem &p) { return p.d > 96 ? 32 : 64; }

bool chunk_supported(const Problem &p, int chunk) {
  if (chunk != 16 && chunk != 32 && chunk != 64) return false;
  if (p.d > 96 && chunk > 32) return false;  // LDS budget of the WY kernel
  return p.d == 32 || p.d == 64 || p.d == 96 || p.d == 128;
}

size_t chunk_workspace_bytes(const Problem &p, int chunk, bool records) {
  return make_plan(p, chunk, records).total;
}

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
// k_gram: Gram_p = sum_{t in segment p} u_t u_t^T (segments 0..P-2) and, for fp32 inputs,
// nk_p = sum phi(k_t) (for bf16 inputs the A side forms these sums from the keys it stages)
// bf16 inputs: v_mfma_f32_16x16x32_bf16 on the raw inputs (every product exact in fp32),
// tokens staged 64 at a time as they are (token rows, 16-byte copies) and read by feature
// with the transposing load ds_read_b64_tr_b16; fp32 inputs: v_mfma_f32_16x16x4_f32, tokens
// transposed and packed at staging so each lane's operand is one 16-byte LDS read.  The next
// block's 16-byte global loads are issued before the current block is multiplied.
// ------------------------------------------------------------------------------------

template <int D, typename TIn>
__global__ void __launch_bounds__(256)
k_gram(const TIn *__restrict__ u, const TIn *__restrict__ k, float *__restrict__ M,
       float *__restrict__ nk, int64_t T, int64_t L, int64_t P) {
  constexpr int NT16 = D / 16;
  constexpr int NTILE = NT16 * (NT16 + 1) / 2;
  constexpr int TPW = (NTILE + 3) / 4;
  constexpr int TB = 64;
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr bool NEEDK = !BF;          // phi(k) sums here only for fp32 inputs
  using IO = io<TIn>;
  using vec_t = typename IO::vec_t;
  constexpr int VW = IO::kVec;
  constexpr int UB = TB * D / VW;      // vectors per array per block
  constexpr int PU = UB / 256;         // per thread (exact for every supported D)
  static_assert(UB % 256 == 0, "block staging must tile the threads");
  constexpr int LDR = D + 8;           // bf16 token rows (52-word rows at d = 96)
  __shared__ __attribute__((aligned(16))) uint16_t sUb[BF ? TB : 1][BF ? LDR : 1];
  __shared__ __attribute__((aligned(16))) float sUf[BF ? 1 : TB / 4][BF ? 1 : D + 1][4];

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
  // Unit ui = tid + 256 i covers token ui % 64 and features (ui / 64) * VW .. + VW.
  float nka[PU][VW];
#pragma unroll
  for (int i = 0; i < PU; ++i)
#pragma unroll
    for (int e = 0; e < VW; ++e) nka[i][e] = 0.f;
  vec_t pu[PU], pk[PU];
  auto prefetch = [&](int64_t t0) {
    const int nt = static_cast<int>(std::min<int64_t>(TB, te - t0));
#pragma unroll
    for (int i = 0; i < PU; ++i) {
      const int ui = tid + 256 * i;
      const int c = ui % TB, f0 = (ui / TB) * VW;
      const bool ok = c < nt;
      pu[i] = ok ? *reinterpret_cast<const vec_t *>(us + (t0 + c) * D + f0) : vec_t{};
      if constexpr (NEEDK) pk[i] = ok ? *reinterpret_cast<const vec_t *>(ks + (t0 + c) * D + f0) : vec_t{};
    }
  };
  prefetch(tb);
  for (int64_t t0 = tb; t0 < te; t0 += TB) {
    const int nt = static_cast<int>(std::min<int64_t>(TB, te - t0));
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PU; ++i) {
      const int ui = tid + 256 * i;
      const int c = ui % TB, f0 = (ui / TB) * VW;
      if constexpr (BF) {
        *reinterpret_cast<uint4 *>(&sUb[c][f0]) = pu[i];
      } else {
        float x[VW];
        IO::unpack(pu[i], x);
#pragma unroll
        for (int e = 0; e < VW; ++e) sUf[c / 4][f0 + e][c % 4] = x[e];
      }
      if constexpr (NEEDK) {
        float kx[VW];
        IO::unpack(pk[i], kx);
        if (c < nt)
#pragma unroll
          for (int e = 0; e < VW; ++e) nka[i][e] += phi(kx[e]);
      }
    }
    __syncthreads();
    if (t0 + TB < te) prefetch(t0 + TB);
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      if (wave + 4 * m < NTILE) {
        const int fi = 16 * ti_i[m] + li, fj = 16 * ti_j[m] + li;
        if constexpr (BF) {
          // lane (li, gq): U[32 kk + 8 gq + e][16 ti + li], e = 0..7, for both operands
#pragma unroll
          for (int kk = 0; kk < TB / 32; ++kk) {
            const int r0 = 32 * kk + 8 * gq;
            const bf16x8_t a = ld_tr4x2(&sUb[0][0], LDR, r0, r0 + 4, 16 * ti_i[m], li);
            const bf16x8_t b = ld_tr4x2(&sUb[0][0], LDR, r0, r0 + 4, 16 * ti_j[m], li);
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[m], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int kt = 0; kt < TB / 16; ++kt) {
            const float4 a = *reinterpret_cast<const float4 *>(&sUf[4 * kt + gq][fi][0]);
            const float4 b = *reinterpret_cast<const float4 *>(&sUf[4 * kt + gq][fj][0]);
            acc[m] = mfma_f32_16x16x4(a.x, b.x, acc[m]);
            acc[m] = mfma_f32_16x16x4(a.y, b.y, acc[m]);
            acc[m] = mfma_f32_16x16x4(a.z, b.z, acc[m]);
            acc[m] = mfma_f32_16x16x4(a.w, b.w, acc[m]);
          }
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
  // phi(k) sums: lanes of a wave share the feature block and differ in the token.
  if constexpr (NEEDK)
#pragma unroll
  for (int i = 0; i < PU; ++i) {
    const int f0 = ((tid + 256 * i) / TB) * VW;
#pragma unroll
    for (int e = 0; e < VW; ++e) {
      const float tot = wave_sum(nka[i][e]);
      if (lane == 0) nk[(s * P + p) * D + f0 + e] = tot;
    }
  }
}

// ------------------------------------------------------------------------------------
// k_prefix: M_p <- M_0 + sum_{p' < p} Gram_p' (fp64 sums), nk_p <- n_0 + sum_{p'<p} nk_p',
// with M_0 = lambda0 I and n_0 = 0, or a carried state's A_0^{-1} (Minit) and n_0.
// ------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
k_prefix(float *__restrict__ M, float *__restrict__ nk, int64_t P, float lambda0,
         const float *__restrict__ Minit, const float *__restrict__ n0, int with_n,
         double *__restrict__ Md) {
  const int64_t s = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  if (e < D * D) {
    const double init = Minit != nullptr ? static_cast<double>(Minit[s * D * D + e])
                        : (e / D) == (e % D) ? static_cast<double>(lambda0) : 0.0;
    float *base = M + s * P * D * D + e;
    double acc = 0.0;
    // 16 segments' Grams are loaded before any of them is replaced by its prefix, so the
    // scan waits for one memory latency per 16 segments rather than one per segment.  With
    // Md the prefixes go there in fp64 instead (M keeps the Grams).
    for (int64_t p0 = 0; p0 < P; p0 += 16) {
      float g[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) g[i] = (p0 + i + 1 < P) ? base[(p0 + i) * D * D] : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (p0 + i < P) {
          if (Md != nullptr)
            Md[(s * P + p0 + i) * D * D + e] = acc + init;
          else
            base[(p0 + i) * D * D] = static_cast<float>(acc + init);
        }
        acc += g[i];
      }
    }
  }
  if (with_n && blockIdx.y == 0 && threadIdx.x < D) {
    const double init = n0 != nullptr ? static_cast<double>(n0[s * D + threadIdx.x]) : 0.0;
    float *base = nk + s * P * D + threadIdx.x;
    double acc = 0.0;
    for (int64_t p0 = 0; p0 < P; p0 += 16) {
      float g[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) g[i] = (p0 + i + 1 < P) ? base[(p0 + i) * D] : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (p0 + i < P) base[(p0 + i) * D] = static_cast<float>(acc + init);
        acc += g[i];
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// k_inv64: M_p <- (Md_p)^{-1} in fp64 (Gauss-Jordan without pivoting, Md_p SPD), rounded once
// to fp32.  For callers that need the segment-start inverse penalty to fp32 accuracy whatever
// the conditioning of lambda0 I + Gram (the fp32 inversion loses about cond * 2^-24).
// Thread (ri, cj) = (tid / 16, tid % 16) holds rows ri + 16 a and columns cj + 16 b; pivot row
// and column are broadcast through LDS, double buffered (one barrier per pivot).
// ------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) k_inv64(const double *__restrict__ Md, float *__restrict__ M,
                                               int64_t P) {
  constexpr int NR = D / 16;
  __shared__ double rowk[2][D], colk[2][D];
  const int64_t s = blockIdx.x, p = blockIdx.y;
  const int tid = threadIdx.x, ri = tid >> 4, cj = tid & 15;
  const double *src = Md + (s * P + p) * D * D;
  double a[NR][NR];
#pragma unroll
  for (int x = 0; x < NR; ++x)
#pragma unroll
    for (int y = 0; y < NR; ++y) a[x][y] = src[(ri + 16 * x) * D + cj + 16 * y];
  for (int k = 0; k < D; ++k) {
    const int b = k & 1, kx = k >> 4, kr = k & 15;
    // Register indices stay compile-time constants: the pivot's block of rows (columns) is
    // picked by a chain of selects, not by indexing, which would put the matrix in scratch
    // memory; the threads of the pivot row (column) then write their values in one guarded
    // region instead of one per element.
    if (ri == kr) {
#pragma unroll
      for (int y = 0; y < NR; ++y) {
        double v = a[0][y];
#pragma unroll
        for (int x = 1; x < NR; ++x) v = (x == kx) ? a[x][y] : v;
        rowk[b][cj + 16 * y] = v;
      }
    }
    if (cj == kr) {
#pragma unroll
      for (int x = 0; x < NR; ++x) {
        double v = a[x][0];
#pragma unroll
        for (int y = 1; y < NR; ++y) v = (y == kx) ? a[x][y] : v;
        colk[b][ri + 16 * x] = v;
      }
    }
    __syncthreads();
    // In-place Gauss-Jordan step with r = the pivot row scaled by 1/pivot, its pivot entry
    // 1/pivot, and c_i = A[i][k] (-1 for the pivot row):  A[i][j] <- keep * A[i][j] - c_i r_j,
    // keep = 0 on the pivot row and the pivot column.  So the pivot row becomes r, the pivot
    // column -A[i][k]/pivot, and every other entry A[i][j] - A[i][k] A[k][j]/pivot: one fma and
    // one select per entry.
    const double ip = 1.0 / rowk[b][k];
    double ry[NR], cx[NR];
#pragma unroll
    for (int y = 0; y < NR; ++y) {
      const int j = cj + 16 * y;
      ry[y] = (j == k) ? ip : rowk[b][j] * ip;
    }
#pragma unroll
    for (int x = 0; x < NR; ++x) {
      const int i = ri + 16 * x;
      cx[x] = (i == k) ? -1.0 : colk[b][i];
    }
#pragma unroll
    for (int x = 0; x < NR; ++x) {
      const bool prow = ri + 16 * x == k;
#pragma unroll
      for (int y = 0; y < NR; ++y) {
        const bool keep = !prow && cj + 16 * y != k;
        a[x][y] = fma(-cx[x], ry[y], keep ? a[x][y] : 0.0);
      }
    }
  }
  float *dst = M + (s * P + p) * D * D;
#pragma unroll
  for (int x = 0; x < NR; ++x)
#pragma unroll
    for (int y = 0; y < NR; ++y) dst[(ri + 16 * x) * D + cj + 16 * y] = static_cast<float>(a[x][y]);
}

// ------------------------------------------------------------------------------------
// k_sym_copy: dst_s = (A_s + A_s^T) / 2 for every stream s (src [streams][D][D], dst matrices
// dst_stride floats apart): a carried A_0, symmetrised, where the path starts from it.
// ------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
k_sym_copy(const float *__restrict__ src, float *__restrict__ dst, int64_t dst_stride) {
  const int64_t s = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  if (e < D * D) {
    const int i = e / D, j = e % D;
    const float *a = src + s * D * D;
    dst[s * dst_stride + e] = 0.5f * (a[i * D + j] + a[j * D + i]);
  }
}

// ------------------------------------------------------------------------------------
// k_inv: M_p <- M_p^{-1} (block Gauss-Jordan without pivoting on 16 x 16 blocks; M_p is
// SPD), symmetrised.  The nb x nb blocks live in MFMA accumulators spread over 4 waves.
// Elimination step kb: invert the diagonal block P (one wave, scalar Gauss-Jordan), then
//   row panel    A[kb][j] <- P^{-1} A[kb][j]
//   trailing     A[i][j]  <- A[i][j] - A[i][kb] (P^{-1} A[kb][j])
//   column panel A[i][kb] <- -A[i][kb] P^{-1},   A[kb][kb] <- P^{-1}
// with every block product on v_mfma_f32_16x16x4_f32 (operands packed k-minor in LDS).
// ------------------------------------------------------------------------------------
template <int D>
// The symmetrisation buffer lies over the elimination buffers (it is used after the last block
// step only), and at d = 96 the kernel is held to 128 VGPRs: four workgroups per CU, not two.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 96 ? 4 : 1)))
k_inv(float *__restrict__ M, int64_t P) {
  constexpr int NB = D / 16;
  constexpr int NOWN = (NB * NB + 3) / 4;  // blocks per wave
  union Lds {
    struct {
      float Pd[16][17];         // diagonal block, scalar GJ
      float PiA[4][16][4];      // P^-1 as A operand [k/4][i][k%4]
      float PiB[4][16][4];      // P^-1 as B operand [k/4][j][k%4]
      float CP[NB][4][16][4];   // column panel (A operands)
      float RP[NB][4][16][4];   // row panel (B operands)
    } e;
    float sym[D][D + 1];        // the result, symmetrised at the end
  };
  __shared__ __attribute__((aligned(16))) Lds lds;
  auto &Pd = lds.e.Pd;
  auto &PiA = lds.e.PiA;
  auto &PiB = lds.e.PiB;
  auto &CP = lds.e.CP;
  auto &RP = lds.e.RP;
  auto &sym = lds.sym;
  const int64_t s = blockIdx.x, p = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, gq = lane >> 4;
  float *base = M + (s * P + p) * D * D;

  // Block n = wave + 4 m is (n / NB, n % NB); acc element r = A[16 bi + 4 gq + r][16 bj + li].
  f4_t acc[NOWN];
#pragma unroll
  for (int m = 0; m < NOWN; ++m) {
    const int n = wave + 4 * m;
    if (n < NB * NB) {
      const int bi = n / NB, bj = n % NB;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[m][r] = base[(16 * bi + 4 * gq + r) * D + 16 * bj + li];
    }
  }
  for (int kb = 0; kb < NB; ++kb) {
    __syncthreads();
    // (1) publish the diagonal block and the column panel
#pragma unroll
    for (int m = 0; m < NOWN; ++m) {
      const int n = wave + 4 * m;
      if (n < NB * NB && n % NB == kb) {
        const int bi = n / NB;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (bi == kb) Pd[4 * gq + r][li] = acc[m][r];
          CP[bi][li / 4][4 * gq + r][li % 4] = acc[m][r];  // C[i'][k]: i' = 4gq + r, k = li
        }
      }
    }
    __syncthreads();
    // (2) P^{-1} by scalar Gauss-Jordan in one wave: lane owns row lane/4, columns 4(lane%4)..
    if (wave == 0) {
      const int i = lane >> 2, j0 = 4 * (lane & 3);
      float e[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) e[c] = Pd[i][j0 + c];
      for (int kk = 0; kk < 16; ++kk) {
        const float piv = 1.0f / Pd[kk][kk];
        const float cik = Pd[i][kk];
        float rkj[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) rkj[c] = Pd[kk][j0 + c];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = j0 + c;
          if (i == kk)
            e[c] = (j == kk) ? piv : e[c] * piv;
          else if (j == kk)
            e[c] = -cik * piv;
          else
            e[c] = fmaf(-cik * piv, rkj[c], e[c]);
          Pd[i][j] = e[c];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = j0 + c;
        PiA[j / 4][i][j % 4] = e[c];  // A operand: element (row i, k = j)
        PiB[i / 4][j][i % 4] = e[c];  // B operand: element (k = i, col j)
      }
    }
    __syncthreads();
    // (3) row panel: A[kb][j] <- P^{-1} A[kb][j]; publish as B operands.
#pragma unroll
    for (int m = 0; m < NOWN; ++m) {
      const int n = wave + 4 * m;
      if (n < NB * NB && n / NB == kb && n % NB != kb) {
        const int bj = n % NB;
        const float4 a4 = *reinterpret_cast<const float4 *>(&PiA[gq][li][0]);
        f4_t r4 = f4_zero();
        r4 = mfma_f32_16x16x4(a4.x, acc[m][0], r4);
        r4 = mfma_f32_16x16x4(a4.y, acc[m][1], r4);
        r4 = mfma_f32_16x16x4(a4.z, acc[m][2], r4);
        r4 = mfma_f32_16x16x4(a4.w, acc[m][3], r4);
        acc[m] = r4;
        *reinterpret_cast<float4 *>(&RP[bj][gq][li][0]) = make_float4(r4[0], r4[1], r4[2], r4[3]);
      }
    }
    __syncthreads();
    // (4) trailing blocks and the column panel.
#pragma unroll
    for (int m = 0; m < NOWN; ++m) {
      const int n = wave + 4 * m;
      if (n < NB * NB) {
        const int bi = n / NB, bj = n % NB;
        if (bi == kb) {
          if (bj == kb) {
            const float4 pv = *reinterpret_cast<const float4 *>(&PiB[gq][li][0]);
            acc[m] = f4_t{pv.x, pv.y, pv.z, pv.w};
          }
        } else {
          const float4 c4 = *reinterpret_cast<const float4 *>(&CP[bi][gq][li][0]);
          if (bj == kb) {
            const float4 b4 = *reinterpret_cast<const float4 *>(&PiB[gq][li][0]);
            f4_t r4 = f4_zero();
            r4 = mfma_f32_16x16x4(-c4.x, b4.x, r4);
            r4 = mfma_f32_16x16x4(-c4.y, b4.y, r4);
            r4 = mfma_f32_16x16x4(-c4.z, b4.z, r4);
            r4 = mfma_f32_16x16x4(-c4.w, b4.w, r4);
            acc[m] = r4;
          } else {
            const float4 b4 = *reinterpret_cast<const float4 *>(&RP[bj][gq][li][0]);
            acc[m] = mfma_f32_16x16x4(-c4.x, b4.x, acc[m]);
            acc[m] = mfma_f32_16x16x4(-c4.y, b4.y, acc[m]);
            acc[m] = mfma_f32_16x16x4(-c4.z, b4.z, acc[m]);
            acc[m] = mfma_f32_16x16x4(-c4.w, b4.w, acc[m]);
          }
        }
      }
    }
  }
  // Symmetrise: A <- (A + A^T) / 2.
  __syncthreads();
#pragma unroll
  for (int m = 0; m < NOWN; ++m) {
    const int n = wave + 4 * m;
    if (n < NB * NB) {
      const int bi = n / NB, bj = n % NB;
#pragma unroll
      for (int r = 0; r < 4; ++r) sym[16 * bi + 4 * gq + r][16 * bj + li] = acc[m][r];
    }
  }
  __syncthreads();
  for (int e = tid; e < D * D; e += 256) {
    const int i = e / D, j = e % D;
    base[e] = 0.5f * (sym[i][j] + sym[j][i]);
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
  static constexpr int RING = 4;                // tokens in flight in registers
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

// With REC the kernel also writes the backward's token records it holds (z, ahat, delta,
// ||A khat||, 1/||k||, den) and the A half of the state checkpoints.
template <int D, typename TIn, bool REC = false>
__global__ void __launch_bounds__(AsideCfg<D>::NT)
k_aside(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ u,
        const float *__restrict__ A0, const float *__restrict__ nk0, float *__restrict__ alpha,
        float *__restrict__ rkden, float *__restrict__ A_final, float *__restrict__ n_final,
        int64_t S, int64_t T, int64_t L, int64_t P, float eps, float *__restrict__ brec,
        float *__restrict__ bck, float *__restrict__ bnend) {
  using C = AsideCfg<D>;
  using IO = io<TIn>;
  using vec_t = typename IO::vec_t;
  constexpr int VW = IO::kVec;
  constexpr int VPA = D / VW;                    // vectors per array per token
  constexpr int NV = 3 * VPA;                    // u, k, q vectors per token
  constexpr int PV = (NV + C::LA - 1) / C::LA;   // vectors per lane per token
  __shared__ __attribute__((aligned(16))) float sU[C::UPB][2][D];
  __shared__ __attribute__((aligned(16))) float sK[C::UPB][2][D];
  __shared__ __attribute__((aligned(16))) float sQ[C::UPB][2][D];  // phi(q)
  __shared__ __attribute__((aligned(16))) float sW[C::UPB][D];
  __shared__ float sRed[2][C::NWA][3];

  const int tid = threadIdx.x;
  const int unit_in_blk = tid / C::LA;
  const int lu = tid % C::LA;  // lane within the unit
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * C::UPB + unit_in_blk;
  if (unit >= S * P) return;  // whole unit (a single wave when UPB > 1) leaves together
  const int64_t s = unit / P, p = unit % P;
  const int h = lu & 1, g = lu >> 1, c0 = h * C::CW;
  const int wside = lu / kWave;
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const TIn *base_in[3] = {u + s * T * D, k + s * T * D, q + s * T * D};
  float *al = alpha + s * T * D;
  float *rd = rkden + s * T * 2;
  float *W = sW[unit_in_blk];
  constexpr int RF = BwRec<D>::F;
  float *brs = REC ? brec + s * T * RF : nullptr;
  float *bcs = REC ? bck + s * ((T + kBwCk - 1) / kBwCk) * 2 * D * D + D * D : nullptr;  // A halves

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

  // Ring of RING tokens in flight: ring[i % RING] holds token tb + i's raw vectors.
  vec_t ring[C::RING][PV];
  auto fetch = [&](int64_t t, vec_t *dst) {
#pragma unroll
    for (int i = 0; i < PV; ++i) {
      const int vi = lu + i * C::LA;
      const bool ok = vi < NV && t < te;
      const int arr = vi / VPA, f0 = (vi % VPA) * VW;
      dst[i] = ok ? *reinterpret_cast<const vec_t *>(base_in[arr < 3 ? arr : 0] + t * D + f0) : vec_t{};
    }
  };
#pragma unroll
  for (int i = 0; i < C::RING; ++i) fetch(tb + i, ring[i]);

  // Token step; RS is the token's ring slot (t - tb) % RING, a compile-time constant so that
  // the compiler knows which loads each step waits for (a slot chosen at run time made every
  // step wait for all outstanding memory operations, the previous steps' stores included).
  static_assert(C::RING == 4, "the token loop below is unrolled by four");
  auto step = [&](const int64_t t, auto rslot) {
    constexpr int RS = decltype(rslot)::value;
    const int slot = RS & 1;
    float *U = sU[unit_in_blk][slot];
    float *K = sK[unit_in_blk][slot];
    float *Q = sQ[unit_in_blk][slot];
    // (a) token t from the ring into LDS (fp32; phi applied to q).
    {
      const vec_t *cur = ring[RS];
#pragma unroll
      for (int i = 0; i < PV; ++i) {
        const int vi = lu + i * C::LA;
        if (vi < NV) {
          const int arr = vi / VPA, f0 = (vi % VPA) * VW;
          float x[VW];
          IO::unpack(cur[i], x);
          float *dst = arr == 0 ? U : (arr == 1 ? K : Q);
          if (arr == 2)
#pragma unroll
            for (int e = 0; e < VW; ++e) x[e] = phi(x[e]);
#pragma unroll
          for (int e = 0; e < VW; e += 4)
            *reinterpret_cast<float4 *>(&dst[f0 + e]) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
        }
      }
      // (b) refill this ring slot with token t + RING.
      fetch(t + C::RING, ring[RS]);
    }
    unit_sync<C::NWA>();
    // (c) readout normaliser n_t = n_{t-1} + phi(k_t); partial of n_t . phi(q_t).
    float dp = 0.f;
#pragma unroll
    for (int f = 0; f < C::NF; ++f) {
      const int feat = lu + f * C::LA;
      if (feat < D) {
        nrun[f] += phi(K[feat]);
        dp = fmaf(nrun[f], Q[feat], dp);
      }
    }
    // (d) Sherman-Morrison step.
    float z[C::RPL], a[C::RPL];
#pragma unroll
    for (int r = 0; r < C::RPL; ++r) { z[r] = 0.f; a[r] = 0.f; }
    float kk = 0.f;
#pragma unroll
    for (int m = 0; m < C::CW / 4; ++m) {
      const float4 u4 = *reinterpret_cast<const float4 *>(&U[c0 + 4 * m]);
      const float4 k4 = *reinterpret_cast<const float4 *>(&K[c0 + 4 * m]);
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
      sd = fmaf(U[row], z[r], sd);
      sg = fmaf(K[row] * rk, z[r], sg);
    }
    if (h) { sd = 0.f; sg = 0.f; }
    sd = wave_sum(sd);
    sg = wave_sum(sg);
    dp = wave_sum(dp);
    if constexpr (C::NWA > 1) {
      if ((lu & (kWave - 1)) == 0) {
        sRed[0][wside][0] = sd; sRed[0][wside][1] = sg; sRed[0][wside][2] = dp;
      }
      __syncthreads();
      sd = 0.f; sg = 0.f; dp = 0.f;
#pragma unroll
      for (int w = 0; w < C::NWA; ++w) {
        sd += sRed[0][w][0]; sg += sRed[0][w][1]; dp += sRed[0][w][2];
      }
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
    if (lu == 0) *reinterpret_cast<float2 *>(&rd[t * 2]) = make_float2(rk, dp + eps);
    if constexpr (REC) {
      float *rr = brs + t * RF;
      if (h == 0)
#pragma unroll
        for (int r = 0; r < C::RPL; ++r) {
          const int row = g + r * C::HALF;
          rr[BwRec<D>::Z + row] = z[r];
          rr[BwRec<D>::AH + row] = y[r] * inv;
        }
      if (lu == 0) {
        rr[BwRec<D>::SC] = delta;
        rr[BwRec<D>::SC + 1] = sy > 0.f ? sqrtf(sy) : 0.f;
        rr[BwRec<D>::SC + 2] = rk;
        rr[BwRec<D>::SC + 3] = dp + eps;
      }
    }
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
    if (REC && ((t + 1) % kBwCk == 0 || t == te - 1)) {  // A after a checkpoint token
      float *dst = bcs + (t / kBwCk) * 2 * D * D;
#pragma unroll
      for (int r = 0; r < C::RPL; ++r)
#pragma unroll
        for (int m = 0; m < C::CW / 4; ++m)
          *reinterpret_cast<float4 *>(&dst[(g + r * C::HALF) * D + c0 + 4 * m]) =
              make_float4(Mr[r][4 * m], Mr[r][4 * m + 1], Mr[r][4 * m + 2], Mr[r][4 * m + 3]);
    }
    if constexpr (C::NWA > 1) __syncthreads();  // W and the LDS slots are rewritten next
  };
  int64_t t = tb;
  for (; t + C::RING <= te; t += C::RING) {
    step(t, std::integral_constant<int, 0>{});
    step(t + 1, std::integral_constant<int, 1>{});
    step(t + 2, std::integral_constant<int, 2>{});
    step(t + 3, std::integral_constant<int, 3>{});
  }
  if (t < te) step(t, std::integral_constant<int, 0>{});
  if (t + 1 < te) step(t + 1, std::integral_constant<int, 1>{});
  if (t + 2 < te) step(t + 2, std::integral_constant<int, 2>{});
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
  if (n_final != nullptr && p == P - 1) {
#pragma unroll
    for (int f = 0; f < C::NF; ++f) {
      const int feat = lu + f * C::LA;
      if (feat < D) n_final[s * D + feat] = nrun[f];
    }
  }
  if constexpr (REC) {  // n after the segment (the backward's records)
#pragma unroll
    for (int f = 0; f < C::NF; ++f) {
      const int feat = lu + f * C::LA;
      if (feat < D) bnend[(s * P + p) * D + feat] = nrun[f];
    }
  }
}

// ------------------------------------------------------------------------------------
// k_swy: the S recurrence of one segment in WY form, one 16-row slice of the state per wave.
//   FINAL: state S (d rows) from the true segment start; writes outputs and S_T.
//   MAP:   state Pi (blockIdx.z = 0, from I, no values) or B (blockIdx.z = 1, from 0 with
//          the values v); writes the segment map.
// The state is held transposed (X^T, d x 16 per wave) in MFMA accumulators.
//
// LDS operands are packed "k-minor": element (k, i) of an MFMA operand lives at
// [k / 4][i][k % 4], so the four k-steps a lane feeds in one 16-slice are one float4.
// ------------------------------------------------------------------------------------
template <int D, int CH, bool FINAL>
struct SwyCfg {
  static constexpr int NWV = D / 16;    // waves = 16-row state slices per workgroup
  static constexpr int NT = NWV * kWave;
  static constexpr int NCT = CH / 16;   // 16-token tiles per chunk
  static constexpr int NFT = D / 16;    // 16-feature tiles
  static constexpr int NKT = NCT * (NCT + 1) / 2;
  static constexpr int DP = D + 1;      // padded feature count of the token-packed ahat
};

__device__ __forceinline__ float4 lds4(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}

// With REC (final pass only) the kernel writes r and o of the backward's token records and the
// S half of the state checkpoints in place of the outputs.
template <int D, int CH, bool FINAL, typename TIn, bool REC = false>
__global__ void __launch_bounds__((SwyCfg<D, CH, FINAL>::NT))
k_swy(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
      const float *__restrict__ alpha, const float *__restrict__ rkden,
      const float *__restrict__ s0, float *__restrict__ pib, TIn *__restrict__ out,
      float *__restrict__ S_final, int64_t T, int64_t L, int64_t P, float *__restrict__ brec,
      float *__restrict__ bck) {
  static_assert(FINAL || !REC, "records come from the final pass");
  using C = SwyCfg<D, CH, FINAL>;
  using IO = io<TIn>;
  using vec_t = typename IO::vec_t;
  constexpr int VW = IO::kVec;
  // [f/4][c][f%4]: khat, phi(q), ahat packed by feature; [c/4][f][c%4]: ahat packed by token.
  __shared__ __attribute__((aligned(16))) float KhP[D / 4][CH][4];
  __shared__ __attribute__((aligned(16))) float AlP[D / 4][CH][4];
  __shared__ __attribute__((aligned(16))) float FqP[FINAL ? D / 4 : 1][CH][4];
  __shared__ __attribute__((aligned(16))) float AcP[CH / 4][C::DP][4];
  // [c''/4][c][c''%4]: -(strict lower of Kh ahat^T) and lower(Fq ahat^T), packed by column.
  __shared__ __attribute__((aligned(16))) float KaP[CH / 4][CH][4];
  __shared__ __attribute__((aligned(16))) float QaP[FINAL ? CH / 4 : 1][CH][4];
  // Inverses of the unit-lower diagonal 16-blocks of I + Ka: [b][k/4][i][k%4].
  __shared__ __attribute__((aligned(16))) float InvP[C::NCT][4][16][4];
  __shared__ __attribute__((aligned(16))) TIn sV[CH][D];   // the chunk's values (input dtype)
  __shared__ float sRden[CH];                                // 1 / readout denominator

  const int64_t s = blockIdx.x, p = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, gq = lane >> 4;
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const TIn *ks = k + s * T * D;
  const TIn *vs = v + s * T * D;
  const TIn *qs = q + s * T * D;
  const float *als = alpha + s * T * D;
  const float *rds = rkden + s * T * 2;
  constexpr int RF = BwRec<D>::F;
  float *brs = REC ? brec + s * T * RF : nullptr;
  float *bcs = REC ? bck + s * ((T + kBwCk - 1) / kBwCk) * 2 * D * D : nullptr;  // S halves

  const bool pi_rows = !FINAL && blockIdx.z == 0;
  const int rowbase = 16 * wave;
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

  // Register prefetch of a chunk: 16-byte vectors of k, q, v and float4 of ahat; lanes run
  // over consecutive tokens so the packed LDS writes are contiguous.
  constexpr int UK = CH * D / VW;
  constexpr int UA = CH * D / 4;
  constexpr int PK = (UK + C::NT - 1) / C::NT;
  constexpr int PA = (UA + C::NT - 1) / C::NT;
  vec_t pk[PK], pq[FINAL ? PK : 1], pv[PK];
  float prk[PK];
  float4 pa[PA];
  float pden = 1.f;
  auto prefetch = [&](int64_t cs) {
    const int mm = static_cast<int>(std::min<int64_t>(CH, te - cs));
#pragma unroll
    for (int i = 0; i < PK; ++i) {
      const int ui = tid + i * C::NT;
      const int c = ui % CH, f0 = (ui / CH) * VW;
      const bool ok = ui < UK && c < mm;
      const int64_t off = (cs + c) * D + f0;
      pk[i] = ok ? *reinterpret_cast<const vec_t *>(ks + off) : vec_t{};
      prk[i] = ok ? rds[(cs + c) * 2] : 0.f;
      if constexpr (FINAL) pq[i] = ok ? *reinterpret_cast<const vec_t *>(qs + off) : vec_t{};
      pv[i] = (ok && has_v) ? *reinterpret_cast<const vec_t *>(vs + off) : vec_t{};
    }
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int ui = tid + i * C::NT;
      const int c = ui % CH, f0 = (ui / CH) * 4;
      const bool ok = ui < UA && c < mm;
      pa[i] = ok ? *reinterpret_cast<const float4 *>(als + (cs + c) * D + f0)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if constexpr (FINAL) pden = (tid < mm) ? rds[(cs + tid) * 2 + 1] : 1.f;
  };
  prefetch(tb);

  for (int64_t c0 = tb; c0 < te; c0 += CH) {
    const int m = static_cast<int>(std::min<int64_t>(CH, te - c0));
    __syncthreads();
    // ---- stage the chunk from registers -----------------------------------------------
#pragma unroll
    for (int i = 0; i < PK; ++i) {
      const int ui = tid + i * C::NT;
      if (ui < UK) {
        const int c = ui % CH, f0 = (ui / CH) * VW;
        float kf[VW];
        IO::unpack(pk[i], kf);
#pragma unroll
        for (int e = 0; e < VW; e += 4)
          *reinterpret_cast<float4 *>(&KhP[(f0 + e) / 4][c][0]) =
              make_float4(kf[e] * prk[i], kf[e + 1] * prk[i], kf[e + 2] * prk[i], kf[e + 3] * prk[i]);
        if constexpr (FINAL) {
          float qf[VW];
          IO::unpack(pq[i], qf);
          const bool ok = c < m;
#pragma unroll
          for (int e = 0; e < VW; e += 4)
            *reinterpret_cast<float4 *>(&FqP[(f0 + e) / 4][c][0]) =
                ok ? make_float4(phi(qf[e]), phi(qf[e + 1]), phi(qf[e + 2]), phi(qf[e + 3]))
                   : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        *reinterpret_cast<vec_t *>(&sV[c][f0]) = pv[i];
      }
    }
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int ui = tid + i * C::NT;
      if (ui < UA) {
        const int c = ui % CH, f0 = (ui / CH) * 4;
        *reinterpret_cast<float4 *>(&AlP[f0 / 4][c][0]) = pa[i];
        AcP[c / 4][f0 + 0][c % 4] = pa[i].x;
        AcP[c / 4][f0 + 1][c % 4] = pa[i].y;
        AcP[c / 4][f0 + 2][c % 4] = pa[i].z;
        AcP[c / 4][f0 + 3][c % 4] = pa[i].w;
      }
    }
    if constexpr (FINAL)
      if (tid < CH) sRden[tid] = 1.0f / pden;
    __syncthreads();
    // ---- shared chunk products (diagonal tiles first; each diagonal Ka tile's wave also
    //      inverts its unit-lower block) ------------------------------------------------
    for (int job = wave; job < (FINAL ? 2 : 1) * C::NKT; job += C::NWV) {
      const bool isq = job >= C::NKT;
      const int jj = isq ? job - C::NKT : job;
      int ct, ct2;
      if (jj < C::NCT) {
        ct = ct2 = jj;                          // diagonal tiles
      } else {
        int t = jj - C::NCT;                    // strictly-lower tiles, row by row
        ct = 1;
        while (t >= ct) { t -= ct; ++ct; }
        ct2 = t;
      }
      f4_t acc = f4_zero();
#pragma unroll
      for (int kt = 0; kt < C::NFT; ++kt) {
        const float4 a4 = isq ? lds4(&FqP[FINAL ? 4 * kt + gq : 0][16 * ct + li][0])
                              : lds4(&KhP[4 * kt + gq][16 * ct + li][0]);
        const float4 b4 = lds4(&AlP[4 * kt + gq][16 * ct2 + li][0]);
        acc = mfma_f32_16x16x4(a4.x, b4.x, acc);
        acc = mfma_f32_16x16x4(a4.y, b4.y, acc);
        acc = mfma_f32_16x16x4(a4.z, b4.z, acc);
        acc = mfma_f32_16x16x4(a4.w, b4.w, acc);
      }
      // acc[r] = product[c = 16 ct + 4 gq + r][c'' = 16 ct2 + li]
      const int cc = 16 * ct2 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * gq + r;
        float val = acc[r];
        if (ct == ct2 && (isq ? (li > i) : (li >= i))) val = 0.f;
        if (isq) {
          if constexpr (FINAL) QaP[cc / 4][16 * ct + i][cc % 4] = val;
        } else {
          KaP[cc / 4][16 * ct + i][cc % 4] = -val;
        }
      }
      if (!isq && ct == ct2) {
        // (I + Ka_bb)^{-1} by forward substitution in lanes 0..15 (column j = lane).
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < 16) {
          const int b = ct, j = lane;
          float x[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float a = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int i2 = 0; i2 < i; ++i2) {
              const int c2 = 16 * b + i2;
              a = fmaf(KaP[c2 / 4][16 * b + i][c2 % 4], x[i2], a);  // KaP holds -Ka
            }
            x[i] = a;
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) InvP[b][j / 4][i][j % 4] = x[i];  // Inv[i][j] = x_j[i]
        }
      }
    }
    __syncthreads();
    // ---- this wave's rows -------------------------------------------------------------
    f4_t E[C::NCT];
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) {
      f4_t acc = f4_zero();
#pragma unroll
      for (int kt = 0; kt < C::NFT; ++kt) {
        const float4 a4 = lds4(&KhP[4 * kt + gq][16 * ct + li][0]);
        acc = mfma_f32_16x16x4(a4.x, X[kt][0], acc);
        acc = mfma_f32_16x16x4(a4.y, X[kt][1], acc);
        acc = mfma_f32_16x16x4(a4.z, X[kt][2], acc);
        acc = mfma_f32_16x16x4(a4.w, X[kt][3], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float vv = has_v ? load_elem(&sV[0][0], (16 * ct + 4 * gq + r) * D + rowbase + li) : 0.f;
        acc[r] = vv - acc[r];
      }
      E[ct] = acc;  // R = Vx - Kh X^T
    }
    // The next chunk's loads fly during the solve, the readout and the state update.
    if (c0 + CH < te) prefetch(c0 + CH);
    // E = (I + Ka)^{-1} R by block forward substitution (KaP holds -Ka).
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) {
      f4_t acc = E[ct];
#pragma unroll
      for (int ct2 = 0; ct2 < ct; ++ct2) {
        const float4 a4 = lds4(&KaP[4 * ct2 + gq][16 * ct + li][0]);
        acc = mfma_f32_16x16x4(a4.x, E[ct2][0], acc);
        acc = mfma_f32_16x16x4(a4.y, E[ct2][1], acc);
        acc = mfma_f32_16x16x4(a4.z, E[ct2][2], acc);
        acc = mfma_f32_16x16x4(a4.w, E[ct2][3], acc);
      }
      const float4 i4 = lds4(&InvP[ct][gq][li][0]);
      f4_t e = f4_zero();
      e = mfma_f32_16x16x4(i4.x, acc[0], e);
      e = mfma_f32_16x16x4(i4.y, acc[1], e);
      e = mfma_f32_16x16x4(i4.z, acc[2], e);
      e = mfma_f32_16x16x4(i4.w, acc[3], e);
      E[ct] = e;
    }
    if constexpr (REC) {  // r_t = v_t - S_{t-1} khat_t: the rows of E
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 16 * ct + 4 * gq + r;
          if (c < m) brs[(c0 + c) * RF + BwRec<D>::R + rowbase + li] = E[ct][r];
        }
    }
    if constexpr (FINAL) {
      // Num = Fq X_start^T + lower(Fq ahat^T) E, then o = Num / den.
      TIn *os = REC ? nullptr : out + s * T * D;
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct) {
        f4_t acc = f4_zero();
#pragma unroll
        for (int kt = 0; kt < C::NFT; ++kt) {
          const float4 a4 = lds4(&FqP[4 * kt + gq][16 * ct + li][0]);
          acc = mfma_f32_16x16x4(a4.x, X[kt][0], acc);
          acc = mfma_f32_16x16x4(a4.y, X[kt][1], acc);
          acc = mfma_f32_16x16x4(a4.z, X[kt][2], acc);
          acc = mfma_f32_16x16x4(a4.w, X[kt][3], acc);
        }
#pragma unroll
        for (int ct2 = 0; ct2 <= ct; ++ct2) {
          const float4 a4 = lds4(&QaP[4 * ct2 + gq][16 * ct + li][0]);
          acc = mfma_f32_16x16x4(a4.x, E[ct2][0], acc);
          acc = mfma_f32_16x16x4(a4.y, E[ct2][1], acc);
          acc = mfma_f32_16x16x4(a4.z, E[ct2][2], acc);
          acc = mfma_f32_16x16x4(a4.w, E[ct2][3], acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 16 * ct + 4 * gq + r;
          if constexpr (REC) {
            if (c < m) brs[(c0 + c) * RF + BwRec<D>::O + rowbase + li] = acc[r] * sRden[c];  // o, fp32
          } else {
            if (c < m) store_elem(os, (c0 + c) * D + rowbase + li, acc[r] * sRden[c]);
          }
        }
      }
    }
    // X^T += ahat^T E.
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
      for (int ft = 0; ft < C::NFT; ++ft) {
        const float4 a4 = lds4(&AcP[4 * ct + gq][16 * ft + li][0]);
        X[ft] = mfma_f32_16x16x4(a4.x, E[ct][0], X[ft]);
        X[ft] = mfma_f32_16x16x4(a4.y, E[ct][1], X[ft]);
        X[ft] = mfma_f32_16x16x4(a4.z, E[ct][2], X[ft]);
        X[ft] = mfma_f32_16x16x4(a4.w, E[ct][3], X[ft]);
      }
    if (REC && ((c0 + m) % kBwCk == 0 || c0 + m == te)) {  // S after a checkpoint token
      float *dst = bcs + ((c0 + m - 1) / kBwCk) * 2 * D * D;
#pragma unroll
      for (int ft = 0; ft < C::NFT; ++ft)
        *reinterpret_cast<float4 *>(&dst[(rowbase + li) * D + 16 * ft + 4 * gq]) =
            make_float4(X[ft][0], X[ft][1], X[ft][2], X[ft][3]);
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
// k_sprefix: S_0 = 0, S_{p+1} = S_p Pi_p + B_p.  A row of S_{p+1} depends only on the same
// row of S_p, so each workgroup scans one 16-row tile of one stream: grid (streams, D/16).
// Wave w owns output columns 16w..16w+15 (S^T in MFMA accumulators: X[r] = S[row li]
// [16w + 4gq + r]) and reads its 96 x 16 column slice of Pi_p straight from memory in the
// A-operand layout, four (two at d = 128) segments ahead.  The row tile of S_p is exchanged between the waves
// through a double-buffered LDS copy (one barrier per segment).
// ------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(D / 16 * kWave)
k_sprefix(const float *__restrict__ pib, float *__restrict__ s0, int64_t P,
          const float *__restrict__ S0, float *__restrict__ nk, const float *__restrict__ n0,
          float *__restrict__ n_final, float *__restrict__ n_end) {
  constexpr int NFT = D / 16;
  __shared__ __attribute__((aligned(16))) float Xs[2][D / 4][16][4];  // S^T[f'][row], f' % 4 minor
  const int64_t s = blockIdx.x;
  // bf16 inputs: the readout normaliser at every segment start, n_p = n_0 + sum_{p' < p} nk_p'
  // (nk_p' = the sum of phi(k) over segment p', formed by the A side), in place, in fp64
  // sums, and n_T when wanted.
  if (nk != nullptr && blockIdx.y == 0 && threadIdx.x < D) {
    const int f = threadIdx.x;
    double acc = n0 != nullptr ? static_cast<double>(n0[s * D + f]) : 0.0;
    float *base = nk + s * P * D + f;
    for (int64_t p0 = 0; p0 < P; p0 += 16) {
      float g[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) g[i] = (p0 + i < P) ? base[(p0 + i) * D] : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (p0 + i < P) base[(p0 + i) * D] = static_cast<float>(acc);
        acc += g[i];
        // n after segment p0 + i (the backward's records)
        if (n_end != nullptr && p0 + i < P) n_end[(s * P + p0 + i) * D + f] = static_cast<float>(acc);
      }
    }
    if (n_final != nullptr) n_final[s * D + f] = static_cast<float>(acc);
  }
  const int rt = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, gq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = 16 * rt + li, col = 16 * w + 4 * gq;
  // S at the first segment start: 0, or a carried S_0
  const float4 st0 = S0 != nullptr ? *reinterpret_cast<const float4 *>(&S0[s * D * D + row * D + col])
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
  *reinterpret_cast<float4 *>(&s0[(s * P) * D * D + row * D + col]) = st0;
  *reinterpret_cast<float4 *>(&Xs[0][4 * w + gq][li][0]) = st0;
  // a[slot][kt][e] = Pi[16 kt + 4 gq + e][16 w + li];  b[slot] = B[row][col .. col + 3].
  // Segment p's map lives in slot p % NSL and is loaded NSL segments ahead, so a step waits for
  // memory only when a load takes longer than NSL steps.
  constexpr int NSL = (D <= 96) ? 4 : 2;  // register budget at d = 128
  float a[NSL][NFT][4];
  float4 b[NSL];
  auto load = [&](int64_t pseg, int slot) {
    const float *Pi = pib + (s * P + pseg) * 2 * D * D;
#pragma unroll
    for (int kt = 0; kt < NFT; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) a[slot][kt][e] = Pi[(16 * kt + 4 * gq + e) * D + 16 * w + li];
    b[slot] = *reinterpret_cast<const float4 *>(&Pi[D * D + row * D + col]);
  };
#pragma unroll
  for (int i = 0; i < NSL; ++i)
    if (i + 1 < P) load(i, i);
  for (int64_t p0 = 0; p0 + 1 < P; p0 += NSL)
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    const int64_t p = p0 + i;
    if (p + 1 >= P) break;
    const int cur = static_cast<int>(p & 1);
    float ac[NFT][4];
#pragma unroll
    for (int kt = 0; kt < NFT; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) ac[kt][e] = a[i][kt][e];
    f4_t y[4] = {f4_t{b[i].x, b[i].y, b[i].z, b[i].w}, f4_zero(), f4_zero(), f4_zero()};
    __syncthreads();
    if (p + NSL + 1 < P) load(p + NSL, i);
    // Y^T[f][row] = B^T[f][row] + sum_f' Pi[f'][f] S^T[f'][row], four independent chains
#pragma unroll
    for (int kt = 0; kt < NFT; ++kt) {
      const float4 x = *reinterpret_cast<const float4 *>(&Xs[cur][4 * kt + gq][li][0]);
      y[0] = mfma_f32_16x16x4(ac[kt][0], x.x, y[0]);
      y[1] = mfma_f32_16x16x4(ac[kt][1], x.y, y[1]);
      y[2] = mfma_f32_16x16x4(ac[kt][2], x.z, y[2]);
      y[3] = mfma_f32_16x16x4(ac[kt][3], x.w, y[3]);
    }
    float4 o;
    o.x = (y[0][0] + y[1][0]) + (y[2][0] + y[3][0]);
    o.y = (y[0][1] + y[1][1]) + (y[2][1] + y[3][1]);
    o.z = (y[0][2] + y[1][2]) + (y[2][2] + y[3][2]);
    o.w = (y[0][3] + y[1][3]) + (y[2][3] + y[3][3]);
    *reinterpret_cast<float4 *>(&Xs[cur ^ 1][4 * w + gq][li][0]) = o;
    *reinterpret_cast<float4 *>(&s0[(s * P + p + 1) * D * D + row * D + col]) = o;
  }
}

// ------------------------------------------------------------------------------------
// Host launch
// ------------------------------------------------------------------------------------
template <int D, int CH, typename TIn>
static hipError_t launch_chunk_t(const Problem &pr, const ChunkPlan &pl, const void *q,
                                 const void *k, const void *v, const void *u, void *out,
                                 const StateIO &sio, char *ws, hipStream_t st, bool states_only,
                                 double *Md, const BwRecords *rec = nullptr) {
  if (rec != nullptr && states_only) return hipErrorInvalidValue;
  const TIn *qq = static_cast<const TIn *>(q);
  const TIn *kk = static_cast<const TIn *>(k);
  const TIn *vv = static_cast<const TIn *>(v);
  const TIn *uu = static_cast<const TIn *>(u);
  TIn *oo = static_cast<TIn *>(out);
  float *Mw = reinterpret_cast<float *>(ws + pl.off_m);
  float *nkw = reinterpret_cast<float *>(ws + pl.off_nk);
  float *alw = reinterpret_cast<float *>(ws + pl.off_alpha);
  // bf16 inputs: ahat as its two bf16 terms, each token's row [hi d | lo d] (same bytes)
  uint16_t *alh = reinterpret_cast<uint16_t *>(ws + pl.off_alpha);
  float *rdw = reinterpret_cast<float *>(ws + pl.off_rkden);
  float *pbw = reinterpret_cast<float *>(ws + pl.off_pib);
  float *s0w = reinterpret_cast<float *>(ws + pl.off_s0);
  float *miw = reinterpret_cast<float *>(ws + pl.off_minv);
  float *S_final = sio.S_final, *A_final = sio.A_final, *n_final = sio.n_final;
  const unsigned S = static_cast<unsigned>(pl.S), P = static_cast<unsigned>(pl.P);
  const dim3 gmat(S, (D * D + 255) / 256);

  if (P > 1) {
    VLA_LAUNCH("k_gram", (k_gram<D, TIn>), dim3(S, P - 1), dim3(256), 0, st, uu, kk, Mw, nkw,
                       pl.T, pl.L, pl.P);
  }
  if (sio.A0 != nullptr) {  // M_0 = A_0^{-1} for the segment prefix
    VLA_LAUNCH("k_sym_copy", (k_sym_copy<D>), gmat, dim3(256), 0, st, sio.A0, miw,
               static_cast<int64_t>(D) * D);
    VLA_LAUNCH("k_inv", (k_inv<D>), dim3(S, 1), dim3(256), 0, st, miw, int64_t(1));
  }
  constexpr bool BF = sizeof(TIn) == 2;  // bf16: the A side forms the segment sums of phi(k)
  VLA_LAUNCH("k_prefix", (k_prefix<D>), gmat, dim3(256), 0, st, Mw, nkw, pl.P, pr.lambda0,
             sio.A0 != nullptr ? static_cast<const float *>(miw) : nullptr, sio.n0, BF ? 0 : 1, Md);
  if (Md != nullptr)
    VLA_LAUNCH("k_inv64", (k_inv64<D>), dim3(S, P), dim3(256), 0, st, static_cast<const double *>(Md),
               Mw, pl.P);
  else
    VLA_LAUNCH("k_inv", (k_inv<D>), dim3(S, P), dim3(256), 0, st, Mw, pl.P);
  if (sio.A0 != nullptr) {  // the first segment starts from A_0 itself
    VLA_LAUNCH("k_sym_copy", (k_sym_copy<D>), gmat, dim3(256), 0, st, sio.A0, Mw,
               static_cast<int64_t>(pl.P) * D * D);
  }
  if constexpr (sizeof(TIn) == 2) {
    // bf16 inputs: chunked A side on the bf16 matrix cores.
    // Three-term operands when the Sherman-Morrison steps cancel strongly: from A_0 = I / lambda0
    // with lambda0 < d / 256 (unit-variance inputs then give cancellation factors above ~256,
    // which two-term operands, 16 significant bits, cannot absorb).
    const bool three = sio.A0 == nullptr && pr.lambda0 < static_cast<float>(D) / 256.0f;
    // d = 96, two-term operands, an even number of streams: the same segment of two streams per
    // workgroup (twelve waves, three per SIMD), in the A side and in the final pass
    constexpr int NP = D == 96 ? 2 : 1;
    const bool pair = NP == 2 && S % 2 == 0;
    if (rec != nullptr) {  // with the backward's records (z, ahat, delta, ||A khat||, A checkpoints)
      if (three)
        VLA_LAUNCH("k_aside_wy", (k_aside_wy<D, 3, true>), dim3(S, P), dim3(AwyCfg<D, 3>::NT), 0, st,
                   qq, kk, uu, Mw, nkw, alh, rdw, A_final, pl.T, pl.L, pl.P, pr.eps, rec->rec, rec->ck);
      else if (pair)
        VLA_LAUNCH("k_aside_wy", (k_aside_wy<D, 2, true, NP>), dim3(S / NP, P), dim3(NP * AwyCfg<D, 2>::NT),
                   0, st, qq, kk, uu, Mw, nkw, alh, rdw, A_final, pl.T, pl.L, pl.P, pr.eps, rec->rec,
                   rec->ck);
      else
        VLA_LAUNCH("k_aside_wy", (k_aside_wy<D, 2, true>), dim3(S, P), dim3(AwyCfg<D, 2>::NT), 0, st,
                   qq, kk, uu, Mw, nkw, alh, rdw, A_final, pl.T, pl.L, pl.P, pr.eps, rec->rec, rec->ck);
    } else if (three) {
      VLA_LAUNCH("k_aside_wy", (k_aside_wy<D, 3>), dim3(S, P), dim3(AwyCfg<D, 3>::NT), 0, st, qq,
                 kk, uu, Mw, nkw, alh, rdw, A_final, pl.T, pl.L, pl.P, pr.eps,
                 static_cast<float *>(nullptr), static_cast<float *>(nullptr));
    } else if (pair) {
      VLA_LAUNCH("k_aside_wy", (k_aside_wy<D, 2, false, NP>), dim3(S / NP, P), dim3(NP * AwyCfg<D, 2>::NT),
                 0, st, qq, kk, uu, Mw, nkw, alh, rdw, A_final, pl.T, pl.L, pl.P, pr.eps,
                 static_cast<float *>(nullptr), static_cast<float *>(nullptr));
    } else {
      VLA_LAUNCH("k_aside_wy", (k_aside_wy<D, 2>), dim3(S, P), dim3(AwyCfg<D, 2>::NT), 0, st, qq,
                 kk, uu, Mw, nkw, alh, rdw, A_final, pl.T, pl.L, pl.P, pr.eps,
                 static_cast<float *>(nullptr), static_cast<float *>(nullptr));
    }
  } else {
    using AC = AsideCfg<D>;
    const int64_t units = pl.S * pl.P;
    const unsigned blocks = static_cast<unsigned>((units + AC::UPB - 1) / AC::UPB);
    if (rec != nullptr)  // with the backward's records (z, ahat, scalars, A checkpoints)
      VLA_LAUNCH("k_aside", (k_aside<D, TIn, true>), dim3(blocks), dim3(AC::NT), 0, st, qq, kk, uu, Mw,
                 nkw, alw, rdw, A_final, n_final, pl.S, pl.T, pl.L, pl.P, pr.eps, rec->rec, rec->ck,
                 rec->n_end);
    else
      VLA_LAUNCH("k_aside", (k_aside<D, TIn>), dim3(blocks), dim3(AC::NT), 0, st, qq, kk, uu, Mw,
                 nkw, alw, rdw, A_final, n_final, pl.S, pl.T, pl.L, pl.P, pr.eps,
                 static_cast<float *>(nullptr), static_cast<float *>(nullptr), static_cast<float *>(nullptr));
  }
  if constexpr (sizeof(TIn) == 2) {
    // bf16 inputs: S side on the bf16 matrix cores.  The map pass covers the segments
    // p < npre (with the backward's records all of them: the backward reads every segment's
    // Pi but the first's) and leaves its tiles for the final pass to load.
    const unsigned npre = rec != nullptr ? P : P - 1;
    uint16_t *tlw = pl.tiles && rec == nullptr ? reinterpret_cast<uint16_t *>(ws + pl.off_tiles) : nullptr;
    const int64_t npf = static_cast<int64_t>(npre);
    if (P > 1) {
      VLA_LAUNCH("k_swy_map", (k_swyb<D, CH, false>), dim3(S, npre),
                 dim3(SwbCfg<D, CH, false>::NT), 0, st, qq, kk, vv, alh, rdw, s0w, pbw, oo,
                 S_final, static_cast<const float *>(nullptr), pl.T, pl.L, pl.P,
                 static_cast<float *>(nullptr), static_cast<float *>(nullptr), tlw, int64_t(0));
    }
    VLA_LAUNCH("k_sprefix", (k_sprefix<D>), dim3(S, D / 16), dim3(D / 16 * kWave), 0, st, pbw,
               s0w, pl.P, sio.S0, nkw, sio.n0, n_final, rec != nullptr ? rec->n_end : nullptr);
    if (states_only) return hipGetLastError();
    // The final pass runs in chunks of at most 32 tokens whatever the map pass uses: its
    // workgroup then fits twice per CU (54 KB of LDS and 127 VGPRs at d = 96), and the
    // segment maps it starts from do not depend on either pass's chunking.
    constexpr int CF = CH < 32 ? CH : 32;
    // d = 96 and an even number of streams: the same segment of two streams per workgroup
    constexpr int NP = D == 96 ? 2 : 1;
    const bool pair = NP == 2 && S % 2 == 0;
    if (rec != nullptr && pair)  // the backward's records (r, o, 1/||k||, den, S checkpoints)
      VLA_LAUNCH("k_swy_final", (k_swyb<D, CF, true, true, NP>), dim3(S / NP, P),
                 dim3(NP * SwbCfg<D, CF, true>::NT), 0, st, qq, kk, vv, alh, rdw, s0w, pbw,
                 static_cast<TIn *>(nullptr), S_final, nkw, pl.T, pl.L, pl.P, rec->rec, rec->ck, tlw, npf);
    else if (rec != nullptr)
      VLA_LAUNCH("k_swy_final", (k_swyb<D, CF, true, true>), dim3(S, P), dim3(SwbCfg<D, CF, true>::NT),
                 0, st, qq, kk, vv, alh, rdw, s0w, pbw, static_cast<TIn *>(nullptr), S_final, nkw, pl.T,
                 pl.L, pl.P, rec->rec, rec->ck, tlw, npf);
    else if (pair)
      VLA_LAUNCH("k_swy_final", (k_swyb<D, CF, true, false, NP>), dim3(S / NP, P),
                 dim3(NP * SwbCfg<D, CF, true>::NT), 0, st, qq, kk, vv, alh, rdw, s0w, pbw, oo, S_final,
                 nkw, pl.T, pl.L, pl.P, static_cast<float *>(nullptr), static_cast<float *>(nullptr), tlw,
                 npf);
    else
      VLA_LAUNCH("k_swy_final", (k_swyb<D, CF, true>), dim3(S, P), dim3(SwbCfg<D, CF, true>::NT), 0,
                 st, qq, kk, vv, alh, rdw, s0w, pbw, oo, S_final, nkw, pl.T, pl.L, pl.P,
                 static_cast<float *>(nullptr), static_cast<float *>(nullptr), tlw, npf);
  } else {
    if (P > 1) {
      VLA_LAUNCH("k_swy_map", (k_swy<D, CH, false, TIn>), dim3(S, rec != nullptr ? P : P - 1, 2),
                 dim3(SwyCfg<D, CH, false>::NT), 0, st, qq, kk, vv, alw, rdw, s0w, pbw, oo,
                 S_final, pl.T, pl.L, pl.P, static_cast<float *>(nullptr), static_cast<float *>(nullptr));
    }
    VLA_LAUNCH("k_sprefix", (k_sprefix<D>), dim3(S, D / 16), dim3(D / 16 * kWave), 0, st, pbw,
               s0w, pl.P, sio.S0, static_cast<float *>(nullptr), static_cast<const float *>(nullptr),
               static_cast<float *>(nullptr), static_cast<float *>(nullptr));
    if (states_only) return hipGetLastError();
    if (rec != nullptr)  // the backward's records (r, o) and S checkpoints
      VLA_LAUNCH("k_swy_final", (k_swy<D, CH, true, TIn, true>), dim3(S, P),
                 dim3(SwyCfg<D, CH, true>::NT), 0, st, qq, kk, vv, alw, rdw, s0w, pbw,
                 static_cast<TIn *>(nullptr), S_final, pl.T, pl.L, pl.P, rec->rec, rec->ck);
    else
      VLA_LAUNCH("k_swy_final", (k_swy<D, CH, true, TIn>), dim3(S, P),
                 dim3(SwyCfg<D, CH, true>::NT), 0, st, qq, kk, vv, alw, rdw, s0w, pbw, oo, S_final,
                 pl.T, pl.L, pl.P, static_cast<float *>(nullptr), static_cast<float *>(nullptr));
  }
  return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_chunk_dt(const Problem &pr, const ChunkPlan &pl, const void *q,
                                  const void *k, const void *v, const void *u, void *out,
                                  const StateIO &sio, char *ws, hipStream_t st, bool states_only,
                                  double *Md, const BwRecords *rec = nullptr) {
#define VLA_CASE(DD, CC)                                                                      \
  if (pr.d == DD && pl.C == CC)                                                               \
    return launch_chunk_t<DD, CC, TIn>(pr, pl, q, k, v, u, out, sio, ws, st, states_only, Md, rec);
  VLA_CASE(32, 16) VLA_CASE(32, 32) VLA_CASE(32, 64)
  VLA_CASE(64, 16) VLA_CASE(64, 32) VLA_CASE(64, 64)
  VLA_CASE(96, 16) VLA_CASE(96, 32) VLA_CASE(96, 64)
  VLA_CASE(128, 16) VLA_CASE(128, 32)
#undef VLA_CASE
  return hipErrorInvalidValue;
}

// Streams [h, h + n) of a call: the same segments (L and P of the whole call's plan, so every
// stream's arithmetic is the same as in one launch over all streams), every workspace array
// and every input, output and state pointer moved to stream h (all are stream-major).
static hipError_t launch_chunk_group(const Problem &p, const ChunkPlan &pl, int64_t h, int64_t n,
                                     const void *q, const void *k, const void *v, const void *u,
                                     void *out, const StateIO &st, char *w, hipStream_t stream) {
  const size_t D = static_cast<size_t>(pl.D), P = static_cast<size_t>(pl.P);
  const size_t T = static_cast<size_t>(pl.T), hs = static_cast<size_t>(h);
  ChunkPlan g = pl;
  g.S = n;
  g.off_m += hs * P * D * D * 4;
  g.off_nk += hs * P * D * 4;
  g.off_alpha += hs * T * D * 4;
  g.off_rkden += hs * T * 2 * 4;
  g.off_pib += hs * P * 2 * D * D * 4;
  g.off_s0 += hs * P * D * D * 4;
  g.off_minv += hs * D * D * 4;
  g.off_tiles += hs * static_cast<size_t>(swb_tile_blocks(pl.T)) * kSwbTileBlock * 2;
  Problem gp = p;
  gp.streams = n;
  const size_t tok = hs * T * D * (p.dtype == Dtype::F32 ? 4 : 2);
  auto in = [&](const void *x) { return static_cast<const void *>(static_cast<const char *>(x) + tok); };
  auto mat = [&](auto *x, size_t per) { return x != nullptr ? x + hs * per : x; };
  StateIO gs;
  gs.S0 = mat(st.S0, D * D);
  gs.A0 = mat(st.A0, D * D);
  gs.n0 = mat(st.n0, D);
  gs.S_final = mat(st.S_final, D * D);
  gs.A_final = mat(st.A_final, D * D);
  gs.n_final = mat(st.n_final, D);
  void *o = static_cast<char *>(out) + tok;
  if (p.dtype == Dtype::F32)
    return launch_chunk_dt<float>(gp, g, in(q), in(k), in(v), in(u), o, gs, w, stream, false, nullptr);
  return launch_chunk_dt<bf16_t>(gp, g, in(q), in(k), in(v), in(u), o, gs, w, stream, false, nullptr);
}

// The library's second HIP stream on the current device: created once, default priority,
// not synchronised with the legacy null stream (ordering comes from events only).  nullptr if
// it cannot be created.
static hipStream_t side_stream() {
  static std::mutex mu;
  static std::vector<hipStream_t> per_device;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (static_cast<int>(per_device.size()) <= dev) per_device.resize(dev + 1, nullptr);
  if (per_device[dev] == nullptr) {
    hipStream_t s = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess) per_device[dev] = s;
  }
  return per_device[dev];
}

// Whether a call's streams run as two groups on two HIP streams.  Each pass then ends in two
// partly filled last waves of workgroups instead of one, and each group's short scan passes
// (k_prefix, k_inv, k_sprefix: a few hundred workgroups) run beside the other group's long
// ones.  On 32 streams x 131072 tokens at d = 96 this takes about 3 % off the call, on
// 32 x 43008 at d = 128 about 8 %; below about 2^20 tokens per call the extra launches and
// events cost more than the overlap gains (4 x 8 x 4096 at d = 64: 2 % slower).  Not used
// while the stream is being captured into a graph.
static bool split_in_two(const Problem &p, hipStream_t stream) {
  if (p.streams < 2 || p.streams * p.T < (int64_t(1) << 20)) return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();  // not a failure of this call
    return false;
  }
  return cs == hipStreamCaptureStatusNone;
}

hipError_t launch_chunk(const Problem &p, int chunk, const void *q, const void *k,
                        const void *v, const void *u, void *out, const StateIO &st, void *ws,
                        hipStream_t stream, bool may_split) {
  if (!chunk_supported(p, chunk)) return hipErrorInvalidValue;
  const ChunkPlan pl = make_plan(p, chunk);
  char *w = static_cast<char *>(ws);
  hipStream_t side = may_split && split_in_two(p, stream) ? side_stream() : nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  if (side != nullptr &&
      (hipEventCreateWithFlags(&fork, hipEventDisableTiming) != hipSuccess ||
       hipEventCreateWithFlags(&join, hipEventDisableTiming) != hipSuccess ||
       hipEventRecord(fork, stream) != hipSuccess ||
       hipStreamWaitEvent(side, fork, 0) != hipSuccess)) {
    // no second stream after all: one launch over all streams on the caller's stream (a
    // recorded fork event that the side stream waits for orders nothing of this call)
    if (fork != nullptr) (void)hipEventDestroy(fork);
    if (join != nullptr) (void)hipEventDestroy(join);
    (void)hipGetLastError();
    side = nullptr;
  }
  if (side == nullptr) return launch_chunk_group(p, pl, 0, p.streams, q, k, v, u, out, st, w, stream);
  const int64_t h = p.streams / 2;
  hipError_t e0 = launch_chunk_group(p, pl, 0, h, q, k, v, u, out, st, w, stream);
  hipError_t e1 = launch_chunk_group(p, pl, h, p.streams - h, q, k, v, u, out, st, w, side);
  // the caller's stream waits for the side stream's group whatever happened above, so that
  // nothing of this call is still running on it once the caller's stream has passed
  hipError_t e2 = hipEventRecord(join, side);
  if (e2 == hipSuccess) e2 = hipStreamWaitEvent(stream, join, 0);
  (void)hipEventDestroy(fork);
  (void)hipEventDestroy(join);
  if (e0 != hipSuccess) return e0;
  if (e1 != hipSuccess) return e1;
  return e2;
}

void chunk_segments(const Problem &p, int chunk, int64_t *L, int64_t *P) {
  const ChunkPlan pl = make_plan(p, chunk);
  *L = pl.L;
  *P = pl.P;
}

hipError_t launch_chunk_states(const Problem &p, int chunk, const void *q, const void *k,
                               const void *v, const void *u, void *ws, double *Md,
                               hipStream_t stream, ChunkStates *cs) {
  if (!chunk_supported(p, chunk)) return hipErrorInvalidValue;
  const ChunkPlan pl = make_plan(p, chunk, true);
  char *w = static_cast<char *>(ws);
  cs->S_seg = reinterpret_cast<float *>(w + pl.off_s0);
  cs->A_seg = reinterpret_cast<float *>(w + pl.off_m);
  cs->n_seg = reinterpret_cast<float *>(w + pl.off_nk);
  cs->pib = reinterpret_cast<float *>(w + pl.off_pib);
  cs->L = pl.L;
  cs->P = pl.P;
  const StateIO none{};
  if (p.dtype == Dtype::F32) return launch_chunk_dt<float>(p, pl, q, k, v, u, nullptr, none, w, stream, true, Md);
  return launch_chunk_dt<bf16_t>(p, pl, q, k, v, u, nullptr, none, w, stream, true, Md);
}

hipError_t launch_chunk_records(const Problem &p, int chunk, const void *q, const void *k,
                                const void *v, const void *u, void *ws, double *Md,
                                hipStream_t stream, const BwRecords &rec, ChunkStates *cs) {
  if (!chunk_supported(p, chunk)) return hipErrorInvalidValue;
  const ChunkPlan pl = make_plan(p, chunk, true);
  char *w = static_cast<char *>(ws);
  cs->S_seg = reinterpret_cast<float *>(w + pl.off_s0);
  cs->A_seg = reinterpret_cast<float *>(w + pl.off_m);
  cs->n_seg = reinterpret_cast<float *>(w + pl.off_nk);
  cs->pib = reinterpret_cast<float *>(w + pl.off_pib);
  cs->L = pl.L;
  cs->P = pl.P;
  const StateIO none{};
  if (p.dtype == Dtype::F32) return launch_chunk_dt<float>(p, pl, q, k, v, u, nullptr, none, w, stream, false, Md, &rec);
  return launch_chunk_dt<bf16_t>(p, pl, q, k, v, u, nullptr, none, w, stream, false, Md, &rec);
}

hipError_t launch_matrix_prefix(const Problem &p, float *M, int64_t P, const float *Minit,
                                hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.streams), static_cast<unsigned>((p.d * p.d + 255) / 256));
#define VLA_CASE(DD)                                                                          \
  if (p.d == DD) {                                                                            \
    VLA_LAUNCH("k_prefix", (k_prefix<DD>), grid, dim3(256), 0, st, M, static_cast<float *>(nullptr), \
               P, 0.0f, Minit, static_cast<const float *>(nullptr), 0, static_cast<double *>(nullptr)); \
    return hipGetLastError();                                                                 \
  }
  VLA_CASE(32) VLA_CASE(64) VLA_CASE(96) VLA_CASE(128)
#undef VLA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_affine_prefix(const Problem &p, const float *pib, float *s0, int64_t P,
                                const float *S0, float *nk, const float *n0, hipStream_t st) {
  const unsigned S = static_cast<unsigned>(p.streams);
#define VLA_CASE(DD)                                                                          \
  if (p.d == DD) {                                                                            \
    VLA_LAUNCH("k_sprefix", (k_sprefix<DD>), dim3(S, DD / 16), dim3(DD / 16 * kWave), 0, st,  \
               pib, s0, P, S0, nk, n0, static_cast<float *>(nullptr), static_cast<float *>(nullptr)); \
    return hipGetLastError();                                                                 \
  }
  VLA_CASE(32) VLA_CASE(64) VLA_CASE(96) VLA_CASE(128)
#undef VLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace vla
