// S side of the chunked path on the bf16 matrix cores (bf16 inputs).
//
// The residual update S <- S + (v - S khat) ahat^T (VLA summary §2.3 steps 3-4) and the
// ratio readout (§2.4) over a chunk of CH tokens, in UT/WY form.  The chunk's triangular
// system (I + Ka) E = R, Ka the strict lower part of Khat Ahat^T, is solved left-looking in
// steps of two 16-token tiles (a, b): with X^T the state slice before the step,
//   R_t = V_t - Khat_t X^T                       (t = a, b)
//   E_a = (I + Ka_aa)^{-1} R_a
//   E_b = (I + Ka_bb)^{-1} (R_b - Ka_ba E_a)
//   Num_t = Phi(q)_t X^T + sum_{t' <= t} Qa_tt' E_t',  o = Num / den   (final pass only)
//   X^T += Ahat_a^T E_a + Ahat_b^T E_b
// (Qa the lower part of Phi(q) Ahat^T); blocks further below the diagonal act through the
// updated state.  The workgroup's waves share only the tiles Ka_aa, Ka_ba, Ka_bb (with the
// inverses of I + Ka_tt) and the matching Qa tiles.  Every product runs on
// v_mfma_f32_16x16x32_bf16.  Raw k and v are exact bf16; khat = rk * k is applied after the
// product.  ahat, phi(q), the state, Ka, Qa and E are fp32 values split into two bf16 terms
// (hi + lo, about 16 significant bits) multiplied term pair by term pair with fp32
// accumulation, which keeps each product's relative error near 2^-16.  ahat arrives already
// split (the A side writes each token's row as [hi d | lo d]) and is staged by token as it is.
#pragma once

#include "vla_common.h"
#include "vla_mfma.h"

namespace vla {

template <int D, int CH, bool FINAL>
struct SwbCfg {
  static constexpr int NWV = D / 16;          // 16-row state slices
  // The final pass runs one wave per slice; the segment-map pass runs the Pi rows (waves
  // 0..NWV-1) and the B rows (waves NWV..2 NWV-1) of one segment in the same workgroup,
  // which share the staged chunk, the Ka tiles and the block inverses.
  static constexpr int NWT = FINAL ? NWV : 2 * NWV;
  static constexpr int NT = NWT * kWave;
  static constexpr int NCT = CH / 16;         // 16-token tiles per chunk
  static constexpr int NPR = (NCT + 1) / 2;   // steps of two tiles
  static constexpr int NOD = NCT / 2;         // steps with both tiles (one off-diagonal tile)
  static constexpr int NFT = D / 16;          // 16-feature tiles
  static constexpr int NKS = D / 32;          // 32-feature slices
  static constexpr int NKT = NCT * (NCT + 1) / 2;
  static constexpr int LDF = D + 8;           // bf16 row stride of token rows
  static constexpr int LDI = 24;              // bf16 row stride of the 16 x 16 inverses
  static_assert(D % 32 == 0, "feature dimension must be a multiple of 32");
};

template <int D, int CH, bool FINAL>
struct SwbLds {
  using C = SwbCfg<D, CH, FINAL>;
  static constexpr int QR = FINAL ? CH : 1;
  uint16_t sK[CH][C::LDF];                    // raw k, by token
  uint16_t sV[CH][C::LDF];                    // raw v, by token
  uint16_t sAt[2][CH][C::LDF];                // ahat terms, by token (read transposed for the state update)
  uint16_t sFq[2][QR][C::LDF];                // phi(q) terms, by token (final pass)
  // 16 x 16 tiles as two bf16 terms, stored transposed ([col][row]): a lane writes its column
  // with wide stores, and the A operands are read back with the transposing load.
  uint16_t InvS[2][C::NCT][16][C::LDI];       // (I + Ka_b)^{-1}
  uint16_t QaD[2][FINAL ? C::NCT : 1][16][C::LDI];  // Qa_tt (final pass)
  uint16_t KaO[2][C::NOD > 0 ? C::NOD : 1][16][C::LDI];  // -Ka_ba of each step
  uint16_t QaO[2][FINAL && C::NOD > 0 ? C::NOD : 1][16][C::LDI];  // Qa_ba (final pass)
  alignas(16) float np[FINAL ? D : 4];        // normaliser at the segment start
  float rk[CH];                               // 1 / ||k||
  float rden[CH];                             // readout denominator (its reciprocal once complete)
  float dpart[FINAL ? CH : 1][FINAL ? D / 32 : 1];  // phi(q) . n_p over 32 features of a token
};

// Tiles shared by the two S passes.  The inverses (I + Ka_tt)^{-1} of the 16-token diagonal
// tiles and the off-diagonal tiles -Ka_ba of each 32-token block depend only on that block's
// tokens (k, ahat, 1/||k||), not on the chunking, so the map pass (chunks of 32 or 64) writes
// them and the final pass (chunks of 32) loads them for every segment the map pass covered
// instead of forming them again.  Per stream and 32-token block (blocks counted from the
// stream's first token): [3 tiles: inverse of tile 0, of tile 1, -Ka_10][2 bf16 terms]
// [16 columns][16 rows], each tile as the passes keep it in LDS (transposed), 3 KB a block.
constexpr int kSwbTileBlock = 3 * 2 * 16 * 16;  // uint16 per 32-token block
__host__ __device__ inline int64_t swb_tile_blocks(int64_t T) { return (T + 31) / 32; }
inline bool swb_shares_tiles(bool fp32_inputs, int64_t P, int chunk) {
  return !fp32_inputs && P > 1 && chunk >= 32;
}

// The final pass at d <= 96 is held to 128 VGPRs (four waves per SIMD), so that two of its
// workgroups share a CU.  A workgroup's waves are placed from the first SIMD on, so two
// six-wave workgroups (d = 96) put four waves on two SIMDs and two on the others.  NSEG = 2
// runs the same segment of two streams (2 s' and 2 s' + 1 for blockIdx.x = s') in one
// workgroup of twice the waves, each half with its own LDS: at d = 96 twelve waves, three on
// every SIMD.  Every stream has the same T, so the two halves run the same chunks and meet at
// every barrier.  On 32 x 131072 tokens at d = 96, in one launch, 1.85 -> 1.64 ms.
template <int D, bool FINAL, int NSEG = 1>
constexpr int swb_waves_per_simd() { return NSEG == 2 ? 3 : (FINAL && D <= 96) ? 4 : 1; }

// With REC (final pass only) the kernel writes its part of the backward's token records (r and
// o in fp32, 1/||k||, den) and the S half of the state checkpoints (brec, bck: BwRec layout) in
// place of the outputs.
template <int D, int CH, bool FINAL, bool REC = false, int NSEG = 1>
__global__ void __launch_bounds__((NSEG * SwbCfg<D, CH, FINAL>::NT))
__attribute__((amdgpu_waves_per_eu(swb_waves_per_simd<D, FINAL, NSEG>())))
k_swyb(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k, const bf16_t *__restrict__ v,
       const uint16_t *__restrict__ ahat, const float *__restrict__ rkden,
       const float *__restrict__ s0, float *__restrict__ pib, bf16_t *__restrict__ out,
       float *__restrict__ S_final, const float *__restrict__ nstart, int64_t T, int64_t L,
       int64_t P, float *__restrict__ brec, float *__restrict__ bck, uint16_t *__restrict__ tiles,
       int64_t npre) {
  static_assert(FINAL || !REC, "records come from the final pass");
  using C = SwbCfg<D, CH, FINAL>;
  constexpr int NT = C::NT, NCT = C::NCT, NFT = C::NFT, NKS = C::NKS;
  constexpr int TQ = SwbLds<D, CH, FINAL>::QR * C::LDF;
  constexpr int TA = CH * C::LDF;
  constexpr int TQD = (FINAL ? NCT : 1) * 16 * C::LDI;
  constexpr int NOD = C::NOD, NPR = C::NPR;
  constexpr int TKO = (NOD > 0 ? NOD : 1) * 16 * C::LDI;
  constexpr int TQO = (FINAL && NOD > 0 ? NOD : 1) * 16 * C::LDI;
  constexpr int TI = NCT * 16 * C::LDI;
  static_assert(NSEG == 1 || NSEG == 2, "one or two streams per workgroup");
  __shared__ __attribute__((aligned(16))) SwbLds<D, CH, FINAL> shs[NSEG];
  // the workgroup's half (its stream), uniform over each wave
  const int half = NSEG == 1 ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / NT);
  SwbLds<D, CH, FINAL> &sh = shs[half];

  const int64_t s = static_cast<int64_t>(blockIdx.x) * NSEG + half, p = blockIdx.y;
  const int tid = static_cast<int>(threadIdx.x) - NT * half, lane = tid & 63, li = lane & 15, gq = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tb = p * L, te = std::min<int64_t>(T, tb + L);
  const uint16_t *ks = reinterpret_cast<const uint16_t *>(k) + s * T * D;
  const uint16_t *vs = reinterpret_cast<const uint16_t *>(v) + s * T * D;
  const uint16_t *qs = reinterpret_cast<const uint16_t *>(q) + s * T * D;
  const uint16_t *als = ahat + s * T * 2 * D;
  const float *rds = rkden + s * T * 2;
  constexpr int RF = BwRec<D>::F;
  float *brs = REC ? brec + s * T * RF : nullptr;
  float *bcs = REC ? bck + s * ((T + kBwCk - 1) / kBwCk) * 2 * D * D : nullptr;  // S halves

  // the shared tiles: written by the map pass (chunks of 32 or 64 tokens), read by the final
  // pass (chunks of 32) for the segments p < npre that the map pass covered
  static_assert(CH % 32 == 0 || CH == 16, "chunks of 16, 32 or 64 tokens");
  // (not with the backward's records: that final pass forms its own tiles)
  constexpr bool TSH = CH >= 32 && (!FINAL || CH == 32) && !REC;
  uint16_t *tls = (TSH && tiles != nullptr) ? tiles + s * swb_tile_blocks(T) * kSwbTileBlock : nullptr;
  const bool pre = FINAL && tls != nullptr && p < npre;

  const bool pi_rows = !FINAL && wave < C::NWV;
  const int rowbase = 16 * (wave % C::NWV);
  const bool has_v = FINAL || !pi_rows;

  // X[ft][r] = S[rowbase + li][16 ft + 4 gq + r]: a 16-row slice of S, transposed.
  f4_t X[NFT];
  if constexpr (FINAL) {
    const float *st = s0 + (s * P + p) * D * D;
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
      const float4 x = *reinterpret_cast<const float4 *>(&st[(rowbase + li) * D + 16 * ft + 4 * gq]);
      X[ft] = f4_t{x.x, x.y, x.z, x.w};
    }
  } else {
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        X[ft][r] = (pi_rows && rowbase + li == 16 * ft + 4 * gq + r) ? 1.f : 0.f;
  }

  // Register prefetch of a chunk: 16-byte row pieces of k, q, v (features fastest) and
  // float4 of ahat for two consecutive tokens (token pairs fastest, so the by-feature LDS
  // writes are contiguous 32-bit words).  Loads
  // past the segment read row 0 instead and are zeroed when staged, so no load result is
  // selected on (which would make the load wait at once).
  constexpr int RV = D / 8;                   // uint4 per token row
  constexpr int UK = CH * RV;
  constexpr int RA = 2 * D / 8;               // uint4 per token row of ahat terms
  constexpr int UA = CH * RA;
  constexpr int PK = (UK + NT - 1) / NT;
  constexpr int PA = (UA + NT - 1) / NT;
  uint4 pk[PK], pq[FINAL ? PK : 1], pv[PK];
  uint4 pa[PA];
  // final pass: units tid, tid + NT, ... (16 bytes each) of the chunk's shared tiles
  constexpr int UT = kSwbTileBlock / 8, PT = (UT + NT - 1) / NT;
  uint4 ptl[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) ptl[i] = make_uint4(0u, 0u, 0u, 0u);
  float prk = 0.f, pden = 1.f;
  // Per-lane offsets are 32-bit (one stream's rows span far less than 4 GiB) from a
  // workgroup-uniform base, so each load needs one offset register.
  auto prefetch = [&](int64_t cs, int tid) {
    const int mm = static_cast<int>(std::min<int64_t>(CH, te - cs));
    const uint16_t *kc = ks + cs * D, *qc = qs + cs * D, *vc = vs + cs * D;
    const uint16_t *ac = als + cs * 2 * D;
    const float *rc = rds + cs * 2;
#pragma unroll
    for (int i = 0; i < PK; ++i) {
      const int ui = tid + i * NT;
      const int c = ui / RV, f0 = (ui % RV) * 8;
      const uint32_t off = (ui < UK && c < mm) ? static_cast<uint32_t>(c * D + f0) : 0u;
      pk[i] = *reinterpret_cast<const uint4 *>(kc + off);
      if constexpr (FINAL) pq[i] = *reinterpret_cast<const uint4 *>(qc + off);
      pv[i] = *reinterpret_cast<const uint4 *>(vc + off);
    }
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int ui = tid + i * NT;
      const int c = ui / RA, j0 = (ui % RA) * 8;
      const uint32_t off = (ui < UA && c < mm) ? static_cast<uint32_t>(c * 2 * D + j0) : 0u;
      pa[i] = *reinterpret_cast<const uint4 *>(ac + off);
    }
    const uint32_t toff = (tid < mm) ? static_cast<uint32_t>(tid * 2) : 0u;
    prk = rc[toff];
    if constexpr (FINAL) pden = rc[toff + 1];
    if constexpr (FINAL && TSH)  // units of the 32-token block at cs: 8 of its uint16 each
      if (pre)
#pragma unroll
        for (int i = 0; i < PT; ++i)
          if (tid + i * NT < UT)
            ptl[i] = *reinterpret_cast<const uint4 *>(tls + (cs / 32) * kSwbTileBlock + 8 * (tid + i * NT));
  };
  prefetch(tb, tid);
  if constexpr (FINAL)  // phi(q) . n_p completes the A side's denominators (see below)
    for (int f = tid; f < D; f += NT) sh.np[f] = nstart[(s * P + p) * D + f];

  for (int64_t c0 = tb; c0 < te; c0 += CH) {
    const int m = static_cast<int>(std::min<int64_t>(CH, te - c0));
    // Opaque per-chunk copies of the lane indices: the addresses derived from them are
    // recomputed each chunk rather than hoisted out of the loop and kept (or spilled).
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o - NT * half, lane = tid & 63, li = lane & 15, gq = lane >> 4;
    __syncthreads();
    // ---- stage the chunk ------------------------------------------------------------------
#pragma unroll
    for (int i = 0; i < PK; ++i) {
      const int ui = tid + i * NT;
      if (ui < UK) {
        const int c = ui / RV, f0 = (ui % RV) * 8;
        const bool okv = c < m;
        *reinterpret_cast<uint4 *>(&sh.sK[c][f0]) = keep_if(c < m, pk[i]);
        *reinterpret_cast<uint4 *>(&sh.sV[c][f0]) = keep_if(okv, pv[i]);
        if constexpr (FINAL) {
          float qf[8];
          io<bf16_t>::unpack(pq[i], qf);
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[e] = c < m ? phi(qf[e]) : 0.f;
          // The A side's denominators count the normaliser from the segment start only;
          // den = phi(q) . n_p + (A side's value), n_p the normaliser at the segment start:
          // this thread's 8 features of the dot product, in fp32 (summed in the tile phase).
          const float4 n0 = *reinterpret_cast<const float4 *>(&sh.np[f0]);
          const float4 n1 = *reinterpret_cast<const float4 *>(&sh.np[f0 + 4]);
          float part = ((qf[0] * n0.x + qf[1] * n0.y) + (qf[2] * n0.z + qf[3] * n0.w)) +
                       ((qf[4] * n1.x + qf[5] * n1.y) + (qf[6] * n1.z + qf[7] * n1.w));
          // lanes ui ^ 1, ui ^ 2 stage the neighbouring 8-feature pieces of the same token
          // (d / 8 is a multiple of 4, and so is every unit count here): one sum per 32 features
          part = part + dpp_xor1(part);
          part = part + dpp_xor2(part);
          if ((ui & 3) == 0) sh.dpart[c][f0 / 32] = part;
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            uint32_t t2[2];
            split_pk<2>(qf[e], qf[e + 1], t2);
            hw[e / 2] = t2[0];
            lw[e / 2] = t2[1];
          }
          *reinterpret_cast<uint4 *>(&sh.sFq[0][c][f0]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
          *reinterpret_cast<uint4 *>(&sh.sFq[1][c][f0]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int ui = tid + i * NT;
      if (ui < UA) {
        const int c = ui / RA, j0 = (ui % RA) * 8;
        const int term = j0 / D, f0 = j0 % D;
        *reinterpret_cast<uint4 *>(&sh.sAt[term][c][f0]) = keep_if(c < m, pa[i]);
      }
    }
    if (tid < CH) {
      sh.rk[tid] = tid < m ? prk : 0.f;
      if constexpr (FINAL) sh.rden[tid] = tid < m ? pden : 1.f;  // completed in the tile phase
    }
    if constexpr (FINAL && TSH) {  // the block's tiles into the slots the Ka jobs would fill
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int u = tid + i * NT;
        if (pre && u < UT) {
          const int tile = u >> 6, term = (u >> 5) & 1, row = (u >> 1) & 15, h8 = u & 1;
          uint16_t *dst = tile < 2 ? &sh.InvS[term][tile][row][8 * h8] : &sh.KaO[term][0][row][8 * h8];
          *reinterpret_cast<uint4 *>(dst) = ptl[i];
        }
        asm volatile("" ::"v"(ptl[i].x));
      }
    }
    // Every prefetched register counts as used here, in every thread (lanes that stage nothing
    // included), so no load is still pending when the next prefetch reuses the registers: the
    // compiler then need not wait for the stores issued since.
    asm volatile("" ::"v"(prk), "v"(pden));
#pragma unroll
    for (int i = 0; i < PK; ++i) {
      asm volatile("" ::"v"(pk[i].x), "v"(pv[i].x));
      if constexpr (FINAL) asm volatile("" ::"v"(pq[i].x));
    }
#pragma unroll
    for (int i = 0; i < PA; ++i) asm volatile("" ::"v"(pa[i].x));
    __syncthreads();
    // ---- shared tile products: Ka_tt (each with the inverse of I + Ka_tt), Ka_ba and, in
    //      the final pass, Qa_tt and Qa_ba --------------------------------------------------
    //      jobs: [0, NCT) Ka_tt, [NCT, NCT + NOD) Ka_ba, then Qa_tt, Qa_ba
    constexpr int NKJ = NCT + NOD;
    constexpr int NJOB = (FINAL ? 2 : 1) * NKJ;
    // with the shared tiles staged, the final pass runs the Qa jobs only
    for (int job = (pre ? NKJ : 0) + wave; job < NJOB; job += C::NWT) {
      const bool isq = job >= NKJ;
      const int jk = isq ? job - NKJ : job;
      const bool diag = jk < NCT;
      const int ct = diag ? jk : 2 * (jk - NCT) + 1;   // row tile
      const int ct2 = diag ? jk : 2 * (jk - NCT);      // column tile
      // Operands first, then one independent MFMA chain per feature slice.
      f4_t acc;
      {
        Split2 b[NKS];
#pragma unroll
        for (int ksl = 0; ksl < NKS; ++ksl) {
          const int fa = 32 * ksl + 4 * gq;
          // Ahat[16 ct2 + li][fa + e], [fa + 16 + e]
          b[ksl] = ld2_4x2(&sh.sAt[0][16 * ct2 + li][fa], &sh.sAt[0][16 * ct2 + li][fa + 16], TA);
        }
        f4_t part[NKS];
        if (isq) {
          if constexpr (FINAL) {
            Split2 a[NKS];
#pragma unroll
            for (int ksl = 0; ksl < NKS; ++ksl) {
              const int fa = 32 * ksl + 4 * gq;
              a[ksl] = ld2_4x2(&sh.sFq[0][16 * ct + li][fa], &sh.sFq[0][16 * ct + li][fa + 16], TQ);
            }
#pragma unroll
            for (int ksl = 0; ksl < NKS; ++ksl) part[ksl] = mm2_ss(a[ksl], b[ksl], f4_zero());
          }
        } else {
          bf16x8_t a[NKS];
#pragma unroll
          for (int ksl = 0; ksl < NKS; ++ksl) {
            const int fa = 32 * ksl + 4 * gq;
            a[ksl] = ld_bf4x2(&sh.sK[16 * ct + li][fa], &sh.sK[16 * ct + li][fa + 16]);
          }
#pragma unroll
          for (int ksl = 0; ksl < NKS; ++ksl) part[ksl] = mm2_xs(a[ksl], b[ksl], f4_zero());
        }
        acc = part[0];
#pragma unroll
        for (int ksl = 1; ksl < NKS; ++ksl) acc += part[ksl];
      }
      // acc[r] = product[i = 4 gq + r][i'' = li] of tile (ct, ct2): this lane's column li,
      // rows 4 gq .. 4 gq + 3, stored transposed as one 8-byte piece per term.
      {
        const int i = 4 * gq;
        if (isq) {
          if constexpr (FINAL) {
            f4_t v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = diag && li > i + r ? 0.f : acc[r];
            const Split2h t = split2_4h(v);
            uint16_t *dst = diag ? &sh.QaD[0][ct][li][i] : &sh.QaO[0][jk - NCT][li][i];
            const int ts = diag ? TQD : TQO;
            *reinterpret_cast<uint2 *>(dst) = t.h;
            *reinterpret_cast<uint2 *>(dst + ts) = t.l;
          }
        } else {
          if (diag) {
            // (I + Ka_b)^{-1} by forward substitution, column j = li in every lane group (lanes
            // 0..15 keep theirs).  M = -Ka_b with rows scaled by 1/||k|| is first stored by
            // column in fp32 over this tile's InvS slots (the inverse overwrites them at the
            // end): columns 0..11 in the term-0 slot, 12..15 in the term-1 slot, 16 floats
            // each.  Pivot q then reads column q with broadcast loads (every lane the same
            // address), one column ahead of its use.
            float *mc0 = reinterpret_cast<float *>(&sh.InvS[0][ct][0][0]);
            float *mc1 = reinterpret_cast<float *>(&sh.InvS[1][ct][0][0]);
            {
              f4_t nv;
#pragma unroll
              for (int e = 0; e < 4; ++e) nv[e] = -acc[e] * sh.rk[16 * ct + i + e];
              float *dstc = (li < 12 ? mc0 + 16 * li : mc1 + 16 * (li - 12)) + i;
              *reinterpret_cast<f4_t *>(dstc) = nv;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            auto col = [&](int q, f4_t (&c)[4]) {
              const float *src = q < 12 ? mc0 + 16 * q : mc1 + 16 * (q - 12);
#pragma unroll
              for (int g = 0; g < 4; ++g)
                if (4 * g + 3 > q) c[g] = *reinterpret_cast<const f4_t *>(src + 4 * g);
            };
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == li) ? 1.f : 0.f;
            f4_t cc[2][4];
            col(0, cc[0]);
#pragma unroll
            for (int q = 0; q < 15; ++q) {
              if (q + 1 < 15) col(q + 1, cc[(q + 1) & 1]);
              __builtin_amdgcn_sched_barrier(0);  // one column of loads in flight at a time
#pragma unroll
              for (int r = q + 1; r < 16; ++r) x[r] = fmaf(cc[q & 1][r >> 2][r & 3], x[q], x[r]);
              // x[q + 1] is final: formed here in every lane, not sunk into the store branch
              asm volatile("" : "+v"(x[q + 1]));
              __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lane < 16) {
              // column j of the inverse, transposed: row j of InvS, 16 values per term
              uint32_t w[8][2];
#pragma unroll
              for (int r = 0; r < 16; r += 2) split_pk<2>(x[r], x[r + 1], w[r / 2]);
#pragma unroll
              for (int term = 0; term < 2; ++term) {
                uint4 *dst = reinterpret_cast<uint4 *>(&sh.InvS[term][ct][lane][0]);
                dst[0] = make_uint4(w[0][term], w[1][term], w[2][term], w[3][term]);
                dst[1] = make_uint4(w[4][term], w[5][term], w[6][term], w[7][term]);
              }
            }
          } else {
            f4_t nk;
#pragma unroll
            for (int r = 0; r < 4; ++r) nk[r] = -acc[r] * sh.rk[16 * ct + i + r];
            const Split2h t = split2_4h(nk);
            *reinterpret_cast<uint2 *>(&sh.KaO[0][jk - NCT][li][i]) = t.h;
            *reinterpret_cast<uint2 *>(&sh.KaO[1][jk - NCT][li][i]) = t.l;
          }
        }
      }
    }
    if constexpr (FINAL) {
      // Complete the denominators (the staging threads' partial dot products phi(q) . n_p,
      // summed in a fixed order) and keep their reciprocals, on the last wave (a light tile job).
      if (wave == C::NWT - 1 && lane < CH) {
        float dn = 0.f;
#pragma unroll
        for (int g = 0; g < D / 32; ++g) dn += sh.dpart[lane][g];
        const float den = sh.rden[lane] + dn;
        sh.rden[lane] = 1.0f / den;
        if constexpr (REC)
          if (lane < m) {
            brs[(c0 + lane) * RF + BwRec<D>::SC + 2] = sh.rk[lane];
            brs[(c0 + lane) * RF + BwRec<D>::SC + 3] = den;
          }
      }
    }
    __syncthreads();
    if constexpr (!FINAL && TSH) {  // the map pass hands its tiles to the final pass
      if (tls != nullptr) {
        constexpr int NBK = CH / 32, UNITS = kSwbTileBlock / 8;  // 32-token blocks, uint4 each
        for (int u = tid; u < NBK * UNITS; u += NT) {
          const int bb = u / UNITS, r = u % UNITS;
          const int tile = r >> 6, term = (r >> 5) & 1, row = (r >> 1) & 15, h8 = r & 1;
          if (c0 + 32 * bb < te) {
            const uint16_t *src = tile < 2 ? &sh.InvS[term][2 * bb + tile][row][8 * h8]
                                           : &sh.KaO[term][bb][row][8 * h8];
            *reinterpret_cast<uint4 *>(tls + (c0 / 32 + bb) * kSwbTileBlock + 8 * r) =
                *reinterpret_cast<const uint4 *>(src);
          }
        }
      }
    }
    // ---- this wave's rows: two tiles per step ---------------------------------------------
    // The next chunk's loads fly during the steps.
    if (c0 + CH < te) prefetch(c0 + CH, tid);
    uint16_t *os = REC ? nullptr : reinterpret_cast<uint16_t *>(out) + (s * T + c0) * D;
#pragma unroll
    for (int pr = 0; pr < NPR; ++pr) {
      const int ta = 2 * pr, tbb = 2 * pr + 1;
      const bool two = tbb < NCT;
      // Operands of the step's products over features, loaded up front so that one LDS
      // latency covers them all: K_t (and Phi(q)_t in the final pass) for both tiles.
      bf16x8_t aK[2][NKS];
      Split2 aQ[FINAL ? 2 : 1][NKS];
      float vv[2][4], rkv[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ct = 2 * pr + h;
        if (ct >= NCT) continue;
#pragma unroll
        for (int ksl = 0; ksl < NKS; ++ksl) {
          const int fa = 32 * ksl + 4 * gq;
          aK[h][ksl] = ld_bf4x2(&sh.sK[16 * ct + li][fa], &sh.sK[16 * ct + li][fa + 16]);
          if constexpr (FINAL)
            aQ[h][ksl] = ld2_4x2(&sh.sFq[0][16 * ct + li][fa], &sh.sFq[0][16 * ct + li][fa + 16], TQ);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 16 * ct + 4 * gq + r;
          vv[h][r] = has_v ? bf_val(sh.sV[c][rowbase + li]) : 0.f;
          rkv[h][r] = sh.rk[c];
        }
      }
      // The state slice before this step as the B operand of products over features.
      Split2 xs[NKS];
#pragma unroll
      for (int ksl = 0; ksl < NKS; ++ksl) {
        float t8[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) { t8[r] = X[2 * ksl][r]; t8[4 + r] = X[2 * ksl + 1][r]; }
        xs[ksl] = split2(t8);
      }
      // R_t = V_t - rk (K_t X^T) and, in the final pass, Phi(q)_t X^T (independent of the
      // solve): four accumulation chains.
      f4_t R[2], numq[2] = {f4_zero(), f4_zero()};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ct = 2 * pr + h;
        if (ct >= NCT) continue;
        f4_t acc = f4_zero();
#pragma unroll
        for (int ksl = 0; ksl < NKS; ++ksl) {
          acc = mm2_xs(aK[h][ksl], xs[ksl], acc);
          if constexpr (FINAL) numq[h] = mm2_ss(aQ[h][ksl], xs[ksl], numq[h]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) R[h][r] = fmaf(-rkv[h][r], acc[r], vv[h][r]);
      }
      // Ahat^T operands of the state update, loaded while the solve runs.
      Split2 aT[NFT];
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        // Ahat[ca + e][16 ft + li] and Ahat[ca + 16 + e][16 ft + li]: the token rows, transposed
        const int ca = 16 * ta + 4 * gq;
        if (two) {
          aT[ft].h = ld_tr4x2(&sh.sAt[0][0][0], C::LDF, ca, ca + 16, 16 * ft, li);
          aT[ft].l = ld_tr4x2(&sh.sAt[1][0][0], C::LDF, ca, ca + 16, 16 * ft, li);
        } else {
          aT[ft].h = ld_tr4z(&sh.sAt[0][0][0], C::LDF, ca, 16 * ft, li);
          aT[ft].l = ld_tr4z(&sh.sAt[1][0][0], C::LDF, ca, 16 * ft, li);
        }
      }
      // E_a = (I + Ka_aa)^{-1} R_a;  E_b = (I + Ka_bb)^{-1} (R_b - Ka_ba E_a)
      f4_t E[2];
      E[0] = mm2h_ss(ld2_tr4h(&sh.InvS[0][ta][0][0], C::LDI, TI, gq, li), split2_4h(R[0]), f4_zero());
      const Split2h esa = split2_4h(E[0]);
      Split2h esb = esa;
      if (two) {
        const f4_t rb = mm2h_ss(ld2_tr4h(&sh.KaO[0][pr][0][0], C::LDI, TKO, gq, li), esa, R[1]);
        E[1] = mm2h_ss(ld2_tr4h(&sh.InvS[0][tbb][0][0], C::LDI, TI, gq, li), split2_4h(rb), f4_zero());
        esb = split2_4h(E[1]);
      }
      if constexpr (REC) {  // r_t = v_t - S_{t-1} khat_t: the rows of E
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ct = 2 * pr + h;
          if (ct >= NCT) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int c = 16 * ct + 4 * gq + r;
            if (c < m) brs[(c0 + c) * RF + BwRec<D>::R + rowbase + li] = E[h][r];
          }
        }
      }
      if constexpr (FINAL) {
        // Num_t = Phi(q)_t X^T + sum_{t' <= t} Qa_tt' E_t', then o = Num / den.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ct = 2 * pr + h;
          if (ct >= NCT) continue;
          f4_t num = mm2h_ss(ld2_tr4h(&sh.QaD[0][ct][0][0], C::LDI, TQD, gq, li), h ? esb : esa, numq[h]);
          if (h) num = mm2h_ss(ld2_tr4h(&sh.QaO[0][pr][0][0], C::LDI, TQO, gq, li), esa, num);
          if constexpr (REC) {  // o in fp32 (no output is written)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int c = 16 * ct + 4 * gq + r;
              if (c < m) brs[(c0 + c) * RF + BwRec<D>::O + rowbase + li] = num[r] * sh.rden[c];
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const int c = 16 * ct + 4 * gq + r;
              const uint32_t o2 = pk_bf16(num[r] * sh.rden[c], num[r + 1] * sh.rden[c + 1]);
              if (c < m) os[static_cast<uint32_t>(c * D + rowbase + li)] = static_cast<uint16_t>(o2);
              if (c + 1 < m) os[static_cast<uint32_t>((c + 1) * D + rowbase + li)] = static_cast<uint16_t>(o2 >> 16);
            }
          }
        }
      }
      // X^T += Ahat_a^T E_a + Ahat_b^T E_b  (one 32-token product)
      Split2 ep;
      ep.h = __builtin_bit_cast(bf16x8_t, make_uint4(esa.h.x, esa.h.y, two ? esb.h.x : 0u, two ? esb.h.y : 0u));
      ep.l = __builtin_bit_cast(bf16x8_t, make_uint4(esa.l.x, esa.l.y, two ? esb.l.x : 0u, two ? esb.l.y : 0u));
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) X[ft] = mm2_ss(aT[ft], ep, X[ft]);
    }
    if (REC && ((c0 + m) % kBwCk == 0 || c0 + m == te)) {  // S after a checkpoint token
      float *dst = bcs + ((c0 + m - 1) / kBwCk) * 2 * D * D;
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
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
    for (int ft = 0; ft < NFT; ++ft)
      *reinterpret_cast<float4 *>(&dst[(rowbase + li) * D + 16 * ft + 4 * gq]) =
          make_float4(X[ft][0], X[ft][1], X[ft][2], X[ft][3]);
  }
}

}  // namespace vla
