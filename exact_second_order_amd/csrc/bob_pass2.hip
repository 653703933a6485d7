// Pass 2 of the BoB schedule: recompute score tiles and accumulate all four
// gradients, with no N x N tensor outside on-chip memory.
//
// FlashBoB (arXiv 2609.24089), Abstract: once the two row scalars are known,
// every output is an affine map of recomputed tiles, so a second pass can
// rebuild S, P and the first-backward tiles block by block (FlashAttention-
// style score recomputation) and contract them straight into the outputs.
// Per (query i, key j), with row scalars LSE, D, c, r from pass 1:
//   P   = exp(s S - LSE)                  S = Q K^T
//   dS  = P (dP - D)                      dP = dO V^T
//   A   = P (G - c)                       G = s (gQ K^T + Q gK^T)
//   dS2 = dS (G - c) + P (H - r)          H = dO gV^T
//   gradK  += s (dS2^T Q + dS^T gQ)       gradV  += A^T dO
//   gradQ  += s (dS2 K + dS gK)           graddO += A V + P gV
//
// Schedule (gfx950): one workgroup (4 waves) owns a block of BC keys for the
// whole kernel and streams the query sequence in blocks of BR rows.
//   * K, gK, V, gV of the key block are staged once in LDS; each wave keeps
//     the operands it reuses every step in registers.
//   * Step 1 (recompute): each wave builds 32-key x 32-query blocks of
//     S^T, G^T, dP^T, H^T with MFMA (lane <-> query, so the four row scalars
//     are per-lane registers), forms P, dS, dS2, A in registers and stores
//     them to LDS as [query][key] tiles.
//   * Step 2 (key-side outputs): gradK and gradV of the key block live in
//     registers for the whole kernel; each step contracts the tiles over the
//     query block. The tiles and Q, gQ, dO are read transposed with gfx950
//     LDS transpose loads (ds_read_b64_tr_b16).
//   * Step 3 (query-side outputs): gradQ and graddO of the query block are
//     contracted over the key block and added to device memory with fp32
//     atomics (one add per element per key block; pass 1 zeroed them).
// Waves split step 3 by output (gradQ or graddO) and by halves of d, so no
// cross-wave reduction is needed anywhere.

#include "bob_device.h"

namespace flashbob {

template <typename T, int D_, int BC_, int BR_>
struct Pass2Cfg {
  static constexpr int D = D_, BC = BC_, BR = BR_;
  static constexpr int PAD = 16 / (int)sizeof(T);  // 16 bytes of row padding (LDS banks)
  static constexpr int LDK = D + PAD;              // [key][d] rows
  static constexpr int LDQ = D + PAD;              // [query][d] rows
  static constexpr int LDT = BC + PAD;             // [query][key] tile rows
  static constexpr int NKB = BC / 32, NQB = BR / 32, NDB = D / 32;
  static constexpr int NCH = D / 16;
  static constexpr int NREC = NKB * NQB;           // 32x32 recompute blocks per step
  static constexpr int REC_PER_WAVE = (NREC + 3) / 4;
  static constexpr int FQ_NDB = NDB * NKB / 4;     // d-blocks of gradK/gradV per wave
  static constexpr int FK_NDB = NDB / 2;           // d-blocks of gradQ or graddO per wave
  static constexpr bool RESIDENT_A = sizeof(T) == 2;  // keep recompute operands in VGPRs
  static_assert(4 % NKB == 0, "a wave must keep one key sub-block");
  static_assert((NDB * NKB) % 4 == 0, "key-side outputs must split over 4 waves");
  static_assert(NDB % 2 == 0, "query-side outputs split d in halves");
  static constexpr size_t LDS_BYTES =
      sizeof(T) * (size_t)(4 * BC * LDK + 3 * BR * LDQ + 4 * BR * LDT) + 4 * BR * sizeof(float);
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU");
};

template <typename Cfg, typename T>
__global__ __launch_bounds__(256, 1) void bob_pass2_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const T* __restrict__ gQ, const T* __restrict__ gK, const T* __restrict__ gV,
    const float* __restrict__ lse, const float* __restrict__ Dv, const float* __restrict__ cv,
    const float* __restrict__ rv, float* __restrict__ gradQ, float* __restrict__ gradK,
    float* __restrict__ gradV, float* __restrict__ graddO, int N, int nkblk, float scale) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int D = Cfg::D, BC = Cfg::BC, BR = Cfg::BR;
  constexpr int LDK = Cfg::LDK, LDQ = Cfg::LDQ, LDT = Cfg::LDT;
  constexpr int NKB = Cfg::NKB, NQB = Cfg::NQB, NCH = Cfg::NCH;
  constexpr int FQ_NDB = Cfg::FQ_NDB, FK_NDB = Cfg::FK_NDB;

  __shared__ __attribute__((aligned(16))) T sK[4][BC][LDK];  // K, gK, V, gV of the key block
  __shared__ __attribute__((aligned(16))) T sQ[3][BR][LDQ];  // Q, gQ, dO of the query block
  __shared__ __attribute__((aligned(16))) T sT[4][BR][LDT];  // P, dS, dS2, A as [query][key]
  __shared__ float sS[4][BR];                                // LSE*log2e, D, c, r

  const int head = blockIdx.x / nkblk;
  const int kblk = blockIdx.x % nkblk;
  const size_t hoff = (size_t)head * N * D;
  const size_t soff = (size_t)head * N;
  const int k0 = kblk * BC;
  const int nk = min(BC, N - k0);
  const int w = wave_id(), l = lane_id(), h = l >> 5, col = l & 31;

  copy_rows_to_lds<T, BC, D, 256>(&sK[0][0][0], LDK, K + hoff + (size_t)k0 * D, nk);
  copy_rows_to_lds<T, BC, D, 256>(&sK[1][0][0], LDK, gK + hoff + (size_t)k0 * D, nk);
  copy_rows_to_lds<T, BC, D, 256>(&sK[2][0][0], LDK, V + hoff + (size_t)k0 * D, nk);
  copy_rows_to_lds<T, BC, D, 256>(&sK[3][0][0], LDK, gV + hoff + (size_t)k0 * D, nk);
  __syncthreads();

  // this wave's 32-key sub-block (recompute and key-side outputs)
  const int rkb = w % NKB;
  // recompute A operands (lane <-> key, k over d)
  F aK[Cfg::RESIDENT_A ? NCH : 1], agK[Cfg::RESIDENT_A ? NCH : 1];
  F aV[Cfg::RESIDENT_A ? NCH : 1], agV[Cfg::RESIDENT_A ? NCH : 1];
  if constexpr (Cfg::RESIDENT_A) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      aK[c] = ld_rows(&sK[0][rkb * 32][16 * c], LDK);
      agK[c] = ld_rows(&sK[1][rkb * 32][16 * c], LDK);
      aV[c] = ld_rows(&sK[2][rkb * 32][16 * c], LDK);
      agV[c] = ld_rows(&sK[3][rkb * 32][16 * c], LDK);
    }
  }
  // query-side B operands (lane <-> d, k over keys): K, gK for gradQ waves,
  // V, gV for graddO waves
  const int fk_which = w >> 1;
  const int fk_db0 = (w & 1) * FK_NDB;
  F bX[FK_NDB][BC / 16], bY[FK_NDB][BC / 16];
#pragma unroll
  for (int j = 0; j < FK_NDB; ++j) {
#pragma unroll
    for (int c = 0; c < BC / 16; ++c) {
      const int dcol = (fk_db0 + j) * 32;
      bX[j][c] = ld_cols(&sK[fk_which ? 2 : 0][16 * c][dcol], LDK);
      bY[j][c] = ld_cols(&sK[fk_which ? 3 : 1][16 * c][dcol], LDK);
    }
  }
  // key-side accumulators
  const int fq_db0 = (w / NKB) * FQ_NDB;
  f32x16 accK[FQ_NDB], accV[FQ_NDB];
#pragma unroll
  for (int j = 0; j < FQ_NDB; ++j) {
    accK[j] = f32x16{};
    accV[j] = f32x16{};
  }

  const float sl2 = scale * kLog2e;
  const bool key_tail = nk < BC;
  float* const qout = fk_which ? graddO : gradQ;
  const float qscale = fk_which ? 1.f : scale;

  for (int q0 = 0; q0 < N; q0 += BR) {
    const int nq = min(BR, N - q0);
    __syncthreads();  // the previous step's readers of sQ, sT, sS are done
    copy_rows_to_lds<T, BR, D, 256>(&sQ[0][0][0], LDQ, Q + hoff + (size_t)q0 * D, nq);
    copy_rows_to_lds<T, BR, D, 256>(&sQ[1][0][0], LDQ, gQ + hoff + (size_t)q0 * D, nq);
    copy_rows_to_lds<T, BR, D, 256>(&sQ[2][0][0], LDQ, dO + hoff + (size_t)q0 * D, nq);
    if (threadIdx.x < BR) {
      const int i = threadIdx.x;
      const bool ok = i < nq;
      const size_t o = soff + q0 + i;
      // rows past the end get LSE = +inf, hence P = 0 and all-zero tiles
      sS[0][i] = ok ? lse[o] * kLog2e : INFINITY;
      sS[1][i] = ok ? Dv[o] : 0.f;
      sS[2][i] = ok ? cv[o] : 0.f;
      sS[3][i] = ok ? rv[o] : 0.f;
    }
    __syncthreads();

    // ---- step 1: recompute tiles of this wave's blocks, store P, dS, dS2, A
#pragma unroll
    for (int t = 0; t < Cfg::REC_PER_WAVE; ++t) {
      const int b = w + 4 * t;
      if (b < Cfg::NREC) {
        const int qb = b / NKB;
        f32x16 S = {}, G = {}, dP = {}, H = {};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const F bq = ld_rows(&sQ[0][qb * 32][16 * c], LDQ);
          const F bgq = ld_rows(&sQ[1][qb * 32][16 * c], LDQ);
          const F bdo = ld_rows(&sQ[2][qb * 32][16 * c], LDQ);
          F ak, agk, av, agv;
          if constexpr (Cfg::RESIDENT_A) {
            ak = aK[c];
            agk = agK[c];
            av = aV[c];
            agv = agV[c];
          } else {
            ak = ld_rows(&sK[0][rkb * 32][16 * c], LDK);
            agk = ld_rows(&sK[1][rkb * 32][16 * c], LDK);
            av = ld_rows(&sK[2][rkb * 32][16 * c], LDK);
            agv = ld_rows(&sK[3][rkb * 32][16 * c], LDK);
          }
          E::mma(S, ak, bq);
          E::mma(G, ak, bgq);
          E::mma(G, agk, bq);
          E::mma(dP, av, bdo);
          E::mma(H, agv, bdo);
        }
        const int qi = qb * 32 + col;  // this lane's query within the block
        const float l2 = sS[0][qi], Dq = sS[1][qi], cq = sS[2][qi], rq = sS[3][qi];
        T* tP = &sT[0][qi][rkb * 32 + 4 * h];
        T* tdS = &sT[1][qi][rkb * 32 + 4 * h];
        T* tdS2 = &sT[2][qi][rkb * 32 + 4 * h];
        T* tA = &sT[3][qi][rkb * 32 + 4 * h];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float p[4], ds[4], ds2[4], a[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * g + e;
            float pe = fast_exp2(fmaf(S[i], sl2, -l2));
            if (key_tail && rkb * 32 + acc_row(h, i) >= nk) pe = 0.f;
            const float dse = pe * (dP[i] - Dq);
            const float ge = fmaf(G[i], scale, -cq);
            p[e] = pe;
            ds[e] = dse;
            a[e] = pe * ge;
            ds2[e] = fmaf(dse, ge, pe * (H[i] - rq));
          }
          st4(tP + 8 * g, p[0], p[1], p[2], p[3]);
          st4(tdS + 8 * g, ds[0], ds[1], ds[2], ds[3]);
          st4(tdS2 + 8 * g, ds2[0], ds2[1], ds2[2], ds2[3]);
          st4(tA + 8 * g, a[0], a[1], a[2], a[3]);
        }
      }
    }
    __syncthreads();

    // ---- step 2: key-side outputs over this query block
#pragma unroll
    for (int c = 0; c < BR / 16; ++c) {
      const F tds2 = ld_cols(&sT[2][16 * c][rkb * 32], LDT);  // lane <-> key, k over queries
      const F tds = ld_cols(&sT[1][16 * c][rkb * 32], LDT);
      const F ta = ld_cols(&sT[3][16 * c][rkb * 32], LDT);
#pragma unroll
      for (int j = 0; j < FQ_NDB; ++j) {
        const int dcol = (fq_db0 + j) * 32;
        const F bq = ld_cols(&sQ[0][16 * c][dcol], LDQ);  // lane <-> d, k over queries
        const F bgq = ld_cols(&sQ[1][16 * c][dcol], LDQ);
        const F bdo = ld_cols(&sQ[2][16 * c][dcol], LDQ);
        E::mma(accK[j], tds2, bq);
        E::mma(accK[j], tds, bgq);
        E::mma(accV[j], ta, bdo);
      }
    }

    // ---- step 3: query-side outputs of this query block over the key block
    f32x16 accO[NQB][FK_NDB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int j = 0; j < FK_NDB; ++j) accO[qb][j] = f32x16{};
#pragma unroll
    for (int c = 0; c < BC / 16; ++c) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        // lane <-> query, k over keys: dS2 and dS (gradQ) or A and P (graddO)
        const F t1 = ld_rows(&sT[fk_which ? 3 : 2][qb * 32][16 * c], LDT);
        const F t2 = ld_rows(&sT[fk_which ? 0 : 1][qb * 32][16 * c], LDT);
#pragma unroll
        for (int j = 0; j < FK_NDB; ++j) {
          E::mma(accO[qb][j], t1, bX[j][c]);
          E::mma(accO[qb][j], t2, bY[j][c]);
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int j = 0; j < FK_NDB; ++j) {
        const int dcol = (fk_db0 + j) * 32 + col;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qrow = qb * 32 + acc_row(h, i);
          if (qrow < nq)
            unsafeAtomicAdd(qout + hoff + (size_t)(q0 + qrow) * D + dcol, qscale * accO[qb][j][i]);
        }
      }
    }
  }

  // key-side outputs of this key block
#pragma unroll
  for (int j = 0; j < FQ_NDB; ++j) {
    const int dcol = (fq_db0 + j) * 32 + col;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int krow = rkb * 32 + acc_row(h, i);
      if (krow < nk) {
        const size_t o = hoff + (size_t)(k0 + krow) * D + dcol;
        gradK[o] = scale * accK[j][i];
        gradV[o] = accV[j][i];
      }
    }
  }
}

template <typename T, int D, int BC, int BR>
static hipError_t launch_cfg(const void* Q, const void* K, const void* V, const void* dO, const void* gQ,
                             const void* gK, const void* gV, const float* stats, float* gradQ, float* gradK,
                             float* gradV, float* graddO, int BH, int N, float scale, hipStream_t stream) {
  using Cfg = Pass2Cfg<T, D, BC, BR>;
  const int nkblk = (N + BC - 1) / BC;
  const long long nblocks = (long long)nkblk * BH;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t BHN = (size_t)BH * N;
  bob_pass2_kernel<Cfg, T><<<dim3((unsigned)nblocks), dim3(256), 0, stream>>>(
      (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, (const T*)gQ, (const T*)gK, (const T*)gV, stats,
      stats + BHN, stats + 2 * BHN, stats + 3 * BHN, gradQ, gradK, gradV, graddO, N, nkblk, scale);
  return hipGetLastError();
}

// Tile shapes per (element type, d): the LDS budget (160 KB) sets BC x BR.
template <typename T, int D>
hipError_t launch_pass2(const void* Q, const void* K, const void* V, const void* dO, const void* gQ,
                        const void* gK, const void* gV, const float* stats, float* gradQ, float* gradK,
                        float* gradV, float* graddO, int BH, int N, float scale, hipStream_t stream) {
  if constexpr (sizeof(T) == 2 && D == 64)
    return launch_cfg<T, 64, 128, 32>(Q, K, V, dO, gQ, gK, gV, stats, gradQ, gradK, gradV, graddO, BH, N, scale,
                                      stream);
  else if constexpr (sizeof(T) == 2 && D == 128)
    return launch_cfg<T, 128, 64, 64>(Q, K, V, dO, gQ, gK, gV, stats, gradQ, gradK, gradV, graddO, BH, N, scale,
                                      stream);
  else if constexpr (D == 64)
    return launch_cfg<T, 64, 64, 32>(Q, K, V, dO, gQ, gK, gV, stats, gradQ, gradK, gradV, graddO, BH, N, scale,
                                     stream);
  else
    return launch_cfg<T, 128, 32, 32>(Q, K, V, dO, gQ, gK, gV, stats, gradQ, gradK, gradV, graddO, BH, N, scale,
                                      stream);
}

#define FLASHBOB_INST_PASS2(T, D)                                                                            \
  template hipError_t launch_pass2<T, D>(const void*, const void*, const void*, const void*, const void*,    \
                                         const void*, const void*, const float*, float*, float*, float*,     \
                                         float*, int, int, float, hipStream_t);
FLASHBOB_INST_PASS2(bf16, 64)
FLASHBOB_INST_PASS2(bf16, 128)
FLASHBOB_INST_PASS2(float, 64)
FLASHBOB_INST_PASS2(float, 128)

}  // namespace flashbob
