// Pass 1 of the BoB schedule: per-query row scalars (LSE, D, c, r).
//
// FlashBoB (arXiv 2609.24089), Abstract: two row-wise scalars fix every BoB
// output through affine maps; they are gathered in a first pass over the key
// sequence, ahead of the pass that accumulates the outputs. With
// G = s (gQ K^T + Q gK^T), H = dO gV^T and P = softmax(s Q K^T):
//   D = rowsum(P o dP)                (first-backward scalar, dP = dO V^T)
//   c = rowsum(P o G)
//   r = rowsum(dS o G) + rowsum(P o H),  dS = P o (dP - D)
// One sweep suffices: with Pt = exp(S - m) under a running max m (online
// softmax normaliser), accumulate l = sum Pt, aD = sum Pt dP, ac = sum Pt G,
// ae = sum Pt dP G, ah = sum Pt H, and finish with D = aD/l, c = ac/l,
// r = ae/l - D c + ah/l, LSE = m + ln l.
//
// Schedule (gfx950): a workgroup of 4 waves owns 128 queries, 32 per wave,
// and streams key blocks of 64 rows through LDS. Each wave computes the
// transposed tiles S^T, G^T, dP^T, H^T (keys x its 32 queries) with MFMA, so
// every lane holds one query column and 16 of the block's keys: all five
// sums stay in per-lane registers with no cross-lane traffic inside the loop;
// the two half-waves (which hold different keys) merge once at the end.

#include "bob_device.h"

namespace flashbob {

template <typename T, int D>
struct RowstatsCfg {
  static constexpr int BQ = 128;             // queries per workgroup (4 waves x 32)
  static constexpr int BK = 64;              // keys per LDS stage
  static constexpr int LDK = D + 16 / (int)sizeof(T);  // padded LDS row (elements)
  static constexpr int NCH = D / 16;         // 16-wide k chunks over d
};

// One fragment (16 k values of d) of a query row held by this lane; zero for
// rows past the sequence end.
__device__ __forceinline__ bf16x8 load_row_frag(const bf16* row, bool valid, int c) {
  bf16x8 f = {};
  if (valid) f = *reinterpret_cast<const bf16x8*>(row + 16 * c + 8 * (lane_id() >> 5));
  return f;
}

__device__ __forceinline__ f32x8 load_row_frag(const float* row, bool valid, int c) {
  f32x8 f = {};
  const int h = lane_id() >> 5;
  if (valid) {
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = row[16 * c + Elem<float>::kmap(h, s)];
  }
  return f;
}

// Running sums of one lane: one query, the keys of its half-wave. Level-1
// sums are scaled to the current running max m and absorb one 32-key block at
// a time (block sums first, so the sequential chain per block is 16 terms);
// every kFlush blocks they move into level-2 sums kept at their own max m2.
// At 262144 keys this keeps every fp32 chain at a few hundred additions
// instead of 131072.
struct OnlineSums {
  float m = -INFINITY, l = 0.f, aD = 0.f, ac = 0.f, ae = 0.f, ah = 0.f;
  float m2 = -INFINITY, l2 = 0.f, aD2 = 0.f, ac2 = 0.f, ae2 = 0.f, ah2 = 0.f;

  // level-1 -> level-2 (both end up scaled to m)
  __device__ __forceinline__ void flush() {
    const float mu = (m == -INFINITY) ? 0.f : m;
    const float c2 = fast_exp2(m2 - mu);
    l2 = fmaf(l2, c2, l);
    aD2 = fmaf(aD2, c2, aD);
    ac2 = fmaf(ac2, c2, ac);
    ae2 = fmaf(ae2, c2, ae);
    ah2 = fmaf(ah2, c2, ah);
    m2 = m;
    l = aD = ac = ae = ah = 0.f;
  }
};

constexpr int kFlush = 64;  // blocks per level-1 chain

// Online accumulation of one 32-key block (per lane: 16 keys of one query).
// In the TAIL variant keys at relative index >= nvalid_rel are masked out.
template <bool TAIL>
__device__ __forceinline__ void online_update(const f32x16& S, const f32x16& G, const f32x16& dP,
                                              const f32x16& H, float sl2, bool pos_scale, int nvalid_rel,
                                              OnlineSums& st) {
  const int h = lane_id() >> 5;
  // block extreme of the raw score (the max of s*S is s*max S for s >= 0,
  // s*min S otherwise)
  float ext = pos_scale ? -INFINITY : INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool ok = !TAIL || acc_row(h, i) < nvalid_rel;
    if (ok) ext = pos_scale ? fmaxf(ext, S[i]) : fminf(ext, S[i]);
  }
  const float mb = (ext == INFINITY || ext == -INFINITY) ? -INFINITY : ext * sl2;
  const float mn = fmaxf(st.m, mb);
  const float mu = (mn == -INFINITY) ? 0.f : mn;
  const float alpha = fast_exp2(st.m - mu);
  float bl = 0.f, bD = 0.f, bc = 0.f, be = 0.f, bh = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float p = fast_exp2(fmaf(S[i], sl2, -mu));
    if (TAIL && acc_row(h, i) >= nvalid_rel) p = 0.f;
    const float t = p * dP[i];
    bl += p;
    bD += t;
    bc = fmaf(p, G[i], bc);
    be = fmaf(t, G[i], be);
    bh = fmaf(p, H[i], bh);
  }
  st.l = fmaf(st.l, alpha, bl);
  st.aD = fmaf(st.aD, alpha, bD);
  st.ac = fmaf(st.ac, alpha, bc);
  st.ae = fmaf(st.ae, alpha, be);
  st.ah = fmaf(st.ah, alpha, bh);
  st.m = mn;
}

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void rowstats_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const T* __restrict__ gQ, const T* __restrict__ gK, const T* __restrict__ gV, float* __restrict__ lse_out,
    float* __restrict__ D_out, float* __restrict__ c_out, float* __restrict__ r_out,
    float* __restrict__ zero_a, float* __restrict__ zero_b, int N, int nqblk, float scale) {
  using Cfg = RowstatsCfg<T, D>;
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int BK = Cfg::BK, LDK = Cfg::LDK, NCH = Cfg::NCH;
  __shared__ __attribute__((aligned(16))) T sK[4][BK][LDK];  // K, gK, V, gV rows of the stage

  const int head = blockIdx.x / nqblk;
  const int qblk = blockIdx.x % nqblk;
  const size_t hoff = (size_t)head * N * D;
  const int w = wave_id(), l = lane_id(), h = l >> 5;
  const int qw = qblk * Cfg::BQ + 32 * w;  // first query of this wave
  const int q = qw + (l & 31);            // this lane's query
  const bool qvalid = q < N;

  // B operands of the wave's 32 queries (lane <-> query, k over d)
  F fQ[NCH], fgQ[NCH], fdO[NCH];
  {
    const T* rq = Q + hoff + (size_t)q * D;
    const T* rgq = gQ + hoff + (size_t)q * D;
    const T* rdo = dO + hoff + (size_t)q * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      fQ[c] = load_row_frag(rq, qvalid, c);
      fgQ[c] = load_row_frag(rgq, qvalid, c);
      fdO[c] = load_row_frag(rdo, qvalid, c);
    }
  }

  // zero the atomically accumulated outputs of this workgroup's query rows
  if (zero_a != nullptr) {
    const int r0 = qblk * Cfg::BQ;
    const int nrows = min(Cfg::BQ, N - r0);
    float4* za = reinterpret_cast<float4*>(zero_a + hoff + (size_t)r0 * D);
    float4* zb = reinterpret_cast<float4*>(zero_b + hoff + (size_t)r0 * D);
    const int nvec = nrows * D / 4;
    for (int i = threadIdx.x; i < nvec; i += 256) {
      za[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      zb[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }

  const float sl2 = scale * kLog2e;
  const bool pos_scale = scale >= 0.f;
  OnlineSums st;
  int nblk = 0;

  for (int k0 = 0; k0 < N; k0 += BK) {
    const int nk = min(BK, N - k0);
    __syncthreads();
    copy_rows_to_lds<T, BK, D, 256>(&sK[0][0][0], LDK, K + hoff + (size_t)k0 * D, nk);
    copy_rows_to_lds<T, BK, D, 256>(&sK[1][0][0], LDK, gK + hoff + (size_t)k0 * D, nk);
    copy_rows_to_lds<T, BK, D, 256>(&sK[2][0][0], LDK, V + hoff + (size_t)k0 * D, nk);
    copy_rows_to_lds<T, BK, D, 256>(&sK[3][0][0], LDK, gV + hoff + (size_t)k0 * D, nk);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb) {
      if (kb * 32 >= nk) break;
      f32x16 S = {}, G = {}, dP = {}, H = {};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const F ak = ld_rows(&sK[0][kb * 32][16 * c], LDK);
        const F agk = ld_rows(&sK[1][kb * 32][16 * c], LDK);
        const F av = ld_rows(&sK[2][kb * 32][16 * c], LDK);
        const F agv = ld_rows(&sK[3][kb * 32][16 * c], LDK);
        E::mma(S, ak, fQ[c]);
        E::mma(G, ak, fgQ[c]);
        E::mma(G, agk, fQ[c]);
        E::mma(dP, av, fdO[c]);
        E::mma(H, agv, fdO[c]);
      }
      const int nrel = nk - kb * 32;
      if (nrel >= 32)
        online_update<false>(S, G, dP, H, sl2, pos_scale, nrel, st);
      else
        online_update<true>(S, G, dP, H, sl2, pos_scale, nrel, st);
      if (++nblk == kFlush) {
        st.flush();
        nblk = 0;
      }
    }
  }
  st.flush();
  const float m = st.m, lsum = st.l2, aD = st.aD2, ac = st.ac2, ae = st.ae2, ah = st.ah2;

  // merge the two half-waves (same query column, disjoint keys)
  const float m2 = __shfl_xor(m, 32), l2 = __shfl_xor(lsum, 32);
  const float aD2 = __shfl_xor(aD, 32), ac2 = __shfl_xor(ac, 32);
  const float ae2 = __shfl_xor(ae, 32), ah2 = __shfl_xor(ah, 32);
  const float mm = fmaxf(m, m2);
  const float mu = (mm == -INFINITY) ? 0.f : mm;
  const float e1 = fast_exp2(m - mu), e2 = fast_exp2(m2 - mu);
  const float L = lsum * e1 + l2 * e2;
  const float AD = aD * e1 + aD2 * e2, AC = ac * e1 + ac2 * e2;
  const float AE = ae * e1 + ae2 * e2, AH = ah * e1 + ah2 * e2;
  if (h == 0 && qvalid) {
    const float inv = 1.f / L;
    const float Dq = AD * inv;
    const float cq = scale * AC * inv;
    const float rq = scale * AE * inv - Dq * cq + AH * inv;
    const size_t o = (size_t)head * N + q;
    lse_out[o] = (mm + log2f(L)) * kLn2;
    D_out[o] = Dq;
    c_out[o] = cq;
    r_out[o] = rq;
  }
}

template <typename T, int D>
hipError_t launch_rowstats(const void* Q, const void* K, const void* V, const void* dO, const void* gQ,
                           const void* gK, const void* gV, float* lse, float* Dv, float* cv, float* rv,
                           float* zero_a, float* zero_b, int BH, int N, float scale, hipStream_t stream) {
  using Cfg = RowstatsCfg<T, D>;
  const int nqblk = (N + Cfg::BQ - 1) / Cfg::BQ;
  const long long nblocks = (long long)nqblk * BH;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  rowstats_kernel<T, D><<<dim3((unsigned)nblocks), dim3(256), 0, stream>>>(
      (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, (const T*)gQ, (const T*)gK, (const T*)gV, lse, Dv,
      cv, rv, zero_a, zero_b, N, nqblk, scale);
  return hipGetLastError();
}

template hipError_t launch_rowstats<bf16, 64>(const void*, const void*, const void*, const void*, const void*,
                                              const void*, const void*, float*, float*, float*, float*, float*,
                                              float*, int, int, float, hipStream_t);
template hipError_t launch_rowstats<bf16, 128>(const void*, const void*, const void*, const void*, const void*,
                                               const void*, const void*, float*, float*, float*, float*, float*,
                                               float*, int, int, float, hipStream_t);
template hipError_t launch_rowstats<float, 64>(const void*, const void*, const void*, const void*, const void*,
                                               const void*, const void*, float*, float*, float*, float*, float*,
                                               float*, int, int, float, hipStream_t);
template hipError_t launch_rowstats<float, 128>(const void*, const void*, const void*, const void*, const void*,
                                                const void*, const void*, float*, float*, float*, float*, float*,
                                                float*, int, int, float, hipStream_t);

}  // namespace flashbob
