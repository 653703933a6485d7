// Query-major kernels of the BoB schedule: pass 1 (row scalars) and the
// query side of pass 2 (gradQ, graddO). Both sweep the whole key sequence for
// a block of queries, so they share one kernel template.
//
// FlashBoB (arXiv 2609.24089), Abstract: two row-wise scalars fix every BoB
// output through affine maps; a first pass gathers them, a second pass
// recomputes the score tiles (FlashAttention-style recomputation) and turns
// them into the outputs, never holding an N x N tensor off chip.
//
// With S = Q K^T, P = exp(s S - LSE), dP = dO V^T, G = s (gQ K^T + Q gK^T),
// H = dO gV^T:
//   pass 1:  D = rowsum(P o dP),  c = rowsum(P o G),
//            r = rowsum(dS o G) + rowsum(P o H),  dS = P o (dP - D).
//            One sweep with an online running max m: accumulate
//            l = sum Pt, aD = sum Pt dP, ac = sum Pt G, ae = sum Pt dP G,
//            ah = sum Pt H (Pt = exp(s S - m)), then D = aD/l, c = ac/l,
//            r = ae/l - D c + ah/l, LSE = m + ln l. (SAVED: m is fixed at a
//            saved log-sum-exp of the row for the whole sweep. PRE: Q and gQ
//            arrive scaled by s, G is s G, and ae = sum Pt (dP G + H) holds
//            both of r's sums.)
//   pass 2q: dS  = P (dP - D),  A = P (G - c),  dS2 = dS (G - c) + P (H - r),
//            gradQ = s (dS2 K + dS gK),  graddO = A V + P gV.
//            Pass 1 hands the scalars over as LSE log2(e), -D, -c/s and -r
//            (the key-major kernel starts its dP, G, H accumulators from them;
//            in bf16 this one starts dP and H from -D and -r, and with PRE G
//            from -c).
//            FIRST: also the first-backward dQ = s dS K.
//
// gfx950 schedule: a workgroup of 4 waves (8 in bf16 d = 64 pass 2q) owns 32
// queries per wave and streams the keys in 32-row stages (K, gK, V, gV)
// through two LDS buffers, issuing each stage's global reads one stage ahead.
// Per 32-key block a wave builds the transposed tiles S^T, G^T,
// dP^T, H^T (keys x its queries) with MFMA; the accumulator layout then puts
// one query per lane, so the row scalars are per-lane registers. In pass 2q
// the elementwise results (P, dS, dS2, A) go straight from the accumulator
// registers into the next MFMAs as B operands (k = keys, in the accumulator's
// row order); the A operands K^T, gK^T, V^T, gV^T come from the LDS stage via
// transpose reads in the same k order. gradQ^T and graddO^T stay in registers
// for the whole sweep (no atomics, no cross-wave reduction) and leave through
// LDS in whole-line stores.

#include <cmath>
#include <type_traits>

#include "bob_device.h"

namespace flashbob {

template <typename T, int D_, bool GRADQ, bool FIRST = false>
struct QueryCfg {
  static constexpr int D = D_;
  static constexpr int BK = 32;                        // keys per LDS stage (one MFMA block)
  static constexpr int LDK = D + 16 / (int)sizeof(T);  // padded LDS row (elements)
  static constexpr int NCH = D / 16;                   // 16-wide k chunks over d
  static constexpr int NDB = D / 32;                   // 32-row blocks of d
  // pass 2q at d >= 256: each query block is handled by OSPLIT workgroups,
  // each accumulating its own share of the output columns (the score tiles
  // are recomputed by each), so the d-wide operands stay in registers beside
  // accumulators for only part of d
  static constexpr int OSPLIT = (GRADQ && D >= 256) ? 2 : 1;
  static constexpr int NDBO = NDB / OSPLIT;            // 32-row blocks of d per workgroup
  // bf16 d = 64, 128 and 256 stage tiles with direct global->LDS loads into
  // swizzled unpadded rows (no staging registers; above d = 64 a tile is d/64
  // swizzled 32 x 64 pieces), which the transposing LDS reads take without
  // bank conflicts; the other variants stage through registers into padded
  // rows. Two waves per SIMD (<= 256 registers: the second wave hides the
  // first one's latencies and overlaps its VALU work with the other's MFMAs)
  // where the per-wave state fits: bf16 d = 64, pass 1 in bf16 at every d (a
  // few bytes spill at d = 96, 128, still faster), and d = 32; the rest run
  // one wave per SIMD.
  static constexpr bool SWZ = sizeof(T) == 2 && (D == 64 || D == 128 || D == 256);
  static constexpr bool SWZ64 = SWZ && D == 64;
  static constexpr bool OCC2 = SWZ64 || (!GRADQ && sizeof(T) == 2) || D == 32;
  // Waves per workgroup, each owning 32 queries: bf16 d = 64 pass 2q runs
  // eight (the two waves of each SIMD in one workgroup), so each K, gK, V, gV
  // stage is fetched into LDS once per 256 queries instead of once per 128:
  // the chip runs these sweeps at its power limit, and the global -> LDS
  // traffic is a measurable part of the energy per block. Pass 1 keeps four
  // (see OCC; eight at two waves per SIMD measured slower).
  static constexpr int NW = (SWZ64 && GRADQ) ? 8 : 4;
  static constexpr int BQ = 32 * NW;                   // queries per workgroup
  // waves per SIMD: pass 1 in bf16 at d = 64 fits 168 registers and runs
  // three, which hides more of each wave's exp and MFMA latency than two
  // (the first-backward dQ accumulator fits two waves per SIMD at bf16 d = 64,
  // with the operand fragments packed into the score tiles; elsewhere its
  // kernels run one)
  static constexpr int OCC = (FIRST && !SWZ64) ? 1 : (!GRADQ && SWZ64) ? 3 : OCC2 ? 2 : 1;
  static constexpr int NBUF = 2;                       // stage n in use, stage n+1 arriving
  static constexpr int STAGE = 4 * BK * (SWZ ? D : LDK);  // elements of one stage
  static constexpr size_t LDS_BYTES = NBUF * STAGE * sizeof(T);
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// One fragment (16 k values of d) of a row held by this lane; zero for rows
// past the sequence end.
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

// ---------------------------------------------------------------------------
// pass 1 running sums of one lane (one query, the keys of its half-wave).
// Level-1 sums are scaled to the current running max m and absorb one 32-key
// block at a time (block sums first); every kFlush blocks they move into
// level-2 sums kept at their own max m2 every kFlush blocks. At 262144 keys
// this keeps every fp32 chain at a few hundred additions instead of 131072.
struct OnlineSums {
  float m = -INFINITY, l = 0.f, aD = 0.f, ac = 0.f, ae = 0.f, ah = 0.f;
  float m2 = -INFINITY, l2 = 0.f, aD2 = 0.f, ac2 = 0.f, ae2 = 0.f, ah2 = 0.f;

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

// Online accumulation of one 32-key block (per lane: 16 keys of one query),
// in two calls: chunk 0 first takes the block maximum and rescales, then each
// chunk adds its 8 keys. In the TAIL variant keys at relative index
// >= nvalid_rel are masked out. FIXED: the row's saved log-sum-exp serves as
// the maximum for the whole sweep (p <= 1 throughout), so there is neither a
// block maximum nor a rescale. PRE: S and G arrive scaled by s (the kernel
// scaled Q and gQ), so ae takes the whole sum P (dP G + H) that r needs
// (one fma fewer per element) and ah stays zero.
template <bool TAIL, bool FIXED, bool PRE>
__device__ __forceinline__ void online_chunk(int cc, const f32x16& S, const f32x16& G, const f32x16& dP,
                                             const f32x16& H, float sl2, int nvalid_rel, OnlineSums& st,
                                             float& mu) {
  const int h = lane_id() >> 5;
  if (cc == 0 && !FIXED) {
    // block maximum of x = S * scale * log2(e); the caller makes the scale
    // non-negative (sl2 >= 0), so it is the maximum of S times sl2
    float mb = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = !TAIL || acc_row(h, i) < nvalid_rel;
      if (ok) mb = fmaxf(mb, S[i]);
    }
    mb *= sl2;
    const float mn = fmaxf(st.m, mb);
    mu = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = fast_exp2(st.m - mu);
    st.l *= alpha;
    st.aD *= alpha;
    st.ac *= alpha;
    st.ae *= alpha;
    st.ah *= alpha;
    st.m = mn;
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int i = 8 * cc + s;
    float p = fast_exp2(fmaf(S[i], sl2, -mu));
    if (TAIL && acc_row(h, i) >= nvalid_rel) p = 0.f;
    if constexpr (PRE) {
      st.l += p;
      st.aD = fmaf(p, dP[i], st.aD);
      st.ac = fmaf(p, G[i], st.ac);
      st.ae = fmaf(p, fmaf(dP[i], G[i], H[i]), st.ae);
    } else {
      const float t = p * dP[i];
      st.l += p;
      st.aD += t;
      st.ac = fmaf(p, G[i], st.ac);
      st.ae = fmaf(t, G[i], st.ae);
      st.ah = fmaf(p, H[i], st.ah);
    }
  }
}

// pass 2q elementwise step of one 16-key chunk cc of a 32-key block, turned
// into B operands (k = keys in accumulator row order). Dq, cq, rq are -D, -c,
// -r of the lane's query. TAIL masks keys at relative index >= nvalid_rel.
template <typename T, bool TAIL>
__device__ __forceinline__ void query_chunk(int cc, const f32x16& S, const f32x16& G, const f32x16& dP,
                                            const f32x16& H, float sl2, float scale, float l2, float Dq,
                                            float cq, float rq, int nvalid_rel, typename Elem<T>::frag& fP,
                                            typename Elem<T>::frag& fdS, typename Elem<T>::frag& fdS2,
                                            typename Elem<T>::frag& fA) {
  const int h = lane_id() >> 5;
  f32x8 P, dS, dS2, A;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int i = 8 * cc + s;
    float p = fast_exp2(fmaf(S[i], sl2, -l2));
    if (TAIL && acc_row(h, i) >= nvalid_rel) p = 0.f;
    const float ds = p * (dP[i] + Dq);
    const float g = fmaf(G[i], scale, cq);
    P[s] = p;
    dS[s] = ds;
    A[s] = p * g;
    dS2[s] = fmaf(ds, g, p * (H[i] + rq));
  }
  to_frag(fP, P);
  to_frag(fdS, dS);
  to_frag(fdS2, dS2);
  to_frag(fA, A);
}

// The same step for bf16 operands, done in place: the results of chunk cc
// are rounded pair by pair and written back into the tiles' own registers,
// P into S, dS into dP, A into G and dS2 into H, at words 8 cc .. 8 cc + 3
// (pair s2 reads words 8 cc + 2 s2, + 1 and writes word 8 cc + s2, which the
// same or an earlier pair has already read). The chunk's bf16 operand
// fragments are then those four words of each tile (packed_frag), and no
// separate fragment registers are live. With SHIFTED, dP and H arrive
// already shifted by the row's -D and -r (their accumulators start from
// them); otherwise Dq and rq (-D and -r) are added here. GSCALED: G arrives
// as s G - c (pre-scaled operands, accumulator started from -c).
template <bool TAIL, bool SHIFTED, bool GSCALED = false>
__device__ __forceinline__ void query_chunk_inplace(int cc, f32x16& S, f32x16& G, f32x16& dP, f32x16& H,
                                                    float sl2, float scale, float l2, float Dq, float cq,
                                                    float rq, int nvalid_rel) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  auto pack = [](float a, float b) __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
  };
  const int h = lane_id() >> 5;
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    float vp[2], vds[2], va[2], vd2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 8 * cc + 2 * s2 + e;
      float p = fast_exp2(fmaf(S[i], sl2, -l2));
      if (TAIL && acc_row(h, i) >= nvalid_rel) p = 0.f;
      const float ds = p * (SHIFTED ? dP[i] : dP[i] + Dq);
      const float g = GSCALED ? G[i] : fmaf(G[i], scale, cq);
      vp[e] = p;
      vds[e] = ds;
      va[e] = p * g;
      vd2[e] = fmaf(ds, g, p * (SHIFTED ? H[i] : H[i] + rq));
    }
    S[8 * cc + s2] = pack(vp[0], vp[1]);
    dP[8 * cc + s2] = pack(vds[0], vds[1]);
    G[8 * cc + s2] = pack(va[0], va[1]);
    H[8 * cc + s2] = pack(vd2[0], vd2[1]);
  }
}

// Words 8 cc .. 8 cc + 3 of a tile as a bf16 operand fragment.
__device__ __forceinline__ bf16x8 packed_frag(const f32x16& t, int cc) {
  return __builtin_bit_cast(bf16x8, cc == 0 ? __builtin_shufflevector(t, t, 0, 1, 2, 3)
                                            : __builtin_shufflevector(t, t, 8, 9, 10, 11));
}

// FIRST (pass 2q only): also return the first-backward dQ = s dS K (one more
// product per block against the K^T operand already read; the extra
// accumulator needs the one-wave-per-SIMD register budget).
// PRE (bf16 pass 1 and plain pass 2q, |s| a power of two in (0, 1]): Q and gQ
// are scaled by s (pass 1: |s|, after its sign flip) in registers, exactly
// short of elements pushed below the normal range, so S and G come out of
// the MFMAs scaled; pass 2q then starts G from the row's -c like dP and H.
template <typename T, int D, bool GRADQ, bool FIRST, bool SAVED, bool PRE = false>
__global__ __launch_bounds__((QueryCfg<T, D, GRADQ, FIRST>::NW * 64),
                             (QueryCfg<T, D, GRADQ, FIRST>::OCC * 4 / QueryCfg<T, D, GRADQ, FIRST>::NW))
void query_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const T* __restrict__ gQ, const T* __restrict__ gK, const T* __restrict__ gV, float* __restrict__ lse,
    float* __restrict__ Dv, float* __restrict__ cv, float* __restrict__ rv, void* __restrict__ gradQ,
    void* __restrict__ graddO, void* __restrict__ dQo, const float* __restrict__ lse_in, int N, int nqblk,
    float scale, int lse_natural, int causal, int G, int out_bf16) {
  static_assert(!(SAVED && GRADQ), "a saved log-sum-exp replaces pass 1's running maximum only");
  static_assert(!PRE || (sizeof(T) == 2 && !FIRST), "pre-scaled operands: bf16 pass 1 and plain pass 2q");
  using Cfg = QueryCfg<T, D, GRADQ, FIRST>;
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int BK = Cfg::BK, LDK = Cfg::LDK, NCH = Cfg::NCH, NDB = Cfg::NDB, NBUF = Cfg::NBUF;
  constexpr bool SWZ = Cfg::SWZ, SWZ64 = Cfg::SWZ64;
  constexpr int ROWLEN = SWZ ? D : LDK;
  // [NBUF][4][BK][ROWLEN]: K, gK, V, gV of a stage
  __shared__ __attribute__((aligned(16))) T smem[NBUF * Cfg::STAGE];
  auto sK = [&](int b, int t, int row, int col) __attribute__((always_inline)) { return smem + ((b * 4 + t) * BK + row) * ROWLEN + col; };
  auto tile = [&](int b, int t) __attribute__((always_inline)) { return smem + (b * 4 + t) * BK * ROWLEN; };
  // (SWZ: from the 64-column half c16 / 4, resp. col0 / 64, of the tile)
  auto lds_rows = [&](int b, int t, int row0, int c16) __attribute__((always_inline)) -> typename Elem<T>::frag {
    if constexpr (SWZ) return ld_rows_sw(tile(b, t) + 2048 * (c16 >> 2), row0, c16 & 3);
    else return ld_rows(sK(b, t, row0, 16 * c16), LDK);
  };
  auto lds_cols = [&](int b, int t, int krow0, int col0) __attribute__((always_inline)) -> typename Elem<T>::frag {
    if constexpr (SWZ) return ld_cols_perm_sw(tile(b, t) + 2048 * (col0 >> 6), krow0, col0 & 63);
    else return ld_cols_perm(sK(b, t, krow0, col0), LDK);
  };

  // causal: the longest sweeps (the last query blocks) start first, across
  // all heads at once (consecutive workgroups take the same block of
  // successive heads)
  // (OSPLIT: consecutive workgroups share a query block and split its output
  // columns; part = which share)
  constexpr int OSPLIT = Cfg::OSPLIT, NDBO = Cfg::NDBO;
  const int part = OSPLIT > 1 ? (int)(blockIdx.x % OSPLIT) : 0;
  const unsigned bid = OSPLIT > 1 ? blockIdx.x / OSPLIT : blockIdx.x;
  const int nheads = (int)((OSPLIT > 1 ? gridDim.x / OSPLIT : gridDim.x) / nqblk);
  const int head = causal ? (int)(bid % nheads) : (int)(bid / nqblk);
  const int qblk = causal ? nqblk - 1 - (int)(bid / nheads) : (int)(bid % nqblk);
  const size_t hoff = (size_t)head * N * D;         // query head (Q, dO, gQ, outputs)
  const size_t koff = (size_t)(head / G) * N * D;   // its key/value head (groups of G)
  const int w = wave_id(), l = lane_id(), h = l >> 5, col = l & 31;
  const int q = qblk * Cfg::BQ + 32 * w + col;  // this lane's query
  const bool qvalid = q < N;
  const int qlim = causal ? min(N, q + 1) : N;    // keys [0, qlim) are visible to it

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

  // Pass 1 works with |scale|: for a negative scale it negates Q and gQ, which
  // leaves s S and s G unchanged and lets the online maximum be taken on S.
  const float sgn = (!GRADQ && scale < 0.f) ? -1.f : 1.f;
  if (sgn < 0.f) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      negate(fQ[c]);
      negate(fgQ[c]);
    }
  }
  scale *= sgn;
  if constexpr (PRE) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      scale_frag(fQ[c], scale);
      scale_frag(fgQ[c], scale);
    }
  }
  const float sl2 = (PRE ? 1.f : scale) * kLog2e;
  OnlineSums st;  // pass 1 state
  float mu = 0.f;  // pass 1: the running max used for the current block
  if constexpr (SAVED) {
    // the saved natural-log LSE of the row, in the base-2 units of x = s S log2(e)
    if (qvalid) st.m = lse_in[(size_t)head * N + q] * kLog2e;
    else st.m = 0.f;
    mu = st.m;
  }
  // pass 2q state: the lane's row scalars and the output accumulators
  // (gradQ^T, graddO^T: d rows x the wave's 32 queries)
  // (pass-2 form: LSE * log2(e), -D, -c, -r)
  float l2 = INFINITY, Dq = 0.f, cq = 0.f, rq = 0.f;
  f32x16 accQ[GRADQ ? NDBO : 1], accO[GRADQ ? NDBO : 1], accdQ[FIRST ? NDBO : 1];
  if constexpr (GRADQ) {
    if (qvalid) {
      const size_t o = (size_t)head * N + q;
      l2 = lse[o];
      Dq = Dv[o];
      cq = scale * cv[o];
      rq = rv[o];
    }
#pragma unroll
    for (int j = 0; j < NDBO; ++j) {
      accQ[j] = f32x16{};
      accO[j] = f32x16{};
      if constexpr (FIRST) accdQ[j] = f32x16{};
    }
  }

  const int nblk = (N + BK - 1) / BK;  // 32-key blocks = stages
  // Key blocks visited and how many of them need no mask. Causal: the
  // workgroup's queries q0 .. q0+BQ-1 see keys 0 .. q0+BQ-1, and blocks
  // wholly below q0 are visible to all of them; the blocks across the
  // diagonal mask per lane at the key limit qlim = q + 1 (the masked path
  // also covers a partial last block).
  const bool last_partial = N % BK != 0;
  const int q0 = qblk * Cfg::BQ;
  const int nvis = causal ? min(nblk, (q0 + Cfg::BQ + BK - 1) / BK) : nblk;
  const int nfull = causal ? min(nvis, q0 / BK) : (last_partial ? nblk - 1 : nblk);
  // staging of stage n: prefetch() issues its global reads (into registers,
  // or straight into its LDS buffer when SWZ); commit() makes it visible to
  // this wave's later LDS accesses (register store, or wait for the loads).
  // A stage past the last visible block is an empty buffer (zeros, no memory
  // access), so every iteration can prefetch its successor.
  RowPrefetch<T, SWZ ? 0 : BK, D, 256> pk, pgk, pv, pgv;
  auto prefetch = [&](int n) __attribute__((always_inline)) {
    const int k0 = n < nvis ? n * BK : 0;
    const int nk = n < nvis ? min(BK, N - k0) : 0;
    if constexpr (SWZ && Cfg::NW == 8) {
      // wave w: rows 8 (w % 4) .. + 7 of K and V (w < 4) or of gK and gV
      const int b = n & (NBUF - 1);
      const int rg = w & 3;
      load_rows8_sw(tile(b, w >> 2), (w < 4 ? K : gK) + koff + (size_t)k0 * D, nk, rg);
      load_rows8_sw(tile(b, 2 + (w >> 2)), (w < 4 ? V : gV) + koff + (size_t)k0 * D, nk, rg);
    } else if constexpr (SWZ64) {
      const int b = n & (NBUF - 1);
      load_tile_sw(tile(b, 0), K + koff + (size_t)k0 * D, nk);
      load_tile_sw(tile(b, 1), gK + koff + (size_t)k0 * D, nk);
      load_tile_sw(tile(b, 2), V + koff + (size_t)k0 * D, nk);
      load_tile_sw(tile(b, 3), gV + koff + (size_t)k0 * D, nk);
    } else if constexpr (SWZ) {
      const int b = n & (NBUF - 1);
      const T* const src[4] = {K, gK, V, gV};
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int hf = 0; hf < D / 64; ++hf)
          load_half_sw(tile(b, t), src[t] + koff + (size_t)k0 * D, nk, D * (int)sizeof(T), hf);
    } else {
      pk.load(K + koff + (size_t)k0 * D, nk);
      pgk.load(gK + koff + (size_t)k0 * D, nk);
      pv.load(V + koff + (size_t)k0 * D, nk);
      pgv.load(gV + koff + (size_t)k0 * D, nk);
    }
  };
  auto commit = [&](int n) __attribute__((always_inline)) {
    if constexpr (SWZ) {
      wait_vmem();
    } else {
      const int b = n & (NBUF - 1);
      pk.store(sK(b, 0, 0, 0), LDK);
      pgk.store(sK(b, 1, 0, 0), LDK);
      pv.store(sK(b, 2, 0, 0), LDK);
      pgv.store(sK(b, 3, 0, 0), LDK);
    }
  };

  // S^T, G^T, dP^T, H^T of block n (keys x this wave's queries)
  struct Tiles {
    f32x16 S, G, dP, H;
  };
  // d-chunks [c0, c1) of the recompute products of block n
  // bf16 pass 2q packs the operand fragments into the score tiles' own
  // registers (query_chunk_inplace); fp32 keeps them apart
  constexpr bool INPLACE = GRADQ && sizeof(T) == 2;
  // start dP and H from -D and -r: two fewer VALU operations per element,
  // left out where the first-backward accumulator leaves no registers for it
  constexpr bool SHIFTED = INPLACE && !FIRST;
  auto recompute = [&](int n, Tiles& t, int c0, int c1) __attribute__((always_inline)) {
    const int b = n & (NBUF - 1);
    if (c0 == 0) {
      t.S = f32x16{};
      if constexpr (GRADQ && PRE)  // s G - c: the lane's -c
        t.G = f32x16{cq, cq, cq, cq, cq, cq, cq, cq, cq, cq, cq, cq, cq, cq, cq, cq};
      else
        t.G = f32x16{};
      if constexpr (SHIFTED) {
        // the row's -D and -r (one query per lane: a broadcast)
        t.dP = f32x16{Dq, Dq, Dq, Dq, Dq, Dq, Dq, Dq, Dq, Dq, Dq, Dq, Dq, Dq, Dq, Dq};
        t.H = f32x16{rq, rq, rq, rq, rq, rq, rq, rq, rq, rq, rq, rq, rq, rq, rq, rq};
      } else {
        t.dP = f32x16{};
        t.H = f32x16{};
      }
    }
#pragma unroll
    for (int c = c0; c < c1; ++c) {
      const F ak = lds_rows(b, 0, 0, c);  // lane <-> key, k over d
      const F agk = lds_rows(b, 1, 0, c);
      const F av = lds_rows(b, 2, 0, c);
      const F agv = lds_rows(b, 3, 0, c);
      E::mma(t.S, ak, fQ[c]);
      E::mma(t.G, ak, fgQ[c]);
      E::mma(t.G, agk, fQ[c]);
      E::mma(t.dP, av, fdO[c]);
      E::mma(t.H, agv, fdO[c]);
    }
  };
  struct Frags {
    F P[2], dS[2], dS2[2], A[2];
  };
  // elementwise work of 16-key chunk cc of block n: online sums (pass 1) or
  // operand fragments (pass 2q); TAIL masks keys past the sequence end
  auto elementwise = [&](auto tail, int n, int cc, Tiles& t, Frags& f) __attribute__((always_inline)) {
    constexpr bool TAIL = decltype(tail)::value;
    const int nrel = qlim - n * BK;
    if constexpr (!GRADQ)
      online_chunk<TAIL, SAVED, PRE>(cc, t.S, t.G, t.dP, t.H, sl2, nrel, st, mu);
    else if constexpr (INPLACE)
      query_chunk_inplace<TAIL, SHIFTED, PRE>(cc, t.S, t.G, t.dP, t.H, sl2, scale, l2, Dq, cq, rq, nrel);
    else
      query_chunk<T, TAIL>(cc, t.S, t.G, t.dP, t.H, sl2, scale, l2, Dq, cq, rq, nrel, f.P[cc], f.dS[cc],
                           f.dS2[cc], f.A[cc]);
  };
  // output products of 16-key chunk cc of block n (pass 2q)
  auto outputs = [&](int n, int cc, const Tiles& t, const Frags& f) __attribute__((always_inline)) {
    if constexpr (GRADQ) {
      const int b = n & (NBUF - 1);
      F fP, fdS, fdS2, fA;
      if constexpr (INPLACE) {
        fP = packed_frag(t.S, cc);
        fdS = packed_frag(t.dP, cc);
        fdS2 = packed_frag(t.H, cc);
        fA = packed_frag(t.G, cc);
      } else {
        fP = f.P[cc];
        fdS = f.dS[cc];
        fdS2 = f.dS2[cc];
        fA = f.A[cc];
      }
#pragma unroll
      for (int j = 0; j < NDBO; ++j) {
        // lane <-> d, k over this chunk's keys (accumulator row order); this
        // workgroup's share of the columns starts at block part * NDBO
        const int jd = 32 * (part * NDBO + j);
        const F tK = lds_cols(b, 0, 16 * cc, jd);
        const F tgK = lds_cols(b, 1, 16 * cc, jd);
        const F tV = lds_cols(b, 2, 16 * cc, jd);
        const F tgV = lds_cols(b, 3, 16 * cc, jd);
        E::mma(accQ[j], tK, fdS2);
        E::mma(accQ[j], tgK, fdS);
        E::mma(accO[j], tV, fA);
        E::mma(accO[j], tgV, fP);
        if constexpr (FIRST) E::mma(accdQ[j], tK, fdS);
      }
    }
  };

  prefetch(0);  // nblk >= 1
  commit(0);
  __syncthreads();

  using F0 = std::integral_constant<bool, false>;
  using F1 = std::integral_constant<bool, true>;
  const int nsteady = nfull;
  Tiles t;
  Frags f;
  // one iteration per 32-key block; the unmasked ones are branch-free, so
  // each is one straight-line block the scheduler can interleave freely (the
  // last one prefetches an empty stage rather than taking a code path of its
  // own)
  auto iteration = [&](auto tail, int n) __attribute__((always_inline)) {
    prefetch(n + 1);  // its buffer last held stage n-1, read in iteration n-1
    recompute(n, t, 0, NCH);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      elementwise(tail, n, cc, t, f);
      outputs(n, cc, t, f);
    }
    commit(n + 1);
    __syncthreads();
  };
  // pass 1 flushes its level-1 sums every kFlush blocks (outside the
  // branch-free inner loop)
  // (n0 is a multiple of kFlush and the steady iterations go in pairs from
  // it, so every stage buffer index below is a compile-time constant)
  for (int n0 = 0; n0 < nsteady; n0 += kFlush) {
    const int n1 = min(n0 + kFlush, nsteady);
    const int npairs = (n1 - n0) >> 1;
    for (int i = 0; i < npairs; ++i) {
      iteration(F0{}, n0 + 2 * i);
      iteration(F0{}, n0 + 2 * i + 1);
    }
    if ((n1 - n0) & 1) iteration(F0{}, n1 - 1);
    if constexpr (!GRADQ) st.flush();
  }
  // masked blocks: the causal diagonal (at most BQ/BK of them) and a partial
  // last block
  for (int n = nsteady; n < nvis; ++n) iteration(F1{}, n);

  if constexpr (!GRADQ) {
    st.flush();
    // merge the two half-waves (same query column, disjoint keys)
    const float m = st.m, lsum = st.l2, aD = st.aD2, ac = st.ac2, ae = st.ae2, ah = st.ah2;
    const float mo = __shfl_xor(m, 32), lo = __shfl_xor(lsum, 32);
    const float aDo = __shfl_xor(aD, 32), aco = __shfl_xor(ac, 32);
    const float aeo = __shfl_xor(ae, 32), aho = __shfl_xor(ah, 32);
    const float mm = fmaxf(m, mo);
    const float mu = (mm == -INFINITY) ? 0.f : mm;
    const float e1 = fast_exp2(m - mu), e2 = fast_exp2(mo - mu);
    const float L = lsum * e1 + lo * e2;
    const float AD = aD * e1 + aDo * e2, AC = ac * e1 + aco * e2;
    const float AE = ae * e1 + aeo * e2, AH = ah * e1 + aho * e2;
    if (h == 0 && qvalid) {
      const float inv = 1.f / L;
      const float Dr = AD * inv;
      // scale is |s| here and G carried the sign of s, so c = |s| AC / L and
      // c / s = sgn AC / L (PRE: G is s G already, and AE holds s AE + AH)
      const float cr = PRE ? AC * inv : scale * AC * inv;
      const float cbar = PRE ? sgn * AC * inv / scale : sgn * AC * inv;
      const float rr = PRE ? AE * inv - Dr * cr : scale * AE * inv - Dr * cr + AH * inv;
      const size_t o = (size_t)head * N + q;
      const float lse2 = mm + log2f(L);
      if (lse_natural) {  // the row statistics themselves
        lse[o] = lse2 * kLn2;
        Dv[o] = Dr;
        cv[o] = cr;
        rv[o] = rr;
      } else {  // pass-2 form: LSE * log2(e), -D, -c/s, -r
        lse[o] = lse2;
        Dv[o] = -Dr;
        cv[o] = -cbar;
        rv[o] = -rr;
      }
    }
  } else {
    // accQ[j] slot i holds d = 32 j + acc_row(h, i) of this lane's query;
    // each 32 x 32 block goes out through LDS (the stage buffers are free:
    // the last iteration ended with a barrier)
    static_assert(Cfg::LDS_BYTES >= (size_t)Cfg::NW * 4096, "output staging fits the stage buffers");
    float* xs = reinterpret_cast<float*>(smem) + 1024 * w;
    const int q0w = qblk * Cfg::BQ + 32 * w;  // the wave's first query
    const size_t base = hoff + (size_t)q0w * D;
    const int nrows = min(32, N - q0w);
#pragma unroll
    for (int j = 0; j < NDBO; ++j) {
      const int col0 = 32 * (part * NDBO + j);
      store_block_lds(xs, accQ[j], scale, gradQ, base, D, col0, nrows, out_bf16);
      store_block_lds(xs, accO[j], 1.f, graddO, base, D, col0, nrows, out_bf16);
      if constexpr (FIRST) store_block_lds(xs, accdQ[j], scale, dQo, base, D, col0, nrows, out_bf16);
    }
  }
}

template <typename T, int D, bool GRADQ, bool FIRST, bool SAVED>
hipError_t launch_query(const void* Q, const void* K, const void* V, const void* dO, const void* gQ,
                        const void* gK, const void* gV, float* lse, float* Dv, float* cv, float* rv,
                        void* gradQ, void* graddO, void* dQ, const float* lse_in, int BH, int N, float scale,
                        int lse_natural, int causal, int G, int out_bf16, hipStream_t stream) {
  using Cfg = QueryCfg<T, D, GRADQ, FIRST>;
  const int nqblk = (N + Cfg::BQ - 1) / Cfg::BQ;
  const long long nblocks = (long long)nqblk * BH * Cfg::OSPLIT;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // bf16 pass 1 and plain pass 2q at d = 64 with |s| = 2^-k (k = 0 .. 59):
  // the pre-scaled variant
  auto kern = query_kernel<T, D, GRADQ, FIRST, SAVED, false>;
  if constexpr (!FIRST && sizeof(T) == 2 && D == 64) {
    int e = 0;
    const float a = std::fabs(scale);
    if (a > 0.f && a <= 1.f && std::frexp(a, &e) == 0.5f && e >= -58) kern = query_kernel<T, D, GRADQ, FIRST, SAVED, true>;
  }
  kern<<<dim3((unsigned)nblocks), dim3(Cfg::NW * 64), 0, stream>>>(
      (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, (const T*)gQ, (const T*)gK, (const T*)gV, lse, Dv,
      cv, rv, gradQ, graddO, dQ, lse_in, N, nqblk, scale, lse_natural, causal, G, out_bf16);
  return hipGetLastError();
}

#define FLASHBOB_INST_QUERY(T, D, G, F, S)                                                                \
  template hipError_t launch_query<T, D, G, F, S>(const void*, const void*, const void*, const void*,      \
                                                  const void*, const void*, const void*, float*, float*,   \
                                                  float*, float*, void*, void*, void*, const float*, int,  \
                                                  int, float, int, int, int, int, hipStream_t);
// Pass 1 and pass 2q instantiations are built as separate objects (pass 1
// with MFMA results kept in VGPRs, which its register budget allows).
// Pass 1: plain and with a saved log-sum-exp; pass 2q: plain and with the
// first-backward dQ.
#define FLASHBOB_INST_QUERY_DIMS(G, F, S)  \
  FLASHBOB_INST_QUERY(bf16, 32, G, F, S)   \
  FLASHBOB_INST_QUERY(bf16, 64, G, F, S)   \
  FLASHBOB_INST_QUERY(bf16, 96, G, F, S)   \
  FLASHBOB_INST_QUERY(bf16, 128, G, F, S)  \
  FLASHBOB_INST_QUERY(bf16, 256, G, F, S)  \
  FLASHBOB_INST_QUERY(float, 32, G, F, S)  \
  FLASHBOB_INST_QUERY(float, 64, G, F, S)  \
  FLASHBOB_INST_QUERY(float, 96, G, F, S)  \
  FLASHBOB_INST_QUERY(float, 128, G, F, S)
#ifndef FLASHBOB_QUERY_PASS2
FLASHBOB_INST_QUERY_DIMS(false, false, false)
FLASHBOB_INST_QUERY_DIMS(false, false, true)
#endif
#ifndef FLASHBOB_QUERY_PASS1
FLASHBOB_INST_QUERY_DIMS(true, false, false)
FLASHBOB_INST_QUERY_DIMS(true, true, false)
#endif

}  // namespace flashbob
