// Key-major kernel of the BoB schedule: the key side of pass 2 (gradK, gradV).
//
// FlashBoB (arXiv 2609.24089), Abstract: with the two row scalars known from
// the first pass, every output is an affine map of recomputed tiles. For the
// key-side outputs, per (query i, key j):
//   P = exp(s S - LSE),  dS = P (dP - D),  A = P (G - c),
//   dS2 = dS (G - c) + P (H - r),
//   gradK_j = s sum_i (dS2_ij Q_i + dS_ij gQ_i),   gradV_j = sum_i A_ij dO_i,
// with S = Q K^T, dP = dO V^T, G = s (gQ K^T + Q gK^T), H = dO gV^T.
//
// gfx950 schedule: a workgroup of 4 waves (8 in bf16 d = 64) owns 32 keys per
// wave and streams the queries (Q, gQ, dO and their row scalars) in 32-row stages
// through two LDS buffers, issuing each stage's global reads one stage ahead.
// Per 32-query block a wave builds S, G, dP, H (queries x its keys) with
// MFMA, so each lane holds one key and 16 queries. The dP, G and H
// accumulators start from the queries' row scalars (-D, -c/s, -r, read from
// LDS as broadcast reads), so the MFMAs deliver dP - D, G/s - c/s and H - r
// and the elementwise step has no per-element subtractions left; LSE enters
// the exponent. P, dS, dS2, A then feed the next
// MFMAs straight from the accumulator registers as B operands (k = queries in
// accumulator row order), against Q^T, gQ^T, dO^T read from the LDS stage with
// transpose loads in the same order. gradK^T and gradV^T (FIRST: also the
// first-backward dK^T = s dS^T Q and dV^T = P^T dO) stay in registers for the
// whole sweep and leave through LDS in whole-line stores. The masked blocks
// (causal diagonal, partial blocks) run apart from a branch-free pair loop over
// the rest.

#include <type_traits>

#include "bob_device.h"

namespace flashbob {

template <typename T, int D_, bool FIRST = false>
struct KeyCfg {
  static constexpr int D = D_;
  static constexpr int BQ = 32;                        // queries per LDS stage (one MFMA block)
  static constexpr int LDQ = D + 16 / (int)sizeof(T);  // padded LDS row (elements)
  static constexpr int NCH = D / 16, NDB = D / 32;
  // d >= 256: each key block is handled by OSPLIT workgroups, each
  // accumulating its own share of gradK, gradV's columns (the score tiles are
  // recomputed by each), so the key-side operands stay in registers beside
  // accumulators for only part of d (two shares fit once the stage tiles load
  // straight into LDS and the operand fragments live in the score tiles: 13
  // products instead of the 23 of four; the first backward's extra
  // accumulators still need four)
  static constexpr int OSPLIT = D >= 256 ? (FIRST ? 4 : 2) : 1;
  static constexpr int NDBO = NDB / OSPLIT;  // 32-row blocks of d per workgroup
  // same staging choices as the query-major kernel; two waves per SIMD for
  // bf16 d = 64 (with the first backward too: its dK, dV accumulators fit once
  // the operand fragments are packed into the score tiles and more key-side
  // tensors live in LDS) and for d = 32 (FIRST: one wave)
  // (d = 128, 256: a stage tile is d/64 swizzled 32 x 64 pieces)
  static constexpr bool SWZ = sizeof(T) == 2 && (D == 64 || D == 128 || D == 256);
  static constexpr bool SWZ64 = SWZ && D == 64;
  static constexpr bool OCC2 = SWZ64 || (D == 32 && !FIRST);
  static constexpr int NBUF = 2;                       // stage n in use, stage n+1 arriving
  // SWZ: which of the wave's K, gK, V, gV operand tensors (bits 0..3) live in
  // LDS instead of registers (every per-block LDS read costs energy): none in
  // the plain kernel, whose operand fragments are packed into the score tiles'
  // registers; with the first backward's accumulators gK, V and gV (with gK
  // alone the loop still spills)
  static constexpr int KLDS = (OCC2 && SWZ64 && FIRST) ? 0xE : 0;
  static constexpr int NKLDS = __builtin_popcount(KLDS);
  // Waves per workgroup, each owning 32 keys: with two waves per SIMD at
  // bf16 d = 64 both go in one workgroup of eight, so each Q, gQ, dO stage is
  // fetched into LDS once per 256 keys instead of once per 128 (the chip runs
  // these sweeps at its power limit, and that traffic costs energy per block)
  static constexpr int NW = (OCC2 && SWZ64) ? 8 : 4;
  static constexpr int BC = 32 * NW;                   // keys per workgroup
  static constexpr int ROWLEN = SWZ ? D : LDQ;
  static constexpr int QSTAGE = 3 * BQ * ROWLEN;       // Q, gQ, dO elements of one stage
  // floats per row-scalar slot of a stage: SWZ loads a slot with one 4-byte
  // buffer load per lane of a wave, so its slot spans 64 floats (lanes 32..63
  // read past the stage's rows, get zeros, and write them to the padding)
  static constexpr int SLOT = SWZ ? 64 : BQ;
  static constexpr int SSTAGE = 4 * SLOT;              // row scalars of one stage (floats)
  // the LDS-resident key-side tiles (NKLDS per wave, 32 x D each) follow the
  // stage buffers
  static constexpr size_t KSIDE = (size_t)NW * NKLDS * 32 * D * sizeof(T);
  static constexpr size_t STAGE_BYTES = NBUF * (QSTAGE * sizeof(T) + SSTAGE * sizeof(float));
  // (at least the epilogue's 4 KB of output staging per wave)
  static constexpr size_t LDS_BYTES =
      STAGE_BYTES + KSIDE > (size_t)NW * 4096 ? STAGE_BYTES + KSIDE : (size_t)NW * 4096;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ bf16x8 load_key_frag(const bf16* row, bool valid, int c) {
  bf16x8 f = {};
  if (valid) f = *reinterpret_cast<const bf16x8*>(row + 16 * c + 8 * (lane_id() >> 5));
  return f;
}

__device__ __forceinline__ f32x8 load_key_frag(const float* row, bool valid, int c) {
  f32x8 f = {};
  const int h = lane_id() >> 5;
  if (valid) {
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = row[16 * c + Elem<float>::kmap(h, s)];
  }
  return f;
}

// A per-query-row vector of the stage (LDS) laid out as an accumulator: slot
// i holds row acc_row(h, i), i.e. four broadcast reads of 4 consecutive rows.
__device__ __forceinline__ f32x16 rows_as_acc(const float* v) {
  const int h = lane_id() >> 5;
  f32x16 a;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(v + 8 * g + 4 * h);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[4 * g + e] = x[e];
  }
  return a;
}

// Elementwise step of 16-query chunk cc of a 32-query block (slot i <-> query
// row acc_row(h, i), lane <-> key), turned into B operands with k = queries.
// dP, G, H arrive already shifted by their row scalars (the accumulators
// start at -D, -c/s, -r): dP - D, G/s - c/s, H - r. TAIL zeroes P for keys
// past the sequence end and for query rows outside [q_lo, nq_rel) (q_lo: the
// causal mask, query row >= this lane's key; otherwise <= 0).
template <typename T, bool TAIL, bool FIRST>
__device__ __forceinline__ void key_chunk(int cc, const f32x16& S, const f32x16& G, const f32x16& dP,
                                          const f32x16& H, const float* sl, float sl2, float scale, bool kvalid,
                                          int q_lo, int nq_rel, typename Elem<T>::frag& fdS,
                                          typename Elem<T>::frag& fdS2, typename Elem<T>::frag& fA,
                                          typename Elem<T>::frag& fP) {
  const int h = lane_id() >> 5;
  f32x8 dS, dS2, A, P;
#pragma unroll
  for (int gg = 0; gg < 2; ++gg) {
    const int g = 2 * cc + gg;
    const int r0 = 8 * g + 4 * h;  // this lane-half's 4 consecutive query rows
    const f32x4 L4 = *reinterpret_cast<const f32x4*>(sl + r0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * g + e, s = 4 * gg + e;
      float p = fast_exp2(fmaf(S[i], sl2, -L4[e]));
      if (TAIL && (!kvalid || r0 + e >= nq_rel || r0 + e < q_lo)) p = 0.f;
      const float ds = p * dP[i];
      const float gv = G[i] * scale;
      dS[s] = ds;
      A[s] = p * gv;
      dS2[s] = fmaf(ds, gv, p * H[i]);
      if constexpr (FIRST) P[s] = p;
    }
  }
  to_frag(fdS, dS);
  to_frag(fdS2, dS2);
  to_frag(fA, A);
  if constexpr (FIRST) to_frag(fP, P);
}

// The same step for bf16 operands, done in place: the results of chunk cc
// are rounded pair by pair and written back into the tiles' own registers
// (dS into dP, A into G, dS2 into H and, with the first backward, P into S) at
// words 8 cc .. 8 cc + 3: pair s2 reads words 8 cc + 2 s2, + 1 and writes
// word 8 cc + s2, which the same or an earlier pair has already read. The
// chunk's bf16 operand fragments are then those four words of each tile.
template <bool TAIL, bool FIRST>
__device__ __forceinline__ void key_chunk_inplace(int cc, f32x16& S, f32x16& G, f32x16& dP, f32x16& H,
                                                  const float* sl, float sl2, float scale, bool kvalid, int q_lo,
                                                  int nq_rel) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  auto pack = [](float a, float b) __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
  };
  const int h = lane_id() >> 5;
#pragma unroll
  for (int gg = 0; gg < 2; ++gg) {
    const int g = 2 * cc + gg;
    const int r0 = 8 * g + 4 * h;  // this lane-half's 4 consecutive query rows
    const f32x4 L4 = *reinterpret_cast<const f32x4*>(sl + r0);
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      float vds[2], va[2], vd2[2], vp[2];
#pragma unroll
      for (int e1 = 0; e1 < 2; ++e1) {
        const int e = 2 * e2 + e1, i = 4 * g + e;
        float p = fast_exp2(fmaf(S[i], sl2, -L4[e]));
        if (TAIL && (!kvalid || r0 + e >= nq_rel || r0 + e < q_lo)) p = 0.f;
        const float ds = p * dP[i];
        const float gv = G[i] * scale;
        vds[e1] = ds;
        va[e1] = p * gv;
        vd2[e1] = fmaf(ds, gv, p * H[i]);
        vp[e1] = p;
      }
      const int o = 8 * cc + 2 * gg + e2;
      dP[o] = pack(vds[0], vds[1]);
      G[o] = pack(va[0], va[1]);
      H[o] = pack(vd2[0], vd2[1]);
      if constexpr (FIRST) S[o] = pack(vp[0], vp[1]);
    }
  }
}

// Words 8 cc .. 8 cc + 3 of a tile as a bf16 operand fragment.
__device__ __forceinline__ bf16x8 packed_frag(const f32x16& t, int cc) {
  return __builtin_bit_cast(bf16x8, cc == 0 ? __builtin_shufflevector(t, t, 0, 1, 2, 3)
                                            : __builtin_shufflevector(t, t, 8, 9, 10, 11));
}

// FIRST: also return the first-backward dK = s dS^T Q and dV = P^T dO (two
// more products per block against operands already read).
template <typename T, int D, bool FIRST>
__global__ __launch_bounds__((KeyCfg<T, D, FIRST>::NW * 64),
                             ((KeyCfg<T, D, FIRST>::OCC2 ? 2 : 1) * 4 / KeyCfg<T, D, FIRST>::NW)) void key_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const T* __restrict__ gQ, const T* __restrict__ gK, const T* __restrict__ gV,
    const float* __restrict__ lse2, const float* __restrict__ Dv, const float* __restrict__ cv,
    const float* __restrict__ rv, void* __restrict__ gradK, void* __restrict__ gradV, void* __restrict__ dKo,
    void* __restrict__ dVo, int N, int nkblk, float scale, int causal, int G, int out_bf16) {
  using Cfg = KeyCfg<T, D, FIRST>;
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int BQ = Cfg::BQ, LDQ = Cfg::LDQ, NCH = Cfg::NCH, NDB = Cfg::NDB, NBUF = Cfg::NBUF;
  constexpr int ROWLEN = Cfg::ROWLEN;
  constexpr bool SWZ = Cfg::SWZ;
  // [NBUF][3][BQ][ROWLEN] Q, gQ, dO rows, then [NBUF][4][BQ] row scalars.
  // (Addresses are always formed from the __shared__ array itself so that
  // they stay LDS addresses.)
  __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
  auto tile = [&](int b, int t) __attribute__((always_inline)) { return reinterpret_cast<T*>(smem) + (b * 3 + t) * BQ * ROWLEN; };
  auto sQ = [&](int b, int t, int row, int col) __attribute__((always_inline)) { return tile(b, t) + row * ROWLEN + col; };
  auto sS = [&](int b, int t) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(smem + NBUF * Cfg::QSTAGE * sizeof(T)) + (b * 4 + t) * Cfg::SLOT;
  };
  auto lds_rows = [&](int b, int t, int c16) __attribute__((always_inline)) -> F {
    if constexpr (SWZ) return ld_rows_sw(tile(b, t) + 2048 * (c16 >> 2), 0, c16 & 3);
    else return ld_rows(sQ(b, t, 0, 16 * c16), LDQ);
  };
  auto lds_cols = [&](int b, int t, int krow0, int col0) __attribute__((always_inline)) -> F {
    if constexpr (SWZ) return ld_cols_perm_sw(tile(b, t) + 2048 * (col0 >> 6), krow0, col0 & 63);
    else return ld_cols_perm(sQ(b, t, krow0, col0), LDQ);
  };

  // causal: the longest sweeps (the first key blocks) start first, across all
  // key/value heads at once
  // (OSPLIT: consecutive workgroups share a key block and split its output
  // columns; part = which share)
  constexpr int OSPLIT = Cfg::OSPLIT, NDBO = Cfg::NDBO;
  const int part = OSPLIT > 1 ? (int)(blockIdx.x % OSPLIT) : 0;
  const unsigned bid = OSPLIT > 1 ? blockIdx.x / OSPLIT : blockIdx.x;
  const int nheads = (int)((OSPLIT > 1 ? gridDim.x / OSPLIT : gridDim.x) / nkblk);
  const int head = causal ? (int)(bid % nheads) : (int)(bid / nkblk);
  const int kblk = causal ? (int)(bid / nheads) : (int)(bid % nkblk);
  // key/value head `head`; the query heads of its group are head * G + g
  const size_t hoff = (size_t)head * N * D;
  size_t qoff = 0, soff = 0;  // query head of the current group member
  // the row scalar this wave (SWZ) or thread (otherwise) stages, of that member
  const float* stat_src = nullptr;
  const int w = wave_id(), l = lane_id(), h = l >> 5, col = l & 31;
  const int key = kblk * Cfg::BC + 32 * w + col;  // this lane's key
  const bool kvalid = key < N;
  const bool ktail = kblk * Cfg::BC + Cfg::BC > N;
  // LDS tile of key-side tensor t (a KLDS member)
  auto ktile = [&](int t) __attribute__((always_inline)) {
    const int slot = __builtin_popcount(Cfg::KLDS & ((1 << t) - 1));
    return reinterpret_cast<T*>(smem + Cfg::STAGE_BYTES) + (w * Cfg::NKLDS + slot) * 32 * D;
  };

  // B operands of the wave's 32 keys (lane <-> key, k over d): registers, or
  // (KLDS members) this wave's LDS tiles, which keeps the kernel within its
  // register budget
  constexpr int KLDS = Cfg::KLDS;
  F bK[(KLDS & 1) ? 1 : NCH], bgK[(KLDS & 2) ? 1 : NCH], bV[(KLDS & 4) ? 1 : NCH], bgV[(KLDS & 8) ? 1 : NCH];
  {
    const int k0w = kblk * Cfg::BC + 32 * w;
    const int nkw = max(1, min(32, N - k0w));  // waves wholly past the end copy row N-1 (masked)
    const size_t rw = hoff + (size_t)min(k0w, N - 1) * D;
    const size_t ro = hoff + (size_t)key * D;
    const T* const srcs[4] = {K, gK, V, gV};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (SWZ) {
        if (KLDS & (1 << t)) load_tile_sw_wave(ktile(t), srcs[t] + rw, nkw);
      }
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if constexpr (!(KLDS & 1)) bK[c] = load_key_frag(K + ro, kvalid, c);
      if constexpr (!(KLDS & 2)) bgK[c] = load_key_frag(gK + ro, kvalid, c);
      if constexpr (!(KLDS & 4)) bV[c] = load_key_frag(V + ro, kvalid, c);
      if constexpr (!(KLDS & 8)) bgV[c] = load_key_frag(gV + ro, kvalid, c);
    }
  }
  auto keyop = [&](int t, int c) __attribute__((always_inline)) -> F {
    if constexpr (SWZ) {
      if (KLDS & (1 << t)) return ld_rows_sw(ktile(t), 0, c);
    }
    return t == 0 ? bK[(KLDS & 1) ? 0 : c]
                  : t == 1 ? bgK[(KLDS & 2) ? 0 : c] : t == 2 ? bV[(KLDS & 4) ? 0 : c] : bgV[(KLDS & 8) ? 0 : c];
  };
  // gradK^T, gradV^T: d rows x the wave's 32 keys
  f32x16 accK[NDBO], accV[NDBO], accdK[FIRST ? NDBO : 1], accdV[FIRST ? NDBO : 1];
#pragma unroll
  for (int j = 0; j < NDBO; ++j) {
    accK[j] = f32x16{};
    accV[j] = f32x16{};
    if constexpr (FIRST) {
      accdK[j] = f32x16{};
      accdV[j] = f32x16{};
    }
  }
  const float sl2 = scale * kLog2e;
  const int nblk = (N + BQ - 1) / BQ;  // 32-query blocks = stages

  // staging of stage n (Q, gQ, dO rows and their row scalars)
  RowPrefetch<T, SWZ ? 0 : BQ, D, 256> pq, pg, pd;
  float pstat = 0.f;
  auto prefetch = [&](int n) __attribute__((always_inline)) {
    const int q0 = n * BQ;
    const int nq = min(BQ, N - q0);
    if constexpr (SWZ) {
      const int b = n & (NBUF - 1);
      if constexpr (Cfg::NW == 8) {
        // wave w: rows 8 (w % 4) .. + 7 of Q and dO (w < 4), or of gQ and
        // row scalar w % 4 (w >= 4)
        const int rg = w & 3;
        if (w < 4) {
          load_rows8_sw(tile(b, 0), Q + qoff + (size_t)q0 * D, nq, rg);
          load_rows8_sw(tile(b, 2), dO + qoff + (size_t)q0 * D, nq, rg);
        } else {
          load_rows8_sw(tile(b, 1), gQ + qoff + (size_t)q0 * D, nq, rg);
        }
      } else if constexpr (D == 64) {
        load_tile_sw(tile(b, 0), Q + qoff + (size_t)q0 * D, nq);
        load_tile_sw(tile(b, 1), gQ + qoff + (size_t)q0 * D, nq);
        load_tile_sw(tile(b, 2), dO + qoff + (size_t)q0 * D, nq);
      } else {
        const T* const src[3] = {Q, gQ, dO};
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
          for (int hf = 0; hf < D / 64; ++hf)
            load_half_sw(tile(b, t), src[t] + qoff + (size_t)q0 * D, nq, D * (int)sizeof(T), hf);
      }
      // wave w (four waves) or w + 4 (eight) fetches row scalar w
      // (LSE*log2e, -D, -c/s, -r) of the stage's queries: lane L -> row L,
      // written at LDS float L of sS(b, w); rows past the end (and lanes
      // 32..63) read as zero
      typedef __attribute__((address_space(3))) void lds_void;
      auto load_scalars = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_rsrc(stat_src + q0, nq * 4), (lds_void*)sS(b, w & 3), 4,
                                                 4 * l, 0, 0, 0);
      };
      if constexpr (Cfg::NW == 4)
        load_scalars();
      else if (w >= 4)
        load_scalars();
    } else {
      pq.load(Q + qoff + (size_t)q0 * D, nq);
      pg.load(gQ + qoff + (size_t)q0 * D, nq);
      pd.load(dO + qoff + (size_t)q0 * D, nq);
      // thread -> (scalar (tid / BQ) % 4, row tid % BQ); threads 128..255 repeat
      // 0..127 (same values to the same LDS slots), so there is no branch.
      // Queries past the end get LSE = +inf (hence P = 0) and zero scalars;
      // the row index is clamped so every load stays in bounds.
      const int i = threadIdx.x % BQ;
      const float v = stat_src[q0 + min(i, nq - 1)];
      pstat = i < nq ? v : (((threadIdx.x / BQ) & 3) == 0 ? INFINITY : 0.f);
    }
  };
  auto commit = [&](int n) __attribute__((always_inline)) {
    if constexpr (SWZ) {
      wait_vmem();
    } else {
      const int b = n & (NBUF - 1);
      pq.store(sQ(b, 0, 0, 0), LDQ);
      pg.store(sQ(b, 1, 0, 0), LDQ);
      pd.store(sQ(b, 2, 0, 0), LDQ);
      sS(b, (threadIdx.x / BQ) & 3)[threadIdx.x % BQ] = pstat;
    }
  };

  struct Tiles {
    f32x16 S, G, dP, H;
  };
  // d-chunks [c0, c1) of S, G/s - c/s, dP - D, H - r of query block n
  // (queries x this wave's keys): the accumulators start from the stage's row
  // scalars
  auto recompute = [&](int n, Tiles& t, int c0, int c1) __attribute__((always_inline)) {
    const int b = n & (NBUF - 1);
    if (c0 == 0) {
      t.S = f32x16{};
      t.dP = rows_as_acc(sS(b, 1));
      t.G = rows_as_acc(sS(b, 2));
      t.H = rows_as_acc(sS(b, 3));
    }
#pragma unroll
    for (int c = c0; c < c1; ++c) {
      const F aq = lds_rows(b, 0, c);  // lane <-> query, k over d
      const F agq = lds_rows(b, 1, c);
      const F ado = lds_rows(b, 2, c);
      const F k = keyop(0, c);
      E::mma(t.S, aq, k);
      E::mma(t.G, agq, k);
      E::mma(t.G, aq, keyop(1, c));
      E::mma(t.dP, ado, keyop(2, c));
      E::mma(t.H, ado, keyop(3, c));
    }
  };
  // bf16 packs the operand fragments into the score tiles' own registers
  // (key_chunk_inplace); fp32 keeps them apart
  constexpr bool INPLACE = sizeof(T) == 2;
  struct Frags {
    F dS[2], dS2[2], A[2], P[FIRST ? 2 : 1];
  };
  // TAIL: masks keys past the end (the whole sweep of the last key block)
  // and query rows past the end (last query block)
  auto elementwise = [&](auto tail, int n, int cc, Tiles& t, Frags& f) __attribute__((always_inline)) {
    constexpr bool TAIL = decltype(tail)::value;
    const int b = n & (NBUF - 1);
    if constexpr (INPLACE)
      key_chunk_inplace<TAIL, FIRST>(cc, t.S, t.G, t.dP, t.H, sS(b, 0), sl2, scale, kvalid,
                                     causal ? key - n * BQ : 0, N - n * BQ);
    else
      key_chunk<T, TAIL, FIRST>(cc, t.S, t.G, t.dP, t.H, sS(b, 0), sl2, scale, kvalid, causal ? key - n * BQ : 0,
                                N - n * BQ, f.dS[cc], f.dS2[cc], f.A[cc], f.P[FIRST ? cc : 0]);
  };
  auto outputs = [&](int n, int cc, const Tiles& t, const Frags& f0) __attribute__((always_inline)) {
    const int b = n & (NBUF - 1);
    Frags f;
    if constexpr (INPLACE) {
      f.dS[cc] = packed_frag(t.dP, cc);
      f.dS2[cc] = packed_frag(t.H, cc);
      f.A[cc] = packed_frag(t.G, cc);
      if constexpr (FIRST) f.P[cc] = packed_frag(t.S, cc);
    } else {
      f = f0;
    }
#pragma unroll
    for (int j = 0; j < NDBO; ++j) {
      // lane <-> d, k over this chunk's queries (accumulator row order); this
      // workgroup's share of the columns starts at block part * NDBO
      const int jd = 32 * (part * NDBO + j);
      const F tQ = lds_cols(b, 0, 16 * cc, jd);
      const F tgQ = lds_cols(b, 1, 16 * cc, jd);
      const F tdO = lds_cols(b, 2, 16 * cc, jd);
      E::mma(accK[j], tQ, f.dS2[cc]);
      E::mma(accK[j], tgQ, f.dS[cc]);
      E::mma(accV[j], tdO, f.A[cc]);
      if constexpr (FIRST) {
        E::mma(accdK[j], tQ, f.dS[cc]);
        E::mma(accdV[j], tdO, f.P[cc]);
      }
    }
  };

  // Query blocks visited: causal starts at the block of the workgroup's
  // first key (queries before it see none of these keys) and masks the
  // BC / BQ blocks across the diagonal; the rest see every key.
  const int nstart = causal ? kblk * (Cfg::BC / BQ) : 0;  // even
  const int ndiag = causal ? min(nblk, nstart + Cfg::BC / BQ) : 0;

  using F0 = std::integral_constant<bool, false>;
  using F1 = std::integral_constant<bool, true>;
  const bool last_partial = N % BQ != 0;
  Tiles t;
  Frags f;
  // sweep the queries of each member of the key/value head's group in turn
  // (gradK, gradV sum over them)
  for (int g = 0; g < G; ++g) {
    qoff = (size_t)(head * G + g) * N * D;
    soff = (size_t)(head * G + g) * N;
    {
      const int si = SWZ ? (w & 3) : (int)(threadIdx.x / BQ) & 3;
      stat_src = (si == 0 ? lse2 : si == 1 ? Dv : si == 2 ? cv : rv) + soff;
    }
    prefetch(nstart);  // nstart < nblk; the previous member's last barrier freed both buffers
    commit(nstart);
    __syncthreads();
    // Blocks in ascending order. The masked ones take the masked elementwise
    // path: the causal diagonal [nstart, ndiag), a partial last query block,
    // and every block of a partial key block (ktail). The unmasked stretch
    // between them runs as a branch-free pair loop (no mask test, the next
    // stage always prefetched), so each pair is one straight-line block the
    // scheduler can interleave.
    const int mask_end = ktail ? nblk : min(ndiag, nblk);  // masked head [nstart, mask_end)
    const int clean_end = ktail ? nblk : max(mask_end, nblk - (last_partial ? 1 : 0));  // unmasked up to here
    // one 32-query block n: TAIL selects the masked path, PF prefetches stage
    // n + 1 (into the buffer that last held stage n - 1, read in block n - 1)
#define FLASHBOB_KEY_BLOCK(n, TAIL, PF)               \
  {                                                   \
    if (PF) prefetch((n) + 1);                        \
    recompute((n), t, 0, NCH);                        \
    _Pragma("unroll") for (int cc = 0; cc < 2; ++cc) { \
      elementwise(TAIL, (n), cc, t, f);               \
      outputs((n), cc, t, f);                         \
    }                                                 \
    if (PF) commit((n) + 1);                          \
    __syncthreads();                                  \
  }
    for (int n = nstart; n < mask_end; ++n) FLASHBOB_KEY_BLOCK(n, F1{}, n + 1 < nblk)
    // pairs from the even mask_end, so the stage buffer index of each half is a
    // compile-time constant; both halves have a next stage
    int i = mask_end >> 1;
    for (; 2 * i + 2 <= clean_end && 2 * i + 2 < nblk; ++i) {
      FLASHBOB_KEY_BLOCK(2 * i, F0{}, true)
      FLASHBOB_KEY_BLOCK(2 * i + 1, F0{}, true)
    }
    // the rest of the unmasked stretch (at most two blocks; mask_end is odd only
    // when the masked head runs to nblk, and then this stretch is empty)
    for (int n = max(2 * i, mask_end); n < clean_end; ++n) FLASHBOB_KEY_BLOCK(n, F0{}, n + 1 < nblk)
    if (!ktail && last_partial && nblk - 1 >= mask_end) FLASHBOB_KEY_BLOCK(nblk - 1, F1{}, false)
#undef FLASHBOB_KEY_BLOCK
  }

  // accK[j] slot i holds d = 32 j + acc_row(h, i) of this lane's key; each
  // 32 x 32 block goes out through LDS (free: the last block ended with a
  // barrier and prefetched nothing)
  static_assert(Cfg::LDS_BYTES >= (size_t)Cfg::NW * 4096, "output staging fits the LDS");
  float* xs = reinterpret_cast<float*>(smem) + 1024 * w;
  const int k0w = kblk * Cfg::BC + 32 * w;  // the wave's first key
  const size_t base = hoff + (size_t)k0w * D;
  const int nrows = min(32, N - k0w);
#pragma unroll
  for (int j = 0; j < NDBO; ++j) {
    const int col0 = 32 * (part * NDBO + j);
    store_block_lds(xs, accK[j], scale, gradK, base, D, col0, nrows, out_bf16);
    store_block_lds(xs, accV[j], 1.f, gradV, base, D, col0, nrows, out_bf16);
    if constexpr (FIRST) {
      store_block_lds(xs, accdK[j], scale, dKo, base, D, col0, nrows, out_bf16);
      store_block_lds(xs, accdV[j], 1.f, dVo, base, D, col0, nrows, out_bf16);
    }
  }
}

template <typename T, int D, bool FIRST>
hipError_t launch_key(const void* Q, const void* K, const void* V, const void* dO, const void* gQ, const void* gK,
                      const void* gV, const float* lse2, const float* Dv, const float* cv, const float* rv,
                      void* gradK, void* gradV, void* dK, void* dV, int BHkv, int N, float scale, int causal,
                      int G, int out_bf16, hipStream_t stream) {
  using Cfg = KeyCfg<T, D, FIRST>;
  const int nkblk = (N + Cfg::BC - 1) / Cfg::BC;
  const long long nblocks = (long long)nkblk * BHkv * Cfg::OSPLIT;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  key_kernel<T, D, FIRST><<<dim3((unsigned)nblocks), dim3(Cfg::NW * 64), 0, stream>>>(
      (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, (const T*)gQ, (const T*)gK, (const T*)gV, lse2, Dv, cv,
      rv, gradK, gradV, dK, dV, N, nkblk, scale, causal, G, out_bf16);
  return hipGetLastError();
}

#define FLASHBOB_INST_KEY(T, D, F)                                                                         \
  template hipError_t launch_key<T, D, F>(const void*, const void*, const void*, const void*, const void*, \
                                          const void*, const void*, const float*, const float*,             \
                                          const float*, const float*, void*, void*, void*, void*, int, int, \
                                          float, int, int, int, hipStream_t);
#define FLASHBOB_INST_KEY_DIMS(F) \
  FLASHBOB_INST_KEY(bf16, 32, F)  \
  FLASHBOB_INST_KEY(bf16, 64, F)  \
  FLASHBOB_INST_KEY(bf16, 96, F)  \
  FLASHBOB_INST_KEY(bf16, 128, F) \
  FLASHBOB_INST_KEY(bf16, 256, F) \
  FLASHBOB_INST_KEY(float, 32, F) \
  FLASHBOB_INST_KEY(float, 64, F) \
  FLASHBOB_INST_KEY(float, 96, F) \
  FLASHBOB_INST_KEY(float, 128, F)
FLASHBOB_INST_KEY_DIMS(false)
FLASHBOB_INST_KEY_DIMS(true)

}  // namespace flashbob
