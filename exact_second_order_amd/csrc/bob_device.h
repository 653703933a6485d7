// Device building blocks for the gfx950 (CDNA4) BoB kernels: MFMA fragment
// types, LDS fragment loaders, exp2, wave exchange. Every kernel works on
// 32 x 32 output blocks held in the v_mfma_f32_32x32x* accumulator layout:
//
//   lane l, accumulator slot i  ->  row 8*(i/4) + 4*(l/32) + (i%4),  col l%32
//
// An operand "fragment" is one 32-row x 16-k slab of an A or B operand, eight
// values per lane: lane l holds row (A) or column (B) l%32 and the k indices
//   bf16 (one v_mfma_f32_32x32x16_bf16):       k = 8*(l/32) + s,  s = 0..7
//   fp32 (eight v_mfma_f32_32x32x2f32 steps):  k = 2*s + (l/32), s = 0..7
// Both operands of a product use the same k mapping, so a fragment pair
// always contracts the right k indices together.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flashbob {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __bf16 bf16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// (read from the first lane, so that it and everything derived from it stays
// in scalar registers)
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Row of the accumulator layout held by (lane half h, slot i).
__device__ __forceinline__ constexpr int acc_row(int h, int i) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// ---------------------------------------------------------------------------
// element type traits: fragment type, MFMA, conversions

template <typename T>
struct Elem;

template <>
struct Elem<bf16> {
  using frag = bf16x8;
  static constexpr int kmap(int h, int s) { return 8 * h + s; }
  __device__ __forceinline__ static void mma(f32x16& c, const frag& a, const frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static float to_f32(bf16 x) { return (float)x; }
  __device__ __forceinline__ static bf16 from_f32(float x) { return (bf16)x; }
};

template <>
struct Elem<float> {
  using frag = f32x8;
  static constexpr int kmap(int h, int s) { return 2 * s + h; }
  __device__ __forceinline__ static void mma(f32x16& c, const frag& a, const frag& b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], c, 0, 0, 0);
  }
  __device__ __forceinline__ static float to_f32(float x) { return x; }
  __device__ __forceinline__ static float from_f32(float x) { return x; }
};

// ---------------------------------------------------------------------------
// LDS fragment loads.
//
// ld_rows: the matrix is stored with the fragment's row index as the storage
//   row and k along the storage row: lane reads row l%32 at columns kmap.
// ld_cols: the matrix is stored with k as the storage row and the fragment's
//   row/column index along the storage row (the transposed case).
// `p` points at element [row0][k0] (ld_rows) or [k0][col0] (ld_cols); `ld` is
// the storage row stride in elements.

__device__ __forceinline__ bf16x8 ld_rows(const bf16* p, int ld) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x8*>(p + (l & 31) * ld + 8 * (l >> 5));
}

__device__ __forceinline__ f32x8 ld_rows(const float* p, int ld) {
  const int l = lane_id();
  const float* q = p + (l & 31) * ld + (l >> 5);
  f32x8 v;
#pragma unroll
  for (int s = 0; s < 8; ++s) v[s] = q[2 * s];
  return v;
}

// gfx950 ds_read_b64_tr_b16: inside each group of 16 lanes, lane i's slot e
// receives element i%4 of the 8-byte read issued by lane 4*e + i/4. Lane j of
// a group therefore reads storage row k0 + j/4 at columns c0 + 4*(j%4) .. +3,
// and lane i ends up with column c0 + i at storage rows k0 .. k0+3.
__device__ __forceinline__ bf16x8 ld_cols(const bf16* p, int ld) {
  const int l = lane_id();
  const int g = l >> 4, j = l & 15;
  const int col = 16 * (g & 1) + 4 * (j & 3);
  const int krow = 8 * (g >> 1) + (j >> 2);
  const bf16* a0 = p + krow * ld + col;
  const bf16* a1 = a0 + 4 * ld;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a1));
  // whole-vector reinterpretation (no per-element bf16 accesses)
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x8 ld_cols(const float* p, int ld) {
  const int l = lane_id();
  const float* q = p + (l >> 5) * ld + (l & 31);
  f32x8 v;
#pragma unroll
  for (int s = 0; s < 8; ++s) v[s] = q[2 * s * ld];
  return v;
}

// ---------------------------------------------------------------------------
// Accumulator blocks as MFMA operands.
//
// A 32 x 32 accumulator block C (rows = the contraction index of the next
// product) can feed the next MFMA as its B operand without leaving registers:
// 16-row chunk cc of C is held by slots 8*cc .. 8*cc+7, and slot s of lane
// half h is row 16*cc + kperm(h, s). The other operand of that product must
// present its k index in the same order, which ld_cols_perm does.

__device__ __forceinline__ constexpr int kperm(int h, int s) { return 8 * (s >> 2) + 4 * h + (s & 3); }

// Chunk cc of an accumulator block as an operand fragment (values rounded to
// the element type).
__device__ __forceinline__ f32x8 acc_chunk(const f32x16& c, int cc) {
  return cc == 0 ? __builtin_shufflevector(c, c, 0, 1, 2, 3, 4, 5, 6, 7)
                 : __builtin_shufflevector(c, c, 8, 9, 10, 11, 12, 13, 14, 15);
}

__device__ __forceinline__ void acc_to_frag(bf16x8& f, const f32x16& c, int cc) {
  f = __builtin_convertvector(acc_chunk(c, cc), bf16x8);  // round to nearest even
}

__device__ __forceinline__ void acc_to_frag(f32x8& f, const f32x16& c, int cc) { f = acc_chunk(c, cc); }

// Eight fp32 values (one accumulator chunk) as an operand fragment.
__device__ __forceinline__ void to_frag(bf16x8& f, const f32x8& v) { f = __builtin_convertvector(v, bf16x8); }
__device__ __forceinline__ void to_frag(f32x8& f, const f32x8& v) { f = v; }

// Like ld_cols (storage rows = k), but slot s of lane half h holds storage row
// kperm(h, s): rows 4h..4h+3 and 8+4h..8+4h+3 of the 16-row chunk.
__device__ __forceinline__ bf16x8 ld_cols_perm(const bf16* p, int ld) {
  const int l = lane_id();
  const int g = l >> 4, j = l & 15;
  const int col = 16 * (g & 1) + 4 * (j & 3);
  const int krow = 4 * (g >> 1) + (j >> 2);
  const bf16* a0 = p + krow * ld + col;
  const bf16* a1 = a0 + 8 * ld;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a1));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x8 ld_cols_perm(const float* p, int ld) {
  const int l = lane_id();
  const int h = l >> 5;
  const float* q = p + (l & 31);
  f32x8 v;
#pragma unroll
  for (int s = 0; s < 8; ++s) v[s] = q[kperm(h, s) * ld];
  return v;
}

// ---------------------------------------------------------------------------
// Swizzled 32 x 64 bf16 stage tiles (128-byte rows, no padding).
//
// The 16-byte chunk c of row r is stored at chunk position c ^ swz(r). swz
// gives rows of equal parity 8 distinct positions (so 16 lanes reading one
// column chunk of 16 rows hit 64 distinct banks) and puts rows r and r + 2 in
// different 64-byte halves (so the 4-row x 32-byte footprint of a transpose
// read is conflict free as well).

__device__ __forceinline__ constexpr int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ const bf16* sw_addr(const bf16* t, int row, int col) {
  return t + row * 64 + 8 * ((col >> 3) ^ swz(row)) + (col & 7);
}

// ld_rows on a swizzled tile: lane reads row row0 + l%32 at k = 16*c16 + kmap.
__device__ __forceinline__ bf16x8 ld_rows_sw(const bf16* t, int row0, int c16) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x8*>(sw_addr(t, row0 + (l & 31), 16 * c16 + 8 * (l >> 5)));
}

// ld_cols_perm on a swizzled tile: storage rows krow0 .. krow0+15 are k (in
// kperm order), lane reads column col0 + l%32.
__device__ __forceinline__ bf16x8 ld_cols_perm_sw(const bf16* t, int krow0, int col0) {
  const int l = lane_id();
  const int g = l >> 4, j = l & 15;
  const int col = col0 + 16 * (g & 1) + 4 * (j & 3);
  const int kr = krow0 + 4 * (g >> 1) + (j >> 2);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)sw_addr(t, kr, col));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)sw_addr(t, kr + 8, col));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Raw buffer resource over `bytes` bytes at p: loads at byte offsets past the
// end return zero. (Word 3 is the gfx9-family raw-buffer format.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Direct global -> LDS copy of a 32 x 64 bf16 tile into swizzled layout, one
// buffer_load_dwordx4 ... lds per wave: wave w fills rows 8w .. 8w+7 (the
// hardware writes lane L's 16 bytes at LDS chunk L of the wave's window, so
// lane L fetches the global chunk that belongs there). The source is a buffer
// of `nvalid` rows, so rows at or past nvalid arrive as zeros (callers mask
// them); the per-lane offset is loop-invariant and the rest is scalar.
__device__ __forceinline__ void load_tile_sw(bf16* t, const bf16* src, int nvalid) {
  const int l = lane_id(), w = wave_id();
  const int row = 8 * w + (l >> 3);
  const int c = (l & 7) ^ swz(row);
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_rsrc(src, nvalid * 128), (lds_void*)(t + 8 * w * 64), 16,
                                           row * 128 + 16 * c, 0, 0, 0);
}

// The same copy for one 64-column half of a 32-row tile of a tensor with
// `pitch` bytes per row (d = 128: two such halves make a stage tile, 2048
// elements apart): wave w fills rows 8w .. 8w+7 of the half starting at
// column 64 * half. Rows at or past nvalid arrive as zeros.
__device__ __forceinline__ void load_half_sw(bf16* t, const bf16* src, int nvalid, int pitch, int half) {
  const int l = lane_id(), w = wave_id();
  const int row = 8 * w + (l >> 3);
  const int c = (l & 7) ^ swz(row);
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_rsrc(src + 64 * half, nvalid * pitch),
                                           (lds_void*)(t + 2048 * half + 8 * w * 64), 16, row * pitch + 16 * c, 0,
                                           0, 0);
}

// Rows 8 rg .. 8 rg + 7 of the same swizzled 32 x 64 tile by one direct
// global -> LDS load of the calling wave (for workgroups of more than four
// waves, which split a stage's tiles differently); rows at or past nvalid
// arrive as zeros (nvalid = 0: no memory access at all).
__device__ __forceinline__ void load_rows8_sw(bf16* t, const bf16* src, int nvalid, int rg) {
  const int l = lane_id();
  const int row = 8 * rg + (l >> 3);
  const int c = (l & 7) ^ swz(row);
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_rsrc(src, nvalid * 128), (lds_void*)(t + 8 * rg * 64), 16,
                                           row * 128 + 16 * c, 0, 0, 0);
}

// The same copy of a 32 x 64 tile done by one wave alone (4 loads).
__device__ __forceinline__ void load_tile_sw_wave(bf16* t, const bf16* src, int nvalid) {
  const int l = lane_id();
  typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = 8 * p + (l >> 3);
    const int c = (l & 7) ^ swz(row);
    const int srow = row < nvalid ? row : nvalid - 1;
    __builtin_amdgcn_global_load_lds((const void*)(src + srow * 64 + 8 * c), (lds_void*)(t + 8 * p * 64), 16,
                                     0, 0);
  }
}

// Negate an operand fragment in place (sign bits only, exact).
__device__ __forceinline__ void negate(bf16x8& f) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  f = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, f) ^ 0x80008000u);
}
__device__ __forceinline__ void negate(f32x8& f) {
  typedef unsigned u32x8 __attribute__((ext_vector_type(8)));
  f = __builtin_bit_cast(f32x8, __builtin_bit_cast(u32x8, f) ^ 0x80000000u);
}

// Multiply every element by a power of two a. Only the exponent changes, so
// the result is exact unless it falls below the normal range (2^-126), where
// it is rounded and stays negligible beside any normal term.
__device__ __forceinline__ void scale_frag(bf16x8& f, float a) {
  typedef float f32x8v __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
  const f32x8v x = __builtin_convertvector(__builtin_bit_cast(bf16x8v, f), f32x8v) * a;
  f = __builtin_bit_cast(bf16x8, __builtin_convertvector(x, bf16x8v));
}

// Wait for this wave's outstanding global loads, including direct-to-LDS ones.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Store four consecutive elements (one accumulator slot group) to LDS.
__device__ __forceinline__ void st4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}

__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}

// Store four consecutive output elements at element index i of an output
// tensor held in float32, or in bf16 (rounded to nearest even) when bf16out.
__device__ __forceinline__ void store_out4(void* base, size_t i, float a, float b, float c, float d, int bf16out) {
  if (bf16out)
    st4(static_cast<bf16*>(base) + i, a, b, c, d);
  else
    st4(static_cast<float*>(base) + i, a, b, c, d);
}

// Store one 32 x 32 output block of a wave (32 rows: this lane's row l % 32;
// 32 columns col0 .. col0 + 31, slot i of the lane half h holding column
// col0 + acc_row(h, i)) times `os`, through the wave's 4 KB of LDS `xs`, so
// each global store instruction writes whole rows of the block (eight lanes
// per 128-byte row) instead of 16 bytes in each of 64 rows: partially written
// cache lines that every workgroup leaves at once otherwise reach HBM more
// than once. Rows at or past nrows are not stored. Contains workgroup
// barriers: every wave of the workgroup calls it the same number of times,
// with the LDS free.
__device__ __forceinline__ void store_block_lds(float* xs, const f32x16& a, float os, void* out, size_t base,
                                                int ld, int col0, int nrows, int bf16out) {
  typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
  const int l = lane_id(), r = l & 31, h = l >> 5;
  // 16-byte chunk k of row r at position k ^ (r & 7): conflict-free both ways
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int k = 2 * g + h;
    const f32x4_t v = {os * a[4 * g], os * a[4 * g + 1], os * a[4 * g + 2], os * a[4 * g + 3]};
    *reinterpret_cast<f32x4_t*>(xs + 32 * r + 4 * (k ^ (r & 7))) = v;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = 8 * it + (l >> 3), k = l & 7;
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(xs + 32 * row + 4 * (k ^ (row & 7)));
    if (row < nrows) store_out4(out, base + (size_t)row * ld + col0 + 4 * k, v[0], v[1], v[2], v[3], bf16out);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// global -> LDS row copies (16 bytes per lane per step), zero rows past `nrows`

// Register-staged copy of a [ROWS][COLS] row block (16 bytes per lane per
// step): load() issues the global reads early, store() writes LDS later, so
// the global latency hides behind the work done in between.
template <typename T, int ROWS, int COLS, int NTHREADS>
struct RowPrefetch {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int VPR = COLS / VEC;
  static_assert(COLS % VEC == 0, "rows are whole 16-byte vectors");
  static constexpr int TOTAL = ROWS * VPR;                     // vectors to copy
  static constexpr int NIT = (TOTAL + NTHREADS - 1) / NTHREADS;  // ROWS = 0: unused placeholder
  // whether the steps do not split evenly (d = 32, 96 in bf16): the surplus
  // steps then repeat real ones (index mod TOTAL), storing the same values to
  // the same LDS slots, so no step needs a guard
  static constexpr bool RAGGED = TOTAL % NTHREADS != 0;
  __device__ __forceinline__ static int step_index(int it) {
    const int idx = it * NTHREADS + (int)threadIdx.x;
    return RAGGED ? idx % TOTAL : idx;
  }
  typedef __attribute__((__vector_size__(16))) int v4i;
  v4i r[NIT > 0 ? NIT : 1];

  // Raw buffer loads over the valid rows only: rows past nrows_valid read as
  // zero without a branch, so the caller's loop body stays one basic block.
  __device__ __forceinline__ void load(const T* src, int nrows_valid) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, nrows_valid * COLS * (int)sizeof(T));
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = step_index(it);
      const int row = idx / VPR, cv = idx % VPR;
      r[it] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                          rs, (row * COLS + cv * VEC) * (int)sizeof(T), 0, 0));
    }
  }
  __device__ __forceinline__ void store(T* dst, int ldd) const {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = step_index(it);
      const int row = idx / VPR, cv = idx % VPR;
      *reinterpret_cast<v4i*>(dst + row * ldd + cv * VEC) = r[it];
    }
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace flashbob
