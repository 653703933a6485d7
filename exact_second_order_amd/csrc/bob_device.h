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
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

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

// ---------------------------------------------------------------------------
// global -> LDS row copies (16 bytes per lane per step), zero rows past `nrows`

template <typename T, int ROWS, int COLS, int NTHREADS>
__device__ __forceinline__ void copy_rows_to_lds(T* dst, int ldd, const T* src, int nrows_valid) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int VPR = COLS / VEC;  // vectors per row
  constexpr int TOTAL = ROWS * VPR;
  static_assert(TOTAL % NTHREADS == 0, "copy must split evenly over the workgroup");
  typedef __attribute__((__vector_size__(16))) int v4i;
#pragma unroll
  for (int it = 0; it < TOTAL / NTHREADS; ++it) {
    const int idx = it * NTHREADS + (int)threadIdx.x;
    const int r = idx / VPR, cv = idx % VPR;
    v4i v = {0, 0, 0, 0};
    if (r < nrows_valid) v = *reinterpret_cast<const v4i*>(src + (size_t)r * COLS + cv * VEC);
    *reinterpret_cast<v4i*>(dst + r * ldd + cv * VEC) = v;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace flashbob
