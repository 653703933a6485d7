// Operand preparation for the bf16 d = 64 pass-2 kernels: row-transposed
// copies of the [rows][64] tensors that the output products contract (K, gK,
// V, gV for the query side; Q, gQ, dO for the key side).
//
// The output products of pass 2 contract a score-derived tile (held in the
// MFMA accumulator layout, k = the rows of the sweep's block) against the
// other side's rows, so their A operands need 8 rows of one column per lane.
// From a row-major tile that is a transpose read (ds_read_b64_tr_b16: 8 bytes
// per lane); from these copies (layout of tposed_pos) it is one 16-byte read,
// half the LDS instructions and twice the LDS bandwidth per instruction.
// Rows at or past the sequence end are stored as zeros.

#include "bob_device.h"

namespace flashbob {

// Source and destination tensors of one launch (kernel argument, by value).
struct TposeArgs {
  const bf16* src[7];
  bf16* dst[7];
};

// One workgroup per (32-row block, slice, tensor): stage the block through LDS
// and write it out in the layout of tposed_pos, 16 bytes per thread.
__global__ __launch_bounds__(256) void transpose_blocks_kernel(TposeArgs a, int N, int nblk) {
  __shared__ __attribute__((aligned(16))) bf16 tile[32 * 64];
  const int blk = blockIdx.x, slice = blockIdx.y, t = blockIdx.z;
  // (uniform select, so the argument table is read with scalar loads)
  const bf16* sp = a.src[0];
  bf16* dp = a.dst[0];
#pragma unroll
  for (int i = 1; i < 7; ++i)
    if (t == i) {
      sp = a.src[i];
      dp = a.dst[i];
    }
  const bf16* s = sp + (size_t)slice * N * 64;
  bf16* o = dp + ((size_t)slice * nblk + blk) * 2048;
  const int tid = threadIdx.x;
  {
    const int r = tid >> 3, c8 = (tid & 7) * 8;  // 8 elements of row r
    const int row = blk * 32 + r;
    typedef __attribute__((__vector_size__(16))) int v4i;
    v4i v = {};
    if (row < N) v = *reinterpret_cast<const v4i*>(s + (size_t)row * 64 + c8);
    *reinterpret_cast<v4i*>(tile + r * 64 + c8) = v;
  }
  __syncthreads();
  // thread tid writes elements [8 tid, 8 tid + 8) of the output block: the
  // 8 rows kperm(h, 0..7) of chunk cc at column d (tposed_pos inverted)
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int idx = 8 * tid + e;
    const int cc = idx >> 10, d = (idx >> 4) & 63, pos = idx & 15;
    const int hh = pos >> 3, sl = pos & 7;
    const int h = hh ^ ((d >> 3) & 1);  // position 8 hh + sl = tposed_pos(cc, d, h, sl) - base
    const int k = kperm(h, sl);
    v[e] = tile[(16 * cc + k) * 64 + d];
  }
  *reinterpret_cast<bf16x8*>(o + 8 * tid) = v;
}

// Transposed copies of n (1..7) tensors of `slices` [N][64] slices each;
// dst[i] receives slices * ceil(N / 32) blocks of 2048 elements.
hipError_t launch_transpose_blocks(const bf16* const* src, bf16* const* dst, int n, int slices, int N,
                                   hipStream_t stream) {
  if (n <= 0 || n > 7 || slices <= 0 || N <= 0) return hipSuccess;
  if (slices > 65535) return hipErrorInvalidConfiguration;
  const int nblk = (N + 31) / 32;
  TposeArgs a{};
  for (int i = 0; i < n; ++i) {
    a.src[i] = src[i];
    a.dst[i] = dst[i];
  }
  transpose_blocks_kernel<<<dim3((unsigned)nblk, (unsigned)slices, (unsigned)n), dim3(256), 0, stream>>>(a, N, nblk);
  return hipGetLastError();
}

}  // namespace flashbob
