// Sustained bf16 MFMA throughput of this GPU under its power limit: every
// SIMD runs one wave of back-to-back v_mfma_f32_32x32x16_bf16 on eight
// independent accumulators, with operands that change from one instruction to
// the next (random-normal bf16 values, as in the BoB sweeps) or stay zero.
// A kernel doing the same MFMA work and anything else besides cannot beat the
// random-operand figure: the chip lowers its clock to stay within its power
// budget, and the MFMA pipe alone draws most of it. The same stream of
// v_mfma_f32_16x16x32_bf16 (16-row tiles) is measured too, to show whether
// the other tile shape spends less energy per flop.
//
// Standalone program (built next to the library, run by bench.py after its
// timed region). Prints one JSON object: TFLOP/s, the shader clock over the
// run (s_memtime against the 100 MHz s_memrealtime) and the MFMA busy
// fraction at that clock, for random and for zero operands, per instruction.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kWaves = 4;  // one workgroup of four waves per CU: one wave per SIMD

// Roughly N(0, 1): a centred sum of four uniforms from a PCG-style hash.
__device__ float normalish(unsigned x) {
  float s = 0.f;
  for (int k = 0; k < 4; ++k) {
    x = x * 747796405u + 2891336453u;
    unsigned w = ((x >> ((x >> 28u) + 4u)) ^ x) * 277803737u;
    w = (w >> 22u) ^ w;
    s += (float)(w >> 8) * (1.f / 16777216.f);
  }
  return (s - 2.f) * 1.7320508f;
}

// The two instructions: 32x32x16 (16 accumulator registers, 32768 flops) and
// 16x16x32 (4 registers, 16384 flops); both take 8 bf16 of A and of B per lane.
struct M32 {
  typedef f32x16 acc;
  static constexpr int kRegs = 16;
  static constexpr double kFlops = 32768.0;
  static constexpr const char* kName = "v_mfma_f32_32x32x16_bf16";
  __device__ static acc mma(bf16x8 a, bf16x8 b, acc c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
};
struct M16 {
  typedef f32x4 acc;
  static constexpr int kRegs = 4;
  static constexpr double kFlops = 16384.0;
  static constexpr const char* kName = "v_mfma_f32_16x16x32_bf16";
  __device__ static acc mma(bf16x8 a, bf16x8 b, acc c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
};

// iters is a multiple of 8; the operand rotation is unrolled so every register
// index is a compile-time constant. Writes out[gid] once per thread and
// clk[2 * wave], clk[2 * wave + 1] once per wave.
template <typename M, bool ZERO>
__global__ __launch_bounds__(kWaves * 64) void mfma_stream(float* out, unsigned long long* clk, int iters) {
  const int t = threadIdx.x, gid = blockIdx.x * (kWaves * 64) + t;
  bf16x8 a[8], b[8];
  for (int s = 0; s < 8; ++s)
    for (int i = 0; i < 8; ++i) {
      a[s][i] = (__bf16)(ZERO ? 0.f : normalish(gid * 131 + s * 17 + i));
      b[s][i] = (__bf16)(ZERO ? 0.f : normalish(gid * 977 + s * 29 + i + 100000));
    }
  typename M::acc acc[8];
  for (int j = 0; j < 8; ++j)
    for (int i = 0; i < M::kRegs; ++i) acc[j][i] = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it += 8) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] = M::mma(a[m], b[(m + r) & 7], acc[m]);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int j = 0; j < 8; ++j)
    for (int i = 0; i < M::kRegs; ++i) s += acc[j][i];
  out[gid] = s;
  if ((t & 63) == 0) {
    const int wv = blockIdx.x * kWaves + (t >> 6);
    clk[2 * wv] = t1 - t0;
    clk[2 * wv + 1] = r1 - r0;
  }
}

#define CHECK(x)                                                                         \
  do {                                                                                   \
    hipError_t e_ = (x);                                                                 \
    if (e_ != hipSuccess) {                                                              \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                \
      std::exit(1);                                                                      \
    }                                                                                    \
  } while (0)

struct Result {
  double tflops, ghz, busy;
};

template <typename M, bool ZERO>
Result run(int ncu, int iters) {
  const int nwg = ncu, nthr = nwg * kWaves * 64, nwave = nwg * kWaves;
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  CHECK(hipMalloc(&out, (size_t)nthr * sizeof(float)));
  CHECK(hipMalloc(&clk, (size_t)nwave * 2 * sizeof(unsigned long long)));
  mfma_stream<M, ZERO><<<nwg, kWaves * 64>>>(out, clk, 64);  // warm-up
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0));
  mfma_stream<M, ZERO><<<nwg, kWaves * 64>>>(out, clk, iters);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  std::vector<unsigned long long> c((size_t)nwave * 2);
  CHECK(hipMemcpy(c.data(), clk, c.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
  double cyc = 0, rt = 0;
  for (size_t i = 0; i < c.size(); i += 2) {
    cyc += (double)c[i];
    rt += (double)c[i + 1];
  }
  const double flops = (double)nwave * iters * 8 * M::kFlops;
  Result r;
  r.tflops = flops / (ms * 1e-3) / 1e12;
  r.ghz = cyc / rt * 0.1;  // memrealtime ticks at 100 MHz
  // a SIMD retires at most 1024 bf16 flops per cycle (one 32x32x16 MFMA per
  // 32 cycles, one 16x16x32 per 16)
  r.busy = flops / (ms * 1e-3) / (r.ghz * 1e9 * 1024.0 * 4 * ncu);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  CHECK(hipFree(out));
  CHECK(hipFree(clk));
  return r;
}

}  // namespace

int main(int argc, char** argv) {
  // iterations per wave (multiple of 8): 200000 is about 0.3 s on MI355X
  const int iters = argc > 1 ? (std::atoi(argv[1]) / 8) * 8 : 200000;
  if (iters <= 0) return 2;
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int ncu = prop.multiProcessorCount;
  // the 16x16x32 stream does half the flops per instruction: twice the
  // instructions for about the same run time
  const Result r = run<M32, false>(ncu, iters), z = run<M32, true>(ncu, iters);
  const Result r16 = run<M16, false>(ncu, 2 * iters), z16 = run<M16, true>(ncu, 2 * iters);
  std::printf(
      "{\"instruction\": \"%s\", \"cus\": %d, \"iters_per_wave\": %d, "
      "\"random\": {\"tflops\": %.1f, \"sclk_ghz\": %.3f, \"mfma_busy\": %.3f}, "
      "\"zero\": {\"tflops\": %.1f, \"sclk_ghz\": %.3f, \"mfma_busy\": %.3f}, "
      "\"%s\": {\"random\": {\"tflops\": %.1f, \"sclk_ghz\": %.3f, \"mfma_busy\": %.3f}, "
      "\"zero\": {\"tflops\": %.1f, \"sclk_ghz\": %.3f, \"mfma_busy\": %.3f}}}\n",
      M32::kName, ncu, iters, r.tflops, r.ghz, r.busy, z.tflops, z.ghz, z.busy, M16::kName, r16.tflops, r16.ghz,
      r16.busy, z16.tflops, z16.ghz, z16.busy);
  return 0;
}
