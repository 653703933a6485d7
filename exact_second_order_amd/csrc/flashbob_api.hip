// Host side of the C ABI declared in include/flashbob.h: argument checks
// (all before any HIP call), workspace split, and the kernel launches of the
// BoB schedule on the caller's stream: pass 1 (row scalars), then the two
// halves of pass 2 (query side: gradQ, graddO; key side: gradK, gradV).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>

#include "flashbob.h"

namespace flashbob {
typedef __bf16 bf16;
template <typename T, int D, bool GRADQ, bool FIRST, bool SAVED>
hipError_t launch_query(const void* Q, const void* K, const void* V, const void* dO, const void* gQ,
                        const void* gK, const void* gV, float* lse, float* Dv, float* cv, float* rv,
                        void* gradQ, void* graddO, void* dQ, const float* lse_in, int BH, int N, float scale,
                        int lse_natural, int causal, int G, int out_bf16, hipStream_t stream);
template <typename T, int D, bool FIRST>
hipError_t launch_key(const void* Q, const void* K, const void* V, const void* dO, const void* gQ, const void* gK,
                      const void* gV, const float* lse2, const float* Dv, const float* cv, const float* rv,
                      void* gradK, void* gradV, void* dK, void* dV, int BHkv, int N, float scale, int causal,
                      int G, int out_bf16, hipStream_t stream);
}  // namespace flashbob

namespace {

thread_local std::string g_last_hip_error = "no HIP error recorded";

int hip_fail(hipError_t e) {
  g_last_hip_error = std::string(hipGetErrorName(e)) + ": " + hipGetErrorString(e);
  return FLASHBOB_ERR_HIP;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Shared validation. On success fills the element count of one tensor.
int check_common(const void* const* ins, int B, int H, int N, int d, float scale, int dtype, size_t* numel) {
  if (B < 0 || H < 0 || N < 0) return FLASHBOB_ERR_SHAPE;
  // the dtype first: the head dims supported depend on it
  if (dtype != FLASHBOB_F32 && dtype != FLASHBOB_BF16) return FLASHBOB_ERR_DTYPE;
  // d = 256 in bf16 only: an fp32 stage at d = 256 needs more than the 160 KB of LDS
  if (d != 32 && d != 64 && d != 96 && d != 128 && !(d == 256 && dtype == FLASHBOB_BF16))
    return FLASHBOB_ERR_UNSUPPORTED_D;
  if (!std::isfinite(scale)) return FLASHBOB_ERR_SCALE;
  // B*H*N*d < 2^62 (fits every index computed in size_t) and B*H*N < 2^31
  const unsigned __int128 n = (unsigned __int128)B * H * N * d;
  if (n >= ((unsigned __int128)1 << 62)) return FLASHBOB_ERR_SHAPE;
  if ((unsigned __int128)B * H * N >= ((unsigned __int128)1 << 31)) return FLASHBOB_ERR_SHAPE;
  if ((long long)B * H >= (1LL << 31)) return FLASHBOB_ERR_SHAPE;
  *numel = (size_t)n;
  if (*numel == 0) return FLASHBOB_OK;
  for (int i = 0; i < 7; ++i) {
    if (ins[i] == nullptr) return FLASHBOB_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(ins[i]) % 16) return FLASHBOB_ERR_ALIGN;
  }
  return FLASHBOB_OK;
}

// ins: the seven inputs with their byte sizes; outs: nout outputs with theirs.
int check_outputs(const void* const* ins, const size_t* in_bytes, int nin, void* const* outs,
                  const size_t* out_bytes, int nout) {
  for (int i = 0; i < nout; ++i) {
    if (outs[i] == nullptr) return FLASHBOB_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(outs[i]) % 16) return FLASHBOB_ERR_ALIGN;
  }
  for (int i = 0; i < nout; ++i) {
    const Range ro{reinterpret_cast<uintptr_t>(outs[i]), reinterpret_cast<uintptr_t>(outs[i]) + out_bytes[i]};
    for (int j = 0; j < nin; ++j) {
      const Range ri{reinterpret_cast<uintptr_t>(ins[j]), reinterpret_cast<uintptr_t>(ins[j]) + in_bytes[j]};
      if (overlaps(ro, ri)) return FLASHBOB_ERR_ALIAS;
    }
    for (int j = i + 1; j < nout; ++j) {
      const Range rj{reinterpret_cast<uintptr_t>(outs[j]), reinterpret_cast<uintptr_t>(outs[j]) + out_bytes[j]};
      if (overlaps(ro, rj)) return FLASHBOB_ERR_ALIAS;
    }
  }
  return FLASHBOB_OK;
}

// The three kernels of the schedule, dispatched on (element type, d).
enum Stage {
  kPass1 = FLASHBOB_STAGE_PASS1,
  kPass2Query = FLASHBOB_STAGE_PASS2_QUERY,
  kPass2Key = FLASHBOB_STAGE_PASS2_KEY,
};

// Everything one flashbob_bob_ex call hands its kernels besides the inputs.
struct Call {
  int stages, causal;
  const float* lse_in;  // the rows' saved log-sum-exp for pass 1, or null
  float* stats;         // workspace: [4][B*H*N] row scalars
  void *gradQ, *gradK, *gradV, *graddO;
  void *dQ, *dK, *dV;   // first-backward outputs, or null
  int out_bf16;         // outputs stored as bf16 instead of float32
  int BH, G, N;
  float scale;
  hipStream_t stream;
};

template <typename T, int D>
hipError_t run_stages(const void* const* in, const Call& c) {
  const size_t BHN = (size_t)c.BH * c.N;
  // workspace row scalars: LSE * log2(e), D, c, r
  float *lse = c.stats, *Dv = c.stats + BHN, *cv = c.stats + 2 * BHN, *rv = c.stats + 3 * BHN;
  const bool first = c.dQ != nullptr;
  hipError_t e = hipSuccess;
  if (c.stages & kPass1) {
    e = c.lse_in ? flashbob::launch_query<T, D, false, false, true>(in[0], in[1], in[2], in[3], in[4], in[5], in[6],
                                                                    lse, Dv, cv, rv, nullptr, nullptr, nullptr,
                                                                    c.lse_in, c.BH, c.N, c.scale, 0, c.causal, c.G,
                                                                    0, c.stream)
                 : flashbob::launch_query<T, D, false, false, false>(in[0], in[1], in[2], in[3], in[4], in[5],
                                                                     in[6], lse, Dv, cv, rv, nullptr, nullptr,
                                                                     nullptr, nullptr, c.BH, c.N, c.scale, 0,
                                                                     c.causal, c.G, 0, c.stream);
    if (e != hipSuccess) return e;
  }
  if (c.stages & kPass2Query) {
    e = first ? flashbob::launch_query<T, D, true, true, false>(in[0], in[1], in[2], in[3], in[4], in[5], in[6],
                                                                lse, Dv, cv, rv, c.gradQ, c.graddO, c.dQ, nullptr,
                                                                c.BH, c.N, c.scale, 0, c.causal, c.G, c.out_bf16,
                                                                c.stream)
              : flashbob::launch_query<T, D, true, false, false>(in[0], in[1], in[2], in[3], in[4], in[5], in[6],
                                                                 lse, Dv, cv, rv, c.gradQ, c.graddO, nullptr,
                                                                 nullptr, c.BH, c.N, c.scale, 0, c.causal, c.G,
                                                                 c.out_bf16, c.stream);
    if (e != hipSuccess) return e;
  }
  if (c.stages & kPass2Key) {
    e = first ? flashbob::launch_key<T, D, true>(in[0], in[1], in[2], in[3], in[4], in[5], in[6], lse, Dv, cv, rv,
                                                 c.gradK, c.gradV, c.dK, c.dV, c.BH / c.G, c.N, c.scale, c.causal,
                                                 c.G, c.out_bf16, c.stream)
              : flashbob::launch_key<T, D, false>(in[0], in[1], in[2], in[3], in[4], in[5], in[6], lse, Dv, cv, rv,
                                                  c.gradK, c.gradV, nullptr, nullptr, c.BH / c.G, c.N, c.scale,
                                                  c.causal, c.G, c.out_bf16, c.stream);
  }
  return e;
}

template <typename T>
struct TypeTag {
  using type = T;
};
template <int D>
using DimTag = std::integral_constant<int, D>;

// Calls f(TypeTag<T>{}, DimTag<D>{}) for the element type and head dim of a
// call (both validated before: d is one of the supported head dims).
template <typename Fn>
hipError_t on_type_and_dim(int dtype, int d, Fn&& f) {
  auto dims = [&](auto t) -> hipError_t {
    switch (d) {
      case 32: return f(t, DimTag<32>{});
      case 64: return f(t, DimTag<64>{});
      case 96: return f(t, DimTag<96>{});
      case 256:
        if constexpr (std::is_same_v<typename decltype(t)::type, __bf16>) return f(t, DimTag<256>{});
        else return hipErrorInvalidValue;  // refused by the argument checks
      default: return f(t, DimTag<128>{});
    }
  };
  return dtype == FLASHBOB_BF16 ? dims(TypeTag<__bf16>{}) : dims(TypeTag<float>{});
}

hipError_t dispatch(int dtype, int d, const void* const* in, const Call& c) {
  return on_type_and_dim(dtype, d, [&](auto t, auto dd) {
    return run_stages<typename decltype(t)::type, decltype(dd)::value>(in, c);
  });
}

template <typename T, int D>
hipError_t rowstats_launch(const void* const* in, float* lse, float* Dv, float* cv, float* rv, int BH, int G,
                           int N, float scale, int causal, hipStream_t st) {
  return flashbob::launch_query<T, D, false, false, false>(in[0], in[1], in[2], in[3], in[4], in[5], in[6], lse,
                                                           Dv, cv, rv, nullptr, nullptr, nullptr, nullptr, BH, N,
                                                           scale, 1, causal, G, 0, st);
}

hipError_t dispatch_rowstats(int dtype, int d, int causal, const void* const* in, float* lse, float* Dv, float* cv,
                             float* rv, int BH, int G, int N, float scale, hipStream_t st) {
  return on_type_and_dim(dtype, d, [&](auto t, auto dd) {
    return rowstats_launch<typename decltype(t)::type, decltype(dd)::value>(in, lse, Dv, cv, rv, BH, G, N, scale,
                                                                            causal, st);
  });
}

// Key/value heads: 1 <= H_kv <= H with H a multiple of H_kv (any H_kv when H
// is 0). Query-side tensors hold B*H*N*d elements, key/value-side ones
// B*H_kv*N*d.
int check_kv_heads(int H, int H_kv) {
  if (H_kv < 0 || (H > 0 && (H_kv == 0 || H % H_kv != 0))) return FLASHBOB_ERR_SHAPE;
  return FLASHBOB_OK;
}

void tensor_bytes(size_t numel_q, size_t numel_kv, size_t esz, size_t* in_bytes) {
  const bool q_side[7] = {true, false, false, true, true, false, false};  // Q K V dO gQ gK gV
  for (int i = 0; i < 7; ++i) in_bytes[i] = (q_side[i] ? numel_q : numel_kv) * esz;
}

size_t stats_bytes(int B, int H, int N) {
  const size_t raw = (size_t)4 * sizeof(float) * (size_t)B * (size_t)H * (size_t)N;
  return (raw + 255) & ~(size_t)255;
}

// Static row-scalar buffer of flashbob_bob_noalloc: one copy per GPU the
// library runs on, found through hipGetSymbolAddress (in host code the array
// name is only a stand-in for the device address, never used directly).
static __device__ __align__(256) unsigned char scratch[FLASHBOB_NOALLOC_SCRATCH_BYTES];
static_assert((size_t)FLASHBOB_NOALLOC_SCRATCH_BYTES >= (size_t)16 * FLASHBOB_NOALLOC_MAX_ROWS,
              "four float32 scalars per query row");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device current on this thread (looked
// up once per device).
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_fail(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (p == nullptr) return hip_fail(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLASHBOB_OK;
}

}  // namespace

extern "C" {

size_t flashbob_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return stats_bytes(B, H, N);
}

int flashbob_bob_ex(const void* Q, const void* K, const void* V, const void* dO, const void* gQ, const void* gK,
                    const void* gV, void* gradQ, void* gradK, void* gradV, void* graddO, void* dQ, void* dK,
                    void* dV, const float* lse_in, int B, int H, int H_kv, int N, int d, float scale, int dtype,
                    int flags, int stages, void* workspace, size_t workspace_bytes, void* stream) {
  constexpr int kKnownFlags = FLASHBOB_CAUSAL | FLASHBOB_FIRST_BACKWARD | FLASHBOB_SAVED_LSE | FLASHBOB_BF16_OUTPUTS;
  if ((flags & ~kKnownFlags) != 0 || stages <= 0 || (stages & ~FLASHBOB_STAGES_ALL) != 0)
    return FLASHBOB_ERR_FLAGS;
  const bool first = (flags & FLASHBOB_FIRST_BACKWARD) != 0;
  const bool saved = (flags & FLASHBOB_SAVED_LSE) != 0;
  const bool bf16_out = (flags & FLASHBOB_BF16_OUTPUTS) != 0;
  const void* ins[8] = {Q, K, V, dO, gQ, gK, gV, lse_in};
  size_t numel = 0;
  int rc = check_common(ins, B, H, N, d, scale, dtype, &numel);
  if (rc == FLASHBOB_OK) rc = check_kv_heads(H, H_kv);
  if (rc != FLASHBOB_OK || numel == 0) return rc;
  const size_t esz = dtype == FLASHBOB_BF16 ? 2 : 4;
  const size_t osz = bf16_out ? 2 : 4;  // output element size
  const size_t numel_kv = numel / (size_t)H * (size_t)H_kv;
  const size_t ws_need = stats_bytes(B, H, N);
  if (workspace == nullptr) return FLASHBOB_ERR_NULL;
  if (workspace_bytes < ws_need) return FLASHBOB_ERR_WORKSPACE;
  if (saved) {  // one float per query row, read as scalars: 4-byte alignment
    if (lse_in == nullptr) return FLASHBOB_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(lse_in) % 4) return FLASHBOB_ERR_ALIGN;
  }
  size_t ib[8];
  tensor_bytes(numel, numel_kv, esz, ib);
  ib[7] = numel / (size_t)d * 4;  // lse_in: B*H*N floats
  void* outs[8] = {gradQ, gradK, gradV, graddO, workspace, dQ, dK, dV};
  const size_t ob[8] = {numel * osz, numel_kv * osz, numel_kv * osz, numel * osz, ws_need,
                        numel * osz, numel_kv * osz, numel_kv * osz};
  // dQ, dK, dV are outputs only with their flag, lse_in an input only with its
  rc = check_outputs(ins, ib, saved ? 8 : 7, outs, ob, first ? 8 : 5);
  if (rc != FLASHBOB_OK) return rc;
  Call c{};
  c.stages = stages;
  c.causal = (flags & FLASHBOB_CAUSAL) ? 1 : 0;
  c.lse_in = saved ? lse_in : nullptr;
  c.stats = static_cast<float*>(workspace);
  c.gradQ = gradQ;
  c.gradK = gradK;
  c.gradV = gradV;
  c.graddO = graddO;
  if (first) {
    c.dQ = dQ;
    c.dK = dK;
    c.dV = dV;
  }
  c.out_bf16 = bf16_out ? 1 : 0;
  c.BH = B * H;
  c.G = H / H_kv;
  c.N = N;
  c.scale = scale;
  c.stream = static_cast<hipStream_t>(stream);
  const hipError_t e = dispatch(dtype, d, ins, c);
  return e == hipSuccess ? FLASHBOB_OK : hip_fail(e);
}

int flashbob_bob(const void* Q, const void* K, const void* V, const void* dO, const void* gQ, const void* gK,
                 const void* gV, float* gradQ, float* gradK, float* gradV, float* graddO, int B, int H, int N,
                 int d, float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return flashbob_bob_ex(Q, K, V, dO, gQ, gK, gV, gradQ, gradK, gradV, graddO, nullptr, nullptr, nullptr, nullptr,
                         B, H, H, N, d, scale, dtype, 0,
                         FLASHBOB_STAGES_ALL, workspace, workspace_bytes, stream);
}

int flashbob_bob_noalloc(const void* Q, const void* K, const void* V, const void* dO, const void* gQ,
                         const void* gK, const void* gV, float* gradQ, float* gradK, float* gradV,
                         float* graddO, int B, int H, int N, int d, float scale, int dtype, void* stream) {
  // every argument check before the HIP call that finds the buffer
  const void* ins[7] = {Q, K, V, dO, gQ, gK, gV};
  size_t numel = 0;
  int rc = check_common(ins, B, H, N, d, scale, dtype, &numel);
  if (rc != FLASHBOB_OK || numel == 0) return rc;
  if ((long long)B * H * N > FLASHBOB_NOALLOC_MAX_ROWS) return FLASHBOB_ERR_SCRATCH;
  const size_t esz = dtype == FLASHBOB_BF16 ? 2 : 4;
  size_t ib[7];
  tensor_bytes(numel, numel, esz, ib);
  void* outs[4] = {gradQ, gradK, gradV, graddO};
  const size_t ob[4] = {numel * 4, numel * 4, numel * 4, numel * 4};
  rc = check_outputs(ins, ib, 7, outs, ob, 4);
  if (rc != FLASHBOB_OK) return rc;
  void* ws = nullptr;
  rc = scratch_on_current_device(&ws);
  if (rc != FLASHBOB_OK) return rc;
  return flashbob_bob_ex(Q, K, V, dO, gQ, gK, gV, gradQ, gradK, gradV, graddO, nullptr, nullptr, nullptr, nullptr,
                         B, H, H, N, d, scale, dtype, 0, FLASHBOB_STAGES_ALL, ws, FLASHBOB_NOALLOC_SCRATCH_BYTES,
                         stream);
}

int flashbob_bob_pass1(const void* Q, const void* K, const void* V, const void* dO, const void* gQ,
                       const void* gK, const void* gV, float* gradQ, float* gradK, float* gradV, float* graddO,
                       int B, int H, int N, int d, float scale, int dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return flashbob_bob_ex(Q, K, V, dO, gQ, gK, gV, gradQ, gradK, gradV, graddO, nullptr, nullptr, nullptr, nullptr,
                         B, H, H, N, d, scale, dtype, 0,
                         FLASHBOB_STAGE_PASS1, workspace, workspace_bytes, stream);
}

int flashbob_bob_pass2_query(const void* Q, const void* K, const void* V, const void* dO, const void* gQ,
                             const void* gK, const void* gV, float* gradQ, float* gradK, float* gradV,
                             float* graddO, int B, int H, int N, int d, float scale, int dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return flashbob_bob_ex(Q, K, V, dO, gQ, gK, gV, gradQ, gradK, gradV, graddO, nullptr, nullptr, nullptr, nullptr,
                         B, H, H, N, d, scale, dtype, 0,
                         FLASHBOB_STAGE_PASS2_QUERY, workspace, workspace_bytes, stream);
}

int flashbob_bob_pass2_key(const void* Q, const void* K, const void* V, const void* dO, const void* gQ,
                           const void* gK, const void* gV, float* gradQ, float* gradK, float* gradV,
                           float* graddO, int B, int H, int N, int d, float scale, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return flashbob_bob_ex(Q, K, V, dO, gQ, gK, gV, gradQ, gradK, gradV, graddO, nullptr, nullptr, nullptr, nullptr,
                         B, H, H, N, d, scale, dtype, 0,
                         FLASHBOB_STAGE_PASS2_KEY, workspace, workspace_bytes, stream);
}

int flashbob_rowstats_ex(const void* Q, const void* K, const void* V, const void* dO, const void* gQ,
                         const void* gK, const void* gV, float* lse, float* Dv, float* cv, float* rv, int B, int H,
                         int H_kv, int N, int d, float scale, int dtype, int flags, void* stream) {
  if ((flags & ~FLASHBOB_CAUSAL) != 0) return FLASHBOB_ERR_FLAGS;
  const void* ins[7] = {Q, K, V, dO, gQ, gK, gV};
  size_t numel = 0;
  int rc = check_common(ins, B, H, N, d, scale, dtype, &numel);
  if (rc == FLASHBOB_OK) rc = check_kv_heads(H, H_kv);
  if (rc != FLASHBOB_OK || numel == 0) return rc;
  const size_t esz = dtype == FLASHBOB_BF16 ? 2 : 4;
  size_t ib[7];
  tensor_bytes(numel, numel / (size_t)H * (size_t)H_kv, esz, ib);
  const size_t vb = (size_t)B * H * N * sizeof(float);
  void* outs[4] = {lse, Dv, cv, rv};
  const size_t ob[4] = {vb, vb, vb, vb};
  rc = check_outputs(ins, ib, 7, outs, ob, 4);
  if (rc != FLASHBOB_OK) return rc;
  // pass 1 writing the plain row scalars into the caller's four vectors
  const hipError_t e = dispatch_rowstats(dtype, d, (flags & FLASHBOB_CAUSAL) ? 1 : 0, ins, lse, Dv, cv, rv, B * H,
                                         H / H_kv, N, scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLASHBOB_OK : hip_fail(e);
}

int flashbob_rowstats(const void* Q, const void* K, const void* V, const void* dO, const void* gQ,
                      const void* gK, const void* gV, float* lse, float* Dv, float* cv, float* rv, int B, int H,
                      int N, int d, float scale, int dtype, void* stream) {
  return flashbob_rowstats_ex(Q, K, V, dO, gQ, gK, gV, lse, Dv, cv, rv, B, H, H, N, d, scale, dtype, 0, stream);
}

const char* flashbob_strerror(int code) {
  switch (code) {
    case FLASHBOB_OK: return "ok";
    case FLASHBOB_ERR_NULL: return "a required pointer is NULL";
    case FLASHBOB_ERR_SHAPE: return "invalid shape (negative size or too many elements)";
    case FLASHBOB_ERR_UNSUPPORTED_D: return "unsupported head dimension (d must be 32, 64, 96 or 128, or 256 with bf16 inputs)";
    case FLASHBOB_ERR_UNSUPPORTED_N: return "unsupported sequence length";
    case FLASHBOB_ERR_DTYPE: return "unknown dtype";
    case FLASHBOB_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FLASHBOB_ERR_WORKSPACE: return "workspace too small";
    case FLASHBOB_ERR_ALIAS: return "an output overlaps an input, the workspace or another output";
    case FLASHBOB_ERR_SCALE: return "scale is not finite";
    case FLASHBOB_ERR_FLAGS: return "unknown flag bits or an empty or unknown stage set";
    case FLASHBOB_ERR_SCRATCH: return "B*H*N exceeds the static buffer of flashbob_bob_noalloc (1048576 query rows)";
    case FLASHBOB_ERR_HIP: return g_last_hip_error.c_str();
    default: return "unknown error code";
  }
}

int flashbob_version(void) { return 104; }

}  // extern "C"
