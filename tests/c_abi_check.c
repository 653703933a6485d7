/* A plain C caller of the BoB C ABI (include/flashbob.h): no torch, no C++.
 *
 * usage: c_abi_check B H N d dtype scale causal in_dir out_dir
 *   dtype 0 = float32, 1 = bf16 (raw bits); causal 0 or 1.
 * Reads in_dir/{Q,K,V,dO,gQ,gK,gV}.bin (B*H*N*d elements each, row-major
 * [B, H, N, d]), runs one call on the default stream (flashbob_bob, or
 * flashbob_bob_ex with FLASHBOB_CAUSAL), and writes out_dir/{gradQ,gradK,
 * gradV,graddO}.bin as float32. Also checks that a bad head dim is rejected
 * before any HIP call. Exit status 0 on success; any failure prints its cause.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "flashbob.h"

#define HIP_OK(call)                                                                \
  do {                                                                              \
    hipError_t e_ = (call);                                                         \
    if (e_ != hipSuccess) {                                                         \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));             \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

static const char* kIn[7] = {"Q", "K", "V", "dO", "gQ", "gK", "gV"};
static const char* kOut[4] = {"gradQ", "gradK", "gradV", "graddO"};

static int read_file(const char* dir, const char* name, void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s.bin", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return 1;
  }
  size_t got = fread(buf, 1, bytes, f);
  fclose(f);
  if (got != bytes) {
    fprintf(stderr, "%s: read %zu of %zu bytes\n", path, got, bytes);
    return 1;
  }
  return 0;
}

static int write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s.bin", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(buf, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    if (f) fclose(f);
    return 1;
  }
  fclose(f);
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 10) {
    fprintf(stderr, "usage: %s B H N d dtype scale causal in_dir out_dir\n", argv[0]);
    return 2;
  }
  const int B = atoi(argv[1]), H = atoi(argv[2]), N = atoi(argv[3]), d = atoi(argv[4]);
  const int dtype = atoi(argv[5]), causal = atoi(argv[7]);
  const float scale = (float)atof(argv[6]);
  const char *in_dir = argv[8], *out_dir = argv[9];
  /* stdout is a pipe under the test runner: unbuffered, so nothing printed is
     lost if the process ends abnormally; progress goes to stderr */
  setvbuf(stdout, NULL, _IONBF, 0);
#define STEP(msg) fprintf(stderr, "c_abi_check: %s\n", msg)
  if (B <= 0 || H <= 0 || N <= 0 || (dtype != FLASHBOB_F32 && dtype != FLASHBOB_BF16)) {
    fprintf(stderr, "bad arguments\n");
    return 2;
  }
  const size_t numel = (size_t)B * H * N * d;
  const size_t esz = dtype == FLASHBOB_BF16 ? 2 : 4;

  void* host = malloc(numel * 4);
  void* dev_in[7] = {0};
  float* dev_out[4] = {0};
  if (!host) return 1;
  for (int i = 0; i < 7; ++i) {
    if (read_file(in_dir, kIn[i], host, numel * esz)) return 1;
    HIP_OK(hipMalloc(&dev_in[i], numel * esz));
    HIP_OK(hipMemcpy(dev_in[i], host, numel * esz, hipMemcpyHostToDevice));
  }
  for (int i = 0; i < 4; ++i) HIP_OK(hipMalloc((void**)&dev_out[i], numel * 4));
  STEP("inputs on the device");
  const size_t ws_bytes = flashbob_workspace_bytes(B, H, N, d);
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, ws_bytes));

  /* argument checks run before any HIP work: d = 80 is refused */
  int rc = flashbob_bob(dev_in[0], dev_in[1], dev_in[2], dev_in[3], dev_in[4], dev_in[5], dev_in[6], dev_out[0],
                        dev_out[1], dev_out[2], dev_out[3], B, H, N, 80, scale, dtype, ws, ws_bytes, NULL);
  if (rc != FLASHBOB_ERR_UNSUPPORTED_D) {
    fprintf(stderr, "d = 80 returned %d, expected %d\n", rc, FLASHBOB_ERR_UNSUPPORTED_D);
    return 1;
  }

  if (causal)
    rc = flashbob_bob_ex(dev_in[0], dev_in[1], dev_in[2], dev_in[3], dev_in[4], dev_in[5], dev_in[6], dev_out[0],
                         dev_out[1], dev_out[2], dev_out[3], NULL, NULL, NULL, NULL, B, H, H, N, d, scale, dtype,
                         FLASHBOB_CAUSAL, FLASHBOB_STAGES_ALL, ws, ws_bytes, NULL);
  else
    rc = flashbob_bob(dev_in[0], dev_in[1], dev_in[2], dev_in[3], dev_in[4], dev_in[5], dev_in[6], dev_out[0],
                      dev_out[1], dev_out[2], dev_out[3], B, H, N, d, scale, dtype, ws, ws_bytes, NULL);
  if (rc != FLASHBOB_OK) {
    fprintf(stderr, "flashbob call failed: %d (%s)\n", rc, flashbob_strerror(rc));
    return 1;
  }
  STEP("call enqueued");
  HIP_OK(hipDeviceSynchronize());
  STEP("call finished");
  for (int i = 0; i < 4; ++i) {
    HIP_OK(hipMemcpy(host, dev_out[i], numel * 4, hipMemcpyDeviceToHost));
    if (write_file(out_dir, kOut[i], host, numel * 4)) return 1;
  }
  STEP("outputs written");
  for (int i = 0; i < 7; ++i) HIP_OK(hipFree(dev_in[i]));
  for (int i = 0; i < 4; ++i) HIP_OK(hipFree(dev_out[i]));
  HIP_OK(hipFree(ws));
  free(host);
  printf("c_abi_check: ok (version %d)\n", flashbob_version());
  return 0;
}
