/*
 * A C caller of libfgfp8 with no Python or PyTorch in the process: device
 * memory from the HIP runtime, the product path through the C ABI only.
 *
 *   c_caller A.bin B.bin M N K OUT_PREFIX
 *
 * A.bin: bf16 [M][K], B.bin: bf16 [N][K] (raw little-endian bit patterns).
 * Runs quantize_fp8_groups on A, quantize_fp8_blocks on B, fp8_gemm_nt, and
 * fp8_linear_nt on A's first row (M = 1, the fused decode kernel), all on the
 * legacy default stream, and writes OUT_PREFIX.{q,sa,qb,sb,d,d1}.bin.  Any
 * failure prints a message and exits non-zero.
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fgfp8.h"

#define HIP_OK(x)                                                                  \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(2);                                                                     \
    }                                                                              \
  } while (0)
#define FG_OK(x)                                                                   \
  do {                                                                             \
    int r_ = (x);                                                                  \
    if (r_ != FGFP8_OK) {                                                          \
      fprintf(stderr, "fgfp8 error %d: %s (line %d)\n", r_, fgfp8_last_error(), __LINE__); \
      exit(3);                                                                     \
    }                                                                              \
  } while (0)

static void* read_file(const char* path, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(4); }
  void* p = malloc(bytes ? bytes : 1);
  if (!p || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(4); }
  fclose(f);
  return p;
}

static void write_dev(const char* prefix, const char* name, const void* dev, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s.%s.bin", prefix, name);
  void* h = malloc(bytes ? bytes : 1);
  if (!h) exit(5);
  HIP_OK(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(h, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(5); }
  fclose(f);
  free(h);
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes ? bytes : 16));
  return p;
}

int main(int argc, char** argv) {
  if (argc != 7) { fprintf(stderr, "usage: %s A.bin B.bin M N K OUT_PREFIX\n", argv[0]); return 1; }
  const int64_t m = atoll(argv[3]), n = atoll(argv[4]), k = atoll(argv[5]);
  const char* out = argv[6];
  if (m <= 0 || n <= 0 || k <= 0 || k % 128) { fprintf(stderr, "bad sizes\n"); return 1; }
  const int64_t sa_ld = (m + 3) / 4 * 4, kb = k / 128, nb = (n + 127) / 128;
  void* ha = read_file(argv[1], (size_t)(m * k * 2));
  void* hb = read_file(argv[2], (size_t)(n * k * 2));

  void* x = dev_alloc((size_t)(m * k * 2));
  void* w = dev_alloc((size_t)(n * k * 2));
  void* q = dev_alloc((size_t)(m * k));
  float* sa = (float*)dev_alloc((size_t)(kb * sa_ld * 4));
  void* qb = dev_alloc((size_t)(n * k));
  float* sb = (float*)dev_alloc((size_t)(nb * kb * 4));
  void* d = dev_alloc((size_t)(m * n * 2));
  void* d1 = dev_alloc((size_t)(n * 2));
  HIP_OK(hipMemcpy(x, ha, (size_t)(m * k * 2), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(w, hb, (size_t)(n * k * 2), hipMemcpyHostToDevice));

  FG_OK(quantize_fp8_groups(x, m, k, q, sa, sa_ld, NULL));
  FG_OK(quantize_fp8_blocks(w, n, k, qb, sb, NULL));
  FG_OK(fp8_gemm_nt(q, sa, sa_ld, qb, sb, d, m, n, k, NULL));
  FG_OK(fp8_linear_nt(x, 1, k, qb, sb, n, d1, NULL, NULL, 0, NULL));
  /* a rejected call reports, and enqueues nothing */
  if (fp8_gemm_nt(q, sa, sa_ld, qb, sb, d, m, n, k + 1, NULL) != FGFP8_EINVAL || !strstr(fgfp8_last_error(), "128")) {
    fprintf(stderr, "bad K was not rejected\n");
    return 6;
  }
  HIP_OK(hipDeviceSynchronize());

  write_dev(out, "q", q, (size_t)(m * k));
  write_dev(out, "sa", sa, (size_t)(kb * sa_ld * 4));
  write_dev(out, "qb", qb, (size_t)(n * k));
  write_dev(out, "sb", sb, (size_t)(nb * kb * 4));
  write_dev(out, "d", d, (size_t)(m * n * 2));
  write_dev(out, "d1", d1, (size_t)(n * 2));
  printf("c_caller ok m=%lld n=%lld k=%lld\n", (long long)m, (long long)n, (long long)k);
  free(ha);
  free(hb);
  return 0;
}
