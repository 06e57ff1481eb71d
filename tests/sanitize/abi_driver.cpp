// Host-side checks of the C ABI's argument validation, device check and
// error reporting, built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code (tests/test_host_sanitizers.py).  Every call here is
// refused before any kernel launch: bad shapes, null or misaligned pointers,
// bad leading dimensions and workspace sizes are rejected with FGFP8_EINVAL,
// and valid calls on a machine without a gfx950 device with FGFP8_ENODEV.
// Empty problems return FGFP8_OK without touching the device.
#include <cstdio>
#include <cstring>
#include <string>

#include "fgfp8.h"

static int failures = 0;

static void expect(int got, int want, const char* what, const char* needle = nullptr) {
  const char* msg = fgfp8_last_error();
  const bool ok = got == want && (needle == nullptr || std::strstr(msg, needle) != nullptr);
  if (!ok) {
    std::printf("FAIL %s: got %d (want %d), last error \"%s\"\n", what, got, want, msg);
    failures++;
  }
}

int main(int argc, char** argv) {
  // a device is present only when asked to expect one
  const bool have_device = argc > 1 && std::strcmp(argv[1], "device") == 0;
  const int dev_rc = have_device ? FGFP8_OK : FGFP8_ENODEV;
  alignas(256) static unsigned char buf[1 << 16];
  void* P = buf;                 // 256-byte aligned, never dereferenced by a refused call
  void* Q = buf + 4;             // misaligned
  float* F = reinterpret_cast<float*>(buf);

  // quantize_fp8_groups
  expect(quantize_fp8_groups(P, 4, 100, P, F, 4, nullptr), FGFP8_EINVAL, "groups k%128", "multiple of 128");
  expect(quantize_fp8_groups(P, 5, 128, P, F, 5, nullptr), FGFP8_EINVAL, "groups sa_ld%4", "sa_ld");
  expect(quantize_fp8_groups(P, 8, 128, P, F, 4, nullptr), FGFP8_EINVAL, "groups sa_ld<m", "sa_ld");
  expect(quantize_fp8_groups(P, -1, 128, P, F, 4, nullptr), FGFP8_EINVAL, "groups m<0", "out of range");
  expect(quantize_fp8_groups(P, 4, int64_t(1) << 24, P, F, 4, nullptr), FGFP8_EINVAL, "groups huge k", "exceeds");
  expect(quantize_fp8_groups(nullptr, 4, 128, P, F, 4, nullptr), FGFP8_EINVAL, "groups null", "null");
  expect(quantize_fp8_groups(Q, 4, 128, P, F, 4, nullptr), FGFP8_EINVAL, "groups misaligned", "aligned");
  expect(quantize_fp8_groups(nullptr, 0, 128, nullptr, nullptr, 0, nullptr), FGFP8_OK, "groups empty");
  if (!have_device) expect(quantize_fp8_groups(P, 4, 128, P, F, 4, nullptr), FGFP8_ENODEV, "groups no device", "device");
  // quantize_fp8_blocks
  expect(quantize_fp8_blocks(P, 10, 130, P, F, nullptr), FGFP8_EINVAL, "blocks k");
  expect(quantize_fp8_blocks(P, 10, 128, nullptr, F, nullptr), FGFP8_EINVAL, "blocks null");
  expect(quantize_fp8_blocks(P, 10, 128, P, F + 1, nullptr), FGFP8_EINVAL, "blocks misaligned");
  // fp8_gemm_nt and its workspace form
  expect(fp8_gemm_nt(P, F, 6, P, F, P, 8, 16, 256, nullptr), FGFP8_EINVAL, "gemm sa_ld", "sa_ld");
  expect(fp8_gemm_nt(P, F, 8, P, F, P, 8, 16, 200, nullptr), FGFP8_EINVAL, "gemm k");
  expect(fp8_gemm_nt(P, F, 8, P, F, nullptr, 8, 16, 256, nullptr), FGFP8_EINVAL, "gemm null d", "null");
  expect(fp8_gemm_nt(P, F, 8, Q, F, P, 8, 16, 256, nullptr), FGFP8_EINVAL, "gemm misaligned b");
  expect(fp8_gemm_nt(nullptr, nullptr, 0, nullptr, nullptr, nullptr, 0, 16, 256, nullptr), FGFP8_OK, "gemm empty");
  if (!have_device) expect(fp8_gemm_nt(P, F, 8, P, F, P, 8, 16, 256, nullptr), FGFP8_ENODEV, "gemm no device");
  expect(fp8_gemm_nt_ws(P, F, 2048, P, F, P, 2048, 4096, 12288, buf + 16, 1 << 26, nullptr), FGFP8_EINVAL,
         "gemm_ws misaligned workspace", "256-byte");
  expect(fp8_gemm_nt_ws(P, F, 2048, P, F, P, 2048, 4096, 12288, P, -1, nullptr), FGFP8_EINVAL, "gemm_ws bytes<0");
  if (fp8_gemm_nt_workspace_bytes(2048, 4096, 12288) <= 0) {
    std::printf("FAIL workspace query\n");
    failures++;
  }
  if (fp8_gemm_nt_workspace_bytes(2048, 4096, 100) != 0) {
    std::printf("FAIL workspace query on a bad k\n");
    failures++;
  }
  // grouped, masked, FP8 output, MX
  expect(m_grouped_fp8_gemm_nt_contiguous(P, F, 200, (const int32_t*)P, P, F, 2, P, 200, 16, 256, nullptr),
         FGFP8_EINVAL, "grouped m%128", "multiple of 128");
  expect(m_grouped_fp8_gemm_nt_contiguous(P, F, 256, (const int32_t*)P, P, F, 0, P, 256, 16, 256, nullptr),
         FGFP8_EINVAL, "grouped groups", "num_groups");
  expect(m_grouped_fp8_gemm_nt_masked(P, F, 64, (const int32_t*)P, P, F, 2, 30, 8, P, 16, 256, nullptr),
         FGFP8_EINVAL, "masked max_m%4", "max_m");
  expect(fp8_gemm_nt_fp8_out(P, F, 8, P, F, P, F, 8, nullptr, 8, 100, 256, nullptr), FGFP8_EINVAL,
         "fp8 out n%128");
  expect(quantize_fp8_mx(P, 5, 128, P, (int32_t*)P, 5, nullptr), FGFP8_EINVAL, "mx sa_ld");
  expect(fp8_gemm_nt_mx(P, (const int32_t*)P, 8, P, (const int32_t*)P, 12, P, 8, 16, 256, nullptr), FGFP8_EINVAL,
         "mx sb_ld");
  // MoE calls
  const int64_t mpm = moe_max_padded_rows(100, 4, 8);
  const int64_t ws = moe_route_workspace_bytes(100, 8);
  expect(moe_route_contiguous((const int32_t*)P, 100, 9, 8, (int32_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, mpm,
                              P, ws, nullptr),
         FGFP8_EINVAL, "route topk", "topk");
  expect(moe_route_contiguous((const int32_t*)P, 100, 4, 8, (int32_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P,
                              mpm - 128, P, ws, nullptr),
         FGFP8_EINVAL, "route m_pad_max", "m_pad_max");
  expect(moe_route_contiguous((const int32_t*)P, 100, 4, 8, (int32_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, mpm,
                              P, ws - 4, nullptr),
         FGFP8_EINVAL, "route workspace", "workspace");
  expect(moe_route_contiguous_noalloc((const int32_t*)P, int64_t(1) << 20, 1, 2048, (int32_t*)P, (int32_t*)P,
                                      (int32_t*)P, (int32_t*)P, moe_max_padded_rows(int64_t(1) << 20, 1, 2048), nullptr),
         FGFP8_EINVAL, "noalloc route beyond the fixed workspace", "fixed");
  expect(moe_combine(P, 10, 12, (const int32_t*)P, F, 4, 2, P, nullptr), FGFP8_EINVAL, "combine hdim", "hdim");
  expect(silu_mul_quantize(P, 8, 100, (const int32_t*)P, P, F, 8, nullptr), FGFP8_EINVAL, "silu inter");
  expect(fp8_linear_nt(P, 32, 256, P, F, 64, P, nullptr, nullptr, 0, nullptr), FGFP8_EINVAL, "linear workspace",
         "workspace");
  expect(fp8_linear_nt(P, 4, 256, P, F, 64, P, P, nullptr, 4, nullptr), FGFP8_EINVAL, "linear q without sa",
         "together");
  if (!have_device) expect(fp8_linear_nt(P, 4, 256, P, F, 64, P, nullptr, nullptr, 0, nullptr), dev_rc, "linear no device");
  // diagnostics: truncation into a small buffer, and the last-error text
  char small[8];
  expect(fgfp8_describe_gemm(2048, 4096, 4096, small, sizeof small), FGFP8_OK, "describe");
  if (std::strlen(small) != sizeof small - 1) {
    std::printf("FAIL describe truncation: \"%s\"\n", small);
    failures++;
  }
  expect(fgfp8_describe_gemm(2048, 4096, 4096, nullptr, 16), FGFP8_EINVAL, "describe null");
  expect(fgfp8_describe_gemm(2048, 4096, 100, small, sizeof small), FGFP8_EINVAL, "describe bad k");
  // a long message must be truncated safely, and reading it twice is stable
  std::string a = fgfp8_last_error(), b = fgfp8_last_error();
  if (a != b || a.empty()) {
    std::printf("FAIL last error not stable\n");
    failures++;
  }
  if (failures == 0) std::printf("all ABI checks passed\n");
  return failures == 0 ? 0 : 1;
}
