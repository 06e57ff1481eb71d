// The C ABI of libfgfp8 (declared in include/fgfp8.h): argument validation,
// device check, kernel plan choice, launch on the caller's stream.  No call
// allocates, frees, synchronizes or reads device memory on the host.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/fgfp8.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device verdict: 0 unknown, 1 gfx950, 2 other.  Device ids beyond the
// table are checked on every call.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];

int check_device(const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(FGFP8_ENODEV, "%s: no HIP device (%s)", who, hipGetErrorString(e));
  }
  int known = dev < kMaxDevices ? g_device_ok[dev].load(std::memory_order_relaxed) : 0;
  if (known == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(FGFP8_ENODEV, "%s: cannot query device %d (%s)", who, dev, hipGetErrorString(e));
    }
    known = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (dev < kMaxDevices) g_device_ok[dev].store(known, std::memory_order_relaxed);
    if (known == 2) return fail(FGFP8_ENODEV, "%s: device %d is %s, not gfx950", who, dev, prop.gcnArchName);
  }
  if (known != 1) return fail(FGFP8_ENODEV, "%s: device %d is not gfx950", who, dev);
  return FGFP8_OK;
}

int launched(hipError_t e, const char* who) {
  if (e != hipSuccess) return fail(FGFP8_ELAUNCH, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
  return FGFP8_OK;
}

// K is below 2^24 so that a tile's operand bytes (256 rows * K) fit the
// 32-bit record counts and offsets of the buffer resources the kernels use
// (at K = 2^24 exactly, 256 * K wraps to zero).
constexpr int64_t kMaxK = (int64_t(1) << 24) - 128;
constexpr int64_t kMaxRows = int64_t(1) << 31;

int check_k(const char* who, int64_t k) {
  if (k <= 0 || k % 128 != 0) return fail(FGFP8_EINVAL, "%s: k=%lld must be a positive multiple of 128", who, (long long)k);
  if (k > kMaxK) return fail(FGFP8_EINVAL, "%s: k=%lld exceeds %lld", who, (long long)k, (long long)kMaxK);
  return FGFP8_OK;
}

int check_sa(const char* who, int64_t m, int64_t k, int64_t sa_ld) {
  if (sa_ld < m || sa_ld % 4 != 0 || sa_ld < 0)
    return fail(FGFP8_EINVAL, "%s: sa_ld=%lld must be a non-negative multiple of 4 and >= m=%lld", who,
                (long long)sa_ld, (long long)m);
  if ((k / 128) * sa_ld * 4 >= (int64_t(1) << 31))
    return fail(FGFP8_EINVAL, "%s: activation scale array (k/128 * sa_ld floats) exceeds 2 GiB", who);
  return FGFP8_OK;
}

bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v && *v && strcmp(v, "0") != 0;
}

}  // namespace

extern "C" {

const char* fgfp8_last_error(void) { return g_last_error.c_str(); }

namespace {

int quantize_groups_impl(const char* who, bool ue8m0, const void* x_bf16, int64_t m, int64_t k, void* q_e4m3,
                         float* sa, int64_t sa_ld, void* stream) {
  if (m < 0 || m >= kMaxRows) return fail(FGFP8_EINVAL, "%s: m=%lld out of range", who, (long long)m);
  if (int rc = check_k(who, k)) return rc;
  if (int rc = check_sa(who, m, k, sa_ld)) return rc;
  if (m == 0) return FGFP8_OK;  // empty: nothing to enqueue, pointers may be null
  if (!x_bf16 || !q_e4m3 || !sa) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(x_bf16) || !aligned16(q_e4m3) || !aligned16(sa))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  return launched(fgfp8::launch_quantize_groups(x_bf16, m, k, q_e4m3, sa, sa_ld, (hipStream_t)stream, ue8m0), who);
}

int quantize_fp8_groups_masked(const void* x_bf16, const int32_t* masked_m, int32_t num_groups, int64_t max_m,
                               int64_t k, void* q_e4m3, float* sa, int64_t sa_ld, void* stream) {
  const char* who = "quantize_fp8_groups_masked";
  if (num_groups < 1) return fail(FGFP8_EINVAL, "%s: num_groups=%d must be >= 1", who, (int)num_groups);
  if (max_m < 0 || max_m % 4 != 0 || (int64_t)num_groups * max_m >= kMaxRows)
    return fail(FGFP8_EINVAL, "%s: max_m=%lld must be a non-negative multiple of 4 (and num_groups * max_m < 2^31)",
                who, (long long)max_m);
  if (int rc = check_k(who, k)) return rc;
  if (int rc = check_sa(who, (int64_t)num_groups * max_m, k, sa_ld)) return rc;
  if (max_m == 0) return FGFP8_OK;
  if (!x_bf16 || !masked_m || !q_e4m3 || !sa) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(x_bf16) || !aligned16(masked_m) || !aligned16(q_e4m3) || !aligned16(sa))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  return launched(fgfp8::launch_quantize_groups_masked(x_bf16, masked_m, num_groups, max_m, k, q_e4m3, sa, sa_ld,
                                                       (hipStream_t)stream),
                  who);
}

int quantize_blocks_impl(const char* who, bool ue8m0, const void* w_bf16, int64_t n, int64_t k, void* q_e4m3,
                         float* sb, void* stream) {
  if (n < 0 || (n + 127) / 128 > 65535) return fail(FGFP8_EINVAL, "%s: n=%lld out of range", who, (long long)n);
  if (int rc = check_k(who, k)) return rc;
  if (n == 0) return FGFP8_OK;
  if (!w_bf16 || !q_e4m3 || !sb) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(w_bf16) || !aligned16(q_e4m3) || !aligned16(sb))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  return launched(fgfp8::launch_quantize_blocks(w_bf16, n, k, q_e4m3, sb, (hipStream_t)stream, ue8m0), who);
}

int gemm_impl(const char* who, bool ue8m0, const void* a_e4m3, const float* sa, int64_t sa_ld, const void* b_e4m3,
              const float* sb, void* d_bf16, int64_t m, int64_t n, int64_t k, void* stream, void* workspace = nullptr,
              int64_t workspace_bytes = 0) {
  if (m < 0 || m >= kMaxRows || n < 0 || n >= kMaxRows)
    return fail(FGFP8_EINVAL, "%s: m=%lld n=%lld out of range", who, (long long)m, (long long)n);
  if (int rc = check_k(who, k)) return rc;
  if (int rc = check_sa(who, m, k, sa_ld)) return rc;
  if (m == 0 || n == 0) return FGFP8_OK;
  if (!a_e4m3 || !sa || !b_e4m3 || !sb || !d_bf16) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(a_e4m3) || !aligned16(sa) || !aligned16(b_e4m3) || !aligned16(sb) || !aligned16(d_bf16))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(FGFP8_EINVAL, "%s: workspace must be 256-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  fgfp8::GemmPlan plan = fgfp8::plan_gemm(m, n, k);
  if (workspace != nullptr && !ue8m0) {
    const fgfp8::GemmPlan wp = fgfp8::plan_gemm_ws(m, n, k);
    if (wp.kind == fgfp8::kGemmTile256x256SplitK2 && workspace_bytes >= fgfp8::gemm_splitk_workspace_bytes(m, n))
      plan = wp;
  }
  if (env_flag("FGFP8_PRINT_CONFIG"))
    fprintf(stderr, "[fgfp8] %s m=%lld n=%lld k=%lld: %s split=%d\n", who, (long long)m, (long long)n, (long long)k,
            fgfp8::gemm_kind_name(plan.kind), plan.split);
  const hipStream_t st = (hipStream_t)stream;
  if (plan.kind == fgfp8::kGemmTile256x256SplitK2)
    return launched(fgfp8::launch_gemm_splitk(a_e4m3, sa, sa_ld, b_e4m3, sb, d_bf16, m, n, k, workspace, st), who);
  return launched(ue8m0 ? fgfp8::launch_gemm_ue8m0(plan, a_e4m3, sa, sa_ld, b_e4m3, sb, d_bf16, m, n, k, st)
                        : fgfp8::launch_gemm(plan, a_e4m3, sa, sa_ld, b_e4m3, sb, d_bf16, m, n, k, st),
                  who);
}

}  // namespace

int quantize_fp8_groups(const void* x_bf16, int64_t m, int64_t k, void* q_e4m3, float* sa, int64_t sa_ld,
                        void* stream) {
  return quantize_groups_impl("quantize_fp8_groups", false, x_bf16, m, k, q_e4m3, sa, sa_ld, stream);
}

int quantize_fp8_groups_ue8m0(const void* x_bf16, int64_t m, int64_t k, void* q_e4m3, float* sa, int64_t sa_ld,
                              void* stream) {
  return quantize_groups_impl("quantize_fp8_groups_ue8m0", true, x_bf16, m, k, q_e4m3, sa, sa_ld, stream);
}

int quantize_fp8_blocks(const void* w_bf16, int64_t n, int64_t k, void* q_e4m3, float* sb, void* stream) {
  return quantize_blocks_impl("quantize_fp8_blocks", false, w_bf16, n, k, q_e4m3, sb, stream);
}

int quantize_fp8_blocks_ue8m0(const void* w_bf16, int64_t n, int64_t k, void* q_e4m3, float* sb, void* stream) {
  return quantize_blocks_impl("quantize_fp8_blocks_ue8m0", true, w_bf16, n, k, q_e4m3, sb, stream);
}

int fp8_gemm_nt_ue8m0(const void* a_e4m3, const float* sa, int64_t sa_ld, const void* b_e4m3, const float* sb,
                      void* d_bf16, int64_t m, int64_t n, int64_t k, void* stream) {
  return gemm_impl("fp8_gemm_nt_ue8m0", true, a_e4m3, sa, sa_ld, b_e4m3, sb, d_bf16, m, n, k, stream);
}

int fp8_gemm_nt(const void* a_e4m3, const float* sa, int64_t sa_ld, const void* b_e4m3, const float* sb,
                void* d_bf16, int64_t m, int64_t n, int64_t k, void* stream) {
  return gemm_impl("fp8_gemm_nt", false, a_e4m3, sa, sa_ld, b_e4m3, sb, d_bf16, m, n, k, stream);
}

int64_t fp8_gemm_nt_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 128 != 0 || m >= kMaxRows || n >= kMaxRows || k > kMaxK) return 0;
  const fgfp8::GemmPlan wp = fgfp8::plan_gemm_ws(m, n, k);
  return wp.kind == fgfp8::kGemmTile256x256SplitK2 ? fgfp8::gemm_splitk_workspace_bytes(m, n) : 0;
}

int fp8_gemm_nt_ws(const void* a_e4m3, const float* sa, int64_t sa_ld, const void* b_e4m3, const float* sb,
                   void* d_bf16, int64_t m, int64_t n, int64_t k, void* workspace, int64_t workspace_bytes,
                   void* stream) {
  if (workspace_bytes < 0) return fail(FGFP8_EINVAL, "fp8_gemm_nt_ws: negative workspace_bytes");
  return gemm_impl("fp8_gemm_nt_ws", false, a_e4m3, sa, sa_ld, b_e4m3, sb, d_bf16, m, n, k, stream,
                   workspace_bytes > 0 ? workspace : nullptr, workspace_bytes);
}

int m_grouped_fp8_gemm_nt_contiguous(const void* a_e4m3, const float* sa, int64_t sa_ld, const int32_t* m_indices,
                                     const void* b_e4m3, const float* sb, int32_t num_groups, void* d_bf16,
                                     int64_t m, int64_t n, int64_t k, void* stream) {
  const char* who = "m_grouped_fp8_gemm_nt_contiguous";
  if (m < 0 || m >= kMaxRows || m % 128 != 0)
    return fail(FGFP8_EINVAL, "%s: m=%lld must be a non-negative multiple of 128", who, (long long)m);
  if (n < 0 || n >= kMaxRows) return fail(FGFP8_EINVAL, "%s: n=%lld out of range", who, (long long)n);
  if (num_groups < 1) return fail(FGFP8_EINVAL, "%s: num_groups=%d must be >= 1", who, (int)num_groups);
  if (int rc = check_k(who, k)) return rc;
  if (int rc = check_sa(who, m, k, sa_ld)) return rc;
  if (m == 0 || n == 0) return FGFP8_OK;
  if (!a_e4m3 || !sa || !m_indices || !b_e4m3 || !sb || !d_bf16) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(a_e4m3) || !aligned16(sa) || !aligned16(m_indices) || !aligned16(b_e4m3) || !aligned16(sb) ||
      !aligned16(d_bf16))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  if (env_flag("FGFP8_PRINT_CONFIG"))
    fprintf(stderr, "[fgfp8] m_grouped_fp8_gemm_nt_contiguous m=%lld n=%lld k=%lld groups=%d: %s\n", (long long)m,
            (long long)n, (long long)k, (int)num_groups, fgfp8::gemm_kind_name(fgfp8::plan_grouped_gemm(m, n, k)));
  return launched(fgfp8::launch_grouped_gemm(a_e4m3, sa, sa_ld, m_indices, b_e4m3, sb, num_groups, d_bf16, m, n, k,
                                             (hipStream_t)stream),
                  who);
}

int fp8_gemm_nt_fp8_out(const void* a_e4m3, const float* sa, int64_t sa_ld, const void* b_e4m3, const float* sb,
                        void* q_e4m3, float* sd, int64_t sd_ld, void* d_bf16, int64_t m, int64_t n, int64_t k,
                        void* stream) {
  const char* who = "fp8_gemm_nt_fp8_out";
  if (m < 0 || m >= kMaxRows) return fail(FGFP8_EINVAL, "%s: m=%lld out of range", who, (long long)m);
  if (n < 0 || n >= kMaxRows || n % 128 != 0)
    return fail(FGFP8_EINVAL, "%s: n=%lld must be a non-negative multiple of 128", who, (long long)n);
  if (int rc = check_k(who, k)) return rc;
  if (int rc = check_sa(who, m, k, sa_ld)) return rc;
  if (sd_ld < m || sd_ld % 4 != 0 || sd_ld < 0 || (n / 128) * sd_ld * 4 >= (int64_t(1) << 31))
    return fail(FGFP8_EINVAL,
                "%s: sd_ld=%lld must be a non-negative multiple of 4, >= m=%lld (and n/128 * sd_ld < 2^29)", who,
                (long long)sd_ld, (long long)m);
  if (m == 0 || n == 0) return FGFP8_OK;
  if (!a_e4m3 || !sa || !b_e4m3 || !sb || !q_e4m3 || !sd) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(a_e4m3) || !aligned16(sa) || !aligned16(b_e4m3) || !aligned16(sb) || !aligned16(q_e4m3) ||
      !aligned16(sd) || (d_bf16 && !aligned16(d_bf16)))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  const fgfp8::GemmKind kind = fgfp8::plan_tiles(m, n, k);
  if (env_flag("FGFP8_PRINT_CONFIG"))
    fprintf(stderr, "[fgfp8] fp8_gemm_nt_fp8_out m=%lld n=%lld k=%lld: %s\n", (long long)m, (long long)n,
            (long long)k, fgfp8::gemm_kind_name(kind));
  return launched(fgfp8::launch_gemm_fp8out(kind, a_e4m3, sa, sa_ld, b_e4m3, sb, q_e4m3, sd, sd_ld, d_bf16, m, n, k,
                                            (hipStream_t)stream),
                  who);
}

static int masked_impl(const char* who, const void* a_e4m3, const float* sa, int64_t sa_ld, const int32_t* masked_m,
                       const void* b_e4m3, const float* sb, int32_t num_groups, int64_t max_m, int64_t expected_m,
                       void* d_bf16, int64_t n, int64_t k, void* stream, void* workspace, int64_t workspace_bytes) {
  if (num_groups < 1) return fail(FGFP8_EINVAL, "%s: num_groups=%d must be >= 1", who, (int)num_groups);
  if (max_m < 0 || max_m % 4 != 0 || (int64_t)num_groups * max_m >= kMaxRows)
    return fail(FGFP8_EINVAL, "%s: max_m=%lld must be a non-negative multiple of 4 (and num_groups * max_m < 2^31)",
                who, (long long)max_m);
  if (n < 0 || n >= kMaxRows) return fail(FGFP8_EINVAL, "%s: n=%lld out of range", who, (long long)n);
  if (int rc = check_k(who, k)) return rc;
  if (int rc = check_sa(who, (int64_t)num_groups * max_m, k, sa_ld)) return rc;
  if (workspace_bytes < 0) return fail(FGFP8_EINVAL, "%s: negative workspace_bytes", who);
  if (workspace_bytes > 0 && (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
    return fail(FGFP8_EINVAL, "%s: the workspace must be a non-null, 256-byte aligned pointer", who);
  if (max_m == 0 || n == 0) return FGFP8_OK;
  if (!a_e4m3 || !sa || !masked_m || !b_e4m3 || !sb || !d_bf16) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(a_e4m3) || !aligned16(sa) || !aligned16(masked_m) || !aligned16(b_e4m3) || !aligned16(sb) ||
      !aligned16(d_bf16))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  const fgfp8::GemmKind kind = fgfp8::plan_masked(num_groups, max_m, expected_m, n);
  const bool split = workspace_bytes >= fgfp8::masked_split_workspace_bytes() &&
                     fgfp8::masked_split_walk(kind, num_groups, max_m, expected_m, n);
  if (env_flag("FGFP8_PRINT_CONFIG"))
    fprintf(stderr, "[fgfp8] %s groups=%d max_m=%lld expected_m=%lld n=%lld k=%lld: %s%s\n", who, (int)num_groups,
            (long long)max_m, (long long)expected_m, (long long)n, (long long)k,
            split ? "tail-split " : "", fgfp8::gemm_kind_name(kind));
  if (split)
    return launched(fgfp8::launch_masked_gemm_split(kind, a_e4m3, sa, sa_ld, masked_m, b_e4m3, sb, num_groups, max_m,
                                                    d_bf16, n, k, workspace, (hipStream_t)stream),
                    who);
  return launched(fgfp8::launch_masked_gemm(kind, a_e4m3, sa, sa_ld, masked_m, b_e4m3, sb, num_groups, max_m, d_bf16,
                                            n, k, (hipStream_t)stream),
                  who);
}

int m_grouped_fp8_gemm_nt_masked(const void* a_e4m3, const float* sa, int64_t sa_ld, const int32_t* masked_m,
                                 const void* b_e4m3, const float* sb, int32_t num_groups, int64_t max_m,
                                 int64_t expected_m, void* d_bf16, int64_t n, int64_t k, void* stream) {
  return masked_impl("m_grouped_fp8_gemm_nt_masked", a_e4m3, sa, sa_ld, masked_m, b_e4m3, sb, num_groups, max_m,
                     expected_m, d_bf16, n, k, stream, nullptr, 0);
}

int64_t m_grouped_fp8_gemm_nt_masked_workspace_bytes(int32_t num_groups, int64_t max_m, int64_t n, int64_t k) {
  if (num_groups < 1 || max_m <= 0 || n <= 0 || k <= 0 || k % 128 != 0 || k > kMaxK) return 0;
  return fgfp8::masked_split_workspace_bytes();
}

int m_grouped_fp8_gemm_nt_masked_ws(const void* a_e4m3, const float* sa, int64_t sa_ld, const int32_t* masked_m,
                                    const void* b_e4m3, const float* sb, int32_t num_groups, int64_t max_m,
                                    int64_t expected_m, void* d_bf16, int64_t n, int64_t k, void* workspace,
                                    int64_t workspace_bytes, void* stream) {
  return masked_impl("m_grouped_fp8_gemm_nt_masked_ws", a_e4m3, sa, sa_ld, masked_m, b_e4m3, sb, num_groups, max_m,
                     expected_m, d_bf16, n, k, stream, workspace, workspace_bytes);
}

int quantize_fp8_mx(const void* x_bf16, int64_t m, int64_t k, void* q_e4m3, int32_t* s, int64_t s_ld,
                    void* stream) {
  const char* who = "quantize_fp8_mx";
  if (m < 0 || m >= kMaxRows) return fail(FGFP8_EINVAL, "%s: m=%lld out of range", who, (long long)m);
  if (int rc = check_k(who, k)) return rc;
  if (int rc = check_sa(who, m, k, s_ld)) return rc;
  if (m == 0) return FGFP8_OK;
  if (!x_bf16 || !q_e4m3 || !s) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(x_bf16) || !aligned16(q_e4m3) || !aligned16(s))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  return launched(fgfp8::launch_quantize_mx(x_bf16, m, k, q_e4m3, s, s_ld, (hipStream_t)stream), who);
}

int fp8_gemm_nt_mx(const void* a_e4m3, const int32_t* sa, int64_t sa_ld, const void* b_e4m3, const int32_t* sb,
                   int64_t sb_ld, void* d_bf16, int64_t m, int64_t n, int64_t k, void* stream) {
  const char* who = "fp8_gemm_nt_mx";
  if (m < 0 || m >= kMaxRows || n < 0 || n >= kMaxRows)
    return fail(FGFP8_EINVAL, "%s: m=%lld n=%lld out of range", who, (long long)m, (long long)n);
  if (int rc = check_k(who, k)) return rc;
  if (int rc = check_sa(who, m, k, sa_ld)) return rc;
  if (sb_ld < n || sb_ld % 4 != 0 || sb_ld < 0 || (k / 128) * sb_ld * 4 >= (int64_t(1) << 31))
    return fail(FGFP8_EINVAL, "%s: sb_ld=%lld must be a non-negative multiple of 4, >= n=%lld (and k/128 * sb_ld < 2^29)",
                who, (long long)sb_ld, (long long)n);
  if (m == 0 || n == 0) return FGFP8_OK;
  if (!a_e4m3 || !sa || !b_e4m3 || !sb || !d_bf16) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(a_e4m3) || !aligned16(sa) || !aligned16(b_e4m3) || !aligned16(sb) || !aligned16(d_bf16))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  const fgfp8::GemmKind kind = fgfp8::plan_tiles(m, n, k);
  if (env_flag("FGFP8_PRINT_CONFIG"))
    fprintf(stderr, "[fgfp8] fp8_gemm_nt_mx m=%lld n=%lld k=%lld: %s\n", (long long)m, (long long)n, (long long)k,
            fgfp8::gemm_kind_name(kind));
  return launched(fgfp8::launch_gemm_mx(kind, a_e4m3, sa, sa_ld, b_e4m3, sb, sb_ld, d_bf16, m, n, k,
                                        (hipStream_t)stream),
                  who);
}

int64_t moe_route_workspace_bytes(int64_t tokens, int32_t num_experts) {
  if (tokens < 0 || num_experts < 1) return -1;
  return fgfp8::moe_route_workspace_bytes(tokens, num_experts);
}

int64_t moe_max_padded_rows(int64_t tokens, int32_t topk, int32_t num_experts) {
  if (tokens < 0 || topk < 1 || num_experts < 1) return -1;
  return (tokens * topk + (int64_t)num_experts * 127 + 127) / 128 * 128;
}

int moe_route_contiguous(const int32_t* topk_idx, int64_t tokens, int32_t topk, int32_t num_experts, int32_t* counts,
                         int32_t* m_indices, int32_t* token_of_row, int32_t* row_of, int64_t m_pad_max,
                         void* workspace, int64_t workspace_bytes, void* stream) {
  const char* who = "moe_route_contiguous";
  if (tokens < 0 || tokens >= kMaxRows) return fail(FGFP8_EINVAL, "%s: tokens=%lld out of range", who, (long long)tokens);
  if (topk < 1 || topk > 8) return fail(FGFP8_EINVAL, "%s: topk=%d must be 1..8", who, (int)topk);
  if (num_experts < 1 || num_experts > 2048)
    return fail(FGFP8_EINVAL, "%s: num_experts=%d must be 1..2048", who, (int)num_experts);
  const int64_t need_rows = moe_max_padded_rows(tokens, topk, num_experts);
  if (m_pad_max < need_rows || m_pad_max % 128 != 0 || m_pad_max >= kMaxRows)
    return fail(FGFP8_EINVAL, "%s: m_pad_max=%lld must be a multiple of 128 and >= %lld", who, (long long)m_pad_max,
                (long long)need_rows);
  if (workspace_bytes < fgfp8::moe_route_workspace_bytes(tokens, num_experts))
    return fail(FGFP8_EINVAL, "%s: workspace of %lld bytes, need %lld", who, (long long)workspace_bytes,
                (long long)fgfp8::moe_route_workspace_bytes(tokens, num_experts));
  if (!counts || !m_indices || !token_of_row || !workspace || (tokens > 0 && (!topk_idx || !row_of)))
    return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (int rc = check_device(who)) return rc;
  return launched(fgfp8::launch_moe_route(topk_idx, tokens, topk, num_experts, counts, m_indices, token_of_row, row_of,
                                          m_pad_max, workspace, (hipStream_t)stream),
                  who);
}

int moe_route_contiguous_noalloc(const int32_t* topk_idx, int64_t tokens, int32_t topk, int32_t num_experts,
                                 int32_t* counts, int32_t* m_indices, int32_t* token_of_row, int32_t* row_of,
                                 int64_t m_pad_max, void* stream) {
  const char* who = "moe_route_contiguous_noalloc";
  if (tokens < 0 || tokens >= kMaxRows) return fail(FGFP8_EINVAL, "%s: tokens=%lld out of range", who, (long long)tokens);
  if (topk < 1 || topk > 8) return fail(FGFP8_EINVAL, "%s: topk=%d must be 1..8", who, (int)topk);
  if (num_experts < 1 || num_experts > 2048)
    return fail(FGFP8_EINVAL, "%s: num_experts=%d must be 1..2048", who, (int)num_experts);
  const int64_t need_rows = moe_max_padded_rows(tokens, topk, num_experts);
  if (m_pad_max < need_rows || m_pad_max % 128 != 0 || m_pad_max >= kMaxRows)
    return fail(FGFP8_EINVAL, "%s: m_pad_max=%lld must be a multiple of 128 and >= %lld", who, (long long)m_pad_max,
                (long long)need_rows);
  const int64_t need = fgfp8::moe_route_workspace_bytes(tokens, num_experts);
  if (need > fgfp8::moe_route_scratch_bytes())
    return fail(FGFP8_EINVAL,
                "%s: tokens=%lld with num_experts=%d need %lld bytes of routing workspace, beyond the fixed %lld "
                "(use moe_route_contiguous with a workspace of its own)",
                who, (long long)tokens, (int)num_experts, (long long)need, (long long)fgfp8::moe_route_scratch_bytes());
  if (!counts || !m_indices || !token_of_row || (tokens > 0 && (!topk_idx || !row_of)))
    return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (int rc = check_device(who)) return rc;
  void* ws = nullptr;
  const hipError_t e = fgfp8::moe_route_scratch(&ws);
  if (e != hipSuccess)
    return fail(FGFP8_ELAUNCH, "%s: cannot find the routing workspace on this device: %s", who, hipGetErrorString(e));
  return launched(fgfp8::launch_moe_route(topk_idx, tokens, topk, num_experts, counts, m_indices, token_of_row, row_of,
                                          m_pad_max, ws, (hipStream_t)stream),
                  who);
}

int64_t moe_route_noalloc_max_workspace_bytes(void) { return fgfp8::moe_route_scratch_bytes(); }

int moe_gather_quantize(const void* x_bf16, int64_t tokens, int64_t k, const int32_t* token_of_row, int64_t m_pad_max,
                        void* q_e4m3, float* sa, int64_t sa_ld, void* stream) {
  const char* who = "moe_gather_quantize";
  if (m_pad_max < 0 || m_pad_max >= kMaxRows) return fail(FGFP8_EINVAL, "%s: m_pad_max out of range", who);
  if (tokens < 0 || tokens >= kMaxRows) return fail(FGFP8_EINVAL, "%s: tokens out of range", who);
  if (int rc = check_k(who, k)) return rc;
  if (int rc = check_sa(who, m_pad_max, k, sa_ld)) return rc;
  if (m_pad_max == 0) return FGFP8_OK;
  if ((tokens > 0 && !x_bf16) || !token_of_row || !q_e4m3 || !sa) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(x_bf16) || !aligned16(q_e4m3) || !aligned16(sa))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  return launched(fgfp8::launch_moe_gather_quantize(x_bf16, tokens, k, token_of_row, m_pad_max, q_e4m3, sa, sa_ld,
                                                    (hipStream_t)stream),
                  who);
}

int moe_gather_quantize_tokens(const void* x_bf16, int64_t tokens, int64_t k, int32_t topk, const int32_t* row_of,
                               const int32_t* token_of_row, int64_t m_pad_max, void* q_e4m3, float* sa, int64_t sa_ld,
                               void* stream) {
  const char* who = "moe_gather_quantize_tokens";
  if (m_pad_max < 0 || m_pad_max >= kMaxRows) return fail(FGFP8_EINVAL, "%s: m_pad_max out of range", who);
  if (tokens < 0 || tokens >= kMaxRows / 8) return fail(FGFP8_EINVAL, "%s: tokens out of range", who);
  if (topk < 1 || topk > 8) return fail(FGFP8_EINVAL, "%s: topk=%d must be in [1, 8]", who, (int)topk);
  if (int rc = check_k(who, k)) return rc;
  if (int rc = check_sa(who, m_pad_max, k, sa_ld)) return rc;
  if (m_pad_max == 0) return FGFP8_OK;
  if ((tokens > 0 && (!x_bf16 || !row_of)) || !token_of_row || !q_e4m3 || !sa)
    return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(x_bf16) || !aligned16(q_e4m3) || !aligned16(sa))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  return launched(fgfp8::launch_moe_gather_quantize_tokens(x_bf16, tokens, k, topk, row_of, token_of_row, m_pad_max,
                                                           q_e4m3, sa, sa_ld, (hipStream_t)stream),
                  who);
}

int silu_mul_quantize(const void* h_bf16, int64_t m, int64_t inter, const int32_t* m_indices, void* q_e4m3, float* sa,
                      int64_t sa_ld, void* stream) {
  const char* who = "silu_mul_quantize";
  if (m < 0 || m >= kMaxRows) return fail(FGFP8_EINVAL, "%s: m=%lld out of range", who, (long long)m);
  if (int rc = check_k(who, inter)) return rc;
  if (int rc = check_sa(who, m, inter, sa_ld)) return rc;
  if (m == 0) return FGFP8_OK;
  if (!h_bf16 || !m_indices || !q_e4m3 || !sa) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(h_bf16) || !aligned16(q_e4m3) || !aligned16(sa))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  return launched(fgfp8::launch_moe_silu_mul_quantize(h_bf16, m, inter, m_indices, q_e4m3, sa, sa_ld,
                                                      (hipStream_t)stream),
                  who);
}

int moe_gate_up_silu_quantize(const void* a_e4m3, const float* sa, int64_t sa_ld, const int32_t* m_indices,
                              const void* w1_e4m3, const float* sb1, int32_t num_groups, void* q_e4m3, float* sq,
                              int64_t sq_ld, int64_t m, int64_t inter, int64_t k, void* stream) {
  const char* who = "moe_gate_up_silu_quantize";
  if (m < 0 || m >= kMaxRows || m % 128 != 0)
    return fail(FGFP8_EINVAL, "%s: m=%lld must be a non-negative multiple of 128", who, (long long)m);
  if (num_groups < 1) return fail(FGFP8_EINVAL, "%s: num_groups=%d must be >= 1", who, (int)num_groups);
  if (int rc = check_k(who, k)) return rc;
  if (int rc = check_k(who, inter)) return rc;
  if ((inter + 128) * k >= (int64_t(1) << 31))
    return fail(FGFP8_EINVAL, "%s: (inter + 128) * k must stay below 2^31", who);
  if (int rc = check_sa(who, m, k, sa_ld)) return rc;
  if (int rc = check_sa(who, m, inter, sq_ld)) return rc;
  if (m == 0) return FGFP8_OK;
  if (!a_e4m3 || !sa || !m_indices || !w1_e4m3 || !sb1 || !q_e4m3 || !sq)
    return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(a_e4m3) || !aligned16(sa) || !aligned16(m_indices) || !aligned16(w1_e4m3) || !aligned16(sb1) ||
      !aligned16(q_e4m3) || !aligned16(sq))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  return launched(fgfp8::launch_grouped_gemm_silu(a_e4m3, sa, sa_ld, m_indices, w1_e4m3, sb1, num_groups, q_e4m3,
                                                  sq, sq_ld, m, inter, k, (hipStream_t)stream),
                  who);
}

int moe_combine(const void* y_bf16, int64_t y_rows, int64_t hdim, const int32_t* row_of, const float* topk_weights,
                int64_t tokens, int32_t topk, void* out_bf16, void* stream) {
  const char* who = "moe_combine";
  if (y_rows < 0 || y_rows >= kMaxRows) return fail(FGFP8_EINVAL, "%s: y_rows out of range", who);
  if (tokens < 0 || tokens >= kMaxRows) return fail(FGFP8_EINVAL, "%s: tokens out of range", who);
  if (topk < 1 || topk > 8) return fail(FGFP8_EINVAL, "%s: topk=%d must be 1..8", who, (int)topk);
  if (hdim <= 0 || hdim % 8 != 0) return fail(FGFP8_EINVAL, "%s: hdim=%lld must be a positive multiple of 8", who, (long long)hdim);
  if (tokens == 0) return FGFP8_OK;
  if ((y_rows > 0 && !y_bf16) || !row_of || !topk_weights || !out_bf16)
    return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(y_bf16) || !aligned16(out_bf16))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  return launched(fgfp8::launch_moe_combine(y_bf16, y_rows, hdim, row_of, topk_weights, tokens, topk, out_bf16,
                                            (hipStream_t)stream),
                  who);
}

// The kernel form fp8_linear_nt runs for m rows (act_out: the quantized
// activation is wanted too): "lds4" (m <= 4: the activation quantized into
// LDS by every workgroup), "lds16" (the three-slab form, the same up to 16
// rows), "registers" (each wave quantizes its K range in registers), or
// nullptr for quantize_fp8_groups followed by fp8_gemm_nt.
static const char* linear_form(int64_t m, int64_t n, int64_t k, bool act_out) {
  if (fgfp8::decode_fused_wide(m, n, k, act_out)) return "lds16";
  if (m <= fgfp8::kFusedLdsMaxM)
    return k <= fgfp8::kFusedLdsMaxK && getenv("FGFP8_DECODE_XQ") == nullptr ? "lds4" : "registers";
  if (m <= fgfp8::kFusedMaxM && !act_out) return "registers";
  return nullptr;
}

int fp8_linear_nt(const void* x_bf16, int64_t m, int64_t k, const void* b_e4m3, const float* sb, int64_t n,
                  void* d_bf16, void* q_e4m3, float* sa, int64_t sa_ld, void* stream) {
  const char* who = "fp8_linear_nt";
  if (m < 0 || m >= kMaxRows || n < 0 || n >= kMaxRows)
    return fail(FGFP8_EINVAL, "%s: m=%lld n=%lld out of range", who, (long long)m, (long long)n);
  if (int rc = check_k(who, k)) return rc;
  if (m == 0 || n == 0) return FGFP8_OK;
  if (!x_bf16 || !b_e4m3 || !sb || !d_bf16) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if ((q_e4m3 == nullptr) != (sa == nullptr))
    return fail(FGFP8_EINVAL, "%s: q_e4m3 and sa must be given together", who);
  const char* form = linear_form(m, n, k, q_e4m3 != nullptr);
  const bool fused = form != nullptr;
  if (!fused && q_e4m3 == nullptr)
    return fail(FGFP8_EINVAL, "%s: m=%lld k=%lld needs the q_e4m3/sa workspace", who, (long long)m, (long long)k);
  if (q_e4m3 != nullptr) {
    if (int rc = check_sa(who, m, k, sa_ld)) return rc;
    if (!aligned16(q_e4m3) || !aligned16(sa)) return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  }
  if (!aligned16(x_bf16) || !aligned16(b_e4m3) || !aligned16(sb) || !aligned16(d_bf16))
    return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  if (fused) {
    if (env_flag("FGFP8_PRINT_CONFIG"))
      fprintf(stderr, "[fgfp8] fp8_linear_nt m=%lld n=%lld k=%lld: fused decode split=%d form=%s\n", (long long)m,
              (long long)n, (long long)k, fgfp8::decode_split(m, n, k), form);
    return launched(fgfp8::launch_decode_fused(x_bf16, b_e4m3, sb, d_bf16, m, n, k, q_e4m3, sa, sa_ld,
                                               (hipStream_t)stream),
                    who);
  }
  if (int rc = launched(fgfp8::launch_quantize_groups(x_bf16, m, k, q_e4m3, sa, sa_ld, (hipStream_t)stream), who))
    return rc;
  const fgfp8::GemmPlan plan = fgfp8::plan_gemm(m, n, k);
  return launched(fgfp8::launch_gemm(plan, q_e4m3, sa, sa_ld, b_e4m3, sb, d_bf16, m, n, k, (hipStream_t)stream), who);
}

int fgfp8_stream_read(const void* src, int64_t bytes, void* out, int64_t out_bytes, void* stream) {
  const char* who = "fgfp8_stream_read";
  const int64_t unit = fgfp8::stream_read_unit_bytes();
  if (bytes < 0 || bytes % unit != 0 || out_bytes < 4096)
    return fail(FGFP8_EINVAL, "%s: bytes=%lld must be a multiple of %lld and out_bytes >= 4096", who,
                (long long)bytes, (long long)unit);
  if (bytes == 0) return FGFP8_OK;
  if (!src || !out) return fail(FGFP8_EINVAL, "%s: null pointer", who);
  if (!aligned16(src) || !aligned16(out)) return fail(FGFP8_EINVAL, "%s: base pointers must be 16-byte aligned", who);
  if (int rc = check_device(who)) return rc;
  return launched(fgfp8::launch_stream_read(src, bytes, out, out_bytes, (hipStream_t)stream), who);
}

static void describe_plan(int64_t m, int64_t n, int64_t k, char* buf, size_t len) {
  const fgfp8::GemmPlan plan = fgfp8::plan_gemm(m, n, k);
  const char* walk = fgfp8::plan_persistent(plan, m, n, k) ? " persistent" : "";
  const fgfp8::GemmPlan wp = fgfp8::plan_gemm_ws(m, n, k);
  if (wp.kind != plan.kind)
    snprintf(buf, (size_t)len, "%s split=%d%s; with workspace: %s", fgfp8::gemm_kind_name(plan.kind), plan.split,
             walk, fgfp8::gemm_kind_name(wp.kind));
  else if (plan.kind == fgfp8::kGemmDecode && fgfp8::decode_plan(m, n, k).slabs > 1)
    snprintf(buf, (size_t)len, "%s split=%d slabs=%d", fgfp8::gemm_kind_name(plan.kind), plan.split,
             fgfp8::decode_plan(m, n, k).slabs);
  else
    snprintf(buf, (size_t)len, "%s split=%d%s", fgfp8::gemm_kind_name(plan.kind), plan.split, walk);
}

int fgfp8_describe_gemm(int64_t m, int64_t n, int64_t k, char* buf, int64_t len) {
  if (!buf || len <= 0) return fail(FGFP8_EINVAL, "fgfp8_describe_gemm: null or empty buffer");
  if (m <= 0 || n <= 0 || k <= 0 || k % 128) return fail(FGFP8_EINVAL, "fgfp8_describe_gemm: bad shape");
  describe_plan(m, n, k, buf, (size_t)len);
  return FGFP8_OK;
}

int fgfp8_describe_grouped(int64_t m, int64_t n, int64_t k, char* buf, int64_t len) {
  if (!buf || len <= 0) return fail(FGFP8_EINVAL, "fgfp8_describe_grouped: null or empty buffer");
  if (m <= 0 || m % 128 || n <= 0 || k <= 0 || k % 128) return fail(FGFP8_EINVAL, "fgfp8_describe_grouped: bad shape");
  snprintf(buf, (size_t)len, "%s%s", fgfp8::gemm_kind_name(fgfp8::plan_grouped_gemm(m, n, k)),
           fgfp8::plan_grouped_walk(m, n, k) ? " persistent" : "");
  return FGFP8_OK;
}

int fgfp8_describe_linear(int64_t m, int64_t n, int64_t k, int act_out, char* buf, int64_t len) {
  if (!buf || len <= 0) return fail(FGFP8_EINVAL, "fgfp8_describe_linear: null or empty buffer");
  if (m <= 0 || n <= 0 || k <= 0 || k % 128) return fail(FGFP8_EINVAL, "fgfp8_describe_linear: bad shape");
  const char* form = linear_form(m, n, k, act_out != 0);
  if (form != nullptr) {
    const fgfp8::DecodePlan p = fgfp8::decode_plan(m, n, k);
    snprintf(buf, (size_t)len, "fused act-quant + decode_splitk_slab16 split=%d slabs=%d form=%s", p.ks,
             strcmp(form, "lds16") == 0 ? 3 : (strcmp(form, "registers") == 0 ? 1 : p.slabs), form);
    return FGFP8_OK;
  }
  if (act_out == 0)
    return fail(FGFP8_EINVAL, "fgfp8_describe_linear: m=%lld needs the q_e4m3/sa workspace", (long long)m);
  char plan[160];
  describe_plan(m, n, k, plan, sizeof plan);
  snprintf(buf, (size_t)len, "quantize_fp8_groups + %s", plan);
  return FGFP8_OK;
}

}  // extern "C"
