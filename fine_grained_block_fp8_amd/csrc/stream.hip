// A plain streaming read of device memory, as a measurement aid: the rate a
// kernel that only reads contiguous memory reaches at a given size is the
// practical ceiling for the HBM-bound kernels (the decode product streams
// its weight exactly once per call).  Every lane keeps kInFlight 16-byte
// loads in flight, workgroups stride over the buffer, and each thread folds
// what it read into one XOR it stores at the end, so no load can be dropped.

#include "common.hpp"
#include "kernels.hpp"

namespace fgfp8 {

constexpr int kStreamThreads = 256;
constexpr int kInFlight = 8;
constexpr int64_t kStreamUnit = (int64_t)kStreamThreads * 16 * kInFlight;  // bytes per workgroup step

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint8_t* __restrict__ src, int64_t units,
                                                                     uint4* __restrict__ out) {
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const uint4* p = reinterpret_cast<const uint4*>(src + u * kStreamUnit) + threadIdx.x;
    uint4 v[kInFlight];
#pragma unroll
    for (int i = 0; i < kInFlight; i++) v[i] = p[i * kStreamThreads];
#pragma unroll
    for (int i = 0; i < kInFlight; i++) {
      acc.x ^= v[i].x;
      acc.y ^= v[i].y;
      acc.z ^= v[i].z;
      acc.w ^= v[i].w;
    }
  }
  out[(int64_t)blockIdx.x * kStreamThreads + threadIdx.x] = acc;
}

int64_t stream_read_unit_bytes() { return kStreamUnit; }

hipError_t launch_stream_read(const void* src, int64_t bytes, void* out, int64_t out_bytes, hipStream_t stream) {
  const int64_t units = bytes / kStreamUnit;
  int64_t grid = out_bytes / (kStreamThreads * 16);
  if (grid > units) grid = units;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(stream_read_kernel, dim3((uint32_t)grid), dim3(kStreamThreads), 0, stream,
                     static_cast<const uint8_t*>(src), units, static_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace fgfp8
