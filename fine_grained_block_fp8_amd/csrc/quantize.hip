// Activation (1x128 group) and weight (128x128 block) quantization to E4M3
// with FP32 scales, for gfx950.
//
// Recipe: per-(1x128) activation scales and per-(128x128) weight scales
// (deepgemm-rust README, "What's implemented" table, fp8_gemm_nt row); every
// 128-element run of a row gets its own FP8 scale, and the scales are laid
// out one K group after another with the row count rounded up to four
// (Linnet "Backend plugins" page, plugin module docstring).  Scale s = fl32(amax/448),
// 1 for an all-zero group; element code = E4M3_RNE(fl32(x / s)).  The UE8M0
// variants round s up to a power of two (the Blackwell path's UE8M0 scale
// factors, deepgemm-rust README key techniques) and are otherwise the same;
// the MX variant takes one such scale per 1x32 block (the README's gran-32
// recipe) and stores E8M0 codes.

#include "common.hpp"
#include "kernels.hpp"

namespace fgfp8 {

// ---------------------------------------------------------------- groups
// A wave quantizes a block of 4 rows x 4 groups.  In step i it reads row
// r0 + i, groups g0 .. g0+3: 1 KB contiguous, the 16 lanes of DPP row j
// holding group g0 + j (8 bf16 = 16 bytes per lane), so a group's amax is a
// 16-lane DPP reduction.  All four rows are loaded before any is quantized
// (four 16-byte loads in flight per lane).  After the four steps, lane 16j
// holds the scales of group g0 + j for rows r0 .. r0+3 -- four consecutive
// floats of the MN-major scale column -- and stores them at once.  Waves are
// numbered row-block-major so that neighbouring waves read neighbouring
// kilobytes of the same rows.  The kernel is bound by HBM: 2 bytes in and 1
// byte out per element.
//
// MASKED (a dispatch buffer of groups of max_m rows, max_m % 4 == 0): only
// rows r < counts[group] of each group (clamped to [0, max_m]) count; m is
// then the row of the group's end, so rows past the count are neither read
// nor written, and a wave whose four rows are all past it exits at once.
constexpr int kQgWaves = 4;

// Rows r0 .. r0 + 3 (those < m) and groups 4 gq .. 4 gq + 3 of x, one wave.
template <bool UE8M0>
__device__ __forceinline__ void quantize_block4(const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
                                                float* __restrict__ sa, int64_t m, int64_t k, int64_t sa_ld,
                                                int64_t r0, int64_t gq, int lane) {
  const int64_t g = gq * 4 + (lane >> 4);
  const bool g_ok = g < k / kGroup;
  const int64_t col = g * kGroup + (lane & 15) * 8;
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; i++)
    v[i] = (g_ok && r0 + i < m) ? *reinterpret_cast<const uint4*>(x + (r0 + i) * k + col) : make_uint4(0, 0, 0, 0);
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t amax_bits = row16_max_u32(absmax8_bits(v[i]));
    s[i] = UE8M0 ? group_scale_ue8m0(__uint_as_float(amax_bits)) : group_scale(__uint_as_float(amax_bits));
    const double r = 1.0 / (double)s[i];
    const uint2 o = quantize8(v[i], r);
    if (g_ok && r0 + i < m) *reinterpret_cast<uint2*>(q + (r0 + i) * k + col) = o;
  }
  if (g_ok && (lane & 15) == 0) {
    float* dst = sa + g * sa_ld + r0;
    if (r0 + 4 <= m) {
      *reinterpret_cast<float4*>(dst) = make_float4(s[0], s[1], s[2], s[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (r0 + i < m) dst[i] = s[i];
    }
  }
}

template <bool UE8M0, bool MASKED = false>
__global__ __launch_bounds__(kQgWaves * 64) void quantize_groups_kernel(const uint16_t* __restrict__ x,
                                                                         uint8_t* __restrict__ q,
                                                                         float* __restrict__ sa, int64_t m, int64_t k,
                                                                         int64_t sa_ld, int64_t group_quads,
                                                                         int64_t total_blocks,
                                                                         const int32_t* __restrict__ counts = nullptr,
                                                                         int64_t max_m = 0) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * kQgWaves + (threadIdx.x >> 6);
  if (blk >= total_blocks) return;  // wave-uniform
  const int64_t r0 = (blk / group_quads) * 4;
  if constexpr (MASKED) {
    const int64_t grp = r0 / max_m;  // the block's four rows share a group
    int c = __builtin_amdgcn_readfirstlane(counts[grp]);
    c = c < 0 ? 0 : (c > max_m ? (int)max_m : c);
    m = grp * max_m + c;
    if (r0 >= m) return;  // wave-uniform
  }
  quantize_block4<UE8M0>(x, q, sa, m, k, sa_ld, r0, blk % group_quads, lane);
}

hipError_t launch_quantize_groups(const void* x, int64_t m, int64_t k, void* q, float* sa, int64_t sa_ld,
                                  hipStream_t stream, bool ue8m0) {
  const int64_t row_blocks = (m + 3) / 4;
  const int64_t group_quads = (k / kGroup + 3) / 4;
  const int64_t total = row_blocks * group_quads;
  const int64_t blocks = (total + kQgWaves - 1) / kQgWaves;
  if (ue8m0)
    hipLaunchKernelGGL(quantize_groups_kernel<true>, dim3((uint32_t)blocks), dim3(kQgWaves * 64), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<uint8_t*>(q), sa, m, k, sa_ld, group_quads, total);
  else
    hipLaunchKernelGGL(quantize_groups_kernel<false>, dim3((uint32_t)blocks), dim3(kQgWaves * 64), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<uint8_t*>(q), sa, m, k, sa_ld, group_quads, total);
  return hipGetLastError();
}

// The masked form over a bounded grid: every workgroup forms the exclusive
// prefix sums of the groups' live 4-row blocks (ceil(count / 4)) in LDS, and
// its waves stride over the live (row block, group quad) tasks only, finding
// a task's group by binary search.  Launching one wave per possible task
// instead costs a count load per wave even where every row is past the
// count (most of a dispatch buffer).  Up to kFlatMaxGroups groups.
constexpr int kFlatMaxGroups = 1024;

__global__ __launch_bounds__(256) void quantize_groups_masked_flat_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ sa, const int32_t* __restrict__ counts,
    int num_groups, int64_t max_m, int64_t k, int64_t sa_ld, int64_t group_quads) {
  __shared__ int64_t pre[kFlatMaxGroups + 1];
  __shared__ int64_t wave_sum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // thread t owns groups 4t .. 4t + 3
  int64_t mine[4], local = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int g = 4 * tid + i;
    int c = g < num_groups ? counts[g] : 0;
    c = c < 0 ? 0 : (c > max_m ? (int)max_m : c);
    mine[i] = (c + 3) / 4;
    local += mine[i];
  }
  int64_t incl = local;  // inclusive scan over the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int64_t base = 0;
  for (int w = 0; w < wave; w++) base += wave_sum[w];
  int64_t run = base + incl - local;  // exclusive prefix of group 4t
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int g = 4 * tid + i;
    if (g < num_groups) pre[g] = run;
    run += mine[i];
  }
  if (tid == 255) pre[num_groups] = run;  // the total (groups past num_groups count zero)
  __syncthreads();
  const int64_t tasks = pre[num_groups] * group_quads;
  const int64_t stride = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t < tasks; t += stride) {  // uniform per wave
    const int64_t rb = t / group_quads, gq = t % group_quads;
    int lo = 0, hi = num_groups - 1;  // the last group with pre[g] <= rb
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= rb) lo = mid;
      else hi = mid - 1;
    }
    int c = counts[lo];
    c = c < 0 ? 0 : (c > max_m ? (int)max_m : c);
    const int64_t r0 = lo * max_m + 4 * (rb - pre[lo]);
    quantize_block4<false>(x, q, sa, lo * max_m + c, k, sa_ld, r0, gq, lane);
  }
}

hipError_t launch_quantize_groups_masked(const void* x, const int32_t* masked_m, int32_t num_groups, int64_t max_m,
                                         int64_t k, void* q, float* sa, int64_t sa_ld, hipStream_t stream) {
  const int64_t m = (int64_t)num_groups * max_m;
  const int64_t group_quads = (k / kGroup + 3) / 4;
  const int64_t total = m / 4 * group_quads;
  const int64_t blocks = (total + kQgWaves - 1) / kQgWaves;
  if (num_groups <= kFlatMaxGroups) {
    const int64_t grid = blocks < 2048 ? blocks : 2048;
    hipLaunchKernelGGL(quantize_groups_masked_flat_kernel, dim3((uint32_t)grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<uint8_t*>(q), sa, masked_m, (int)num_groups,
                       max_m, k, sa_ld, group_quads);
  } else {
    hipLaunchKernelGGL((quantize_groups_kernel<false, true>), dim3((uint32_t)blocks), dim3(kQgWaves * 64), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<uint8_t*>(q), sa, m, k, sa_ld, group_quads, total,
                       masked_m, max_m);
  }
  return hipGetLastError();
}

// -------------------------------------------------------------------- MX
// The MX recipe: one power-of-two scale per 1x32 block of a row (the UE8M0
// rule over the block's amax), E8M0 codes packed four to an int32 per row
// and 128-column chunk (byte j = block 4c + j), MN-major s[c][row].  Same
// wave layout as quantize_groups_kernel: a 16-lane quarter holds one 128-
// column chunk of a row, 8 values per lane, so a 4-lane quad holds one
// 32-block and its amax is a two-step lane exchange; lane 0 of the quarter
// gathers the four codes.  Serves activations and weights alike (a weight's
// blocks run along its rows, per output column).
__global__ __launch_bounds__(kQgWaves * 64) void quantize_mx_kernel(const uint16_t* __restrict__ x,
                                                                    uint8_t* __restrict__ q, int32_t* __restrict__ s,
                                                                    int64_t m, int64_t k, int64_t s_ld,
                                                                    int64_t group_quads, int64_t total_blocks) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * kQgWaves + (threadIdx.x >> 6);
  if (blk >= total_blocks) return;  // wave-uniform
  const int64_t r0 = (blk / group_quads) * 4;
  const int64_t g = (blk % group_quads) * 4 + (lane >> 4);
  const bool g_ok = g < k / kGroup;
  const int64_t col = g * kGroup + (lane & 15) * 8;
  const int quarter = lane & ~15;
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; i++)
    v[i] = (g_ok && r0 + i < m) ? *reinterpret_cast<const uint4*>(x + (r0 + i) * k + col) : make_uint4(0, 0, 0, 0);
  uint32_t packed[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    uint32_t am = absmax8_bits(v[i]);
    am = max(am, (uint32_t)__shfl_xor((int)am, 1));
    am = max(am, (uint32_t)__shfl_xor((int)am, 2));
    const float sc = group_scale_ue8m0(__uint_as_float(am));
    const double r = 1.0 / (double)sc;
    const uint2 o = quantize8(v[i], r);
    if (g_ok && r0 + i < m) *reinterpret_cast<uint2*>(q + (r0 + i) * k + col) = o;
    const int code = e8m0_of(sc);
    packed[i] = (uint32_t)__shfl(code, quarter) | ((uint32_t)__shfl(code, quarter + 4) << 8) |
                ((uint32_t)__shfl(code, quarter + 8) << 16) | ((uint32_t)__shfl(code, quarter + 12) << 24);
  }
  if (g_ok && (lane & 15) == 0) {
    int32_t* dst = s + g * s_ld + r0;
    if (r0 + 4 <= m) {
      *reinterpret_cast<int4*>(dst) = make_int4((int)packed[0], (int)packed[1], (int)packed[2], (int)packed[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (r0 + i < m) dst[i] = (int)packed[i];
    }
  }
}

hipError_t launch_quantize_mx(const void* x, int64_t m, int64_t k, void* q, int32_t* s, int64_t s_ld,
                              hipStream_t stream) {
  const int64_t group_quads = (k / kGroup + 3) / 4;
  const int64_t total = (m + 3) / 4 * group_quads;
  const int64_t blocks = (total + kQgWaves - 1) / kQgWaves;
  hipLaunchKernelGGL(quantize_mx_kernel, dim3((uint32_t)blocks), dim3(kQgWaves * 64), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<uint8_t*>(q), s, m, k, s_ld, group_quads, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------- blocks
// One workgroup per 128x128 block: thread t owns 64 elements of row t/2; the
// block amax is a wave shuffle reduction followed by an LDS combine across the
// four waves.  Offline (weights are quantized once), so simplicity wins.
template <bool UE8M0>
__global__ __launch_bounds__(256) void quantize_blocks_kernel(const uint16_t* __restrict__ w, uint8_t* __restrict__ q,
                                                              float* __restrict__ sb, int64_t n, int64_t k) {
  __shared__ uint32_t red[4];
  const int t = threadIdx.x;
  const int64_t kb = blockIdx.x, nb = blockIdx.y;
  const int64_t row = nb * kGroup + (t >> 1);
  const int64_t col = kb * kGroup + (t & 1) * 64;
  const bool valid = row < n;
  uint4 v[8];
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    v[i] = valid ? *reinterpret_cast<const uint4*>(w + row * k + col + 8 * i) : make_uint4(0, 0, 0, 0);
    am = max(am, absmax8_bits(v[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off));
  if ((t & 63) == 0) red[t >> 6] = am;
  __syncthreads();
  am = max(max(red[0], red[1]), max(red[2], red[3]));
  const float s = UE8M0 ? group_scale_ue8m0(__uint_as_float(am)) : group_scale(__uint_as_float(am));
  const double r = 1.0 / (double)s;
  if (valid) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const uint2 a = quantize8(v[i], r), b = quantize8(v[i + 1], r);
      *reinterpret_cast<uint4*>(q + row * k + col + 8 * i) = make_uint4(a.x, a.y, b.x, b.y);
    }
  }
  if (t == 0) sb[nb * (k / kGroup) + kb] = s;
}

hipError_t launch_quantize_blocks(const void* w, int64_t n, int64_t k, void* q, float* sb, hipStream_t stream,
                                  bool ue8m0) {
  const int64_t nbk = k / kGroup, nbn = (n + kGroup - 1) / kGroup;
  if (ue8m0)
    hipLaunchKernelGGL(quantize_blocks_kernel<true>, dim3((uint32_t)nbk, (uint32_t)nbn), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(w), static_cast<uint8_t*>(q), sb, n, k);
  else
    hipLaunchKernelGGL(quantize_blocks_kernel<false>, dim3((uint32_t)nbk, (uint32_t)nbn), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(w), static_cast<uint8_t*>(q), sb, n, k);
  return hipGetLastError();
}

}  // namespace fgfp8
